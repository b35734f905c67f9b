/*
 * starkv.h -- C ABI of libstarkv.so: attention that reads a compressed latent
 * KV cache directly (STAR-KV), for AMD Instinct MI355X (gfx950).
 *
 * What is stored and computed follows the technical review of arXiv
 * 2606.08382 ("STAR-KV: Learning the Rank Is Only Half of KV Cache
 * Compression"):
 *   - keys are per-KV-head low-rank latents and values one joint low-rank
 *     latent shared by all heads (section 5, eq. 9 and eq. 12);
 *   - reconstruction is K_g = Z_k,g B_key[g]^T, V = Z_v B_value^T in the
 *     row-vector convention of eq. 2 (section 2.2), V_g being the g-th block
 *     of head_dim columns of V;
 *   - latents may be block-wise Walsh-Hadamard rotated and are stored with the
 *     leading quarter of the channels at 4 bits and the rest at 3 bits
 *     (section 6.1, eq. 13 and eq. 14);
 *   - the calls follow Algorithm 2 (section 6.2): project and rotate latents,
 *     quantize and append them, then score against the latent keys, apply the
 *     softmax, multiply the stacked head probabilities by the shared latent
 *     values and apply the head-specific value factors -- without ever
 *     writing reconstructed keys or values to memory.
 * Query head h reads KV head g(h) = h / (n_q_heads / n_kv_heads).
 *
 * Conventions for every entry point:
 *   - Pointers marked (host) are host memory; every other pointer is device
 *     memory on the current HIP device, 16-byte aligned.
 *   - The caller allocates and frees everything (cache, inputs, outputs,
 *     workspace).  The library allocates no device memory on these calls.
 *     Its only state is host-side: a memo of the runtime's occupancy answer
 *     per decode kernel and device (mutex-guarded, filled on first use), from
 *     which the automatic split count is derived.  (starkv_decode_noalloc
 *     below is the exception: it uses a fixed device array of the library.)
 *   - Compute calls are asynchronous on `stream` and never synchronize.
 *   - Arguments are validated on the host before any HIP call; a failed
 *     validation returns a negative status and touches no memory.  A kernel
 *     launch failure returns STARKV_ELAUNCH.  No C++ exception crosses the ABI.
 *   - Inputs must be finite; otherwise results are unspecified.  Decode
 *     keeps three intermediates in fp16 (the projected query q~, the
 *     4/3-bit value operand P * 2^k * group scale with P <= 4 and 2^k <= 64,
 *     and each split's partial rows divided by their exp-sum), so:
 *       - quantized caches: latents within the fp16 range (their scale and
 *         zero are fp16), and value group scales below 256 (a 3-bit group's
 *         range below ~1.8e3, a 4-bit group's below ~1.5e4);
 *       - BF16 caches: softmax-weighted averages of the value latents (the
 *         partial rows) within the fp16 range, |.| < 65504.
 *     Measured within these limits (value latents scaled 1e-3 .. 1e5, key
 *     latents 1e-2 .. 1e3, queries sharpened 32x) the output stays within
 *     2e-3 of the fp64 oracle relative to its largest entry.
 *   - Calls that overlap on the same cache buffers race; calls on disjoint
 *     buffers may run concurrently on different streams.
 */
#ifndef STARKV_H
#define STARKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define STARKV_API __attribute__((visibility("default")))
#else
#define STARKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STARKV_OK = 0,
  STARKV_EINVAL = -1,       /* bad pointer, size, range or enum value */
  STARKV_EUNSUPPORTED = -2, /* valid shape the library has no kernel for */
  STARKV_ECAPACITY = -3,    /* tokens past max_tokens */
  STARKV_EWORKSPACE = -4,   /* workspace missing or too small */
  STARKV_ELAUNCH = -5       /* a HIP launch or query failed */
} starkv_status;

typedef enum {
  STARKV_CACHE_F32 = 0,  /* fp32 latents, no quantization */
  STARKV_CACHE_BF16 = 1, /* bf16 latents (round to nearest even) */
  STARKV_CACHE_Q43 = 2   /* 4-bit leading quarter, 3-bit rest, groups of at
                            most 32 channels, fp16 scale and zero per group */
} starkv_cache_dtype;

/* (host) Shape of one attention layer and its cache.
 *
 * The quantized cache (STARKV_CACHE_Q43) follows section 6.1 of the review:
 * the retained latent channels split into a leading (outlier) block and a
 * trailing (inlier) block, each optionally Walsh-Hadamard rotated on its own
 * (eq. 13) and stored at its own precision (eq. 14), with an asymmetric
 * fp16 scale and zero per group of at most group_size consecutive channels
 * of one token inside one block.  The five layout fields below state that
 * split explicitly; the library has kernels for hi_bits = 4, lo_bits = 3,
 * group_size = 32, key_hi_channels = key_rank / 4 and value_hi_channels =
 * value_rank / 4 (the model card's top_fraction = 0.25 recipe, 3.25 bits per
 * channel on average), and for the same fields with lo_bits = 4 (a uniform
 * 4-bit cache: the 4-bit cache of the review's speed figures, section 6.1
 * after eq. 14), and returns STARKV_EUNSUPPORTED for any other combination
 * (a 20:80 split
 * among them).  For F32 / BF16 caches the five fields must be 0. */
typedef struct starkv_config {
  int32_t batch;       /* B */
  int32_t n_q_heads;   /* Hq <= 32, a multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv; Hq / Hkv in {1, 2, 4, 8}; for Q43, Hkv in
                          {1, 2, 4, 8, 16, 32} with a decode kernel for the
                          (Hq / Hkv, Hkv) pair (starkv_decode_splits returns
                          0 when there is none) */
  int32_t head_dim;    /* d_h, a multiple of 16, <= 256 */
  int32_t key_rank;    /* r_k per KV head: <= 64 and a multiple of 8 for
                          F32/BF16; exactly 32 for Q43 */
  int32_t value_rank;  /* R_v, joint over n_kv_heads*head_dim value dims:
                          a multiple of 32, <= 1024 (Q43: multiple of 256) */
  int32_t max_tokens;  /* cache capacity T_max, a multiple of 64 */
  int32_t cache_dtype; /* starkv_cache_dtype */
  int32_t hi_bits;     /* Q43: bits of the leading block (4) */
  int32_t lo_bits;     /* Q43: bits of the trailing block (3, or 4 for a
                          uniform 4-bit cache) */
  int32_t group_size;  /* Q43: channels per quantization group (32) */
  int32_t key_hi_channels;   /* Q43: leading key channels per head at
                                hi_bits (key_rank / 4) */
  int32_t value_hi_channels; /* Q43: leading value channels at hi_bits
                                (value_rank / 4) */
  int32_t rotate;      /* Q43 only: 1 = latents are block-Hadamard rotated
                          by starkv_append before quantization (eq. 13); the
                          factors passed to decode/prefill stay unrotated */
  int32_t num_splits;  /* decode token splits per sequence; 0 = automatic */
  float rope_theta;    /* 0: no rotary position embedding.  > 0: RoPE base
                          (section 5.3 and Algorithm 2 step 4c: keys stay
                          pre-RoPE latents, reconstructed and rotated inside
                          the scoring); see starkv_decode and
                          starkv_prefill */
  const int32_t* key_ranks; /* (host) NULL: every KV head has key_rank
                          channels.  Otherwise n_kv_heads per-head ranks
                          (section 4 / Fig. 2: learned per-head ranks; eq. 15
                          sums them), each a multiple of 8 and <= key_rank.
                          F32/BF16: the key cache stores head g with
                          key_ranks[g] channels.  Q43: every head keeps its
                          32-channel key tile, the channels past its rank
                          zero (section 6.2: rank rounding to a supported
                          kernel tile, eq. 15's padding term).  Either way
                          z_key rows stay key_rank wide and B_key stays
                          [Hkv][d_h][key_rank]; entries past a head's rank
                          are ignored */
} starkv_config;

/* Device buffers of one layer's cache.  Byte layout ("format v1", tiles of
 * 64 tokens):
 *   F32/BF16: key [B][Hkv][T_max/64][r_k/8][64 tokens][8 channels],
 *             value [B][T_max/64][R_v/32][8 token blocks][32 channels]
 *             [8 tokens] (token u of a tile, channel 32g + m: group g,
 *             block u/8, [m][u%8]); key_meta and value_meta are unused
 *             (may be NULL).
 *   Q43:      key  [B][T_max/64][Hkv] blocks of 832 B (4-bit plane u32[64],
 *             3-bit planes u32[64], u32[64], u8[64], token-major);
 *             key_meta [B][T_max/64][Hkv][64][4] fp16 (scale_hi, zero_hi,
 *             scale_lo, zero_lo);
 *             value [B][T_max/64] blocks of 26*R_v B (per 32-channel group,
 *             channel-major runs of 32 tokens, 4-bit groups first);
 *             value_meta [B][T_max/64][2][R_v/32][64] fp16 (scales, zeros).
 *   Q43 with lo_bits = 4 (uniform 4-bit): key blocks of 1024 B (four 4-bit
 *             planes u32[64], plane p holding channels 8p .. 8p+7 of each
 *             token at bits 4c, the layout of the 4/3-bit cache's 4-bit
 *             plane); value blocks of 32*R_v B (every group in the 4-bit
 *             run layout); metadata as above.
 * Sizes are returned by starkv_cache_bytes. */
typedef struct starkv_cache {
  void* key;
  void* key_meta;
  void* value;
  void* value_meta;
} starkv_cache;

/* Buffer ids for starkv_cache_bytes. */
enum { STARKV_BUF_KEY = 0, STARKV_BUF_KEY_META = 1, STARKV_BUF_VALUE = 2,
       STARKV_BUF_VALUE_META = 3 };
/* Operation ids for starkv_workspace_bytes. */
enum { STARKV_OP_DECODE = 0, STARKV_OP_PREFILL = 1 };

/* (host) Bytes of one cache buffer for `cfg`; 0 if cfg is invalid or the
 * buffer is unused.  The quantized payload equals eq. 15 of the review
 * (B T b_bar / 8 (Hkv r_k + R_v) with b_bar = 3.25, or 4 for a uniform 4-bit
 * cache) with no padding term; the
 * metadata is 4 bytes per (token, group). */
STARKV_API size_t starkv_cache_bytes(const starkv_config* cfg, int32_t buffer);

/* (host) Workspace bytes needed by starkv_decode (op STARKV_OP_DECODE,
 * n_tokens = largest seq_len that will be passed) or starkv_prefill (op
 * STARKV_OP_PREFILL, n_tokens = chunk length).  0 on invalid arguments or
 * for a configuration the operation has no kernel for. */
STARKV_API size_t starkv_workspace_bytes(const starkv_config* cfg, int32_t op,
                              int32_t n_tokens);

/* (host) Number of token splits starkv_decode uses for seq_len tokens. */
STARKV_API int32_t starkv_decode_splits(const starkv_config* cfg, int32_t seq_len);

/* Latent append (review Algorithm 2, step 3: quantize and append).
 * Stores tokens [pos, pos+n) of every sequence:
 *   z_key   fp32 [B][n][Hkv][r_k]  key latents (unrotated if cfg->rotate)
 *   z_value fp32 [B][n][R_v]       joint value latents
 * F32 copies; BF16 rounds to nearest even; Q43 optionally applies the
 * block-Hadamard rotation (fp32 fast transform, butterfly strides 1, 2, 4,
 * ..., then a multiply by the fp32 value nearest 1/sqrt(m)), then quantizes
 * each (token, group): zero = fp16(min) rounded down, scale =
 * fp16((max - zero) / (2^bits - 1)) rounded up, code = clamp(rint((x - zero)
 * / scale)) -- all in IEEE fp32, bit-reproducible.  Only the bits and
 * metadata of the appended tokens change.
 * Errors: EINVAL (null pointer, n < 0, pos < 0), ECAPACITY (pos + n >
 * max_tokens), EUNSUPPORTED. n == 0 is a no-op returning STARKV_OK. */
STARKV_API int starkv_append(const starkv_config* cfg, const starkv_cache* cache,
                  const float* z_key, const float* z_value, int32_t pos,
                  int32_t n, hipStream_t stream);

/* Decode attention (review Algorithm 2, steps 4-7; section 5.3, eq. 12):
 *   q       [B][Hq][d_h]          bf16 (fp32 for an F32 cache)
 *   B_key   [Hkv][d_h][r_k]       bf16 (fp32 for an F32 cache), unrotated
 *   B_value [Hkv*d_h][R_v]        bf16 (fp32 for an F32 cache), unrotated
 *   out     [B][Hq][d_h]          fp32
 * out[b,h] = softmax_t(sm_scale * q[b,h] . K_g(h)[t]) V_g(h) over the first
 * seq_len cached tokens, computed in latent space: q is projected into the
 * key latent, scores and an online softmax run over token splits, the joint
 * value contraction P Z_v runs on MFMA, the splits are merged with the
 * attention decomposition theorem and the result is up-projected by
 * B_value's head block.  Workspace: starkv_workspace_bytes(cfg, DECODE,
 * seq_len) bytes.
 * Errors: EINVAL (null pointer, seq_len < 1), ECAPACITY (seq_len >
 * max_tokens), EWORKSPACE, EUNSUPPORTED, ELAUNCH. */
STARKV_API int starkv_decode(const starkv_config* cfg, const starkv_cache* cache,
                  int32_t seq_len, const void* q, const void* B_key,
                  const void* B_value, float sm_scale, float* out,
                  void* workspace, size_t ws_bytes, hipStream_t stream);

/* One decode step (review Algorithm 2, steps 3-7): append tokens [pos,
 * pos + n) of every sequence, then decode over seq_len = pos + n tokens --
 * exactly starkv_append followed by starkv_decode (same bytes, same output),
 * but the append and the query projection share one launch (they are
 * independent; every cache kind except rotary keys), which saves launches
 * and overlaps their memory latencies.  Arguments as in those two calls;
 * n == 0 decodes only.
 * Workspace: starkv_workspace_bytes(cfg, DECODE, pos + n).
 * Errors: EINVAL (pos < 0, n < 0, null or misaligned pointer), ECAPACITY
 * (pos + n > max_tokens), EWORKSPACE, EUNSUPPORTED, ELAUNCH. */
STARKV_API int starkv_decode_step(const starkv_config* cfg,
                                  const starkv_cache* cache, const float* z_key,
                                  const float* z_value, int32_t pos, int32_t n,
                                  const void* q, const void* B_key,
                                  const void* B_value, float sm_scale,
                                  float* out, void* workspace, size_t ws_bytes,
                                  hipStream_t stream);

/* starkv_decode_step that also records events[0..4] on `stream`: before the
 * append (and query projection), before the split kernel, before the merge,
 * before the up-projection and after it (as starkv_decode_profiled). */
STARKV_API int starkv_decode_step_profiled(
    const starkv_config* cfg, const starkv_cache* cache, const float* z_key,
    const float* z_value, int32_t pos, int32_t n, const void* q,
    const void* B_key, const void* B_value, float sm_scale, float* out,
    void* workspace, size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/* starkv_decode that also records events[0..4] (host array of created
 * hipEvent_t) on `stream`: before the query projection, before the split
 * kernel, before the merge, before the value up-projection and after it, so
 * a caller can time each kernel on the stream it runs on.  Where the merge
 * and the up-projection run as one kernel (fp16 partials, R_v <= 256,
 * d_h <= 128, at most 64 splits), events[3] and events[4] are both recorded
 * after it.  With rotary keys (rope_theta > 0) events[0] is recorded right
 * before the rotary score kernel instead (after the position table and the
 * query coefficients), so events[0..1] time that kernel alone.  Same
 * arguments, results and errors as starkv_decode; EINVAL if events is NULL. */
STARKV_API int starkv_decode_profiled(const starkv_config* cfg,
                                      const starkv_cache* cache,
                                      int32_t seq_len, const void* q,
                                      const void* B_key, const void* B_value,
                                      float sm_scale, float* out,
                                      void* workspace, size_t ws_bytes,
                                      hipStream_t stream, hipEvent_t* events);

/* ---- paged and ragged 4/3-bit caches (vLLM-style KV blocks) -----------
 * The cache buffers are a pool of B * (max_tokens / 64) pages, each holding
 * one 64-token tile of every KV head (the tile layout of the Q43 format
 * above: key [page][Hkv][832 B], key_meta [page][Hkv][64][4], value
 * [page][26 R_v B], value_meta [page][2][R_v/32][64]); starkv_cache_bytes
 * gives their sizes.  page_table (device, int32 [B][pages_per_seq]) maps tile
 * t of sequence b to its page; the contiguous cache is the table
 * page(b, t) = b * (max_tokens / 64) + t.  Table entries are clamped into the
 * pool on the device (a bad entry reads or writes a wrong page, never outside
 * the buffers).  Q43 caches only; EUNSUPPORTED otherwise. */

/* Append one token per sequence, each at its own position positions[b]
 * (device int32 [B], clamped on the device to [0, pages_per_seq * 64)):
 *   z_key fp32 [B][Hkv][r_k], z_value fp32 [B][R_v]; quantized, rotated and
 *   packed exactly as starkv_append does.
 * Errors: EINVAL (null / misaligned pointer, pages_per_seq < 1), EUNSUPPORTED,
 * ELAUNCH. */
STARKV_API int starkv_append_paged(const starkv_config* cfg,
                                   const starkv_cache* cache,
                                   const int32_t* page_table,
                                   int32_t pages_per_seq,
                                   const int32_t* positions, const float* z_key,
                                   const float* z_value, hipStream_t stream);

/* starkv_decode over a paged pool with ragged lengths: sequence b attends to
 * its first seq_lens[b] tokens (device int32 [B], clamped on the device to
 * [0, max_seq_len]; a length of 0 gives an all-zero output row).  The splits
 * are laid out for max_seq_len (host), which must be <= max_tokens and
 * <= pages_per_seq * 64.  With rotary keys the query of sequence b sits at
 * position seq_lens[b] - 1.  Workspace: starkv_workspace_bytes(cfg, DECODE,
 * max_seq_len).  Other arguments, results and errors as starkv_decode. */
STARKV_API int starkv_decode_paged(const starkv_config* cfg,
                                   const starkv_cache* cache,
                                   const int32_t* page_table,
                                   int32_t pages_per_seq,
                                   const int32_t* seq_lens, int32_t max_seq_len,
                                   const void* q, const void* B_key,
                                   const void* B_value, float sm_scale,
                                   float* out, void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* starkv_prefill over a paged pool (same page layout as starkv_append_paged):
 * every sequence b has the same ctx_len and chunk, and its tile t lives in
 * pool page page_table[b * pages_per_seq + t] (device int32, clamped on the
 * device into the pool).  The chunk's latents are appended at [ctx_len,
 * ctx_len + chunk) of each sequence's pages, then attended to as in
 * starkv_prefill.  pages_per_seq * 64 must cover ctx_len + chunk.
 * Workspace: starkv_workspace_bytes(cfg, PREFILL, chunk).  Other arguments,
 * results and errors as starkv_prefill; EINVAL also for a null or
 * misaligned page table or too few pages per sequence. */
STARKV_API int starkv_prefill_paged(const starkv_config* cfg,
                                    const starkv_cache* cache,
                                    const int32_t* page_table,
                                    int32_t pages_per_seq, int32_t ctx_len,
                                    int32_t chunk, const void* x, int32_t hidden,
                                    const void* A_key, const void* A_value,
                                    const void* q, const void* B_key,
                                    const void* B_value, float sm_scale,
                                    float* out, float* z_debug, void* workspace,
                                    size_t ws_bytes, hipStream_t stream);

/* ---- value/output factor fusion and the head sum (review section 5.3,
 * eq. 12 read right to left; Algorithm 2, steps 7-8) ---------------------
 * eq. 12: p_h (Z_V U_h^T) O_h = (p_h Z_V)(U_h^T O_h).  The right-hand factor
 * F_h = B_value[g(h)]^T O_h (R_v x hidden per query head, O_h = rows h*d_h
 * .. h*d_h + d_h - 1 of the output projection W_o [Hq*d_h][hidden], row-vector
 * convention y = o W_o) is prepared once; decode then ends in the hidden
 * size: y[b] = sum_h obar[b, h] F_h, obar[b, h] = softmax_t(scores) Z_v the
 * per-head attention row in the (unrotated) value latent.
 * Shapes: BF16 or Q43 caches (bf16 factors), hidden a multiple of 128;
 * EUNSUPPORTED otherwise.  F's layout is opaque to callers: it is written by
 * starkv_fuse_value_output and read by starkv_decode_hidden only (bf16,
 * [hidden/16][Hq*R_v/8][16][8]). */

/* (host) Bytes of the fused factor F for `hidden`; 0 if unsupported. */
STARKV_API size_t starkv_fused_factor_bytes(const starkv_config* cfg,
                                            int32_t hidden);

/* F_h = B_value[g(h)]^T O_h for every query head, fp32 accumulation of bf16
 * products, rounded to bf16 (nearest even).  B_value [Hkv*d_h][R_v] bf16
 * (unrotated, as in starkv_decode), W_o [Hq*d_h][hidden] bf16, F device
 * buffer of starkv_fused_factor_bytes(cfg, hidden) bytes.
 * Errors: EINVAL (null / misaligned pointer, hidden < 1), EUNSUPPORTED,
 * ELAUNCH. */
STARKV_API int starkv_fuse_value_output(const starkv_config* cfg,
                                        const void* B_value, const void* W_o,
                                        int32_t hidden, void* F,
                                        hipStream_t stream);

/* (host) Workspace bytes of starkv_decode_hidden; 0 if unsupported. */
STARKV_API size_t starkv_decode_hidden_workspace_bytes(const starkv_config* cfg,
                                                       int32_t seq_len,
                                                       int32_t hidden);

/* Decode that ends in the hidden size: the query projection, split scores
 * and online softmax, P Z_v on MFMA and the split merge of starkv_decode,
 * then y = obar_flat [B][Hq*R_v] x F [Hq*R_v][hidden] (the per-head value
 * factors and the sum over heads as one GEMM; obar fp32 split into bf16 high
 * and low parts, fp32 accumulation, K slices summed in a fixed order).
 *   q, B_key as in starkv_decode; F from starkv_fuse_value_output;
 *   y fp32 [B][hidden].
 * Errors: as starkv_decode; EUNSUPPORTED for the shapes above. */
STARKV_API int starkv_decode_hidden(const starkv_config* cfg,
                                    const starkv_cache* cache, int32_t seq_len,
                                    const void* q, const void* B_key,
                                    const void* F, int32_t hidden,
                                    float sm_scale, float* y, void* workspace,
                                    size_t ws_bytes, hipStream_t stream);

/* starkv_decode_hidden that also records events[0..5] (host array of
 * created hipEvent_t) on `stream`: before the query projection, before the
 * split kernel, before the merge, before the hidden GEMM, before the K-slice
 * reduction and after it.  Same arguments, results and errors; EINVAL if
 * events is NULL. */
STARKV_API int starkv_decode_hidden_profiled(
    const starkv_config* cfg, const starkv_cache* cache, int32_t seq_len,
    const void* q, const void* B_key, const void* F, int32_t hidden,
    float sm_scale, float* y, void* workspace, size_t ws_bytes,
    hipStream_t stream, hipEvent_t* events);

/* For callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * starkv_decode -- same arguments except the workspace, same kernels, same
 * results and errors -- but the workspace is a fixed array of the library,
 * starkv_noalloc_scratch_bytes() = 64 MiB per device, held from the first
 * call on a device until the process ends.  The call allocates nothing.
 * Its first call on a device asks the runtime for that device's array
 * address (a HIP call, done once per device).  Every call on one device
 * shares its array: calls that overlap on one device (different streams, or
 * different threads) race and give undefined results; calls on one stream
 * are ordered.  Nothing in the array needs to start at zero: each call
 * writes everything it reads.
 * Errors: as starkv_decode; STARKV_EWORKSPACE when the shape needs more than
 * starkv_noalloc_scratch_bytes() (starkv_workspace_bytes(cfg, DECODE,
 * seq_len) tells), checked on the host before any HIP call. */
STARKV_API int starkv_decode_noalloc(const starkv_config* cfg,
                                     const starkv_cache* cache,
                                     int32_t seq_len, const void* q,
                                     const void* B_key, const void* B_value,
                                     float sm_scale, float* out,
                                     hipStream_t stream);

/* (host) Size of the fixed scratch array starkv_decode_noalloc uses. */
STARKV_API size_t starkv_noalloc_scratch_bytes(void);

/* Chunked causal prefill of one chunk (review Algorithm 2, steps 1-3, then
 * causal attention over the stored cache):
 *   x       bf16 [B][C][D]          hidden states of the chunk
 *   A_key   bf16 [D][Hkv*r_k]       key down-projection (unrotated)
 *   A_value bf16 [D][R_v]           value down-projection (unrotated)
 *   q       bf16 [B][C][Hq][d_h]    queries of the chunk
 *   B_key, B_value as in starkv_decode
 *   out     fp32 [B][C][Hq][d_h]
 *   z_debug fp32 [B][C][Hkv*r_k + R_v] or NULL: the projected latents
 * Projects Z = x A, appends it at [ctx_len, ctx_len + C) exactly as
 * starkv_append would, then query i (absolute position ctx_len + i) attends
 * to cached positions 0 .. ctx_len + i.  With rope_theta > 0 (review
 * section 5.3, Algorithm 2 steps 4b-4c) the keys of every visible position
 * are reconstructed from the stored latents (k = B_key[g] z) and rotated at
 * their positions, query i is rotated at ctx_len + i, and the scores run
 * over d_h channels; the values are not rotated.  The values enter in one
 * of eq. 12's two orders, chosen from the shape alone: when
 * C * Hq * (R_v - d_h) > Hkv * d_h * R_v and d_h is 64 or 128, the values of
 * every visible position are reconstructed once per call (Z_v B_value^T per
 * KV head, fp16) and the attention contracts over d_h, writing out
 * directly; otherwise it contracts the probabilities with the joint value
 * latent and up-projects (the decode order).  Workspace:
 * starkv_workspace_bytes(cfg, PREFILL, C) (with rotary keys it holds fp16
 * keys of d_h channels for every position, B * max_tokens * Hkv * d_h * 2
 * bytes, instead of the 32-channel latents; with reconstructed values, the
 * fp16 values B * max_tokens * Hkv * d_h * 2 bytes and the fp16 value
 * latents B * max_tokens * R_v * 2 bytes instead of the fp32 partial rows
 * B * C * Hq * R_v * 4 bytes).  Because the two orders need different
 * buffers, the size is not monotone in C: query it for every chunk length
 * a caller uses (or take the largest over them).
 * Errors: EINVAL, ECAPACITY (ctx_len + C > max_tokens), EWORKSPACE,
 * ELAUNCH; EUNSUPPORTED unless the cache is Q43 with r_k = 32, Hq / Hkv in
 * {1, 2, 4, 8}, R_v a multiple of 256 up to 1024, D a multiple of 64, and
 * either (no rotary keys) Hq a multiple of 8 and d_h a multiple of 64 up to
 * 256, or (rotary keys) d_h = 128 with Hq even or d_h = 64 with Hq a
 * multiple of 4. */
STARKV_API int starkv_prefill(const starkv_config* cfg, const starkv_cache* cache,
                   int32_t ctx_len, int32_t chunk, const void* x,
                   int32_t hidden, const void* A_key, const void* A_value,
                   const void* q, const void* B_key, const void* B_value,
                   float sm_scale, float* out, float* z_debug,
                   void* workspace, size_t ws_bytes, hipStream_t stream);

/* starkv_prefill that also records events[0..5] (host array of created
 * hipEvent_t) on `stream`: before the latent projection, before the append,
 * before the query projection, before the causal attention kernel, before
 * the normalisation + value up-projection and after it.  Same arguments,
 * results and errors as starkv_prefill; EINVAL if events is NULL. */
STARKV_API int starkv_prefill_profiled(const starkv_config* cfg,
                                       const starkv_cache* cache,
                                       int32_t ctx_len, int32_t chunk,
                                       const void* x, int32_t hidden,
                                       const void* A_key, const void* A_value,
                                       const void* q, const void* B_key,
                                       const void* B_value, float sm_scale,
                                       float* out, float* z_debug,
                                       void* workspace, size_t ws_bytes,
                                       hipStream_t stream, hipEvent_t* events);

/* Measurement helper, not a step of the method: reads `bytes` bytes of the
 * device buffer `src` once with non-temporal 16-byte loads, the way the
 * decode split kernel streams the cache, so that the split kernel's
 * bandwidth can be set against the measured streaming-read ceiling.
 * `sink` (device, one uint32) is written only in the rare case that the
 * XOR of a thread's data equals a fixed value; its content is meaningless.
 * src 16-byte aligned, sink 4-byte aligned, bytes a non-zero multiple of
 * 16; EINVAL otherwise, ELAUNCH if the launch fails (also when bytes / 16
 * needs more than 2^31 - 1 workgroups of 512).  Async on `stream`. */
STARKV_API int starkv_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                  hipStream_t stream);

/* (host) Static description of a status code. */
STARKV_API const char* starkv_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* STARKV_H */
