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
 *     workspace).  The library keeps no state between calls and allocates
 *     nothing.
 *   - Compute calls are asynchronous on `stream` and never synchronize.
 *   - Arguments are validated on the host before any HIP call; a failed
 *     validation returns a negative status and touches no memory.  A kernel
 *     launch failure returns STARKV_ELAUNCH.  No C++ exception crosses the ABI.
 *   - Inputs must be finite and latents must lie within the fp16 range for the
 *     quantized cache; otherwise results are unspecified.
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
  STARKV_EUNSUPPORTED = -2, /* valid shape this build has no kernel for */
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

/* (host) Shape of one attention layer and its cache. */
typedef struct starkv_config {
  int32_t batch;       /* B */
  int32_t n_q_heads;   /* Hq <= 32, a multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv; Hq / Hkv in {1, 2, 4, 8}; Q43 with Hkv > 4
                          needs Hkv a multiple of 4 */
  int32_t head_dim;    /* d_h, a multiple of 16, <= 256 */
  int32_t key_rank;    /* r_k per KV head: <= 64 and a multiple of 8 for
                          F32/BF16; exactly 32 for Q43 */
  int32_t value_rank;  /* R_v, joint over n_kv_heads*head_dim value dims:
                          a multiple of 32, <= 1024 (Q43: multiple of 256) */
  int32_t max_tokens;  /* cache capacity T_max, a multiple of 64 */
  int32_t cache_dtype; /* starkv_cache_dtype */
  int32_t rotate;      /* Q43 only: 1 = latents are block-Hadamard rotated
                          by starkv_append before quantization (eq. 13); the
                          factors passed to decode/prefill stay unrotated */
  int32_t num_splits;  /* decode token splits per sequence; 0 = automatic */
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
 * (B T b_bar / 8 (Hkv r_k + R_v) with b_bar = 3.25) with no padding term; the
 * metadata is 4 bytes per (token, group). */
STARKV_API size_t starkv_cache_bytes(const starkv_config* cfg, int32_t buffer);

/* (host) Workspace bytes needed by starkv_decode (op STARKV_OP_DECODE,
 * n_tokens = largest seq_len that will be passed) or starkv_prefill (op
 * STARKV_OP_PREFILL, n_tokens = chunk length).  0 on invalid arguments. */
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

/* starkv_decode that also records events[0..4] (host array of created
 * hipEvent_t) on `stream`: before the query projection, before the split
 * kernel, before the merge, before the value up-projection and after it, so
 * a caller can time each kernel on the stream it runs on.  Where the merge
 * and the up-projection run as one kernel (fp16 partials, R_v <= 256,
 * d_h <= 128, at most 64 splits), events[3] and events[4] are both recorded
 * after it.  Same arguments, results and errors as starkv_decode; EINVAL if
 * events is NULL. */
STARKV_API int starkv_decode_profiled(const starkv_config* cfg,
                                      const starkv_cache* cache,
                                      int32_t seq_len, const void* q,
                                      const void* B_key, const void* B_value,
                                      float sm_scale, float* out,
                                      void* workspace, size_t ws_bytes,
                                      hipStream_t stream, hipEvent_t* events);

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
 * to cached positions 0 .. ctx_len + i.  Workspace:
 * starkv_workspace_bytes(cfg, PREFILL, C).
 * Errors: EINVAL, ECAPACITY (ctx_len + C > max_tokens), EWORKSPACE,
 * ELAUNCH; EUNSUPPORTED unless the cache is Q43 with r_k = 32, Hq a multiple
 * of 8, Hq / Hkv in {1, 2, 4, 8}, R_v a multiple of 256 up to 1024, d_h a
 * multiple of 64 up to 256 and D a multiple of 64. */
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
