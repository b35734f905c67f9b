// Internal declarations shared by the HIP translation units of libstarkv.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/starkv.h"

namespace starkv {

constexpr int kTile = 64;          // tokens per cache tile (format v1)
// Bytes of one quantized key tile of one KV head: 4/3-bit (832: a 4-bit
// plane, two 3-bit planes and a remainder byte per token) or uniform 4-bit
// (1024: four 4-bit planes), and of one value tile (26 or 32 bytes per
// latent channel).
__host__ __device__ constexpr int key_block_bytes(int lo_bits) { return lo_bits == 4 ? 1024 : 832; }
__host__ __device__ constexpr int value_tile_bytes(int rv, int lo_bits) {
  return (lo_bits == 4 ? 32 : 26) * rv;
}
constexpr int kMaxQHeads = 32;     // rows of the stacked-head P operand
constexpr int kDecodeWaves = 8;    // waves per decode workgroup
constexpr int kMaxSplits = 1024;   // decode token splits per sequence
constexpr int kComputeUnits = 256;  // MI355X compute units (split-count sizing)

// Shape of one call, copied by value into every kernel.
struct Dims {
  int B, Hq, Hkv, G, dh, rk, rv, Tmax, NT, dtype, rotate;
  int lob;           // quantized caches: bits of the trailing block (3 or 4)
  float rope_theta;  // 0: no rotary position embedding
  // Paged / ragged 4/3-bit caches (all null / 0 for the contiguous layout):
  const int32_t* pages = nullptr;  // device [B][pages_per_seq]: tile -> pool page
  int pages_per_seq = 0;
  const int32_t* lens = nullptr;   // device [B]: tokens of each sequence (decode)
  const int32_t* positions = nullptr;  // device [B]: append position of each sequence
  // Key rank of each KV head and the channel offset of its key region
  // (per-head ranks; for uniform ranks krank[g] = rk, kpre[g] = g * rk);
  // kpre[Hkv] = sum of the ranks.
  uint8_t krank[kMaxQHeads];
  uint16_t kpre[kMaxQHeads + 1];
};

// Element offset, in an unquantized key buffer, of the 8-channel chunk c of
// token u of tile `tile` of KV head g of sequence b.  Layout: per sequence,
// the KV heads' regions one after the other, head g's region
// [NT][r_g/8][64 tokens][8 channels] (with uniform ranks this is
// [B][Hkv][NT][r_k/8][64][8]).
__host__ __device__ inline size_t plain_key_offset(const Dims& d, int b, int g, int tile,
                                                   int c, int u) {
  return (size_t)d.NT * kTile * ((size_t)b * d.kpre[d.Hkv] + d.kpre[g]) +
         ((size_t)tile * (d.krank[g] / 8) + c) * (kTile * 8) + (size_t)u * 8;
}

// Index of the 64-token tile `tile` of sequence b in the cache buffers: the
// contiguous layout b * NT + tile, or the page the table maps it to (clamped
// into the pool of B * NT pages, so a bad table entry selects a wrong page but
// never an address outside the buffers).
__host__ __device__ inline size_t tile_index(const Dims& d, int b, int tile) {
  if (!d.pages) return (size_t)b * d.NT + tile;
  const int t = tile < 0 ? 0 : (tile < d.pages_per_seq ? tile : d.pages_per_seq - 1);
  int p = d.pages[(size_t)b * d.pages_per_seq + t];
  const int n_pages = d.B * d.NT;
  p = p < 0 ? 0 : (p >= n_pages ? n_pages - 1 : p);
  return (size_t)p;
}
// Tokens of sequence b: its own length (ragged batches, clamped to
// [0, max_len]) or the call's common length.
__host__ __device__ inline int seq_len_of(const Dims& d, int b, int max_len) {
  if (!d.lens) return max_len;
  const int n = d.lens[b];
  return n < 0 ? 0 : (n > max_len ? max_len : n);
}

inline Dims make_dims(const starkv_config& c) {
  Dims d;
  d.B = c.batch;
  d.Hq = c.n_q_heads;
  d.Hkv = c.n_kv_heads;
  d.G = c.n_q_heads / c.n_kv_heads;
  d.dh = c.head_dim;
  d.rk = c.key_rank;
  d.rv = c.value_rank;
  d.Tmax = c.max_tokens;
  d.NT = c.max_tokens / kTile;
  d.dtype = c.cache_dtype;
  d.rotate = c.rotate;
  d.lob = c.cache_dtype == STARKV_CACHE_Q43 ? c.lo_bits : 0;
  d.rope_theta = c.rope_theta;
  int off = 0;
  for (int g = 0; g < kMaxQHeads; ++g) {
    const int r = g < c.n_kv_heads ? (c.key_ranks ? c.key_ranks[g] : c.key_rank) : 0;
    d.krank[g] = (uint8_t)r;
    d.kpre[g] = (uint16_t)off;
    off += r;
  }
  d.kpre[kMaxQHeads] = (uint16_t)off;
  if (c.n_kv_heads < kMaxQHeads) d.kpre[c.n_kv_heads] = (uint16_t)off;
  return d;
}

// Workspace of the rotary-key scores (offsets from DecodeWs::rope_off).
struct RopeWs {
  size_t mrec, trig, s_rel, m_tile, m_split, total;
};
// Workspace carve-up of one decode call (byte offsets, 256-aligned).
struct DecodeWs {
  size_t qt, part_o, part_ml, obar, rope_off, total;
  RopeWs rope;
  int splits;
};
DecodeWs decode_ws_layout(const Dims& d, int splits, int seq_len);
// Decode split workgroups that stay resident on one compute unit together
// (1 when it cannot be asked, e.g. without a device).
int decode_groups_per_cu(const Dims& d);
int choose_splits(const starkv_config& c, int seq_len);
// Host validation of a decode call short of the workspace (api.cpp): status,
// and on success the workspace layout the call needs.
int validate_decode(const starkv_config* cfg, const starkv_cache* cache,
                    int32_t seq_len, const void* q, const void* B_key,
                    const void* B_value, const float* out, DecodeWs* lay);

// Launchers; each returns hipSuccess or the launch error.
hipError_t launch_append(const Dims& d, const starkv_cache& cache,
                         const float* zk, const float* zv, int pos, int n,
                         hipStream_t s);
// Decode launches.  With `qproj_done` the query records are already in the
// workspace (written by launch_append_qproj) and the query projection is not
// launched again; with `first_mark_done` the caller has recorded events[0];
// with `latent_only` the call stops after the merge, leaving the merged,
// unrotated rows obar [B][Hq][R_v] fp32 at ws + lay.obar (no up-projection).
hipError_t launch_decode(const Dims& d, const starkv_cache& cache, int seq_len,
                         const void* q, const void* bk, const void* bv,
                         float sm_scale, float* out, char* ws,
                         const DecodeWs& lay, hipStream_t s,
                         hipEvent_t* events = nullptr, bool qproj_done = false,
                         bool first_mark_done = false, bool latent_only = false);
// Rotary-key scores (rope.hip).
struct RopeArgs {
  Dims d;
  int seq_len, splits, tiles_per_split;
  const void* key;
  const uint16_t* kmeta;
  const void* mrec;      // fp16 query coefficient fragments
  const void* trig;      // fp16 position trig fragments
  void* s_rel;           // fp16 [B][Hq][NT*64]
  float* m_tile;         // [B][Hq][NT]
  float* m_split;        // [B][splits][Hq]
};
bool rope_supported(const Dims& d);
size_t rope_ws_bytes(const Dims& d, int seq_len, int splits, RopeWs* w);
hipError_t launch_rope_scores(const Dims& d, const starkv_cache& cache, int seq_len,
                              const void* q, const void* bk, float sm_scale,
                              char* ws, const RopeWs& rw, int splits,
                              int tiles_per_split, hipStream_t s,
                              hipEvent_t before_scores = nullptr);
// Value/output factor fusion and the head sum (oproj.hip).
int hidden_k_slices(const Dims& d, int D);
hipError_t launch_fuse_vo(const Dims& d, const void* bv, const void* w_o, int D,
                          void* F, hipStream_t s);
// events (optional): [0] after the GEMM, [1] after the K-slice reduction.
hipError_t launch_hidden(const Dims& d, const float* obar, const void* F, int D,
                         float* part_y, float* y, hipStream_t s,
                         hipEvent_t* events = nullptr);
// One launch for the append of tokens [pos, pos+n) of a 4/3-bit cache and the
// decode query projection into `qt` (the workspace's query records).
hipError_t launch_append_qproj(const Dims& d, const starkv_cache& cache,
                               const float* zk, const float* zv, int pos, int n,
                               const void* q, const void* bk, float qscale,
                               void* qt, hipStream_t s);
// The same for an unquantized (fp32 / bf16) cache.
hipError_t launch_append_qproj_plain(const Dims& d, const starkv_cache& cache,
                                     const float* zk, const float* zv, int pos, int n,
                                     const void* q, const void* bk, float qscale,
                                     void* qt, hipStream_t s);

// Workspace carve-up of one prefill call (byte offsets, 256-aligned).
struct PrefillWs {
  size_t zk, zv, qt, kd, part_o, part_ml, bvr, zvd, bvh, vt, total;
};
// Whether a prefill chunk reconstructs the values once per call (eq. 12 in
// its left-hand order) instead of contracting with the joint latent.
bool prefill_reconstructs(const Dims& d, int chunk);
PrefillWs prefill_ws_layout(const Dims& d, int chunk);
hipError_t launch_prefill(const Dims& d, const starkv_cache& cache,
                          int ctx_len, int chunk, const void* x, int hidden,
                          const void* ak, const void* av, const void* q,
                          const void* bk, const void* bv, float sm_scale,
                          float* out, float* z_debug, char* ws,
                          const PrefillWs& lay, hipStream_t s,
                          hipEvent_t* events = nullptr);
bool prefill_supported(const Dims& d);
// A decode split kernel exists for the shape (decode.hip).
bool decode_supported(const Dims& d);

// Streaming-read measurement pass (stream.hip).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);

// fp32 value nearest to 1/sqrt(m) for a Walsh-Hadamard block of m channels
// (m a power of two, 1 <= m <= kMaxRotBlock); 0 otherwise, which the host
// validation never lets through (a zero would show as an all-zero output,
// not as a plausible wrong one).
constexpr int kMaxRotBlock = 1024;
__host__ __device__ inline float inv_sqrt_pow2(int m) {
  switch (m) {
    case 1: return 1.0f;
    case 2: return __builtin_bit_cast(float, 0x3F3504F3u);
    case 4: return 0.5f;
    case 8: return __builtin_bit_cast(float, 0x3EB504F3u);
    case 16: return 0.25f;
    case 32: return __builtin_bit_cast(float, 0x3E3504F3u);
    case 64: return 0.125f;
    case 128: return __builtin_bit_cast(float, 0x3DB504F3u);
    case 256: return 0.0625f;
    case 512: return __builtin_bit_cast(float, 0x3D3504F3u);
    case 1024: return 0.03125f;
    default: return 0.0f;
  }
}

__host__ __device__ inline int pow2_divisor(int n) { return n & -n; }

}  // namespace starkv
