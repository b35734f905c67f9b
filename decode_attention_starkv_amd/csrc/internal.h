// Internal declarations shared by the HIP translation units of libstarkv.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/starkv.h"

namespace starkv {

constexpr int kTile = 64;          // tokens per cache tile (format v1)
constexpr int kKeyBlock = 832;     // bytes of one Q43 key tile of one KV head
constexpr int kMaxQHeads = 32;     // rows of the stacked-head P operand
constexpr int kDecodeWaves = 8;    // waves per decode workgroup
constexpr int kMaxSplits = 1024;   // decode token splits per sequence

// Shape of one call, copied by value into every kernel.
struct Dims {
  int B, Hq, Hkv, G, dh, rk, rv, Tmax, NT, dtype, rotate;
};

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
  return d;
}

// Workspace carve-up of one decode call (byte offsets, 256-aligned).
struct DecodeWs {
  size_t qt, part_o, part_ml, obar, total;
  int splits;
};
DecodeWs decode_ws_layout(const Dims& d, int splits);
// Decode split workgroups that stay resident on one compute unit together
// (1 when it cannot be asked, e.g. without a device).
int decode_groups_per_cu(const Dims& d);
int choose_splits(const starkv_config& c, int seq_len);

// Launchers; each returns hipSuccess or the launch error.
hipError_t launch_append(const Dims& d, const starkv_cache& cache,
                         const float* zk, const float* zv, int pos, int n,
                         hipStream_t s);
hipError_t launch_decode(const Dims& d, const starkv_cache& cache, int seq_len,
                         const void* q, const void* bk, const void* bv,
                         float sm_scale, float* out, char* ws,
                         const DecodeWs& lay, hipStream_t s,
                         hipEvent_t* events = nullptr);

// Workspace carve-up of one prefill call (byte offsets, 256-aligned).
struct PrefillWs {
  size_t zk, zv, qt, kd, part_o, part_ml, bvr, total;
};
PrefillWs prefill_ws_layout(const Dims& d, int chunk);
hipError_t launch_prefill(const Dims& d, const starkv_cache& cache,
                          int ctx_len, int chunk, const void* x, int hidden,
                          const void* ak, const void* av, const void* q,
                          const void* bk, const void* bv, float sm_scale,
                          float* out, float* z_debug, char* ws,
                          const PrefillWs& lay, hipStream_t s,
                          hipEvent_t* events = nullptr);
bool prefill_supported(const Dims& d);

// Streaming-read measurement pass (stream.hip).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);

// fp32 value nearest to 1/sqrt(m) for the Walsh-Hadamard block sizes used.
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
    default: return 0.0625f;  // 256
  }
}

__host__ __device__ inline int pow2_divisor(int n) { return n & -n; }

}  // namespace starkv
