// Host side of the C ABI: argument validation (before any HIP call), cache
// and workspace sizes, split selection and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <limits>

#include "internal.h"

namespace starkv {
namespace {

// Structural validity (EINVAL) and supported shapes (EUNSUPPORTED).
int check_config(const starkv_config* c) {
  if (!c) return STARKV_EINVAL;
  if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 1 || c->key_rank < 1 || c->value_rank < 1 ||
      c->max_tokens < kTile || c->max_tokens % kTile != 0 ||
      c->n_q_heads % c->n_kv_heads != 0 || c->num_splits < 0 ||
      c->cache_dtype < STARKV_CACHE_F32 || c->cache_dtype > STARKV_CACHE_Q43 ||
      (c->rotate != 0 && c->rotate != 1))
    return STARKV_EINVAL;
  const int g = c->n_q_heads / c->n_kv_heads;
  if (c->n_q_heads > kMaxQHeads || (g != 1 && g != 2 && g != 4 && g != 8))
    return STARKV_EUNSUPPORTED;
  if (c->head_dim % 16 != 0 || c->head_dim > 256) return STARKV_EUNSUPPORTED;
  if (c->value_rank % 32 != 0 || c->value_rank > 1024) return STARKV_EUNSUPPORTED;
  if (c->cache_dtype == STARKV_CACHE_Q43) {
    if (c->key_rank != 32 || c->value_rank % 256 != 0 ||
        (c->n_kv_heads > 4 && c->n_kv_heads % 4 != 0))
      return STARKV_EUNSUPPORTED;
  } else {
    if (c->rotate) return STARKV_EUNSUPPORTED;
    if (c->key_rank % 8 != 0 || c->key_rank > 64) return STARKV_EUNSUPPORTED;
  }
  return STARKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_cache(const starkv_config* c, const starkv_cache* cache) {
  if (!cache || !cache->key || !cache->value) return STARKV_EINVAL;
  if (!aligned16(cache->key) || !aligned16(cache->value)) return STARKV_EINVAL;
  if (c->cache_dtype == STARKV_CACHE_Q43 &&
      (!cache->key_meta || !cache->value_meta || !aligned16(cache->key_meta) ||
       !aligned16(cache->value_meta)))
    return STARKV_EINVAL;
  return STARKV_OK;
}

size_t cache_bytes(const starkv_config& c, int which) {
  const size_t B = c.batch, H = c.n_kv_heads, T = c.max_tokens, NT = T / kTile;
  const size_t rk = c.key_rank, rv = c.value_rank;
  if (c.cache_dtype == STARKV_CACHE_Q43) {
    switch (which) {
      case STARKV_BUF_KEY: return B * H * NT * kKeyBlock;
      case STARKV_BUF_KEY_META: return B * H * NT * kTile * 8;
      case STARKV_BUF_VALUE: return B * NT * rv * 26;
      case STARKV_BUF_VALUE_META: return B * NT * 2 * (rv / 32) * kTile * 2;
      default: return 0;
    }
  }
  const size_t es = c.cache_dtype == STARKV_CACHE_F32 ? 4 : 2;
  switch (which) {
    case STARKV_BUF_KEY: return B * H * T * rk * es;
    case STARKV_BUF_VALUE: return B * NT * rv * kTile * es;
    default: return 0;
  }
}

// MI355X has 256 compute units; the split count fills every unit with as
// many decode workgroups as stay resident on it.
constexpr int kComputeUnits = 256;

}  // namespace

int choose_splits(const starkv_config& c, int seq_len) {
  const int n_tiles = (seq_len + kTile - 1) / kTile;
  const int groups = kComputeUnits * decode_groups_per_cu(make_dims(c));
  int s = c.num_splits > 0 ? c.num_splits : (groups + c.batch - 1) / c.batch;
  s = std::max(1, std::min(std::min(s, n_tiles), kMaxSplits));
  const int tps = (n_tiles + s - 1) / s;
  return (n_tiles + tps - 1) / tps;  // no empty splits
}

}  // namespace starkv

using namespace starkv;

extern "C" {

size_t starkv_cache_bytes(const starkv_config* cfg, int32_t buffer) {
  if (check_config(cfg) != STARKV_OK) return 0;
  return cache_bytes(*cfg, buffer);
}

size_t starkv_workspace_bytes(const starkv_config* cfg, int32_t op,
                              int32_t n_tokens) {
  if (check_config(cfg) != STARKV_OK || n_tokens < 1) return 0;
  const Dims d = make_dims(*cfg);
  if (op == STARKV_OP_DECODE) {
    if (n_tokens > cfg->max_tokens) return 0;
    return decode_ws_layout(d, choose_splits(*cfg, n_tokens)).total;
  }
  if (op == STARKV_OP_PREFILL) return prefill_ws_layout(d, n_tokens).total;
  return 0;
}

int32_t starkv_decode_splits(const starkv_config* cfg, int32_t seq_len) {
  if (check_config(cfg) != STARKV_OK || seq_len < 1) return 0;
  return choose_splits(*cfg, seq_len);
}

int starkv_append(const starkv_config* cfg, const starkv_cache* cache,
                  const float* z_key, const float* z_value, int32_t pos,
                  int32_t n, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != STARKV_OK) return st;
  if ((st = check_cache(cfg, cache)) != STARKV_OK) return st;
  if (pos < 0 || n < 0) return STARKV_EINVAL;
  if ((int64_t)pos + n > cfg->max_tokens) return STARKV_ECAPACITY;
  if (n == 0) return STARKV_OK;
  if (!z_key || !z_value || !aligned16(z_key) || !aligned16(z_value))
    return STARKV_EINVAL;
  hipError_t e = launch_append(make_dims(*cfg), *cache, z_key, z_value, pos, n, stream);
  return e == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

static int decode_impl(const starkv_config* cfg, const starkv_cache* cache,
                       int32_t seq_len, const void* q, const void* B_key,
                       const void* B_value, float sm_scale, float* out,
                       void* workspace, size_t ws_bytes, hipStream_t stream,
                       hipEvent_t* events) {
  int st = check_config(cfg);
  if (st != STARKV_OK) return st;
  if ((st = check_cache(cfg, cache)) != STARKV_OK) return st;
  if (seq_len < 1) return STARKV_EINVAL;
  if (seq_len > cfg->max_tokens) return STARKV_ECAPACITY;
  if (!q || !B_key || !B_value || !out || !aligned16(q) || !aligned16(B_key) ||
      !aligned16(B_value) || !aligned16(out))
    return STARKV_EINVAL;
  const Dims d = make_dims(*cfg);
  const DecodeWs lay = decode_ws_layout(d, choose_splits(*cfg, seq_len));
  if (!workspace || !aligned16(workspace) || ws_bytes < lay.total)
    return STARKV_EWORKSPACE;
  hipError_t e = launch_decode(d, *cache, seq_len, q, B_key, B_value, sm_scale,
                               out, static_cast<char*>(workspace), lay, stream,
                               events);
  return e == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

int starkv_decode(const starkv_config* cfg, const starkv_cache* cache,
                  int32_t seq_len, const void* q, const void* B_key,
                  const void* B_value, float sm_scale, float* out,
                  void* workspace, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(cfg, cache, seq_len, q, B_key, B_value, sm_scale, out,
                     workspace, ws_bytes, stream, nullptr);
}

int starkv_decode_profiled(const starkv_config* cfg, const starkv_cache* cache,
                           int32_t seq_len, const void* q, const void* B_key,
                           const void* B_value, float sm_scale, float* out,
                           void* workspace, size_t ws_bytes,
                           hipStream_t stream, hipEvent_t* events) {
  if (!events) return STARKV_EINVAL;
  return decode_impl(cfg, cache, seq_len, q, B_key, B_value, sm_scale, out,
                     workspace, ws_bytes, stream, events);
}

static int prefill_impl(const starkv_config* cfg, const starkv_cache* cache,
                        int32_t ctx_len, int32_t chunk, const void* x,
                        int32_t hidden, const void* A_key, const void* A_value,
                        const void* q, const void* B_key, const void* B_value,
                        float sm_scale, float* out, float* z_debug, void* workspace,
                        size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  int st = check_config(cfg);
  if (st != STARKV_OK) return st;
  if ((st = check_cache(cfg, cache)) != STARKV_OK) return st;
  if (ctx_len < 0 || chunk < 1 || hidden < 1) return STARKV_EINVAL;
  if ((int64_t)ctx_len + chunk > cfg->max_tokens) return STARKV_ECAPACITY;
  if (!x || !A_key || !A_value || !q || !B_key || !B_value || !out ||
      !aligned16(x) || !aligned16(A_key) || !aligned16(A_value) ||
      !aligned16(q) || !aligned16(B_key) || !aligned16(B_value) ||
      !aligned16(out) || (z_debug && !aligned16(z_debug)))
    return STARKV_EINVAL;
  const Dims d = make_dims(*cfg);
  if (hidden % 64 != 0 || !prefill_supported(d)) return STARKV_EUNSUPPORTED;
  const PrefillWs lay = prefill_ws_layout(d, chunk);
  if (!workspace || !aligned16(workspace) || ws_bytes < lay.total)
    return STARKV_EWORKSPACE;
  hipError_t e = launch_prefill(d, *cache, ctx_len, chunk, x, hidden, A_key,
                                A_value, q, B_key, B_value, sm_scale, out,
                                z_debug, static_cast<char*>(workspace), lay,
                                stream, events);
  if (e == hipErrorNotSupported) return STARKV_EUNSUPPORTED;
  return e == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

int starkv_prefill(const starkv_config* cfg, const starkv_cache* cache,
                   int32_t ctx_len, int32_t chunk, const void* x,
                   int32_t hidden, const void* A_key, const void* A_value,
                   const void* q, const void* B_key, const void* B_value,
                   float sm_scale, float* out, float* z_debug, void* workspace,
                   size_t ws_bytes, hipStream_t stream) {
  return prefill_impl(cfg, cache, ctx_len, chunk, x, hidden, A_key, A_value, q,
                      B_key, B_value, sm_scale, out, z_debug, workspace,
                      ws_bytes, stream, nullptr);
}

int starkv_prefill_profiled(const starkv_config* cfg, const starkv_cache* cache,
                            int32_t ctx_len, int32_t chunk, const void* x,
                            int32_t hidden, const void* A_key,
                            const void* A_value, const void* q,
                            const void* B_key, const void* B_value,
                            float sm_scale, float* out, float* z_debug,
                            void* workspace, size_t ws_bytes,
                            hipStream_t stream, hipEvent_t* events) {
  if (!events) return STARKV_EINVAL;
  return prefill_impl(cfg, cache, ctx_len, chunk, x, hidden, A_key, A_value, q,
                      B_key, B_value, sm_scale, out, z_debug, workspace,
                      ws_bytes, stream, events);
}

int starkv_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || !aligned16(src) || reinterpret_cast<uintptr_t>(sink) % 4 != 0 ||
      bytes == 0 || bytes % 16 != 0)
    return STARKV_EINVAL;
  return launch_stream_read(src, bytes, sink, stream) == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

const char* starkv_strerror(int status) {
  switch (status) {
    case STARKV_OK: return "success";
    case STARKV_EINVAL: return "invalid argument";
    case STARKV_EUNSUPPORTED: return "unsupported shape or cache type";
    case STARKV_ECAPACITY: return "tokens exceed cache capacity";
    case STARKV_EWORKSPACE: return "workspace missing or too small";
    case STARKV_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
