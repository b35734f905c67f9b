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
      (c->rotate != 0 && c->rotate != 1) || !(c->rope_theta >= 0.0f) ||
      c->rope_theta == std::numeric_limits<float>::infinity())
    return STARKV_EINVAL;
  const bool quant = c->cache_dtype == STARKV_CACHE_Q43;
  if (quant) {
    // the precision split of section 6.1: two blocks, each at its own width
    if (c->hi_bits < 1 || c->hi_bits > 8 || c->lo_bits < 1 || c->lo_bits > 8 ||
        c->group_size < 1 || c->key_hi_channels < 0 ||
        c->key_hi_channels > c->key_rank || c->value_hi_channels < 0 ||
        c->value_hi_channels > c->value_rank)
      return STARKV_EINVAL;
  } else if (c->hi_bits != 0 || c->lo_bits != 0 || c->group_size != 0 ||
             c->key_hi_channels != 0 || c->value_hi_channels != 0) {
    return STARKV_EINVAL;   // unquantized caches have no precision split
  }
  if (c->key_ranks) {
    if (c->n_kv_heads > kMaxQHeads) return STARKV_EUNSUPPORTED;
    for (int g = 0; g < c->n_kv_heads; ++g)
      if (c->key_ranks[g] < 8 || c->key_ranks[g] % 8 != 0 ||
          c->key_ranks[g] > c->key_rank)
        return STARKV_EINVAL;
    // quantized caches pad every head to the 32-channel key tile (eq. 15's
    // padding term): ranks are checked against key_rank = 32 above
  }
  // rotary keys: quantized caches (decode: rope.hip, prefill: prefill.hip),
  // head_dim 64 or 128
  if (c->rope_theta > 0.0f &&
      (!quant || (c->head_dim != 64 && c->head_dim != 128)))
    return STARKV_EUNSUPPORTED;
  const int g = c->n_q_heads / c->n_kv_heads;
  if (c->n_q_heads > kMaxQHeads || (g != 1 && g != 2 && g != 4 && g != 8))
    return STARKV_EUNSUPPORTED;
  if (c->head_dim % 16 != 0 || c->head_dim > 256) return STARKV_EUNSUPPORTED;
  if (c->value_rank % 32 != 0 || c->value_rank > 1024) return STARKV_EUNSUPPORTED;
  if (quant) {
    if (c->key_rank != 32 || c->value_rank % 256 != 0 ||
        (c->n_kv_heads > 4 && c->n_kv_heads % 4 != 0))
      return STARKV_EUNSUPPORTED;
    // the 4/3-bit split, or both blocks at 4 bits (uniform 4-bit cache)
    if (c->hi_bits != 4 || (c->lo_bits != 3 && c->lo_bits != 4) || c->group_size != 32 ||
        c->key_hi_channels != c->key_rank / 4 ||
        c->value_hi_channels != c->value_rank / 4)
      return STARKV_EUNSUPPORTED;
    // the rotation blocks (largest power of two dividing each block width)
    // stay within one wave's 256 channels, where the inverse rotation of
    // the merge runs in registers
    if (c->rotate && (pow2_divisor(c->value_hi_channels) > 256 ||
                      pow2_divisor(c->value_rank - c->value_hi_channels) > 256 ||
                      pow2_divisor(c->key_hi_channels) > 8 ||
                      pow2_divisor(c->key_rank - c->key_hi_channels) > 8))
      return STARKV_EUNSUPPORTED;
  } else {
    if (c->rotate) return STARKV_EUNSUPPORTED;
    if (c->key_rank % 8 != 0 || c->key_rank > 64) return STARKV_EUNSUPPORTED;
  }
  return STARKV_OK;
}

// The configuration is valid and a decode kernel exists for it.
int check_decode_config(const starkv_config* c) {
  const int st = check_config(c);
  if (st != STARKV_OK) return st;
  return decode_supported(make_dims(*c)) ? STARKV_OK : STARKV_EUNSUPPORTED;
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
      case STARKV_BUF_KEY: return B * H * NT * key_block_bytes(c.lo_bits);
      case STARKV_BUF_KEY_META: return B * H * NT * kTile * 8;
      case STARKV_BUF_VALUE: return B * NT * value_tile_bytes((int)rv, c.lo_bits);
      case STARKV_BUF_VALUE_META: return B * NT * 2 * (rv / 32) * kTile * 2;
      default: return 0;
    }
  }
  const size_t es = c.cache_dtype == STARKV_CACHE_F32 ? 4 : 2;
  size_t rsum = H * rk;   // eq. 15: the sum of the per-head key ranks
  if (c.key_ranks) {
    rsum = 0;
    for (int g = 0; g < c.n_kv_heads; ++g) rsum += c.key_ranks[g];
  }
  switch (which) {
    case STARKV_BUF_KEY: return B * T * rsum * es;
    case STARKV_BUF_VALUE: return B * NT * rv * kTile * es;
    default: return 0;
  }
}

}  // namespace

// The split count fills every compute unit with as many decode workgroups
// as stay resident on it.
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
    if (!decode_supported(d)) return 0;
    if (n_tokens > cfg->max_tokens) return 0;
    return decode_ws_layout(d, choose_splits(*cfg, n_tokens), n_tokens).total;
  }
  if (op == STARKV_OP_PREFILL) {
    if (!prefill_supported(d)) return 0;
    return prefill_ws_layout(d, n_tokens).total;
  }
  return 0;
}

int32_t starkv_decode_splits(const starkv_config* cfg, int32_t seq_len) {
  if (check_decode_config(cfg) != STARKV_OK || seq_len < 1) return 0;
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

}  // extern "C"

namespace starkv {

// Everything starkv_decode checks before it looks at the workspace.
int validate_decode(const starkv_config* cfg, const starkv_cache* cache,
                    int32_t seq_len, const void* q, const void* B_key,
                    const void* B_value, const float* out, DecodeWs* lay) {
  int st = check_decode_config(cfg);
  if (st != STARKV_OK) return st;
  if ((st = check_cache(cfg, cache)) != STARKV_OK) return st;
  if (seq_len < 1) return STARKV_EINVAL;
  if (seq_len > cfg->max_tokens) return STARKV_ECAPACITY;
  if (!q || !B_key || !B_value || !out || !aligned16(q) || !aligned16(B_key) ||
      !aligned16(B_value) || !aligned16(out))
    return STARKV_EINVAL;
  *lay = decode_ws_layout(make_dims(*cfg), choose_splits(*cfg, seq_len), seq_len);
  return STARKV_OK;
}

}  // namespace starkv

extern "C" {

static int decode_impl(const starkv_config* cfg, const starkv_cache* cache,
                       int32_t seq_len, const void* q, const void* B_key,
                       const void* B_value, float sm_scale, float* out,
                       void* workspace, size_t ws_bytes, hipStream_t stream,
                       hipEvent_t* events) {
  DecodeWs lay;
  const int st = validate_decode(cfg, cache, seq_len, q, B_key, B_value, out, &lay);
  if (st != STARKV_OK) return st;
  if (!workspace || !aligned16(workspace) || ws_bytes < lay.total)
    return STARKV_EWORKSPACE;
  hipError_t e = launch_decode(make_dims(*cfg), *cache, seq_len, q, B_key, B_value,
                               sm_scale, out, static_cast<char*>(workspace), lay,
                               stream, events);
  return e == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

static int decode_step_impl(const starkv_config* cfg, const starkv_cache* cache,
                            const float* z_key, const float* z_value, int32_t pos,
                            int32_t n, const void* q, const void* B_key,
                            const void* B_value, float sm_scale, float* out,
                            void* workspace, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t* events) {
  if (pos < 0 || n < 0) return STARKV_EINVAL;
  if ((int64_t)pos + n > std::numeric_limits<int32_t>::max()) return STARKV_ECAPACITY;
  DecodeWs lay;
  const int st = validate_decode(cfg, cache, pos + n, q, B_key, B_value, out, &lay);
  if (st != STARKV_OK) return st;
  if (n > 0 && (!z_key || !z_value || !aligned16(z_key) || !aligned16(z_value)))
    return STARKV_EINVAL;
  if (!workspace || !aligned16(workspace) || ws_bytes < lay.total)
    return STARKV_EWORKSPACE;
  const Dims d = make_dims(*cfg);
  char* ws = static_cast<char*>(workspace);
  if (events) (void)hipEventRecord(events[0], stream);
  hipError_t e = hipSuccess;
  bool fused = false;
  if (n > 0) {
    if (d.dtype == STARKV_CACHE_Q43 && d.rope_theta == 0.0f) {
      e = launch_append_qproj(d, *cache, z_key, z_value, pos, n, q, B_key,
                              sm_scale * 1.4426950408889634f, ws + lay.qt, stream);
      fused = true;
    } else if (d.dtype != STARKV_CACHE_Q43) {
      e = launch_append_qproj_plain(d, *cache, z_key, z_value, pos, n, q, B_key,
                                    sm_scale * 1.4426950408889634f, ws + lay.qt, stream);
      fused = true;
    } else {
      e = launch_append(d, *cache, z_key, z_value, pos, n, stream);
    }
    if (e != hipSuccess) return STARKV_ELAUNCH;
  }
  e = launch_decode(d, *cache, pos + n, q, B_key, B_value, sm_scale, out, ws, lay,
                    stream, events, fused, true);
  return e == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

int starkv_decode_step(const starkv_config* cfg, const starkv_cache* cache,
                       const float* z_key, const float* z_value, int32_t pos,
                       int32_t n, const void* q, const void* B_key,
                       const void* B_value, float sm_scale, float* out,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  return decode_step_impl(cfg, cache, z_key, z_value, pos, n, q, B_key, B_value,
                          sm_scale, out, workspace, ws_bytes, stream, nullptr);
}

int starkv_decode_step_profiled(const starkv_config* cfg, const starkv_cache* cache,
                                const float* z_key, const float* z_value,
                                int32_t pos, int32_t n, const void* q,
                                const void* B_key, const void* B_value,
                                float sm_scale, float* out, void* workspace,
                                size_t ws_bytes, hipStream_t stream,
                                hipEvent_t* events) {
  if (!events) return STARKV_EINVAL;
  return decode_step_impl(cfg, cache, z_key, z_value, pos, n, q, B_key, B_value,
                          sm_scale, out, workspace, ws_bytes, stream, events);
}

// ------------------------------------------- value/output fusion, head sum

static bool hidden_ok(const starkv_config* cfg, int32_t hidden) {
  return cfg->cache_dtype != STARKV_CACHE_F32 && hidden >= 128 && hidden % 128 == 0;
}

size_t starkv_fused_factor_bytes(const starkv_config* cfg, int32_t hidden) {
  if (check_config(cfg) != STARKV_OK || !hidden_ok(cfg, hidden)) return 0;
  return (size_t)cfg->n_q_heads * cfg->value_rank * hidden * 2;
}

int starkv_fuse_value_output(const starkv_config* cfg, const void* B_value,
                             const void* W_o, int32_t hidden, void* F,
                             hipStream_t stream) {
  const int st = check_config(cfg);
  if (st != STARKV_OK) return st;
  if (hidden < 1) return STARKV_EINVAL;
  if (!hidden_ok(cfg, hidden)) return STARKV_EUNSUPPORTED;
  if (!B_value || !W_o || !F || !aligned16(B_value) || !aligned16(W_o) || !aligned16(F))
    return STARKV_EINVAL;
  return launch_fuse_vo(make_dims(*cfg), B_value, W_o, hidden, F, stream) == hipSuccess
             ? STARKV_OK : STARKV_ELAUNCH;
}

static size_t hidden_extra(const Dims& d, int32_t hidden) {
  return (size_t)hidden_k_slices(d, hidden) * d.B * hidden * 4;
}

size_t starkv_decode_hidden_workspace_bytes(const starkv_config* cfg,
                                            int32_t seq_len, int32_t hidden) {
  const size_t base = starkv_workspace_bytes(cfg, STARKV_OP_DECODE, seq_len);
  if (base == 0 || !hidden_ok(cfg, hidden)) return 0;
  return base + hidden_extra(make_dims(*cfg), hidden);
}

static int decode_hidden_impl(const starkv_config* cfg, const starkv_cache* cache,
                              int32_t seq_len, const void* q, const void* B_key,
                              const void* F, int32_t hidden, float sm_scale, float* y,
                              void* workspace, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t* events) {
  DecodeWs lay;
  // F stands in for B_value in the common checks
  int st = validate_decode(cfg, cache, seq_len, q, B_key, F, y, &lay);
  if (st != STARKV_OK) return st;
  if (hidden < 1) return STARKV_EINVAL;
  if (!hidden_ok(cfg, hidden)) return STARKV_EUNSUPPORTED;
  const Dims d = make_dims(*cfg);
  const size_t need = lay.total + hidden_extra(d, hidden);
  if (!workspace || !aligned16(workspace) || ws_bytes < need) return STARKV_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipError_t e = launch_decode(d, *cache, seq_len, q, B_key, nullptr, sm_scale, nullptr,
                               ws, lay, stream, events, false, false, true);
  if (e != hipSuccess) return STARKV_ELAUNCH;
  e = launch_hidden(d, reinterpret_cast<const float*>(ws + lay.obar), F, hidden,
                    reinterpret_cast<float*>(ws + lay.total), y, stream,
                    events ? events + 4 : nullptr);
  return e == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

int starkv_decode_hidden(const starkv_config* cfg, const starkv_cache* cache,
                         int32_t seq_len, const void* q, const void* B_key,
                         const void* F, int32_t hidden, float sm_scale, float* y,
                         void* workspace, size_t ws_bytes, hipStream_t stream) {
  return decode_hidden_impl(cfg, cache, seq_len, q, B_key, F, hidden, sm_scale, y,
                            workspace, ws_bytes, stream, nullptr);
}

int starkv_decode_hidden_profiled(const starkv_config* cfg, const starkv_cache* cache,
                                  int32_t seq_len, const void* q, const void* B_key,
                                  const void* F, int32_t hidden, float sm_scale,
                                  float* y, void* workspace, size_t ws_bytes,
                                  hipStream_t stream, hipEvent_t* events) {
  if (!events) return STARKV_EINVAL;
  return decode_hidden_impl(cfg, cache, seq_len, q, B_key, F, hidden, sm_scale, y,
                            workspace, ws_bytes, stream, events);
}

// ------------------------------------------------ paged and ragged caches

int starkv_append_paged(const starkv_config* cfg, const starkv_cache* cache,
                        const int32_t* page_table, int32_t pages_per_seq,
                        const int32_t* positions, const float* z_key,
                        const float* z_value, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != STARKV_OK) return st;
  if ((st = check_cache(cfg, cache)) != STARKV_OK) return st;
  if (cfg->cache_dtype != STARKV_CACHE_Q43) return STARKV_EUNSUPPORTED;
  if (!page_table || !positions || pages_per_seq < 1 || !z_key || !z_value ||
      !aligned16(z_key) || !aligned16(z_value) ||
      reinterpret_cast<uintptr_t>(page_table) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(positions) % 4 != 0)
    return STARKV_EINVAL;
  Dims d = make_dims(*cfg);
  d.pages = page_table;
  d.pages_per_seq = pages_per_seq;
  d.positions = positions;
  hipError_t e = launch_append(d, *cache, z_key, z_value, 0, 1, stream);
  return e == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

int starkv_decode_paged(const starkv_config* cfg, const starkv_cache* cache,
                        const int32_t* page_table, int32_t pages_per_seq,
                        const int32_t* seq_lens, int32_t max_seq_len, const void* q,
                        const void* B_key, const void* B_value, float sm_scale,
                        float* out, void* workspace, size_t ws_bytes,
                        hipStream_t stream) {
  DecodeWs lay;
  int st = validate_decode(cfg, cache, max_seq_len, q, B_key, B_value, out, &lay);
  if (st != STARKV_OK) return st;
  if (cfg->cache_dtype != STARKV_CACHE_Q43) return STARKV_EUNSUPPORTED;
  if (!page_table || !seq_lens || pages_per_seq < 1 ||
      (int64_t)pages_per_seq * kTile < max_seq_len ||
      reinterpret_cast<uintptr_t>(page_table) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(seq_lens) % 4 != 0)
    return STARKV_EINVAL;
  if (!workspace || !aligned16(workspace) || ws_bytes < lay.total)
    return STARKV_EWORKSPACE;
  Dims d = make_dims(*cfg);
  d.pages = page_table;
  d.pages_per_seq = pages_per_seq;
  d.lens = seq_lens;
  hipError_t e = launch_decode(d, *cache, max_seq_len, q, B_key, B_value, sm_scale, out,
                               static_cast<char*>(workspace), lay, stream);
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
                        size_t ws_bytes, hipStream_t stream, hipEvent_t* events,
                        const int32_t* page_table = nullptr, int32_t pages_per_seq = 0) {
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
  Dims d = make_dims(*cfg);
  if (hidden % 64 != 0 || !prefill_supported(d)) return STARKV_EUNSUPPORTED;
  if (page_table) {
    // every sequence's positions [0, ctx_len + chunk) must have pages
    if (pages_per_seq < 1 || (int64_t)pages_per_seq * kTile < (int64_t)ctx_len + chunk ||
        reinterpret_cast<uintptr_t>(page_table) % 4 != 0)
      return STARKV_EINVAL;
    d.pages = page_table;
    d.pages_per_seq = pages_per_seq;
  }
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

int starkv_prefill_paged(const starkv_config* cfg, const starkv_cache* cache,
                         const int32_t* page_table, int32_t pages_per_seq,
                         int32_t ctx_len, int32_t chunk, const void* x, int32_t hidden,
                         const void* A_key, const void* A_value, const void* q,
                         const void* B_key, const void* B_value, float sm_scale,
                         float* out, float* z_debug, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  if (!page_table) return STARKV_EINVAL;
  return prefill_impl(cfg, cache, ctx_len, chunk, x, hidden, A_key, A_value, q,
                      B_key, B_value, sm_scale, out, z_debug, workspace, ws_bytes,
                      stream, nullptr, page_table, pages_per_seq);
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
