// Chunked causal prefill over the latent cache.
#include "internal.h"

namespace starkv {

static size_t align256p(size_t x) { return (x + 255) & ~(size_t)255; }

PrefillWs prefill_ws_layout(const Dims& d, int chunk) {
  PrefillWs w;
  size_t off = 0;
  w.z = off;
  off += align256p((size_t)d.B * chunk * (d.Hkv * d.rk + d.rv) * 4);
  w.qt = off;
  w.part = off;
  w.total = off;
  return w;
}

hipError_t launch_prefill(const Dims&, const starkv_cache&, int, int,
                          const void*, int, const void*, const void*,
                          const void*, const void*, const void*, float, float*,
                          float*, char*, const PrefillWs&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace starkv
