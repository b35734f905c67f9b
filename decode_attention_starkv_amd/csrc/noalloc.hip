// starkv_decode_noalloc: decode with the library's own fixed device scratch
// array in place of a caller workspace, for callers that cannot allocate
// (code under stream capture, tight serving loops, harnesses that forbid
// allocation).  Same kernels as starkv_decode.
//
// The array is a file-scope __device__ variable, so every device the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol: its device address is
// asked of the runtime (hipGetSymbolAddress) once per device, with that device
// current, on the first call there, and only that address is ever handed to
// kernels.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "internal.h"

namespace starkv {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on device `dev` (current), or nullptr if the
// runtime cannot give it.
char* scratch_on(int dev) {
  static std::mutex mu;
  static std::map<int, char*> known;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = known.find(dev);
  if (it != known.end()) return it->second;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return nullptr;
  }
  known[dev] = static_cast<char*>(p);
  return static_cast<char*>(p);
}

}  // namespace
}  // namespace starkv

using namespace starkv;

extern "C" {

size_t starkv_noalloc_scratch_bytes(void) { return kScratchBytes; }

int starkv_decode_noalloc(const starkv_config* cfg, const starkv_cache* cache,
                          int32_t seq_len, const void* q, const void* B_key,
                          const void* B_value, float sm_scale, float* out,
                          hipStream_t stream) {
  DecodeWs lay;
  const int st = validate_decode(cfg, cache, seq_len, q, B_key, B_value, out, &lay);
  if (st != STARKV_OK) return st;
  if (lay.total > kScratchBytes) return STARKV_EWORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return STARKV_ELAUNCH;
  char* ws = scratch_on(dev);
  if (!ws) return STARKV_ELAUNCH;
  const hipError_t e = launch_decode(make_dims(*cfg), *cache, seq_len, q, B_key,
                                     B_value, sm_scale, out, ws, lay, stream);
  return e == hipSuccess ? STARKV_OK : STARKV_ELAUNCH;
}

}  // extern "C"
