// Streaming-read ceiling: the bandwidth at which the device streams a large
// buffer once with non-temporal 16-byte loads, as the decode split kernel
// streams the cache.  A measurement helper, not a step of the method.
#include "internal.h"

namespace starkv {
namespace {

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 512;

// One non-temporal 16-byte load per thread over a grid that covers the
// buffer (the fastest of the launch shapes measured: fewer loads per thread
// on more workgroups stream faster); the XOR of the data is written only if
// it equals a fixed value, so the load cannot be removed and the write
// practically never happens.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4s* __restrict__ src,
                                                                     size_t n,
                                                                     uint32_t* __restrict__ sink) {
  const size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  if (i >= n) return;
  const u32x4s v = __builtin_nontemporal_load(src + i);
  const uint32_t x = v[0] ^ v[1] ^ v[2] ^ v[3];
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n = bytes / 16;
  const size_t blocks = (n + kStreamThreads - 1) / kStreamThreads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  stream_read_kernel<<<(unsigned)blocks, kStreamThreads, 0, s>>>(
      static_cast<const u32x4s*>(src), n, sink);
  return hipGetLastError();
}

}  // namespace starkv
