// Device-side helpers shared by the decode and prefill kernels (gfx950).
#pragma once

#include "internal.h"

namespace starkv {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTwo24 = 16777216.0f;
// The running max used for the probabilities is only moved when a tile's max
// exceeds it by more than this (log2 units), so probabilities stay <= 2^8 and
// the accumulators are rescaled rarely.
constexpr float kLazy = 8.0f;
constexpr int kQ43Rec = 20;   // dwords per (b, h) query record, Q43
constexpr int kPlainRec = 64; // floats per (b, h) query record, F32/BF16
// Cache-policy bits of a non-temporal load.
constexpr int kNonTemporal = 2;

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x += __shfl_xor(x, s);
  return x;
}
__device__ inline float f16v(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ inline float bf16v(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
__device__ inline void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Row of the 32x32 MFMA accumulator held in register v of a lane.
__device__ inline int acc_row(int v, int lane) {
  return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
}

// 16 fp16 pairs (tokens 2p, 2p+1) of one channel's 32-token value run:
// 4-bit run in 4 words, 3-bit run in 3 words (see the format description).
template <bool kFour>
__device__ inline uint32_t run_pair(const u32x4& w, int p) {
  if constexpr (kFour) {
    return (w[p >> 2] >> (4 * (p & 3))) & 0x000F000Fu;
  } else {
    if (p < 15) return (w[p / 5] >> (3 * (p % 5))) & 0x00070007u;
    return ((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) |
           ((w[2] >> 13) & 0x00040004u);
  }
}

// One Q43 key tile of one KV head as seen by one lane (= token): the 4-bit
// and 3-bit codes as fp16 pairs (raw bits, i.e. k * 2^-24) in the order of
// the query record, and the group scales (times 2^24) and zeros.
struct KeyLane {
  uint32_t ph[4], pl[12];
  float s_hi, z_hi, s_lo, z_lo;
};

// kc: the lane's hi word, lo0 word, lo1 word, lo2 byte and its two meta
// words (s_hi | z_hi << 16, s_lo | z_lo << 16).
__device__ inline KeyLane unpack_key_lane(const uint32_t (&kc)[6]) {
  KeyLane k;
  const uint32_t whi = kc[0], w0 = kc[1], w1 = kc[2], r8 = kc[3];
  k.s_hi = f16v(kc[4] & 0xFFFFu) * kTwo24;
  k.z_hi = f16v(kc[4] >> 16);
  k.s_lo = f16v(kc[5] & 0xFFFFu) * kTwo24;
  k.z_lo = f16v(kc[5] >> 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) k.ph[i] = (whi >> (4 * i)) & 0x000F000Fu;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    k.pl[i] = (w0 >> (3 * i)) & 0x00070007u;
    k.pl[5 + i] = (w1 >> (3 * i)) & 0x00070007u;
  }
  const uint32_t R = r8 | (((w0 >> 15) & 1u) << 8) | ((w0 >> 31) << 9) |
                     (((w1 >> 15) & 1u) << 10) | ((w1 >> 31) << 11);
  k.pl[10] = (R & 7u) | (((R >> 6) & 7u) << 16);
  k.pl[11] = ((R >> 3) & 7u) | (((R >> 9) & 7u) << 16);
  return k;
}

// Latent score (log2 units, pre-scaled) of one key lane against one Q43
// query record (16 fp16 pairs, then the sums of the hi and lo query parts).
__device__ inline float key_score(const KeyLane& k, const uint32_t* rec) {
  float ah = 0.0f, al = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ah = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, k.ph[i]),
                                __builtin_bit_cast(h2, rec[i]), ah, false);
#pragma unroll
  for (int i = 0; i < 12; ++i)
    al = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, k.pl[i]),
                                __builtin_bit_cast(h2, rec[4 + i]), al, false);
  const float qs_hi = __builtin_bit_cast(float, rec[16]);
  const float qs_lo = __builtin_bit_cast(float, rec[17]);
  return fmaf(k.s_hi, ah, fmaf(k.z_hi, qs_hi, fmaf(k.s_lo, al, k.z_lo * qs_lo)));
}

}  // namespace starkv
