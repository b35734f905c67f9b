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
// The Q43 decode contraction scales P by up to 2^6 (the in-place field
// weights) before the per-group scale: its running max moves at 2^2, so
// that P times the weight stays <= 2^8 as elsewhere.
constexpr float kLazyQ43 = 2.0f;
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

// fp16 pair p (tokens 2p, 2p + 1 as the two 16-bit halves) of one channel's
// 32-token value run, read in place for the decode contraction.  Run layout:
// a 4-bit run is 4 words, word p / 4 holding pair p at bit 4 (p % 4) of
// each half; a 3-bit run is 3 words, word p / 5 holding pair p < 15 at bit
// 3 (p % 5) of each half, and pair 15 (tokens 30, 31) has its three bits in
// bits 15 / 31 of the three words.
//   - A field at bit b <= 6 of a 16-bit half is the fp16 subnormal
//     c * 2^(b-24) after one AND; the fields above it are first shifted down
//     by 8 (4-bit runs) or 9 (3-bit runs) bits.
//   - The product's other operand carries run_pair_weight(p) = 2^(K-b), b
//     the bit at which pair p's field is read (K = 4 for 4-bit runs, 6 for
//     3-bit runs), so every product comes out in units of 2^(K-24).
//   - Pair 15 of a 3-bit run is assembled from its three one-bit fields
//     (weight 2^6).
template <bool kFour>
__device__ inline uint32_t run_pair_inplace(const u32x4& w, int p) {
  if constexpr (kFour) {
    const uint32_t x = (p & 2) ? (w[p >> 2] >> 8) : w[p >> 2];
    return x & ((p & 1) ? 0x00F000F0u : 0x000F000Fu);
  } else {
    if (p < 15) {
      const int f = p % 5;
      const uint32_t x = f >= 3 ? (w[p / 5] >> 9) : w[p / 5];
      return x & (f == 0 || f == 3 ? 0x00070007u : f == 1 || f == 4 ? 0x00380038u : 0x01C001C0u);
    }
    return ((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) |
           ((w[2] >> 13) & 0x00040004u);
  }
}
template <bool kFour>
__host__ __device__ constexpr float run_pair_weight(int p) {
  if (kFour) return (p & 1) ? 1.0f : 16.0f;
  if (p == 15) return 64.0f;
  return p % 5 == 0 || p % 5 == 3 ? 64.0f : p % 5 == 1 || p % 5 == 4 ? 8.0f : 1.0f;
}

// One Q43 key tile of one KV head as seen by one lane (= token), as 17 fp16
// pairs whose halves hold codes (or parts of codes) in place: a field with
// value c at bit p <= 7 of a half reads as the subnormal c * 2^(p-24), so
// the query record carries the matching 2^-p and no field is shifted down.
// mhi / mlo: the meta words (s | z << 16, fp16) of the 4-bit and the 3-bit
// group.
struct KeyLane {
  uint32_t pr[17];
  uint32_t mhi, mlo;
};

// kc: the lane's hi word, lo0 word, lo1 word, lo2 byte and its two meta
// words.  Word layout: hi = channels 0-3 (low half) and 4-7 (high half) as
// nibbles; lo0 / lo1 = channels 8-12 / 13-17 (low) and 18-22 / 23-27 (high)
// as 3-bit fields at bits 0, 3, .., 12 of each half; the byte holds channels
// 28, 29 and the two low bits of 30; bit 15 of lo0 is the top bit of 30 and
// bit 31 of lo0, bits 15 and 31 of lo1 are the three bits of 31.
__device__ inline KeyLane unpack_key_lane(const uint32_t (&kc)[6]) {
  KeyLane k;
  const uint32_t whi = kc[0], r8 = kc[3];
  k.pr[0] = whi & 0x000F000Fu;              // ch 0, 4 at bit 0
  k.pr[1] = whi & 0x00F000F0u;              // ch 1, 5 at bit 4
  const uint32_t wh8 = whi >> 8;
  k.pr[2] = wh8 & 0x000F000Fu;              // ch 2, 6 at bit 0
  k.pr[3] = wh8 & 0x00F000F0u;              // ch 3, 7 at bit 4
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t w = kc[1 + i];
    k.pr[4 + 5 * i] = w & 0x00070007u;      // fields 0 at bit 0
    k.pr[5 + 5 * i] = w & 0x00380038u;      // fields 1 at bit 3
    k.pr[6 + 5 * i] = w & 0x01C001C0u;      // fields 2 at bit 6
    const uint32_t t = w >> 9;
    k.pr[7 + 5 * i] = t & 0x00070007u;      // fields 3 at bit 0
    k.pr[8 + 5 * i] = t & 0x00380038u;      // fields 4 at bit 3
  }
  const uint32_t x = r8 | (r8 << 16);
  k.pr[14] = x & 0x00380007u;               // ch 28 at bit 0, ch 29 at bit 3
  // ch 30 at bit 6 (two byte bits + bit 15 of lo0 moved to bit 8), bit 0
  // of ch 31 (bit 31 of lo0) at bit 8 of the high half
  k.pr[15] = ((kc[1] >> 7) & 0x01000100u) | (r8 & 0xC0u);
  k.pr[16] = (kc[2] >> 15) & 0x00010001u;   // bits 1 and 2 of ch 31
  k.mhi = kc[4];
  k.mlo = kc[5];
  return k;
}

// The same for a uniform 4-bit key tile: kc holds the lane's four nibble
// planes (plane p: channels 8p .. 8p+3 in the low half, 8p+4 .. 8p+7 in the
// high half) and its two meta words; pair 4p + k is read like pair k of the
// 4-bit plane above, and pair 16 is zero.
__device__ inline KeyLane unpack_key_lane_u4(const uint32_t (&kc)[6]) {
  KeyLane k;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t w = kc[p], w8 = w >> 8;
    k.pr[4 * p] = w & 0x000F000Fu;
    k.pr[4 * p + 1] = w & 0x00F000F0u;
    k.pr[4 * p + 2] = w8 & 0x000F000Fu;
    k.pr[4 * p + 3] = w8 & 0x00F000F0u;
  }
  k.pr[16] = 0u;
  k.mhi = kc[4];
  k.mlo = kc[5];
  return k;
}

// Latent score of one key lane against one Q43 query record (17 fp16
// pairs, then the sums of the hi and lo query parts times 2^-24), in units
// of 2^-24 (log2 domain, pre-scaled):
//   s_hi (q_hi . k_hi 2^-24) + s_lo (q_lo . k_lo 2^-24) + (z_hi sum q_hi + z_lo sum q_lo) 2^-24
__device__ inline float key_score(const KeyLane& k, const uint32_t* rec) {
  float ah = 0.0f, al = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ah = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, k.pr[i]),
                                __builtin_bit_cast(h2, rec[i]), ah, false);
#pragma unroll
  for (int i = 4; i < 17; ++i)
    al = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, k.pr[i]),
                                __builtin_bit_cast(h2, rec[i]), al, false);
  const h2 mh = __builtin_bit_cast(h2, k.mhi), ml = __builtin_bit_cast(h2, k.mlo);
  const float qs_hi = __builtin_bit_cast(float, rec[17]);
  const float qs_lo = __builtin_bit_cast(float, rec[18]);
  return fmaf((float)mh[0], ah,
              fmaf((float)ml[0], al, fmaf((float)mh[1], qs_hi, (float)ml[1] * qs_lo)));
}

// Rotary frequency of pair p, theta^(-2 p / dh), in fp64.
__device__ inline double rope_freq(int p, int dh, double log2_theta) {
  return exp2(-2.0 * p / dh * log2_theta);
}

// sin / cos of the rotary angle pos * w, reduced modulo 2 pi in fp64; the
// hardware sine and cosine take the angle in turns, here in [0, 1).
__device__ inline void rope_sincos(int pos, double w, float* c, float* s) {
  const double a = (double)pos * w;
  const double turns = a * 0.15915494309189535;     // 1 / (2 pi)
  const float frac = (float)(turns - floor(turns));
  *c = __builtin_amdgcn_cosf(frac);
  *s = __builtin_amdgcn_sinf(frac);
}

// sin / cos of the rotary angle of pair p at position pos,
// pos * theta^(-2 p / dh)
__device__ inline void rope_angle(int pos, int p, int dh, double log2_theta, float* c,
                                  float* s) {
  rope_sincos(pos, rope_freq(p, dh, log2_theta), c, s);
}

}  // namespace starkv
