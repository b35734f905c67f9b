// Query projection into the key latent (Algorithm 2 of the technical review
// of arXiv 2606.08382, step 4 read through eq. 2: q K^T = (q B_key) Z^T), as
// a block-level device function: decode.hip launches it on its own, and the
// decode step kernel of append.hip shares one launch between it and the
// append of the new tokens.
#pragma once

#include "device.h"

namespace starkv {

// ------------------------------------------------------------------ qproj --

// One block of 256 threads per (b, h) = bh: the threads split the d_h contraction into
// chunks (each thread loads its q entries and factor entries together, so
// the kernel makes one round trip to memory), the chunks are summed, then
// wave 0 rotates, scales and packs the record.
// A Q43 record holds the 17 fp16 pairs that meet the in-place code fields of
// the key words (each entry times 2^-p for a field at bit p; channel 31
// split over three one-bit fields), then sum(q_hi) 2^-24 and
// sum(q_lo) 2^-24 as fp32.  For a uniform 4-bit cache the pairs are those
// of the four nibble planes (pair 4p + k: channels 8p + k and 8p + k + 4),
// and pair 16 is zero.
template <int FMT>
__device__ inline void qproj_block(const void* __restrict__ q,
                                   const void* __restrict__ bk, const Dims& d,
                                   float qscale, void* __restrict__ qt, int bh) {
  __shared__ float part[256];
  __shared__ _Float16 sq[32];
  const int g = (bh % d.Hq) / d.G;
  const int t = threadIdx.x;
  const size_t qrow = (size_t)bh * d.dh;
  const int rkp = d.rk <= 32 ? 32 : 64;
  const int c = t % rkp, chunk = t / rkp, nch = 256 / rkp;
  const int klen = (d.dh + nch - 1) / nch;
  float acc = 0.0f;
  const int rank = d.krank[g];       // B_key is [Hkv][d_h][r_k] with r_k the largest rank
  if (c < rank) {
    const int k0 = chunk * klen, k1 = min(d.dh, k0 + klen);
#pragma unroll 16
    for (int k = k0; k < k1; ++k) {
      const size_t bi = ((size_t)g * d.dh + k) * d.rk + c;
      const float bv = FMT == STARKV_CACHE_F32 ? static_cast<const float*>(bk)[bi]
                                               : bf16v(static_cast<const uint16_t*>(bk)[bi]);
      const float qv = FMT == STARKV_CACHE_F32 ? static_cast<const float*>(q)[qrow + k]
                                               : bf16v(static_cast<const uint16_t*>(q)[qrow + k]);
      acc = fmaf(qv, bv, acc);
    }
  }
  part[t] = acc;
  __syncthreads();
  if (t >= 64) return;
  float v = 0.0f;
  if (t < rkp)
    for (int ch = 0; ch < nch; ++ch) v += part[ch * rkp + t];
  if (FMT == STARKV_CACHE_Q43 && d.rotate) {
    // stored key latents are rotated by blocks of 8 (hi block 0-7, lo
    // blocks 8-15, 16-23, 24-31): rotate q~ the same way (eq. 13).
#pragma unroll
    for (int s = 1; s < 8; s <<= 1) {
      float p = __shfl_xor(v, s);
      v = (t & s) ? p - v : v + p;
    }
    v *= inv_sqrt_pow2(8);
  }
  v *= qscale;
  if (FMT != STARKV_CACHE_Q43) {
    // the whole record: entries past r_k are zeros (the split kernels read
    // key rows in 8-channel chunks and may pad them)
    static_cast<float*>(qt)[(size_t)bh * kPlainRec + t] = t < rank ? v : 0.0f;
    return;
  }
  if (t < 32) sq[t] = (_Float16)v;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  uint32_t* rec = static_cast<uint32_t*>(qt) + (size_t)bh * kQ43Rec;
  const float qsum_scale = 1.0f / kTwo24;
  if (t < 17) {
    int a, cc;        // channels of the low and the high half
    float sa, sc;     // their field weights (2^-bit position, or the bit's weight)
    if (d.lob == 4) {
      // pair k of plane p = t / 4 as in the 4-bit plane below; pair 16
      // meets no field and is stored as zero
      a = t < 16 ? 8 * (t >> 2) + (t & 3) : 0;
      cc = a + 4;
      sa = sc = (t & 1) ? 1.0f / 16.0f : 1.0f;
    } else if (t < 4) {
      // channels 0-3 / 4-7; odd pairs sit at bit 4 of their byte
      a = t;
      cc = t + 4;
      sa = sc = (t & 1) ? 1.0f / 16.0f : 1.0f;
    } else if (t < 14) {
      const int i = (t - 4) / 5, f = (t - 4) % 5;
      a = 8 + 5 * i + f;
      cc = 18 + 5 * i + f;
      sa = sc = f == 1 || f == 4 ? 1.0f / 8.0f : f == 2 ? 1.0f / 64.0f : 1.0f;
    } else if (t == 14) {
      a = 28; cc = 29; sa = 1.0f; sc = 1.0f / 8.0f;
    } else if (t == 15) {
      a = 30; cc = 31; sa = 1.0f / 64.0f; sc = 1.0f / 256.0f;
    } else {
      a = 31; cc = 31; sa = 2.0f; sc = 4.0f;
    }
    const _Float16 lo = (_Float16)((float)sq[a] * sa);
    const _Float16 hi = (_Float16)((float)sq[cc] * sc);
    rec[t] = d.lob == 4 && t == 16 ? 0u
                                   : (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                                         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  if (t == 32) {
    float s = 0.0f;
    for (int k = 0; k < 8; ++k) s += (float)sq[k];
    rec[17] = __builtin_bit_cast(uint32_t, s * qsum_scale);
  } else if (t == 33) {
    float s = 0.0f;
    for (int k = 8; k < 32; ++k) s += (float)sq[k];
    rec[18] = __builtin_bit_cast(uint32_t, s * qsum_scale);
  }
}


}  // namespace starkv
