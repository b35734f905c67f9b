// Decode attention over the latent cache -- steps 4-7 of Algorithm 2 in the
// technical review of arXiv 2606.08382 (section 6.2), without a key or value
// cache ever being reconstructed in memory.
//
//   qproj   q~ = q B_key[g] (d_h -> r_k), rotated like the stored latents and
//           pre-scaled by sm_scale*log2(e): the score q K^T equals q~ Z^T
//           (eq. 2 read right to left).
//   split   per (sequence, token split): latent scores, online softmax, then
//           the stacked-head probabilities P [Hq x tokens] times the shared
//           value latent Z_v on MFMA (section 5.3: "Computing P Z_V turns
//           multiple vector-style reductions into a matrix multiplication").
//   merge   partial (m, l, o) of the splits combined by the attention
//           decomposition theorem (CaliDrop review: attention over disjoint
//           token subsets, weighted by each subset's share of the exp-sum),
//           then the rotation undone.
//   vproj   o_h = o~_h B_value[g]^T (eq. 12: the value factor is applied
//           after aggregation, so its cost does not grow with context).
//
// Quantized codes enter fp16 dot products and MFMA as raw bit patterns, i.e.
// as fp16 subnormals k * 2^-24, exactly; the 2^24 and the per-group scale and
// zero are folded outside the inner products:
//   keys:   q~ . z_hat = s * 2^24 * (q~ . k 2^-24) + z * sum(q~)
//   values: P Z_hat    = 2^24 * ((P * s) k 2^-24) + P z      (per 32-ch group)
#include "internal.h"

namespace starkv {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTwo24 = 16777216.0f;
// The running max used for the probabilities is only moved when a tile's max
// exceeds it by more than this (log2 units), so probabilities stay <= 2^8 and
// the accumulators are rescaled rarely.
constexpr float kLazy = 8.0f;
constexpr int kQ43Rec = 20;   // dwords per (b, h) query record, Q43
constexpr int kPlainRec = 64; // floats per (b, h) query record, F32/BF16

struct SplitArgs {
  Dims d;
  int seq_len, splits, tiles_per_split;
  const void* key;
  const uint16_t* kmeta;
  const void* value;
  const uint16_t* vmeta;
  const void* qt;
  float* part_o;
  float* part_ml;
};

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

// ------------------------------------------------------------------ qproj --

template <int FMT>
__global__ __launch_bounds__(64) void qproj_kernel(const void* __restrict__ q,
                                                   const void* __restrict__ bk,
                                                   Dims d, float qscale,
                                                   void* __restrict__ qt) {
  const int bh = blockIdx.x;
  const int b = bh / d.Hq, h = bh % d.Hq, g = h / d.G;
  const int lane = threadIdx.x;
  float acc = 0.0f;
  if (lane < d.rk) {
    for (int k = 0; k < d.dh; ++k) {
      float qv, bv;
      size_t qi = ((size_t)b * d.Hq + h) * d.dh + k;
      size_t bi = ((size_t)g * d.dh + k) * d.rk + lane;
      if (FMT == STARKV_CACHE_F32) {
        qv = static_cast<const float*>(q)[qi];
        bv = static_cast<const float*>(bk)[bi];
      } else {
        qv = bf16v(static_cast<const uint16_t*>(q)[qi]);
        bv = bf16v(static_cast<const uint16_t*>(bk)[bi]);
      }
      acc = fmaf(qv, bv, acc);
    }
  }
  if (FMT == STARKV_CACHE_Q43 && d.rotate) {
    // stored key latents are rotated by blocks of 8 (hi block 0-7, lo
    // blocks 8-15, 16-23, 24-31): rotate q~ the same way (eq. 13).
#pragma unroll
    for (int s = 1; s < 8; s <<= 1) {
      float p = __shfl_xor(acc, s);
      acc = (lane & s) ? p - acc : acc + p;
    }
    acc *= inv_sqrt_pow2(8);
  }
  acc *= qscale;
  if (FMT != STARKV_CACHE_Q43) {
    if (lane < d.rk) static_cast<float*>(qt)[(size_t)bh * kPlainRec + lane] = acc;
    return;
  }
  __shared__ _Float16 sq[32];
  if (lane < 32) sq[lane] = (_Float16)acc;
  __syncthreads();
  uint32_t* rec = static_cast<uint32_t*>(qt) + (size_t)bh * kQ43Rec;
  if (lane < 16) {
    int a, c;  // channel pair (a -> low half, c -> high half)
    if (lane < 4) { a = lane; c = lane + 4; }
    else if (lane < 9) { a = 8 + (lane - 4); c = 8 + 10 + (lane - 4); }
    else if (lane < 14) { a = 8 + 5 + (lane - 9); c = 8 + 15 + (lane - 9); }
    else if (lane == 14) { a = 8 + 20; c = 8 + 22; }
    else { a = 8 + 21; c = 8 + 23; }
    uint32_t lo = __builtin_bit_cast(uint16_t, sq[a]);
    uint32_t hi = __builtin_bit_cast(uint16_t, sq[c]);
    rec[lane] = lo | (hi << 16);
  } else if (lane == 16) {
    float s = 0.0f;
    for (int c = 0; c < 8; ++c) s += (float)sq[c];
    rec[16] = __builtin_bit_cast(uint32_t, s);
  } else if (lane == 17) {
    float s = 0.0f;
    for (int c = 8; c < 32; ++c) s += (float)sq[c];
    rec[17] = __builtin_bit_cast(uint32_t, s);
  }
}

// ------------------------------------------------------------ key scores --

// Scores of one 64-token tile for the G query heads of KV head kh; lane = token.
template <int FMT, int G>
__device__ inline void score_tile(const SplitArgs& a, int b, int kh, int tile,
                                  int lane, float* sc) {
  const Dims& d = a.d;
  if constexpr (FMT == STARKV_CACHE_Q43) {
    const size_t blk = ((size_t)b * d.Hkv + kh) * d.NT + tile;
    const uint8_t* kb = static_cast<const uint8_t*>(a.key) + blk * kKeyBlock;
    const uint32_t whi = reinterpret_cast<const uint32_t*>(kb)[lane];
    const uint32_t w0 = reinterpret_cast<const uint32_t*>(kb + 256)[lane];
    const uint32_t w1 = reinterpret_cast<const uint32_t*>(kb + 512)[lane];
    const uint32_t r8 = kb[768 + lane];
    const uint2 mt = reinterpret_cast<const uint2*>(a.kmeta)[blk * kTile + lane];
    const float s_hi = f16v(mt.x & 0xFFFFu) * kTwo24, z_hi = f16v(mt.x >> 16);
    const float s_lo = f16v(mt.y & 0xFFFFu) * kTwo24, z_lo = f16v(mt.y >> 16);
    uint32_t ph[4], pl[12];
#pragma unroll
    for (int i = 0; i < 4; ++i) ph[i] = (whi >> (4 * i)) & 0x000F000Fu;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      pl[i] = (w0 >> (3 * i)) & 0x00070007u;
      pl[5 + i] = (w1 >> (3 * i)) & 0x00070007u;
    }
    const uint32_t R = r8 | (((w0 >> 15) & 1u) << 8) | ((w0 >> 31) << 9) |
                       (((w1 >> 15) & 1u) << 10) | ((w1 >> 31) << 11);
    pl[10] = (R & 7u) | (((R >> 6) & 7u) << 16);
    pl[11] = ((R >> 3) & 7u) | (((R >> 9) & 7u) << 16);
    const uint32_t* recs = static_cast<const uint32_t*>(a.qt) +
                           ((size_t)b * d.Hq + (size_t)kh * G) * kQ43Rec;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const uint32_t* rec = recs + j * kQ43Rec;
      float ah = 0.0f, al = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ah = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, ph[i]),
                                    __builtin_bit_cast(h2, rec[i]), ah, false);
#pragma unroll
      for (int i = 0; i < 12; ++i)
        al = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pl[i]),
                                    __builtin_bit_cast(h2, rec[4 + i]), al, false);
      const float qs_hi = __builtin_bit_cast(float, rec[16]);
      const float qs_lo = __builtin_bit_cast(float, rec[17]);
      sc[j] = fmaf(s_hi, ah, fmaf(z_hi, qs_hi, fmaf(s_lo, al, z_lo * qs_lo)));
    }
  } else {
    const size_t row = (((size_t)b * d.Hkv + kh) * d.Tmax + (size_t)tile * kTile + lane) * d.rk;
    const float* recs = static_cast<const float*>(a.qt) +
                        ((size_t)b * d.Hq + (size_t)kh * G) * kPlainRec;
    float acc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.0f;
    for (int c0 = 0; c0 < d.rk; c0 += 8) {
      float z[8];
      if constexpr (FMT == STARKV_CACHE_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.key) + row + c0);
        float4 u = p[0], v = p[1];
        z[0] = u.x; z[1] = u.y; z[2] = u.z; z[3] = u.w;
        z[4] = v.x; z[5] = v.y; z[6] = v.z; z[7] = v.w;
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.key) + row + c0);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[2 * e] = __builtin_bit_cast(float, w[e] << 16);
          z[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float* qr = recs + j * kPlainRec + c0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j] = fmaf(qr[e], z[e], acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) sc[j] = acc[j];
  }
}

// ------------------------------------------------------------ split kernel --

// Row of the 32x32 MFMA accumulator held in register v of a lane.
__device__ inline int acc_row(int v, int lane) {
  return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
}

template <int FMT, int G>
__global__ __launch_bounds__(512) void split_kernel(SplitArgs a) {
  constexpr int NW = kDecodeWaves;
  constexpr int KVI = G >= 4 ? 1 : 4 / G;  // KV heads per wave (Hq <= 32)
  constexpr bool kQ = FMT == STARKV_CACHE_Q43;
  constexpr int PS = kQ ? 72 : 68;          // P row stride (elements)
  const Dims& d = a.d;

  __shared__ __attribute__((aligned(16))) float p_raw[2 * 32 * 68];
  __shared__ float alpha_l[2][32];
  __shared__ int flag_l[2];
  __shared__ float bias_l[32][33];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int b = blockIdx.y, sp = blockIdx.x;
  const int n_tiles = (a.seq_len + kTile - 1) / kTile;
  const int tile0 = sp * a.tiles_per_split;
  const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);
  const int GV = d.rv / 32;                 // value column tiles / groups
  const int NH = kQ ? d.rv / 128 : 0;       // 4-bit value groups

  for (int i = tid; i < 2 * 32 * 68; i += 512) p_raw[i] = 0.0f;
  if (tid < 64) alpha_l[tid >> 5][tid & 31] = 1.0f;
  if (tid < 2) flag_l[tid] = -1;
  for (int i = tid; i < 32 * 33; i += 512) (&bias_l[0][0])[i] = 0.0f;
  __syncthreads();

  float m_ref[KVI * G], l_lane[KVI * G];
#pragma unroll
  for (int i = 0; i < KVI * G; ++i) { m_ref[i] = -INFINITY; l_lane[i] = 0.0f; }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  f32x16 bacc = f32x16{};

  const int j = lane >> 5, m = lane & 31;

  for (int tile = tile0, it = 0; tile < tile1; ++tile, ++it) {
    const int buf = it & 1;
    const int rem = a.seq_len - tile * kTile;     // valid tokens in this tile
    const bool valid = lane < rem;
    // ------------------------------------------------------------ scores
#pragma unroll
    for (int ki = 0; ki < KVI; ++ki) {
      const int kh = wave + ki * NW;
      if (kh < d.Hkv) {
        float sc[G];
        score_tile<FMT, G>(a, b, kh, tile, lane, sc);
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
          const int h = kh * G + jj;
          const float x = valid ? sc[jj] : -INFINITY;
          const float mt = wave_max(x);
          float mr = m_ref[ki * G + jj];
          float alpha = 1.0f;
          if (mt > mr + kLazy) {
            alpha = exp2f(mr - mt);
            mr = mt;
            m_ref[ki * G + jj] = mt;
          }
          const float p = exp2f(x - mr);
          l_lane[ki * G + jj] = fmaf(l_lane[ki * G + jj], alpha, p);
          if constexpr (kQ)
            reinterpret_cast<_Float16*>(p_raw)[(buf * 32 + h) * PS + lane] = (_Float16)p;
          else
            p_raw[(buf * 32 + h) * PS + lane] = p;
          if (lane == 0) {
            alpha_l[buf][h] = alpha;
            if (alpha != 1.0f) flag_l[buf] = it;
          }
        }
      }
    }
    lds_barrier();
    // ------------------------------------------------------------ values
    if (flag_l[buf] == it) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float al = alpha_l[buf][acc_row(v, lane)];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[ni][v] *= al;
        bacc[v] *= al;
      }
    }
    const bool partial = rem < kTile;
    if constexpr (kQ) {
      const _Float16* prow = reinterpret_cast<const _Float16*>(p_raw) + (buf * 32 + m) * PS + 32 * j;
      h8 A[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) A[r] = *reinterpret_cast<const h8*>(prow + 8 * r);
      const uint8_t* vt = static_cast<const uint8_t*>(a.value) + ((size_t)b * d.NT + tile) * 26 * d.rv;
      const _Float16* vm = reinterpret_cast<const _Float16*>(a.vmeta) + ((size_t)b * d.NT + tile) * 2 * GV * kTile;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int n = wave + ni * NW;
        if (n < GV) {
          uint32_t pr[16];
          if (n < NH) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(vt + (size_t)n * 1024 + (32 * j + m) * 16);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int i = 0; i < 4; ++i) pr[4 * r + i] = (w[r] >> (4 * i)) & 0x000F000Fu;
          } else {
            const uint32_t* wp = reinterpret_cast<const uint32_t*>(
                vt + (size_t)NH * 1024 + (size_t)(n - NH) * 768 + (32 * j + m) * 12);
            const uint32_t w0 = wp[0], w1 = wp[1], w2 = wp[2];
#pragma unroll
            for (int i = 0; i < 5; ++i) {
              pr[i] = (w0 >> (3 * i)) & 0x00070007u;
              pr[5 + i] = (w1 >> (3 * i)) & 0x00070007u;
              pr[10 + i] = (w2 >> (3 * i)) & 0x00070007u;
            }
            pr[15] = ((w0 >> 15) & 0x00010001u) | ((w1 >> 14) & 0x00020002u) |
                     ((w2 >> 13) & 0x00040004u);
          }
          const _Float16* sp_ = vm + (size_t)n * kTile + 32 * j;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            h8 S = *reinterpret_cast<const h8*>(sp_ + 8 * r);
            if (partial) {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (32 * j + 8 * r + e >= rem) S[e] = (_Float16)0.0f;
            }
            const h8 Ap = A[r] * S;
            const u32x4 bw = {pr[4 * r], pr[4 * r + 1], pr[4 * r + 2], pr[4 * r + 3]};
            acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ap, __builtin_bit_cast(h8, bw), acc[ni], 0, 0, 0);
          }
        }
      }
      if (wave == it % NW) {  // zero-point term P z, one wave per tile
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          h8 Z = h8{};
          if (m < GV) Z = *reinterpret_cast<const h8*>(vm + (size_t)(GV + m) * kTile + 32 * j + 8 * r);
          if (partial) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (32 * j + 8 * r + e >= rem) Z[e] = (_Float16)0.0f;
          }
          bacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[r], Z, bacc, 0, 0, 0);
        }
      }
    } else if constexpr (FMT == STARKV_CACHE_BF16) {
      const float* prow = p_raw + (buf * 32 + m) * PS + 32 * j;
      bf8 Ah[4], Al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = prow[8 * r + e];
          const __bf16 hi = (__bf16)p;
          Ah[r][e] = hi;
          Al[r][e] = (__bf16)(p - (float)hi);
        }
      const uint16_t* vbase = static_cast<const uint16_t*>(a.value);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int n = wave + ni * NW;
        if (n < GV) {
          const uint16_t* zp = vbase + (((size_t)b * d.NT + tile) * d.rv + n * 32 + m) * kTile + 32 * j;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bf8 Z = *reinterpret_cast<const bf8*>(zp + 8 * r);
            if (partial) {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (32 * j + 8 * r + e >= rem) Z[e] = (__bf16)0.0f;
            }
            acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah[r], Z, acc[ni], 0, 0, 0);
            acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al[r], Z, acc[ni], 0, 0, 0);
          }
        }
      }
    } else {
      const float* prow = p_raw + (buf * 32 + m) * PS + 32 * j;
      const float* vbase = static_cast<const float*>(a.value);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int n = wave + ni * NW;
        if (n < GV) {
          const float* zp = vbase + (((size_t)b * d.NT + tile) * d.rv + n * 32 + m) * kTile + 32 * j;
          for (int r = 0; r < 32; ++r) {
            const float z = (partial && 32 * j + r >= rem) ? 0.0f : zp[r];
            acc[ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(prow[r], z, acc[ni], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---------------------------------------------------------------- finish
  if constexpr (kQ) {
#pragma unroll
    for (int v = 0; v < 16; ++v) atomicAdd(&bias_l[acc_row(v, lane)][m], bacc[v]);
  }
  __syncthreads();
  const size_t obase = ((size_t)b * a.splits + sp) * d.Hq;
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int n = wave + ni * NW;
    if (n < GV) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = acc_row(v, lane);
        if (row < d.Hq) {
          float val = acc[ni][v];
          if constexpr (kQ) val = fmaf(val, kTwo24, bias_l[row][n]);
          a.part_o[(obase + row) * d.rv + n * 32 + m] = val;
        }
      }
    }
  }
#pragma unroll
  for (int ki = 0; ki < KVI; ++ki) {
    const int kh = wave + ki * NW;
    if (kh < d.Hkv) {
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const float l = wave_sum(l_lane[ki * G + jj]);
        if (lane == 0) {
          const int h = kh * G + jj;
          a.part_ml[(obase + h) * 2] = m_ref[ki * G + jj];
          a.part_ml[(obase + h) * 2 + 1] = l;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ merge --

__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    Dims d, int splits,
                                                    float* __restrict__ obar) {
  __shared__ float buf[1024];
  const int bh = blockIdx.x;
  const int b = bh / d.Hq, h = bh % d.Hq;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s)
    mx = fmaxf(mx, part_ml[(((size_t)b * splits + s) * d.Hq + h) * 2]);
  float L = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const size_t k = (((size_t)b * splits + s) * d.Hq + h) * 2;
    const float l = part_ml[k + 1];
    if (l > 0.0f) L += exp2f(part_ml[k] - mx) * l;
  }
  const float inv = 1.0f / L;
  for (int c = threadIdx.x; c < d.rv; c += 256) {
    float o = 0.0f;
    for (int s = 0; s < splits; ++s) {
      const size_t k = (((size_t)b * splits + s) * d.Hq + h);
      const float l = part_ml[k * 2 + 1];
      if (l > 0.0f) o = fmaf(exp2f(part_ml[k * 2] - mx), part_o[k * d.rv + c], o);
    }
    buf[c] = o * inv;
  }
  if (d.dtype == STARKV_CACHE_Q43 && d.rotate) {
    // undo the block rotation of the stored value latents: (Z H) H = Z (eq. 13)
    const int mb = pow2_divisor(d.rv / 4);
    for (int hs = 1; hs < mb; hs <<= 1) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < d.rv / 2; idx += 256) {
        const int i = (idx / hs) * 2 * hs + (idx % hs);
        const float x = buf[i], y = buf[i + hs];
        buf[i] = x + y;
        buf[i + hs] = x - y;
      }
    }
    __syncthreads();
    const float c = inv_sqrt_pow2(mb);
    for (int i = threadIdx.x; i < d.rv; i += 256) buf[i] *= c;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d.rv; c += 256) obar[(size_t)bh * d.rv + c] = buf[c];
}

// ------------------------------------------------------------------ vproj --

// out[b, h, dd] = sum_c obar[b, h, c] * B_value[g*d_h + dd, c]; one workgroup
// per (head, 16 output rows) reads those B_value rows once for every b.
template <int FMT>
__global__ __launch_bounds__(256) void vproj_kernel(const float* __restrict__ obar,
                                                    const void* __restrict__ bv,
                                                    Dims d, float* __restrict__ out) {
  const int h = blockIdx.x, g = h / d.G;
  const int r0 = blockIdx.y * 16 + (threadIdx.x & 7) * 2;
  for (int b = threadIdx.x >> 3; b < d.B; b += 32) {
    const float* ob = obar + ((size_t)b * d.Hq + h) * d.rv;
    float o0 = 0.0f, o1 = 0.0f;
    const size_t row0 = ((size_t)g * d.dh + r0) * d.rv;
    for (int c = 0; c < d.rv; c += 8) {
      const float4 x0 = *reinterpret_cast<const float4*>(ob + c);
      const float4 x1 = *reinterpret_cast<const float4*>(ob + c + 4);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      float w0[8], w1[8];
      if (FMT == STARKV_CACHE_F32) {
        const float* p0 = static_cast<const float*>(bv) + row0 + c;
        const float* p1 = p0 + d.rv;
#pragma unroll
        for (int e = 0; e < 8; ++e) { w0[e] = p0[e]; w1[e] = p1[e]; }
      } else {
        const uint4 u0 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(bv) + row0 + c);
        const uint4 u1 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(bv) + row0 + d.rv + c);
        const uint32_t a0[4] = {u0.x, u0.y, u0.z, u0.w}, a1[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w0[2 * e] = __builtin_bit_cast(float, a0[e] << 16);
          w0[2 * e + 1] = __builtin_bit_cast(float, a0[e] & 0xFFFF0000u);
          w1[2 * e] = __builtin_bit_cast(float, a1[e] << 16);
          w1[2 * e + 1] = __builtin_bit_cast(float, a1[e] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) { o0 = fmaf(xs[e], w0[e], o0); o1 = fmaf(xs[e], w1[e], o1); }
    }
    float* dst = out + ((size_t)b * d.Hq + h) * d.dh + r0;
    dst[0] = o0;
    dst[1] = o1;
  }
}

template <int FMT>
hipError_t launch_split(int G, dim3 grid, const SplitArgs& sa, hipStream_t s) {
  switch (G) {
    case 1: split_kernel<FMT, 1><<<grid, 512, 0, s>>>(sa); break;
    case 2: split_kernel<FMT, 2><<<grid, 512, 0, s>>>(sa); break;
    case 4: split_kernel<FMT, 4><<<grid, 512, 0, s>>>(sa); break;
    default: split_kernel<FMT, 8><<<grid, 512, 0, s>>>(sa); break;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t decode_fmt(const Dims& d, const starkv_cache& cache, int seq_len,
                      const void* q, const void* bk, const void* bv,
                      float sm_scale, float* out, char* ws, const DecodeWs& lay,
                      hipStream_t s) {
  void* qt = ws + lay.qt;
  float* part_o = reinterpret_cast<float*>(ws + lay.part_o);
  float* part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
  float* obar = reinterpret_cast<float*>(ws + lay.obar);
  qproj_kernel<FMT><<<d.B * d.Hq, 64, 0, s>>>(q, bk, d, sm_scale * kLog2e, qt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SplitArgs sa;
  sa.d = d;
  sa.seq_len = seq_len;
  sa.splits = lay.splits;
  const int n_tiles = (seq_len + kTile - 1) / kTile;
  sa.tiles_per_split = (n_tiles + lay.splits - 1) / lay.splits;
  sa.key = cache.key;
  sa.kmeta = static_cast<const uint16_t*>(cache.key_meta);
  sa.value = cache.value;
  sa.vmeta = static_cast<const uint16_t*>(cache.value_meta);
  sa.qt = qt;
  sa.part_o = part_o;
  sa.part_ml = part_ml;
  e = launch_split<FMT>(d.G, dim3(lay.splits, d.B), sa, s);
  if (e != hipSuccess) return e;
  merge_kernel<<<d.B * d.Hq, 256, 0, s>>>(part_o, part_ml, d, lay.splits, obar);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  vproj_kernel<FMT><<<dim3(d.Hq, d.dh / 16), 256, 0, s>>>(obar, bv, d, out);
  return hipGetLastError();
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeWs decode_ws_layout(const Dims& d, int splits) {
  DecodeWs w;
  w.splits = splits;
  size_t off = 0;
  w.qt = off;
  off += align256((size_t)d.B * d.Hq * kPlainRec * 4);
  w.part_o = off;
  off += align256((size_t)d.B * splits * d.Hq * d.rv * 4);
  w.part_ml = off;
  off += align256((size_t)d.B * splits * d.Hq * 2 * 4);
  w.obar = off;
  off += align256((size_t)d.B * d.Hq * d.rv * 4);
  w.total = off;
  return w;
}

hipError_t launch_decode(const Dims& d, const starkv_cache& cache, int seq_len,
                         const void* q, const void* bk, const void* bv,
                         float sm_scale, float* out, char* ws,
                         const DecodeWs& lay, hipStream_t s) {
  switch (d.dtype) {
    case STARKV_CACHE_F32:
      return decode_fmt<STARKV_CACHE_F32>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s);
    case STARKV_CACHE_BF16:
      return decode_fmt<STARKV_CACHE_BF16>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s);
    default:
      return decode_fmt<STARKV_CACHE_Q43>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s);
  }
}

}  // namespace starkv
