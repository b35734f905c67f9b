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
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "device.h"

namespace starkv {
namespace {


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

// ------------------------------------------------------------------ qproj --

// One workgroup per (b, h): 256 threads split the d_h contraction into
// chunks (each thread loads its q entries and factor entries together, so
// the kernel makes one round trip to memory), the chunks are summed, then
// wave 0 rotates, scales and packs the record.
// A Q43 record holds the 17 fp16 pairs that meet the in-place code fields of
// the key words (each entry times 2^-p for a field at bit p; channel 31
// split over three one-bit fields), then sum(q_hi) 2^-24 and
// sum(q_lo) 2^-24 as fp32.
template <int FMT>
__global__ __launch_bounds__(256) void qproj_kernel(const void* __restrict__ q,
                                                    const void* __restrict__ bk,
                                                    Dims d, float qscale,
                                                    void* __restrict__ qt) {
  __shared__ float part[256];
  __shared__ _Float16 sq[32];
  const int bh = blockIdx.x;
  const int g = (bh % d.Hq) / d.G;
  const int t = threadIdx.x;
  const size_t qrow = (size_t)bh * d.dh;
  const int rkp = d.rk <= 32 ? 32 : 64;
  const int c = t % rkp, chunk = t / rkp, nch = 256 / rkp;
  const int klen = (d.dh + nch - 1) / nch;
  float acc = 0.0f;
  if (c < d.rk) {
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
    static_cast<float*>(qt)[(size_t)bh * kPlainRec + t] = t < d.rk ? v : 0.0f;
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
    if (t < 4) {
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
    rec[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
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

// ---------------------------------------------------- fp32 / bf16 split --

// Scores of one 64-token tile for the G query heads of KV head kh from an
// unquantized cache; lane = token, the key row (RK channels, of which the
// first d.rk are real) loaded whole, query records read from LDS.
template <int FMT, int G, int RK>
__device__ inline void score_tile_plain(const SplitArgs& a, const float* qrec,
                                        int b, int kh, int tile, int lane,
                                        float* sc) {
  const Dims& d = a.d;
  // chunk c of this token's key row: [b][kh][tile][c][lane][8 channels]
  const size_t row0 = (((size_t)b * d.Hkv + kh) * d.NT + tile) * (d.rk / 8) * (kTile * 8) + lane * 8;
  // the record offset is made opaque per call so the records are read from
  // LDS where they are used instead of being held in registers across tiles
  int rec_off = kh * G * kPlainRec;
  __asm__ volatile("" : "+s"(rec_off));
  const float* recs = qrec + rec_off;
  constexpr int NC = RK / 8;              // 8-channel chunks
  constexpr int CW = FMT == STARKV_CACHE_F32 ? 8 : 4;   // dwords per chunk
  if constexpr (G * RK > 64) {
    // many heads per key row: one chunk at a time, all G products per chunk
    float acc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.0f;
#pragma unroll 1
    for (int c = 0; c < NC && 8 * c < d.rk; ++c) {
      float z[8];
      const size_t row = row0 + (size_t)c * (kTile * 8);
      if constexpr (FMT == STARKV_CACHE_F32) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.key) + row);
        const u32x4 u = __builtin_nontemporal_load(p), v = __builtin_nontemporal_load(p + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // vector elements go through scalars before the bit-cast (a
          // bit-cast of an ext_vector element is lowered as one of element 0)
          const uint32_t wu = u[e], wv = v[e];
          z[e] = __builtin_bit_cast(float, wu);
          z[4 + e] = __builtin_bit_cast(float, wv);
        }
      } else {
        const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            static_cast<const uint16_t*>(a.key) + row));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = u[e];
          z[2 * e] = __builtin_bit_cast(float, w << 16);
          z[2 * e + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j] = fmaf(recs[j * kPlainRec + 8 * c + e], z[e], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) sc[j] = acc[j];
    return;
  }
  uint32_t kw[NC][CW];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    // chunks past r_k (when RK rounds it up) are neither read nor used
    const bool live = 8 * c < d.rk;
    const size_t row = row0 + (size_t)(live ? c : 0) * (kTile * 8);
    if constexpr (FMT == STARKV_CACHE_F32) {
      const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.key) + row);
      const u32x4 u = live ? __builtin_nontemporal_load(p) : u32x4{};
      const u32x4 v = live ? __builtin_nontemporal_load(p + 1) : u32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kw[c][e] = u[e];
        kw[c][4 + e] = v[e];
      }
    } else {
      const u32x4 u = live ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                 static_cast<const uint16_t*>(a.key) + row))
                           : u32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) kw[c][e] = u[e];
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    // one head at a time: its record is read right before its products
    __builtin_amdgcn_sched_barrier(0);
    const float* qr = recs + j * kPlainRec;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float z;
        if constexpr (FMT == STARKV_CACHE_F32) z = __builtin_bit_cast(float, kw[c][e]);
        else z = __builtin_bit_cast(float, (e & 1) ? kw[c][e >> 1] & 0xFFFF0000u
                                                   : kw[c][e >> 1] << 16);
        acc = fmaf(qr[8 * c + e], z, acc);
      }
    sc[j] = acc;
  }
}

// Online-softmax update of one query head over one tile (lane = token):
// the reference max moves only when a score exceeds it by more than 2^kLazy,
// decided by a wave vote, so the common tile needs no reduction.
__device__ inline float softmax_step(float x, float& mr, float& l, float& alpha,
                                     bool& moved) {
  alpha = 1.0f;
  moved = false;
  if (__builtin_amdgcn_ballot_w64(x > mr + kLazy) != 0) {
    const float mt = wave_max(x);
    alpha = exp2f(mr - mt);
    mr = mt;
    l *= alpha;
    moved = true;
  }
  const float p = exp2f(x - mr);
  l += p;
  return p;
}

// Split kernel for unquantized caches: 8 waves, each scores KVI KV heads
// (lane = token) and then contracts NI value groups (32 channels each) with
// the stacked-head P tile on MFMA.  A tile's value operands are requested
// before its scores are computed, so both streams are in flight together.
// bf16 caches write fp16 partial rows divided by their own l; fp32 caches
// write unnormalised fp32 rows.
template <int FMT, int G, int RK>
__global__ __launch_bounds__(512) void split_kernel(SplitArgs a) {
  constexpr int NW = kDecodeWaves;
  constexpr int KVI = G >= 4 ? 1 : 4 / G;  // KV heads per wave (Hq <= 32)
  constexpr int NI = kMaxQHeads * 32 / 32 / NW;   // value groups per wave (R_v <= 1024)
  constexpr int PS = 68;                    // P row stride (floats)
  constexpr bool kBF = FMT == STARKV_CACHE_BF16;
  // bf16 value operands requested before the scores where registers allow
  // (one query head per KV head, key rows of <= 32 channels); else at use
  constexpr bool kPreV = kBF && G == 1 && RK <= 32;
  const Dims& d = a.d;

  __shared__ __attribute__((aligned(16))) float p_raw[2 * 32 * PS];
  __shared__ __attribute__((aligned(16))) float qrec[32 * kPlainRec];
  __shared__ float alpha_l[2][32];
  __shared__ int flag_l[2];
  __shared__ float l_row[32];
  // bf16 caches: per-wave staging of the fp16 partial rows (32 rows of the
  // wave's NI groups, padded rows) for 16-byte stores
  constexpr int kStg = kBF ? NI * 32 + 8 : 8;
  __shared__ __attribute__((aligned(16))) _Float16 stg[kBF ? NW : 1][32][kStg];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int b = blockIdx.y, sp = blockIdx.x;
  const int n_tiles = (a.seq_len + kTile - 1) / kTile;
  const int tile0 = sp * a.tiles_per_split;
  const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);
  const int GV = d.rv / 32;

  for (int i = tid; i < 2 * 32 * PS; i += 512) p_raw[i] = 0.0f;
  for (int i = tid; i < d.Hq * kPlainRec; i += 512)
    qrec[i] = static_cast<const float*>(a.qt)[(size_t)b * d.Hq * kPlainRec + i];
  if (tid < 64) alpha_l[tid >> 5][tid & 31] = 1.0f;
  if (tid < 2) flag_l[tid] = -1;
  __syncthreads();

  float m_ref[KVI * G], l_lane[KVI * G];
#pragma unroll
  for (int i = 0; i < KVI * G; ++i) { m_ref[i] = -INFINITY; l_lane[i] = 0.0f; }
  f32x16 acc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) acc[i] = f32x16{};
  const int j = lane >> 5, m = lane & 31;

  for (int tile = tile0, it = 0; tile < tile1; ++tile, ++it) {
    const int buf = it & 1;
    const int rem = a.seq_len - tile * kTile;
    const bool valid = lane < rem;
    const bool partial = rem < kTile;
    // value operands of this tile (bf16): 4 K-steps of 8 tokens per group
    bf8 Zv[NI][4];
    auto load_values = [&]() {
      const uint16_t* vbase = static_cast<const uint16_t*>(a.value);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int n = wave + ni * NW;
        // K-step r, lane half j: tokens 16r + 8j .. +7 = token block 2r + j
        const uint16_t* zp =
            vbase + (((size_t)b * d.NT + tile) * GV + min(n, GV - 1)) * (8 * 256) + (j * 32 + m) * 8;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Zv[ni][r] = n < GV ? __builtin_nontemporal_load(reinterpret_cast<const bf8*>(zp + r * 512))
                             : bf8{};
      }
    };
    if constexpr (kPreV) load_values();
#pragma unroll
    for (int ki = 0; ki < KVI; ++ki) {
      const int kh = wave + ki * NW;
      if (kh < d.Hkv) {
        float sc[G];
        score_tile_plain<FMT, G, RK>(a, qrec, b, kh, tile, lane, sc);
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
          const int h = kh * G + jj;
          float alpha;
          bool moved;
          const float p = softmax_step(valid ? sc[jj] : -INFINITY, m_ref[ki * G + jj],
                                       l_lane[ki * G + jj], alpha, moved);
          p_raw[(buf * 32 + h) * PS + lane] = p;
          if (lane == 0) {
            alpha_l[buf][h] = alpha;
            if (moved) flag_l[buf] = it;
          }
        }
      }
    }
    lds_barrier();
    if (flag_l[buf] == it) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float al = alpha_l[buf][acc_row(v, lane)];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[ni][v] *= al;
      }
    }
    if constexpr (kBF) {
      if constexpr (!kPreV) load_values();
      const float* prow = p_raw + (buf * 32 + m) * PS + 8 * j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // P as bf16 high and low parts (two products per K-step); K-step r,
        // lane half j covers tokens 16r + 8j .. +7
        bf8 Ah, Al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = prow[16 * r + e];
          const __bf16 hi = (__bf16)p;
          Ah[e] = hi;
          Al[e] = (__bf16)(p - (float)hi);
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int n = wave + ni * NW;
          if (n < GV) {
            bf8 Z = Zv[ni][r];
            if (partial) {
              // unused cache slots never reach the operands
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (16 * r + 8 * j + e >= rem) Z[e] = (__bf16)0.0f;
            }
            acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Z, acc[ni], 0, 0, 0);
            acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al, Z, acc[ni], 0, 0, 0);
          }
        }
      }
    } else {
      // fp32 products, K = 2: step r, lane half j is token 32j + r
      const float* prow = p_raw + (buf * 32 + m) * PS + 32 * j;
      const float* vbase = static_cast<const float*>(a.value);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int n = wave + ni * NW;
        if (n < GV) {
          const float* zp = vbase + (((size_t)b * d.NT + tile) * GV + n) * (8 * 256) + m * 8;
          for (int r = 0; r < 32; ++r) {
            const int u = 32 * j + r;
            const float z = (partial && u >= rem) ? 0.0f : zp[(u >> 3) * 256 + (u & 7)];
            acc[ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(prow[r], z, acc[ni], 0, 0, 0);
          }
        }
      }
    }
  }

  const size_t obase = ((size_t)b * a.splits + sp) * d.Hq;
#pragma unroll
  for (int ki = 0; ki < KVI; ++ki) {
    const int kh = wave + ki * NW;
    if (kh < d.Hkv) {
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        const float l = wave_sum(l_lane[ki * G + jj]);
        if (lane == 0) {
          const int h = kh * G + jj;
          l_row[h] = l;
          a.part_ml[(obase + h) * 2] = m_ref[ki * G + jj];
          a.part_ml[(obase + h) * 2 + 1] = l;
        }
      }
    }
  }
  lds_barrier();   // l of every head
  if constexpr (kBF) {
    // rows divided by their l, as fp16, through LDS into 16-byte streaming
    // stores of whole 32-channel group segments
    float inv_l[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float l = l_row[acc_row(v, lane)];
      inv_l[v] = l > 0.0f ? __builtin_amdgcn_rcpf(l) : 0.0f;   // rows go out as fp16
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        stg[wave][acc_row(v, lane)][ni * 32 + m] = (_Float16)(acc[ni][v] * inv_l[v]);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): own staging writes done
    __builtin_amdgcn_wave_barrier();
    _Float16* po = reinterpret_cast<_Float16*>(a.part_o);
#pragma unroll
    for (int k = 0; k < 32 * NI * 4 / 64; ++k) {
      const int c = lane + 64 * k;
      const int row = c / (NI * 4), q = c % (NI * 4);
      const int ni = q >> 2, part = q & 3;
      const int n = wave + ni * NW;
      if (row < d.Hq && n < GV) {
        const h8 o = *reinterpret_cast<const h8*>(&stg[wave][row][ni * 32 + part * 8]);
        __builtin_nontemporal_store(o, reinterpret_cast<h8*>(po + (obase + row) * d.rv + n * 32 + part * 8));
      }
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = wave + ni * NW;
      if (n < GV) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = acc_row(v, lane);
          if (row < d.Hq) a.part_o[(obase + row) * d.rv + n * 32 + m] = acc[ni][v];
        }
      }
    }
  }
}

// ------------------------------------------------------------- Q43 split --

// s_waitcnt vmcnt(N) for a compile-time N.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Copy `bytes` from global to LDS with one wave: direct-to-LDS loads, 1 KB
// per instruction, always ceil(bytes / 1024) instructions.  The cache is read
// exactly once per call, so the loads are non-temporal: streaming past L2 and
// the Infinity Cache measures ~1.5x the bandwidth of cache-allocating loads.
__device__ inline void wave_dma(const uint8_t* src, uint8_t* lds_dst, int bytes, int lane) {
  for (int k = 0; k * 1024 < bytes; ++k) {
    const int off = k * 1024 + lane * 16;
    if (off < bytes)
      __builtin_amdgcn_global_load_lds(
          src + off, (__attribute__((address_space(3))) void*)(lds_dst + k * 1024), 16, 0,
          kNonTemporal);
  }
}

constexpr int kValueSlots = 4;     // LDS ring slots per value wave
constexpr int kValueAhead = kValueSlots - 1;   // tiles staged ahead of use
// Value ring of a kernel whose value waves own NIV groups each (R_v = 128 NIV,
// NIV <= 8); sized per NIV so that small value ranks leave room for a second
// workgroup on the compute unit.
// one slot: the 4-bit wave's codes + scales + zeros, then the three 3-bit
// waves' (1024 + 128 + 128 and 768 + 128 + 128 bytes per group)
constexpr int hi_region(int niv) { return niv * 1280; }
constexpr int lo_region(int niv) { return niv * 1024; }
constexpr int slot_bytes(int niv) { return hi_region(niv) + 3 * lo_region(niv); }
// fp32 row stride of the epilogue's per-wave staging of partial rows (kept
// in the value ring): 32 rows of 32 NIV columns, padded so the two row halves
// a store instruction writes fall in different LDS banks
constexpr int stage_row(int niv) { return niv * 32 + 8; }
constexpr int ring_bytes(int niv) {
  return kValueSlots * slot_bytes(niv) > 4 * 32 * stage_row(niv) * 4
             ? kValueSlots * slot_bytes(niv)
             : 4 * 32 * stage_row(niv) * 4;
}

// Q43 split kernel, warp-specialized.  Workgroup = (sequence b, token split),
// 8 waves; waves w and w+4 share a SIMD.
//   score waves 0-3: wave s owns KV heads s, s+4, ... (KVS of them); lane =
//     token; key codes (loaded two barrier periods ahead into alternating
//     register sets) are read in place as fp16 pairs (one AND per field
//     pair, the field weights carried by the query record) and meet the
//     query pairs in v_dot2_f32_f16; p = exp2(score - m_ref) goes to a
//     2-slot LDS ring as the stacked-head P tile (32 rows, fp16).
//   value waves 4-7: wave v owns the NIV value groups v*NIV .. v*NIV+NIV-1
//     (32 channels each, one MFMA column tile); since R_v/4 channels are
//     4-bit, value wave 0 holds exactly the 4-bit groups.  Each value wave
//     streams its own groups' codes, scales and zeros into a private 4-slot
//     LDS ring (direct-to-LDS, non-temporal) three tiles ahead, so it waits
//     on its own loads only.  A = P * scale in fp16, B = codes as fp16
//     subnormals, mfma 32x32x16; P x zero adds the zero points, and a column
//     of ones in that product gives each head's exp-sum l.
// One barrier per tile hands P over: while the value waves contract tile t,
// the score waves already score tile t+1.
template <int G, int KVS, int NIV>
__global__ __launch_bounds__(512) void split_q43_kernel(SplitArgs a) {
  constexpr int PS = 72;                        // P row stride (halves)
  constexpr bool kFourW0 = true;                // value wave 0: 4-bit groups
  constexpr int kDmaHi = NIV + 2 * ((NIV * 128 + 1023) / 1024);
  constexpr int kDmaLo = (NIV * 768 + 1023) / 1024 + 2 * ((NIV * 128 + 1023) / 1024);
  (void)kFourW0;
  const Dims& d = a.d;

  constexpr int kHiRegion = hi_region(NIV), kLoRegion = lo_region(NIV);
  constexpr int kSlotBytes = slot_bytes(NIV), kStageRow = stage_row(NIV);
  __shared__ __attribute__((aligned(16))) uint8_t vring[ring_bytes(NIV)];
  __shared__ __attribute__((aligned(16))) _Float16 p_l[2][32 * PS];
  __shared__ __attribute__((aligned(16))) uint32_t qrec[kMaxQHeads * kQ43Rec];
  __shared__ float alpha_l[2][32];
  __shared__ int flag_l[2];
  __shared__ float bias_l[32][33];
  __shared__ float l_row[32];
  __shared__ __attribute__((aligned(16))) _Float16 zo_l[2 * kTile];   // zeros, then ones

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int b = blockIdx.y, sp = blockIdx.x;
  const int n_tiles = (a.seq_len + kTile - 1) / kTile;
  const int tile0 = sp * a.tiles_per_split;
  const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);
  const int GV = 4 * NIV;            // value groups
  const int NH = NIV;                // 4-bit value groups
  // Two workgroups share a compute unit when R_v is small, and issue
  // arbitration favours the older one; the grid's second half (which lands
  // as the second workgroup of each unit) runs at the higher wave priority.
  if ((blockIdx.y * gridDim.x + blockIdx.x) >= (gridDim.x * gridDim.y) / 2)
    __builtin_amdgcn_s_setprio(1);
  const int j = lane >> 5, m = lane & 31;

  for (int i = tid; i < 2 * 32 * PS / 8; i += 512) reinterpret_cast<h8*>(&p_l[0][0])[i] = h8{};
  for (int i = tid; i < d.Hq * kQ43Rec; i += 512)
    qrec[i] = static_cast<const uint32_t*>(a.qt)[(size_t)b * d.Hq * kQ43Rec + i];
  if (tid < 64) alpha_l[tid >> 5][tid & 31] = 1.0f;
  if (tid < 2) flag_l[tid] = -1;
  for (int i = tid; i < 32 * 33; i += 512) (&bias_l[0][0])[i] = 0.0f;
  if (tid < 32) l_row[tid] = 1.0f;
  if (tid < 2 * kTile) zo_l[tid] = tid < kTile ? (_Float16)0.0f : (_Float16)1.0f;
  __syncthreads();

  const size_t obase = ((size_t)b * a.splits + sp) * d.Hq;

  if (wave < 4) {
    // ================================================================ scores
    const int sw = wave;
    const bool has_keys = sw < d.Hkv;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.key);
    const u32x2* kmeta = reinterpret_cast<const u32x2*>(a.kmeta);
    uint32_t kA[KVS][6], kB[KVS][6];
    auto load_keys = [&](int tile, uint32_t (&dst)[KVS][6]) {
#pragma unroll
      for (int ki = 0; ki < KVS; ++ki) {
        const int kh = sw + ki * 4;
        const size_t blk = ((size_t)b * d.NT + tile) * d.Hkv + kh;
        const uint8_t* kb = kbase + blk * kKeyBlock;
        dst[ki][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb) + lane);
        dst[ki][1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 256) + lane);
        dst[ki][2] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 512) + lane);
        dst[ki][3] = __builtin_nontemporal_load(kb + 768 + lane);
        const u32x2 mt = __builtin_nontemporal_load(kmeta + blk * kTile + lane);
        dst[ki][4] = mt[0];
        dst[ki][5] = mt[1];
      }
    };
    // m_ref: reference max (log2 units); thr = (m_ref + kLazyQ43) 2^-24, the
    // move threshold in the 2^-24 units the scores come in
    float m_ref[KVS * G], thr[KVS * G];
#pragma unroll
    for (int i = 0; i < KVS * G; ++i) {
      m_ref[i] = -INFINITY;
      thr[i] = -INFINITY;
    }
    // Groups of 4 or more query heads per KV head score on MFMA 4x4x4 (16
    // blocks of 4 tokens): B = the lane's own key fields (column = token),
    // A = the query records read from LDS (row = query head; lane 4b + i
    // reads head i of a set of 4), so that a lane receives its token's
    // scores of the 4 heads in 4 registers.  K step s takes field pairs 2s,
    // 2s + 1: steps 0-1 the 4-bit part, steps 2-8 the 3-bit part (pair 17
    // is zero on both sides).
    constexpr int kSets = G >= 4 ? G / 4 : 0;
    constexpr int kSetsA = kSets > 0 ? kSets : 1;
    typedef _Float16 h4v __attribute__((ext_vector_type(4)));
    float qsh[KVS][kSetsA][4], qsl[KVS][kSetsA][4];
    if constexpr (kSets > 0) {
#pragma unroll
      for (int ki = 0; ki < KVS; ++ki)
#pragma unroll
        for (int st = 0; st < kSets; ++st)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t* rv = qrec + ((sw + ki * 4) * G + st * 4 + v) * kQ43Rec;
            qsh[ki][st][v] = __builtin_bit_cast(float, rv[17]);
            qsl[ki][st][v] = __builtin_bit_cast(float, rv[18]);
          }
    }

    // scores of tile `tile` into P slot `slot`; `it` = its index in the split
    auto score = [&](int tile, int it, int slot, const uint32_t (&kc)[KVS][6]) {
      const int rem = a.seq_len - tile * kTile;
      const bool valid = lane < rem;
      float x[KVS * G];   // scores times 2^-24
#pragma unroll
      for (int ki = 0; ki < KVS; ++ki) {
        const KeyLane kl = unpack_key_lane(kc[ki]);
        if constexpr (kSets > 0) {
          const h2 mh = __builtin_bit_cast(h2, kl.mhi), ml = __builtin_bit_cast(h2, kl.mlo);
#pragma unroll
          for (int st = 0; st < kSets; ++st) {
            const uint32_t* rq = qrec + ((sw + ki * 4) * G + st * 4 + (lane & 3)) * kQ43Rec;
            f32x4 dh = {0.0f, 0.0f, 0.0f, 0.0f}, dl = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < 9; ++k) {
              const h4v qa = __builtin_bit_cast(
                  h4v, k < 8 ? *reinterpret_cast<const u32x2*>(rq + 2 * k) : u32x2{rq[16], 0u});
              const h4v kb = __builtin_bit_cast(
                  h4v, u32x2{kl.pr[2 * k], k < 8 ? kl.pr[2 * k + 1] : 0u});
              if (k < 2) dh = __builtin_amdgcn_mfma_f32_4x4x4f16(qa, kb, dh, 0, 0, 0);
              else dl = __builtin_amdgcn_mfma_f32_4x4x4f16(qa, kb, dl, 0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float sc =
                  fmaf((float)mh[0], dh[v],
                       fmaf((float)ml[0], dl[v],
                            fmaf((float)mh[1], qsh[ki][st][v], (float)ml[1] * qsl[ki][st][v])));
              x[ki * G + st * 4 + v] = valid ? sc : -INFINITY;
            }
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < G; ++jj) {
            const float sc = key_score(kl, qrec + ((sw + ki * 4) * G + jj) * kQ43Rec);
            x[ki * G + jj] = valid ? sc : -INFINITY;
          }
        }
      }
      bool big = false;
#pragma unroll
      for (int i = 0; i < KVS * G; ++i) big |= x[i] > thr[i];
      if (__builtin_amdgcn_ballot_w64(big) != 0) {
        // rare: some head's reference max must move up
#pragma unroll
        for (int i = 0; i < KVS * G; ++i) {
          const int h = (sw + (i / G) * 4) * G + (i % G);
          float alpha = 1.0f;
          if (__builtin_amdgcn_ballot_w64(x[i] > thr[i]) != 0) {
            const float mt = wave_max(x[i]) * kTwo24;
            alpha = exp2f(m_ref[i] - mt);
            m_ref[i] = mt;
            thr[i] = (mt + kLazyQ43) * (1.0f / kTwo24);
            if (lane == 0) flag_l[slot] = it;
          }
          if (lane == 0) alpha_l[slot][h] = alpha;
        }
      } else if (lane < KVS * G) {
        const int i = lane;
        alpha_l[slot][(sw + (i / G) * 4) * G + (i % G)] = 1.0f;
      }
#pragma unroll
      for (int i = 0; i < KVS * G; ++i) {
        const int h = (sw + (i / G) * 4) * G + (i % G);
        const float p = __builtin_amdgcn_exp2f(fmaf(x[i], kTwo24, -m_ref[i]));
        p_l[slot][h * PS + lane] = (_Float16)p;
      }
    };

    // Keys alternate between two register sets (tile tile0 + k in set k & 1):
    // iteration it scores tile tile0 + it + 1 and refills its set with tile
    // tile0 + it + 3, so codes arrive two barrier periods before use.  One
    // barrier per iteration, as in the value waves.
    const int n_it = tile1 - tile0;
    if (n_it > 0 && has_keys) {
      load_keys(tile0, kA);
      if (n_it > 1) load_keys(tile0 + 1, kB);
      score(tile0, 0, 0, kA);
      if (n_it > 2) load_keys(tile0 + 2, kA);
    }
    lds_barrier();
    for (int it = 0; it < n_it; it += 2) {
      if (it + 1 < n_it && has_keys) {
        score(tile0 + it + 1, it + 1, (it + 1) & 1, kB);
        if (it + 3 < n_it) load_keys(tile0 + it + 3, kB);
      }
      lds_barrier();
      if (it + 1 >= n_it) break;
      if (it + 2 < n_it && has_keys) {
        score(tile0 + it + 2, it + 2, (it + 2) & 1, kA);
        if (it + 4 < n_it) load_keys(tile0 + it + 4, kA);
      }
      lds_barrier();
    }
    // the running max of each head; its exp-sum l comes out of the value
    // waves' zero-point product (a column of ones)
    if (has_keys && lane == 0) {
#pragma unroll
      for (int i = 0; i < KVS * G; ++i) {
        const int h = (sw + (i / G) * 4) * G + (i % G);
        a.part_ml[(obase + h) * 2] = m_ref[i];
      }
    }
    // the value waves add their zero-point terms and l; the (m, l) stores
    // need not complete before the barrier, so it waits on LDS only
    lds_barrier();
  } else {
    // ================================================================ values
    const int vw = wave - 4;
    const int n0 = vw * NIV;                 // first value group of this wave
    const bool four = vw == 0;
    const int code_bytes = NIV * (four ? 1024 : 768);
    const int code_off = four ? 0 : NH * 1024 + (n0 - NH) * 768;
    const int meta_bytes = NIV * kTile * 2;   // one plane of this wave's groups
    const uint8_t* vbase = static_cast<const uint8_t*>(a.value);
    const uint8_t* vmbase = reinterpret_cast<const uint8_t*>(a.vmeta);
    const size_t tile_bytes = (size_t)26 * 32 * GV;
    const size_t meta_tile = (size_t)2 * GV * kTile * 2;
    uint8_t* ring = vring + (four ? 0 : kHiRegion + (vw - 1) * kLoRegion);

    auto stage = [&](int tile, int slot) {
      const size_t t = (size_t)b * d.NT + tile;
      uint8_t* dst = ring + slot * kSlotBytes;
      wave_dma(vbase + t * tile_bytes + code_off, dst, code_bytes, lane);
      wave_dma(vmbase + t * meta_tile + (size_t)n0 * kTile * 2, dst + code_bytes, meta_bytes, lane);
      wave_dma(vmbase + t * meta_tile + (size_t)(GV + n0) * kTile * 2,
               dst + code_bytes + meta_bytes, meta_bytes, lane);
    };
    // The whole tile loop is instantiated once per code width so that the
    // accumulators of the two variants never meet in one live range.
    auto run_values = [&](auto fourc) {
    constexpr bool kFour = decltype(fourc)::value;
    f32x16 acc[NIV];
#pragma unroll
    for (int i = 0; i < NIV; ++i) acc[i] = f32x16{};
    f32x16 bacc = f32x16{};

    for (int k = 0; k < kValueAhead && tile0 + k < tile1; ++k) stage(tile0 + k, k);
    lds_barrier();      // P of the first tile is ready
    for (int tile = tile0, it = 0; tile < tile1; ++tile, ++it) {
      const int pslot = it & 1;
      const int vslot = it % kValueSlots;
      if (tile + kValueAhead < tile1) stage(tile + kValueAhead, (it + kValueAhead) % kValueSlots);
      // wait for this tile's stage: the later stages may stay in flight
      constexpr int kDma = kFour ? kDmaHi : kDmaLo;
      switch (min(kValueAhead, tile1 - 1 - tile)) {
        case 3: wait_vmcnt<3 * kDma>(); break;
        case 2: wait_vmcnt<2 * kDma>(); break;
        case 1: wait_vmcnt<kDma>(); break;
        default: wait_vmcnt<0>(); break;
      }
      uint8_t* vt = ring + vslot * kSlotBytes;
      _Float16* sc_l = reinterpret_cast<_Float16*>(vt + code_bytes);
      _Float16* zr_l = sc_l + NIV * kTile;
      const int rem = a.seq_len - tile * kTile;
      if (rem < kTile) {
        // last, partial tile: zero the missing tokens' scales and zeros so
        // unused cache bytes never reach the MFMA operands
        for (int i = lane; i < 2 * NIV * kTile; i += 64)
          if ((i & (kTile - 1)) >= rem) sc_l[i] = (_Float16)0.0f;
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
      }
      if (flag_l[pslot] == it) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float al = alpha_l[pslot][acc_row(v, lane)];
#pragma unroll
          for (int ni = 0; ni < NIV; ++ni) acc[ni][v] *= al;
          bacc[v] *= al;
        }
      }
      const _Float16* prow = &p_l[pslot][m * PS + 32 * j];
      h8 A[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) A[r] = *reinterpret_cast<const h8*>(prow + 8 * r);
      // zero points of this wave's groups: columns n0 .. n0+NIV-1; the
      // 4-bit wave (n0 = 0) also sums P into column NIV: l of every head,
      // rescaled with the accumulators and made of the same fp16 P
      // (other columns read a row of zeros: no masked loads)
      {
        const bool zcol = m >= n0 && m < n0 + NIV;
        const _Float16* zsrc = zcol ? zr_l + (m - n0) * kTile
                                    : (kFour && m == NIV) ? zo_l + kTile : zo_l;
        h8 Z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) Z[r] = *reinterpret_cast<const h8*>(zsrc + 32 * j + 8 * r);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          bacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[r], Z[r], bacc, 0, 0, 0);
      }
      // P times the in-place field weights of the token pairs of step r
      // (powers of two: exact); shared by all groups of the wave
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        h8 F;
#pragma unroll
        for (int e = 0; e < 8; ++e) F[e] = (_Float16)run_pair_weight<kFour>(4 * r + e / 2);
        A[r] = A[r] * F;
      }
      {
        // two column tiles at a time: their MFMAs are independent
#pragma unroll
        for (int n2 = 0; n2 < NIV; n2 += 2) {
          u32x4 W[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int ni = n2 + q;
            if constexpr (kFour) {
              W[q] = *reinterpret_cast<const u32x4*>(vt + ni * 1024 + (32 * j + m) * 16);
            } else {
              const uint32_t* wp = reinterpret_cast<const uint32_t*>(vt + ni * 768 + (32 * j + m) * 12);
              W[q] = u32x4{wp[0], wp[1], wp[2], 0u};
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int ni = n2 + q;
              const h8 S = *reinterpret_cast<const h8*>(sc_l + ni * kTile + 32 * j + 8 * r);
              const u32x4 bw = {run_pair_inplace<kFour>(W[q], 4 * r),
                                run_pair_inplace<kFour>(W[q], 4 * r + 1),
                                run_pair_inplace<kFour>(W[q], 4 * r + 2),
                                run_pair_inplace<kFour>(W[q], 4 * r + 3)};
              acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[r] * S, __builtin_bit_cast(h8, bw),
                                                              acc[ni], 0, 0, 0);
            }
          }
        }
      }
      lds_barrier();
    }
    // zero-point sums of this wave's own columns: one writer per entry
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (m >= n0 && m < n0 + NIV) bias_l[acc_row(v, lane)][m] = bacc[v];
    if (kFour && m == NIV) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = acc_row(v, lane);
        l_row[row] = bacc[v];
        if (row < d.Hq) a.part_ml[(obase + row) * 2 + 1] = bacc[v];
      }
    }
    // bias and l complete; no wave uses the value ring any more (every stage
    // was waited for in the last iteration)
    lds_barrier();
    // The partial rows, divided by their l (so that fp16 holds them), go
    // out through LDS (this wave's region of the ring) as 16-byte stores of
    // whole row segments instead of 2-byte scatters.
    float* st = reinterpret_cast<float*>(vring) + vw * 32 * kStageRow;
    float inv_l[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float l = l_row[acc_row(v, lane)];
      inv_l[v] = l > 0.0f ? __builtin_amdgcn_rcpf(l) : 0.0f;   // rows go out as fp16
    }
#pragma unroll
    for (int ni = 0; ni < NIV; ++ni) {
      const int n = n0 + ni;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = acc_row(v, lane);
        // products came in units of 2^-20 (4-bit runs) or 2^-18 (3-bit)
        st[row * kStageRow + ni * 32 + m] =
            fmaf(acc[ni][v], kFour ? 1048576.0f : 262144.0f, bias_l[row][n]) * inv_l[v];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): own staging writes done
    __builtin_amdgcn_wave_barrier();
    constexpr int kChunks = NIV * 4;       // 16-byte (8 x fp16) chunks per row segment
    _Float16* po = reinterpret_cast<_Float16*>(a.part_o);
    for (int c = lane; c < 32 * kChunks; c += 64) {
      const int row = c / kChunks, k = c % kChunks;
      if (row < d.Hq) {
        const float4 x0 = *reinterpret_cast<const float4*>(st + row * kStageRow + 8 * k);
        const float4 x1 = *reinterpret_cast<const float4*>(st + row * kStageRow + 8 * k + 4);
        const h8 o = {(_Float16)x0.x, (_Float16)x0.y, (_Float16)x0.z, (_Float16)x0.w,
                      (_Float16)x1.x, (_Float16)x1.y, (_Float16)x1.z, (_Float16)x1.w};
        // streaming stores: the partials are read once, by the merge
        __builtin_nontemporal_store(o, reinterpret_cast<h8*>(po + (obase + row) * d.rv + n0 * 32 + 8 * k));
      }
    }
    };
    if (four) run_values(std::true_type{});
    else run_values(std::false_type{});
  }
}

// The Q43 split kernel for a shape: G query heads per KV head, KVS KV heads
// per score wave, NIV value groups per value wave.
using SplitFn = void (*)(SplitArgs);

template <int G, int KVS>
SplitFn q43_kernel_niv(int NIV) {
  switch (NIV) {
    case 2: return split_q43_kernel<G, KVS, 2>;
    case 4: return split_q43_kernel<G, KVS, 4>;
    case 6: return split_q43_kernel<G, KVS, 6>;
    case 8: return split_q43_kernel<G, KVS, 8>;
    default: return nullptr;
  }
}

SplitFn q43_kernel(const Dims& d) {
  const int NIV = d.rv / 128;
  const int KVS = d.Hkv >= 4 ? d.Hkv / 4 : 1;
  switch (d.G * 16 + KVS) {
    case 1 * 16 + 1: return q43_kernel_niv<1, 1>(NIV);
    case 1 * 16 + 2: return q43_kernel_niv<1, 2>(NIV);
    case 1 * 16 + 4: return q43_kernel_niv<1, 4>(NIV);
    case 1 * 16 + 8: return q43_kernel_niv<1, 8>(NIV);
    case 2 * 16 + 1: return q43_kernel_niv<2, 1>(NIV);
    case 2 * 16 + 2: return q43_kernel_niv<2, 2>(NIV);
    case 2 * 16 + 4: return q43_kernel_niv<2, 4>(NIV);
    case 4 * 16 + 1: return q43_kernel_niv<4, 1>(NIV);
    case 4 * 16 + 2: return q43_kernel_niv<4, 2>(NIV);
    case 8 * 16 + 1: return q43_kernel_niv<8, 1>(NIV);
    default: return nullptr;
  }
}

hipError_t launch_q43(const Dims& d, dim3 grid, const SplitArgs& sa, hipStream_t s) {
  const SplitFn k = q43_kernel(d);
  if (!k) return hipErrorNotSupported;
  hipLaunchKernelGGL(k, grid, dim3(512), 0, s, sa);
  return hipGetLastError();
}

// ------------------------------------------------------------------ merge --

// 4 consecutive partial values as fp32 (fp32 partials: one 16-byte load;
// fp16 partials: one 8-byte load).
__device__ inline float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline float4 load4(const _Float16* p) {
  // the partials are read exactly once
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  // element picks go through scalars: a bit-cast applied directly to an
  // ext_vector element is lowered as a cast of element 0
  const uint32_t w0 = w[0], w1 = w[1];
  const h2 a = __builtin_bit_cast(h2, w0), b = __builtin_bit_cast(h2, w1);
  return float4{(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
}

// One workgroup per (b, h): weights of the splits from their (m, l) (wave
// reductions), the weighted sum of their partial outputs (4 consecutive
// channels per thread), then the inverse rotation in registers: a rotation
// block has at most 256 channels = one wave's 64 lanes, so its butterflies
// are in-register (strides 1, 2) or lane shuffles (strides 4 .. 128).  fp32
// partials are unnormalised sums (weight 2^(m_s - m)); fp16 partials are
// already divided by their own l_s (weight 2^(m_s - m) * l_s).
template <typename PT>
__global__ __launch_bounds__(256) void merge_kernel(const PT* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    Dims d, int splits,
                                                    float* __restrict__ obar) {
  constexpr bool kNormalised = std::is_same<PT, _Float16>::value;
  __shared__ float ms[kMaxSplits];
  const int bh = blockIdx.x;
  const int b = bh / d.Hq, h = bh % d.Hq;
  const int t = threadIdx.x, lane = t & 63;
  const int c = 4 * t;
  const size_t stride = (size_t)d.Hq * d.rv;
  const PT* src = part_o + ((size_t)b * splits * d.Hq + h) * d.rv + min(c, d.rv - 4);
  // (m, l) of split `lane` first, then the rows of the first kPre splits
  // (clamped addresses: every load is issued, so the wait for (m, l) does
  // not cover the rows)
  const float2 ml0 = *reinterpret_cast<const float2*>(
      part_ml + (((size_t)b * splits + min(lane, splits - 1)) * d.Hq + h) * 2);
  // (fp32 partials come with one split per row in the prefill: one row)
  constexpr int kPre = kNormalised ? 16 : 1;
  float4 xp[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) xp[u] = load4(src + (size_t)min(u, splits - 1) * stride);
  // every wave reduces the same (m, l) values; wave 0 publishes the weights
  float mx = lane < splits ? ml0.x : -INFINITY;
  for (int s = lane + 64; s < splits; s += 64)
    mx = fmaxf(mx, part_ml[(((size_t)b * splits + s) * d.Hq + h) * 2]);
  mx = wave_max(mx);
  float L = 0.0f;
  if (lane < splits) {
    const float wgt = ml0.y > 0.0f ? exp2f(ml0.x - mx) : 0.0f;
    if (t < 64) ms[lane] = kNormalised ? wgt * ml0.y : wgt;
    L = wgt * ml0.y;
  }
  for (int s = lane + 64; s < splits; s += 64) {
    const size_t k = (((size_t)b * splits + s) * d.Hq + h) * 2;
    const float l = part_ml[k + 1];
    const float wgt = l > 0.0f ? exp2f(part_ml[k] - mx) : 0.0f;
    if (t < 64) ms[s] = kNormalised ? wgt * l : wgt;
    L = fmaf(wgt, l, L);
  }
  const float inv = 1.0f / wave_sum(L);
  __syncthreads();
  float4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  if (c < d.rv) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const float wgt = u < splits ? ms[u] : 0.0f;
      o.x = fmaf(wgt, xp[u].x, o.x);
      o.y = fmaf(wgt, xp[u].y, o.y);
      o.z = fmaf(wgt, xp[u].z, o.z);
      o.w = fmaf(wgt, xp[u].w, o.w);
    }
    int s = kPre;
    for (; s + 8 <= splits; s += 8) {
      float4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = load4(src + (size_t)(s + u) * stride);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wgt = ms[s + u];
        o.x = fmaf(wgt, x[u].x, o.x);
        o.y = fmaf(wgt, x[u].y, o.y);
        o.z = fmaf(wgt, x[u].z, o.z);
        o.w = fmaf(wgt, x[u].w, o.w);
      }
    }
    for (; s < splits; ++s) {
      const float4 x = load4(src + (size_t)s * stride);
      const float wgt = ms[s];
      o.x = fmaf(wgt, x.x, o.x);
      o.y = fmaf(wgt, x.y, o.y);
      o.z = fmaf(wgt, x.z, o.z);
      o.w = fmaf(wgt, x.w, o.w);
    }
    o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
  }
  if (d.dtype == STARKV_CACHE_Q43 && d.rotate) {
    // undo the block rotation of the stored value latents: (Z H) H = Z (eq. 13)
    const int mb = pow2_divisor(d.rv / 4);
    // strides 1 and 2: inside the thread's 4 channels
    float a0 = o.x + o.y, a1 = o.x - o.y, a2 = o.z + o.w, a3 = o.z - o.w;
    o = float4{a0 + a2, a1 + a3, a0 - a2, a1 - a3};
    // strides 4 .. mb/2: partner channels sit 1 .. mb/8 lanes away
    for (int hs = 4; hs < mb; hs <<= 1) {
      const int dl = hs >> 2;
      const float4 p = {__shfl_xor(o.x, dl), __shfl_xor(o.y, dl), __shfl_xor(o.z, dl),
                        __shfl_xor(o.w, dl)};
      if (c & hs) o = float4{p.x - o.x, p.y - o.y, p.z - o.z, p.w - o.w};
      else o = float4{o.x + p.x, o.y + p.y, o.z + p.z, o.w + p.w};
    }
    const float cst = inv_sqrt_pow2(mb);
    o.x *= cst; o.y *= cst; o.z *= cst; o.w *= cst;
  }
  if (c < d.rv) *reinterpret_cast<float4*>(obar + (size_t)bh * d.rv + c) = o;
}

// ------------------------------------------------------------------ vproj --

// out[b, h, r] = sum_c obar[b, h, c] * B_value[g*d_h + r, c] on MFMA 16x16x32
// bf16: one workgroup per (head, 16 rows, 16 sequences); its 4 waves take
// interleaved 32-wide K steps (several loads in flight each) and their
// partial tiles are summed through LDS.  obar (fp32) is split into bf16 high
// and low parts; fp32 factors are split the same way.
constexpr int kVprojWaves = 4;

template <int FMT>
__global__ __launch_bounds__(64 * kVprojWaves) void vproj_kernel(
    const float* __restrict__ obar, const void* __restrict__ bv, Dims d,
    float* __restrict__ out) {
  __shared__ f32x4 red[kVprojWaves - 1][64];
  const int h = blockIdx.x, g = h / d.G;
  const int r0 = blockIdx.y * 16, b0 = blockIdx.z * 16;
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i16 = l & 15, ks = l >> 4;
  const int bb = b0 + i16;
  const float* arow = obar + ((size_t)min(bb, d.B - 1) * d.Hq + h) * d.rv + ks * 8;
  const size_t brow = ((size_t)g * d.dh + r0 + i16) * d.rv + ks * 8;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // this wave's K-steps k0 = 32 (w + 4 s) < rv (s < 8 as rv <= 1024): all
  // operand loads of all steps are issued before the first product; steps
  // past rv multiply zeros
  constexpr int kSteps = 1024 / (32 * kVprojWaves);
  float4 xa[kSteps], xb[kSteps];
  bf8 bw[kSteps];
  f32x4 bwf[kSteps][2];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int k0 = 32 * (w + kVprojWaves * st);
    const bool on = k0 < d.rv;
    xa[st] = on ? *reinterpret_cast<const float4*>(arow + k0) : float4{0.0f, 0.0f, 0.0f, 0.0f};
    xb[st] = on ? *reinterpret_cast<const float4*>(arow + k0 + 4) : float4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (FMT == STARKV_CACHE_F32) {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(bv) + brow + k0);
      bwf[st][0] = on ? p[0] : f32x4{};
      bwf[st][1] = on ? p[1] : f32x4{};
    } else {
      bw[st] = on ? *reinterpret_cast<const bf8*>(static_cast<const uint16_t*>(bv) + brow + k0)
                  : bf8{};
    }
  }
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const float xs[8] = {xa[st].x, xa[st].y, xa[st].z, xa[st].w,
                         xb[st].x, xb[st].y, xb[st].z, xb[st].w};
    bf8 ah, al;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = bb < d.B ? xs[e] : 0.0f;
      ah[e] = (__bf16)x;
      al[e] = (__bf16)(x - (float)ah[e]);
    }
    if constexpr (FMT == STARKV_CACHE_F32) {
      bf8 bh, bl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = bwf[st][e >> 2][e & 3];
        bh[e] = (__bf16)v;
        bl[e] = (__bf16)(v - (float)bh[e]);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    } else {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw[st], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw[st], acc, 0, 0, 0);
    }
  }
  if (w > 0) red[w - 1][l] = acc;
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int i = 0; i < kVprojWaves - 1; ++i) acc += red[i][l];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int ob = b0 + ks * 4 + v;   // row of C = sequence, column = output row
    if (ob < d.B) out[((size_t)ob * d.Hq + h) * d.dh + r0 + i16] = acc[v];
  }
}

// ----------------------------------------------------- merge + vproj --

// Merge and up-projection in one workgroup per (KV head g, sequence b), for
// fp16 partials, value ranks up to 256 and d_h up to 128: the factor block
// of one KV head (d_h x R_v bf16, at most 64 KiB) is then read once per
// sequence from L2 and the two dependent launches become one.
//   - Wave w merges query heads w, w + 4, .. of the group as merge_kernel
//     does (lane = split for (m, l); 4 channels per lane; the inverse value
//     rotation in registers and lane shuffles) and stages each merged row in
//     LDS as bf16 high and low parts.
//   - Then wave w takes output columns 16 rb .. 16 rb + 15 (rb = w, w + 4)
//     on MFMA 16x16x32 bf16: rows = the group's query heads (padded to 16
//     with zero rows), K = R_v; its factor rows are requested before the
//     merge starts.
constexpr int kMvRows = 16;
constexpr int kMvMaxRv = 256;
constexpr int kMvPad = 8;

bool merge_vproj_fits(const Dims& d, int splits) {
  return d.dtype != STARKV_CACHE_F32 && d.rv <= kMvMaxRv && d.rv % 32 == 0 &&
         d.G <= kMvRows && splits <= 64 && d.dh % 16 == 0 && d.dh <= 128;
}

__global__ __launch_bounds__(256) void merge_vproj_kernel(
    const _Float16* __restrict__ part_o, const float* __restrict__ part_ml,
    const uint16_t* __restrict__ bv, Dims d, int splits, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) __bf16 oh[kMvRows][kMvMaxRv + kMvPad];
  __shared__ __attribute__((aligned(16))) __bf16 ol[kMvRows][kMvMaxRv + kMvPad];
  __shared__ float ms[4][64];
  const int g = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int n16 = lane & 15, kq = lane >> 4;
  const int ksteps = d.rv / 32;

  // factor rows of this wave's output columns: B[k][n] = B_value[g d_h +
  // 16 rb + n][k], 8 consecutive k per lane
  bf8 bw[2][kMvMaxRv / 32];
#pragma unroll
  for (int ri = 0; ri < 2; ++ri) {
    const int rb = w + 4 * ri;
    const bool on = 16 * rb < d.dh;
    const uint16_t* brow = bv + ((size_t)g * d.dh + 16 * min(rb, d.dh / 16 - 1) + n16) * d.rv + 8 * kq;
#pragma unroll
    for (int ks = 0; ks < kMvMaxRv / 32; ++ks)
      bw[ri][ks] = on && ks < ksteps ? *reinterpret_cast<const bf8*>(brow + 32 * ks) : bf8{};
  }
  // zero rows past the group's heads
  for (int i = t; i < (kMvRows - d.G) * (d.rv / 8); i += 256) {
    const int row = d.G + i / (d.rv / 8), c8 = 8 * (i % (d.rv / 8));
    *reinterpret_cast<bf8*>(&oh[row][c8]) = bf8{};
    *reinterpret_cast<bf8*>(&ol[row][c8]) = bf8{};
  }

  const size_t stride = (size_t)d.Hq * d.rv;
  const int c = 4 * lane;
  for (int i = w; i < d.G; i += 4) {
    const int h = g * d.G + i;
    const _Float16* src = part_o + ((size_t)b * splits * d.Hq + h) * d.rv + min(c, d.rv - 4);
    const float2 ml0 = *reinterpret_cast<const float2*>(
        part_ml + (((size_t)b * splits + min(lane, splits - 1)) * d.Hq + h) * 2);
    float4 xp[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) xp[u] = load4(src + (size_t)min(u, splits - 1) * stride);
    const float mx = wave_max(lane < splits ? ml0.x : -INFINITY);
    float wl = 0.0f;
    if (lane < splits && ml0.y > 0.0f) wl = exp2f(ml0.x - mx) * ml0.y;
    ms[w][lane] = wl;
    const float inv = 1.0f / wave_sum(wl);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's weights
    __builtin_amdgcn_wave_barrier();
    float4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float wgt = u < splits ? ms[w][u] : 0.0f;
      o.x = fmaf(wgt, xp[u].x, o.x);
      o.y = fmaf(wgt, xp[u].y, o.y);
      o.z = fmaf(wgt, xp[u].z, o.z);
      o.w = fmaf(wgt, xp[u].w, o.w);
    }
    for (int s = 16; s < splits; ++s) {
      const float4 x = load4(src + (size_t)s * stride);
      const float wgt = ms[w][s];
      o.x = fmaf(wgt, x.x, o.x);
      o.y = fmaf(wgt, x.y, o.y);
      o.z = fmaf(wgt, x.z, o.z);
      o.w = fmaf(wgt, x.w, o.w);
    }
    o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
    if (d.dtype == STARKV_CACHE_Q43 && d.rotate) {
      // undo the block rotation of the stored value latents (eq. 13)
      const int mb = pow2_divisor(d.rv / 4);
      float a0 = o.x + o.y, a1 = o.x - o.y, a2 = o.z + o.w, a3 = o.z - o.w;
      o = float4{a0 + a2, a1 + a3, a0 - a2, a1 - a3};
      for (int hs = 4; hs < mb; hs <<= 1) {
        const int dl = hs >> 2;
        const float4 p = {__shfl_xor(o.x, dl), __shfl_xor(o.y, dl), __shfl_xor(o.z, dl),
                          __shfl_xor(o.w, dl)};
        if (c & hs) o = float4{p.x - o.x, p.y - o.y, p.z - o.z, p.w - o.w};
        else o = float4{o.x + p.x, o.y + p.y, o.z + p.z, o.w + p.w};
      }
      const float cst = inv_sqrt_pow2(mb);
      o.x *= cst; o.y *= cst; o.z *= cst; o.w *= cst;
    }
    if (c < d.rv) {
      const float v[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 hi = (__bf16)v[e];
        oh[i][c + e] = hi;
        ol[i][c + e] = (__bf16)(v[e] - (float)hi);
      }
    }
  }
  __syncthreads();

#pragma unroll
  for (int ri = 0; ri < 2; ++ri) {
    const int rb = w + 4 * ri;
    if (16 * rb >= d.dh) break;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kMvMaxRv / 32; ++ks) {
      if (ks >= ksteps) break;
      const bf8 ah = *reinterpret_cast<const bf8*>(&oh[n16][32 * ks + 8 * kq]);
      const bf8 al = *reinterpret_cast<const bf8*>(&ol[n16][32 * ks + 8 * kq]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw[ri][ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw[ri][ks], acc, 0, 0, 0);
    }
    // C[row = query head 4 kq + v][column = output row 16 rb + n16]
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 4 * kq + v;
      if (row < d.G)
        out[((size_t)b * d.Hq + g * d.G + row) * d.dh + 16 * rb + n16] = acc[v];
    }
  }
}

template <int FMT>
hipError_t launch_split(const Dims& d, dim3 grid, const SplitArgs& sa, hipStream_t s) {
  if constexpr (FMT == STARKV_CACHE_Q43) {
    return launch_q43(d, grid, sa, s);
  } else {
    // key rows of up to 16 / 32 / 64 channels (d.rk is a multiple of 8)
    const int rkc = d.rk <= 16 ? 16 : d.rk <= 32 ? 32 : 64;
    switch (d.G * 128 + rkc) {
      case 1 * 128 + 16: split_kernel<FMT, 1, 16><<<grid, 512, 0, s>>>(sa); break;
      case 1 * 128 + 32: split_kernel<FMT, 1, 32><<<grid, 512, 0, s>>>(sa); break;
      case 1 * 128 + 64: split_kernel<FMT, 1, 64><<<grid, 512, 0, s>>>(sa); break;
      case 2 * 128 + 16: split_kernel<FMT, 2, 16><<<grid, 512, 0, s>>>(sa); break;
      case 2 * 128 + 32: split_kernel<FMT, 2, 32><<<grid, 512, 0, s>>>(sa); break;
      case 2 * 128 + 64: split_kernel<FMT, 2, 64><<<grid, 512, 0, s>>>(sa); break;
      case 4 * 128 + 16: split_kernel<FMT, 4, 16><<<grid, 512, 0, s>>>(sa); break;
      case 4 * 128 + 32: split_kernel<FMT, 4, 32><<<grid, 512, 0, s>>>(sa); break;
      case 4 * 128 + 64: split_kernel<FMT, 4, 64><<<grid, 512, 0, s>>>(sa); break;
      case 8 * 128 + 16: split_kernel<FMT, 8, 16><<<grid, 512, 0, s>>>(sa); break;
      case 8 * 128 + 32: split_kernel<FMT, 8, 32><<<grid, 512, 0, s>>>(sa); break;
      default: split_kernel<FMT, 8, 64><<<grid, 512, 0, s>>>(sa); break;
    }
    return hipGetLastError();
  }
}

template <int FMT>
hipError_t decode_fmt(const Dims& d, const starkv_cache& cache, int seq_len,
                      const void* q, const void* bk, const void* bv,
                      float sm_scale, float* out, char* ws, const DecodeWs& lay,
                      hipStream_t s, hipEvent_t* ev) {
  void* qt = ws + lay.qt;
  float* part_o = reinterpret_cast<float*>(ws + lay.part_o);
  float* part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
  float* obar = reinterpret_cast<float*>(ws + lay.obar);
  auto mark = [&](int i) { if (ev) (void)hipEventRecord(ev[i], s); };
  mark(0);
  qproj_kernel<FMT><<<d.B * d.Hq, 256, 0, s>>>(q, bk, d, sm_scale * kLog2e, qt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(1);
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
  e = launch_split<FMT>(d, dim3(lay.splits, d.B), sa, s);
  if (e != hipSuccess) return e;
  mark(2);
  if (FMT != STARKV_CACHE_F32 && merge_vproj_fits(d, lay.splits)) {
    // one kernel for both steps; the up-projection's event pair is empty
    merge_vproj_kernel<<<dim3(d.Hkv, d.B), 256, 0, s>>>(
        reinterpret_cast<const _Float16*>(part_o), part_ml, static_cast<const uint16_t*>(bv),
        d, lay.splits, out);
    e = hipGetLastError();
    mark(3);
    mark(4);
    return e;
  }
  if constexpr (FMT == STARKV_CACHE_F32)
    merge_kernel<float><<<d.B * d.Hq, 256, 0, s>>>(part_o, part_ml, d, lay.splits, obar);
  else   // fp16 partial rows, each divided by its own l
    merge_kernel<_Float16><<<d.B * d.Hq, 256, 0, s>>>(
        reinterpret_cast<const _Float16*>(part_o), part_ml, d, lay.splits, obar);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(3);
  vproj_kernel<FMT><<<dim3(d.Hq, d.dh / 16, (d.B + 15) / 16), 64 * kVprojWaves, 0, s>>>(obar, bv, d, out);
  e = hipGetLastError();
  mark(4);
  return e;
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int decode_groups_per_cu(const Dims& d) {
  if (d.dtype != STARKV_CACHE_Q43) return 1;
  const SplitFn k = q43_kernel(d);
  if (!k) return 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  // asked once per kernel instantiation and device
  static std::mutex mu;
  static std::map<std::pair<SplitFn, int>, int> known;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = known.find({k, dev});
  if (it != known.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(k), 512, 0) != hipSuccess || n < 1) {
    (void)hipGetLastError();   // no device to ask: one group per unit
    return 1;
  }
  known[{k, dev}] = n;
  return n;
}

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
                         const DecodeWs& lay, hipStream_t s, hipEvent_t* ev) {
  switch (d.dtype) {
    case STARKV_CACHE_F32:
      return decode_fmt<STARKV_CACHE_F32>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s, ev);
    case STARKV_CACHE_BF16:
      return decode_fmt<STARKV_CACHE_BF16>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s, ev);
    default:
      return decode_fmt<STARKV_CACHE_Q43>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s, ev);
  }
}

}  // namespace starkv
