// Decode attention over the latent cache -- steps 4-7 of Algorithm 2 in the
// technical review of arXiv 2606.08382 (section 6.2), without a key or value
// cache ever being reconstructed in memory.
//
//   qproj   q~ = q B_key[g] (d_h -> r_k), rotated like the stored latents and
//           pre-scaled by sm_scale*log2(e): the score q K^T equals q~ Z^T
//           (eq. 2 read right to left).
//   split   per (sequence, token split): latent scores, online softmax, then
//           the stacked-head probabilities P [Hq x tokens] times the shared
//           value latent Z_v on MFMA (section 5.3 / eq. 12: stacking the
//           heads' probability rows makes the per-head weighted sums one
//           matrix product against the shared latent).
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
#include "qproj.h"
#include "split_q43.h"

namespace starkv {
namespace {




// ------------------------------------------------------------------ qproj --

template <int FMT>
__global__ __launch_bounds__(256) void qproj_kernel(const void* __restrict__ q,
                                                    const void* __restrict__ bk,
                                                    Dims d, float qscale,
                                                    void* __restrict__ qt) {
  qproj_block<FMT>(q, bk, d, qscale, qt, blockIdx.x);
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
  const size_t row0 = plain_key_offset(d, b, kh, tile, 0, lane);
  const int rank = d.krank[kh];            // this KV head's key rank
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
    for (int c = 0; c < NC && 8 * c < rank; ++c) {
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
    // chunks past the head's rank (RK rounds the largest up) are neither
    // read nor used
    const bool live = 8 * c < rank;
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
  // value slice blockIdx.z of gridDim.z: this workgroup contracts value
  // groups [g_lo, g_hi) only (every slice scores all heads)
  const int GVs = GV / (int)gridDim.z;
  const int g_lo = (int)blockIdx.z * GVs, g_hi = g_lo + GVs;

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
        const int n = g_lo + wave + ni * NW;
        // K-step r, lane half j: tokens 16r + 8j .. +7 = token block 2r + j
        const uint16_t* zp =
            vbase + (((size_t)b * d.NT + tile) * GV + min(n, g_hi - 1)) * (8 * 256) + (j * 32 + m) * 8;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Zv[ni][r] = n < g_hi ? __builtin_nontemporal_load(reinterpret_cast<const bf8*>(zp + r * 512))
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
          const int n = g_lo + wave + ni * NW;
          if (n < g_hi) {
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
        const int n = g_lo + wave + ni * NW;
        if (n < g_hi) {
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
          if (blockIdx.z == 0) {   // the same (m, l) in every value slice
            a.part_ml[(obase + h) * 2] = m_ref[ki * G + jj];
            a.part_ml[(obase + h) * 2 + 1] = l;
          }
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
      const int n = g_lo + wave + ni * NW;
      if (row < d.Hq && n < g_hi) {
        const h8 o = *reinterpret_cast<const h8*>(&stg[wave][row][ni * 32 + part * 8]);
        __builtin_nontemporal_store(o, reinterpret_cast<h8*>(po + (obase + row) * d.rv + n * 32 + part * 8));
      }
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = g_lo + wave + ni * NW;
      if (n < g_hi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = acc_row(v, lane);
          if (row < d.Hq) a.part_o[(obase + row) * d.rv + n * 32 + m] = acc[ni][v];
        }
      }
    }
  }
}

SplitFn q43_kernel(const Dims& d) {
  if (d.lob == 4) return d.rope_theta > 0.0f ? u4_rope_kernel(d) : u4_kernel(d);
  return d.rope_theta > 0.0f ? q43_rope_kernel(d) : q43_kernel_select<false, false>(d);
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

// Rows of partials a merge lane keeps in flight: 16 fp16 rows, 8 fp32 rows.
template <typename PT>
constexpr int merge_batch() { return std::is_same<PT, _Float16>::value ? 16 : 8; }
// Waves of a merge workgroup that share one block of 256 channels: 1 while
// one batch holds every split, then 2, then 4 (the splits dealt out among
// them, so that a lane's chain of row loads stays short).
__host__ __device__ inline int merge_wsplit(int splits, int batch) {
  return splits <= batch ? 1 : splits <= 2 * batch ? 2 : 4;
}

// One workgroup per (b, h, 4 / W blocks of 256 channels), W = merge_wsplit:
// the weights of the splits from their (m, l) (wave reductions), then each
// of the W waves of a channel block sums the splits s = k, k + W, k + 2W, ...
// (k its index among them) with kBatch rows in flight per lane (4
// consecutive channels per lane); their sums meet in LDS, and the first
// wave of the block scales by 1 / L, undoes the block rotation and stores.
// A rotation block has at most 256 channels, i.e. one wave's 64 lanes: its
// butterflies are in registers (strides 1, 2) or lane shuffles (strides
// 4 .. 128).  fp32 partials are unnormalised sums (weight 2^(m_s - m)); fp16
// partials are already divided by their own l_s (weight 2^(m_s - m) * l_s).
template <typename PT>
__global__ __launch_bounds__(256) void merge_kernel(const PT* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    Dims d, int splits,
                                                    float* __restrict__ obar) {
  constexpr bool kNormalised = std::is_same<PT, _Float16>::value;
  constexpr int kBatch = merge_batch<PT>();
  __shared__ float ms[kMaxSplits];
  __shared__ float4 red[4][64];
  const int bh = blockIdx.x;
  const int b = bh / d.Hq, h = bh % d.Hq;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int W = merge_wsplit(splits, kBatch);
  const int sw = wave % W;                      // the wave's index in its block
  const int c = (blockIdx.y * (4 / W) + wave / W) * 256 + 4 * lane;
  const size_t stride = (size_t)d.Hq * d.rv;
  const PT* src = part_o + ((size_t)b * splits * d.Hq + h) * d.rv + min(c, d.rv - 4);
  // (m, l) of split `lane` first, then this wave's first batch of rows
  // (clamped addresses: every load is issued, so the wait for (m, l) does
  // not cover the rows)
  const float2 ml0 = *reinterpret_cast<const float2*>(
      part_ml + (((size_t)b * splits + min(lane, splits - 1)) * d.Hq + h) * 2);
  float4 xp[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u)
    xp[u] = load4(src + (size_t)min(sw + W * u, splits - 1) * stride);
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
  // a sequence with no token in any split (ragged batches, length 0) gives 0
  const float Lt = wave_sum(L);
  const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
  __syncthreads();
  float4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  auto accumulate = [&](int s0, const float4 (&x)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sp = s0 + sw + W * u;
      const float wgt = sp < splits ? ms[sp] : 0.0f;
      o.x = fmaf(wgt, x[u].x, o.x);
      o.y = fmaf(wgt, x[u].y, o.y);
      o.z = fmaf(wgt, x[u].z, o.z);
      o.w = fmaf(wgt, x[u].w, o.w);
    }
  };
  accumulate(0, xp);
  for (int s0 = W * kBatch; s0 < splits; s0 += W * kBatch) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      xp[u] = load4(src + (size_t)min(s0 + sw + W * u, splits - 1) * stride);
    accumulate(s0, xp);
  }
  if (W > 1) {
    red[wave][lane] = o;
    __syncthreads();
    if (sw != 0) return;
    for (int k = 1; k < W; ++k) {
      const float4 r = red[wave + k][lane];
      o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
    }
  }
  o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
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
    const float wt = wave_sum(wl);
    const float inv = wt > 0.0f ? 1.0f / wt : 0.0f;
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
                      hipStream_t s, hipEvent_t* ev, bool qproj_done,
                      bool first_mark_done, bool latent_only) {
  void* qt = ws + lay.qt;
  float* part_o = reinterpret_cast<float*>(ws + lay.part_o);
  float* part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
  float* obar = reinterpret_cast<float*>(ws + lay.obar);
  auto mark = [&](int i) { if (ev) (void)hipEventRecord(ev[i], s); };
  // a decode step records events[0] itself, before its append
  if (!first_mark_done) mark(0);
  hipError_t e = hipSuccess;
  const int n_tiles = (seq_len + kTile - 1) / kTile;
  const int tiles_per_split = (n_tiles + lay.splits - 1) / lay.splits;
  const bool rope = FMT == STARKV_CACHE_Q43 && d.rope_theta > 0.0f;
  if (rope) {
    // rotary keys: position trig table, rotated query coefficients and the
    // scores of every head and token (rope.hip), read by the split kernel
    // (profiled calls: events[0] is re-recorded right before the score
    // kernel, so that events[0..1] time it alone)
    e = launch_rope_scores(d, cache, seq_len, q, bk, sm_scale, ws + lay.rope_off, lay.rope,
                           lay.splits, tiles_per_split, s, ev ? ev[0] : nullptr);
    if (e != hipSuccess) return e;
  } else if (!qproj_done) {
    qproj_kernel<FMT><<<d.B * d.Hq, 256, 0, s>>>(q, bk, d, sm_scale * kLog2e, qt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mark(1);
  SplitArgs sa;
  sa.d = d;
  sa.seq_len = seq_len;
  sa.splits = lay.splits;
  sa.tiles_per_split = tiles_per_split;
  sa.s_rel = rope ? ws + lay.rope_off + lay.rope.s_rel : nullptr;
  sa.m_tile = rope ? reinterpret_cast<const float*>(ws + lay.rope_off + lay.rope.m_tile) : nullptr;
  sa.m_split = rope ? reinterpret_cast<const float*>(ws + lay.rope_off + lay.rope.m_split) : nullptr;
  sa.key = cache.key;
  sa.kmeta = static_cast<const uint16_t*>(cache.key_meta);
  sa.value = cache.value;
  sa.vmeta = static_cast<const uint16_t*>(cache.value_meta);
  sa.qt = qt;
  sa.part_o = part_o;
  sa.part_ml = part_ml;
  // unquantized caches: when the splits leave compute units idle (short
  // contexts, small batches), each tile's value groups are dealt out among
  // up to 4 workgroups, which all score it: one unit fetches only about
  // 1/256 of the chip's bandwidth, so fewer bytes per workgroup on more
  // units finish sooner
  int vslices = 1;
  if constexpr (FMT != STARKV_CACHE_Q43) {
    const int gv = d.rv / 32;
    // (at least 8 groups per slice: one per wave)
    while (vslices < 4 && lay.splits * d.B * vslices * 2 <= kComputeUnits &&
           gv % (vslices * 2) == 0 && gv / (vslices * 2) >= 8)
      vslices *= 2;
  }
  e = launch_split<FMT>(d, dim3(lay.splits, d.B, vslices), sa, s);
  if (e != hipSuccess) return e;
  mark(2);
  if (FMT != STARKV_CACHE_F32 && !latent_only && merge_vproj_fits(d, lay.splits)) {
    // one kernel for both steps; the up-projection's event pair is empty
    merge_vproj_kernel<<<dim3(d.Hkv, d.B), 256, 0, s>>>(
        reinterpret_cast<const _Float16*>(part_o), part_ml, static_cast<const uint16_t*>(bv),
        d, lay.splits, out);
    e = hipGetLastError();
    mark(3);
    mark(4);
    return e;
  }
  // channels per merge workgroup: 4 / W blocks of 256
  const int mw = merge_wsplit(lay.splits, FMT == STARKV_CACHE_F32 ? merge_batch<float>()
                                                                  : merge_batch<_Float16>());
  const dim3 mgrid(d.B * d.Hq, (d.rv + 256 * (4 / mw) - 1) / (256 * (4 / mw)));
  if constexpr (FMT == STARKV_CACHE_F32)
    merge_kernel<float><<<mgrid, 256, 0, s>>>(part_o, part_ml, d, lay.splits, obar);
  else   // fp16 partial rows, each divided by its own l
    merge_kernel<_Float16><<<mgrid, 256, 0, s>>>(
        reinterpret_cast<const _Float16*>(part_o), part_ml, d, lay.splits, obar);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(3);
  if (latent_only) return hipSuccess;   // obar (unrotated) is the result
  vproj_kernel<FMT><<<dim3(d.Hq, d.dh / 16, (d.B + 15) / 16), 64 * kVprojWaves, 0, s>>>(obar, bv, d, out);
  e = hipGetLastError();
  mark(4);
  return e;
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool decode_supported(const Dims& d) {
  if (d.rope_theta > 0.0f && !rope_supported(d)) return false;
  return d.dtype != STARKV_CACHE_Q43 || q43_kernel(d) != nullptr;
}

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

DecodeWs decode_ws_layout(const Dims& d, int splits, int seq_len) {
  DecodeWs w;
  w.splits = splits;
  size_t off = 0;
  w.qt = off;
  off += align256((size_t)d.B * d.Hq * kPlainRec * 4);
  w.part_o = off;
  // partial rows: fp32 for an F32 cache, fp16 (divided by l) otherwise
  off += align256((size_t)d.B * splits * d.Hq * d.rv * (d.dtype == STARKV_CACHE_F32 ? 4 : 2));
  w.part_ml = off;
  off += align256((size_t)d.B * splits * d.Hq * 2 * 4);
  w.obar = off;
  off += align256((size_t)d.B * d.Hq * d.rv * 4);
  w.rope_off = off;
  w.rope = RopeWs{};
  if (d.dtype == STARKV_CACHE_Q43 && d.rope_theta > 0.0f)
    off += rope_ws_bytes(d, seq_len, splits, &w.rope);
  w.total = off;
  return w;
}

hipError_t launch_decode(const Dims& d, const starkv_cache& cache, int seq_len,
                         const void* q, const void* bk, const void* bv,
                         float sm_scale, float* out, char* ws,
                         const DecodeWs& lay, hipStream_t s, hipEvent_t* ev,
                         bool qproj_done, bool first_mark_done, bool latent_only) {
  switch (d.dtype) {
    case STARKV_CACHE_F32:
      return decode_fmt<STARKV_CACHE_F32>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s, ev, qproj_done, first_mark_done, latent_only);
    case STARKV_CACHE_BF16:
      return decode_fmt<STARKV_CACHE_BF16>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s, ev, qproj_done, first_mark_done, latent_only);
    default:
      return decode_fmt<STARKV_CACHE_Q43>(d, cache, seq_len, q, bk, bv, sm_scale, out, ws, lay, s, ev, qproj_done, first_mark_done, latent_only);
  }
}

}  // namespace starkv
