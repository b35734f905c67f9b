// Value/output factor fusion and the head sum -- Algorithm 2, steps 7-8 of
// the technical review of arXiv 2606.08382, with section 5.3, eq. 12 read
// right to left: p_h (Z_V U_h^T) O_h = (p_h Z_V)(U_h^T O_h), the right-hand
// factor prepared once, offline.
//
//   fuse_vo    F_h = B_value[g(h)]^T O_h  (R_v x D per query head, bf16),
//              O_h = rows h*d_h .. h*d_h + d_h - 1 of W_o [Hq*d_h, D]; stored
//              "N-blocked": [D/16][Hq*R_v/8][16 columns][8 k] so that a
//              64-lane load of MFMA B operands reads 1 KB contiguously.
//   hidden     y[b, :] = sum_h obar[b, h, :] F_h = obar_flat [B, Hq*R_v] x
//              F [Hq*R_v, D]: a split-K GEMM on MFMA 16x16x32 bf16 (obar fp32
//              split into bf16 high and low parts), K slices summed by a
//              second small kernel in a fixed order (deterministic).
//
// The fused factor holds Hq*R_v*D values: at R_v > d_h it is larger than
// B_value and W_o together, so decoding through it reads more bytes than the
// up-projection followed by W_o would; it is what eq. 12 prescribes, and its
// cost is measured, not assumed.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "device.h"

namespace starkv {
namespace {

constexpr int kHidWaves = 4;        // waves per hidden-GEMM workgroup
constexpr int kHidCols = 32;        // output columns per wave (two 16-wide tiles)

__device__ inline float bf16_to_f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// F[k = h R_v + r][n] for 8 consecutive r (one 16-byte store) and one column
// n per thread; fp32 accumulation of the d_h bf16 products, then RNE to bf16.
__global__ __launch_bounds__(256) void fuse_vo_kernel(const uint16_t* __restrict__ bv,
                                                      const uint16_t* __restrict__ w_o,
                                                      Dims d, int D,
                                                      uint16_t* __restrict__ F) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int kb = blockIdx.y;                 // k / 8
  const int K = d.Hq * d.rv;
  if (n >= D) return;
  const int k0 = kb * 8;
  const int h = k0 / d.rv, r0 = k0 % d.rv, g = h / d.G;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = 0; i < d.dh; ++i) {
    const float o = bf16_to_f(w_o[((size_t)h * d.dh + i) * D + n]);
    const uint16_t* brow = bv + ((size_t)g * d.dh + i) * d.rv + r0;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(bf16_to_f(brow[e]), o, acc[e]);
  }
  bf8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (__bf16)acc[e];
  const size_t idx = (((size_t)(n / 16) * (K / 8) + kb) * 16 + (n % 16)) * 8;
  *reinterpret_cast<bf8*>(F + idx) = v;
}

// Partial y for K slice blockIdx.y: wave w of workgroup x owns columns
// (4x + w) * 32 .. +31 (two 16x16 output tiles) and NRB blocks of 16 rows
// (sequences) starting at row 16 NRB blockIdx.z, so F is streamed once per
// NRB row blocks.  A = obar rows (fp32 -> bf16 high + low), B = F fragments.
// The K slice is walked in chunks of kAhead steps of 32, double-buffered:
// the loads of chunk c + 1 are issued before chunk c is multiplied (a
// scheduling barrier keeps them there), so a wave always has a chunk in
// flight.
template <int NRB>
__global__ __launch_bounds__(64 * kHidWaves) void hidden_gemm_kernel(
    const float* __restrict__ obar, const uint16_t* __restrict__ F, Dims d, int D,
    int k_slice, float* __restrict__ part_y) {
  constexpr int kAhead = NRB == 4 ? 2 : 4;
  const int K = d.Hq * d.rv;
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c0 = (blockIdx.x * kHidWaves + w) * kHidCols;
  if (c0 >= D) return;
  const int ks = blockIdx.y;
  const int kbeg = ks * k_slice, kend = kbeg + k_slice;
  const int m = l & 15, kq = l >> 4;
  const int rb0 = blockIdx.z * 16 * NRB;
  const float* arow[NRB];
  bool live[NRB];
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
    const int b = rb0 + 16 * r + m;
    live[r] = b < d.B;
    arow[r] = obar + (size_t)min(b, d.B - 1) * K + kq * 8;
  }
  const uint16_t* fcol0 = F + (((size_t)(c0 / 16) * (K / 8) + kq) * 16 + m) * 8;
  const uint16_t* fcol1 = fcol0 + (size_t)(K / 8) * 16 * 8;
  f32x4 acc[NRB][2];
#pragma unroll
  for (int r = 0; r < NRB; ++r) acc[r][0] = acc[r][1] = f32x4{};
  auto step = [&](const float4 (&x0)[NRB], const float4 (&x1)[NRB], const bf8& f0,
                  const bf8& f1) {
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const float xs[8] = {x0[r].x, x0[r].y, x0[r].z, x0[r].w,
                           x1[r].x, x1[r].y, x1[r].z, x1[r].w};
      bf8 ah, al;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = live[r] ? xs[e] : 0.0f;
        ah[e] = (__bf16)x;
        al[e] = (__bf16)(x - (float)ah[e]);
      }
      acc[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, f0, acc[r][0], 0, 0, 0);
      acc[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, f0, acc[r][0], 0, 0, 0);
      acc[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, f1, acc[r][1], 0, 0, 0);
      acc[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, f1, acc[r][1], 0, 0, 0);
    }
  };
  struct Chunk {
    float4 a0[kAhead][NRB], a1[kAhead][NRB];
    bf8 b0[kAhead], b1[kAhead];
  };
  auto load_chunk = [&](Chunk& c, int kc) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int k = kc + 32 * u;
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        c.a0[u][r] = *reinterpret_cast<const float4*>(arow[r] + k);
        c.a1[u][r] = *reinterpret_cast<const float4*>(arow[r] + k + 4);
      }
      // F is read once: streaming loads keep it out of the caches
      c.b0[u] = __builtin_nontemporal_load(
          reinterpret_cast<const bf8*>(fcol0 + (size_t)(k / 8) * 16 * 8));
      c.b1[u] = __builtin_nontemporal_load(
          reinterpret_cast<const bf8*>(fcol1 + (size_t)(k / 8) * 16 * 8));
    }
  };
  auto use_chunk = [&](const Chunk& c) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) step(c.a0[u], c.a1[u], c.b0[u], c.b1[u]);
  };
  constexpr int kChunk = 32 * kAhead;
  const int n_chunks = (kend - kbeg) / kChunk;
  int k0 = kbeg;
  if (n_chunks > 0) {
    Chunk ca, cb;
    load_chunk(ca, k0);
    int c = 0;
    for (; c + 2 <= n_chunks; c += 2) {
      load_chunk(cb, k0 + kChunk);
      __builtin_amdgcn_sched_barrier(0);
      use_chunk(ca);
      if (c + 2 < n_chunks) load_chunk(ca, k0 + 2 * kChunk);
      __builtin_amdgcn_sched_barrier(0);
      use_chunk(cb);
      k0 += 2 * kChunk;
    }
    if (c < n_chunks) {   // odd count: the last chunk is in ca
      __builtin_amdgcn_sched_barrier(0);
      use_chunk(ca);
      k0 += kChunk;
    }
  }
  // the rest of the slice, one step at a time
  for (; k0 < kend; k0 += 32) {
    float4 x0[NRB], x1[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      x0[r] = *reinterpret_cast<const float4*>(arow[r] + k0);
      x1[r] = *reinterpret_cast<const float4*>(arow[r] + k0 + 4);
    }
    const bf8 f0 = *reinterpret_cast<const bf8*>(fcol0 + (size_t)(k0 / 8) * 16 * 8);
    const bf8 f1 = *reinterpret_cast<const bf8*>(fcol1 + (size_t)(k0 / 8) * 16 * 8);
    step(x0, x1, f0, f1);
  }
  // D[row = sequence 4 kq + i][column = m] of each tile
#pragma unroll
  for (int r = 0; r < NRB; ++r)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ob = rb0 + 16 * r + 4 * kq + i;
        if (ob < d.B) part_y[((size_t)ks * d.B + ob) * D + c0 + 16 * t + m] = acc[r][t][i];
      }
}

__global__ __launch_bounds__(256) void hidden_reduce_kernel(const float* __restrict__ part_y,
                                                            int n_slices, size_t n,
                                                            float* __restrict__ y) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int k = 0; k < n_slices; ++k) s += part_y[(size_t)k * n + i];
  y[i] = s;
}

}  // namespace

int hidden_k_slices(const Dims& d, int D) {
  const int K = d.Hq * d.rv;
  const int groups = (D + kHidWaves * kHidCols - 1) / (kHidWaves * kHidCols);
  // slices of whole 4-step chunks where K allows it
  int ks = 1;
  while (ks * 2 * groups <= 512 && K % (ks * 2 * 32 * 4) == 0) ks *= 2;
  return ks;
}

hipError_t launch_fuse_vo(const Dims& d, const void* bv, const void* w_o, int D,
                          void* F, hipStream_t s) {
  const int K = d.Hq * d.rv;
  fuse_vo_kernel<<<dim3((D + 255) / 256, K / 8), 256, 0, s>>>(
      static_cast<const uint16_t*>(bv), static_cast<const uint16_t*>(w_o), d, D,
      static_cast<uint16_t*>(F));
  return hipGetLastError();
}

hipError_t launch_hidden(const Dims& d, const float* obar, const void* F, int D,
                         float* part_y, float* y, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) { if (ev) (void)hipEventRecord(ev[i], s); };
  const int K = d.Hq * d.rv;
  const int ks = hidden_k_slices(d, D);
  const int groups = (D + kHidWaves * kHidCols - 1) / (kHidWaves * kHidCols);
  // row blocks of 16 sequences handled per pass over F: all of them up to 64
  const int nrb_total = (d.B + 15) / 16;
  const int nrb = nrb_total >= 4 ? 4 : nrb_total >= 2 ? 2 : 1;
  const dim3 grid(groups, ks, (nrb_total + nrb - 1) / nrb);
  const uint16_t* Fp = static_cast<const uint16_t*>(F);
  if (nrb == 4)
    hidden_gemm_kernel<4><<<grid, 64 * kHidWaves, 0, s>>>(obar, Fp, d, D, K / ks, part_y);
  else if (nrb == 2)
    hidden_gemm_kernel<2><<<grid, 64 * kHidWaves, 0, s>>>(obar, Fp, d, D, K / ks, part_y);
  else
    hidden_gemm_kernel<1><<<grid, 64 * kHidWaves, 0, s>>>(obar, Fp, d, D, K / ks, part_y);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(0);
  const size_t n = (size_t)d.B * D;
  hidden_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part_y, ks, n, y);
  e = hipGetLastError();
  mark(1);
  return e;
}

}  // namespace starkv
