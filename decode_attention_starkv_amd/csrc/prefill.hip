// Chunked causal prefill over the latent cache: steps 1-3 of Algorithm 2 in
// the technical review of arXiv 2606.08382 (project the chunk's hidden states
// into the latent space, rotate, quantize and append), then causal attention
// of the chunk's queries through the stored, quantized cache.
//
//   gemm      Z = X [A_key | A_value] (bf16 in, fp32 out) on MFMA 32x32x16
//   append    the decode-path append kernels (rotation + 4/3-bit packing)
//   keys      the key latents of every visible position as fp16; with
//             rotary keys, the keys themselves: reconstructed through the
//             key factor and rotated at their positions (section 5.3,
//             Algorithm 2 steps 4b-4c)
//   qproj     q~ for every query of the chunk on MFMA (natural channel
//             order); with rotary keys, the queries rotated at their positions
//   attn      per (128 stacked rows of queries x query heads, up to 512
//             value columns): scores on MFMA (over the 32 latent channels,
//             or the d_h channels of rotary keys) with a lazy online softmax,
//             then P Z_v on MFMA with each wave dequantizing its own value
//             groups straight into MFMA operands (section 5.3, eq. 12)
//   vproj     the attention rows times the value factor rotated like the
//             stored latents, on MFMA, divided by the softmax denominator
#include <type_traits>

#include "device.h"

namespace starkv {
namespace {

// ------------------------------------------------------------------- gemm --

// Z[mat] [M][N] = X [M][D] * A[mat] [D][N], bf16 x bf16 -> fp32, mat = the
// key or the value projection.  Workgroup tile 128 x 128, four
// waves in 2 x 2, each 2 x 2 MFMA 32x32x16 tiles; K steps of 32 staged
// through LDS.  X tiles are read as 16-byte k-runs; A is kept k-major in LDS
// and a lane gathers its 8 k-values of one column with 2-byte reads.
struct GemmArgs {
  const uint16_t* x;
  const uint16_t* a[2];
  float* z[2];
  float* zdbg;       // optional [M][ldd] copy of both outputs side by side
  int M, D, N[2], off[2], ldd;
  int nx, ny;        // column tiles (of the wider projection) and row tiles
};
constexpr int kGT = 128;          // workgroup tile (rows and columns)
constexpr int kGK = 32;           // K step
constexpr int kGXS = kGK + 8;     // X tile row stride (bf16)
constexpr int kGAS = kGT + 8;     // A tile row stride (bf16)

__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kGT * kGXS];
  __shared__ __attribute__((aligned(16))) uint16_t as[kGK * kGAS];
  // XCD-aware order (workgroup L runs on XCD L mod 8): every column tile of
  // both projections for one block of 128 rows runs on one XCD, so that
  // XCD fetches those rows of X once (row blocks padded to a multiple of 8)
  const int L = blockIdx.x, xcd = L & 7, k = L >> 3;
  const int per_row = 2 * g.nx;
  const int yb = 8 * (k / per_row) + xcd;
  const int mat = (k % per_row) / g.nx;
  const int N = g.N[mat];
  const int m0 = yb * kGT, n0 = (k % g.nx) * kGT;
  // past the last row block, or the other projection is wider: uniform exit
  if (yb >= g.ny || n0 >= N) return;
  const uint16_t* A = g.a[mat];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m = lane & 31, j = lane >> 5;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  // one K step = 512 chunks of 16 B from X and 512 from A; 2 + 2 per thread
  u32x4 xr[2], ar[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 2, kc = (c & 3) * 8;
      const int row = m0 + r;
      xr[i] = row < g.M
                  ? *reinterpret_cast<const u32x4*>(g.x + (size_t)row * g.D + k0 + kc)
                  : u32x4{0u, 0u, 0u, 0u};
      const int k = c >> 4, nc = (c & 15) * 8;
      const int col = n0 + nc;
      ar[i] = col < N ? *reinterpret_cast<const u32x4*>(A + (size_t)(k0 + k) * N + col)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 2, kc = (c & 3) * 8;
      *reinterpret_cast<u32x4*>(xs + r * kGXS + kc) = xr[i];
      const int k = c >> 4, nc = (c & 15) * 8;
      *reinterpret_cast<u32x4*>(as + k * kGAS + nc) = ar[i];
    }
  };

  load(0);
  for (int k0 = 0; k0 < g.D; k0 += kGK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + kGK < g.D) load(k0 + kGK);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf8 af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const bf8*>(xs + (wm * 64 + t * 32 + m) * kGXS + s * 16 + j * 8);
        const uint16_t* col = as + (s * 16 + j * 8) * kGAS + wn * 64 + t * 32 + m;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)col[(2 * e) * kGAS] | ((uint32_t)col[(2 * e + 1) * kGAS] << 16);
        bfr[t] = __builtin_bit_cast(bf8, u32x4{w[0], w[1], w[2], w[3]});
      }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
          acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ti], bfr[tj], acc[ti][tj], 0, 0, 0);
    }
  }
  float* z = g.z[mat];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
      const int col = n0 + wn * 64 + tj * 32 + m;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 64 + ti * 32 + acc_row(v, lane);
        if (row < g.M && col < N) {
          z[(size_t)row * N + col] = acc[ti][tj][v];
          if (g.zdbg) g.zdbg[(size_t)row * g.ldd + g.off[mat] + col] = acc[ti][tj][v];
        }
      }
    }
}


// s_waitcnt vmcnt(N) for a compile-time N.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ------------------------------------------------------------- key dequant --

// The stored key latent z + s * code (fp32, channels in their natural
// order, still in the rotated basis when the cache rotates) of position t of
// KV head h of sequence b, from a 4/3-bit or a uniform 4-bit key tile.
__device__ inline void key_latent(const uint8_t* __restrict__ key,
                                  const u32x2* __restrict__ kmeta, const Dims& d, int b,
                                  int t, int h, float (&v)[32]) {
  const int tile = t / kTile, u = t % kTile;
  // the tile's slot: b * NT + tile, or its page in a paged pool
  const size_t blk = tile_index(d, b, tile) * d.Hkv + h;
  const uint8_t* kb = key + blk * key_block_bytes(d.lob);
  const uint32_t whi = reinterpret_cast<const uint32_t*>(kb)[u];
  const uint32_t w0 = reinterpret_cast<const uint32_t*>(kb + 256)[u];
  const uint32_t w1 = reinterpret_cast<const uint32_t*>(kb + 512)[u];
  // the remainder byte (4/3-bit) or the fourth 4-bit plane
  const uint32_t w2 = d.lob == 4 ? reinterpret_cast<const uint32_t*>(kb + 768)[u] : kb[768 + u];
  const uint32_t R = w2 | (((w0 >> 15) & 1u) << 8) | ((w0 >> 31) << 9) |
                     (((w1 >> 15) & 1u) << 10) | ((w1 >> 31) << 11);
  const u32x2 mt = kmeta[blk * kTile + u];
  const uint32_t m0 = mt[0], m1 = mt[1];
  const _Float16 s_hi = __builtin_bit_cast(_Float16, (uint16_t)(m0 & 0xFFFFu));
  const _Float16 z_hi = __builtin_bit_cast(_Float16, (uint16_t)(m0 >> 16));
  const _Float16 s_lo = __builtin_bit_cast(_Float16, (uint16_t)(m1 & 0xFFFFu));
  const _Float16 z_lo = __builtin_bit_cast(_Float16, (uint16_t)(m1 >> 16));
#pragma unroll
  for (int c = 0; c < 8; ++c)
    v[c] = fmaf((float)s_hi, (float)((whi >> (4 * c)) & 15u), (float)z_hi);
  if (d.lob == 4) {
    // uniform 4-bit: channel 8p + c at bits 4c of plane p
    const uint32_t pl[3] = {w0, w1, w2};
#pragma unroll
    for (int i = 0; i < 24; ++i)
      v[8 + i] = fmaf((float)s_lo, (float)((pl[i / 8] >> (4 * (i % 8))) & 15u), (float)z_lo);
  } else {
    // 3-bit channel i (= key channel 8 + i): i < 5 lo0 bits 3i, i < 10 lo1
    // bits 3(i-5), i < 15 lo0 bits 16+3(i-10), i < 20 lo1 bits 16+3(i-15),
    // else bits 3(i-20) of the 12-bit remainder
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      uint32_t code;
      if (i < 5) code = (w0 >> (3 * i)) & 7u;
      else if (i < 10) code = (w1 >> (3 * (i - 5))) & 7u;
      else if (i < 15) code = (w0 >> (16 + 3 * (i - 10))) & 7u;
      else if (i < 20) code = (w1 >> (16 + 3 * (i - 15))) & 7u;
      else code = (R >> (3 * (i - 20))) & 7u;
      v[8 + i] = fmaf((float)s_lo, (float)code, (float)z_lo);
    }
  }
}

// fp16 key latents of positions [0, n) of every sequence and KV head,
// channels in their natural order: [B][T_max][Hkv][32] (64 bytes per token
// and head).  One thread per (sequence, position, KV head).  The attention
// kernel reads them as MFMA operands.
__global__ __launch_bounds__(256) void key_dequant_kernel(const uint8_t* __restrict__ key,
                                                          const u32x2* __restrict__ kmeta,
                                                          Dims d, int n,
                                                          _Float16* __restrict__ kd) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)d.B * n * d.Hkv) return;
  const int h = idx % d.Hkv;
  const int t = (idx / d.Hkv) % n;
  const int b = idx / ((size_t)d.Hkv * n);
  float v[32];
  key_latent(key, kmeta, d, b, t, h, v);
  h8* dst = reinterpret_cast<h8*>(kd + (((size_t)b * d.Tmax + t) * d.Hkv + h) * 32);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    dst[k] = h8{(_Float16)v[8 * k], (_Float16)v[8 * k + 1], (_Float16)v[8 * k + 2],
                (_Float16)v[8 * k + 3], (_Float16)v[8 * k + 4], (_Float16)v[8 * k + 5],
                (_Float16)v[8 * k + 6], (_Float16)v[8 * k + 7]};
}

// ------------------------------------------------------------ rotary keys --

// Rotary keys of positions [0, n) of every sequence and KV head (section 5.3
// of the review, Algorithm 2 steps 4b-4c: the stored keys stay pre-RoPE
// latents, reconstructed and rotated at run time): the stored latent, its
// block rotation undone (eq. 13; the 8-channel Hadamard blocks are
// symmetric), times the key factor (eq. 2: k = B_key[g] z, columns past the
// head's key rank taken as zero), then each pair (i, i + d_h/2) turned by
// the angle of its position.  fp16 [B][T_max][Hkv][d_h], d_h = 64 or 128.
// One block per (64 positions, KV head, sequence): the 64 latents go to LDS
// first; thread (pair i, token group) then keeps rows i and i + d_h/2 of
// B_key[g] in registers and walks its tokens, reading each latent as an LDS
// broadcast.
__global__ __launch_bounds__(256) void rope_key_kernel(const uint8_t* __restrict__ key,
                                                       const u32x2* __restrict__ kmeta,
                                                       const uint16_t* __restrict__ bk,
                                                       Dims d, int n, double log2_theta,
                                                       _Float16* __restrict__ kd) {
  // rows padded to 36 floats: 16-byte aligned for the 16-byte broadcasts
  __shared__ __attribute__((aligned(16))) float zl[kTile][36];
  const int g = blockIdx.y, b = blockIdx.z, t0 = blockIdx.x * kTile;
  const int tid = threadIdx.x;
  if (tid < kTile) {
    float z[32];
    const int t = t0 + tid;
    if (t < n) {
      key_latent(key, kmeta, d, b, t, g, z);
    } else {
#pragma unroll
      for (int c = 0; c < 32; ++c) z[c] = 0.0f;
    }
    if (d.rotate) {
      // z <- H8 z per block of 8 channels (butterflies, then 1/sqrt(8))
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int st = 1; st < 8; st <<= 1)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!(e & st)) {
              const float x = z[8 * blk + e], y = z[8 * blk + e + st];
              z[8 * blk + e] = x + y;
              z[8 * blk + e + st] = x - y;
            }
#pragma unroll
      for (int c = 0; c < 32; ++c) z[c] *= inv_sqrt_pow2(8);
    }
#pragma unroll
    for (int c = 0; c < 32; ++c) zl[tid][c] = z[c];
  }
  __syncthreads();
  const int half = d.dh / 2;                   // pairs: 32 or 64
  const int i = tid % half, grp = tid / half, ngrp = 256 / half;
  const int rank = d.krank[g];
  const double w = rope_freq(i, d.dh, log2_theta);
  // rows i and i + d_h/2 of B_key[g] (32 bf16 each): four 16-byte loads per row
  float b1[32], b2[32];
  {
    const u32x4* r1 = reinterpret_cast<const u32x4*>(bk + ((size_t)g * d.dh + i) * 32);
    const u32x4* r2 = reinterpret_cast<const u32x4*>(bk + ((size_t)g * d.dh + i + half) * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w1 = r1[q], w2 = r2[q];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * q + e;
        const uint32_t h1 = (w1[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const uint32_t h2 = (w2[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        b1[c] = c < rank ? bf16v(h1) : 0.0f;
        b2[c] = c < rank ? bf16v(h2) : 0.0f;
      }
    }
  }
  for (int u = grp; u < kTile; u += ngrp) {
    const int t = t0 + u;
    if (t >= n) break;
    float k1 = 0.0f, k2 = 0.0f;
#pragma unroll
    for (int c4 = 0; c4 < 8; ++c4) {
      const float4 z4 = *reinterpret_cast<const float4*>(&zl[u][4 * c4]);
      k1 = fmaf(b1[4 * c4], z4.x, k1);
      k1 = fmaf(b1[4 * c4 + 1], z4.y, k1);
      k1 = fmaf(b1[4 * c4 + 2], z4.z, k1);
      k1 = fmaf(b1[4 * c4 + 3], z4.w, k1);
      k2 = fmaf(b2[4 * c4], z4.x, k2);
      k2 = fmaf(b2[4 * c4 + 1], z4.y, k2);
      k2 = fmaf(b2[4 * c4 + 2], z4.z, k2);
      k2 = fmaf(b2[4 * c4 + 3], z4.w, k2);
    }
    float cs, sn;
    rope_sincos(t, w, &cs, &sn);
    _Float16* dst = kd + (((size_t)b * d.Tmax + t) * d.Hkv + g) * d.dh;
    dst[i] = (_Float16)(k1 * cs - k2 * sn);
    dst[i + half] = (_Float16)(k1 * sn + k2 * cs);
  }
}

// Rotary queries of the chunk: query i of sequence b (position ctx + i)
// turned pair by pair like the keys and scaled by sm_scale log2(e), fp16
// [rows][Hq][d_h].  One thread per (row, head, pair).
__global__ __launch_bounds__(256) void rope_query_kernel(const uint16_t* __restrict__ q,
                                                         Dims d, int rows, int chunk, int ctx,
                                                         double log2_theta, float qscale,
                                                         _Float16* __restrict__ qn) {
  const int half = d.dh / 2;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)rows * d.Hq * half) return;
  const int i = idx % half;
  const size_t rh = idx / half;                  // row * Hq + head
  const int pos = ctx + (int)((rh / d.Hq) % chunk);
  const float x1 = bf16v(q[rh * d.dh + i]), x2 = bf16v(q[rh * d.dh + i + half]);
  float cs, sn;
  rope_angle(pos, i, d.dh, log2_theta, &cs, &sn);
  qn[rh * d.dh + i] = (_Float16)((x1 * cs - x2 * sn) * qscale);
  qn[rh * d.dh + i + half] = (_Float16)((x1 * sn + x2 * cs) * qscale);
}

// ------------------------------------------------------------------ qproj --

// q~ = q B_k[g] of every (row, head) of the chunk (eq. 2), rotated by blocks
// of 8 channels like the stored key latents (eq. 13) and scaled by
// sm_scale log2(e), as fp16 in natural channel order: [rows][Hq][32].  One
// workgroup per (128 rows, head): 4 waves of 32 rows on MFMA 32x32x16 bf16,
// B_k[g] staged channel-major in LDS.
__global__ __launch_bounds__(256) void prefill_qproj_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ bk,
                                                            Dims d, int rows, float qscale,
                                                            _Float16* __restrict__ qn) {
  __shared__ __attribute__((aligned(16))) uint16_t bt[32 * (256 + 8)];
  const int h = blockIdx.y, g = h / d.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, j = lane >> 5;
  const int bs = d.dh + 8;    // row stride of bt: operand reads spread over the banks
  for (int i = tid; i < d.dh * 32; i += 256) {
    const int k = i >> 5, c = i & 31;
    // channels past the head's key rank have no factor column (zero)
    bt[c * bs + k] = c < d.krank[g] ? bk[((size_t)g * d.dh + k) * 32 + c] : (uint16_t)0;
  }
  __syncthreads();
  const int r0 = blockIdx.x * 128 + wave * 32;
  const uint16_t* qrow = q + ((size_t)min(r0 + m, rows - 1) * d.Hq + h) * d.dh + 8 * j;
  f32x16 acc = f32x16{};
  for (int k0 = 0; k0 < d.dh; k0 += 16) {
    const bf8 av = *reinterpret_cast<const bf8*>(qrow + k0);
    const bf8 bv = *reinterpret_cast<const bf8*>(&bt[m * bs + k0 + 8 * j]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  }
  // lane: channel m of rows acc_row(v, lane); the rotation pairs channels
  // m and m ^ s (lanes m ^ s of the same half)
  const float cst = (d.rotate ? inv_sqrt_pow2(8) : 1.0f) * qscale;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float x = acc[v];
    if (d.rotate) {
#pragma unroll
      for (int st = 1; st < 8; st <<= 1) {
        const float p = __shfl_xor(x, st);
        x = (m & st) ? p - x : x + p;
      }
    }
    const int r = r0 + acc_row(v, lane);
    if (r < rows) qn[((size_t)r * d.Hq + h) * 32 + m] = (_Float16)(x * cst);
  }
}

// ------------------------------------------------------------------ vproj --

// Element (row, head h, channel 32 kb + 16 j + 8 s + 4 i + e) of the
// attention rows, in the order the up-projection's MFMA A operands are read:
// planes of `rows` x 32 bytes per (h, kb, s, i), so that an operand load of
// 32 consecutive rows reads 1 KB of contiguous memory.
__host__ __device__ inline size_t po_index(const Dims& d, size_t rows, int h, size_t row, int c) {
  const int kb = c >> 5, j = (c >> 4) & 1, s = (c >> 3) & 1, i = (c >> 2) & 1, e = c & 3;
  const size_t plane = (((size_t)h * (d.rv / 32) + kb) * 2 + s) * 2 + i;
  return (plane * rows + row) * 8 + j * 4 + e;
}

// B_v' = B_v with every row put through the block rotation of the stored
// value latents (blocks of mb = the largest power of two dividing R_v / 4,
// scaled by 1/sqrt(mb); the rotation is symmetric), so that
// (o' H) B_v^T = o' B_v'^T: the up-projection then takes the still rotated
// attention rows.  Written as bf16 high and low parts in the order the
// up-projection's MFMA B operands are read (bvr_index), so that every
// operand load reads 1 KB of contiguous memory.  One workgroup per row of
// B_v, 4 channels per thread; strides 1 and 2 inside the thread, strides
// 4 .. mb/2 as lane shuffles (mb <= 256 = one wave).
// Element (row g d_h + 32 ct + m, channel 32 kb + 16 j + 8 s + e) of part
// p (0 high, 1 low) of B_v': blocks of 1 KB per (g, kb, p, ct, s), lane
// (m, j) of a block owning 16 bytes.
__host__ __device__ inline size_t bvr_index(const Dims& d, int g, int n, int c, int p) {
  const int ct = n >> 5, m = n & 31;
  const int kb = c >> 5, j = (c >> 4) & 1, s = (c >> 3) & 1, e = c & 7;
  const size_t blk = ((((size_t)g * (d.rv / 32) + kb) * 2 + p) * (d.dh / 32) + ct) * 2 + s;
  return blk * 512 + (m * 2 + j) * 8 + e;
}

__global__ __launch_bounds__(256) void prefill_rotate_bv_kernel(const uint16_t* __restrict__ bv,
                                                                Dims d,
                                                                uint16_t* __restrict__ bvr,
                                                                _Float16* __restrict__ bvh) {
  const size_t row = blockIdx.x;
  const int t = threadIdx.x, c = 4 * t;
  const int cc = min(c, d.rv - 4);
  const uint16_t* src = bv + row * d.rv + cc;
  float o[4] = {bf16v(src[0]), bf16v(src[1]), bf16v(src[2]), bf16v(src[3])};
  if (d.rotate) {
    const int mb = pow2_divisor(d.rv / 4);
    const float a0 = o[0] + o[1], a1 = o[0] - o[1], a2 = o[2] + o[3], a3 = o[2] - o[3];
    o[0] = a0 + a2; o[1] = a1 + a3; o[2] = a0 - a2; o[3] = a1 - a3;
    for (int hs = 4; hs < mb; hs <<= 1) {
      const int dl = hs >> 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __shfl_xor(o[e], dl);
        o[e] = (c & hs) ? p - o[e] : o[e] + p;
      }
    }
    const float cst = inv_sqrt_pow2(mb);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] *= cst;
  }
  if (c < d.rv && bvh) {
    // (B_v H) as fp16 rows [Hkv d_h][R_v], for the value reconstruction
#pragma unroll
    for (int e = 0; e < 4; ++e) bvh[row * d.rv + c + e] = (_Float16)o[e];
  } else if (c < d.rv) {
    const int g = (int)(row / d.dh), n = (int)(row % d.dh);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const __bf16 hi = (__bf16)o[e];
      const __bf16 lo = (__bf16)(o[e] - (float)hi);
      bvr[bvr_index(d, g, n, c + e, 0)] = __builtin_bit_cast(uint16_t, hi);
      bvr[bvr_index(d, g, n, c + e, 1)] = __builtin_bit_cast(uint16_t, lo);
    }
  }
}

// out[row][h][r] = (sum_c po[row, h, c] B_v'[g d_h + r][c]) / l[row][h]: the
// attention rows (unnormalised, still rotated, in the order of po_index)
// times the rotated factor, divided by the softmax denominator.  One workgroup per
// (128 rows, head): 4 waves of 32 rows x d_h columns on MFMA 32x32x16 bf16
// over K = R_v in steps of one channel block; lane (m, j) reads channels
// 16 j .. 16 j + 15 of its row, MFMA s of a step takes channels 16 j + 8 s ..
// in k-slot j.  The fp32 rows are split into bf16 high and low parts: three
// products per step (low x low dropped).
template <int NCT>
__global__ __launch_bounds__(256) void prefill_vproj_kernel(const float* __restrict__ po,
                                                            const float* __restrict__ pml,
                                                            const uint16_t* __restrict__ bvr,
                                                            Dims d, int rows,
                                                            float* __restrict__ out) {
  const int h = blockIdx.y, g = h / d.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, j = lane >> 5;
  const int r0 = blockIdx.x * 128 + wave * 32;
  // this lane's 16 bytes of every operand plane (kb, s, i) of head h
  const float* arow = po + po_index(d, rows, h, min(r0 + m, rows - 1), 16 * j);
  const size_t pstride = (size_t)rows * 8;    // floats from one plane to the next
  // this lane's 16 bytes of every B_v' operand block of head group g
  const uint16_t* bg = bvr + (size_t)g * (d.rv / 32) * 2 * NCT * 2 * 512 + (m * 2 + j) * 8;
  f32x16 acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x16{};
  for (int k0 = 0; k0 < d.rv; k0 += 32) {
    f32x4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)   // plane (kb, s = i / 2, i % 2)
      x[i] = *reinterpret_cast<const f32x4*>(arow + ((size_t)(k0 / 32) * 4 + i) * pstride);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf8 ah, al;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = x[2 * st + (e >> 2)][e & 3];
        ah[e] = (__bf16)xv;
        al[e] = (__bf16)(xv - (float)ah[e]);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        // blocks (kb, p, ct, s) of bvr_index
        const uint16_t* bo = bg + ((((size_t)(k0 / 32) * 2) * NCT + ct) * 2 + st) * 512;
        const bf8 bh = *reinterpret_cast<const bf8*>(bo);
        const bf8 bl = *reinterpret_cast<const bf8*>(bo + (size_t)NCT * 2 * 512);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[ct], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = r0 + acc_row(v, lane);
    if (r >= rows) continue;
    const float l = pml[((size_t)r * d.Hq + h) * 2 + 1];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      out[((size_t)r * d.Hq + h) * d.dh + ct * 32 + m] = acc[ct][v] * inv;
  }
}

hipError_t launch_prefill_vproj(const Dims& d, int rows, const float* po, const float* pml,
                                const uint16_t* bvr, float* out, hipStream_t s) {
  const dim3 grid((rows + 127) / 128, d.Hq);
  switch (d.dh / 32) {
    case 2: prefill_vproj_kernel<2><<<grid, 256, 0, s>>>(po, pml, bvr, d, rows, out); break;
    case 4: prefill_vproj_kernel<4><<<grid, 256, 0, s>>>(po, pml, bvr, d, rows, out); break;
    case 6: prefill_vproj_kernel<6><<<grid, 256, 0, s>>>(po, pml, bvr, d, rows, out); break;
    case 8: prefill_vproj_kernel<8><<<grid, 256, 0, s>>>(po, pml, bvr, d, rows, out); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------- attn --

// A workgroup's stacked P tile has 128 rows: kPQ queries x kPH query heads.
// Both depend on the width DK of the keys it scores against (32 latent
// channels, or d_h channels of rotary keys), so that one tile's keys of the
// workgroup's KV heads stay within kKeySlot.
constexpr int kRows = 128;
constexpr int kPHof(int dk) { return dk == 32 ? 8 : 256 / dk; }   // query heads
constexpr int kPQof(int dk) { return kRows / kPHof(dk); }          // queries
constexpr int kPS = 72;       // P row stride (halves)
constexpr int kMaxRv = 1024;
constexpr int kMaxCols = 512;      // value columns per workgroup (at most)
// bytes of one tile's value scales (or zeros) over the workgroup's groups
constexpr int kMetaHalf = (kMaxCols / 32) * kTile * 2;
// bytes of one tile's value codes over the workgroup's groups: at most 16
// groups of 1024 B (a uniform 4-bit cache; a 4/3-bit block of 512 columns
// holds at most eight 4-bit and eight 3-bit groups, 14 KB)
constexpr int kCodeSlot = 16 * 1024;
// bytes of one tile's fp16 keys of the workgroup's KV heads (8 KV heads of
// 32 latent channels, or 256 / d_h heads of d_h rotary-key channels)
constexpr int kKeySlot = 32 * 1024;

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

struct AttnArgs {
  Dims d;
  int ctx, chunk, n_qb, n_qb_pad, n_hg, n_cb;
  const uint8_t* value;
  const uint16_t* vmeta;
  const _Float16* qn;     // [B*C][Hq][DK] query latents, natural channel order
  const _Float16* kd;     // [B][T_max][Hkv][DK] fp16 keys
  float* part_o;          // B*C x Hq rows of R_v, element order of po_index
  float* part_ml;         // [B*C][Hq][2]
};

// Mask and bias registers of the value unpacking: kept in VGPRs (opaque to
// the compiler) so that mask-and-bias is one v_and_or_b32.
struct UnpackRegs {
  uint32_t m4, m3, bias;
};

// Codes of token pair p of a value run as the fp16 bit patterns of 1024 + k
// in both halves (run layout as described at run_pair_inplace).
template <bool kFour>
__device__ inline uint32_t biased_pair(const u32x4& w, int p, const UnpackRegs& u) {
  if constexpr (kFour) {
    return ((w[p >> 2] >> (4 * (p & 3))) & u.m4) | u.bias;
  } else {
    if (p < 15) return ((w[p / 5] >> (3 * (p % 5))) & u.m3) | u.bias;
    return ((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) |
           ((w[2] >> 13) & 0x00040004u) | u.bias;
  }
}

// One MFMA 32x32x16 B operand of value group run `w` (the lane's channel and
// 32-token half): tokens 8r .. 8r + 7 of the run as z + s * code, one packed
// fp16 FMA per token pair.  S, Z: the scales and zeros of those 8 tokens.
// kMask zeroes tokens past `pmax` (tok: the run's token 8r).
template <bool kFour, bool kMask>
__device__ inline h8 value_frag(const u32x4& w, int r, const u32x4& S, const u32x4& Z,
                                int tok, int pmax, const UnpackRegs& u) {
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // codes as exact fp16 integers: (1024 + k) - 1024
    const h2 kv = __builtin_bit_cast(h2, biased_pair<kFour>(w, 4 * r + q, u)) -
                  h2{1024.0f16, 1024.0f16};
    // element picks go through scalars: a bit-cast applied directly to an
    // ext_vector element is lowered as a cast of element 0
    const uint32_t sb = S[q], zb = Z[q];
    h2 v = __builtin_elementwise_fma(kv, __builtin_bit_cast(h2, sb), __builtin_bit_cast(h2, zb));
    if constexpr (kMask) {
      if (tok + 2 * q > pmax) v[0] = (_Float16)0.0f;
      if (tok + 2 * q + 1 > pmax) v[1] = (_Float16)0.0f;
    }
    o[q] = __builtin_bit_cast(uint32_t, v);
  }
  return __builtin_bit_cast(h8, u32x4{o[0], o[1], o[2], o[3]});
}

// Workgroup = (PQ consecutive queries, PH query heads, R_v / n_cb value
// columns, sequence b), 8 waves; PQ x PH = 128 (16 x 8 for DK = 32 latent
// keys, 64 x 2 for rotary keys of d_h = 128).  Rows of the stacked P tile:
// row = query * PH + head (128 rows = four MFMA row tiles).  Wave w
//   - scores query head w % PH for queries 16 (w / PH) .. + 15 on MFMA
//     16x16x32 (DK / 32 steps) with the keys as the A operand (a lane then
//     holds four consecutive tokens of one query) and a lazy online softmax,
//     writing fp16 probabilities to a P slot;
//   - owns value groups 2w and 2w + 1 of the workgroup's columns for all
//     128 rows: it dequantizes their codes with their scales and zeros
//     straight into MFMA B operands and contracts them with P on MFMA
//     32x32x16.  MFMA r of a tile takes, in k-slot j, tokens 32j + 8r ..
//     32j + 8r + 7: word r of the lane's run.
// Keys, codes, scales and zeros reach LDS by direct-to-LDS loads issued a
// step ahead (keys two tiles ahead); P, alpha and every staging buffer are
// double-buffered, so a tile needs one barrier.
// The column blocks compute the same scores; the first writes (m, l).
// Causal mask: query i (absolute position ctx + i) sees cached positions
// 0 .. ctx + i.  Value tokens past the workgroup's last position are zeroed
// so that unwritten cache bytes never reach the MFMA operands.
template <int G, int DK>
__global__ __launch_bounds__(512) void prefill_attn_kernel(AttnArgs a) {
  constexpr int PH = kPHof(DK), PQ = kPQof(DK);
  constexpr int CPT = DK / 8;             // 16-byte chunks per key row
  constexpr int TPP = 1024 / (DK * 2);    // key rows per 1 KB staging piece
  constexpr int KS = DK / 32;             // K steps of a score MFMA
  // swizzle of a key row's chunks: the 16 rows a score operand read takes
  // fall in 16 different groups of 4 banks
  auto swz = [](int u) { return (u / (16 / CPT)) & (CPT - 1); };
  const Dims& d = a.d;
  __shared__ __attribute__((aligned(16))) _Float16 p_l[2][kRows * kPS];
  __shared__ __attribute__((aligned(16))) uint8_t meta_l[2][2 * kMetaHalf];
  __shared__ __attribute__((aligned(16))) uint8_t code_l[2][kCodeSlot];
  // keys [KV head][token][CPT chunks of 16 B], chunk c of token u at
  // position c ^ swz(u) so that a score operand read (16 tokens, one chunk)
  // touches every bank once
  __shared__ __attribute__((aligned(16))) uint8_t key_l[2][kKeySlot];
  __shared__ __attribute__((aligned(16))) float alpha_l[2][kRows];
  __shared__ int flag_l[2];

  // XCD-aware order: the workgroups of one query block (head groups x
  // column blocks) run on one XCD (blockIdx % 8) and share its L2; the query
  // blocks with the longest causal span start first.
  const int L = blockIdx.x;
  const int xcd = L & 7, k = L >> 3;
  const int per_qb = a.n_cb * a.n_hg;
  const int sub = k % per_qb;
  const int hg = sub % a.n_hg, cb = sub / a.n_hg;
  const int qb = a.n_qb_pad - 1 - ((k / per_qb) * 8 + xcd);
  if (qb >= a.n_qb) return;   // padding workgroup; uniform, before any barrier
  const int b = blockIdx.y;
  const int q0 = qb * PQ;
  const int nq = min(PQ, a.chunk - q0);
  const int pfirst = a.ctx + q0;            // first query's position
  const int pmax = pfirst + nq - 1;         // last position any row may see
  const int tile_last = pmax / kTile;
  const int cols = d.rv / a.n_cb, col0 = cb * cols;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, j = lane >> 5;   // 32x32 operand coordinates
  const int c16 = lane & 15, g16 = lane >> 4;  // 16x16 operand coordinates

  if (tid < 2) flag_l[tid] = -1;
  __syncthreads();

  // ------------------------------------------------------------ score setup
  const int hl = wave % PH;                     // query head within the group
  const int qs = wave / PH;                     // the wave's 16 queries
  const int h = hg * PH + hl;
  const int g = h / G;
  const int qi = 16 * qs + c16;                 // the lane's query
  const int R = qi * PH + hl;                   // its row of the P tile
  // B operands of the score MFMA: query qi, channels 32 ks + 8 g16 .. + 7
  h8 bq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bq[ks] = qi < nq ? *reinterpret_cast<const h8*>(
                           a.qn + (((size_t)b * a.chunk + q0 + qi) * d.Hq + h) * DK + 32 * ks +
                           8 * g16)
                     : h8{};
  // lazy softmax state of query c16 (the same in its four lanes).  The
  // running max starts finite so that exp2(x - m) needs no guard: a row's
  // first real score always moves it (alpha = exp2(-1e30 - m) = 0), and rows
  // of padding queries only ever see -inf (p = 0).
  float m_ref = -1e30f, l_lane = 0.0f;
  // P tile: row R, token u stored at chunk (u / 8) ^ (R / 32) of the row, so
  // that the four row tiles' writes fall in different LDS banks
  auto p_at = [&](int slot, int R, int u) -> _Float16* {
    return &p_l[slot][R * kPS + (((u >> 3) ^ (R >> 5)) << 3) + (u & 7)];
  };
  // A operands of the score MFMA: tokens bl * 16 + c16 of a tile, channels
  // 32 ks + 8 g16 .. + 7 of KV head g (local head g - g0); swz(bl * 16 + c16)
  // = swz(c16)
  const int g0 = hg * PH / G;
  const int key_lane = (g - g0) * (kTile * DK * 2) + c16 * (DK * 2);
  auto key_at = [&](int slot, int bl, int ks) {
    return *reinterpret_cast<const h8*>(
        &key_l[slot][key_lane + bl * 16 * (DK * 2) + (((4 * ks + g16) ^ swz(c16)) << 4)]);
  };
  // (latent keys: the next tile's operands are read ahead of its scores;
  // rotary keys: each 16-token block's operands right before its MFMAs)
  constexpr int KK = DK == 32 ? 4 : 1;
  auto load_keys = [&](int slot, h8 (&kk)[KK]) {
    if constexpr (DK == 32) {
#pragma unroll
      for (int bl = 0; bl < 4; ++bl) kk[bl] = key_at(slot, bl, 0);
    }
  };

  // scores of tile `tile` (index it in the loop) into P slot `slot`
  auto score = [&](int tile, int it, int slot, const h8 (&kk)[KK]) {
    float x[4][4];   // [16-token block][token 4 g16 + v], query qi
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
      f32x4v sc;
      if constexpr (DK == 32) {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kk[bl], bq[0], f32x4v{}, 0, 0, 0);
      } else {
        h8 kb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[ks] = key_at(slot, bl, ks);
        sc = f32x4v{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[ks], bq[ks], sc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) x[bl][v] = sc[v];
    }
    if (tile * kTile + kTile - 1 > pfirst) {   // uniform: some token is hidden
      // last token of the tile query qi sees (none for padding queries)
      const int lim = qi < nq ? pfirst + qi - tile * kTile : -1;
#pragma unroll
      for (int bl = 0; bl < 4; ++bl)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          x[bl][v] = bl * 16 + 4 * g16 + v > lim ? -INFINITY : x[bl][v];
    }
    float tmax = x[0][0];
#pragma unroll
    for (int bl = 0; bl < 4; ++bl)
#pragma unroll
      for (int v = 0; v < 4; ++v) tmax = fmaxf(tmax, x[bl][v]);
    float alpha = 1.0f;
    if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kLazy) != 0) {
      float gm = fmaxf(tmax, __shfl_xor(tmax, 16));
      gm = fmaxf(gm, __shfl_xor(gm, 32));
      if (gm > m_ref + kLazy) {        // the same in the query's four lanes
        alpha = __builtin_amdgcn_exp2f(m_ref - gm);
        m_ref = gm;
        l_lane *= alpha;
        flag_l[slot] = it;
      }
    }
    if (lane < 16) alpha_l[slot][R] = alpha;
    float ls = 0.0f;
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[v] = __builtin_amdgcn_exp2f(x[bl][v] - m_ref);
        ls += p[v];
      }
      *reinterpret_cast<h4*>(p_at(slot, R, bl * 16 + 4 * g16)) =
          h4{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    }
    l_lane += ls;
  };

  // ------------------------------------------------------------ value setup
  const int NG = d.rv / 32;           // value groups
  const int NH = d.lob == 4 ? NG : d.rv / 128;   // 4-bit value groups
  const int ngrp = cols / 32, g_first = col0 / 32;
  const size_t vtile_bytes = value_tile_bytes(d.rv, d.lob);
  const size_t mtile = (size_t)2 * NG * kTile;     // fp16 elements
  const int meta_bytes = ngrp * kTile * 2;
  // Direct-to-LDS staging, in 1 KB pieces spread over the waves: the fp16
  // keys of tile `kt` into key slot kt & 1 (CPT pieces per KV head) and the
  // value codes, scales and zeros of tile `ct` into slot ct & 1.  A key
  // piece is TPP tokens of one head; lane l moves chunk
  // (l % CPT) ^ swz(u) of token u = TPP * piece + l / CPT (the swizzle of
  // key_l).
  auto goff = [&](int gi) { return gi < NH ? gi * 1024 : NH * 1024 + (gi - NH) * 768; };
  const int code_lo = goff(g_first), code_bytes = goff(g_first + ngrp) - code_lo;
  constexpr int KVW = PH / G > 0 ? PH / G : 1;   // KV heads of the workgroup
  const int nkp = CPT * KVW;                   // key pieces
  const int ncp = (code_bytes + 1023) / 1024;  // code pieces
  const int nmp = (meta_bytes + 1023) / 1024;  // pieces per scale / zero plane
  const int key_tl = lane / CPT, key_pos = lane % CPT;
  auto dma = [&](const uint8_t* src, uint8_t* dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  // Pieces are numbered keys first (nkp), then codes (ncp), then scales and
  // zeros (nmp each); wave w issues the pieces p with p % 8 == w.  Each kind
  // has its own loop with its base address set up once per call, so a piece
  // costs an address add and the load.
  auto first_piece = [&](int p0) { return p0 + ((wave - p0) & 7); };
  auto stage = [&](int kt, int ct) {
    if (kt <= tile_last) {
      // piece p: KV head g0 + p / CPT, tokens TPP (p % CPT) .. + TPP - 1 of
      // tile kt
      const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.kd) +
          (((size_t)b * d.Tmax + (size_t)kt * kTile) * d.Hkv + g0) * (DK * 2);
      uint8_t* kdst = &key_l[kt & 1][0];
      for (int p = wave; p < nkp; p += 8) {
        const int kh = p / CPT, blk = p % CPT;
        const int u = blk * TPP + key_tl;
        dma(kbase + ((size_t)u * d.Hkv + kh) * (DK * 2) + ((key_pos ^ swz(u)) << 4),
            kdst + kh * (kTile * DK * 2) + blk * 1024);
      }
    }
    if (ct <= tile_last) {
      const size_t ctix = tile_index(d, b, ct);   // the tile's slot or page
      const uint8_t* cbase = a.value + ctix * vtile_bytes + code_lo + lane * 16;
      uint8_t* cdst = &code_l[ct & 1][0];
      for (int p = first_piece(nkp); p < nkp + ncp; p += 8) {
        const int q = p - nkp;
        if (q * 1024 + lane * 16 < code_bytes) dma(cbase + q * 1024, cdst + q * 1024);
      }
      const uint8_t* mbase = reinterpret_cast<const uint8_t*>(
          a.vmeta + ctix * mtile + (size_t)g_first * kTile) + lane * 16;
      uint8_t* mdst = &meta_l[ct & 1][0];
      for (int p = first_piece(nkp + ncp); p < nkp + ncp + 2 * nmp; p += 8) {
        const int q = p - nkp - ncp;
        const int part = q >= nmp ? 1 : 0, piece = q - part * nmp;   // 0 scales, 1 zeros
        if (piece * 1024 + lane * 16 < meta_bytes)
          dma(mbase + (size_t)part * NG * kTile * 2 + piece * 1024,
              mdst + part * kMetaHalf + piece * 1024);
      }
    }
  };
  const int gw = g_first + 2 * wave;          // the wave's first value group
  const bool active = 2 * wave < ngrp;        // uniform
  const bool four = gw < NH;                  // both groups: NH is even
  const int coff0 = goff(gw) - code_lo, coff1 = goff(gw + 1) - code_lo;

  f32x16 acc[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) acc[rt][gp] = f32x16{};

  UnpackRegs ur{0x000F000Fu, 0x00070007u, 0x64006400u};
  __asm__ volatile("" : "+v"(ur.m4), "+v"(ur.m3), "+v"(ur.bias));

  auto run = [&](auto fourc) {
    constexpr bool kFour = decltype(fourc)::value;
    // the lane's runs (channel m, token half j) of its two groups
    auto load_codes = [&](int slot, u32x4 (&dst)[2]) {
      const uint8_t* base = code_l[slot];
      if constexpr (kFour) {
        dst[0] = *reinterpret_cast<const u32x4*>(base + coff0 + lane * 16);
        dst[1] = *reinterpret_cast<const u32x4*>(base + coff1 + lane * 16);
      } else {
        const uint32_t* p0 = reinterpret_cast<const uint32_t*>(base + coff0 + lane * 12);
        const uint32_t* p1 = reinterpret_cast<const uint32_t*>(base + coff1 + lane * 12);
        dst[0] = u32x4{p0[0], p0[1], p0[2], 0u};
        dst[1] = u32x4{p1[0], p1[1], p1[2], 0u};
      }
    };
    auto contract = [&](int slot, int it, int tile, auto maskc) {
      constexpr bool kMask = decltype(maskc)::value;
      u32x4 cw[2];
      load_codes(slot, cw);
      if (__builtin_amdgcn_readfirstlane(flag_l[slot]) == it) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            // rows acc_row(4 k4 + e, lane) = 8 k4 + 4 j + e
            const f32x4v al = *reinterpret_cast<const f32x4v*>(&alpha_l[slot][rt * 32 + k4 * 8 + j * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[rt][0][4 * k4 + e] *= al[e];
              acc[rt][1][4 * k4 + e] *= al[e];
            }
          }
      }
      // P row rt * 32 + m, tokens 32 j + 8 r: chunk (4 j + r) ^ rt = 4 j + (r ^ rt)
      const _Float16* pa = &p_l[slot][m * kPS + 32 * j];
      const uint8_t* ms = meta_l[slot] + (2 * wave) * (kTile * 2) + 64 * j;
      const int tok0 = tile * kTile + 32 * j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        h8 A[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          A[rt] = *reinterpret_cast<const h8*>(pa + rt * 32 * kPS + (r ^ rt) * 8);
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const int mo = gp * (kTile * 2) + 16 * r;
          const u32x4 S = *reinterpret_cast<const u32x4*>(ms + mo);
          const u32x4 Z = *reinterpret_cast<const u32x4*>(ms + kMetaHalf + mo);
          const h8 Bf = value_frag<kFour, kMask>(cw[gp], r, S, Z, tok0 + 8 * r, pmax, ur);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            acc[rt][gp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[rt], Bf, acc[rt][gp], 0, 0, 0);
        }
      }
    };

    // staging runs two tiles ahead for keys, one for values
    stage(0, 0);
    stage(1, tile_last + 1);
    wait_vmcnt<0>();
    __syncthreads();        // keys of tiles 0, 1 and values of tile 0 in LDS
    {
      h8 kk[KK];
      load_keys(0, kk);
      score(0, 0, 0, kk);
    }
    // One tile: contract tile `tile`, then score tile + 1, with the next
    // stage in flight.  Only the workgroup's last tile can hold tokens past
    // its last position, so only it takes the masked value operands.
    auto step = [&](int tile, auto lastc) {
      constexpr bool kLast = decltype(lastc)::value;
      const int it = tile, cur = it & 1, nxt = cur ^ 1;
      lds_barrier();        // P of `tile`, staging of the previous step visible
      if constexpr (!kLast) stage(tile + 2, tile + 1);
      if (active) contract(cur, it, tile, lastc);
      if constexpr (!kLast) {
        __builtin_amdgcn_sched_barrier(0);
        h8 kk[KK];
        load_keys(nxt, kk);
        score(tile + 1, it + 1, nxt, kk);
        wait_vmcnt<0>();    // this wave's staging landed
      }
    };
    for (int tile = 0; tile < tile_last; ++tile) step(tile, std::false_type{});
    step(tile_last, std::true_type{});
  };
  if (four) run(std::true_type{});
  else run(std::false_type{});

  // ---------------------------------------------------------------- output
  if (active) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = rt * 32 + acc_row(v, lane);
          const int rq = rr / PH, hh = rr % PH;
          if (rq < nq)
            a.part_o[po_index(d, (size_t)d.B * a.chunk, hg * PH + hh,
                              (size_t)b * a.chunk + q0 + rq,
                              col0 + (2 * wave + gp) * 32 + m)] = acc[rt][gp][v];
        }
  }
  if (cb == 0) {
    float l = l_lane + __shfl_xor(l_lane, 16);
    l += __shfl_xor(l, 32);
    if (lane < 16 && qi < nq) {
      const size_t o = (((size_t)b * a.chunk + q0 + qi) * d.Hq + h) * 2;
      a.part_ml[o] = m_ref;
      a.part_ml[o + 1] = l;
    }
  }
}

// ------------------------------------------ reconstructed values (prefill) --
//
// eq. 12 read in its left-hand order for the prefill: p_h (Z_v B_v[h]^T).
// Decode contracts P with the joint latent (2 R_v flop per query, head and
// token) because each token meets one query; a chunk's queries share every
// cached token, so reconstructing the values once per call (2 Hkv d_h R_v
// flop per token) and contracting over d_h (2 d_h per pair) is cheaper as
// soon as C Hq (R_v - d_h) > Hkv d_h R_v.  The stored latents are rotated
// (eq. 13), so the factor is rotated the same way: Z H (B_v H)^T = Z B_v^T.

// Element (sequence b, KV head g, position t, channel c) of the
// reconstructed values: per (b, g, 64-position tile) d_h rows of 64
// positions (fp16).  Within a row, position 32 k + 16 h + 4 q + e (h < 2,
// q < 4, e < 4) sits in 16-byte chunk 4 k + q at half h: a chunk holds the
// eight positions one lane of the attention's value operand takes (the
// k-slots of a score MFMA's output).  Chunk p of channel c is stored at
// chunk p ^ ((c >> 1) & 7), so that an operand read of 16 channels touches
// every LDS bank once.
__host__ __device__ inline size_t vrec_index(const Dims& d, int b, int g, int t, int c) {
  const int u = t % kTile, r = u & 31;
  const int chunk = 4 * (u >> 5) + ((r >> 2) & 3);
  return ((((size_t)b * d.Hkv + g) * d.NT + t / kTile) * d.dh + c) * kTile +
         ((chunk ^ ((c >> 1) & 7)) << 3) + 4 * (r >> 4) + (r & 3);
}

// Value latents of positions [0, n) of every sequence, dequantized from the
// stored tiles (z + s * code per 32-channel group), fp16 [B][T_max][R_v]
// (position-major, still rotated).  One thread per (sequence, tile, group,
// channel m, half j): the 32 positions of one value run.
__global__ __launch_bounds__(256) void value_dequant_kernel(const uint8_t* __restrict__ value,
                                                            const uint16_t* __restrict__ vmeta,
                                                            Dims d, int n,
                                                            _Float16* __restrict__ zv) {
  const int NG = d.rv / 32, NH = d.lob == 4 ? NG : d.rv / 128;
  const int ntn = (n + kTile - 1) / kTile;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)d.B * ntn * NG * 64) return;
  const int run = (int)(idx % 64), m = run & 31, j = run >> 5;
  size_t rest = idx / 64;
  const int grp = (int)(rest % NG);
  rest /= NG;
  const int tile = (int)(rest % ntn), b = (int)(rest / ntn);
  const size_t tix = tile_index(d, b, tile);   // the tile's slot or page
  const uint8_t* tb = value + tix * value_tile_bytes(d.rv, d.lob);
  const bool four = grp < NH;
  uint32_t w[4];
  if (four) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(tb + grp * 1024 + run * 16);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(tb + NH * 1024 + (grp - NH) * 768 + run * 12);
    w[0] = p[0]; w[1] = p[1]; w[2] = p[2]; w[3] = 0u;
  }
  const _Float16* meta = reinterpret_cast<const _Float16*>(vmeta) + tix * (size_t)(2 * NG * kTile);
  const _Float16* sc = meta + grp * kTile + 32 * j;
  const _Float16* ze = meta + (NG + grp) * kTile + 32 * j;
  const int t0 = tile * kTile + 32 * j;
  _Float16* dst = zv + ((size_t)b * d.Tmax + t0) * d.rv + grp * 32 + m;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    // codes of positions 2p and 2p + 1 of the run (the run layout of the
    // append: see run_pair_inplace)
    uint32_t c0, c1;
    if (four) {
      c0 = (w[p >> 2] >> (4 * (p & 3))) & 15u;
      c1 = (w[p >> 2] >> (16 + 4 * (p & 3))) & 15u;
    } else if (p < 15) {
      c0 = (w[p / 5] >> (3 * (p % 5))) & 7u;
      c1 = (w[p / 5] >> (16 + 3 * (p % 5))) & 7u;
    } else {
      c0 = ((w[0] >> 15) & 1u) | ((w[1] >> 14) & 2u) | ((w[2] >> 13) & 4u);
      c1 = ((w[0] >> 31) & 1u) | ((w[1] >> 30) & 2u) | ((w[2] >> 29) & 4u);
    }
    // s * code is exact in fp32 and so is the sum with z: one rounding to fp16
    if (t0 + 2 * p < n)
      dst[(size_t)(2 * p) * d.rv] =
          (_Float16)fmaf((float)sc[2 * p], (float)c0, (float)ze[2 * p]);
    if (t0 + 2 * p + 1 < n)
      dst[(size_t)(2 * p + 1) * d.rv] =
          (_Float16)fmaf((float)sc[2 * p + 1], (float)c1, (float)ze[2 * p + 1]);
  }
}

// V^ = Zv (B_v H)^T of one sequence (blockIdx.z), fp16 x fp16 -> fp32 on
// MFMA 32x32x16, written as fp16 in the order of vrec_index for positions
// [0, 64 ceil(n / 64)) (zeros past n: those rows of Zv read as zero).  Both
// operands are read with the reduction index contiguous: Zv [T][R_v] and
// (B_v H) [Hkv d_h][R_v].  Workgroup tile 128 positions x 128 channels, four
// waves in 2 x 2, K steps of 64 through LDS.
constexpr int kRK = 64;       // K step
constexpr int kRS = kRK + 8;  // LDS row stride (fp16): 16-row reads hit 16 bank groups
__global__ __launch_bounds__(256) void value_recon_kernel(const _Float16* __restrict__ zv,
                                                          const _Float16* __restrict__ bvh,
                                                          Dims d, int n,
                                                          _Float16* __restrict__ vt) {
  __shared__ __attribute__((aligned(16))) _Float16 as[kGT * kRS];
  __shared__ __attribute__((aligned(16))) _Float16 bs[kGT * kRS];
  const int b = blockIdx.z, t0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  const int N = d.Hkv * d.dh, K = d.rv;
  const int tend = ((n + kTile - 1) / kTile) * kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m = lane & 31, j = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
  // one K step: 128 rows x 64 channels of each operand = 1024 runs of 16 B
  u32x4 ar[4], br[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 3, kc = (c & 7) * 8;
      const int t = t0 + r, col = n0 + r;
      ar[i] = t < n ? *reinterpret_cast<const u32x4*>(zv + ((size_t)b * d.Tmax + t) * K + k0 + kc)
                    : u32x4{0u, 0u, 0u, 0u};
      br[i] = col < N ? *reinterpret_cast<const u32x4*>(bvh + (size_t)col * K + k0 + kc)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  };
  load(0);
  for (int k0 = 0; k0 < K; k0 += kRK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&as[r * kRS + kc]) = ar[i];
      *reinterpret_cast<u32x4*>(&bs[r * kRS + kc]) = br[i];
    }
    __syncthreads();
    if (k0 + kRK < K) load(k0 + kRK);
#pragma unroll
    for (int s = 0; s < kRK / 16; ++s) {
      h8 af[2], bf[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        af[x] = *reinterpret_cast<const h8*>(&as[(wm * 64 + x * 32 + m) * kRS + s * 16 + j * 8]);
        bf[x] = *reinterpret_cast<const h8*>(&bs[(wn * 64 + x * 32 + m) * kRS + s * 16 + j * 8]);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[x], bf[y], acc[x][y], 0, 0, 0);
    }
  }
  // lane (m, j): channel column m of its tiles; registers 4q .. 4q + 3 are
  // positions 8q + 4j .. + 3 of the tile, adjacent in vrec_index order: one
  // 8-byte store each
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int col = n0 + wn * 64 + y * 32 + m;
    if (col >= N) continue;
    const int g = col / d.dh, c = col % d.dh;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + wm * 64 + x * 32 + 8 * q + 4 * j;
        if (t >= tend) continue;
        const h4 v = h4{(_Float16)acc[x][y][4 * q], (_Float16)acc[x][y][4 * q + 1],
                        (_Float16)acc[x][y][4 * q + 2], (_Float16)acc[x][y][4 * q + 3]};
        *reinterpret_cast<h4*>(vt + vrec_index(d, b, g, t, c)) = v;
      }
  }
}

struct RecArgs {
  Dims d;
  int ctx, chunk, n_qb, n_qb_pad;
  const _Float16* qn;     // [B*C][Hq][DK] query latents (or rotary queries)
  const _Float16* kd;     // [B][T_max][Hkv][DK] fp16 key latents (or rotary keys)
  const _Float16* vt;     // reconstructed values, vrec_index order
  float* out;             // [B*C][Hq][d_h]
};

// Workgroup = (16 NW / G consecutive queries, the G query heads of one KV
// head g, sequence b), NW waves.  Wave w owns query head w % G for queries
// 16 (w / G) .. + 15 from end to end: it scores them as prefill_attn_kernel
// does (MFMA 16x16x32 over DK key channels, keys as the A operand, lazy
// online softmax), keeps the probabilities in registers and contracts them
// with the KV head's reconstructed values on MFMA 16x16x32 (DH / 16 channel
// tiles, two K steps of 32 positions per tile).  A score MFMA leaves a lane
// four consecutive positions 16 bl + 4 g16 .. + 3 of query c16: those of
// blocks 2k and 2k + 1 are the lane's eight k-values of K step k (A
// operand), and the value operand takes the same positions in the same
// k-slots (two 8-byte reads).  Waves share only the staging: keys and value
// tiles reach LDS by direct-to-LDS loads one tile ahead, one barrier per
// tile.  The rows are divided by their softmax denominators and written to
// out: no partial rows, no up-projection.
template <int G, int DK, int DH, int NW>
__global__ __launch_bounds__(64 * NW) void prefill_attn_rec_kernel(RecArgs a) {
  constexpr int PH = G, PQ = 16 * NW / G;
  constexpr int CPT = DK / 8;             // 16-byte chunks per key row
  constexpr int TPP = 1024 / (DK * 2);    // key rows per 1 KB staging piece
  constexpr int KS = DK / 32;             // K steps of a score MFMA
  constexpr int NCT = DH / 16;            // channel tiles of the contraction
  auto swz = [](int u) { return (u / (16 / CPT)) & (CPT - 1); };
  const Dims& d = a.d;
  __shared__ __attribute__((aligned(16))) uint8_t key_l[2][kTile * DK * 2];
  __shared__ __attribute__((aligned(16))) _Float16 v_l[2][DH * kTile];

  // XCD-aware order (workgroup L runs on XCD L mod 8), the query blocks
  // with the longest causal span first.  With a multiple of 8 KV heads, XCD
  // x takes heads x, x + 8, .., one after the other, each with all of its
  // query blocks: the workgroups that run on an XCD at the same time stream
  // the same key and value tiles through its L2.  Otherwise the KV heads of
  // one query block share an XCD.
  const int L = blockIdx.x;
  const int xcd = L & 7, k = L >> 3;
  int g, qb;
  if (d.Hkv % 8 == 0) {
    g = (k / a.n_qb_pad) * 8 + xcd;
    qb = a.n_qb_pad - 1 - k % a.n_qb_pad;
  } else {
    g = k % d.Hkv;
    qb = a.n_qb_pad - 1 - ((k / d.Hkv) * 8 + xcd);
  }
  if (qb >= a.n_qb) return;   // padding workgroup; uniform, before any barrier
  const int b = blockIdx.y;
  const int q0 = qb * PQ;
  const int nq = min(PQ, a.chunk - q0);
  const int pfirst = a.ctx + q0;
  const int pmax = pfirst + nq - 1;
  const int tile_last = pmax / kTile;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g16 = lane >> 4;

  // ------------------------------------------------------------ score setup
  const int hl = wave % PH, qs = wave / PH;
  const int h = g * G + hl;
  const int qw = 16 * qs;                       // the wave's first query
  const int qi = qw + c16;                      // the lane's query (scores)
  h8 bq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bq[ks] = qi < nq ? *reinterpret_cast<const h8*>(
                           a.qn + (((size_t)b * a.chunk + q0 + qi) * d.Hq + h) * DK + 32 * ks +
                           8 * g16)
                     : h8{};
  // lazy softmax state of query qi (the same in its four lanes); the running
  // max starts finite so that exp2(x - m) needs no guard
  float m_ref = -1e30f, l_lane = 0.0f;
  const int key_lane = c16 * (DK * 2);
  auto key_at = [&](int slot, int bl, int ks) {
    return *reinterpret_cast<const h8*>(
        &key_l[slot][key_lane + bl * 16 * (DK * 2) + (((4 * ks + g16) ^ swz(c16)) << 4)]);
  };
  // value operand of K step kk for channel c: positions 32 kk + 4 g16 .. + 3
  // and 32 kk + 16 + 4 g16 .. + 3, one chunk (4 kk + g16) of the row
  auto v_at = [&](int slot, int c, int kk) {
    return *reinterpret_cast<const h8*>(
        &v_l[slot][c * kTile + (((4 * kk + g16) ^ ((c >> 1) & 7)) << 3)]);
  };

  // ---------------------------------------------------------------- staging
  const int key_tl = lane / CPT, key_pos = lane % CPT;
  auto dma = [&](const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  constexpr int nkp = CPT, nvp = DH / 8;
  auto stage = [&](int t) {   // keys and values of tile t into slot t & 1
    if (t > tile_last) return;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.kd) +
        (((size_t)b * d.Tmax + (size_t)t * kTile) * d.Hkv + g) * (DK * 2);
    for (int p = wave; p < nkp; p += NW) {
      const int u = p * TPP + key_tl;
      dma(kbase + (size_t)u * d.Hkv * (DK * 2) + ((key_pos ^ swz(u)) << 4),
          &key_l[t & 1][p * 1024]);
    }
    const uint8_t* vbase =
        reinterpret_cast<const uint8_t*>(a.vt + vrec_index(d, b, g, t * kTile, 0)) + lane * 16;
    uint8_t* vdst = reinterpret_cast<uint8_t*>(&v_l[t & 1][0]);
    for (int p = nkp + ((wave - nkp) & (NW - 1)); p < nkp + nvp; p += NW)
      dma(vbase + (p - nkp) * 1024, vdst + (p - nkp) * 1024);
  };

  f32x4v acc[NCT];
#pragma unroll
  for (int t = 0; t < NCT; ++t) acc[t] = f32x4v{};

  stage(0);
  wait_vmcnt<0>();
  for (int tile = 0; tile <= tile_last; ++tile) {
    const int slot = tile & 1;
    lds_barrier();        // this tile's staging visible; the other slot free
    stage(tile + 1);
    // scores of the tile: x[bl][v] = position 16 bl + 4 g16 + v, query qi
    // (K-step-major: each step's four key operands are read before its four
    // MFMAs, which go to four different accumulators)
    float x[4][4];
    f32x4v sc[4] = {f32x4v{}, f32x4v{}, f32x4v{}, f32x4v{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      h8 kb[4];
#pragma unroll
      for (int bl = 0; bl < 4; ++bl) kb[bl] = key_at(slot, bl, ks);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bl = 0; bl < 4; ++bl)
        sc[bl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[bl], bq[ks], sc[bl], 0, 0, 0);
    }
#pragma unroll
    for (int bl = 0; bl < 4; ++bl)
#pragma unroll
      for (int v = 0; v < 4; ++v) x[bl][v] = sc[bl][v];
    if (tile * kTile + kTile - 1 > pfirst) {   // uniform: some token is hidden
      const int lim = qi < nq ? pfirst + qi - tile * kTile : -1;
#pragma unroll
      for (int bl = 0; bl < 4; ++bl)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          x[bl][v] = bl * 16 + 4 * g16 + v > lim ? -INFINITY : x[bl][v];
    }
    float tmax = x[0][0];
#pragma unroll
    for (int bl = 0; bl < 4; ++bl)
#pragma unroll
      for (int v = 0; v < 4; ++v) tmax = fmaxf(tmax, x[bl][v]);
    if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kLazy) != 0) {
      float gm = fmaxf(tmax, __shfl_xor(tmax, 16));
      gm = fmaxf(gm, __shfl_xor(gm, 32));
      float alpha = 1.0f;
      if (gm > m_ref + kLazy) {        // the same in the query's four lanes
        alpha = __builtin_amdgcn_exp2f(m_ref - gm);
        m_ref = gm;
        l_lane *= alpha;
      }
      // accumulator rows are queries qw + 4 g16 + v: their alphas sit in
      // lanes 4 g16 + v
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = __shfl(alpha, 4 * g16 + v);
#pragma unroll
        for (int t = 0; t < NCT; ++t) acc[t][v] *= av;
      }
    }
    h8 A[2];
    float ls = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(x[2 * kk + (e >> 2)][e & 3] - m_ref);
        ls += p[e];
      }
      A[kk] = h8{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                 (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
    }
    l_lane += ls;
    // P (16 queries x 64 positions) times the tile's values, four channel
    // tiles at a time: their eight operand reads are issued before their
    // eight MFMAs, which go K-step-major so that consecutive MFMAs are
    // independent
#pragma unroll
    for (int t0 = 0; t0 < NCT; t0 += 4) {
      h8 vo[4][2];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) vo[t][kk] = v_at(slot, 16 * (t0 + t) + c16, kk);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t0 + t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[kk], vo[t][kk], acc[t0 + t], 0, 0, 0);
    }
    wait_vmcnt<0>();      // this wave's staging of the next tile landed
  }

  // ---------------------------------------------------------------- output
  float l = l_lane + __shfl_xor(l_lane, 16);
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rq = qw + 4 * g16 + v;            // this register's query
    const float lv = __shfl(l, 4 * g16 + v);
    if (rq < nq) {
      const float inv = 1.0f / lv;
      float* o = a.out + (((size_t)b * a.chunk + q0 + rq) * d.Hq + h) * DH;
#pragma unroll
      for (int t = 0; t < NCT; ++t) o[16 * t + c16] = acc[t][v] * inv;
    }
  }
}

// Width of the keys the attention kernel scores against: the 32 latent
// channels, or the d_h channels of reconstructed rotary keys.
int attn_key_width(const Dims& d) { return d.rope_theta > 0.0f ? d.dh : 32; }

template <int DK>
hipError_t launch_attn_dk(const Dims& d, dim3 grid, const AttnArgs& aa, hipStream_t s) {
  switch (d.G) {
    case 1: prefill_attn_kernel<1, DK><<<grid, 512, 0, s>>>(aa); break;
    case 2: prefill_attn_kernel<2, DK><<<grid, 512, 0, s>>>(aa); break;
    case 4: prefill_attn_kernel<4, DK><<<grid, 512, 0, s>>>(aa); break;
    case 8: prefill_attn_kernel<8, DK><<<grid, 512, 0, s>>>(aa); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_attn(const Dims& d, dim3 grid, const AttnArgs& aa, hipStream_t s) {
  switch (attn_key_width(d)) {
    case 32: return launch_attn_dk<32>(d, grid, aa, s);
    case 64: return launch_attn_dk<64>(d, grid, aa, s);
    case 128: return launch_attn_dk<128>(d, grid, aa, s);
    default: return hipErrorNotSupported;
  }
}

template <int DK, int DH, int NW>
hipError_t launch_rec_dk(const Dims& d, dim3 grid, const RecArgs& ra, hipStream_t s) {
  switch (d.G) {
    case 1: prefill_attn_rec_kernel<1, DK, DH, NW><<<grid, 64 * NW, 0, s>>>(ra); break;
    case 2: prefill_attn_rec_kernel<2, DK, DH, NW><<<grid, 64 * NW, 0, s>>>(ra); break;
    case 4: prefill_attn_rec_kernel<4, DK, DH, NW><<<grid, 64 * NW, 0, s>>>(ra); break;
    case 8: prefill_attn_rec_kernel<8, DK, DH, NW><<<grid, 64 * NW, 0, s>>>(ra); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

// Waves of a reconstructed-value attention workgroup (16 rows each): 16,
// four per SIMD (every variant fits 128 VGPRs)
int rec_waves(const Dims&) { return 16; }

hipError_t launch_rec(const Dims& d, dim3 grid, const RecArgs& ra, hipStream_t s) {
  const int dk = attn_key_width(d);
  if (dk == 32 && d.dh == 64) return launch_rec_dk<32, 64, 16>(d, grid, ra, s);
  if (dk == 32 && d.dh == 128) return launch_rec_dk<32, 128, 16>(d, grid, ra, s);
  if (dk == 64 && d.dh == 64) return launch_rec_dk<64, 64, 16>(d, grid, ra, s);
  if (dk == 128 && d.dh == 128) return launch_rec_dk<128, 128, 16>(d, grid, ra, s);
  return hipErrorNotSupported;
}

}  // namespace

static size_t align256p(size_t x) { return (x + 255) & ~(size_t)255; }

bool prefill_reconstructs(const Dims& d, int chunk) {
  // the chunk's queries outweigh one reconstruction of every position's
  // values: C Hq (R_v - d_h) > Hkv d_h R_v (flop per cached position)
  return (d.dh == 64 || d.dh == 128) && d.rv > d.dh &&
         (int64_t)chunk * d.Hq * (d.rv - d.dh) > (int64_t)d.Hkv * d.dh * d.rv;
}

PrefillWs prefill_ws_layout(const Dims& d, int chunk) {
  PrefillWs w;
  const size_t M = (size_t)d.B * chunk;
  const bool rec = prefill_reconstructs(d, chunk);
  size_t off = 0;
  w.zk = off;
  off += align256p(M * d.Hkv * d.rk * 4);
  w.zv = off;
  off += align256p(M * d.rv * 4);
  const int dk = attn_key_width(d);
  w.qt = off;   // fp16 query latents (or rotary queries) [rows][Hq][dk]
  off += align256p(M * d.Hq * dk * 2);
  w.kd = off;   // fp16 key latents (or rotary keys) of every cached position, [B][T_max][Hkv][dk]
  off += align256p((size_t)d.B * d.Tmax * d.Hkv * dk * 2);
  w.part_o = w.part_ml = w.bvr = w.zvd = w.bvh = w.vt = 0;
  if (rec) {
    w.zvd = off;  // fp16 value latents of every position, [B][T_max][R_v]
    off += align256p((size_t)d.B * d.Tmax * d.rv * 2);
    w.bvh = off;  // rotated value factor as fp16 rows
    off += align256p((size_t)d.Hkv * d.dh * d.rv * 2);
    w.vt = off;   // reconstructed values, vrec_index order
    off += align256p((size_t)d.B * d.NT * kTile * d.Hkv * d.dh * 2);
  } else {
    w.part_o = off;
    off += align256p(M * d.Hq * d.rv * 4);
    w.part_ml = off;
    off += align256p(M * d.Hq * 2 * 4);
    w.bvr = off;  // rotated value factor, bf16 high then low parts
    off += align256p((size_t)2 * d.Hkv * d.dh * d.rv * 2);
  }
  w.total = off;
  return w;
}

bool prefill_supported(const Dims& d) {
  // rotary keys: reconstructed at d_h = 64 or 128 channels
  if (d.rope_theta > 0.0f && d.dh != 64 && d.dh != 128) return false;
  return d.dtype == STARKV_CACHE_Q43 && d.rk == 32 && d.Hq % kPHof(attn_key_width(d)) == 0 &&
         (d.G == 1 || d.G == 2 || d.G == 4 || d.G == 8) && d.rv % 256 == 0 &&
         d.rv <= kMaxRv && d.dh % 64 == 0 && d.dh <= 256;
}

hipError_t launch_prefill(const Dims& d, const starkv_cache& cache, int ctx_len,
                          int chunk, const void* x, int hidden, const void* ak,
                          const void* av, const void* q, const void* bk,
                          const void* bv, float sm_scale, float* out,
                          float* z_debug, char* ws, const PrefillWs& lay,
                          hipStream_t s, hipEvent_t* ev) {
  if (!prefill_supported(d)) return hipErrorNotSupported;
  auto mark = [&](int i) { if (ev) (void)hipEventRecord(ev[i], s); };
  mark(0);
  const int M = d.B * chunk;
  float* zk = reinterpret_cast<float*>(ws + lay.zk);
  float* zv = reinterpret_cast<float*>(ws + lay.zv);

  // Z = X A for both projections
  GemmArgs ga;
  ga.x = static_cast<const uint16_t*>(x);
  ga.a[0] = static_cast<const uint16_t*>(ak);
  ga.a[1] = static_cast<const uint16_t*>(av);
  ga.z[0] = zk;
  ga.z[1] = zv;
  ga.zdbg = z_debug;
  ga.M = M;
  ga.D = hidden;
  ga.N[0] = d.Hkv * d.rk;
  ga.N[1] = d.rv;
  ga.off[0] = 0;
  ga.off[1] = d.Hkv * d.rk;
  ga.ldd = d.Hkv * d.rk + d.rv;
  const int nmax = ga.N[0] > ga.N[1] ? ga.N[0] : ga.N[1];
  ga.nx = (nmax + kGT - 1) / kGT;
  ga.ny = (M + kGT - 1) / kGT;
  gemm_bf16_kernel<<<(unsigned)(2 * ga.nx * ((ga.ny + 7) / 8 * 8)), 256, 0, s>>>(ga);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(1);

  // rotate, quantize and append the chunk at [ctx_len, ctx_len + chunk)
  e = launch_append(d, cache, zk, zv, ctx_len, chunk, s);
  if (e != hipSuccess) return e;
  mark(2);

  _Float16* kd = reinterpret_cast<_Float16*>(ws + lay.kd);
  _Float16* qn = reinterpret_cast<_Float16*>(ws + lay.qt);
  const int n = ctx_len + chunk;
  if (d.rope_theta > 0.0f) {
    // rotary keys of every position the chunk's queries can see, and the
    // chunk's rotary queries
    const double log2_theta = log2((double)d.rope_theta);
    rope_key_kernel<<<dim3((n + kTile - 1) / kTile, d.Hkv, d.B), 256, 0, s>>>(
        static_cast<const uint8_t*>(cache.key), static_cast<const u32x2*>(cache.key_meta),
        static_cast<const uint16_t*>(bk), d, n, log2_theta, kd);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t items = (size_t)M * d.Hq * (d.dh / 2);
    rope_query_kernel<<<(unsigned)((items + 255) / 256), 256, 0, s>>>(
        static_cast<const uint16_t*>(q), d, M, chunk, ctx_len, log2_theta, sm_scale * kLog2e,
        qn);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    // fp16 key latents of every position the chunk's queries can see
    const size_t items = (size_t)d.B * n * d.Hkv;
    key_dequant_kernel<<<(unsigned)((items + 255) / 256), 256, 0, s>>>(
        static_cast<const uint8_t*>(cache.key), static_cast<const u32x2*>(cache.key_meta), d, n, kd);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // query latents of every (query, head) of the chunk
    prefill_qproj_kernel<<<dim3((M + 127) / 128, d.Hq), 256, 0, s>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(bk), d, M,
        sm_scale * kLog2e, qn);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (prefill_reconstructs(d, chunk)) {
    // values of every visible position reconstructed once (eq. 12, left-hand
    // order), then attention straight into out
    _Float16* zvd = reinterpret_cast<_Float16*>(ws + lay.zvd);
    _Float16* bvh = reinterpret_cast<_Float16*>(ws + lay.bvh);
    _Float16* vt = reinterpret_cast<_Float16*>(ws + lay.vt);
    const int ntn = (n + kTile - 1) / kTile;
    const size_t vitems = (size_t)d.B * ntn * (d.rv / 32) * 64;
    value_dequant_kernel<<<(unsigned)((vitems + 255) / 256), 256, 0, s>>>(
        static_cast<const uint8_t*>(cache.value), static_cast<const uint16_t*>(cache.value_meta),
        d, n, zvd);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    prefill_rotate_bv_kernel<<<d.Hkv * d.dh, 256, 0, s>>>(static_cast<const uint16_t*>(bv), d,
                                                           nullptr, bvh);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    value_recon_kernel<<<dim3((d.Hkv * d.dh + kGT - 1) / kGT, (ntn * kTile + kGT - 1) / kGT, d.B),
                         256, 0, s>>>(zvd, bvh, d, n, vt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    mark(3);
    RecArgs ra;
    ra.d = d;
    ra.ctx = ctx_len;
    ra.chunk = chunk;
    const int pq = 16 * rec_waves(d) / d.G;   // queries per workgroup
    ra.n_qb = (chunk + pq - 1) / pq;
    ra.n_qb_pad = (ra.n_qb + 7) / 8 * 8;
    ra.qn = qn;
    ra.kd = kd;
    ra.vt = vt;
    ra.out = out;
    e = launch_rec(d, dim3(ra.n_qb_pad * d.Hkv, d.B), ra, s);
    if (e != hipSuccess) return e;
    mark(4);
    mark(5);
    return hipSuccess;
  }
  mark(3);

  // causal latent attention
  AttnArgs aa;
  aa.d = d;
  aa.ctx = ctx_len;
  aa.chunk = chunk;
  const int pq = kPQof(attn_key_width(d)), ph = kPHof(attn_key_width(d));
  aa.n_qb = (chunk + pq - 1) / pq;
  aa.n_qb_pad = (aa.n_qb + 7) / 8 * 8;
  aa.n_hg = d.Hq / ph;
  aa.n_cb = d.rv > kMaxCols ? 2 : 1;
  aa.value = static_cast<const uint8_t*>(cache.value);
  aa.vmeta = static_cast<const uint16_t*>(cache.value_meta);
  aa.qn = qn;
  aa.kd = kd;
  aa.part_o = reinterpret_cast<float*>(ws + lay.part_o);
  aa.part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
  e = launch_attn(d, dim3(aa.n_qb_pad * aa.n_hg * aa.n_cb, d.B), aa, s);
  if (e != hipSuccess) return e;
  mark(4);

  // up-project per head through the rotated factor and normalise
  uint16_t* bvr = reinterpret_cast<uint16_t*>(ws + lay.bvr);
  prefill_rotate_bv_kernel<<<d.Hkv * d.dh, 256, 0, s>>>(static_cast<const uint16_t*>(bv), d, bvr,
                                                         nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_prefill_vproj(d, M, aa.part_o, aa.part_ml, bvr, out, s);
  mark(5);
  return e;
}

}  // namespace starkv
