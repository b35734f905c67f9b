// Chunked causal prefill over the latent cache: steps 1-3 of Algorithm 2 in
// the technical review of arXiv 2606.08382 (project the chunk's hidden states
// into the latent space, rotate, quantize and append), then causal attention
// of the chunk's queries through the stored, quantized cache.
//
//   gemm      Z = X [A_key | A_value] (bf16 in, fp32 out) on MFMA 32x32x16
//   append    the decode-path append kernels (rotation + 4/3-bit packing)
//   qproj     q~ for every query of the chunk on MFMA (natural channel order)
//   attn      per (16 queries, 8 query heads, up to 512 value columns):
//             latent scores on MFMA with a lazy online softmax, then P Z_v
//             on MFMA with each wave dequantizing its own value groups
//             straight into MFMA operands (section 5.3, eq. 12)
//   vproj     the attention rows times the value factor rotated like the
//             stored latents, on MFMA, divided by the softmax denominator
#include <type_traits>

#include "device.h"

namespace starkv {
namespace {

// ------------------------------------------------------------------- gemm --

// Z[mat] [M][N] = X [M][D] * A[mat] [D][N], bf16 x bf16 -> fp32.  blockIdx.z
// selects the key or the value projection.  Workgroup tile 128 x 128, four
// waves in 2 x 2, each 2 x 2 MFMA 32x32x16 tiles; K steps of 32 staged
// through LDS.  X tiles are read as 16-byte k-runs; A is kept k-major in LDS
// and a lane gathers its 8 k-values of one column with 2-byte reads.
struct GemmArgs {
  const uint16_t* x;
  const uint16_t* a[2];
  float* z[2];
  float* zdbg;       // optional [M][ldd] copy of both outputs side by side
  int M, D, N[2], off[2], ldd;
};
constexpr int kGT = 128;          // workgroup tile (rows and columns)
constexpr int kGK = 32;           // K step
constexpr int kGXS = kGK + 8;     // X tile row stride (bf16)
constexpr int kGAS = kGT + 8;     // A tile row stride (bf16)

__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kGT * kGXS];
  __shared__ __attribute__((aligned(16))) uint16_t as[kGK * kGAS];
  const int mat = blockIdx.z;
  const int N = g.N[mat];
  const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  if (n0 >= N) return;   // the other projection is wider; uniform exit
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

// fp16 key latents z + s * code of positions [0, n) of every sequence and KV
// head, channels in their natural order: [B][T_max][Hkv][32] (64 bytes per
// token and head).  One thread per (sequence, position, KV head).  The
// attention kernel reads them as MFMA operands.
__global__ __launch_bounds__(256) void key_dequant_kernel(const uint8_t* __restrict__ key,
                                                          const u32x2* __restrict__ kmeta,
                                                          Dims d, int n,
                                                          _Float16* __restrict__ kd) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)d.B * n * d.Hkv) return;
  const int h = idx % d.Hkv;
  const int t = (idx / d.Hkv) % n;
  const int b = idx / ((size_t)d.Hkv * n);
  const int tile = t / kTile, u = t % kTile;
  const size_t blk = ((size_t)b * d.NT + tile) * d.Hkv + h;
  const uint8_t* kb = key + blk * kKeyBlock;
  const uint32_t whi = reinterpret_cast<const uint32_t*>(kb)[u];
  const uint32_t w0 = reinterpret_cast<const uint32_t*>(kb + 256)[u];
  const uint32_t w1 = reinterpret_cast<const uint32_t*>(kb + 512)[u];
  const uint32_t R = kb[768 + u] | (((w0 >> 15) & 1u) << 8) | ((w0 >> 31) << 9) |
                     (((w1 >> 15) & 1u) << 10) | ((w1 >> 31) << 11);
  const u32x2 mt = kmeta[blk * kTile + u];
  const uint32_t m0 = mt[0], m1 = mt[1];
  const _Float16 s_hi = __builtin_bit_cast(_Float16, (uint16_t)(m0 & 0xFFFFu));
  const _Float16 z_hi = __builtin_bit_cast(_Float16, (uint16_t)(m0 >> 16));
  const _Float16 s_lo = __builtin_bit_cast(_Float16, (uint16_t)(m1 & 0xFFFFu));
  const _Float16 z_lo = __builtin_bit_cast(_Float16, (uint16_t)(m1 >> 16));
  _Float16 v[32];
#pragma unroll
  for (int c = 0; c < 8; ++c)
    v[c] = (_Float16)fmaf((float)s_hi, (float)((whi >> (4 * c)) & 15u), (float)z_hi);
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
    v[8 + i] = (_Float16)fmaf((float)s_lo, (float)code, (float)z_lo);
  }
  h8* dst = reinterpret_cast<h8*>(kd + (((size_t)b * d.Tmax + t) * d.Hkv + h) * 32);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    dst[k] = h8{v[8 * k], v[8 * k + 1], v[8 * k + 2], v[8 * k + 3],
                v[8 * k + 4], v[8 * k + 5], v[8 * k + 6], v[8 * k + 7]};
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
    bt[c * bs + k] = bk[((size_t)g * d.dh + k) * 32 + c];
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
                                                                uint16_t* __restrict__ bvr) {
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
  if (c < d.rv) {
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

constexpr int kPQ = 16;       // queries per workgroup
constexpr int kPH = 8;        // query heads per workgroup
constexpr int kRows = kPQ * kPH;   // rows of the stacked P tile
constexpr int kPS = 72;       // P row stride (halves)
constexpr int kMaxRv = 1024;
constexpr int kMaxCols = 512;      // value columns per workgroup (at most)
// bytes of one tile's value scales (or zeros) over the workgroup's groups
constexpr int kMetaHalf = (kMaxCols / 32) * kTile * 2;
// bytes of one tile's value codes over the workgroup's groups (at most
// eight 4-bit and eight 3-bit groups: the 4-bit groups are the first R_v/4
// channels, so no block of 512 columns holds more)
constexpr int kCodeSlot = 8 * 1024 + 8 * 768;
// bytes of one tile's fp16 key latents of the workgroup's KV heads
constexpr int kKeySlot = kPH * kTile * 64;

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

struct AttnArgs {
  Dims d;
  int ctx, chunk, n_qb, n_qb_pad, n_hg, n_cb;
  const uint8_t* value;
  const uint16_t* vmeta;
  const _Float16* qn;     // [B*C][Hq][32] query latents, natural channel order
  const _Float16* kd;     // [B][T_max][Hkv][32] fp16 key latents
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

// Workgroup = (16 consecutive queries, 8 query heads, R_v / n_cb value
// columns, sequence b), 8 waves.  Rows of the stacked P tile: row = query * 8
// + head (128 rows = four MFMA row tiles).  Wave w
//   - scores query head w for the 16 queries on MFMA 16x16x32 with the keys
//     as the A operand (a lane then holds four consecutive tokens of one
//     query) and a lazy online softmax, writing fp16 probabilities to a P
//     slot;
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
template <int G>
__global__ __launch_bounds__(512) void prefill_attn_kernel(AttnArgs a) {
  const Dims& d = a.d;
  __shared__ __attribute__((aligned(16))) _Float16 p_l[2][kRows * kPS];
  __shared__ __attribute__((aligned(16))) uint8_t meta_l[2][2 * kMetaHalf];
  __shared__ __attribute__((aligned(16))) uint8_t code_l[2][kCodeSlot];
  // key latents [KV head][token][4 chunks of 16 B], chunk c of token u at
  // position c ^ ((u >> 2) & 3) so that a score operand read (16 tokens,
  // one chunk) touches every bank once
  __shared__ __attribute__((aligned(16))) uint8_t key_l[2][kKeySlot];
  // the queries' latent vectors in natural channel order (fp16)
  __shared__ __attribute__((aligned(16))) _Float16 qnat[kRows * 32];
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
  const int q0 = qb * kPQ;
  const int nq = min(kPQ, a.chunk - q0);
  const int pfirst = a.ctx + q0;            // first query's position
  const int pmax = pfirst + nq - 1;         // last position any row may see
  const int tile_last = pmax / kTile;
  const int cols = d.rv / a.n_cb, col0 = cb * cols;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, j = lane >> 5;   // 32x32 operand coordinates
  const int c16 = lane & 15, g16 = lane >> 4;  // 16x16 operand coordinates

  // the 16 queries' latent vectors of the 8 heads: one 16-byte piece each
  {
    const int qh = tid >> 2, piece = tid & 3;    // (query, head), 8 channels
    const int qi = qh / kPH;
    h8 v = h8{};
    if (qi < nq)
      v = *reinterpret_cast<const h8*>(
          a.qn + (((size_t)b * a.chunk + q0 + qi) * d.Hq + hg * kPH + qh % kPH) * 32 + piece * 8);
    *reinterpret_cast<h8*>(&qnat[qh * 32 + piece * 8]) = v;
  }
  if (tid < 2) flag_l[tid] = -1;
  __syncthreads();

  // ------------------------------------------------------------ score setup
  const int hl = wave;                          // query head within the group
  const int h = hg * kPH + hl;
  const int g = h / G;
  // B operand of the score MFMA: query c16, channels 8 g16 .. 8 g16 + 7
  const h8 bq = *reinterpret_cast<const h8*>(&qnat[(c16 * kPH + hl) * 32 + g16 * 8]);
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
  // 8 g16 .. 8 g16 + 7 of KV head g (local head g - g0)
  const int g0 = hg * kPH / G;
  const int key_lane = (g - g0) * (kTile * 64) + c16 * 64 + ((g16 ^ (c16 >> 2)) << 4);
  auto load_keys = [&](int slot, h8 (&kk)[4]) {
#pragma unroll
    for (int bl = 0; bl < 4; ++bl)
      kk[bl] = *reinterpret_cast<const h8*>(&key_l[slot][key_lane + bl * 16 * 64]);
  };

  // scores of tile `tile` (index it in the loop) into P slot `slot`
  auto score = [&](int tile, int it, int slot, const h8 (&kk)[4]) {
    float x[4][4];   // [16-token block][token 4 g16 + v], query c16
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
      const f32x4v sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kk[bl], bq, f32x4v{}, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) x[bl][v] = sc[v];
    }
    if (tile * kTile + kTile - 1 > pfirst) {   // uniform: some token is hidden
      // last token of the tile query c16 sees (none for padding queries)
      const int lim = c16 < nq ? pfirst + c16 - tile * kTile : -1;
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
    if (lane < kPQ) alpha_l[slot][c16 * kPH + hl] = alpha;
    float ls = 0.0f;
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[v] = __builtin_amdgcn_exp2f(x[bl][v] - m_ref);
        ls += p[v];
      }
      *reinterpret_cast<h4*>(p_at(slot, c16 * kPH + hl, bl * 16 + 4 * g16)) =
          h4{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    }
    l_lane += ls;
  };

  // ------------------------------------------------------------ value setup
  const int NG = d.rv / 32;           // value groups
  const int NH = d.rv / 128;          // 4-bit value groups
  const int ngrp = cols / 32, g_first = col0 / 32;
  const size_t vtile_bytes = (size_t)26 * d.rv;
  const size_t mtile = (size_t)2 * NG * kTile;     // fp16 elements
  const int meta_bytes = ngrp * kTile * 2;
  // Direct-to-LDS staging, in 1 KB pieces spread over the waves: the fp16
  // keys of tile `kt` into key slot kt & 1 (4 pieces per KV head) and the
  // value codes, scales and zeros of tile `ct` into slot ct & 1.  A key
  // piece is 16 tokens of one head; lane l moves chunk
  // (l & 3) ^ ((l >> 4) & 3) of token l >> 2 (the swizzle of key_l).
  auto goff = [&](int gi) { return gi < NH ? gi * 1024 : NH * 1024 + (gi - NH) * 768; };
  const int code_lo = goff(g_first), code_bytes = goff(g_first + ngrp) - code_lo;
  const int nkp = 4 * (kPH / G);               // key pieces
  const int ncp = (code_bytes + 1023) / 1024;  // code pieces
  const int nmp = (meta_bytes + 1023) / 1024;  // pieces per scale / zero plane
  const int key_src_lane = (lane >> 2) * d.Hkv * 64 + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  auto dma = [&](const uint8_t* src, uint8_t* dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  auto stage = [&](int kt, int ct) {
    const int p_key = kt <= tile_last ? nkp : 0;
    const int p_val = ct <= tile_last ? ncp + 2 * nmp : 0;
    for (int p = wave; p < p_key + p_val; p += 8) {
      if (p < p_key) {
        const int kh = p >> 2, blk = p & 3;
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kd) +
            (((size_t)b * d.Tmax + kt * kTile + blk * 16) * d.Hkv + g0 + kh) * 64 + key_src_lane;
        dma(src, &key_l[kt & 1][kh * (kTile * 64) + blk * 1024]);
      } else if (p < p_key + ncp) {
        const int q = p - p_key;
        const int off = q * 1024 + lane * 16;
        if (off < code_bytes)
          dma(a.value + ((size_t)b * d.NT + ct) * vtile_bytes + code_lo + off,
              &code_l[ct & 1][q * 1024]);
      } else {
        const int q = p - p_key - ncp;
        const int part = q / nmp, piece = q - part * nmp;   // part 0 scales, 1 zeros
        const int off = piece * 1024 + lane * 16;
        if (off < meta_bytes) {
          const uint16_t* mt = a.vmeta + ((size_t)b * d.NT + ct) * mtile +
                               (size_t)(part * NG + g_first) * kTile;
          dma(reinterpret_cast<const uint8_t*>(mt) + off,
              &meta_l[ct & 1][part * kMetaHalf + piece * 1024]);
        }
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
      h8 kk[4];
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
        h8 kk[4];
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
          const int qi = rr >> 3, hh = rr & 7;
          if (qi < nq)
            a.part_o[po_index(d, (size_t)d.B * a.chunk, hg * kPH + hh,
                              (size_t)b * a.chunk + q0 + qi,
                              col0 + (2 * wave + gp) * 32 + m)] = acc[rt][gp][v];
        }
  }
  if (cb == 0) {
    float l = l_lane + __shfl_xor(l_lane, 16);
    l += __shfl_xor(l, 32);
    if (lane < kPQ && c16 < nq) {
      const size_t o = (((size_t)b * a.chunk + q0 + c16) * d.Hq + h) * 2;
      a.part_ml[o] = m_ref;
      a.part_ml[o + 1] = l;
    }
  }
}

hipError_t launch_attn(const Dims& d, dim3 grid, const AttnArgs& aa, hipStream_t s) {
  switch (d.G) {
    case 1: prefill_attn_kernel<1><<<grid, 512, 0, s>>>(aa); break;
    case 2: prefill_attn_kernel<2><<<grid, 512, 0, s>>>(aa); break;
    case 4: prefill_attn_kernel<4><<<grid, 512, 0, s>>>(aa); break;
    case 8: prefill_attn_kernel<8><<<grid, 512, 0, s>>>(aa); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace

static size_t align256p(size_t x) { return (x + 255) & ~(size_t)255; }

PrefillWs prefill_ws_layout(const Dims& d, int chunk) {
  PrefillWs w;
  const size_t M = (size_t)d.B * chunk;
  size_t off = 0;
  w.zk = off;
  off += align256p(M * d.Hkv * d.rk * 4);
  w.zv = off;
  off += align256p(M * d.rv * 4);
  w.qt = off;   // fp16 query latents [rows][Hq][32]
  off += align256p(M * d.Hq * 32 * 2);
  w.kd = off;   // fp16 key latents of every cached position, [B][T_max][Hkv][32]
  off += align256p((size_t)d.B * d.Tmax * d.Hkv * 32 * 2);
  w.part_o = off;
  off += align256p(M * d.Hq * d.rv * 4);
  w.part_ml = off;
  off += align256p(M * d.Hq * 2 * 4);
  w.bvr = off;  // rotated value factor, bf16 high then low parts
  off += align256p((size_t)2 * d.Hkv * d.dh * d.rv * 2);
  w.total = off;
  return w;
}

bool prefill_supported(const Dims& d) {
  return d.dtype == STARKV_CACHE_Q43 && d.rk == 32 && d.Hq % kPH == 0 &&
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
  gemm_bf16_kernel<<<dim3((nmax + kGT - 1) / kGT, (M + kGT - 1) / kGT, 2), 256, 0, s>>>(ga);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(1);

  // rotate, quantize and append the chunk at [ctx_len, ctx_len + chunk)
  e = launch_append(d, cache, zk, zv, ctx_len, chunk, s);
  if (e != hipSuccess) return e;
  mark(2);

  // fp16 key latents of every position the chunk's queries can see
  _Float16* kd = reinterpret_cast<_Float16*>(ws + lay.kd);
  {
    const int n = ctx_len + chunk;
    const size_t items = (size_t)d.B * n * d.Hkv;
    key_dequant_kernel<<<(unsigned)((items + 255) / 256), 256, 0, s>>>(
        static_cast<const uint8_t*>(cache.key), static_cast<const u32x2*>(cache.key_meta), d, n, kd);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  // query latents of every (query, head) of the chunk
  _Float16* qn = reinterpret_cast<_Float16*>(ws + lay.qt);
  prefill_qproj_kernel<<<dim3((M + 127) / 128, d.Hq), 256, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(bk), d, M,
      sm_scale * kLog2e, qn);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(3);

  // causal latent attention
  AttnArgs aa;
  aa.d = d;
  aa.ctx = ctx_len;
  aa.chunk = chunk;
  aa.n_qb = (chunk + kPQ - 1) / kPQ;
  aa.n_qb_pad = (aa.n_qb + 7) / 8 * 8;
  aa.n_hg = d.Hq / kPH;
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
  prefill_rotate_bv_kernel<<<d.Hkv * d.dh, 256, 0, s>>>(static_cast<const uint16_t*>(bv), d, bvr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_prefill_vproj(d, M, aa.part_o, aa.part_ml, bvr, out, s);
  mark(5);
  return e;
}

}  // namespace starkv
