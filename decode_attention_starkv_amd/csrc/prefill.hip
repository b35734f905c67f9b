// Chunked causal prefill over the latent cache: steps 1-3 of Algorithm 2 in
// the technical review of arXiv 2606.08382 (project the chunk's hidden states
// into the latent space, rotate, quantize and append), then causal attention
// of the chunk's queries through the stored, quantized cache.
//
//   gemm      Z = X [A_key | A_value] (bf16 in, fp32 out) on MFMA 32x32x16
//   append    the decode-path append kernels (rotation + 4/3-bit packing)
//   qproj     q~ for every query of the chunk (the decode kernel, rows = B*C)
//   attn      per (16 queries, 8 query heads, half of R_v): latent scores on
//             MFMA with an online softmax, then P Z_v on MFMA against an
//             fp16 value tile dequantized once per workgroup into LDS
//             (section 5.3, eq. 12)
//   merge, vproj   the decode kernels with one split per query row
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

// ------------------------------------------------------------------- attn --

constexpr int kPQ = 16;       // queries per workgroup
constexpr int kPH = 8;        // query heads per workgroup
constexpr int kRows = kPQ * kPH;   // rows of the stacked P tile
constexpr int kPS = 72;       // P row stride (halves)
constexpr int kZRow = 128;    // bytes of one dequantized value channel (64 tokens)
constexpr int kMaxRv = 1024;
constexpr int kHalfRv = kMaxRv / 2;   // value columns per workgroup (at most)

typedef float f32x4v __attribute__((ext_vector_type(4)));

struct AttnArgs {
  Dims d;
  int ctx, chunk, n_qb, n_qb_pad, n_hg;
  const uint8_t* key;
  const u32x2* kmeta;     // per token: (s_hi | z_hi << 16, s_lo | z_lo << 16)
  const uint8_t* value;
  const uint16_t* vmeta;
  const uint32_t* qt;     // [B*C][Hq][kQ43Rec]
  float* part_o;          // [B*C][Hq][R_v]
  float* part_ml;         // [B*C][Hq][2]
};

// Workgroup = (16 consecutive queries, 8 query heads, half of the value
// columns, sequence b), 8 waves.  Rows of the stacked P tile: row = query * 8
// + head (128 rows = four MFMA row tiles).  Per 64-token tile:
//   phase A  all threads dequantize the tile's value latents of this
//            column half into LDS as fp16 (z + s * code: one packed fp16
//            FMA per token pair; rows of 64 tokens, 16-byte chunks swizzled
//            by channel so that MFMA operand reads spread over the banks);
//   barrier
//   phase B  wave w scores tile t+1 for query head w and all 16 queries on
//            MFMA 16x16x32: A = the queries' latent pairs (once with only
//            the 4-bit part, once with only the 3-bit part), B = the raw
//            codes as fp16 subnormals, K slots in the order the packed key
//            words give them; scales and zero points are applied to the
//            two partial dots afterwards; a lazy online softmax writes P to
//            the other P slot.  It also contracts tile t: row tiles 2(w&1),
//            2(w&1)+1 against its R_v/256 value column tiles on MFMA
//            32x32x16 f16;
//   barrier
// The two column halves compute the same scores; the first writes (m, l).
// Causal mask: query i (absolute position ctx + i) sees cached positions
// 0 .. ctx + i.  Value tokens past the workgroup's last position are zeroed
// so that unwritten cache bytes never reach the MFMA operands.
template <int G, int NCT>
__global__ __launch_bounds__(512) void prefill_attn_kernel(AttnArgs a) {
  const Dims& d = a.d;
  __shared__ __attribute__((aligned(16))) uint8_t zt[kHalfRv * kZRow];
  __shared__ __attribute__((aligned(16))) _Float16 p_l[2][kRows * kPS];
  __shared__ __attribute__((aligned(16))) uint32_t qrec[kPQ * kPH * kQ43Rec];
  __shared__ float alpha_l[2][kRows];
  __shared__ int flag_l[2];

  // XCD-aware order: the 8 workgroups of one query block (4 head groups x
  // 2 column halves for 32 heads) run on one XCD (blockIdx % 8) and share
  // its L2; the query blocks with the longest causal span start first.
  const int L = blockIdx.x;
  const int xcd = L & 7, k = L >> 3;
  const int per_qb = 2 * a.n_hg;
  const int sub = k % per_qb;
  const int hg = sub % a.n_hg, cs = sub / a.n_hg;
  const int qb = a.n_qb_pad - 1 - ((k / per_qb) * 8 + xcd);
  if (qb >= a.n_qb) return;   // padding workgroup; uniform, before any barrier
  const int b = blockIdx.y;
  const int q0 = qb * kPQ;
  const int nq = min(kPQ, a.chunk - q0);
  const int pfirst = a.ctx + q0;            // first query's position
  const int pmax = pfirst + nq - 1;         // last position any row may see
  const int tile_last = pmax / kTile;
  const int cols = d.rv / 2, col0 = cs * cols;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, j = lane >> 5;   // 32x32 operand coordinates
  const int c16 = lane & 15, g16 = lane >> 4;  // 16x16 operand coordinates

  for (int i = tid; i < 2 * kRows * kPS; i += 512) (&p_l[0][0])[i] = (_Float16)0.0f;
  for (int i = tid; i < kPQ * kPH * kQ43Rec; i += 512) {
    const int qi = i / (kPH * kQ43Rec), r = i % (kPH * kQ43Rec);
    qrec[i] = qi < nq ? a.qt[(((size_t)b * a.chunk + q0 + qi) * d.Hq + hg * kPH) * kQ43Rec + r]
                      : 0u;
  }
  if (tid < 2 * kRows) (&alpha_l[0][0])[tid] = 1.0f;
  if (tid < 2) flag_l[tid] = -1;
  __syncthreads();

  // ------------------------------------------------------------ score setup
  const int hl = wave;                          // query head within the group
  const int h = hg * kPH + hl;
  const int g = h / G;
  // K group of this lane's 16x16x32 operands: the record holds the 4 hi
  // pairs then the 12 lo pairs (channel order of the key words); K group 0
  // = hi pairs, 1 = lo pairs 0-3, 2 = lo pairs 5-8, 3 = lo pairs 4, 9-11.
  int qidx[4];
  if (g16 == 0) { qidx[0] = 0; qidx[1] = 1; qidx[2] = 2; qidx[3] = 3; }
  else if (g16 == 1) { qidx[0] = 4; qidx[1] = 5; qidx[2] = 6; qidx[3] = 7; }
  else if (g16 == 2) { qidx[0] = 9; qidx[1] = 10; qidx[2] = 11; qidx[3] = 12; }
  else { qidx[0] = 8; qidx[1] = 13; qidx[2] = 14; qidx[3] = 15; }
  // per lane: queries g16*4 + v (v < 4) of the 16x16 result
  float m_ref[4], l_lane[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { m_ref[v] = -INFINITY; l_lane[v] = 0.0f; }

  // scores of tile `tile` (pair index it) into P slot `slot`
  auto score = [&](int tile, int it, int slot) {
    // A operands (rows = queries c16): once with only the 4-bit part of the
    // query pairs, once with only the 3-bit part; and the queries' sums
    h8 a_hi, a_lo;
    {
      const uint32_t* rec = qrec + (c16 * kPH + hl) * kQ43Rec;
      const h8 v = __builtin_bit_cast(h8, u32x4{rec[qidx[0]], rec[qidx[1]], rec[qidx[2]], rec[qidx[3]]});
      a_hi = g16 == 0 ? v : h8{};
      a_lo = g16 == 0 ? h8{} : v;
    }
    float qs_hi[4], qs_lo[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t* rec = qrec + ((g16 * 4 + v) * kPH + hl) * kQ43Rec;
      qs_hi[v] = __builtin_bit_cast(float, rec[16]);
      qs_lo[v] = __builtin_bit_cast(float, rec[17]);
    }
    const size_t blk = ((size_t)b * d.NT + tile) * d.Hkv + g;
    const uint8_t* kb = a.key + blk * kKeyBlock;
    const bool masked = tile * kTile + kTile - 1 > pfirst;   // uniform
    float x[4][4];   // [16-token block][query v]
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
      const int u = bl * 16 + c16;            // token within the tile
      // this lane's 4 code pairs for K group g16
      const uint32_t wa = reinterpret_cast<const uint32_t*>(kb + (g16 == 0 ? 0 : g16 == 2 ? 512 : 256))[u];
      uint32_t bw[4];
      if (g16 < 3) {
        const int sh = g16 == 0 ? 4 : 3;
        const uint32_t mk = g16 == 0 ? 0x000F000Fu : 0x00070007u;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bw[kk] = (wa >> (sh * kk)) & mk;
      } else {
        const uint32_t w1 = reinterpret_cast<const uint32_t*>(kb + 512)[u];
        const uint32_t r8 = kb[768 + u];
        const uint32_t R = r8 | (((wa >> 15) & 1u) << 8) | ((wa >> 31) << 9) |
                           (((w1 >> 15) & 1u) << 10) | ((w1 >> 31) << 11);
        bw[0] = (wa >> 12) & 0x00070007u;
        bw[1] = (w1 >> 12) & 0x00070007u;
        bw[2] = (R & 7u) | (((R >> 6) & 7u) << 16);
        bw[3] = ((R >> 3) & 7u) | (((R >> 9) & 7u) << 16);
      }
      const h8 bv = __builtin_bit_cast(h8, u32x4{bw[0], bw[1], bw[2], bw[3]});
      const f32x4v dh = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, bv, f32x4v{}, 0, 0, 0);
      const f32x4v dl = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, bv, f32x4v{}, 0, 0, 0);
      const u32x2 mt = a.kmeta[blk * kTile + u];
      const uint32_t m0 = mt[0], m1 = mt[1];
      const float s_hi = f16v(m0 & 0xFFFFu) * kTwo24, z_hi = f16v(m0 >> 16);
      const float s_lo = f16v(m1 & 0xFFFFu) * kTwo24, z_lo = f16v(m1 >> 16);
      const int tok = tile * kTile + u;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int q = g16 * 4 + v;
        const float sc = fmaf(s_hi, dh[v], fmaf(z_hi, qs_hi[v], fmaf(s_lo, dl[v], z_lo * qs_lo[v])));
        x[bl][v] = (!masked || (q < nq && tok <= pfirst + q)) ? sc : -INFINITY;
      }
    }
    if (masked) {
#pragma unroll
      for (int bl = 0; bl < 4; ++bl)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (g16 * 4 + v >= nq) x[bl][v] = -INFINITY;
    }
    bool big = false;
#pragma unroll
    for (int bl = 0; bl < 4; ++bl)
#pragma unroll
      for (int v = 0; v < 4; ++v) big |= x[bl][v] > m_ref[v] + kLazy;
    if (__builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float gm = fmaxf(fmaxf(x[0][v], x[1][v]), fmaxf(x[2][v], x[3][v]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
        float alpha = 1.0f;
        if (gm > m_ref[v] + kLazy) {          // uniform in the 16-lane group
          alpha = m_ref[v] == -INFINITY ? 0.0f : exp2f(m_ref[v] - gm);
          m_ref[v] = gm;
          l_lane[v] *= alpha;
          if (c16 == 0) flag_l[slot] = it;
        }
        if (c16 == 0) alpha_l[slot][(g16 * 4 + v) * kPH + hl] = alpha;
      }
    } else if (lane < kPQ) {
      alpha_l[slot][lane * kPH + hl] = 1.0f;
    }
#pragma unroll
    for (int bl = 0; bl < 4; ++bl)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = x[bl][v] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[bl][v] - m_ref[v]);
        l_lane[v] += p;
        p_l[slot][((g16 * 4 + v) * kPH + hl) * kPS + bl * 16 + c16] = (_Float16)p;
      }
  };

  // ----------------------------------------------------- value dequantize
  const int NG = d.rv / 32;           // value groups
  const int NH = d.rv / 128;          // 4-bit value groups
  const size_t vtile_bytes = (size_t)26 * d.rv;
  const size_t mtile = (size_t)2 * NG * kTile;     // fp16 elements
  const int g_first = col0 / 32;      // first value group of this half
  auto dequant = [&](int tile, auto maskc) {
    constexpr bool kMask = decltype(maskc)::value;
    const size_t t = (size_t)b * d.NT + tile;
    const uint8_t* vb = a.value + t * vtile_bytes;
    const uint16_t* vm = a.vmeta + t * mtile;
    const int tok_base = tile * kTile;
    for (int r = tid; r < 2 * cols; r += 512) {
      const int gl = r >> 6, e = r & 63;          // group in the half; (half, channel)
      const int gi = g_first + gl;
      const int jj = e >> 5, c = e & 31;
      const bool four = gi < NH;                  // uniform per wave
      u32x4 w;
      if (four) {
        w = *reinterpret_cast<const u32x4*>(vb + (size_t)gi * 1024 + e * 16);
      } else {
        const uint32_t* pw = reinterpret_cast<const uint32_t*>(vb + (size_t)NH * 1024 +
                                                               (size_t)(gi - NH) * 768 + e * 12);
        w = u32x4{pw[0], pw[1], pw[2], 0u};
      }
      const u32x4* sp = reinterpret_cast<const u32x4*>(vm + (size_t)gi * kTile + 32 * jj);
      const u32x4* zp = reinterpret_cast<const u32x4*>(vm + (size_t)(NG + gi) * kTile + 32 * jj);
      const int ch = gl * 32 + c;                 // column within the half
      uint8_t* row = zt + (size_t)ch * kZRow;
      const int t0 = tok_base + 32 * jj;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const u32x4 S = sp[r4], Z = zp[r4];
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = 4 * r4 + q;
          const uint32_t code = four ? run_pair<true>(w, p) : run_pair<false>(w, p);
          // codes as exact fp16 integers: (1024 + k) - 1024
          const h2 kv = __builtin_bit_cast(h2, code | 0x64006400u) - h2{1024.0f16, 1024.0f16};
          // element picks go through scalars: a bit-cast applied directly
          // to an ext_vector element is lowered as a cast of element 0
          const uint32_t sbits = S[q], zbits = Z[q];
          h2 v = __builtin_elementwise_fma(kv, __builtin_bit_cast(h2, sbits),
                                           __builtin_bit_cast(h2, zbits));
          if constexpr (kMask) {
            const int tk = t0 + 2 * p;
            if (tk > pmax) v[0] = (_Float16)0.0f;
            if (tk + 1 > pmax) v[1] = (_Float16)0.0f;
          }
          o[q] = __builtin_bit_cast(uint32_t, v);
        }
        const int chunk = (4 * jj + r4) ^ (ch & 7);
        *reinterpret_cast<u32x4*>(row + chunk * 16) = u32x4{o[0], o[1], o[2], o[3]};
      }
    }
  };

  // -------------------------------------------------------------- contract
  // Wave w: row tiles rt0 = 2 (w & 1) and rt0 + 1, value column tiles
  // (w >> 1) * NCT .. + NCT - 1 of this half; each value fragment read from
  // LDS feeds two MFMAs and each P fragment NCT.
  const int rt0 = 2 * (wave & 1);
  const int ct0 = (wave >> 1) * NCT;
  f32x16 acc[2][NCT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < NCT; ++i) acc[rt][i] = f32x16{};

  auto contract = [&](int slot, int it) {
    if (flag_l[slot] == it) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float al = alpha_l[slot][(rt0 + rt) * 32 + acc_row(v, lane)];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) acc[rt][ct][v] *= al;
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const h8 A0 = *reinterpret_cast<const h8*>(&p_l[slot][(rt0 * 32 + m) * kPS + 32 * j + 8 * r]);
      const h8 A1 = *reinterpret_cast<const h8*>(&p_l[slot][((rt0 + 1) * 32 + m) * kPS + 32 * j + 8 * r]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint8_t* row = zt + (size_t)((ct0 + ct) * 32 + m) * kZRow;
        const h8 Bv = *reinterpret_cast<const h8*>(row + (((4 * j + r) ^ (m & 7)) * 16));
        acc[0][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, Bv, acc[0][ct], 0, 0, 0);
        acc[1][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, Bv, acc[1][ct], 0, 0, 0);
      }
    }
  };

  score(0, 0, 0);
  for (int tile = 0, it = 0; tile <= tile_last; ++tile, ++it) {
    // only the workgroup's last tile can hold tokens past its last position
    if (tile * kTile + kTile - 1 > pmax) dequant(tile, std::true_type{});
    else dequant(tile, std::false_type{});
    lds_barrier();          // value tile and P of this tile visible
    if (tile < tile_last) score(tile + 1, it + 1, (it + 1) & 1);
    // keep the scoring and the contraction apart (register pressure); the
    // other wave of the SIMD overlaps them
    __builtin_amdgcn_sched_barrier(0);
    contract(it & 1, it);
    lds_barrier();          // value tile and this P slot free
  }

  // ---------------------------------------------------------------- output
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = (rt0 + rt) * 32 + acc_row(v, lane);
        const int qi = rr >> 3, hh = rr & 7;
        if (qi < nq)
          a.part_o[(((size_t)b * a.chunk + q0 + qi) * d.Hq + hg * kPH + hh) * d.rv +
                   col0 + (ct0 + ct) * 32 + m] = acc[rt][ct][v];
      }
    }
  if (cs == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float l = l_lane[v];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o);
      const int q = g16 * 4 + v;
      if (c16 == 0 && q < nq) {
        const size_t o = (((size_t)b * a.chunk + q0 + q) * d.Hq + h) * 2;
        a.part_ml[o] = m_ref[v];
        a.part_ml[o + 1] = l;
      }
    }
  }
}

template <int G>
hipError_t launch_attn_g(int nct, dim3 grid, const AttnArgs& aa, hipStream_t s) {
  switch (nct) {
    case 1: prefill_attn_kernel<G, 1><<<grid, 512, 0, s>>>(aa); break;
    case 2: prefill_attn_kernel<G, 2><<<grid, 512, 0, s>>>(aa); break;
    case 3: prefill_attn_kernel<G, 3><<<grid, 512, 0, s>>>(aa); break;
    case 4: prefill_attn_kernel<G, 4><<<grid, 512, 0, s>>>(aa); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_attn(const Dims& d, dim3 grid, const AttnArgs& aa, hipStream_t s) {
  const int nct = d.rv / 256;
  switch (d.G) {
    case 1: return launch_attn_g<1>(nct, grid, aa, s);
    case 2: return launch_attn_g<2>(nct, grid, aa, s);
    case 4: return launch_attn_g<4>(nct, grid, aa, s);
    case 8: return launch_attn_g<8>(nct, grid, aa, s);
    default: return hipErrorNotSupported;
  }
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
  w.qt = off;
  off += align256p(M * d.Hq * kQ43Rec * 4);
  w.part_o = off;
  off += align256p(M * d.Hq * d.rv * 4);
  w.part_ml = off;
  off += align256p(M * d.Hq * 2 * 4);
  w.obar = off;
  off += align256p(M * d.Hq * d.rv * 4);
  w.total = off;
  return w;
}

bool prefill_supported(const Dims& d) {
  return d.dtype == STARKV_CACHE_Q43 && d.rk == 32 && d.Hq % kPH == 0 &&
         (d.G == 1 || d.G == 2 || d.G == 4 || d.G == 8) && d.rv % 256 == 0 &&
         d.rv <= kMaxRv;
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

  // query records for every (query, head) of the chunk
  Dims dq = d;
  dq.B = M;
  void* qt = ws + lay.qt;
  e = launch_qproj_q43(dq, q, bk, sm_scale, qt, s);
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
  aa.key = static_cast<const uint8_t*>(cache.key);
  aa.kmeta = static_cast<const u32x2*>(cache.key_meta);
  aa.value = static_cast<const uint8_t*>(cache.value);
  aa.vmeta = static_cast<const uint16_t*>(cache.value_meta);
  aa.qt = static_cast<const uint32_t*>(qt);
  aa.part_o = reinterpret_cast<float*>(ws + lay.part_o);
  aa.part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
  e = launch_attn(d, dim3(aa.n_qb_pad * aa.n_hg * 2, d.B), aa, s);
  if (e != hipSuccess) return e;
  mark(4);

  // normalise, undo the value rotation, up-project per head
  e = launch_merge_vproj_q43(dq, aa.part_o, aa.part_ml, 1, bv,
                             reinterpret_cast<float*>(ws + lay.obar), out, s);
  mark(5);
  return e;
}

}  // namespace starkv
