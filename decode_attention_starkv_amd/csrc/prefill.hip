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

__device__ inline void wait_vmcnt0() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// ------------------------------------------------------------------- attn --

constexpr int kPQ = 16;       // queries per workgroup
constexpr int kPH = 8;        // query heads per workgroup
constexpr int kRows = kPQ * kPH;   // rows of the stacked P tile
constexpr int kPS = 72;       // P row stride (halves)
constexpr int kZRow = 128;    // bytes of one dequantized value channel (64 tokens)
constexpr int kMaxRv = 1024;
constexpr int kHalfRv = kMaxRv / 2;   // value columns per workgroup (at most)
// packed value data of one tile and one column half, staged in LDS: codes
// (at most 8 four-bit + 8 three-bit groups), then scales, then zeros
constexpr int kVCodeMax = 8 * 1024 + 8 * 768;
constexpr int kVMetaMax = (kHalfRv / 32) * kTile * 2;
constexpr int kVSlot = kVCodeMax + 2 * kVMetaMax;

typedef float f32x4v __attribute__((ext_vector_type(4)));

struct AttnArgs {
  Dims d;
  int ctx, chunk, n_qb, n_qb_pad, n_hg;
  const uint8_t* key;
  const u32x2* kmeta;     // per token: (s_hi | z_hi << 16, s_lo | z_lo << 16)
  const uint8_t* value;
  const uint16_t* vmeta;
  const uint32_t* qt;     // [B*C][Hq][kQ43Rec]
  const _Float16* kd;     // [B][T_max][Hkv][32] fp16 key latents
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
//            MFMA 16x16x32 (A = the queries' latent vectors, B = the fp16
//            key latents a pre-pass dequantized from the packed cache); a
//            lazy online softmax writes P to the other P slot.  It also
//            contracts tile t: row tiles 2(w&1),
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
  // the queries' latent vectors in natural channel order (fp16)
  __shared__ __attribute__((aligned(16))) _Float16 qnat[kPQ * kPH * 32];
  __shared__ __attribute__((aligned(16))) uint8_t vst[2][kVSlot];
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
  // the query records hold 16 channel pairs (lo half, hi half) in the order
  // of the packed key words; put every channel back in its place
  for (int i = tid; i < kPQ * kPH * 16; i += 512) {
    const int qh = i >> 4, t = i & 15;       // (query, head) and pair
    const int qi = qh / kPH;
    int ca, cb;
    if (t < 4) { ca = t; cb = t + 4; }
    else if (t < 9) { ca = 8 + (t - 4); cb = 18 + (t - 4); }
    else if (t < 14) { ca = 13 + (t - 9); cb = 23 + (t - 9); }
    else if (t == 14) { ca = 28; cb = 30; }
    else { ca = 29; cb = 31; }
    const uint32_t pr = qi < nq
        ? a.qt[(((size_t)b * a.chunk + q0 + qi) * d.Hq + hg * kPH) * kQ43Rec +
               (qh % kPH) * kQ43Rec + t]
        : 0u;
    qnat[qh * 32 + ca] = __builtin_bit_cast(_Float16, (uint16_t)(pr & 0xFFFFu));
    qnat[qh * 32 + cb] = __builtin_bit_cast(_Float16, (uint16_t)(pr >> 16));
  }
  if (tid < 2 * kRows) (&alpha_l[0][0])[tid] = 1.0f;
  if (tid < 2) flag_l[tid] = -1;
  __syncthreads();

  // ------------------------------------------------------------ score setup
  const int hl = wave;                          // query head within the group
  const int h = hg * kPH + hl;
  const int g = h / G;
  // per lane: queries g16*4 + v (v < 4) of the 16x16 result
  float m_ref[4], l_lane[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { m_ref[v] = -INFINITY; l_lane[v] = 0.0f; }
  // P tile: row R, token u stored at chunk (u / 8) ^ (R / 32) of the row, so
  // that the four row tiles' writes fall in different LDS banks
  auto p_at = [&](int slot, int R, int u) -> _Float16* {
    return &p_l[slot][R * kPS + (((u >> 3) ^ (R >> 5)) << 3) + (u & 7)];
  };

  // scores of tile `tile` (index it in the loop) into P slot `slot`: MFMA
  // 16x16x32 with A = the 16 queries' latent vectors, B = 16 tokens' fp16
  // key latents, both in natural channel order
  auto score = [&](int tile, int it, int slot) {
    const h8 aq = *reinterpret_cast<const h8*>(&qnat[(c16 * kPH + hl) * 32 + g16 * 8]);
    const bool masked = tile * kTile + kTile - 1 > pfirst;   // uniform
    const _Float16* kdt = a.kd + (((size_t)b * d.Tmax + tile * kTile) * d.Hkv + g) * 32 + g16 * 8;
    h8 bk[4];
#pragma unroll
    for (int bl = 0; bl < 4; ++bl)
      bk[bl] = *reinterpret_cast<const h8*>(kdt + (size_t)(bl * 16 + c16) * d.Hkv * 32);
    float x[4][4];   // [16-token block][query v]
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
      const f32x4v dq = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bk[bl], f32x4v{}, 0, 0, 0);
      const int tok = tile * kTile + bl * 16 + c16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int q = g16 * 4 + v;
        x[bl][v] = (!masked || (q < nq && tok <= pfirst + q)) ? dq[v] : -INFINITY;
      }
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
        *p_at(slot, (g16 * 4 + v) * kPH + hl, bl * 16 + c16) = (_Float16)p;
      }
  };

  // ----------------------------------------------------- value dequantize
  const int NG = d.rv / 32;           // value groups
  const int NH = d.rv / 128;          // 4-bit value groups
  const size_t vtile_bytes = (size_t)26 * d.rv;
  const size_t mtile = (size_t)2 * NG * kTile;     // fp16 elements
  const int g_first = col0 / 32;      // first value group of this half
  const int ngh = cols / 32;          // value groups of this half
  auto goff = [&](int gi) { return gi < NH ? gi * 1024 : NH * 1024 + (gi - NH) * 768; };
  const int code_lo = goff(g_first), code_bytes = goff(g_first + ngh) - code_lo;
  const int meta_bytes = ngh * kTile * 2;
  // direct-to-LDS copy of one tile's codes, scales and zeros of this half
  // into ring slot `slot`; wave w moves the 1 KB pieces w, w + 8, ...
  auto stage = [&](int tile, int slot) {
    const size_t t = (size_t)b * d.NT + tile;
    const uint8_t* src[3] = {a.value + t * vtile_bytes + code_lo,
                             reinterpret_cast<const uint8_t*>(a.vmeta + t * mtile + (size_t)g_first * kTile),
                             reinterpret_cast<const uint8_t*>(a.vmeta + t * mtile + (size_t)(NG + g_first) * kTile)};
    const int len[3] = {code_bytes, meta_bytes, meta_bytes};
    const int dst[3] = {0, kVCodeMax, kVCodeMax + kVMetaMax};
#pragma unroll
    for (int k = 0; k < 3; ++k)
      for (int piece = wave; piece * 1024 < len[k]; piece += 8) {
        const int off = piece * 1024 + lane * 16;
        if (off < len[k])
          __builtin_amdgcn_global_load_lds(
              src[k] + off,
              (__attribute__((address_space(3))) void*)(&vst[slot][dst[k] + piece * 1024]), 16, 0, 0);
      }
  };
  auto dequant = [&](int tile, int slot, auto maskc) {
    constexpr bool kMask = decltype(maskc)::value;
    const uint8_t* vb = vst[slot];
    const uint16_t* vm_s = reinterpret_cast<const uint16_t*>(vb + kVCodeMax);
    const uint16_t* vm_z = reinterpret_cast<const uint16_t*>(vb + kVCodeMax + kVMetaMax);
    const int tok_base = tile * kTile;
    for (int r = tid; r < 2 * cols; r += 512) {
      const int gl = r >> 6, e = r & 63;          // group in the half; (half, channel)
      const int gi = g_first + gl;
      const int jj = e >> 5, c = e & 31;
      const bool four = gi < NH;                  // uniform per wave
      const uint8_t* gp = vb + goff(gi) - code_lo;
      u32x4 w;
      if (four) {
        w = *reinterpret_cast<const u32x4*>(gp + e * 16);
      } else {
        const uint32_t* pw = reinterpret_cast<const uint32_t*>(gp + e * 12);
        w = u32x4{pw[0], pw[1], pw[2], 0u};
      }
      const u32x4* sp = reinterpret_cast<const u32x4*>(vm_s + gl * kTile + 32 * jj);
      const u32x4* zp = reinterpret_cast<const u32x4*>(vm_z + gl * kTile + 32 * jj);
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
      const h8 A0 = *reinterpret_cast<const h8*>(p_at(slot, rt0 * 32 + m, 32 * j + 8 * r));
      const h8 A1 = *reinterpret_cast<const h8*>(p_at(slot, (rt0 + 1) * 32 + m, 32 * j + 8 * r));
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint8_t* row = zt + (size_t)((ct0 + ct) * 32 + m) * kZRow;
        const h8 Bv = *reinterpret_cast<const h8*>(row + (((4 * j + r) ^ (m & 7)) * 16));
        acc[0][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, Bv, acc[0][ct], 0, 0, 0);
        acc[1][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, Bv, acc[1][ct], 0, 0, 0);
      }
    }
  };

  stage(0, 0);
  score(0, 0, 0);
  wait_vmcnt0();
  __syncthreads();          // packed values of tile 0 in LDS
  for (int tile = 0, it = 0; tile <= tile_last; ++tile, ++it) {
    // packed values of the next tile stream in while this one is processed
    if (tile < tile_last) stage(tile + 1, (it + 1) & 1);
    // only the workgroup's last tile can hold tokens past its last position
    if (tile * kTile + kTile - 1 > pmax) dequant(tile, it & 1, std::true_type{});
    else dequant(tile, it & 1, std::false_type{});
    lds_barrier();          // value tile and P of this tile visible
    if (tile < tile_last) score(tile + 1, it + 1, (it + 1) & 1);
    // keep the scoring and the contraction apart (register pressure); the
    // other wave of the SIMD overlaps them
    __builtin_amdgcn_sched_barrier(0);
    contract(it & 1, it);
    wait_vmcnt0();          // this wave's pieces of the next tile have landed
    lds_barrier();          // value tile and this P slot free; next tile staged
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
  w.kd = off;   // fp16 key latents of every cached position, [B][T_max][Hkv][32]
  off += align256p((size_t)d.B * d.Tmax * d.Hkv * 32 * 2);
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
  aa.kd = kd;
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
