// Chunked causal prefill over the latent cache: steps 1-3 of Algorithm 2 in
// the technical review of arXiv 2606.08382 (project the chunk's hidden states
// into the latent space, rotate, quantize and append), then causal attention
// of the chunk's queries through the stored, quantized cache.
//
//   gemm      Z = X [A_key | A_value] (bf16 in, fp32 out) on MFMA 32x32x16
//   append    the decode-path append kernels (rotation + 4/3-bit packing)
//   qproj     q~ for every query of the chunk (the decode kernel, rows = B*C)
//   attn      per (8 queries, 8 query heads): latent scores with an online
//             softmax, then P Z_v on MFMA against an fp16 value tile
//             dequantized once per workgroup into LDS (section 5.3, eq. 12)
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

constexpr int kPQ = 8;        // queries per workgroup
constexpr int kPH = 8;        // query heads per workgroup
constexpr int kPS = 72;       // P row stride (halves)
constexpr int kZRow = 128;    // bytes of one dequantized value channel (64 tokens)
constexpr int kMaxRv = 1024;

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

// Workgroup = (8 consecutive queries, 8 query heads, sequence b), 8 waves.
// Rows of the stacked P tile: row = query * 8 + head (64 rows, two MFMA row
// tiles).  Per 64-token tile:
//   phase A  all threads dequantize the tile's value latents (all R_v
//            channels) into LDS as fp16: z + s * code, one packed fp16 FMA
//            per token pair, rows of 64 tokens with 16-byte chunks swizzled
//            by channel so that MFMA operand reads spread over the banks;
//   barrier
//   phase B  wave w scores tile t+1 for query head w of the group and all 8
//            queries (lane = token, codes as fp16 pairs in v_dot2, lazy
//            online softmax) into the other P slot, and contracts tile t:
//            both row tiles against its R_v / 256 column tiles on mfma
//            32x32x16 f16;
//   barrier
// Causal mask: query i (absolute position ctx + i) sees cached positions
// 0 .. ctx + i.  Value tokens past the workgroup's last position are zeroed
// so that unwritten cache bytes never reach the MFMA operands.
template <int G, int NCT>
__global__ __launch_bounds__(512) void prefill_attn_kernel(AttnArgs a) {
  const Dims& d = a.d;
  __shared__ __attribute__((aligned(16))) uint8_t zt[kMaxRv * kZRow];
  __shared__ __attribute__((aligned(16))) _Float16 p_l[2][kPQ * kPH * kPS];
  __shared__ __attribute__((aligned(16))) uint32_t qrec[kPQ * kPH * kQ43Rec];
  __shared__ float alpha_l[2][kPQ * kPH];
  __shared__ int flag_l[2];

  // XCD-aware order: consecutive workgroups of one XCD (blockIdx % 8) are
  // the head groups of one query block, so they share value tiles in that
  // XCD's L2; the query blocks with the longest causal span start first.
  const int L = blockIdx.x;
  const int xcd = L & 7, k = L >> 3;
  const int hg = k % a.n_hg;
  const int qb = a.n_qb_pad - 1 - ((k / a.n_hg) * 8 + xcd);
  if (qb >= a.n_qb) return;   // padding workgroup; uniform, before any barrier
  const int b = blockIdx.y;
  const int q0 = qb * kPQ;
  const int nq = min(kPQ, a.chunk - q0);
  const int pmax = a.ctx + q0 + nq - 1;     // last position any row may see
  const int tile_last = pmax / kTile;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, j = lane >> 5;

  for (int i = tid; i < 2 * kPQ * kPH * kPS; i += 512) (&p_l[0][0])[i] = (_Float16)0.0f;
  for (int i = tid; i < kPQ * kPH * kQ43Rec; i += 512) {
    const int qi = i / (kPH * kQ43Rec), r = i % (kPH * kQ43Rec);
    qrec[i] = qi < nq ? a.qt[(((size_t)b * a.chunk + q0 + qi) * d.Hq + hg * kPH) * kQ43Rec + r]
                      : 0u;
  }
  if (tid < 2 * kPQ * kPH) (&alpha_l[0][0])[tid] = 1.0f;
  if (tid < 2) flag_l[tid] = -1;
  __syncthreads();

  // ---------------------------------------------------------------- scores
  const int hl = wave;                          // query head within the group
  const int h = hg * kPH + hl;
  const int g = h / G;
  float m_ref[kPQ], l_lane[kPQ];
#pragma unroll
  for (int i = 0; i < kPQ; ++i) { m_ref[i] = -INFINITY; l_lane[i] = 0.0f; }

  auto score = [&](int tile, int it, int slot) {
    const size_t blk = ((size_t)b * d.NT + tile) * d.Hkv + g;
    const uint8_t* kb = a.key + blk * kKeyBlock;
    uint32_t kc[6];
    kc[0] = reinterpret_cast<const uint32_t*>(kb)[lane];
    kc[1] = reinterpret_cast<const uint32_t*>(kb + 256)[lane];
    kc[2] = reinterpret_cast<const uint32_t*>(kb + 512)[lane];
    kc[3] = kb[768 + lane];
    const u32x2 mt = a.kmeta[blk * kTile + lane];
    kc[4] = mt[0];
    kc[5] = mt[1];
    const KeyLane kl = unpack_key_lane(kc);
    const int tok = tile * kTile + lane;
    float x[kPQ];
#pragma unroll
    for (int qi = 0; qi < kPQ; ++qi) {
      const bool valid = qi < nq && tok <= a.ctx + q0 + qi;
      const float sc = key_score(kl, qrec + (qi * kPH + hl) * kQ43Rec);
      x[qi] = valid ? sc : -INFINITY;
    }
    bool big = false;
#pragma unroll
    for (int qi = 0; qi < kPQ; ++qi) big |= x[qi] > m_ref[qi] + kLazy;
    if (__builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
      for (int qi = 0; qi < kPQ; ++qi) {
        float alpha = 1.0f;
        if (__builtin_amdgcn_ballot_w64(x[qi] > m_ref[qi] + kLazy) != 0) {
          const float mx = wave_max(x[qi]);
          alpha = m_ref[qi] == -INFINITY ? 0.0f : exp2f(m_ref[qi] - mx);
          m_ref[qi] = mx;
          l_lane[qi] *= alpha;
          if (lane == 0) flag_l[slot] = it;
        }
        if (lane == 0) alpha_l[slot][qi * kPH + hl] = alpha;
      }
    } else if (lane < kPQ) {
      alpha_l[slot][lane * kPH + hl] = 1.0f;
    }
#pragma unroll
    for (int qi = 0; qi < kPQ; ++qi) {
      const float p = x[qi] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[qi] - m_ref[qi]);
      l_lane[qi] += p;
      p_l[slot][(qi * kPH + hl) * kPS + lane] = (_Float16)p;
    }
  };

  // ----------------------------------------------------- value dequantize
  const int NG = d.rv / 32;           // value groups
  const int NH = d.rv / 128;          // 4-bit value groups
  const size_t vtile_bytes = (size_t)26 * d.rv;
  const size_t mtile = (size_t)2 * NG * kTile;     // fp16 elements
  auto dequant = [&](int tile, auto maskc) {
    constexpr bool kMask = decltype(maskc)::value;
    const size_t t = (size_t)b * d.NT + tile;
    const uint8_t* vb = a.value + t * vtile_bytes;
    const uint16_t* vm = a.vmeta + t * mtile;
    const int tok_base = tile * kTile;
    for (int r = tid; r < 2 * d.rv; r += 512) {
      const int gi = r >> 6, e = r & 63;          // group; (half, channel) in it
      const int jj = e >> 5, c = e & 31;
      const bool four = gi < NH;                  // uniform per wave
      u32x4 w;
      if (four) {
        w = *reinterpret_cast<const u32x4*>(vb + (size_t)gi * 1024 + e * 16);
      } else {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(vb + (size_t)NH * 1024 +
                                                              (size_t)(gi - NH) * 768 + e * 12);
        w = u32x4{p[0], p[1], p[2], 0u};
      }
      const u32x4* sp = reinterpret_cast<const u32x4*>(vm + (size_t)gi * kTile + 32 * jj);
      const u32x4* zp = reinterpret_cast<const u32x4*>(vm + (size_t)(NG + gi) * kTile + 32 * jj);
      const int ch = gi * 32 + c;
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
  // Wave w owns value column tiles w*NCT .. w*NCT+NCT-1 for both row tiles,
  // so each value fragment read from LDS feeds two MFMAs.
  const int ct0 = wave * NCT;
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
          const float al = alpha_l[slot][rt * 32 + acc_row(v, lane)];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) acc[rt][ct][v] *= al;
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const h8 A0 = *reinterpret_cast<const h8*>(&p_l[slot][m * kPS + 32 * j + 8 * r]);
      const h8 A1 = *reinterpret_cast<const h8*>(&p_l[slot][(32 + m) * kPS + 32 * j + 8 * r]);
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
    lds_barrier();          // Z tile and P of this tile visible
    if (tile < tile_last) score(tile + 1, it + 1, (it + 1) & 1);
    contract(it & 1, it);
    lds_barrier();          // Z tile and this P slot free
  }

  // ---------------------------------------------------------------- output
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = rt * 32 + acc_row(v, lane);
        const int qi = rr >> 3, hh = rr & 7;
        if (qi < nq)
          a.part_o[(((size_t)b * a.chunk + q0 + qi) * d.Hq + hg * kPH + hh) * d.rv +
                   (ct0 + ct) * 32 + m] = acc[rt][ct][v];
      }
    }
#pragma unroll
  for (int qi = 0; qi < kPQ; ++qi) {
    const float l = wave_sum(l_lane[qi]);
    if (lane == 0 && qi < nq) {
      const size_t o = (((size_t)b * a.chunk + q0 + qi) * d.Hq + h) * 2;
      a.part_ml[o] = m_ref[qi];
      a.part_ml[o + 1] = l;
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
  e = launch_attn(d, dim3(aa.n_qb_pad * aa.n_hg, d.B), aa, s);
  if (e != hipSuccess) return e;
  mark(4);

  // normalise, undo the value rotation, up-project per head
  e = launch_merge_vproj_q43(dq, aa.part_o, aa.part_ml, 1, bv,
                             reinterpret_cast<float*>(ws + lay.obar), out, s);
  mark(5);
  return e;
}

}  // namespace starkv
