// Latent append: rotate (optional), quantize and pack new tokens into the
// cache -- step 3 of Algorithm 2 in the technical review of arXiv 2606.08382
// (section 6.2), with the block-wise Hadamard rotation and 4/3-bit mixed
// precision of section 6.1 (eq. 13, eq. 14).
//
// Every floating-point step here is a single IEEE fp32 operation (no FMA
// contraction) so the packed bytes are reproducible bit for bit:
//   rotation: butterflies (a, b) -> (a + b, a - b) at strides 1, 2, 4, ...,
//             then one multiply by the fp32 value nearest 1/sqrt(m);
//   zero  = fp16(min) rounded toward -inf, scale = fp16((max - zero) / L)
//           rounded toward +inf, code = clamp(rint((x - zero) / scale), 0, L).
#include "internal.h"
#include "qproj.h"   // before the pragma: the query projection keeps its own FP rules

#pragma clang fp contract(off)

namespace starkv {
namespace {

__device__ inline uint16_t f16_bits_rn(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ inline float f16_value(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// One representable fp16 value toward -inf.
__device__ inline uint16_t f16_step_down(uint16_t b) {
  if ((b & 0x7FFF) == 0) return 0x8001;
  return (b & 0x8000) ? (uint16_t)(b + 1) : (uint16_t)(b - 1);
}
// One representable fp16 value toward +inf.
__device__ inline uint16_t f16_step_up(uint16_t b) {
  if ((b & 0x7FFF) == 0) return 0x0001;
  return (b & 0x8000) ? (uint16_t)(b - 1) : (uint16_t)(b + 1);
}

struct QParams {
  float zf, sf;
  uint16_t zb, sb;
};

// Zero and scale of a group from its min and max (L = 2^bits - 1).
__device__ inline QParams group_params(float lo, float hi, float levels) {
  QParams p;
  p.zb = f16_bits_rn(lo);
  if (f16_value(p.zb) > lo) p.zb = f16_step_down(p.zb);
  p.zf = f16_value(p.zb);
  float s32 = __fdiv_rn(__fsub_rn(hi, p.zf), levels);
  p.sb = f16_bits_rn(s32);
  if (f16_value(p.sb) < s32) p.sb = f16_step_up(p.sb);
  p.sf = f16_value(p.sb);
  return p;
}

__device__ inline uint32_t code_of(float x, const QParams& p, float levels) {
  if (p.sf == 0.0f) return 0u;
  float q = rintf(__fdiv_rn(__fsub_rn(x, p.zf), p.sf));
  q = fminf(fmaxf(q, 0.0f), levels);
  return (uint32_t)q;
}

// In-register fp32 Walsh-Hadamard transform of 8 consecutive values.
__device__ inline void fwht8(float* x) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = __fadd_rn(a, b);
        x[i + h] = __fsub_rn(a, b);
      }
    }
  }
  const float c = inv_sqrt_pow2(8);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __fmul_rn(x[i], c);
}

// ------------------------------------------------------------ F32 / BF16 --

__device__ inline uint16_t bf16_bits_rn(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One element of the appended keys / values per thread (idx over the
// z_key / z_value rows of the new tokens).
template <bool kBf16>
__device__ inline void plain_key_elem(const float* __restrict__ zk, void* key,
                                      const Dims& d, int pos, int n, size_t idx) {
  size_t total = (size_t)d.B * n * d.Hkv * d.rk;
  if (idx >= total) return;
  int c = idx % d.rk;
  size_t r = idx / d.rk;
  int h = r % d.Hkv;
  r /= d.Hkv;
  int i = r % n;
  int b = r / n;
  // per-head regions [NT][r_g/8][64 tokens][8 channels]; z_key rows are
  // r_k (the largest rank) wide, channels past the head's rank are skipped
  if (c >= d.krank[h]) return;
  const int t = pos + i;
  const size_t dst = plain_key_offset(d, b, h, t / kTile, c / 8, t % kTile) + c % 8;
  if (kBf16)
    static_cast<uint16_t*>(key)[dst] = bf16_bits_rn(zk[idx]);
  else
    static_cast<float*>(key)[dst] = zk[idx];
}

template <bool kBf16>
__device__ inline void plain_value_elem(const float* __restrict__ zv, void* value,
                                        const Dims& d, int pos, int n, size_t idx) {
  size_t total = (size_t)d.B * n * d.rv;
  if (idx >= total) return;
  int c = idx % d.rv;
  size_t r = idx / d.rv;
  int i = r % n;
  int b = r / n;
  int t = pos + i;
  // [B][tile][R_v/32][8 token blocks][32 channels][8 tokens]
  const int u = t % kTile;
  size_t dst = (((((size_t)b * d.NT + t / kTile) * (d.rv / 32) + c / 32) * 8 + u / 8) * 32 +
                c % 32) * 8 + u % 8;
  if (kBf16)
    static_cast<uint16_t*>(value)[dst] = bf16_bits_rn(zv[idx]);
  else
    static_cast<float*>(value)[dst] = zv[idx];
}

template <bool kBf16>
__global__ void append_plain_keys(const float* __restrict__ zk, void* key,
                                  Dims d, int pos, int n) {
  plain_key_elem<kBf16>(zk, key, d, pos, n, (size_t)blockIdx.x * blockDim.x + threadIdx.x);
}

template <bool kBf16>
__global__ void append_plain_values(const float* __restrict__ zv, void* value,
                                    Dims d, int pos, int n) {
  plain_value_elem<kBf16>(zv, value, d, pos, n, (size_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// ------------------------------------------------------------------- Q43 --

// One thread per (batch, token, KV head): 32 key channels, channels 0-7 at
// 4 bits and 8-31 at 3 bits.  The key tile format is token-major, so every
// word written here belongs to this token alone.
__device__ inline void append_q43_keys(const float* __restrict__ zk,
                                       uint8_t* __restrict__ key,
                                       uint16_t* __restrict__ kmeta, const Dims& d,
                                       int pos, int n, size_t idx) {
  size_t total = (size_t)d.B * n * d.Hkv;
  if (idx >= total) return;
  int h = idx % d.Hkv;
  int i = (idx / d.Hkv) % n;
  int b = idx / ((size_t)d.Hkv * n);
  // per-sequence positions (paged caches, one token each, clamped into the
  // sequence's pages) or the common one
  int t = (d.positions ? min(max(d.positions[b], 0), d.pages_per_seq * kTile - 1) : pos) + i;
  int tile = t / kTile, u = t % kTile;

  float x[32];
  const float4* src = reinterpret_cast<const float4*>(zk + idx * 32);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float4 v = src[k];
    x[4 * k] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
  }
  // per-head ranks: the head's latent is padded with zeros to the 32-channel
  // tile (whole blocks of 8, so the rotation never mixes them with its
  // channels)
  const int rank = d.krank[h];
#pragma unroll
  for (int c = 8; c < 32; ++c)
    if (c >= rank) x[c] = 0.0f;
  if (d.rotate) {
    fwht8(x); fwht8(x + 8); fwht8(x + 16); fwht8(x + 24);
  }
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int c = 1; c < 8; ++c) { lo = fminf(lo, x[c]); hi = fmaxf(hi, x[c]); }
  QParams ph = group_params(lo, hi, 15.0f);
  lo = x[8]; hi = x[8];
#pragma unroll
  for (int c = 9; c < 32; ++c) { lo = fminf(lo, x[c]); hi = fmaxf(hi, x[c]); }
  const bool u4 = d.lob == 4;
  const float lo_levels = u4 ? 15.0f : 7.0f;
  QParams pl = group_params(lo, hi, lo_levels);

  uint32_t whi = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) whi |= code_of(x[c], ph, 15.0f) << (4 * c);
  uint32_t q[24];
#pragma unroll
  for (int c = 0; c < 24; ++c) q[c] = code_of(x[8 + c], pl, lo_levels);
  size_t blk = tile_index(d, b, tile) * d.Hkv + h;
  uint16_t* km = kmeta + (blk * kTile + u) * 4;
  if (u4) {
    // uniform 4-bit: four nibble planes, plane p holding channels 8p .. 8p+7
    // at bits 4c (the layout of the 4-bit plane above)
    uint8_t* kb = key + blk * key_block_bytes(4);
    reinterpret_cast<uint32_t*>(kb)[u] = whi;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      uint32_t w = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) w |= q[8 * p + c] << (4 * c);
      reinterpret_cast<uint32_t*>(kb + 256 * (p + 1))[u] = w;
    }
    km[0] = ph.sb; km[1] = ph.zb; km[2] = pl.sb; km[3] = pl.zb;
    return;
  }
  // lo channel i: i<5 -> lo0 bit 3i; 5<=i<10 -> lo1 bit 3(i-5);
  // 10<=i<15 -> lo0 bit 16+3(i-10); 15<=i<20 -> lo1 bit 16+3(i-15);
  // 20<=i<24 -> remainder R bit 3(i-20): R[0:8] = lo2,
  // R8 = lo0 b15, R9 = lo0 b31, R10 = lo1 b15, R11 = lo1 b31.
  uint32_t lo0 = 0, lo1 = 0;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    lo0 |= q[k] << (3 * k);
    lo1 |= q[5 + k] << (3 * k);
    lo0 |= q[10 + k] << (16 + 3 * k);
    lo1 |= q[15 + k] << (16 + 3 * k);
  }
  uint32_t R = q[20] | (q[21] << 3) | (q[22] << 6) | (q[23] << 9);
  lo0 |= ((R >> 8) & 1u) << 15;
  lo0 |= ((R >> 9) & 1u) << 31;
  lo1 |= ((R >> 10) & 1u) << 15;
  lo1 |= ((R >> 11) & 1u) << 31;

  uint8_t* kb = key + blk * key_block_bytes(3);
  reinterpret_cast<uint32_t*>(kb)[u] = whi;
  reinterpret_cast<uint32_t*>(kb + 256)[u] = lo0;
  reinterpret_cast<uint32_t*>(kb + 512)[u] = lo1;
  kb[768 + u] = (uint8_t)(R & 0xFFu);
  km[0] = ph.sb; km[1] = ph.zb; km[2] = pl.sb; km[3] = pl.zb;
}

// One workgroup (4 waves) per (batch, touched tile, block of 256 value
// channels).  Phase 1: each wave takes tokens u = wave, wave+4, ...: lane l
// holds channels l + 64r (r < 4), rotates them (butterflies by lane shuffles
// for strides < 64 and in-register for 64 and 128), quantizes per 32-channel
// group (reduction over half-waves) and writes codes to LDS.  Phase 2: thread
// t packs channel t's runs of 32 tokens, merging with the previous words
// where the token range covers a run only partly.
__device__ inline void append_q43_values(
    const float* __restrict__ zv, uint8_t* __restrict__ value,
    uint16_t* __restrict__ vmeta, const Dims& d, int pos, int n, int cb,
    int tile_off, int b, uint8_t (*codes)[256]) {
  // paged caches: one token per sequence, at its own (clamped) position
  if (d.positions) pos = min(max(d.positions[b], 0), d.pages_per_seq * kTile - 1);
  const int tile = pos / kTile + tile_off;
  const int t0 = tile * kTile;
  const int ulo = max(pos, t0) - t0;
  const int uhi = min(pos + n, t0 + kTile) - t0;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int n_hi = d.rv / 4;
  const int G = d.rv / 32;
  const int m = pow2_divisor(n_hi);  // rotation block size
  const float rc = inv_sqrt_pow2(m);
  uint16_t* vm = vmeta + tile_index(d, b, tile) * 2 * G * kTile;

  // Words of a 32-token run that this append covers only partly keep the
  // other tokens' bits: read them now, so that the read overlaps phase 1
  // instead of following it.  Thread t owns channel cb*256 + t of the tile;
  // no other thread touches its words.
  const int ch = cb * 256 + threadIdx.x;
  const int g = ch / 32, c = ch % 32;
  // leading groups at 4 bits (every group in a uniform 4-bit cache)
  const int NH = d.lob == 4 ? G : n_hi / 32;
  const bool four = g < NH;
  const int nw = four ? 4 : 3;
  uint8_t* vt = value + tile_index(d, b, tile) * value_tile_bytes(d.rv, d.lob);
  uint8_t* grp = four ? vt + (size_t)g * 1024 : vt + (size_t)NH * 1024 + (size_t)(g - NH) * 768;
  uint32_t old[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int a = max(ulo - 32 * j, 0), e = min(uhi - 32 * j, 32);
    if (a < e && !(a == 0 && e == 32)) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(grp + (size_t)(32 * j + c) * nw * 4);
      old[j][0] = src[0];
      old[j][1] = src[1];
      old[j][2] = src[2];
      if (four) old[j][3] = src[3];
    }
  }

  for (int u = ulo + wave; u < uhi; u += 4) {
    const float* src = zv + ((size_t)b * n + (t0 + u - pos)) * d.rv + cb * 256;
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = src[lane + 64 * r];
    if (d.rotate) {
      for (int h = 1; h < m && h < 64; h <<= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = __shfl_xor(x[r], h);
          x[r] = (lane & h) ? __fsub_rn(p, x[r]) : __fadd_rn(x[r], p);
        }
      }
      if (m > 64) {  // stride 64: registers (0,1), (2,3)
        float a0 = x[0], b0 = x[1], a1 = x[2], b1 = x[3];
        x[0] = __fadd_rn(a0, b0); x[1] = __fsub_rn(a0, b0);
        x[2] = __fadd_rn(a1, b1); x[3] = __fsub_rn(a1, b1);
      }
      if (m > 128) {  // stride 128: registers (0,2), (1,3)
        float a0 = x[0], b0 = x[2], a1 = x[1], b1 = x[3];
        x[0] = __fadd_rn(a0, b0); x[2] = __fsub_rn(a0, b0);
        x[1] = __fadd_rn(a1, b1); x[3] = __fsub_rn(a1, b1);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = __fmul_rn(x[r], rc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float lo = x[r], hi = x[r];
#pragma unroll
      for (int s = 1; s < 32; s <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, s));
        hi = fmaxf(hi, __shfl_xor(hi, s));
      }
      const int chr = cb * 256 + lane + 64 * r;
      float levels = chr < n_hi || d.lob == 4 ? 15.0f : 7.0f;
      QParams p = group_params(lo, hi, levels);
      codes[u][lane + 64 * r] = (uint8_t)code_of(x[r], p, levels);
      if ((lane & 31) == 0) {
        const int gr = chr / 32;
        vm[(size_t)gr * kTile + u] = p.sb;
        vm[(size_t)(G + gr) * kTile + u] = p.zb;
      }
    }
  }
  __syncthreads();

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int a = max(ulo - 32 * j, 0), e = min(uhi - 32 * j, 32);
    if (a >= e) continue;
    uint32_t w[4] = {0, 0, 0, 0}, mask[4] = {0, 0, 0, 0};
    if (four) {
      for (int uu = a; uu < e; ++uu) {
        uint32_t k = codes[32 * j + uu][threadIdx.x];
        int v = uu % 8;
        int bit = 16 * (v % 2) + 4 * (v / 2);
        w[uu / 8] |= k << bit;
        mask[uu / 8] |= 0xFu << bit;
      }
    } else {
      for (int uu = a; uu < e; ++uu) {
        uint32_t k = codes[32 * j + uu][threadIdx.x];
        if (uu < 30) {
          int ww = uu % 10;
          int bit = 16 * (ww % 2) + 3 * (ww / 2);
          w[uu / 10] |= k << bit;
          mask[uu / 10] |= 0x7u << bit;
        } else {
          int bit = uu == 30 ? 15 : 31;
#pragma unroll
          for (int kk = 0; kk < 3; ++kk) {
            w[kk] |= ((k >> kk) & 1u) << bit;
            mask[kk] |= 1u << bit;
          }
        }
      }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(grp + (size_t)(32 * j + c) * nw * 4);
    const bool whole = (a == 0 && e == 32);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < nw) dst[k] = whole ? w[k] : ((old[j][k] & ~mask[k]) | w[k]);
  }
}

// Keys and values of one append in a single launch: blocks [0, key_blocks)
// take 256 (batch, token, KV head) key items each, the rest one (block of
// 256 value channels, touched tile, batch) value item each.
__global__ __launch_bounds__(256) void append_q43_kernel(
    const float* __restrict__ zk, const float* __restrict__ zv,
    uint8_t* __restrict__ key, uint16_t* __restrict__ kmeta,
    uint8_t* __restrict__ value, uint16_t* __restrict__ vmeta, Dims d, int pos,
    int n, int key_blocks, int tiles) {
  __shared__ uint8_t codes[kTile][256];
  const int blk = blockIdx.x;
  if (blk < key_blocks) {
    append_q43_keys(zk, key, kmeta, d, pos, n, (size_t)blk * 256 + threadIdx.x);
    return;
  }
  const int vb = blk - key_blocks;
  const int ncb = d.rv / 256;
  const int cb = vb % ncb, rest = vb / ncb;
  append_q43_values(zv, value, vmeta, d, pos, n, cb, rest % tiles, rest / tiles, codes);
}

// A decode step's first launch: the append of the new tokens (blocks
// [0, append_blocks), exactly append_q43_kernel's work) and the query
// projection (one block per (b, h) after them) are independent, so they
// share one launch and their memory latencies overlap.
__global__ __launch_bounds__(256) void step_q43_kernel(
    const float* __restrict__ zk, const float* __restrict__ zv,
    uint8_t* __restrict__ key, uint16_t* __restrict__ kmeta,
    uint8_t* __restrict__ value, uint16_t* __restrict__ vmeta, Dims d, int pos,
    int n, int key_blocks, int tiles, int append_blocks,
    const void* __restrict__ q, const void* __restrict__ bk, float qscale,
    void* __restrict__ qt) {
  __shared__ uint8_t codes[kTile][256];
  const int blk = blockIdx.x;
  if (blk >= append_blocks) {
    qproj_block<STARKV_CACHE_Q43>(q, bk, d, qscale, qt, blk - append_blocks);
    return;
  }
  if (blk < key_blocks) {
    append_q43_keys(zk, key, kmeta, d, pos, n, (size_t)blk * 256 + threadIdx.x);
    return;
  }
  const int vb = blk - key_blocks;
  const int ncb = d.rv / 256;
  const int cb = vb % ncb, rest = vb / ncb;
  append_q43_values(zv, value, vmeta, d, pos, n, cb, rest % tiles, rest / tiles, codes);
}

// The decode step's first launch for an unquantized cache: blocks
// [0, key_blocks) append key elements, the next value_blocks blocks value
// elements, and the last B Hq blocks project the queries.
template <int FMT>
__global__ __launch_bounds__(256) void step_plain_kernel(
    const float* __restrict__ zk, const float* __restrict__ zv, void* key, void* value,
    Dims d, int pos, int n, int key_blocks, int value_blocks,
    const void* __restrict__ q, const void* __restrict__ bk, float qscale,
    void* __restrict__ qt) {
  constexpr bool kBf = FMT == STARKV_CACHE_BF16;
  const int blk = blockIdx.x;
  if (blk < key_blocks) {
    plain_key_elem<kBf>(zk, key, d, pos, n, (size_t)blk * 256 + threadIdx.x);
    return;
  }
  if (blk < key_blocks + value_blocks) {
    plain_value_elem<kBf>(zv, value, d, pos, n, (size_t)(blk - key_blocks) * 256 + threadIdx.x);
    return;
  }
  qproj_block<FMT>(q, bk, d, qscale, qt, blk - key_blocks - value_blocks);
}

}  // namespace

hipError_t launch_append_qproj(const Dims& d, const starkv_cache& cache,
                               const float* zk, const float* zv, int pos, int n,
                               const void* q, const void* bk, float qscale,
                               void* qt, hipStream_t s) {
  const int T = 256;
  const size_t nk = (size_t)d.B * n * d.Hkv;
  const size_t key_blocks = (nk + T - 1) / T;
  const int tiles = (pos + n - 1) / kTile - pos / kTile + 1;
  const size_t append_blocks = key_blocks + (size_t)(d.rv / 256) * tiles * d.B;
  const size_t blocks = append_blocks + (size_t)d.B * d.Hq;
  step_q43_kernel<<<(unsigned)blocks, T, 0, s>>>(
      zk, zv, static_cast<uint8_t*>(cache.key), static_cast<uint16_t*>(cache.key_meta),
      static_cast<uint8_t*>(cache.value), static_cast<uint16_t*>(cache.value_meta), d,
      pos, n, (int)key_blocks, tiles, (int)append_blocks, q, bk, qscale, qt);
  return hipGetLastError();
}

hipError_t launch_append_qproj_plain(const Dims& d, const starkv_cache& cache,
                                     const float* zk, const float* zv, int pos, int n,
                                     const void* q, const void* bk, float qscale,
                                     void* qt, hipStream_t s) {
  const int T = 256;
  const size_t kb = ((size_t)d.B * n * d.Hkv * d.rk + T - 1) / T;
  const size_t vb = ((size_t)d.B * n * d.rv + T - 1) / T;
  const size_t blocks = kb + vb + (size_t)d.B * d.Hq;
  if (d.dtype == STARKV_CACHE_BF16)
    step_plain_kernel<STARKV_CACHE_BF16><<<(unsigned)blocks, T, 0, s>>>(
        zk, zv, cache.key, cache.value, d, pos, n, (int)kb, (int)vb, q, bk, qscale, qt);
  else
    step_plain_kernel<STARKV_CACHE_F32><<<(unsigned)blocks, T, 0, s>>>(
        zk, zv, cache.key, cache.value, d, pos, n, (int)kb, (int)vb, q, bk, qscale, qt);
  return hipGetLastError();
}

hipError_t launch_append(const Dims& d, const starkv_cache& cache,
                         const float* zk, const float* zv, int pos, int n,
                         hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int T = 256;
  if (d.dtype == STARKV_CACHE_Q43) {
    const size_t nk = (size_t)d.B * n * d.Hkv;
    const size_t key_blocks = (nk + T - 1) / T;
    const int tiles = (pos + n - 1) / kTile - pos / kTile + 1;
    const size_t blocks = key_blocks + (size_t)(d.rv / 256) * tiles * d.B;
    append_q43_kernel<<<(unsigned)blocks, T, 0, s>>>(
        zk, zv, static_cast<uint8_t*>(cache.key),
        static_cast<uint16_t*>(cache.key_meta), static_cast<uint8_t*>(cache.value),
        static_cast<uint16_t*>(cache.value_meta), d, pos, n, (int)key_blocks, tiles);
  } else {
    bool bf = d.dtype == STARKV_CACHE_BF16;
    size_t nk = (size_t)d.B * n * d.Hkv * d.rk;
    size_t nv = (size_t)d.B * n * d.rv;
    if (bf) {
      append_plain_keys<true><<<(unsigned)((nk + T - 1) / T), T, 0, s>>>(zk, cache.key, d, pos, n);
      append_plain_values<true><<<(unsigned)((nv + T - 1) / T), T, 0, s>>>(zv, cache.value, d, pos, n);
    } else {
      append_plain_keys<false><<<(unsigned)((nk + T - 1) / T), T, 0, s>>>(zk, cache.key, d, pos, n);
      append_plain_values<false><<<(unsigned)((nv + T - 1) / T), T, 0, s>>>(zv, cache.value, d, pos, n);
    }
  }
  return hipGetLastError();
}

}  // namespace starkv
