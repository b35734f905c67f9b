// Rotary position embedding fused into latent-key scoring -- the technical
// review of arXiv 2606.08382, section 5.3 ("keys are harder"): the stored
// keys stay pre-RoPE latents, and reconstruction, rotation and scoring are
// fused at runtime (Algorithm 2, steps 4b-4d), with no key ever written out.
//
// RoPE variant: channel i < d_h/2 pairs with i + d_h/2 and turns by the angle
// pos * theta^(-2i/d_h).  With q' = R_t q (the query at its position t) and
// k_j = B z_j (B = the KV head's key factor), the score is
//   q' . R_j k_j = sum_{i < d_h/2} cos(j w_i) (A_i . z_j) + sin(j w_i) (C_i . z_j),
//   A_i = q'_i B_i + q'_{i'} B_{i'},   C_i = q'_{i'} B_i - q'_i B_{i'}   (i' = i + d_h/2),
// i.e. per token q~_j = Trig_j M (M = [A; C], d_h x r_k per query head) and
// score_j = q~_j . z_j.  Per call:
//   rope_prep_kernel   one launch for two independent parts:
//                      Trig for positions 0 .. seq_len-1, fp16, already in
//                      the MFMA B-operand order (angles reduced in fp64);
//                      M per (sequence, query head): q rotated to its own
//                      position, A and C, the key latent's block rotation and
//                      sm_scale * log2(e) folded in, fp16 in A-operand order;
//   rope_score_kernel  per (split, group of 8 query heads, sequence): q~ for a
//                      64-token tile on MFMA 32x32x16 (K = d_h), transposed
//                      through LDS so lane = token, then the 32-term dot with
//                      the dequantized latent.  Scores leave as fp16 relative
//                      to the running (exact) max of their head, with that
//                      max per tile and the split's final max.
// The quantized split kernel (4/3-bit or uniform 4-bit) then reads those
// scores instead of computing latent ones (exp2(s_rel + m_tile - m_split)
// <= 1) and runs its value contraction unchanged.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "device.h"

namespace starkv {
namespace {

constexpr int kRopeHeads = 8;     // query heads per score workgroup (4 waves x 2)
constexpr int kQtStride = 36;     // floats per token row of the transpose buffer

// Trig[tile][s][j][lane][e] = T[i = 16 s + 8 (lane / 32) + e][token 64 tile +
// 32 j + lane % 32], T[i][pos] = cos(pos w_i) (i < dh/2), sin(pos w_{i-dh/2}).
// Item x (one thread) is a (pair p, position) and writes its cosine and its
// sine: x's bits are e (3), lane % 32 (5), lane / 32 (1), j (1), then s for
// p = 16 s + 8 (lane / 32) + e, so consecutive items write consecutive
// halves.
__device__ inline void rope_trig_pair(int dh, int n_tiles, double log2_theta,
                                      _Float16* __restrict__ trig, size_t x) {
  const int half = dh / 2;
  const int per_tile = half * kTile;          // items per tile
  if (x >= (size_t)n_tiles * per_tile) return;
  const int tile = (int)(x / per_tile);
  int r = (int)(x % per_tile);
  const int e = r & 7;
  r >>= 3;
  const int u = r & 31;
  r >>= 5;
  const int lh = r & 1;
  r >>= 1;
  const int j = r & 1, sp = r >> 1;
  const int p = 16 * sp + 8 * lh + e;
  const int pos = tile * kTile + 32 * j + u;
  float c, sn;
  rope_angle(pos, p, dh, log2_theta, &c, &sn);
  _Float16* t = trig + (size_t)tile * dh * kTile + (32 * lh + u) * 8 + e;
  t[(size_t)(2 * sp + j) * 512] = (_Float16)c;                     // row i = p
  t[(size_t)(2 * (sp + half / 16) + j) * 512] = (_Float16)sn;      // row i = p + dh/2
}

// M for one (sequence, query head) = bh, in A-operand order
// frag[s][lane][e] = M[i = 16 s + 8 (lane / 32) + e][r = lane % 32].
__device__ inline void rope_qproj_block(const uint16_t* __restrict__ q,
                                        const uint16_t* __restrict__ bk, const Dims& d,
                                        int q_pos, double log2_theta, float qscale,
                                        _Float16* __restrict__ mrec, int bh) {
  __shared__ float qr[256];
  __shared__ float Mf[256][33];
  const int h = bh % d.Hq, g = h / d.G;
  const int t = threadIdx.x;
  const int half = d.dh / 2;
  // the query sits at its sequence's last position (ragged batches: its own)
  if (d.lens) q_pos = seq_len_of(d, bh / d.Hq, q_pos + 1) - 1;
  // q' = R_t q
  if (t < half) {
    float c, s;
    rope_angle(q_pos, t, d.dh, log2_theta, &c, &s);
    const float a = bf16v(q[(size_t)bh * d.dh + t]);
    const float b = bf16v(q[(size_t)bh * d.dh + t + half]);
    qr[t] = a * c - b * s;
    qr[t + half] = a * s + b * c;
  }
  __syncthreads();
  // A (rows i < half) and C (rows half + i), 32 latent channels each
  // (channels past the head's key rank have no factor column: zero)
  const int rank = d.krank[g];
  for (int x = t; x < half * 32; x += 256) {
    const int i = x / 32, r = x % 32;
    const float b0 = r < rank ? bf16v(bk[((size_t)g * d.dh + i) * 32 + r]) : 0.0f;
    const float b1 = r < rank ? bf16v(bk[((size_t)g * d.dh + i + half) * 32 + r]) : 0.0f;
    Mf[i][r] = qr[i] * b0 + qr[i + half] * b1;
    Mf[half + i][r] = qr[i + half] * b0 - qr[i] * b1;
  }
  __syncthreads();
  // stored key latents rotated by blocks of 8 channels (eq. 13): M H
  if (d.rotate) {
    for (int x = t; x < d.dh * 4; x += 256) {
      const int i = x / 4, blk = x % 4;
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = Mf[i][8 * blk + k];
#pragma unroll
      for (int st = 1; st < 8; st <<= 1)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (!(k & st)) {
            const float a = v[k], b = v[k + st];
            v[k] = a + b;
            v[k + st] = a - b;
          }
#pragma unroll
      for (int k = 0; k < 8; ++k) Mf[i][8 * blk + k] = v[k] * inv_sqrt_pow2(8);
    }
    __syncthreads();
  }
  const int ks = d.dh / 16;
  for (int x = t; x < ks * 64 * 8; x += 256) {
    const int e = x & 7, lane = (x >> 3) & 63, s = x >> 9;
    const int i = 16 * s + 8 * (lane >> 5) + e;
    mrec[(size_t)bh * ks * 512 + x] = (_Float16)(Mf[i][lane & 31] * qscale);
  }
}

// The rotary decode's first launch: blocks [0, B Hq) compute the rotated
// query coefficients (a chain of dependent steps each, so they go first and
// overlap the table), the blocks after them fill the trig table.
__global__ __launch_bounds__(256) void rope_prep_kernel(int n_tiles,
                                                        const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ bk, Dims d,
                                                        int q_pos, double log2_theta,
                                                        float qscale,
                                                        _Float16* __restrict__ trig,
                                                        _Float16* __restrict__ mrec) {
  const int blk = blockIdx.x, nq = d.B * d.Hq;
  if (blk < nq) {
    rope_qproj_block(q, bk, d, q_pos, log2_theta, qscale, mrec, blk);
    return;
  }
  rope_trig_pair(d.dh, n_tiles, log2_theta, trig, (size_t)(blk - nq) * 256 + threadIdx.x);
}

template <int N>
__device__ inline void rope_wait_vmcnt() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Scores of one (split, group of 8 query heads, sequence).  Wave w owns
// query heads 8 hg + 2 w and 8 hg + 2 w + 1.  Per 64-token tile: the trig
// fragments come through a 2-slot LDS ring (direct-to-LDS loads one tile
// ahead), each lane loads its own token's key words two tiles ahead.  kU4:
// a uniform 4-bit key tile (four nibble planes) instead of a 4/3-bit one.
template <int DH, bool kU4>
__global__ __launch_bounds__(256) void rope_score_kernel(RopeArgs a) {
  constexpr int KS = DH / 16;
  constexpr int kChunks = KS * 2;              // 1 KB trig chunks per tile
  constexpr int kChunksPerWave = kChunks / 4;
  const Dims& d = a.d;
  __shared__ __attribute__((aligned(16))) h8 trig_l[2][kChunks * 64];
  __shared__ __attribute__((aligned(16))) float qt_l[4][kTile * kQtStride];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int sp = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int seq_len = seq_len_of(d, b, a.seq_len);
  const int n_tiles = (seq_len + kTile - 1) / kTile;
  const int tile0 = sp * a.tiles_per_split;
  const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);
  const int h0 = hg * kRopeHeads + 2 * w;
  const bool on0 = h0 < d.Hq, on1 = h0 + 1 < d.Hq;
  const int g0 = min(h0, d.Hq - 1) / d.G, g1 = min(h0 + 1, d.Hq - 1) / d.G;
  const bool two_kv = g0 != g1;

  // this wave's M fragments (registers for the whole split)
  h8 mf[2][KS];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int h = min(h0 + hh, d.Hq - 1);
    const h8* src = static_cast<const h8*>(a.mrec) + ((size_t)b * d.Hq + h) * KS * 64;
#pragma unroll
    for (int s = 0; s < KS; ++s) mf[hh][s] = src[s * 64 + l];
  }

  const uint8_t* kbase = static_cast<const uint8_t*>(a.key);
  const u32x2* kmeta = reinterpret_cast<const u32x2*>(a.kmeta);
  const uint8_t* tbase = static_cast<const uint8_t*>(a.trig);
  _Float16* srel = static_cast<_Float16*>(a.s_rel);
  auto stage = [&](int tile, int slot) {
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
      const int k = w * kChunksPerWave + c;
      __builtin_amdgcn_global_load_lds(
          tbase + ((size_t)tile * kChunks + k) * 1024 + l * 16,
          (__attribute__((address_space(3))) void*)(&trig_l[slot][k * 64]), 16, 0, 0);
    }
  };
  // the lane's token: 4-bit word, two 3-bit words, remainder byte (kU4:
  // four 4-bit words), meta; three register sets: keys are loaded two tiles
  // ahead
  uint32_t kc[3][2][6];
  auto load_keys = [&](int tile, uint32_t (&dst)[2][6]) {
    const size_t tix = tile_index(d, b, tile) * d.Hkv;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const size_t blk = tix + (kv == 0 ? g0 : g1);
      const uint8_t* kb = kbase + blk * key_block_bytes(kU4 ? 4 : 3);
      dst[kv][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb) + l);
      dst[kv][1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 256) + l);
      dst[kv][2] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 512) + l);
      if constexpr (kU4)
        dst[kv][3] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 768) + l);
      else
        dst[kv][3] = __builtin_nontemporal_load(kb + 768 + l);
      const u32x2 mt = __builtin_nontemporal_load(kmeta + blk * kTile + l);
      dst[kv][4] = mt[0];
      dst[kv][5] = mt[1];
    }
  };
  // loads per issue: 5 per KV head (both sets, the second a duplicate when
  // the wave's heads share one) and the wave's trig chunks
  constexpr int kKeyLoads = 10;

  float m_run[2] = {-INFINITY, -INFINITY};
  float* qt = &qt_l[w][0];
  const size_t tpad = (size_t)d.NT * kTile;

  // one tile: issue the trig of tile + 1 and the keys of tile + 2, wait for
  // this tile's trig (older loads -- its keys included -- are then done),
  // score both heads
  auto step = [&](int tile, int it, const uint32_t (&cur)[2][6], uint32_t (&ahead)[2][6]) {
    const int slot = it & 1;
    const bool more1 = tile + 1 < tile1, more2 = tile + 2 < tile1;
    if (more1) stage(tile + 1, slot ^ 1);
    if (more2) load_keys(tile + 2, ahead);
    // loads issued after this tile's trig: keys(tile+1) [last step],
    // trig(tile+1) and keys(tile+2) [this step]
    if (more2) rope_wait_vmcnt<2 * kKeyLoads + kChunksPerWave>();
    else if (more1) rope_wait_vmcnt<kKeyLoads + kChunksPerWave>();
    else rope_wait_vmcnt<0>();
    lds_barrier();   // every wave's trig chunks of this tile are in LDS

    const h8* tr = &trig_l[slot][0];
    const bool valid = tile * kTile + l < seq_len;
    // q~ tiles of both heads: each trig operand is read once and feeds both
    // heads' MFMAs (four independent accumulators)
    f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const h8 t0 = tr[(2 * s2) * 64 + l], t1 = tr[(2 * s2 + 1) * 64 + l];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(mf[0][s2], t0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(mf[0][s2], t1, acc[0][1], 0, 0, 0);
      if (on1) {
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(mf[1][s2], t0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(mf[1][s2], t1, acc[1][1], 0, 0, 0);
      }
    }
    float zf[32];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bool on = hh == 0 ? on0 : on1;
      if (!on) continue;
      const int h = h0 + hh;
      if (hh == 0 || two_kv) {
        // dequantized latent of the lane's token for this head's KV head
        const uint32_t* k = cur[hh == 1 && two_kv ? 1 : 0];
        const h2 mh = __builtin_bit_cast(h2, k[4]), ml = __builtin_bit_cast(h2, k[5]);
        const float sh = (float)mh[0], zh = (float)mh[1], sl = (float)ml[0], zl = (float)ml[1];
#pragma unroll
        for (int c = 0; c < 8; ++c) zf[c] = fmaf(sh, (float)((k[0] >> (4 * c)) & 15u), zh);
        if constexpr (kU4) {
          // channel 8p + c at bits 4c of plane p
#pragma unroll
          for (int i = 0; i < 24; ++i)
            zf[8 + i] = fmaf(sl, (float)((k[1 + i / 8] >> (4 * (i % 8))) & 15u), zl);
        } else {
          const uint32_t lo0 = k[1], lo1 = k[2];
          const uint32_t rem = (k[3] & 0xFFu) | (((lo0 >> 15) & 1u) << 8) |
                               (((lo0 >> 31) & 1u) << 9) | (((lo1 >> 15) & 1u) << 10) |
                               (((lo1 >> 31) & 1u) << 11);
#pragma unroll
          for (int i = 0; i < 24; ++i) {
            uint32_t code;
            if (i < 5) code = (lo0 >> (3 * i)) & 7u;
            else if (i < 10) code = (lo1 >> (3 * (i - 5))) & 7u;
            else if (i < 15) code = (lo0 >> (16 + 3 * (i - 10))) & 7u;
            else if (i < 20) code = (lo1 >> (16 + 3 * (i - 15))) & 7u;
            else code = (rem >> (3 * (i - 20))) & 7u;
            zf[8 + i] = fmaf(sl, (float)code, zl);
          }
        }
      }
      const f32x16& acc0 = acc[hh][0];
      const f32x16& acc1 = acc[hh][1];
      // D[r][token]: lane l holds token l % 32 (acc0) and 32 + l % 32 (acc1),
      // rows acc_row(v, l); through LDS so that lane = token
#pragma unroll
      for (int v = 0; v < 16; v += 4) {
        const int r = acc_row(v, l);
        *reinterpret_cast<float4*>(qt + (l & 31) * kQtStride + r) =
            float4{acc0[v], acc0[v + 1], acc0[v + 2], acc0[v + 3]};
        *reinterpret_cast<float4*>(qt + (32 + (l & 31)) * kQtStride + r) =
            float4{acc1[v], acc1[v + 1], acc1[v + 2], acc1[v + 3]};
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      float sc = 0.0f;
#pragma unroll
      for (int r = 0; r < 32; r += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qt + l * kQtStride + r);
        sc = fmaf(x.x, zf[r], sc);
        sc = fmaf(x.y, zf[r + 1], sc);
        sc = fmaf(x.z, zf[r + 2], sc);
        sc = fmaf(x.w, zf[r + 3], sc);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);   // reads done before the next head writes
      __builtin_amdgcn_wave_barrier();
      sc = valid ? sc : -INFINITY;
      const float mt = wave_max(sc);
      const float mn = fmaxf(m_run[hh], mt);
      m_run[hh] = mn;
      const float rel = valid ? sc - mn : -INFINITY;
      srel[((size_t)b * d.Hq + h) * tpad + (size_t)tile * kTile + l] = (_Float16)rel;
      if (l == 0) a.m_tile[((size_t)b * d.Hq + h) * d.NT + tile] = mn;
    }
    lds_barrier();   // the slot read here is restaged next step
  };

  // (a split may hold no tile of a shorter sequence: then nothing is loaded,
  // and no direct-to-LDS load is left in flight when the workgroup ends)
  if (tile0 < tile1) {
    load_keys(tile0, kc[0]);
    stage(tile0, 0);
    if (tile0 + 1 < tile1) load_keys(tile0 + 1, kc[1]);
  }
  // three steps per round so that the register sets are named statically
  for (int tile = tile0, it = 0; tile < tile1; tile += 3, it += 3) {
    step(tile, it, kc[0], kc[2]);
    if (tile + 1 >= tile1) break;
    step(tile + 1, it + 1, kc[1], kc[0]);
    if (tile + 2 >= tile1) break;
    step(tile + 2, it + 2, kc[2], kc[1]);
  }
  if (l == 0) {
    if (on0) a.m_split[((size_t)b * a.splits + sp) * d.Hq + h0] = m_run[0];
    if (on1) a.m_split[((size_t)b * a.splits + sp) * d.Hq + h0 + 1] = m_run[1];
  }
}

}  // namespace

bool rope_supported(const Dims& d) {
  return d.dtype == STARKV_CACHE_Q43 && d.rk == 32 && (d.dh == 64 || d.dh == 128);
}

size_t rope_ws_bytes(const Dims& d, int seq_len, int splits, RopeWs* w) {
  const size_t nt = (size_t)(seq_len + kTile - 1) / kTile;
  auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  RopeWs r;
  r.mrec = off;
  off += a256((size_t)d.B * d.Hq * d.dh * 32 * 2);
  r.trig = off;
  off += a256(nt * d.dh * kTile * 2);
  r.s_rel = off;
  off += a256((size_t)d.B * d.Hq * d.NT * kTile * 2);
  r.m_tile = off;
  off += a256((size_t)d.B * d.Hq * d.NT * 4);
  r.m_split = off;
  off += a256((size_t)d.B * splits * d.Hq * 4);
  r.total = off;
  if (w) *w = r;
  return off;
}

hipError_t launch_rope_scores(const Dims& d, const starkv_cache& cache, int seq_len,
                              const void* q, const void* bk, float sm_scale,
                              char* ws, const RopeWs& rw, int splits,
                              int tiles_per_split, hipStream_t s,
                              hipEvent_t before_scores) {
  const double log2_theta = log2((double)d.rope_theta);
  const int n_tiles = (seq_len + kTile - 1) / kTile;
  const size_t n_items = (size_t)n_tiles * (d.dh / 2) * kTile;   // (pair, position)
  const int trig_blocks = (int)((n_items + 255) / 256);
  _Float16* trig = reinterpret_cast<_Float16*>(ws + rw.trig);
  _Float16* mrec = reinterpret_cast<_Float16*>(ws + rw.mrec);
  rope_prep_kernel<<<(unsigned)(trig_blocks + d.B * d.Hq), 256, 0, s>>>(
      n_tiles, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(bk), d,
      seq_len - 1, log2_theta, sm_scale * kLog2e, trig, mrec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RopeArgs a;
  a.d = d;
  a.seq_len = seq_len;
  a.splits = splits;
  a.tiles_per_split = tiles_per_split;
  a.key = cache.key;
  a.kmeta = static_cast<const uint16_t*>(cache.key_meta);
  a.mrec = mrec;
  a.trig = trig;
  a.s_rel = ws + rw.s_rel;
  a.m_tile = reinterpret_cast<float*>(ws + rw.m_tile);
  a.m_split = reinterpret_cast<float*>(ws + rw.m_split);
  const dim3 grid(splits, (d.Hq + kRopeHeads - 1) / kRopeHeads, d.B);
  if (before_scores) (void)hipEventRecord(before_scores, s);
  const bool u4 = d.lob == 4;
  if (d.dh == 64) {
    if (u4) rope_score_kernel<64, true><<<grid, 256, 0, s>>>(a);
    else rope_score_kernel<64, false><<<grid, 256, 0, s>>>(a);
  } else {
    if (u4) rope_score_kernel<128, true><<<grid, 256, 0, s>>>(a);
    else rope_score_kernel<128, false><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace starkv
