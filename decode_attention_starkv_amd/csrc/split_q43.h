// The quantized decode split kernel (rows a-3 and a-4 of the decode path:
// split-T latent scores with an online softmax, and the stacked-head joint
// value contraction P Z_v on MFMA), shared by four translation units:
// decode.hip instantiates the 4/3-bit latent-score kernels, decode_rope.hip
// the 4/3-bit variants that read precomputed rotary scores, decode_u4.hip
// and decode_u4_rope.hip the same two for the uniform 4-bit cache.  Each
// unit gets its own copy of the kernels (anonymous namespace); SplitArgs and
// SplitFn are common.
#pragma once

#include <type_traits>

#include "device.h"

namespace starkv {

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
  // precomputed (rotary) scores, read by the kRope kernels only
  const void* s_rel;        // fp16 [B][Hq][NT*64]
  const float* m_tile;      // [B][Hq][NT]
  const float* m_split;     // [B][splits][Hq]
};

using SplitFn = void (*)(SplitArgs);

// The 4/3-bit split kernel reading precomputed rotary scores for the
// shape, or nullptr (decode_rope.hip).
SplitFn q43_rope_kernel(const Dims& d);
// The uniform 4-bit split kernels (decode_u4.hip, decode_u4_rope.hip).
SplitFn u4_kernel(const Dims& d);
SplitFn u4_rope_kernel(const Dims& d);

namespace {

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

// Value ring of a kernel whose value waves own NIV groups each (R_v = 128 NIV,
// NIV <= 8); sized per NIV so that small value ranks leave room for a second
// workgroup on the compute unit.
// one slot: the 4-bit wave's codes + scales + zeros, then the three other
// waves' (1024 + 128 + 128 bytes per 4-bit group, 768 + 128 + 128 per 3-bit
// group; in a uniform 4-bit cache every wave's groups are 4-bit)
constexpr int hi_region(int niv) { return niv * 1280; }
constexpr int lo_region(int niv, bool u4) { return niv * (u4 ? 1280 : 1024); }
constexpr int slot_bytes(int niv, bool u4) { return hi_region(niv) + 3 * lo_region(niv, u4); }
// LDS ring slots per value wave: 4 (tiles staged three ahead of use); 3
// where four slots would not fit in LDS (uniform 4-bit, R_v = 1024), and for
// R_v <= 256, where a tile is small enough that two tiles in flight keep the
// stream busy and a shorter opening burst lets short splits start sooner
constexpr int value_slots(int niv, bool u4) { return (u4 && niv == 8) || niv <= 2 ? 3 : 4; }
// fp32 row stride of the epilogue's per-wave staging of partial rows (kept
// in the value ring): 32 rows of 32 NIV columns, padded so the two row halves
// a store instruction writes fall in different LDS banks
constexpr int stage_row(int niv) { return niv * 32 + 8; }
constexpr int ring_bytes(int niv, bool u4) {
  return value_slots(niv, u4) * slot_bytes(niv, u4) > 4 * 32 * stage_row(niv) * 4
             ? value_slots(niv, u4) * slot_bytes(niv, u4)
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
//     4-bit, value wave 0 holds exactly the 4-bit groups (kU4: every group
//     is 4-bit).  Each value wave streams its own groups' codes, scales and
//     zeros into a private LDS ring (direct-to-LDS, non-temporal) two or
//     three tiles ahead, so it waits on its own loads only.  A = P * scale in fp16, B = codes as fp16
//     subnormals, mfma 32x32x16; P x zero adds the zero points, and a column
//     of ones in that product gives each head's exp-sum l.
// One barrier per tile hands P over: while the value waves contract tile t,
// the score waves already score tile t+1.
template <int G, int KVS, int NIV, bool kRope, bool kU4>
__global__ __launch_bounds__(512) void split_q43_kernel(SplitArgs a) {
  constexpr int PS = 72;                        // P row stride (halves)
  constexpr int kDmaHi = NIV + 2 * ((NIV * 128 + 1023) / 1024);
  constexpr int kDmaLo = (NIV * 768 + 1023) / 1024 + 2 * ((NIV * 128 + 1023) / 1024);
  constexpr int kValueSlots = value_slots(NIV, kU4);
  constexpr int kValueAhead = kValueSlots - 1;   // tiles staged ahead of use
  constexpr int kKeyBlockBytes = key_block_bytes(kU4 ? 4 : 3);
  const Dims& d = a.d;

  constexpr int kHiRegion = hi_region(NIV), kLoRegion = lo_region(NIV, kU4);
  constexpr int kSlotBytes = slot_bytes(NIV, kU4), kStageRow = stage_row(NIV);
  __shared__ __attribute__((aligned(16))) uint8_t vring[ring_bytes(NIV, kU4)];
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
  // this sequence's tokens (ragged batches: its own length; the splits are
  // laid out for the longest, so a split may hold no tile of it)
  const int seq_len = seq_len_of(d, b, a.seq_len);
  const int n_tiles = (seq_len + kTile - 1) / kTile;
  const int tile0 = sp * a.tiles_per_split;
  const int tile1 = min(n_tiles, tile0 + a.tiles_per_split);
  const int GV = 4 * NIV;            // value groups
  const int NH = kU4 ? GV : NIV;     // 4-bit value groups
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

  if (wave < 4 && kRope) {
    // ===================================================== precomputed scores
    // (rotary position embedding: the scores come from the RoPE score
    // kernel as fp16 values relative to the running max m_tile of their
    // head at that tile; the split's final max m_split makes every
    // probability exp2(s_rel + m_tile - m_split) <= 1, so no accumulator is
    // ever rescaled.)  Same barrier sequence as the latent-score path.
    const int sw = wave;
    const bool has_heads = sw < d.Hkv;
    const size_t tpad = (size_t)d.NT * kTile;
    const uint16_t* srel = static_cast<const uint16_t*>(a.s_rel);
    auto head_of = [&](int i) { return (sw + (i / G) * 4) * G + (i % G); };
    float msplit[KVS * G];
#pragma unroll
    for (int i = 0; i < KVS * G; ++i)
      msplit[i] = has_heads ? a.m_split[((size_t)b * a.splits + sp) * d.Hq + head_of(i)] : 0.0f;
    uint32_t srA[KVS * G], srB[KVS * G];
    float mtA[KVS * G], mtB[KVS * G];
    auto load_pre = [&](int tile, uint32_t (&sr)[KVS * G], float (&mt)[KVS * G]) {
#pragma unroll
      for (int i = 0; i < KVS * G; ++i) {
        const size_t row = (size_t)b * d.Hq + head_of(i);
        sr[i] = __builtin_nontemporal_load(srel + row * tpad + (size_t)tile * kTile + lane);
        mt[i] = a.m_tile[row * d.NT + tile];
      }
    };
    auto score_pre = [&](int tile, int slot, const uint32_t (&sr)[KVS * G],
                         const float (&mt)[KVS * G]) {
      const bool valid = lane < seq_len - tile * kTile;
#pragma unroll
      for (int i = 0; i < KVS * G; ++i) {
        const float x = valid ? f16v(sr[i]) + (mt[i] - msplit[i]) : -INFINITY;
        p_l[slot][head_of(i) * PS + lane] = (_Float16)__builtin_amdgcn_exp2f(x);
      }
    };
    const int n_it = tile1 - tile0;
    if (n_it > 0 && has_heads) {
      load_pre(tile0, srA, mtA);
      if (n_it > 1) load_pre(tile0 + 1, srB, mtB);
      score_pre(tile0, 0, srA, mtA);
      if (n_it > 2) load_pre(tile0 + 2, srA, mtA);
    }
    lds_barrier();
    for (int it = 0; it < n_it; it += 2) {
      if (it + 1 < n_it && has_heads) {
        score_pre(tile0 + it + 1, (it + 1) & 1, srB, mtB);
        if (it + 3 < n_it) load_pre(tile0 + it + 3, srB, mtB);
      }
      lds_barrier();
      if (it + 1 >= n_it) break;
      if (it + 2 < n_it && has_heads) {
        score_pre(tile0 + it + 2, (it + 2) & 1, srA, mtA);
        if (it + 4 < n_it) load_pre(tile0 + it + 4, srA, mtA);
      }
      lds_barrier();
    }
    if (has_heads && lane == 0) {
#pragma unroll
      for (int i = 0; i < KVS * G; ++i) a.part_ml[(obase + head_of(i)) * 2] = msplit[i];
    }
    lds_barrier();
  } else if (wave < 4) {
    // ================================================================ scores
    const int sw = wave;
    const bool has_keys = sw < d.Hkv;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.key);
    const u32x2* kmeta = reinterpret_cast<const u32x2*>(a.kmeta);
    uint32_t kA[KVS][6], kB[KVS][6];
    auto load_keys = [&](int tile, uint32_t (&dst)[KVS][6]) {
      // the tile's slot (page) once per tile, not once per KV head
      const size_t tix = tile_index(d, b, tile) * d.Hkv;
#pragma unroll
      for (int ki = 0; ki < KVS; ++ki) {
        const int kh = sw + ki * 4;
        const size_t blk = tix + kh;
        const uint8_t* kb = kbase + blk * kKeyBlockBytes;
        dst[ki][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb) + lane);
        dst[ki][1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 256) + lane);
        dst[ki][2] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 512) + lane);
        // the remainder byte (4/3-bit) or the fourth nibble plane (kU4)
        if constexpr (kU4)
          dst[ki][3] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kb + 768) + lane);
        else
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
    // 2s + 1: steps 0-1 the leading block, steps 2-8 the trailing block
    // (pair 17 is zero on both sides; kU4 has no pair 16 either and stops
    // after step 7).
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
      const int rem = seq_len - tile * kTile;
      const bool valid = lane < rem;
      float x[KVS * G];   // scores times 2^-24
#pragma unroll
      for (int ki = 0; ki < KVS; ++ki) {
        const KeyLane kl = kU4 ? unpack_key_lane_u4(kc[ki]) : unpack_key_lane(kc[ki]);
        if constexpr (kSets > 0) {
          const h2 mh = __builtin_bit_cast(h2, kl.mhi), ml = __builtin_bit_cast(h2, kl.mlo);
#pragma unroll
          for (int st = 0; st < kSets; ++st) {
            const uint32_t* rq = qrec + ((sw + ki * 4) * G + st * 4 + (lane & 3)) * kQ43Rec;
            f32x4 dh = {0.0f, 0.0f, 0.0f, 0.0f}, dl = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < (kU4 ? 8 : 9); ++k) {
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
    const bool four = kU4 || vw == 0;
    const int code_bytes = NIV * (four ? 1024 : 768);
    const int code_off = four ? n0 * 1024 : NH * 1024 + (n0 - NH) * 768;
    const int meta_bytes = NIV * kTile * 2;   // one plane of this wave's groups
    const uint8_t* vbase = static_cast<const uint8_t*>(a.value);
    const uint8_t* vmbase = reinterpret_cast<const uint8_t*>(a.vmeta);
    const size_t tile_bytes = value_tile_bytes(32 * GV, kU4 ? 4 : 3);
    const size_t meta_tile = (size_t)2 * GV * kTile * 2;
    // this wave's region of each slot: value wave 0's groups (4-bit) first
    uint8_t* ring = vring + (vw == 0 ? 0 : kHiRegion + (vw - 1) * kLoRegion);

    auto stage = [&](int tile, int slot) {
      const size_t t = tile_index(d, b, tile);
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
      const int rem = seq_len - tile * kTile;
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
      // zero points of this wave's groups: columns n0 .. n0+NIV-1; value
      // wave 0 (n0 = 0) also sums P into column NIV: l of every head,
      // rescaled with the accumulators and made of the same fp16 P
      // (other columns read a row of zeros: no masked loads)
      {
        const bool zcol = m >= n0 && m < n0 + NIV;
        const _Float16* zsrc = zcol ? zr_l + (m - n0) * kTile
                                    : (vw == 0 && m == NIV) ? zo_l + kTile : zo_l;
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
    if (vw == 0 && m == NIV) {
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

// The quantized split kernel for a shape: G query heads per KV head, KVS KV
// heads per score wave, NIV value groups per value wave; kRope reads
// precomputed (rotary) scores instead of scoring latent keys; kU4 reads a
// uniform 4-bit cache.
template <int G, int KVS, bool kRope, bool kU4>
SplitFn q43_kernel_niv(int NIV) {
  switch (NIV) {
    case 2: return split_q43_kernel<G, KVS, 2, kRope, kU4>;
    case 4: return split_q43_kernel<G, KVS, 4, kRope, kU4>;
    case 6: return split_q43_kernel<G, KVS, 6, kRope, kU4>;
    case 8: return split_q43_kernel<G, KVS, 8, kRope, kU4>;
    default: return nullptr;
  }
}

template <bool kRope, bool kU4>
SplitFn q43_kernel_select(const Dims& d) {
  const int NIV = d.rv / 128;
  const int KVS = d.Hkv >= 4 ? d.Hkv / 4 : 1;
  switch (d.G * 16 + KVS) {
    case 1 * 16 + 1: return q43_kernel_niv<1, 1, kRope, kU4>(NIV);
    case 1 * 16 + 2: return q43_kernel_niv<1, 2, kRope, kU4>(NIV);
    case 1 * 16 + 4: return q43_kernel_niv<1, 4, kRope, kU4>(NIV);
    case 1 * 16 + 8: return q43_kernel_niv<1, 8, kRope, kU4>(NIV);
    case 2 * 16 + 1: return q43_kernel_niv<2, 1, kRope, kU4>(NIV);
    case 2 * 16 + 2: return q43_kernel_niv<2, 2, kRope, kU4>(NIV);
    case 2 * 16 + 4: return q43_kernel_niv<2, 4, kRope, kU4>(NIV);
    case 4 * 16 + 1: return q43_kernel_niv<4, 1, kRope, kU4>(NIV);
    case 4 * 16 + 2: return q43_kernel_niv<4, 2, kRope, kU4>(NIV);
    case 8 * 16 + 1: return q43_kernel_niv<8, 1, kRope, kU4>(NIV);
    default: return nullptr;
  }
}

}  // namespace
}  // namespace starkv
