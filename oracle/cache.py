"""The latent KV cache in its packed byte form, written from the format spec.

The pages fix what is stored -- per-head key latents and one joint value
latent (technical review of arXiv 2606.08382, section 5.3, eq. 12; section
2.2, eq. 2), rotated and mixed-precision quantized (section 6.1) -- but no
byte layout.  This module implements format v1 (tiles of 64 tokens) on its
own, from the specification below, so that the GPU packer can be checked
against it to the bit.

fp32 / bf16 caches (elements little-endian), in the order one GPU load
instruction reads (64 lanes x 8 consecutive elements):
  key   [B][Hkv][tile][r_k/8][64 tokens][8 channels]
  value [B][tile][R_v/32][8 token blocks][32 channels][8 tokens]
        (element (token u of the tile, channel 32g + m) of group g sits in
        block u // 8 at [m][u % 8])
  (shapes the GPU path does not accept -- r_k not a multiple of 8, R_v not
  a multiple of 32 -- use one chunk of r_k channels / one group of R_v.)

q43 cache (r_k = 32: channels 0-7 at 4 bits, 8-31 at 3 bits; R_v a multiple
of 128: channels [0, R_v/4) at 4 bits, the rest at 3 bits):
  key codes  [B][tile][Hkv] blocks of 832 B, one 64-token tile each (the
      blocks of all KV heads of a tile are contiguous):
      [0,256)   hi  u32[64]: key channel c (0..7) at bits 4c..4c+3
      [256,512) lo0 u32[64]: lo channel i at bits 3i (i<5), 16+3(i-10) (10<=i<15)
      [512,768) lo1 u32[64]: lo channel i at bits 3(i-5) (5<=i<10),
                             16+3(i-15) (15<=i<20)
      [768,832) lo2 u8[64]
      lo channel 20+k (k<4) is bits 3k..3k+2 of a 12-bit remainder R whose
      bits 0-7 are lo2, bit 8 = lo0 bit 15, bit 9 = lo0 bit 31,
      bit 10 = lo1 bit 15, bit 11 = lo1 bit 31.  (lo channel i = key ch 8+i.)
  key meta   [B][tile][Hkv][64][4] fp16: scale_hi, zero_hi, scale_lo, zero_lo
  value codes [B][tile] blocks of 26*R_v B: the 4-bit groups (32 channels
      each) first, then the 3-bit groups; a 4-bit group is
      [half j<2][channel c<32][4 x u32], a 3-bit group [half j][c][3 x u32];
      token 32j+u of the tile, u < 32:
        4-bit: word u//8, bit 16*(v%2) + 4*(v//2) with v = u%8
        3-bit, u < 30: word u//10, bit 16*(w%2) + 3*(w//2) with w = u%10
        3-bit, u = 30: code bit k is bit 15 of word k; u = 31: bit 31 of word k
  value meta [B][tile][2][R_v/32][64] fp16: plane 0 scales, plane 1 zeros.

uniform 4-bit cache (lo_bits = 4; the 4-bit cache of the review's speed
figures, section 6.1 after eq. 14): the same precision blocks, groups and
rotation, both blocks at 4 bits:
  key codes  [B][tile][Hkv] blocks of 1024 B: four u32[64] planes, plane p
      holding key channels 8p .. 8p+7 of each token as nibbles (channel 8p+c
      at bits 4c, the layout of the q43 hi plane);
  value codes [B][tile] blocks of 32*R_v B: every group in the 4-bit run
      layout above.  Metadata as for q43.

Appending tokens [pos, pos+n) changes only the bits and metadata of those
tokens; every other bit of the buffers keeps its previous value.
"""

from __future__ import annotations

import numpy as np

from . import hadamard, quant

TT = 64


# ------------------------------------------------------------------ sizes --

def key_block_bytes(lo_bits=3):
    """Bytes of one packed key tile of one KV head."""
    return 832 if lo_bits == 3 else 1024


def value_tile_bytes(value_rank, lo_bits=3):
    """Bytes of one packed value tile (all groups of one 64-token tile)."""
    return (26 if lo_bits == 3 else 32) * value_rank


def layout(batch, n_kv_heads, key_rank, value_rank, max_tokens, cache,
           key_ranks=None, lo_bits=3):
    """Byte sizes of the four cache buffers.  key_ranks: per-KV-head key
    ranks; an fp32 / bf16 key buffer then holds sum(key_ranks) channels per
    token (the technical review's eq. 15 sums the per-head ranks), a q43 one
    keeps its 32-channel tiles (eq. 15's padding term)."""
    assert max_tokens % TT == 0
    nt = max_tokens // TT
    if cache in ("f32", "bf16"):
        es = 4 if cache == "f32" else 2
        rsum = n_kv_heads * key_rank if key_ranks is None else int(sum(key_ranks))
        return dict(key=batch * max_tokens * rsum * es,
                    key_meta=0,
                    value=batch * nt * value_rank * TT * es,
                    value_meta=0)
    assert cache == "q43" and key_rank == 32 and value_rank % 128 == 0
    assert lo_bits in (3, 4)
    return dict(key=batch * n_kv_heads * nt * key_block_bytes(lo_bits),
                key_meta=batch * n_kv_heads * nt * TT * 8,
                value=batch * nt * value_tile_bytes(value_rank, lo_bits),
                value_meta=batch * nt * 2 * (value_rank // 32) * TT * 2)


# ------------------------------------------------------- bit-level tables --

def _value_bit(u: int, bits: int, k: int):
    """(word, bit) of code bit k of token u (< 32) in a channel's half-run."""
    if bits == 4:
        v = u % 8
        return u // 8, 16 * (v % 2) + 4 * (v // 2) + k
    if u < 30:
        w = u % 10
        return u // 10, 16 * (w % 2) + 3 * (w // 2) + k
    return k, 15 if u == 30 else 31


def _key_lo_bit(i: int, k: int):
    """(plane, bit) of code bit k of lo channel i (< 24); plane 0=lo0, 1=lo1,
    2=lo2 (byte)."""
    if i < 5:
        return 0, 3 * i + k
    if i < 10:
        return 1, 3 * (i - 5) + k
    if i < 15:
        return 0, 16 + 3 * (i - 10) + k
    if i < 20:
        return 1, 16 + 3 * (i - 15) + k
    r = 3 * (i - 20) + k           # bit of the remainder R
    if r < 8:
        return 2, r
    return {8: (0, 15), 9: (0, 31), 10: (1, 15), 11: (1, 31)}[r]


# ------------------------------------------------------------ pack/unpack --

def pack_key_tiles(codes: np.ndarray, lo_bits: int = 3) -> np.ndarray:
    """codes uint8 [N, 64, 32] -> bytes uint8 [N, 832] (lo_bits 3) or
    [N, 1024] (lo_bits 4: four nibble planes)."""
    n = codes.shape[0]
    if lo_bits == 4:
        c = codes.astype(np.uint32)
        out = np.empty((n, 1024), np.uint8)
        for p in range(4):
            w = np.zeros((n, TT), np.uint32)
            for ch in range(8):
                w |= (c[:, :, 8 * p + ch] & 15) << (4 * ch)
            out[:, 256 * p:256 * (p + 1)] = w.astype("<u4").view(np.uint8).reshape(n, 256)
        return out
    c = codes.astype(np.uint32)
    hi = np.zeros((n, TT), np.uint32)
    for ch in range(8):
        hi |= (c[:, :, ch] & 15) << (4 * ch)
    planes = [np.zeros((n, TT), np.uint32) for _ in range(3)]
    for i in range(24):
        for k in range(3):
            p, b = _key_lo_bit(i, k)
            planes[p] |= ((c[:, :, 8 + i] >> k) & 1) << b
    out = np.empty((n, 832), np.uint8)
    out[:, 0:256] = hi.astype("<u4").view(np.uint8).reshape(n, 256)
    out[:, 256:512] = planes[0].astype("<u4").view(np.uint8).reshape(n, 256)
    out[:, 512:768] = planes[1].astype("<u4").view(np.uint8).reshape(n, 256)
    out[:, 768:832] = planes[2].astype(np.uint8)
    return out


def unpack_key_tiles(blob: np.ndarray, lo_bits: int = 3) -> np.ndarray:
    """bytes uint8 [N, 832] (or [N, 1024], lo_bits 4) -> codes uint8
    [N, 64, 32]."""
    n = blob.shape[0]
    blob = np.ascontiguousarray(blob)
    if lo_bits == 4:
        codes = np.zeros((n, TT, 32), np.uint32)
        for p in range(4):
            w = blob[:, 256 * p:256 * (p + 1)].copy().view("<u4").astype(np.uint32)
            for ch in range(8):
                codes[:, :, 8 * p + ch] = (w >> (4 * ch)) & 15
        return codes.astype(np.uint8)
    hi = blob[:, 0:256].copy().view("<u4").astype(np.uint32)
    lo0 = blob[:, 256:512].copy().view("<u4").astype(np.uint32)
    lo1 = blob[:, 512:768].copy().view("<u4").astype(np.uint32)
    lo2 = blob[:, 768:832].astype(np.uint32)
    planes = [lo0, lo1, lo2]
    codes = np.zeros((n, TT, 32), np.uint32)
    for ch in range(8):
        codes[:, :, ch] = (hi >> (4 * ch)) & 15
    for i in range(24):
        for k in range(3):
            p, b = _key_lo_bit(i, k)
            codes[:, :, 8 + i] |= ((planes[p] >> b) & 1) << k
    return codes.astype(np.uint8)


def _value_regions(value_rank: int, lo_bits: int = 3):
    """[(first channel, bits, byte offset, words per run)] per 32-ch group."""
    n_hi = value_rank // 4
    regs, off = [], 0
    for g in range(value_rank // 32):
        bits = 4 if 32 * g < n_hi else lo_bits
        regs.append((32 * g, bits, off, bits))
        off += 2 * 32 * bits * 4
    assert off == value_tile_bytes(value_rank, lo_bits)
    return regs


def pack_value_tiles(codes: np.ndarray, lo_bits: int = 3) -> np.ndarray:
    """codes uint8 [N, 64, R_v] -> bytes uint8 [N, 26*R_v] (32*R_v with
    lo_bits 4)."""
    n, _, rv = codes.shape
    out = np.empty((n, value_tile_bytes(rv, lo_bits)), np.uint8)
    c = codes.astype(np.uint32)
    for c0, bits, off, nw in _value_regions(rv, lo_bits):
        words = np.zeros((n, 2, 32, nw), np.uint32)   # [tile, half, ch, word]
        grp = c[:, :, c0:c0 + 32]                      # [tile, token, ch]
        for j in range(2):
            for u in range(32):
                col = grp[:, 32 * j + u, :]            # [tile, ch]
                for k in range(bits):
                    wd, b = _value_bit(u, bits, k)
                    words[:, j, :, wd] |= ((col >> k) & 1) << b
        size = 2 * 32 * nw * 4
        out[:, off:off + size] = words.astype("<u4").view(np.uint8).reshape(n, size)
    return out


def unpack_value_tiles(blob: np.ndarray, value_rank: int, lo_bits: int = 3) -> np.ndarray:
    """bytes uint8 [N, 26*R_v] (32*R_v with lo_bits 4) -> codes uint8
    [N, 64, R_v]."""
    n = blob.shape[0]
    codes = np.zeros((n, TT, value_rank), np.uint32)
    for c0, bits, off, nw in _value_regions(value_rank, lo_bits):
        size = 2 * 32 * nw * 4
        words = np.ascontiguousarray(blob[:, off:off + size]).view("<u4")
        words = words.astype(np.uint32).reshape(n, 2, 32, nw)
        for j in range(2):
            for u in range(32):
                for k in range(bits):
                    wd, b = _value_bit(u, bits, k)
                    codes[:, 32 * j + u, c0:c0 + 32] |= \
                        ((words[:, j, :, wd] >> b) & 1) << k
    return codes.astype(np.uint8)


# ------------------------------------------------------------ bf16 helper --

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ cache --

class Cache:
    """Byte-exact image of the four cache buffers, with append and read-out."""

    def __init__(self, batch, n_kv_heads, key_rank, value_rank, max_tokens,
                 cache, rotate=False, fill=0, key_ranks=None, lo_bits=3):
        self.B, self.H, self.rk, self.rv = batch, n_kv_heads, key_rank, value_rank
        self.T, self.kind, self.rotate = max_tokens, cache, rotate
        self.lob = lo_bits        # bits of the trailing precision block (q43)
        self.nt = max_tokens // TT
        # per-head key ranks: head g keeps key_ranks[g] channels; key_rank is
        # the largest, the width of the latent rows.  fp32 / bf16 caches
        # store exactly those channels; a q43 cache keeps every head's
        # 32-channel tile with the channels past its rank zero (the review's
        # section 6.2: rank rounding to a supported kernel tile, eq. 15's
        # padding term)
        self.kr = None if key_ranks is None else [int(r) for r in key_ranks]
        assert self.kr is None or all(r % 8 == 0 and 0 < r <= key_rank for r in self.kr)
        sz = layout(batch, n_kv_heads, key_rank, value_rank, max_tokens, cache, key_ranks,
                    lo_bits)
        self.buf = {k: np.full(v, fill, np.uint8) for k, v in sz.items()}

    @classmethod
    def for_workload(cls, w, fill=0, batch=None, max_tokens=None, key_ranks=None):
        return cls(w.batch if batch is None else batch, w.n_kv_heads,
                   w.key_rank, w.value_rank,
                   w.max_tokens if max_tokens is None else max_tokens,
                   w.cache, w.rotate, fill, key_ranks=key_ranks,
                   lo_bits=getattr(w, "lo_bits", 3))

    # -- views -------------------------------------------------------------
    def _elem_views(self):
        """Element views k [B, H, tile, token, r_k/8, 8] and
        v [B, tile, block, token-in-block, group, channel-in-group] over the
        buffers (writes through them land in the buffers)."""
        dt = np.float32 if self.kind == "f32" else np.uint16
        kw = 8 if self.rk % 8 == 0 else self.rk
        gw = 32 if self.rv % 32 == 0 else self.rv
        k = None if self.kr is not None else self.buf["key"].view(dt).reshape(
            self.B, self.H, self.nt, self.rk // kw, TT, kw).transpose(0, 1, 2, 4, 3, 5)
        v = self.buf["value"].view(dt).reshape(
            self.B, self.nt, self.rv // gw, 8, gw, 8).transpose(0, 1, 3, 5, 2, 4)
        return k, v

    def _key_head_view(self, g):
        """Per-head key view [B, tile, token, r_g/8, 8] of a cache with
        per-head ranks: sequence b's key region holds the heads one after the
        other, head g as [tile][r_g/8][64 tokens][8 channels] (writes through
        the view land in the buffer)."""
        dt = np.float32 if self.kind == "f32" else np.uint16
        e = self.buf["key"].view(dt)
        rg, rs = self.kr[g], sum(self.kr)
        base = self.nt * TT * sum(self.kr[:g])
        it = e.itemsize
        v = np.lib.stride_tricks.as_strided(
            e[base:], shape=(self.B, self.nt, rg // 8, TT, 8),
            strides=(self.nt * TT * rs * it, (rg // 8) * TT * 8 * it, TT * 8 * it, 8 * it, it),
            writeable=True)
        return v.transpose(0, 1, 3, 2, 4)

    def _q_views(self):
        """Key views with axes (batch, head, tile, ...) over the tile-major
        buffers (writes through the views land in the buffers)."""
        kb = key_block_bytes(self.lob)
        k = self.buf["key"].reshape(self.B, self.nt, self.H, kb).transpose(0, 2, 1, 3)
        km = self.buf["key_meta"].view(np.uint16).reshape(
            self.B, self.nt, self.H, TT, 4).transpose(0, 2, 1, 3, 4)
        v = self.buf["value"].reshape(self.B, self.nt, value_tile_bytes(self.rv, self.lob))
        vm = self.buf["value_meta"].view(np.uint16).reshape(
            self.B, self.nt, 2, self.rv // 32, TT)
        return k, km, v, vm

    # -- append ------------------------------------------------------------
    def append(self, z_key, z_value, pos, n):
        """Store tokens [pos, pos+n) of every batch element.

        z_key float32 [B, n, Hkv, r_k], z_value float32 [B, n, R_v]
        (technical review, Algorithm 2 step 3: quantize and append)."""
        assert 0 <= pos and pos + n <= self.T
        zk = np.asarray(z_key, np.float32)
        zv = np.asarray(z_value, np.float32)
        if n == 0:
            return
        if self.kind in ("f32", "bf16"):
            k, v = self._elem_views()
            if self.kind == "f32":
                kk, vv = zk, zv
            else:
                kk, vv = to_bf16_bits(zk), to_bf16_bits(zv)
            t = pos + np.arange(n)
            if self.kr is None:
                k[:, :, t // TT, t % TT] = np.transpose(kk, (0, 2, 1, 3)).reshape(
                    self.B, self.H, n, *k.shape[4:])
            else:
                for g, rg in enumerate(self.kr):
                    hv = self._key_head_view(g)
                    hv[:, t // TT, t % TT] = kk[:, :, g, :rg].reshape(self.B, n, rg // 8, 8)
            v[:, t // TT, (t % TT) // 8, t % 8] = vv.reshape(self.B, n, *v.shape[4:])
            return
        if self.kr is not None:
            zk = zk.copy()
            for g, rg in enumerate(self.kr):
                zk[:, :, g, rg:] = 0.0
        if self.rotate:
            zk = hadamard.rotate_latent_f32(zk, self.rk // 4)
            zv = hadamard.rotate_latent_f32(zv, self.rv // 4)
        kq_hi = quant.quantize(zk[..., :8], 4)
        kq_lo = quant.quantize(zk[..., 8:], self.lob)
        nhi = self.rv // 4
        vgr = zv.reshape(self.B, n, self.rv // 32, 32)
        vq4 = quant.quantize(vgr[:, :, :nhi // 32], 4)
        vq3 = quant.quantize(vgr[:, :, nhi // 32:], self.lob)
        kcodes = np.concatenate([kq_hi[0], kq_lo[0]], axis=-1)     # [B,n,H,32]
        vcodes = np.concatenate([vq4[0], vq3[0]], axis=2).reshape(self.B, n, self.rv)
        vscale = np.concatenate([vq4[1], vq3[1]], axis=2)          # [B,n,G]
        vzero = np.concatenate([vq4[2], vq3[2]], axis=2)
        kb, km, vb, vm = self._q_views()
        ta, tb = pos // TT, (pos + n - 1) // TT + 1     # touched tiles
        nt = tb - ta
        # token-in-window index of every stored token of the touched tiles
        win = np.arange(ta * TT, tb * TT) - pos          # [nt*64]
        sel = (win >= 0) & (win < n)
        src = np.clip(win, 0, max(n - 1, 0))
        # keys: unpack the touched tiles, overwrite the appended tokens, repack
        cur = unpack_key_tiles(kb[:, :, ta:tb].reshape(-1, key_block_bytes(self.lob)),
                               self.lob).reshape(self.B, self.H, nt * TT, 32)
        newk = np.transpose(kcodes, (0, 2, 1, 3))[:, :, src]
        cur = np.where(sel[None, None, :, None], newk, cur)
        kb[:, :, ta:tb] = pack_key_tiles(cur.reshape(-1, TT, 32), self.lob).reshape(
            self.B, self.H, nt, key_block_bytes(self.lob))
        meta = np.stack([kq_hi[1], kq_hi[2], kq_lo[1], kq_lo[2]], axis=-1)
        oldm = km[:, :, ta:tb].reshape(self.B, self.H, nt * TT, 4)
        newm = np.transpose(meta, (0, 2, 1, 3))[:, :, src]
        km[:, :, ta:tb] = np.where(sel[None, None, :, None], newm, oldm).reshape(
            self.B, self.H, nt, TT, 4)
        # values
        vtb = value_tile_bytes(self.rv, self.lob)
        curv = unpack_value_tiles(vb[:, ta:tb].reshape(-1, vtb),
                                  self.rv, self.lob).reshape(self.B, nt * TT, self.rv)
        curv = np.where(sel[None, :, None], vcodes[:, src], curv)
        vb[:, ta:tb] = pack_value_tiles(curv.reshape(-1, TT, self.rv), self.lob).reshape(
            self.B, nt, vtb)
        for plane, arr in ((0, vscale), (1, vzero)):
            old_ = np.transpose(vm[:, ta:tb, plane], (0, 2, 1, 3)).reshape(
                self.B, -1, nt * TT)                       # [B, G, nt*64]
            new_ = np.transpose(arr, (0, 2, 1))[:, :, src]
            upd = np.where(sel[None, None, :], new_, old_)
            vm[:, ta:tb, plane] = np.transpose(
                upd.reshape(self.B, -1, nt, TT), (0, 2, 1, 3))

    # -- read-out ----------------------------------------------------------
    def key_latents(self, b, seq_len):
        """Dequantized (stored, i.e. rotated if enabled) key latents
        float64 [seq_len, Hkv, r_k] of batch element b."""
        if self.kind in ("f32", "bf16") and self.kr is not None:
            # channels past a head's rank read as 0
            nt = (seq_len + TT - 1) // TT
            out = np.zeros((seq_len, self.H, self.rk))
            for g, rg in enumerate(self.kr):
                x = self._key_head_view(g)[b, :nt].reshape(nt * TT, rg)[:seq_len]
                x = x if self.kind == "f32" else from_bf16_bits(x)
                out[:, g, :rg] = x
            return out
        if self.kind in ("f32", "bf16"):
            k, _ = self._elem_views()
            nt = (seq_len + TT - 1) // TT
            x = k[b, :, :nt].reshape(self.H, nt * TT, self.rk)[:, :seq_len]
            x = x if self.kind == "f32" else from_bf16_bits(x)
            return np.transpose(x, (1, 0, 2)).astype(np.float64)
        kb, km, _, _ = self._q_views()
        nt = (seq_len + TT - 1) // TT
        codes = unpack_key_tiles(kb[b, :, :nt].reshape(-1, key_block_bytes(self.lob)),
                                 self.lob).reshape(self.H, nt * TT, 32)[:, :seq_len]
        meta = km[b, :, :nt].reshape(self.H, nt * TT, 4)[:, :seq_len]
        # only stored tokens are dequantized (slots past seq_len may hold any
        # bytes, NaN scales included)
        hi = quant.dequantize(codes[..., :8], meta[..., 0], meta[..., 1])
        lo = quant.dequantize(codes[..., 8:], meta[..., 2], meta[..., 3])
        x = np.concatenate([hi, lo], axis=-1)
        return np.transpose(x, (1, 0, 2))

    def value_latents(self, b, seq_len):
        """Dequantized joint value latents float64 [seq_len, R_v]."""
        nt = (seq_len + TT - 1) // TT
        if self.kind in ("f32", "bf16"):
            _, v = self._elem_views()
            x = v[b, :nt].reshape(nt * TT, self.rv)
            x = x if self.kind == "f32" else from_bf16_bits(x)
            return x[:seq_len].astype(np.float64)
        _, _, vb, vm = self._q_views()
        codes = unpack_value_tiles(vb[b, :nt], self.rv, self.lob)  # [nt,64,R]
        g = self.rv // 32
        s = np.transpose(vm[b, :nt, 0], (0, 2, 1))                  # [nt,64,G]
        z = np.transpose(vm[b, :nt, 1], (0, 2, 1))
        codes = codes.reshape(nt * TT, g, 32)[:seq_len]
        s = s.reshape(nt * TT, g)[:seq_len]
        z = z.reshape(nt * TT, g)[:seq_len]
        x = quant.dequantize(codes, s, z)
        return x.reshape(seq_len, self.rv)
