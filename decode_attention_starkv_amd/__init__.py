"""Python binding of libstarkv.so (argument marshalling only).

Every function mirrors an entry point of include/starkv.h and passes device
pointers (torch.Tensor.data_ptr()) and the current HIP stream through ctypes;
all computation happens in the library's HIP kernels.  Importing this module
does not load the library; the first call does, and raises if it is missing
(build it with `python -m decode_attention_starkv_amd.build`).
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstarkv.so")

STARKV_OK = 0
STARKV_EINVAL = -1
STARKV_EUNSUPPORTED = -2
STARKV_ECAPACITY = -3
STARKV_EWORKSPACE = -4
STARKV_ELAUNCH = -5

CACHE_F32, CACHE_BF16, CACHE_Q43 = 0, 1, 2
DTYPES = {"f32": CACHE_F32, "bf16": CACHE_BF16, "q43": CACHE_Q43}
BUF_KEY, BUF_KEY_META, BUF_VALUE, BUF_VALUE_META = 0, 1, 2, 3
OP_DECODE, OP_PREFILL = 0, 1

ENTRY_POINTS = ("starkv_cache_bytes", "starkv_workspace_bytes",
                "starkv_decode_splits", "starkv_append", "starkv_decode",
                "starkv_decode_profiled", "starkv_prefill",
                "starkv_prefill_profiled", "starkv_stream_read", "starkv_strerror",
                "starkv_decode_noalloc", "starkv_noalloc_scratch_bytes",
                "starkv_decode_step", "starkv_decode_step_profiled",
                "starkv_fused_factor_bytes", "starkv_fuse_value_output",
                "starkv_decode_hidden_workspace_bytes", "starkv_decode_hidden",
                "starkv_decode_hidden_profiled", "starkv_append_paged",
                "starkv_decode_paged", "starkv_prefill_paged")


class StarkvConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "key_rank",
        "value_rank", "max_tokens", "cache_dtype", "hi_bits", "lo_bits",
        "group_size", "key_hi_channels", "value_hi_channels", "rotate",
        "num_splits")] + [("rope_theta", ctypes.c_float),
                          ("key_ranks", ctypes.POINTER(ctypes.c_int32))]


class StarkvCache(ctypes.Structure):
    _fields_ = [("key", ctypes.c_void_p), ("key_meta", ctypes.c_void_p),
                ("value", ctypes.c_void_p), ("value_meta", ctypes.c_void_p)]


class StarkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {starkv_strerror(status)} ({status})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libstarkv.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m decode_attention_starkv_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.starkv_cache_bytes.argtypes = [P(StarkvConfig), i32]
    lib.starkv_cache_bytes.restype = sz
    lib.starkv_workspace_bytes.argtypes = [P(StarkvConfig), i32, i32]
    lib.starkv_workspace_bytes.restype = sz
    lib.starkv_decode_splits.argtypes = [P(StarkvConfig), i32]
    lib.starkv_decode_splits.restype = i32
    lib.starkv_append.argtypes = [P(StarkvConfig), P(StarkvCache), vp, vp, i32, i32, vp]
    lib.starkv_append.restype = ctypes.c_int
    lib.starkv_decode.argtypes = [P(StarkvConfig), P(StarkvCache), i32, vp, vp, vp,
                                  f32, vp, vp, sz, vp]
    lib.starkv_decode.restype = ctypes.c_int
    lib.starkv_decode_profiled.argtypes = [P(StarkvConfig), P(StarkvCache), i32, vp, vp,
                                           vp, f32, vp, vp, sz, vp, P(vp)]
    lib.starkv_decode_profiled.restype = ctypes.c_int
    lib.starkv_prefill.argtypes = [P(StarkvConfig), P(StarkvCache), i32, i32, vp, i32,
                                   vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.starkv_prefill.restype = ctypes.c_int
    lib.starkv_prefill_profiled.argtypes = [P(StarkvConfig), P(StarkvCache), i32, i32, vp,
                                            i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, sz,
                                            vp, P(vp)]
    lib.starkv_prefill_profiled.restype = ctypes.c_int
    lib.starkv_stream_read.argtypes = [vp, sz, vp, vp]
    lib.starkv_stream_read.restype = ctypes.c_int
    lib.starkv_decode_step.argtypes = [P(StarkvConfig), P(StarkvCache), vp, vp, i32, i32,
                                       vp, vp, vp, f32, vp, vp, sz, vp]
    lib.starkv_decode_step.restype = ctypes.c_int
    lib.starkv_decode_step_profiled.argtypes = [P(StarkvConfig), P(StarkvCache), vp, vp,
                                                i32, i32, vp, vp, vp, f32, vp, vp, sz,
                                                vp, P(vp)]
    lib.starkv_decode_step_profiled.restype = ctypes.c_int
    lib.starkv_fused_factor_bytes.argtypes = [P(StarkvConfig), i32]
    lib.starkv_fused_factor_bytes.restype = sz
    lib.starkv_fuse_value_output.argtypes = [P(StarkvConfig), vp, vp, i32, vp, vp]
    lib.starkv_fuse_value_output.restype = ctypes.c_int
    lib.starkv_decode_hidden_workspace_bytes.argtypes = [P(StarkvConfig), i32, i32]
    lib.starkv_decode_hidden_workspace_bytes.restype = sz
    lib.starkv_decode_hidden.argtypes = [P(StarkvConfig), P(StarkvCache), i32, vp, vp, vp,
                                         i32, f32, vp, vp, sz, vp]
    lib.starkv_decode_hidden.restype = ctypes.c_int
    lib.starkv_decode_hidden_profiled.argtypes = [P(StarkvConfig), P(StarkvCache), i32, vp,
                                                  vp, vp, i32, f32, vp, vp, sz, vp, P(vp)]
    lib.starkv_decode_hidden_profiled.restype = ctypes.c_int
    lib.starkv_append_paged.argtypes = [P(StarkvConfig), P(StarkvCache), vp, i32, vp, vp,
                                        vp, vp]
    lib.starkv_append_paged.restype = ctypes.c_int
    lib.starkv_decode_paged.argtypes = [P(StarkvConfig), P(StarkvCache), vp, i32, vp, i32,
                                        vp, vp, vp, f32, vp, vp, sz, vp]
    lib.starkv_decode_paged.restype = ctypes.c_int
    lib.starkv_prefill_paged.argtypes = [P(StarkvConfig), P(StarkvCache), vp, i32, i32, i32,
                                         vp, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, sz,
                                         vp]
    lib.starkv_prefill_paged.restype = ctypes.c_int
    lib.starkv_decode_noalloc.argtypes = [P(StarkvConfig), P(StarkvCache), i32, vp, vp,
                                          vp, f32, vp, vp]
    lib.starkv_decode_noalloc.restype = ctypes.c_int
    lib.starkv_noalloc_scratch_bytes.argtypes = []
    lib.starkv_noalloc_scratch_bytes.restype = sz
    lib.starkv_strerror.argtypes = [ctypes.c_int]
    lib.starkv_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def make_config(batch, n_q_heads, n_kv_heads, head_dim, key_rank, value_rank,
                max_tokens, cache_dtype, rotate=False, num_splits=0, *,
                hi_bits=None, lo_bits=None, group_size=None,
                key_hi_channels=None, value_hi_channels=None,
                rope_theta=0.0, key_ranks=None) -> StarkvConfig:
    """starkv_config; the quantized cache's layout fields default to the
    4/3-bit split with the leading quarter of the channels at 4 bits and
    groups of 32 (zeros for unquantized caches)."""
    dt = DTYPES[cache_dtype] if isinstance(cache_dtype, str) else int(cache_dtype)
    quant = dt == CACHE_Q43

    def pick(v, q_default):
        return (q_default if quant else 0) if v is None else int(v)

    cfg = StarkvConfig(batch, n_q_heads, n_kv_heads, head_dim, key_rank,
                       value_rank, max_tokens, dt, pick(hi_bits, 4),
                       pick(lo_bits, 3), pick(group_size, 32),
                       pick(key_hi_channels, key_rank // 4),
                       pick(value_hi_channels, value_rank // 4),
                       int(bool(rotate)), num_splits, float(rope_theta), None)
    if key_ranks is not None:
        arr = (ctypes.c_int32 * len(key_ranks))(*[int(r) for r in key_ranks])
        cfg._key_ranks_buf = arr          # keeps the host array alive
        cfg.key_ranks = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return cfg


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libstarkv must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def starkv_strerror(status: int) -> str:
    return load_library().starkv_strerror(status).decode()


def starkv_cache_bytes(cfg: StarkvConfig, buffer: int) -> int:
    return load_library().starkv_cache_bytes(ctypes.byref(cfg), buffer)


def starkv_workspace_bytes(cfg: StarkvConfig, op: int, n_tokens: int) -> int:
    return load_library().starkv_workspace_bytes(ctypes.byref(cfg), op, n_tokens)


def starkv_decode_splits(cfg: StarkvConfig, seq_len: int) -> int:
    return load_library().starkv_decode_splits(ctypes.byref(cfg), seq_len)


class LatentCache:
    """The four device buffers of one layer's cache (torch uint8 tensors)."""

    def __init__(self, cfg: StarkvConfig, device="cuda", fill: int | None = 0):
        import torch
        self.cfg = cfg
        self.buffers = []
        for which in range(4):
            n = starkv_cache_bytes(cfg, which)
            if n == 0 and which in (BUF_KEY, BUF_VALUE):
                raise StarkvError(STARKV_EINVAL, "LatentCache")
            t = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
            if fill is not None:
                t.fill_(fill)
            self.buffers.append(t)

    @property
    def struct(self) -> StarkvCache:
        return StarkvCache(*(b.data_ptr() for b in self.buffers))

    def nbytes(self) -> int:
        return sum(starkv_cache_bytes(self.cfg, w) for w in range(4))


def starkv_stream_read(src, sink, stream=None) -> None:
    """Measurement helper: stream the whole device tensor `src` once (the
    split kernel's access pattern); `sink` is a device tensor of >= 4 bytes."""
    st = load_library().starkv_stream_read(_ptr(src), src.numel() * src.element_size(),
                                           _ptr(sink), _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_stream_read")


def starkv_append(cfg, cache: LatentCache, z_key, z_value, pos: int,
                  n: int | None = None, stream=None) -> None:
    """z_key fp32 [B, n, Hkv, r_k], z_value fp32 [B, n, R_v] (device)."""
    n = z_key.shape[1] if n is None else n
    cs = cache.struct
    st = load_library().starkv_append(ctypes.byref(cfg), ctypes.byref(cs),
                                      _ptr(z_key), _ptr(z_value), pos, n,
                                      _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_append")


def starkv_decode(cfg, cache: LatentCache, seq_len: int, q, B_key, B_value,
                  sm_scale: float, out, workspace, stream=None) -> None:
    cs = cache.struct
    st = load_library().starkv_decode(
        ctypes.byref(cfg), ctypes.byref(cs), seq_len, _ptr(q), _ptr(B_key),
        _ptr(B_value), sm_scale, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_decode")


def starkv_decode_step(cfg, cache: LatentCache, z_key, z_value, pos: int, q,
                       B_key, B_value, sm_scale: float, out, workspace,
                       n: int | None = None, stream=None, events=None) -> None:
    """Append tokens [pos, pos+n) then decode over pos + n tokens (one
    call); `events`: five timing events (the profiled variant)."""
    n = z_key.shape[1] if n is None else n
    cs = cache.struct
    args = (ctypes.byref(cfg), ctypes.byref(cs), _ptr(z_key), _ptr(z_value), pos, n,
            _ptr(q), _ptr(B_key), _ptr(B_value), sm_scale, _ptr(out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    lib = load_library()
    if events is None:
        st = lib.starkv_decode_step(*args)
    else:
        handles = (ctypes.c_void_p * 5)(*(e.cuda_event for e in events))
        st = lib.starkv_decode_step_profiled(*args, handles)
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_decode_step")


def starkv_fused_factor_bytes(cfg, hidden: int) -> int:
    return load_library().starkv_fused_factor_bytes(ctypes.byref(cfg), hidden)


def starkv_fuse_value_output(cfg, B_value, W_o, hidden: int, F, stream=None) -> None:
    """F_h = B_value[g(h)]^T O_h into the device buffer F (bf16, opaque)."""
    st = load_library().starkv_fuse_value_output(
        ctypes.byref(cfg), _ptr(B_value), _ptr(W_o), hidden, _ptr(F), _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_fuse_value_output")


def starkv_decode_hidden_workspace_bytes(cfg, seq_len: int, hidden: int) -> int:
    return load_library().starkv_decode_hidden_workspace_bytes(ctypes.byref(cfg),
                                                               seq_len, hidden)


def starkv_decode_hidden(cfg, cache: LatentCache, seq_len: int, q, B_key, F,
                         hidden: int, sm_scale: float, y, workspace,
                         stream=None, events=None) -> None:
    """y fp32 [B, hidden] = sum_h obar_h F_h (decode through the fused
    value/output factor); `events`: six timing events (profiled variant)."""
    cs = cache.struct
    args = (ctypes.byref(cfg), ctypes.byref(cs), seq_len, _ptr(q), _ptr(B_key), _ptr(F),
            hidden, sm_scale, _ptr(y), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    lib = load_library()
    if events is None:
        st = lib.starkv_decode_hidden(*args)
    else:
        handles = (ctypes.c_void_p * 6)(*(e.cuda_event for e in events))
        st = lib.starkv_decode_hidden_profiled(*args, handles)
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_decode_hidden")


def starkv_append_paged(cfg, cache: LatentCache, page_table, positions, z_key,
                        z_value, stream=None) -> None:
    """One token per sequence at positions[b] of a paged pool.
    page_table int32 [B, pages_per_seq], positions int32 [B] (device);
    z_key fp32 [B, Hkv, r_k], z_value fp32 [B, R_v]."""
    cs = cache.struct
    st = load_library().starkv_append_paged(
        ctypes.byref(cfg), ctypes.byref(cs), _ptr(page_table), page_table.shape[1],
        _ptr(positions), _ptr(z_key), _ptr(z_value), _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_append_paged")


def starkv_decode_paged(cfg, cache: LatentCache, page_table, seq_lens,
                        max_seq_len: int, q, B_key, B_value, sm_scale: float, out,
                        workspace, stream=None) -> None:
    """Decode over a paged pool with ragged lengths seq_lens int32 [B]."""
    cs = cache.struct
    st = load_library().starkv_decode_paged(
        ctypes.byref(cfg), ctypes.byref(cs), _ptr(page_table), page_table.shape[1],
        _ptr(seq_lens), max_seq_len, _ptr(q), _ptr(B_key), _ptr(B_value), sm_scale,
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_decode_paged")


def starkv_prefill_paged(cfg, cache: LatentCache, page_table, ctx_len: int, chunk: int,
                         x, hidden: int, A_key, A_value, q, B_key, B_value,
                         sm_scale: float, out, workspace, z_debug=None,
                         stream=None) -> None:
    """starkv_prefill over a paged pool (page_table int32 [B, pages_per_seq])."""
    cs = cache.struct
    st = load_library().starkv_prefill_paged(
        ctypes.byref(cfg), ctypes.byref(cs), _ptr(page_table), page_table.shape[1],
        ctx_len, chunk, _ptr(x), hidden, _ptr(A_key), _ptr(A_value), _ptr(q),
        _ptr(B_key), _ptr(B_value), sm_scale, _ptr(out), _ptr(z_debug), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_prefill_paged")


def starkv_decode_noalloc(cfg, cache: LatentCache, seq_len: int, q, B_key,
                          B_value, sm_scale: float, out, stream=None) -> None:
    """starkv_decode with the library's fixed scratch array as workspace."""
    cs = cache.struct
    st = load_library().starkv_decode_noalloc(
        ctypes.byref(cfg), ctypes.byref(cs), seq_len, _ptr(q), _ptr(B_key),
        _ptr(B_value), sm_scale, _ptr(out), _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_decode_noalloc")


def starkv_noalloc_scratch_bytes() -> int:
    return load_library().starkv_noalloc_scratch_bytes()


def starkv_decode_profiled(cfg, cache: LatentCache, seq_len: int, q, B_key,
                           B_value, sm_scale: float, out, workspace, events,
                           stream=None) -> None:
    """events: five torch.cuda.Event(enable_timing=True) recorded by the
    library before/after its four kernels on the launch stream."""
    handles = (ctypes.c_void_p * 5)(*(e.cuda_event for e in events))
    cs = cache.struct
    st = load_library().starkv_decode_profiled(
        ctypes.byref(cfg), ctypes.byref(cs), seq_len, _ptr(q), _ptr(B_key),
        _ptr(B_value), sm_scale, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), handles)
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_decode_profiled")


def starkv_prefill(cfg, cache: LatentCache, ctx_len: int, chunk: int, x,
                   hidden: int, A_key, A_value, q, B_key, B_value,
                   sm_scale: float, out, workspace, z_debug=None,
                   stream=None) -> None:
    cs = cache.struct
    st = load_library().starkv_prefill(
        ctypes.byref(cfg), ctypes.byref(cs), ctx_len, chunk, _ptr(x), hidden,
        _ptr(A_key), _ptr(A_value), _ptr(q), _ptr(B_key), _ptr(B_value),
        sm_scale, _ptr(out), _ptr(z_debug), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_prefill")


def starkv_prefill_profiled(cfg, cache: LatentCache, ctx_len: int, chunk: int,
                            x, hidden: int, A_key, A_value, q, B_key, B_value,
                            sm_scale: float, out, workspace, events,
                            z_debug=None, stream=None) -> None:
    """events: six torch.cuda.Event(enable_timing=True) recorded by the
    library around its launches on the launch stream."""
    handles = (ctypes.c_void_p * 6)(*(e.cuda_event for e in events))
    cs = cache.struct
    st = load_library().starkv_prefill_profiled(
        ctypes.byref(cfg), ctypes.byref(cs), ctx_len, chunk, _ptr(x), hidden,
        _ptr(A_key), _ptr(A_value), _ptr(q), _ptr(B_key), _ptr(B_value),
        sm_scale, _ptr(out), _ptr(z_debug), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), handles)
    if st != STARKV_OK:
        raise StarkvError(st, "starkv_prefill_profiled")


def workspace(cfg, op: int, n_tokens: int, device="cuda"):
    """Allocate a workspace tensor of the size the library asks for."""
    import torch
    n = starkv_workspace_bytes(cfg, op, n_tokens)
    if n == 0:
        raise StarkvError(STARKV_EINVAL, "starkv_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)
