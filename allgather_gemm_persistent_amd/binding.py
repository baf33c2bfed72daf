"""ctypes binding of libagg (include/agg.h): the same entry points, argument marshalling only.

Tensors are accepted wherever the C call takes a device pointer (their data_ptr() is passed),
Python sequences wherever it takes a host array, and torch streams wherever it takes a stream.
Every call returns None or raises AggError carrying the C status code and agg_last_error().
All computation happens in the library; nothing here falls back to another implementation: a
missing or unloadable library is an error.

torch is imported before the library is loaded, so libagg binds to the HIP runtime torch already
loaded (same soname) and torch's stream handles are valid for it.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (load order: torch's HIP runtime first)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libagg.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "agg.h")

AGG_OK, AGG_E_ARG, AGG_E_UNSUPPORTED, AGG_E_HIP, AGG_E_TIMEOUT, AGG_E_STATE = range(6)
AGG_BF16, AGG_FP8_E4M3 = 0, 1
AGG_OVERLAP, AGG_SERIAL, AGG_GEMM_ONLY, AGG_COPY_ONLY = range(4)
MODES = {"overlap": AGG_OVERLAP, "serial": AGG_SERIAL, "gemm_only": AGG_GEMM_ONLY,
         "copy_only": AGG_COPY_ONLY}
DTYPES = {"bf16": AGG_BF16, "fp8": AGG_FP8_E4M3}
MAX_ROW_TILES = 1024

_c_int, _c_i64, _c_u32, _c_u64, _c_f32 = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint32,
                                          ctypes.c_uint64, ctypes.c_float)
_vp, _sz = ctypes.c_void_p, ctypes.c_size_t
_i32p, _u32p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_uint32)

_SIGNATURES = {
    "agg_ctx_create": [_c_int, ctypes.POINTER(_vp)],
    "agg_ctx_destroy": [_vp],
    "agg_ctx_reset": [_vp, _vp],
    "agg_ctx_status": [_vp, _vp, _u32p, _i32p],
    "agg_ctx_epoch": [_vp, _u32p],
    "agg_ctx_set_epoch": [_vp, _c_u32],
    "agg_ctx_set_timeout_us": [_vp, _c_u64],
    "agg_ctx_set_tile": [_vp, _c_int, _c_int],
    "agg_ctx_set_lists": [_vp, _c_int, _c_int],
    "agg_ctx_set_split": [_vp, _c_int],
    "agg_ctx_set_tail": [_vp, _c_int],
    "agg_ctx_set_pull": [_vp, _c_int],
    "agg_ctx_set_producer": [_vp, _c_int, _c_int, _c_int],
    "agg_ctx_last_producer": [_vp, _i32p],
    "agg_set_trace": [_vp, _vp, _sz],
    "agg_ctx_set_timing": [_vp, _c_int],
    "agg_ctx_kernel_times": [_vp, ctypes.POINTER(ctypes.c_float), _c_int, ctypes.POINTER(_c_int)],
    "agg_put_signal": [_vp, _vp, _sz, _vp, _c_u32, _vp],
    "agg_ctx_set_copy_streams": [_vp, _c_int],
    "agg_ctx_set_reserved_cus": [_vp, _c_int],
    "ag_gemm": [_vp, _c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_f32, _c_f32,
                ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _i32p, _c_int, _u32p, _c_int, _vp, _vp],
    "ag_gemm_noalloc": [_vp, _c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_f32, _c_f32,
                        ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _i32p, _c_int, _u32p, _c_int, _vp, _vp],
    "gemm_rs": [_vp, _c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp, _vp, _vp,
                ctypes.POINTER(_vp), _vp, _vp, _vp, _i32p, _c_int, _u32p, _c_int, _vp, _vp],
    "gemm_ar": [_vp, _c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp, _vp, _vp,
                ctypes.POINTER(_vp), _vp, _vp, _vp, _i32p, _c_int, _u32p, _c_int, _vp, _vp],
    "agg_check_ar_args": [_c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp, _vp, _vp,
                          ctypes.POINTER(_vp), _vp, _vp, _vp, _i32p, _c_int, _c_int, _vp, _vp],
    "ffn_chain": [_vp, _c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_int,
                  ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_vp), _vp,
                  _vp, _vp, _i32p, _c_int, _i32p, _c_int, _c_int, _vp, _vp],
    "agg_ctx_set_chain_fused": [_vp, _c_int],
    "agg_kernel_regs": [_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)],
    "agg_tile_shape": [_c_int, _c_int, _c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_int),
                       ctypes.POINTER(_c_int)],
    "agg_tail_split": [_c_int, _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_int, ctypes.POINTER(_c_int),
                       ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)],
    "agg_ag_row_tile_order": [_c_int, _c_int, _c_i64, _c_int, _i32p, _c_int, _c_int, _i32p,
                              _c_int, ctypes.POINTER(_c_int)],
    "agg_rs_row_tile_order": [_c_int, _c_int, _c_i64, _c_int, _i32p, _c_int, _c_int, _i32p,
                              _c_int, ctypes.POINTER(_c_int)],
    "a2a_gemm": [_vp, _c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_f32, _c_f32, _i32p,
                 ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _i32p, _c_int, _u32p, _c_int, _vp, _vp],
    "agg_check_a2a_args": [_c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_f32, _c_f32, _i32p,
                           ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _i32p, _c_int, _c_int, _vp, _vp],
    "agg_a2a_row_tile_order": [_c_int, _c_int, _c_i64, _c_int, _i32p, _i32p, _c_int, _c_int, _i32p,
                               _c_int, ctypes.POINTER(_c_int)],
    "agg_check_ag_args": [_c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_f32, _c_f32,
                          ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _i32p, _c_int, _c_int, _vp, _vp],
    "agg_check_rs_args": [_c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp, _vp, _vp,
                          ctypes.POINTER(_vp), _vp, _vp, _vp, _i32p, _c_int, _c_int, _vp, _vp],
}

_lib = None


class AggError(RuntimeError):
    def __init__(self, code: int, where: str, text: str):
        super().__init__(f"{where} failed with status {code}: {text}")
        self.code = code


def header_functions() -> list:
    """Names of the functions include/agg.h declares."""
    with open(HEADER) as f:
        src = f.read()
    return re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", src, flags=re.M)


def load(path: str | None = None):
    """Load libagg (building it first only if no built library exists) and declare signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        from . import build
        build.build(verbose=False)
    lib = ctypes.CDLL(p)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _c_int
    lib.agg_last_error.argtypes = []
    lib.agg_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _call(name: str, *args) -> None:
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != AGG_OK:
        raise AggError(rc, name, lib.agg_last_error().decode())


# ------------------------------------------------------------------------------ marshalling

def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _checked(items):
    """Device pointers of `items` = [(x, nbytes, what), ...] for a call that touches `nbytes`
    bytes of each x.

    A tensor must be contiguous, hold at least `nbytes` bytes and live on the GPU (every tensor
    is checked for the first two before any for the third); anything else (an int address,
    None) is passed through unchanged and is the caller's responsibility.
    """
    for x, nbytes, what in items:
        if isinstance(x, torch.Tensor):
            if not x.is_contiguous():
                raise AggError(AGG_E_ARG, what, "must be contiguous (the library reads it row-major)")
            have = x.numel() * x.element_size()
            if have < nbytes:
                raise AggError(AGG_E_ARG, what, f"holds {have} bytes, the call touches {nbytes}")
    for x, _, what in items:
        if isinstance(x, torch.Tensor) and x.device.type != "cuda":
            raise AggError(AGG_E_ARG, what, f"must be a device tensor, got {x.device}")
    return [_ptr(x) for x, _, _ in items]


def _stream(s):
    if s is None:
        return None
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def _ptr_array(seq):
    if seq is None:
        return None
    return (_vp * len(seq))(*[_ptr(x) for x in seq])


def _i32_array(seq):
    if seq is None:
        return None, 0
    return (ctypes.c_int32 * len(seq))(*[int(v) for v in seq]), len(seq)


def _u32_array(seq):
    if seq is None:
        return None
    return (ctypes.c_uint32 * len(seq))(*[int(v) for v in seq])


def _mode(mode):
    return MODES[mode] if isinstance(mode, str) else int(mode)


def _dtype(dtype):
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


# ------------------------------------------------------------------------------ entry points

def agg_ctx_create(device: int = 0) -> ctypes.c_void_p:
    out = _vp()
    _call("agg_ctx_create", device, ctypes.byref(out))
    return out


def agg_ctx_destroy(ctx) -> None:
    _call("agg_ctx_destroy", ctx)


def agg_ctx_reset(ctx, stream=None) -> None:
    _call("agg_ctx_reset", ctx, _stream(stream))


def agg_ctx_status(ctx, stream=None):
    """Returns (status, failed_chunk); does not raise on a timeout status."""
    lib = load()
    st, fc = ctypes.c_uint32(), ctypes.c_int32()
    rc = lib.agg_ctx_status(ctx, _stream(stream), ctypes.byref(st), ctypes.byref(fc))
    if rc not in (AGG_OK, AGG_E_TIMEOUT):
        raise AggError(rc, "agg_ctx_status", lib.agg_last_error().decode())
    return st.value, fc.value


def agg_ctx_epoch(ctx) -> int:
    e = ctypes.c_uint32()
    _call("agg_ctx_epoch", ctx, ctypes.byref(e))
    return e.value


def agg_ctx_set_epoch(ctx, epoch: int) -> None:
    _call("agg_ctx_set_epoch", ctx, epoch)


def agg_ctx_set_timeout_us(ctx, timeout_us: int) -> None:
    _call("agg_ctx_set_timeout_us", ctx, timeout_us)


def agg_ctx_set_tile(ctx, bm: int = 0, bn: int = 0) -> None:
    _call("agg_ctx_set_tile", ctx, bm, bn)


def agg_ctx_set_timing(ctx, on=True) -> None:
    """on: False/0 off, True/1 every launch timed, n > 1 every n-th launch timed."""
    _call("agg_ctx_set_timing", ctx, int(on))


def agg_ctx_kernel_times(ctx, max_n: int = 256) -> list:
    """Durations (ms) of the last launches' consumer kernels, oldest first."""
    buf = (ctypes.c_float * max_n)()
    n = _c_int()
    _call("agg_ctx_kernel_times", ctx, buf, max_n, ctypes.byref(n))
    return list(buf[:n.value])


def agg_set_trace(ctx, buf=None, nbytes: int = 0) -> None:
    _call("agg_set_trace", ctx, _ptr(buf), nbytes)


def agg_put_signal(dst, src, nbytes: int, flag, value: int, copy_stream) -> None:
    _call("agg_put_signal", _ptr(dst), _ptr(src), nbytes, _ptr(flag), value, _stream(copy_stream))


def agg_ctx_set_copy_streams(ctx, n: int) -> None:
    _call("agg_ctx_set_copy_streams", ctx, n)


PRODUCERS = {"cu": 0, "sdma": 1, "kernel": 2}


def agg_ctx_set_producer(ctx, kind="cu", copy_wgs: int = 0, piece_kib: int = 0) -> None:
    """Producer of later calls: "cu" (copy jobs inside the persistent kernel), "sdma" (copy
    engines) or "kernel" (a copy kernel beside the persistent kernel)."""
    _call("agg_ctx_set_producer", ctx, PRODUCERS[kind] if isinstance(kind, str) else int(kind),
          copy_wgs, piece_kib)


def agg_ctx_last_producer(ctx):
    """The producer the last call on `ctx` ran ("cu", "sdma", "kernel"), None before the first."""
    v = _c_int(0)
    _call("agg_ctx_last_producer", ctx, ctypes.byref(v))
    names = {i: k for k, i in PRODUCERS.items()}
    return names.get(v.value)


PULL_MODES = {"auto": 0, "off": 1, "on": 2}


def agg_ctx_set_pull(ctx, pull: str = "auto") -> None:
    _call("agg_ctx_set_pull", ctx, PULL_MODES[pull])


def agg_ctx_set_split(ctx, ksplit: int = 0) -> None:
    _call("agg_ctx_set_split", ctx, ksplit)


_TAIL_MODES = {"auto": 0, "off": 1, "on": 2}


def agg_ctx_set_tail(ctx, mode: str = "auto") -> None:
    """Tail split of later ag_gemm / a2a_gemm calls: "auto", "off" or "on"."""
    _call("agg_ctx_set_tail", ctx, _TAIL_MODES[mode] if isinstance(mode, str) else int(mode))


def agg_ctx_set_lists(ctx, lists: int = 8, list_cols: int = 0) -> None:
    _call("agg_ctx_set_lists", ctx, lists, list_cols)


def agg_ctx_set_reserved_cus(ctx, n: int) -> None:
    _call("agg_ctx_set_reserved_cus", ctx, n)


def _ag_ptrs(world, rank, m_shard, n, k, chunk_rows, dtype, peer_src, gather, flags, b, c):
    """Checked device pointers of an ag_gemm call (sizes as include/agg.h states them)."""
    el = 1 if _dtype(dtype) == AGG_FP8_E4M3 else 2
    m = world * m_shard
    cps = m_shard // chunk_rows if chunk_rows > 0 else 0
    items = [(gather, m * k * el, "gather"), (flags, world * cps * 4, "flags"), (b, k * n * el, "b"),
             (c, m * n * 2, "c")]
    if peer_src is not None:
        items += [(p, m_shard * k * el if i != rank else 0, f"peer_src[{i}]")
                  for i, p in enumerate(peer_src)]
    ptrs = _checked(items)
    peers = (_vp * len(peer_src))(*ptrs[4:]) if peer_src is not None else None
    return (peers, *ptrs[:4])


def ag_gemm(ctx, world, rank, m_shard, n, k, chunk_rows, dtype, scale_a, scale_b, peer_src,
            gather, flags, b, c, order=None, delay_us=None, mode="overlap", stream=None,
            copy_stream=None) -> None:
    ordr, n_order = _i32_array(order)
    peers, g, f, bp, cp = _ag_ptrs(world, rank, m_shard, n, k, chunk_rows, dtype, peer_src,
                                   gather, flags, b, c)
    _call("ag_gemm", ctx, world, rank, m_shard, n, k, chunk_rows, _dtype(dtype), scale_a, scale_b,
          peers, g, f, bp, cp, ordr, n_order, _u32_array(delay_us), _mode(mode), _stream(stream),
          _stream(copy_stream))


def ag_gemm_noalloc(ctx, world, rank, m_shard, n, k, chunk_rows, dtype, scale_a, scale_b, peer_src,
                    gather, flags, b, c, order=None, delay_us=None, mode="overlap", stream=None,
                    copy_stream=None) -> None:
    ordr, n_order = _i32_array(order)
    peers, g, f, bp, cp = _ag_ptrs(world, rank, m_shard, n, k, chunk_rows, dtype, peer_src,
                                   gather, flags, b, c)
    _call("ag_gemm_noalloc", ctx, world, rank, m_shard, n, k, chunk_rows, _dtype(dtype), scale_a,
          scale_b, peers, g, f, bp, cp, ordr, n_order, _u32_array(delay_us), _mode(mode),
          _stream(stream), _stream(copy_stream))


def a2a_gemm(ctx, world, rank, cap, n, k, chunk_rows, dtype, scale_a, scale_b, counts, peer_src,
             recv, flags, b, c, order=None, delay_us=None, mode="overlap", stream=None,
             copy_stream=None) -> None:
    """AllToAll (dispatch) + GEMM: slot p of `recv` receives counts[p] rows from source p."""
    if counts is None or len(counts) != world:
        raise AggError(AGG_E_ARG, "a2a_gemm", f"counts must hold {world} entries")
    cnt, _ = _i32_array(counts)
    ordr, n_order = _i32_array(order)
    peers, g, f, bp, cp = _ag_ptrs(world, rank, cap, n, k, chunk_rows, dtype, peer_src, recv, flags, b, c)
    _call("a2a_gemm", ctx, world, rank, cap, n, k, chunk_rows, _dtype(dtype), scale_a, scale_b, cnt,
          peers, g, f, bp, cp, ordr, n_order, _u32_array(delay_us), _mode(mode), _stream(stream),
          _stream(copy_stream))


def _rs_ptrs(world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src, recv, flags, out):
    """Checked device pointers of a gemm_rs call, in its argument order."""
    mb = m // world if world > 0 else 0
    cpb = mb // chunk_rows if chunk_rows > 0 else 0
    items = [(a, m * k * 2, "a"), (b, k * n * 2, "b"), (send, max(world - 1, 0) * mb * n * 4, "send"),
             (send_flags, world * cpb * 4, "send_flags"), (recv, world * mb * n * 4, "recv"),
             (flags, world * cpb * 4, "flags"), (out, mb * n * 4, "out")]
    if peer_src is not None:
        items += [(p, mb * n * 4 if i != rank else 0, f"peer_src[{i}]") for i, p in enumerate(peer_src)]
    ptrs = _checked(items)
    peers = (_vp * len(peer_src))(*ptrs[7:]) if peer_src is not None else None
    return (*ptrs[:4], peers, *ptrs[4:7])


def gemm_rs(ctx, world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src, recv, flags,
            out, order=None, delay_us=None, mode="overlap", stream=None, copy_stream=None) -> None:
    ordr, n_order = _i32_array(order)
    ptrs = _rs_ptrs(world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src, recv,
                    flags, out)
    _call("gemm_rs", ctx, world, rank, m, n, k, chunk_rows, *ptrs, ordr, n_order,
          _u32_array(delay_us), _mode(mode), _stream(stream), _stream(copy_stream))


def _ar_ptrs(world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src, recv, flags, out):
    """Checked device pointers of a gemm_ar call, in its argument order."""
    cpb = m // chunk_rows if chunk_rows > 0 else 0
    items = [(a, m * k * 2, "a"), (b, k * n * 2, "b"), (send, m * n * 4, "send"),
             (send_flags, cpb * 4, "send_flags"), (recv, world * m * n * 4, "recv"),
             (flags, world * cpb * 4, "flags"), (out, m * n * 4, "out")]
    if peer_src is not None:
        items += [(p, m * n * 4 if i != rank else 0, f"peer_src[{i}]") for i, p in enumerate(peer_src)]
    ptrs = _checked(items)
    peers = (_vp * len(peer_src))(*ptrs[7:]) if peer_src is not None else None
    return (*ptrs[:4], peers, *ptrs[4:7])


def gemm_ar(ctx, world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src, recv, flags,
            out, order=None, delay_us=None, mode="overlap", stream=None, copy_stream=None) -> None:
    ordr, n_order = _i32_array(order)
    ptrs = _ar_ptrs(world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src, recv,
                    flags, out)
    _call("gemm_ar", ctx, world, rank, m, n, k, chunk_rows, *ptrs, ordr, n_order,
          _u32_array(delay_us), _mode(mode), _stream(stream), _stream(copy_stream))


def ffn_chain(ctx, world, rank, m_shard, k1, n1, n2, chunk_rows, rs_chunk_rows, peer_src, gather,
              flags, w1, h, w2, send, send_flags, rs_peer_src, recv, rs_flags, out, order=None,
              rs_order=None, mode="overlap", stream=None, copy_stream=None) -> None:
    m = world * m_shard
    cps = m_shard // chunk_rows if chunk_rows > 0 else 0
    cpb = m_shard // rs_chunk_rows if rs_chunk_rows > 0 else 0
    items = [(gather, m * k1 * 2, "gather"), (flags, world * cps * 4, "flags"), (w1, k1 * n1 * 2, "w1"),
             (h, m * n1 * 2, "h"), (w2, n1 * n2 * 2, "w2"),
             (send, max(world - 1, 0) * m_shard * n2 * 4, "send"), (send_flags, world * cpb * 4, "send_flags"),
             (recv, world * m_shard * n2 * 4, "recv"), (rs_flags, world * cpb * 4, "rs_flags"),
             (out, m_shard * n2 * 4, "out")]
    for i, p in enumerate(peer_src or []):
        items.append((p, m_shard * k1 * 2 if i != rank else 0, f"peer_src[{i}]"))
    for i, p in enumerate(rs_peer_src or []):
        items.append((p, m_shard * n2 * 4 if i != rank else 0, f"rs_peer_src[{i}]"))
    ptrs = _checked(items)
    nw = len(peer_src or [])
    peers = (_vp * nw)(*ptrs[10:10 + nw]) if peer_src is not None else None
    rs_peers = (_vp * len(rs_peer_src))(*ptrs[10 + nw:]) if rs_peer_src is not None else None
    ordr, n_order = _i32_array(order)
    rs_ordr, n_rs_order = _i32_array(rs_order)
    _call("ffn_chain", ctx, world, rank, m_shard, k1, n1, n2, chunk_rows, rs_chunk_rows, peers,
          ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], ptrs[5], ptrs[6], rs_peers, ptrs[7], ptrs[8],
          ptrs[9], ordr, n_order, rs_ordr, n_rs_order, _mode(mode), _stream(stream),
          _stream(copy_stream))


def agg_ctx_set_chain_fused(ctx, on: bool = True) -> None:
    _call("agg_ctx_set_chain_fused", ctx, 1 if on else 0)


def agg_tile_shape(op: int, dtype, m: int, n: int, k: int):
    bm, bn = _c_int(), _c_int()
    _call("agg_tile_shape", op, _dtype(dtype), m, n, k, ctypes.byref(bm), ctypes.byref(bn))
    return bm.value, bn.value


def agg_tail_split(bm: int, bn: int, m: int, n: int, n_row_tiles: int, units: int = 256, mode="auto"):
    """(head row tiles, tail tile shape) of the tail split; head 0 = no split."""
    head, tbm, tbn = _c_int(), _c_int(), _c_int()
    _call("agg_tail_split", bm, bn, m, n, n_row_tiles, units,
          _TAIL_MODES[mode] if isinstance(mode, str) else int(mode),
          ctypes.byref(head), ctypes.byref(tbm), ctypes.byref(tbn))
    return head.value, (tbm.value, tbn.value)


def _tile_order(name, world, rank, size, chunk_rows, order, bm):
    ordr, n_order = _i32_array(order)
    cap = MAX_ROW_TILES * 64
    out = (ctypes.c_int32 * cap)()
    n = _c_int()
    _call(name, world, rank, size, chunk_rows, ordr, n_order, bm, out, cap, ctypes.byref(n))
    return list(out[:n.value])


def agg_ag_row_tile_order(world, rank, m_shard, chunk_rows, order, bm) -> list:
    return _tile_order("agg_ag_row_tile_order", world, rank, m_shard, chunk_rows, order, bm)


def agg_rs_row_tile_order(world, rank, m, chunk_rows, order, bm) -> list:
    return _tile_order("agg_rs_row_tile_order", world, rank, m, chunk_rows, order, bm)


def agg_a2a_row_tile_order(world, rank, cap, chunk_rows, counts, order, bm) -> list:
    cnt, _ = _i32_array(counts)
    ordr, n_order = _i32_array(order)
    room = MAX_ROW_TILES * 64
    out = (ctypes.c_int32 * room)()
    n = _c_int()
    _call("agg_a2a_row_tile_order", world, rank, cap, chunk_rows, cnt, ordr, n_order, bm, out, room,
          ctypes.byref(n))
    return list(out[:n.value])


def agg_check_a2a_args(world, rank, cap, n, k, chunk_rows, dtype, scale_a, scale_b, counts, peer_src,
                       recv, flags, b, c, order=None, mode="overlap", stream=None,
                       copy_stream=None) -> int:
    """Returns the status code (does not raise) so tests can check each error code."""
    cnt, _ = _i32_array(counts)
    ordr, n_order = _i32_array(order)
    return load().agg_check_a2a_args(world, rank, cap, n, k, chunk_rows, _dtype(dtype), scale_a,
                                     scale_b, cnt, _ptr_array(peer_src), _ptr(recv), _ptr(flags),
                                     _ptr(b), _ptr(c), ordr, n_order, _mode(mode), _stream(stream),
                                     _stream(copy_stream))


def agg_check_ag_args(world, rank, m_shard, n, k, chunk_rows, dtype, scale_a, scale_b, peer_src,
                      gather, flags, b, c, order=None, mode="overlap", stream=None,
                      copy_stream=None) -> int:
    """Returns the status code (does not raise) so tests can check each error code."""
    ordr, n_order = _i32_array(order)
    return load().agg_check_ag_args(world, rank, m_shard, n, k, chunk_rows, _dtype(dtype), scale_a,
                                    scale_b, _ptr_array(peer_src), _ptr(gather), _ptr(flags),
                                    _ptr(b), _ptr(c), ordr, n_order, _mode(mode), _stream(stream),
                                    _stream(copy_stream))


def agg_check_rs_args(world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src, recv,
                      flags, out, order=None, mode="overlap", stream=None, copy_stream=None) -> int:
    ordr, n_order = _i32_array(order)
    return load().agg_check_rs_args(world, rank, m, n, k, chunk_rows, _ptr(a), _ptr(b), _ptr(send),
                                    _ptr(send_flags), _ptr_array(peer_src), _ptr(recv), _ptr(flags),
                                    _ptr(out), ordr, n_order, _mode(mode), _stream(stream),
                                    _stream(copy_stream))


def last_error() -> str:
    return load().agg_last_error().decode()


def agg_check_ar_args(world, rank, m, n, k, chunk_rows, a, b, send, send_flags, peer_src, recv,
                      flags, out, order=None, mode="overlap", stream=None, copy_stream=None) -> int:
    ordr, n_order = _i32_array(order)
    return load().agg_check_ar_args(world, rank, m, n, k, chunk_rows, _ptr(a), _ptr(b), _ptr(send),
                                    _ptr(send_flags), _ptr_array(peer_src), _ptr(recv), _ptr(flags),
                                    _ptr(out), ordr, n_order, _mode(mode), _stream(stream),
                                    _stream(copy_stream))


def agg_kernel_regs(op: int, dtype, bm: int, bn: int):
    """(GEMM kernel registers per lane, copy kernel registers per lane) as the runtime reports them."""
    g, c = _c_int(), _c_int()
    _call("agg_kernel_regs", op, _dtype(dtype), bm, bn, ctypes.byref(g), ctypes.byref(c))
    return g.value, c.value
