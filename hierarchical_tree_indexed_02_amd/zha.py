"""ctypes binding of libzha.so, the C ABI in include/zha.h.

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  Functions keep the C names; device pointers may be given as
torch tensors (their data_ptr) or integers; streams default to torch's current
stream.  A non-OK status raises ZhaError.  Importing this module fails loudly
when the compiled library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzha.so")

ZHA_OK, ZHA_ERR_INVALID, ZHA_ERR_CAPACITY, ZHA_ERR_NOMEM, ZHA_ERR_UNSUPPORTED, ZHA_ERR_HIP, ZHA_ERR_DEVICE = range(7)
ZHA_F32, ZHA_BF16 = 0, 1
ZHA_SUMMARY_NATIVE, ZHA_SUMMARY_FP8, ZHA_SUMMARY_FP4 = 0, 1, 2
ZHA_ROUTE_GROUP, ZHA_ROUTE_PER_HEAD = 0, 1
ZHA_K_BUILD, ZHA_K_APPEND, ZHA_K_SCORE, ZHA_K_SELECT, ZHA_K_ATTEND, ZHA_K_MERGE, ZHA_K_MASS, ZHA_K_COMPACT = range(1, 9)
KERNEL_NAMES = {1: "build", 2: "append", 3: "score", 4: "select", 5: "attend", 6: "merge", 7: "mass", 8: "compact"}


class zha_tree_desc(Structure):
    _fields_ = [("batch", c_int32), ("n_kv_heads", c_int32), ("n_q_heads", c_int32), ("head_dim", c_int32),
                ("chunk", c_int32), ("levels", c_int32), ("n_refs", c_int32), ("max_tokens", c_int64),
                ("dtype", c_int), ("summary", c_int), ("per_head_routes", c_int32),
                ("max_queries", c_int32)]


class zha_kept(Structure):
    _fields_ = [("counts", c_void_p), ("ids", c_void_p), ("cap", c_int64)]


class ZhaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = f" [{zha_last_error()}]" if status == ZHA_ERR_HIP else ""
        super().__init__(f"{where}: {zha_status_str(status)} (status {status}){detail}")


_lib = None
_i32p = POINTER(c_int32)


def load():
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime with the same soname as the system one; loading
        # torch first makes libzha.so bind to that runtime instead of mapping a second one
        # (two HIP runtimes in one process do not share devices, streams or memory).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libzha.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, st = c_void_p, c_int
        sig = {
            "zha_status_str": (c_char_p, [c_int]),
            "zha_last_error": (c_char_p, []),
            "zha_tree_create": (st, [POINTER(zha_tree_desc), POINTER(c_void_p)]),
            "zha_tree_destroy": (None, [vp]),
            "zha_tree_bytes": (st, [vp, POINTER(c_int64)]),
            "zha_tree_check": (st, [vp, vp]),
            "zha_build": (st, [vp, vp, vp, _i32p, vp]),
            "zha_append": (st, [vp, vp, _i32p, vp]),
            "zha_route": (st, [vp, vp, c_float, c_float, POINTER(zha_kept), vp]),
            "zha_route_ex": (st, [vp, vp, c_float, c_float, c_int, POINTER(zha_kept), vp]),
            "zha_attend": (st, [vp, vp, vp, vp, POINTER(zha_kept), c_float, vp, vp, vp]),
            "zha_route_multi": (st, [vp, vp, c_int32, c_float, c_float, c_int, POINTER(zha_kept), vp]),
            "zha_attend_multi": (st, [vp, vp, c_int32, vp, vp, POINTER(zha_kept), c_float, vp, vp, vp]),
            "zha_dense_decode": (st, [vp, vp, vp, _i32p, c_int32, c_int32, c_int32, c_int32, c_int64, c_int,
                                      c_float, vp, vp, vp, c_size_t, vp]),
            "zha_dense_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int64]),
            "zha_dense_decode_noalloc": (st, [vp, vp, vp, _i32p, c_int32, c_int32, c_int32, c_int32, c_int64, c_int,
                                              c_float, vp, vp, vp]),
            "zha_tree_level_capacity": (st, [vp, c_int32, POINTER(c_int64)]),
            "zha_tree_copy_level": (st, [vp, c_int32, vp, vp, vp]),
            "zha_tree_copy_scales": (st, [vp, c_int32, vp, vp]),
            "zha_route_copy_level": (st, [vp, c_int32, vp, vp, vp, vp]),
            "zha_timing_enable": (st, [vp, c_int32, c_int32]),
            "zha_timing_read": (st, [vp, _i32p, _i32p, POINTER(c_float), c_int32, _i32p]),
            "zha_calibration_copy": (st, [vp, vp, c_int64, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(x) -> int:
    if x is None:
        return 0
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(s) -> int:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    return int(s)


def _check(status: int, where: str) -> None:
    if status != ZHA_OK:
        raise ZhaError(status, where)


def _lens(seq_lens):
    vals = [int(v) for v in seq_lens]
    return (c_int32 * max(len(vals), 1))(*vals)


def zha_status_str(status: int) -> str:
    return load().zha_status_str(int(status)).decode()


def zha_last_error() -> str:
    return load().zha_last_error().decode()


def zha_tree_create(desc: zha_tree_desc) -> int:
    h = c_void_p()
    _check(load().zha_tree_create(ctypes.byref(desc), ctypes.byref(h)), "zha_tree_create")
    return h.value


def zha_tree_destroy(tree: int) -> None:
    load().zha_tree_destroy(tree)


def zha_tree_bytes(tree: int) -> int:
    v = c_int64()
    _check(load().zha_tree_bytes(tree, ctypes.byref(v)), "zha_tree_bytes")
    return v.value


def zha_tree_check(tree: int, stream=None) -> None:
    """Synchronises the stream and raises ZhaError(ZHA_ERR_DEVICE) if a device-side bounded
    wait of the tree's routes gave up since the last check (the mark is cleared)."""
    _check(load().zha_tree_check(tree, _stream(stream)), "zha_tree_check")


def zha_build(tree: int, K, refs, seq_lens, stream=None) -> None:
    _check(load().zha_build(tree, _ptr(K), _ptr(refs), _lens(seq_lens), _stream(stream)), "zha_build")


def zha_append(tree: int, K, new_seq_lens, stream=None) -> None:
    _check(load().zha_append(tree, _ptr(K), _lens(new_seq_lens), _stream(stream)), "zha_append")


def zha_route(tree: int, q, p: float, scale: float, stream=None) -> zha_kept:
    kept = zha_kept()
    _check(load().zha_route(tree, _ptr(q), float(p), float(scale), ctypes.byref(kept), _stream(stream)), "zha_route")
    return kept


def zha_route_ex(tree: int, q, p: float, scale: float, mode: int, stream=None) -> zha_kept:
    kept = zha_kept()
    _check(load().zha_route_ex(tree, _ptr(q), float(p), float(scale), int(mode), ctypes.byref(kept), _stream(stream)),
           "zha_route_ex")
    return kept


def zha_route_multi(tree: int, q, n_queries: int, p: float, scale: float, mode: int, stream=None) -> zha_kept:
    kept = zha_kept()
    _check(load().zha_route_multi(tree, _ptr(q), int(n_queries), float(p), float(scale), int(mode),
                                  ctypes.byref(kept), _stream(stream)), "zha_route_multi")
    return kept


def zha_attend_multi(tree: int, q, n_queries: int, K, V, kept: zha_kept, scale: float, out, lse,
                     stream=None) -> None:
    _check(load().zha_attend_multi(tree, _ptr(q), int(n_queries), _ptr(K), _ptr(V), ctypes.byref(kept),
                                   float(scale), _ptr(out), _ptr(lse), _stream(stream)), "zha_attend_multi")


def zha_attend(tree: int, q, K, V, kept: zha_kept, scale: float, out, lse, stream=None) -> None:
    _check(load().zha_attend(tree, _ptr(q), _ptr(K), _ptr(V), ctypes.byref(kept), float(scale), _ptr(out), _ptr(lse),
                             _stream(stream)), "zha_attend")


def zha_dense_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, max_tokens: int) -> int:
    return int(load().zha_dense_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_tokens))


def zha_dense_decode(q, K, V, seq_lens, batch, n_q_heads, n_kv_heads, head_dim, max_tokens, dtype, scale, out, lse,
                     workspace, workspace_bytes, stream=None) -> None:
    _check(load().zha_dense_decode(_ptr(q), _ptr(K), _ptr(V), _lens(seq_lens), batch, n_q_heads, n_kv_heads,
                                   head_dim, max_tokens, dtype, float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                   int(workspace_bytes), _stream(stream)), "zha_dense_decode")


ZHA_DENSE_SCRATCH_BYTES = 8 << 20


def zha_dense_decode_noalloc(q, K, V, seq_lens, batch, n_q_heads, n_kv_heads, head_dim, max_tokens, dtype, scale, out,
                             lse, stream=None) -> None:
    _check(load().zha_dense_decode_noalloc(_ptr(q), _ptr(K), _ptr(V), _lens(seq_lens), batch, n_q_heads, n_kv_heads,
                                           head_dim, max_tokens, dtype, float(scale), _ptr(out), _ptr(lse),
                                           _stream(stream)), "zha_dense_decode_noalloc")


def zha_tree_level_capacity(tree: int, level: int) -> int:
    v = c_int64()
    _check(load().zha_tree_level_capacity(tree, level, ctypes.byref(v)), "zha_tree_level_capacity")
    return v.value


def zha_tree_copy_level(tree: int, level: int, m_out, b_out, stream=None) -> None:
    _check(load().zha_tree_copy_level(tree, level, _ptr(m_out), _ptr(b_out), _stream(stream)), "zha_tree_copy_level")


def zha_tree_copy_scales(tree: int, level: int, scale_out, stream=None) -> None:
    _check(load().zha_tree_copy_scales(tree, level, _ptr(scale_out), _stream(stream)), "zha_tree_copy_scales")


def zha_route_copy_level(tree: int, level: int, frontier_counts, kept_counts, kept_ids, stream=None) -> None:
    _check(load().zha_route_copy_level(tree, level, _ptr(frontier_counts), _ptr(kept_counts), _ptr(kept_ids),
                                       _stream(stream)), "zha_route_copy_level")


ZHA_TIMING_ALL = -1


def zha_timing_enable(tree: int, kernel_mask: int, level_mask: int = ZHA_TIMING_ALL) -> None:
    _check(load().zha_timing_enable(tree, int(kernel_mask), int(level_mask)), "zha_timing_enable")


def zha_timing_read(tree: int, max_entries: int = 256):
    """Returns [(kernel code, level, ms), ...] of the launches recorded since the last read."""
    k = (c_int32 * max_entries)()
    l = (c_int32 * max_entries)()
    ms = (c_float * max_entries)()
    n = c_int32()
    _check(load().zha_timing_read(tree, k, l, ms, max_entries, ctypes.byref(n)), "zha_timing_read")
    return [(int(k[i]), int(l[i]), float(ms[i])) for i in range(n.value)]


def zha_calibration_copy(dst, src, n16: int, stream=None) -> None:
    _check(load().zha_calibration_copy(_ptr(dst), _ptr(src), int(n16), _stream(stream)), "zha_calibration_copy")
