"""ctypes wrapper of the fp64 CPU oracle (oracle/zha_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the HIP implementation.  The wrapper
only marshals numpy arrays; every step of the method is in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zha_oracle.c")
_LIB = os.path.join(_HERE, "libzha_oracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _bind(path: str):
    L = ctypes.CDLL(path)
    L.zo_tree_tokens.restype = _i64
    L.zo_tree_tokens.argtypes = [_i64, _int]
    L.zo_level_nodes.restype = _i64
    L.zo_level_nodes.argtypes = [_i64, _int, _int]
    L.zo_node_planes.restype = None
    L.zo_node_planes.argtypes = [_f64p, _int, _i64, _i64, _f64p, _int, _f64p, _f64p, _f64p]
    for fn in (L.zo_tree_definition, L.zo_tree_merge):
        fn.restype = None
        fn.argtypes = [_f64p, _i64, _int, _f64p, _int, _int, _int, _f64p, _f64p, _f64p]
    L.zo_select.restype = _i64
    L.zo_select.argtypes = [_f64p, _f64p, _int, _int, _f64p, _int, _i32p, _i64, ctypes.c_double,
                            _i32p, _f64p, _i64p, _f64p]
    L.zo_expand.restype = _i64
    L.zo_expand.argtypes = [_i32p, _i64, _int, _i64, _i32p]
    L.zo_route.restype = None
    L.zo_route.argtypes = [_f64p, _f64p, _i64, _int, _int, _int, _int, _f64p, _int, ctypes.c_double,
                           _i32p, _i64p, _i32p, _i64p]
    L.zo_attend_set.restype = _i64
    L.zo_attend_set.argtypes = [_i64, _int, _i32p, _i64, _i64p]
    L.zo_block_attend_set.restype = _i64
    L.zo_block_attend_set.argtypes = [_i64, _int, _i32p, _i64, _i64, _i64p]
    L.zo_attend.restype = None
    L.zo_attend.argtypes = [_f64p, _int, _int, _f64p, _f64p, _i64p, _i64, _f64p, _f64p]
    L.zo_attend_blockwise.restype = None
    L.zo_attend_blockwise.argtypes = [_f64p, _int, _int, _f64p, _f64p, _i64p, _i64, _i64, _f64p, _f64p]
    L.zo_e4m3_round.restype = ctypes.c_double
    L.zo_e4m3_round.argtypes = [ctypes.c_double]
    L.zo_e4m3_row_exp.restype = _int
    L.zo_e4m3_row_exp.argtypes = [ctypes.c_double]
    L.zo_fp8_rows.restype = None
    L.zo_fp8_rows.argtypes = [_f64p, _i64, _int, _f64p, _f64p]
    L.zo_e2m1_round.restype = ctypes.c_double
    L.zo_e2m1_round.argtypes = [ctypes.c_double]
    L.zo_e2m1_block_exp.restype = _int
    L.zo_e2m1_block_exp.argtypes = [ctypes.c_double]
    L.zo_fp4_rows.restype = None
    L.zo_fp4_rows.argtypes = [_f64p, _i64, _int, _f64p, _f64p]
    for fn in (L.zo_fp8_planes, L.zo_fp4_planes):
        fn.restype = None
        fn.argtypes = [_f64p, _f64p, _f64p, _i64, _int, _int, _f64p, _f64p, _f64p]
    L.zo_num_threads.restype = _int
    L.zo_num_threads.argtypes = []
    L.zo_set_num_threads.restype = None
    L.zo_set_num_threads.argtypes = [_int]
    return L


def lib():
    global _lib
    if _lib is None:
        _lib = _bind(build())
    return _lib


def use_library(path: str | None):
    """Point this wrapper at another build of zha_oracle.c (None: the default build).

    Used by the tests that check the pins against deliberately broken copies of
    the oracle.  Returns the previously bound library handle.
    """
    global _lib
    prev = _lib
    _lib = None if path is None else _bind(path)
    return prev


def restore_library(handle) -> None:
    global _lib
    _lib = handle


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a, t):
    return a.ctypes.data_as(t)


def num_threads() -> int:
    return lib().zo_num_threads()


def set_num_threads(n: int) -> None:
    lib().zo_set_num_threads(int(n))


def tree_tokens(N: int, C: int) -> int:
    return lib().zo_tree_tokens(N, C)


def level_nodes(N: int, C: int, l: int) -> int:
    return lib().zo_level_nodes(N, C, l)


def node_planes(K, t0: int, t1: int, refs):
    """Planes (m [R][d], b [R], lse [R]) of the node covering tokens [t0, t1)."""
    K, refs = _f64(K), _f64(refs)
    R, d = refs.shape
    m = np.empty((R, d)); b = np.empty(R); lse = np.empty(R)
    lib().zo_node_planes(_p(K, _f64p), d, t0, t1, _p(refs, _f64p), R, _p(m, _f64p), _p(b, _f64p), _p(lse, _f64p))
    return m, b, lse


def e4m3_round(x: float) -> float:
    """Nearest OCP fp8 e4m3 value to x (|x| <= 448), ties to even mantissa."""
    return lib().zo_e4m3_round(float(x))


def e4m3_row_exp(amax: float) -> int:
    """Smallest s with amax * 2^-s <= 448 (0 for amax = 0)."""
    return lib().zo_e4m3_row_exp(float(amax))


def fp8_rows(m):
    """fp8 summary storage of rows m [..., d]: (m~ = grid value * 2^s per row, scale 2^s [...])."""
    m = _f64(m)
    shp = m.shape
    d = shp[-1]
    flat = m.reshape(-1, d)
    out = np.empty_like(flat); sc = np.empty(flat.shape[0])
    lib().zo_fp8_rows(_p(flat, _f64p), flat.shape[0], d, _p(out, _f64p), _p(sc, _f64p))
    return out.reshape(shp), sc.reshape(shp[:-1])


def _lowp_planes(fn, m, lse, refs, scale_shape):
    m, lse, refs = _f64(m), _f64(lse), _f64(refs)
    n, R, d = m.shape
    mq = np.empty_like(m); b = np.empty((n, R)); sc = np.empty(scale_shape)
    fn(_p(m, _f64p), _p(lse, _f64p), _p(refs, _f64p), n, R, d, _p(mq, _f64p), _p(b, _f64p), _p(sc, _f64p))
    return mq, b, sc


def fp8_planes(m, lse, refs):
    """Planes with fp8-stored means (zo_fp8_planes): (m~ [n][R][d], b~ = LSE - r.m~ [n][R],
    scale [n][R])."""
    m = _f64(m)
    return _lowp_planes(lib().zo_fp8_planes, m, lse, refs, m.shape[:2])


def e2m1_round(x: float) -> float:
    """Nearest OCP fp4 e2m1 value to x (|x| <= 6), ties to even mantissa."""
    return lib().zo_e2m1_round(float(x))


def e2m1_block_exp(amax: float) -> int:
    """Smallest s with amax * 2^-s <= 6 (0 for amax = 0)."""
    return lib().zo_e2m1_block_exp(float(amax))


def fp4_rows(m):
    """fp4 summary storage of rows m [..., d] (d a multiple of 32): (m~ = grid value * 2^s per
    block of 32 values, scales 2^s [..., d / 32])."""
    m = _f64(m)
    shp = m.shape
    d = shp[-1]
    flat = m.reshape(-1, d)
    out = np.empty_like(flat); sc = np.empty((flat.shape[0], d // 32))
    lib().zo_fp4_rows(_p(flat, _f64p), flat.shape[0], d, _p(out, _f64p), _p(sc, _f64p))
    return out.reshape(shp), sc.reshape(shp[:-1] + (d // 32,))


def fp4_planes(m, lse, refs):
    """Planes with fp4-stored means (zo_fp4_planes): (m~ [n][R][d], b~ = LSE - r.m~ [n][R],
    scales [n][R][d/32])."""
    m = _f64(m)
    return _lowp_planes(lib().zo_fp4_planes, m, lse, refs, m.shape[:2] + (m.shape[2] // 32,))


class Tree:
    """Per-level planes of one unit: m[l] [n_l][R][d], b[l] / lse[l] [n_l][R], l = 1..L."""

    def __init__(self, m_all, b_all, lse_all, counts):
        self.m, self.b, self.lse = {}, {}, {}
        off = 0
        for l, n in enumerate(counts, start=1):
            self.m[l] = m_all[off:off + n]
            self.b[l] = b_all[off:off + n]
            self.lse[l] = lse_all[off:off + n]
            off += n
        self.m_all, self.b_all, self.lse_all = m_all, b_all, lse_all
        self.counts = list(counts)


def _tree(fn, K, refs, C: int, L: int) -> Tree:
    K, refs = _f64(K), _f64(refs)
    N, d = K.shape
    R = refs.shape[0]
    counts = [level_nodes(N, C, l) for l in range(1, L + 1)]
    tot = sum(counts)
    m = np.empty((tot, R, d)); b = np.empty((tot, R)); lse = np.empty((tot, R))
    fn(_p(K, _f64p), N, d, _p(refs, _f64p), R, C, L, _p(m, _f64p), _p(b, _f64p), _p(lse, _f64p))
    return Tree(m, b, lse, counts)


def tree_definition(K, refs, C: int, L: int) -> Tree:
    return _tree(lib().zo_tree_definition, K, refs, C, L)


def tree_merge(K, refs, C: int, L: int) -> Tree:
    return _tree(lib().zo_tree_merge, K, refs, C, L)


def select(m_l, b_l, q, F, p: float):
    """One routing level from frontier F.  Returns (kept ids ascending, w, order, csum)."""
    m_l, b_l, q = _f64(m_l), _f64(b_l), _f64(q)
    F = np.ascontiguousarray(F, dtype=np.int32)
    R, d = m_l.shape[1], m_l.shape[2]
    G = q.shape[0]
    nF = len(F)
    kept = np.empty(max(nF, 1), dtype=np.int32)
    w = np.empty(max(nF, 1)); order = np.empty(max(nF, 1), dtype=np.int64); csum = np.empty(max(nF, 1))
    k = lib().zo_select(_p(m_l, _f64p), _p(b_l, _f64p), R, d, _p(q, _f64p), G, _p(F, _i32p), nF, float(p),
                        _p(kept, _i32p), _p(w, _f64p), _p(order, _i64p), _p(csum, _f64p))
    return kept[:k].copy(), w[:nF], order[:nF], csum[:nF]


def expand(kept, C: int, n_child: int):
    kept = np.ascontiguousarray(kept, dtype=np.int32)
    out = np.empty(max(len(kept) * C, 1), dtype=np.int32)
    n = lib().zo_expand(_p(kept, _i32p), len(kept), C, n_child, _p(out, _i32p))
    return out[:n].copy()


def route(tree: Tree, N: int, C: int, L: int, q, p: float):
    """Full route of one unit.  Returns ({l: frontier ids}, {l: kept ids})."""
    q = _f64(q)
    G, d = q.shape
    R = tree.m_all.shape[1]
    tot = sum(tree.counts)
    F = np.empty(max(tot, 1), dtype=np.int32); K = np.empty(max(tot, 1), dtype=np.int32)
    nF = np.zeros(L, dtype=np.int64); nK = np.zeros(L, dtype=np.int64)
    lib().zo_route(_p(tree.m_all, _f64p), _p(tree.b_all, _f64p), N, d, R, C, L, _p(q, _f64p), G, float(p),
                   _p(F, _i32p), _p(nF, _i64p), _p(K, _i32p), _p(nK, _i64p))
    Fd, Kd, off = {}, {}, 0
    for l, n in enumerate(tree.counts, start=1):
        Fd[l] = F[off:off + nF[l - 1]].copy()
        Kd[l] = K[off:off + nK[l - 1]].copy()
        off += n
    return Fd, Kd


def attend_set(N: int, C: int, kept):
    kept = np.ascontiguousarray(kept, dtype=np.int32)
    out = np.empty(max(N, 1), dtype=np.int64)
    n = lib().zo_attend_set(N, C, _p(kept, _i32p), len(kept), _p(out, _i64p))
    return out[:n].copy()


def block_attend_set(N: int, C: int, kept, t: int):
    """Attention set of query t of a block of queries after N cached tokens: the decode set
    over the cache plus the block's rows N .. N + t (zo_block_attend_set)."""
    kept = np.ascontiguousarray(kept, dtype=np.int32)
    out = np.empty(N + t + 1, dtype=np.int64)
    n = lib().zo_block_attend_set(N, C, _p(kept, _i32p), len(kept), t, _p(out, _i64p))
    return out[:n].copy()


def attend(q, K, V, S):
    """Exact attention of q [G][d] over token set S.  Returns (out [G][d], lse [G])."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    S = np.ascontiguousarray(S, dtype=np.int64)
    G, d = q.shape
    out = np.empty((G, d)); lse = np.empty(G)
    lib().zo_attend(_p(q, _f64p), G, d, _p(K, _f64p), _p(V, _f64p), _p(S, _i64p), len(S),
                    _p(out, _f64p), _p(lse, _f64p))
    return out, lse


def attend_blockwise(q, K, V, S, block: int):
    q, K, V = _f64(q), _f64(K), _f64(V)
    S = np.ascontiguousarray(S, dtype=np.int64)
    G, d = q.shape
    out = np.empty((G, d)); lse = np.empty(G)
    lib().zo_attend_blockwise(_p(q, _f64p), G, d, _p(K, _f64p), _p(V, _f64p), _p(S, _i64p), len(S), block,
                              _p(out, _f64p), _p(lse, _f64p))
    return out, lse


def dense_tokens(N: int):
    return np.arange(N, dtype=np.int64)
