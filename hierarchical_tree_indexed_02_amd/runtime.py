"""Torch-side helpers around the ctypes binding: allocation of output and
inspection buffers on the current device, and a Tree object that owns a
zha_tree handle.  Every computation happens in libzha.so's kernels."""
from __future__ import annotations

import torch

from . import zha

_DT = {torch.bfloat16: zha.ZHA_BF16, torch.float32: zha.ZHA_F32}


def zdtype(t: torch.dtype) -> int:
    if t not in _DT:
        raise ValueError(f"unsupported dtype {t}")
    return _DT[t]


class Tree:
    """One attention layer's summary tree (library-owned device memory)."""

    def __init__(self, batch, n_kv_heads, n_q_heads, head_dim, chunk, levels, n_refs, max_tokens,
                 dtype=torch.bfloat16, summary="native", per_head_routes=False, max_queries=1):
        """summary: "native" (m stored in dtype), "fp8" (e4m3 codes with a power-of-two
        scale per node and reference) or "fp4" (e2m1 codes with a power-of-two scale per block
        of 32 values); fp8 and fp4 need dtype bf16.  per_head_routes: the tree also serves
        routes that give every query head its own kept set (route(..., mode="per_head")).
        max_queries: queries per sequence one route_multi may carry."""
        codes = {"native": zha.ZHA_SUMMARY_NATIVE, "fp8": zha.ZHA_SUMMARY_FP8, "fp4": zha.ZHA_SUMMARY_FP4}
        if summary not in codes:
            raise ValueError(f"unsupported summary storage {summary!r}")
        self.desc = zha.zha_tree_desc(batch, n_kv_heads, n_q_heads, head_dim, chunk, levels, n_refs, max_tokens,
                                      zdtype(dtype),
                                      codes[summary],
                                      1 if per_head_routes else 0, max_queries)
        self.RU = batch * n_kv_heads  # routing units of the last route
        self.dtype = dtype
        self.summary = summary
        self.B, self.Hkv, self.Hq, self.d = batch, n_kv_heads, n_q_heads, head_dim
        self.C, self.L, self.R, self.T = chunk, levels, n_refs, max_tokens
        self.U = batch * n_kv_heads
        self.G = n_q_heads // n_kv_heads
        self.h = zha.zha_tree_create(self.desc)
        self.kept = None
        self.Tq = 1  # queries per sequence of the last route

    def close(self):
        if getattr(self, "h", None):
            zha.zha_tree_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def bytes(self) -> int:
        return zha.zha_tree_bytes(self.h)

    def check(self, stream=None):
        """Synchronises and raises if a device-side bounded wait of a route gave up."""
        zha.zha_tree_check(self.h, stream)

    def build(self, K, refs, seq_lens, stream=None):
        zha.zha_build(self.h, K, refs, seq_lens, stream)

    def append(self, K, new_seq_lens, stream=None):
        zha.zha_append(self.h, K, new_seq_lens, stream)

    def route(self, q, p, scale=1.0, stream=None, mode="group"):
        """mode "group": one kept set per (sequence, KV head); "per_head": one per (sequence,
        query head), each head routed alone.  Routing units are numbered with the head fastest."""
        if mode == "group":
            self.kept = zha.zha_route(self.h, q, p, scale, stream)
            self.RU = self.U
        elif mode == "per_head":
            self.kept = zha.zha_route_ex(self.h, q, p, scale, zha.ZHA_ROUTE_PER_HEAD, stream)
            self.RU = self.U * self.G
        else:
            raise ValueError(f"unknown routing mode {mode!r}")
        self.Tq = 1
        return self.kept

    def route_multi(self, q, p, scale=1.0, stream=None, mode="group"):
        """Routes a block of queries q [B][Tq][Hq][d], each on its own, over the tree as it
        stands (the block's own tokens are not in it).  Routing units are numbered
        ((b * Tq + t) * Hkv + KV head) * hr + head (hr = 1, or G per head)."""
        if mode not in ("group", "per_head"):
            raise ValueError(f"unknown routing mode {mode!r}")
        Tq = int(q.shape[1])
        m = zha.ZHA_ROUTE_GROUP if mode == "group" else zha.ZHA_ROUTE_PER_HEAD
        self.kept = zha.zha_route_multi(self.h, q, Tq, p, scale, m, stream)
        self.Tq = Tq
        self.RU = self.U * Tq * (1 if mode == "group" else self.G)
        return self.kept

    def attend_multi(self, q, K, V, scale=1.0, out=None, lse=None, stream=None):
        """Attention of the block routed by route_multi: query t also reads the block's rows
        N .. N + t of K and V (N: the tree's length).  out [B][Tq][Hq][d], lse [B][Tq][Hq]."""
        Tq = int(q.shape[1])
        if out is None:
            out = torch.empty((self.B, Tq, self.Hq, self.d), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((self.B, Tq, self.Hq), dtype=torch.float32, device=q.device)
        zha.zha_attend_multi(self.h, q, Tq, K, V, self.kept, scale, out, lse, stream)
        return out, lse

    def attend(self, q, K, V, scale=1.0, out=None, lse=None, stream=None):
        if out is None:
            out = torch.empty((self.B, self.Hq, self.d), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((self.B, self.Hq), dtype=torch.float32, device=q.device)
        zha.zha_attend(self.h, q, K, V, self.kept, scale, out, lse, stream)
        return out, lse

    def capacity(self, level: int) -> int:
        return zha.zha_tree_level_capacity(self.h, level)

    def level(self, level: int, device="cuda"):
        """(m [U][cap][R][d] in the tree dtype, b [U][cap][R] fp32) of one level; with fp8
        summaries m holds the decoded values (code times the row's power-of-two scale)."""
        cap = self.capacity(level)
        m = torch.empty((self.U, cap, self.R, self.d), dtype=self.dtype, device=device)
        b = torch.empty((self.U, cap, self.R), dtype=torch.float32, device=device)
        zha.zha_tree_copy_level(self.h, level, m, b)
        return m, b

    def scales(self, level: int, device="cuda"):
        """Scales of one level of a tree with low-precision summaries: fp8 [U][cap][R] (one
        per row), fp4 [U][cap][R][d/32] (one per block of 32 values), fp32."""
        shape = (self.U, self.capacity(level), self.R) + ((self.d // 32,) if self.summary == "fp4" else ())
        sc = torch.empty(shape, dtype=torch.float32, device=device)
        zha.zha_tree_copy_scales(self.h, level, sc)
        return sc

    def route_level(self, level: int, device="cuda"):
        """(frontier counts [RU], kept counts [RU], kept ids [RU][cap]) of the last route, per
        routing unit (RU = U * Tq, times G after a per-head route)."""
        cap = self.capacity(level)
        nf = torch.empty(self.RU, dtype=torch.int32, device=device)
        nk = torch.empty(self.RU, dtype=torch.int32, device=device)
        ids = torch.empty((self.RU, cap), dtype=torch.int32, device=device)
        zha.zha_route_copy_level(self.h, level, nf, nk, ids)
        return nf, nk, ids

    def timing(self, enable=True, kernels=None, levels=None):
        """Record per-launch durations: every launch, or only those of the given kernel
        codes (zha.ZHA_K_*) at the given levels (0 for launches without a level)."""
        km = 0 if not enable else (zha.ZHA_TIMING_ALL if kernels is None else sum(1 << k for k in kernels))
        lm = zha.ZHA_TIMING_ALL if levels is None else sum(1 << l for l in levels)
        zha.zha_timing_enable(self.h, km, lm)

    def timing_read(self):
        return zha.zha_timing_read(self.h)


def dense_decode(q, K, V, seq_lens, n_kv_heads, scale=1.0, workspace=None, out=None, lse=None, stream=None):
    B, Hq, d = q.shape
    T = K.shape[2]
    if workspace is None:
        nb = zha.zha_dense_workspace_bytes(B, Hq, n_kv_heads, d, T)
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    zha.zha_dense_decode(q, K, V, seq_lens, B, Hq, n_kv_heads, d, T, zdtype(q.dtype), scale, out, lse, workspace,
                         workspace.numel(), stream)
    return out, lse
