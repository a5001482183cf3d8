"""zha_dense_decode_noalloc (dense decode with the library's fixed scratch array instead of a
caller workspace) against zha_dense_decode on the same inputs: two calls in a row, the
second smaller, each bit-identical to the workspace entry point (same kernels), and the
first also within the attention tolerance of the oracle.  Needs a gfx950 GPU."""
import sys

import numpy as np
import pytest
import torch

import oracle
import zha_inputs as zi
from hierarchical_tree_indexed_02_amd import zha
from hierarchical_tree_indexed_02_amd.runtime import dense_decode, zdtype

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(cfg, lens, T, dev):
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = zi.queries(cfg, n=1)[0]
    K = torch.zeros((cfg.batch, cfg.n_kv_heads, T, cfg.head_dim), dtype=dt, device=dev)
    V = torch.zeros_like(K)
    host = {}
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            Ku, Vu = zi.unit_kv(cfg, b, g)
            K[b, g, :cfg.n_tokens] = torch.from_numpy(Ku).to(dev, dt)
            V[b, g, :cfg.n_tokens] = torch.from_numpy(Vu).to(dev, dt)
            host[(b, g)] = (Ku[:lens[b]], Vu[:lens[b]])
    return q, torch.from_numpy(q).to(dev, dt), K, V, host


def test_dense_decode_noalloc_matches_workspace_entry_point():
    dev = torch.device("cuda:0")
    cases = [
        ("bf16 B=2 32q/4kv d=128 lens [5000, 3111]",
         zi.get_config("deep_256k", batch=2, n_tokens=5000, n_queries=1, needles_per_unit=4), [5000, 3111]),
        ("f32 B=1 8q/2kv d=64 lens [777] (smaller)",
         zi.get_config("deep_256k", batch=1, n_tokens=800, n_q_heads=8, n_kv_heads=2, head_dim=64, n_queries=1,
                       needles_per_unit=2, dtype="f32"), [777]),
    ]
    for i, (label, cfg, lens) in enumerate(cases):
        say(f"case dense decode without allocation, call {i + 1}: {label}")
        T = cfg.n_tokens
        qh, q, K, V, host = _inputs(cfg, lens, T, dev)
        B, Hq, Hkv, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        out_ws, lse_ws = dense_decode(q, K, V, lens, Hkv, 1.0)
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
        zha.zha_dense_decode_noalloc(q, K, V, lens, B, Hq, Hkv, d, T, zdtype(q.dtype), 1.0, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ws) and torch.equal(lse, lse_ws), "differs from zha_dense_decode"
        G = cfg.group
        worst = 0.0
        for b in range(B):
            for g in range(Hkv):
                Ku, Vu = host[(b, g)]
                o_o, l_o = oracle.attend(qh[b, g * G:(g + 1) * G].astype(np.float64), Ku, Vu, np.arange(lens[b]))
                eo = float(np.max(np.abs(out[b, g * G:(g + 1) * G].cpu().numpy() - o_o)))
                el = float(np.max(np.abs(lse[b, g * G:(g + 1) * G].cpu().numpy() - l_o)))
                assert eo <= 2e-3 and el <= 1e-3, f"unit {(b, g)}: out {eo:.3e} lse {el:.3e}"
                worst = max(worst, eo)
        say(f" bit-identical to the workspace entry point; worst |out - oracle| {worst:.2e}")
