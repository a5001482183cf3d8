"""Host logic of the benchmark's byte accounting: the distinct frontier nodes and attended
tokens that bench.union_counts derives from the kept views of a union route equal those of the
oracle's routes (the sets of the member units' frontiers and attend sets, joined per sequence and
KV head), on ragged lengths, per-head unions and query blocks."""
import numpy as np
import pytest
import torch

import bench
import oracle

C, L, R, d = 4, 3, 4, 16


class KeptViews:
    """Stands in for a routed tree: per-unit frontier counts and kept ids of given routes."""

    def __init__(self, fr, kp):
        self.fr, self.kp = fr, kp
        self.cap = max(1, max(len(k[l]) for k in kp for l in range(1, L + 1)))

    def route_level(self, l):
        nf = torch.tensor([len(f[l]) for f in self.fr], dtype=torch.int32)
        nk = torch.tensor([len(k[l]) for k in self.kp], dtype=torch.int32)
        ids = torch.zeros((len(self.kp), self.cap), dtype=torch.int32)
        for u, k in enumerate(self.kp):
            ids[u, :len(k[l])] = torch.from_numpy(k[l].astype(np.int32))
        return nf, nk, ids


@pytest.mark.parametrize("N", [0, 3, 37, 150, 257])
@pytest.mark.parametrize("hr,Tq", [(1, 1), (4, 1), (1, 3), (2, 2)])
def test_union_counts_match_oracle_routes(N, hr, Tq):
    rng = np.random.default_rng(1000 * N + 10 * hr + Tq)
    B, Hkv = 2, 2
    trees = {}
    for b in range(B):
        for g in range(Hkv):
            K = rng.standard_normal((N, d))
            trees[(b, g)] = oracle.tree_merge(K, rng.standard_normal((R, d)), C, L)
    fr, kp, want_fr, want_tok = [], [], {}, {}
    for u in range(B * Tq * Hkv * hr):
        b, g, t = u // (Tq * Hkv * hr), (u // hr) % Hkv, (u // (Hkv * hr)) % Tq
        F, K = oracle.route(trees[(b, g)], N, C, L, rng.standard_normal((2, d)), 0.7)
        fr.append(F)
        kp.append(K)
        for l in range(1, L + 1):
            want_fr.setdefault(l, set()).update((b, g, int(j)) for j in F[l])
        S = oracle.block_attend_set(N, C, K[1], t) if Tq > 1 else oracle.attend_set(N, C, K[1])
        want_tok.setdefault((b, g), set()).update(S.tolist())
    ufr, tok, fr_unit, _ = bench.union_counts(KeptViews(fr, kp), L, C, hr, Tq, Hkv, [N] * B, Tq > 1)
    assert ufr == {l: len(want_fr.get(l, ())) for l in range(1, L + 1)}
    assert tok == sum(len(v) for v in want_tok.values())
    assert fr_unit == {l: sum(len(f[l]) for f in fr) for l in range(1, L + 1)}


def test_bench_refuses_several_gpus():
    """The benchmark runs on one GPU: asked for more it exits with status 2 and says so."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
