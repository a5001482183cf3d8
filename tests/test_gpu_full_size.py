"""Parity at the full sizes of the two largest workloads, in the launch shapes the
benchmark times (needs a gfx950 GPU; `slow`: minutes of host work in all).

deep_1m: N = 1048576, 32 query heads over 4 KV heads, d = 128, C = 4, L = 7, R = 16,
p = 0.95 -- every unit checked for two decode queries, and dense decode at 1M.

batch8_append_512k: 8 sequences of N = 524288 growing by one row per decode step for
1024 steps, C = 4, L = 6, R = 4; every step appends, then routes and attends at each
p in {0.7, 0.9, 0.99}.  At steps {0, 1, 2, 3, 4, 255, 511, 1023} the route of one p (one
test per p) is checked level by level against the oracle, and the attention over the
GPU's kept lists, for units of three different sequences of the 32-unit launch; after
the last step the appended tree equals a rebuild over the grown cache bit for bit.
The inputs of each workload are generated once per module (each unit from its own
stream, in parallel) and shared by its tests.
"""
import sys

import pytest
import torch

import zha_inputs as zi
from parity import Case, check_build, check_dense, full_check, route_attend
from test_gpu_parity import _valid_equal, selection_levels

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# --------------------------------------------------------------------------------- 1M context

@pytest.fixture(scope="module")
def deep_1m():
    cfg = zi.get_config("deep_1m")
    say("case deep_1m full: N=1048576, 32q/4kv, d=128, C=4 L=7 R=16 p=0.95 (inputs and tree)")
    case = Case(cfg, n_queries=2, host_f64=True)
    tree = case.tree()
    torch.cuda.synchronize()
    yield case, tree
    tree.close()


@pytest.mark.timeout(600)
def test_deep_1m_build_and_dense(deep_1m):
    case, tree = deep_1m
    say("case deep_1m full: build (12 sampled nodes per unit and level) and dense decode, every unit")
    say(" build", check_build(case, tree, sample=12))
    say(" dense worst |out err|", check_dense(case, 0))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", [0, 1])
def test_deep_1m_route_attend(deep_1m, t):
    case, tree = deep_1m
    say(f"case deep_1m full: route and attend of decode query {t}, every unit")
    r, a = full_check(case, tree, t, 0.95)
    say(f" t={t}", r, a)


# ------------------------------------------------------------------ batched decode with growth

C4_STEPS = (0, 1, 2, 3, 4, 255, 511, 1023)
C4_UNITS = {1, 14, 31}  # (sequence, KV head) = (0, 1), (3, 2), (7, 3)


@pytest.fixture(scope="module")
def batch8():
    cfg = zi.get_config("batch8_append_512k")
    say("case batch8_append_512k full: 8 x 524288 (+1024 rows), 32q/4kv, d=128, C=4 L=6 R=4 (inputs)")
    pairs = {(u // cfg.n_kv_heads, u % cfg.n_kv_heads) for u in C4_UNITS}
    case = Case(cfg, n_queries=cfg.append_steps, host_units=pairs, host_f64=True, with_appended=True)
    torch.cuda.synchronize()
    return case


def _decode_steps(case, p_check, rebuild):
    """Builds the tree over the first N rows, then runs the 1024 decode steps (append, then
    route + attend at every p), checking the route at p_check on the sampled steps."""
    cfg = case.cfg
    N, A, B = cfg.n_tokens, cfg.append_steps, cfg.batch
    case.lens = [N] * B
    tree = case.tree()
    for s in range(A):
        lens = [N + s + 1] * B
        tree.append(case.Kd, lens)
        case.lens = lens
        for p in cfg.p:
            if p == p_check and s in C4_STEPS:
                r, a = full_check(case, tree, s, p, units=C4_UNITS)
                say(f" step {s} p={p}: level 1 {r['levels'].get(1)}, ambiguous {r['ambiguous']}, {a}")
            else:
                route_attend(case, tree, s, p)
    tree.check()
    levels = selection_levels(tree, lambda: tree.route(case.qd[A - 1], p_check, 1.0))
    say(f" levels selected by the multi-workgroup path: {levels}")
    assert 1 in levels
    if rebuild:
        full = case.tree()
        torch.cuda.synchronize()
        _valid_equal(case, tree, full)
        say(f" appended tree bitwise equal to a rebuild over {case.lens[0]} tokens")
        full.close()
    tree.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("p_check,rebuild", [(0.7, True), (0.9, False), (0.99, False)])
def test_batch8_append_512k(batch8, p_check, rebuild):
    say(f"case batch8_append_512k full: 1024 decode steps, route parity at p={p_check} on units {sorted(C4_UNITS)}")
    _decode_steps(batch8, p_check, rebuild)
