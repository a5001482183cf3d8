"""Pins of the fp64 oracle: checks against what the pages and the mathematics fix.

Each pin_* function raises AssertionError when the oracle (as currently bound
in the `oracle` module) disagrees with something other than itself: a value
the pages state, a closed form, an invariant, a library routine (scipy's
logsumexp/softmax, transformers' nucleus filter, torch's attention) or brute
force on tiny inputs.  test_oracle_pins.py runs them on the real oracle;
test_oracle_mutants.py runs them on copies of the oracle with planted
mistakes and requires every mistake to be caught.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
from scipy.special import logsumexp, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(seed, N, d, R, G, kscale=1.0, qscale=3.0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((N, d)) * kscale
    V = rng.standard_normal((N, d))
    refs = rng.standard_normal((R, d)) / math.sqrt(d)
    q = rng.standard_normal((G, d)) / math.sqrt(d) * qscale
    return K, V, refs, q


def _node_range(N, C, l, j):
    Nc = (N // C) * C
    span = C ** l
    return j * span, min((j + 1) * span, Nc)


def _close(a, b, rel=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64); b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= rel, f"{what}: max rel err {err:.3e} > {rel:.1e}"


def _read_golden():
    rows = []
    with open(os.path.join(GOLDEN, "tree_geometry.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kv = line.split("|")[0].split()
            rows.append(dict(x.split("=") for x in kv))
    return rows


# --------------------------------------------------------------------- P4

def pin_geometry():
    """A top node covers C^L tokens (4096 at C=4, L=6); ceil(Nc/C^l) nodes per level."""
    rows = _read_golden()
    g = next(r for r in rows if "tokens_per_top_node" in r)
    C, L, span = int(g["chunk"]), int(g["levels"]), int(g["tokens_per_top_node"])
    assert oracle.level_nodes(span, C, L) == 1
    assert oracle.level_nodes(2 * span, C, L) == 2
    K, _, refs, _ = _rand(1, 2 * span, 4, 2, 1)
    t = oracle.tree_definition(K, refs, C, L)
    for j in range(2):
        for r in range(refs.shape[0]):
            want = logsumexp(K[j * span:(j + 1) * span] @ refs[r])
            _close(t.lse[L][j, r], want, 1e-12, "top node log-mass")
    for (N, C, L) in [(1000, 4, 3), (1003, 4, 3), (7, 4, 2), (3, 4, 2), (65536 + 5, 256, 1)]:
        Nc = (N // C) * C
        assert oracle.tree_tokens(N, C) == Nc
        for l in range(1, L + 1):
            assert oracle.level_nodes(N, C, l) == -(-Nc // C ** l), (N, C, l)


# --------------------------------------------------------------------- P2

def pin_tangent_planes():
    """Planes are tangent to A(q) = log sum exp(q.k): exact at q = r, below elsewhere,
    and their slope m equals the gradient of A at r (central differences)."""
    N, C, L, R, d = 300, 4, 3, 3, 8
    K, _, refs, _ = _rand(2, N, d, R, 1, kscale=1.5)
    t = oracle.tree_definition(K, refs, C, L)
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((24, d)) * 0.7
    for l in range(1, L + 1):
        for j in range(t.counts[l - 1]):
            t0, t1 = _node_range(N, C, l, j)
            Kn = K[t0:t1]
            for r in range(R):
                _close(t.lse[l][j, r], logsumexp(Kn @ refs[r]), 1e-12, "LSE_r")
                _close(t.b[l][j, r] + refs[r] @ t.m[l][j, r], logsumexp(Kn @ refs[r]), 1e-12, "T_r(r)")
                A = logsumexp(Kn @ Q.T, axis=0)
                T = t.b[l][j, r] + Q @ t.m[l][j, r]
                assert np.all(T <= A + 1e-12 * np.maximum(1.0, np.abs(A))), "plane above log-mass"
                eps = 1e-5
                grad = np.array([(logsumexp(Kn @ (refs[r] + eps * e)) - logsumexp(Kn @ (refs[r] - eps * e))) / (2 * eps)
                                 for e in np.eye(d)])
                assert np.max(np.abs(grad - t.m[l][j, r])) < 1e-6, "slope != gradient"


# --------------------------------------------------------------------- P3

def pin_merge_equals_definition():
    for (N, C, L) in [(4 * 16 * 3 + 7, 4, 3), (200, 3, 4), (1030, 256, 1), (4 ** 4, 4, 4)]:
        K, _, refs, _ = _rand(4 + N, N, 6, 3, 1)
        a = oracle.tree_definition(K, refs, C, L)
        b = oracle.tree_merge(K, refs, C, L)
        _close(a.m_all, b.m_all, 1e-11, "merge m")
        _close(a.b_all, b.b_all, 1e-11, "merge b")
        _close(a.lse_all, b.lse_all, 1e-11, "merge lse")


# --------------------------------------------------------------------- helpers for routing pins

def _w_direct(tree, l, F, q):
    """Per-node mass by direct formula: mean over heads of softmax over the frontier
    of max_r(b + q.m)."""
    s = np.max(tree.b[l][F][None, :, :] + np.einsum("gd,nrd->gnr", q, tree.m[l][F]), axis=2)  # [G][nF]
    return softmax(s, axis=1).mean(axis=0)


def _bruteforce_select(w, p):
    """Smallest subset with mass >= p * sum(w); among those the largest mass."""
    n = len(w)
    masks = np.array(list(itertools.product([0, 1], repeat=n)), dtype=np.float64)
    mass = masks @ w
    card = masks.sum(axis=1)
    ok = mass >= p * w.sum()
    cmin = card[ok].min()
    cand = np.where(ok & (card == cmin))[0]
    best = cand[np.argmax(mass[cand])]
    return np.nonzero(masks[best])[0]


# --------------------------------------------------------------------- P5

def pin_top_p_minimal():
    N, C, L, R, d, G = 1200, 4, 3, 4, 16, 3
    K, _, refs, q = _rand(5, N, d, R, G, kscale=1.3)
    t = oracle.tree_definition(K, refs, C, L)
    for p in (0.3, 0.7, 0.9, 0.99):
        F, Kp = oracle.route(t, N, C, L, q, p)
        for l in range(L, 0, -1):
            kept, w, order, csum = oracle.select(t.m[l], t.b[l], q, F[l], p)
            assert np.array_equal(kept, Kp[l])
            _close(w.sum(), 1.0, 1e-12, "sum of w")
            _close(w, _w_direct(t, l, F[l], q), 1e-12, "w")
            wk = w[np.isin(F[l], kept)]
            wn = w[~np.isin(F[l], kept)]
            W = w.sum()
            assert wk.sum() >= p * W * (1 - 1e-12), "kept mass < p"
            assert wk.sum() - wk.min() < p * W, "not minimal"
            if len(wn):
                assert wk.min() >= wn.max(), "kept set is not the heaviest nodes"
            assert np.all(np.diff(kept) > 0), "kept ids not ascending"
            if l > 1:
                assert np.array_equal(F[l - 1], np.array([k * C + c for k in kept for c in range(C)
                                                          if k * C + c < t.counts[l - 2]]))


# --------------------------------------------------------------------- P6

def pin_bruteforce_tiny():
    """N <= 256: each level's kept set equals the brute-force minimum-cardinality,
    maximum-mass subset; the output equals softmax attention over S by direct formula."""
    C, L, R, d, G = 4, 2, 2, 8, 2
    for seed, N, p in [(6, 64, 0.5), (7, 64, 0.8), (8, 62, 0.95), (9, 256 - 3, 0.7), (10, 64, 0.9)]:
        K, V, refs, q = _rand(seed, N, d, R, G, kscale=1.5, qscale=4.0)
        t = oracle.tree_definition(K, refs, C, L)
        F, Kp = oracle.route(t, N, C, L, q, p)
        front = np.arange(t.counts[L - 1])
        for l in range(L, 0, -1):
            if len(front) > 16:
                break
            assert np.array_equal(F[l], front)
            w = _w_direct(t, l, front, q)
            bf = front[_bruteforce_select(w, p)]
            assert np.array_equal(np.sort(bf), Kp[l]), (seed, l, bf, Kp[l])
            front = np.array([k * C + c for k in bf for c in range(C) if k * C + c < t.counts[l - 2]]) if l > 1 else None
        S = oracle.attend_set(N, C, Kp[1])
        out, lse = oracle.attend(q, K, V, S)
        logits = q @ K[S].T
        _close(lse, logsumexp(logits, axis=1), 1e-12, "lse")
        _close(out, softmax(logits, axis=1) @ V[S], 1e-12, "out")


# --------------------------------------------------------------------- P7 / P8

def _nucleus_library(logits, p):
    """Kept positions of transformers' nucleus (top-p) filter."""
    import torch
    from transformers.generation.logits_process import TopPLogitsWarper
    x = torch.tensor(np.asarray(logits, dtype=np.float64))[None]
    y = TopPLogitsWarper(top_p=float(p))(None, x)
    return np.nonzero(torch.isfinite(y[0]).numpy())[0]


def _margin_ok(a, p, tol=1e-9):
    pr = np.sort(softmax(a))[::-1]
    return np.min(np.abs(np.cumsum(pr) - p)) > tol


def pin_nucleus_single_tokens():
    """C = 1, L = 1: one token per leaf makes every plane exact, so routing is
    textbook nucleus selection over softmax(q.k); compared with a library filter."""
    d = 16
    for seed, N, p in [(11, 50, 0.9), (12, 200, 0.5), (13, 300, 0.95), (14, 33, 0.75)]:
        K, _, refs, q = _rand(seed, N, d, 1, 1, kscale=1.2, qscale=5.0)
        a = (q @ K.T)[0]
        if not _margin_ok(a, p):
            continue
        t = oracle.tree_definition(K, refs, 1, 1)
        F, Kp = oracle.route(t, N, 1, 1, q, p)
        assert np.array_equal(Kp[1], _nucleus_library(a, p)), seed


def pin_exact_reference():
    """A reference query equal to the query makes the score the exact node log-mass,
    so each level is nucleus selection over true node masses."""
    N, C, L, R, d = 1024, 4, 3, 3, 16
    for seed, p in [(15, 0.9), (16, 0.6), (17, 0.97)]:
        K, _, refs, q = _rand(seed, N, d, R, 1, kscale=1.4, qscale=4.0)
        refs[1] = q[0]
        t = oracle.tree_definition(K, refs, C, L)
        F, Kp = oracle.route(t, N, C, L, q, p)
        for l in range(L, 0, -1):
            a = np.array([logsumexp(K[slice(*_node_range(N, C, l, j))] @ q[0]) for j in F[l]])
            if not _margin_ok(a, p):
                break
            assert np.array_equal(Kp[l], F[l][_nucleus_library(a, p)]), (seed, l)


# --------------------------------------------------------------------- P9

def pin_translation_permutation():
    N, C, L, R, d = 4 * 4 * 4 * 3, 4, 3, 3, 8
    K, _, refs, _ = _rand(18, N, d, R, 1)
    t = oracle.tree_definition(K, refs, C, L)
    u = np.random.default_rng(19).standard_normal(d)
    tu = oracle.tree_definition(K + u, refs, C, L)
    _close(tu.b_all, t.b_all, 1e-10, "b under translation")
    _close(tu.m_all, t.m_all + u, 1e-10, "m under translation")
    perm = np.concatenate([c * C + np.random.default_rng(20 + c).permutation(C) for c in range(N // C)])
    tp = oracle.tree_definition(K[perm], refs, C, L)
    _close(tp.m_all, t.m_all, 1e-12, "m under permutation")
    _close(tp.b_all, t.b_all, 1e-12, "b under permutation")


# --------------------------------------------------------------------- P10

def pin_value_closed_forms():
    N, C, d, G = 333, 4, 8, 3
    K, V, _, q = _rand(21, N, d, 1, G)
    S = oracle.attend_set(N, C, np.array([0, 5, 17, 60], dtype=np.int32))
    c = np.linspace(-1, 1, d)
    out, _ = oracle.attend(q, K, np.tile(c, (N, 1)), S)
    _close(out, np.tile(c, (G, 1)), 1e-12, "constant values")
    Ke = np.tile(K[0], (N, 1))
    out, lse = oracle.attend(q, Ke, V, S)
    _close(out, np.tile(V[S].mean(axis=0), (G, 1)), 1e-12, "equal keys -> mean of V")
    _close(lse, q @ K[0] + math.log(len(S)), 1e-12, "equal keys lse")


# --------------------------------------------------------------------- P11

def pin_equal_masses():
    """All keys equal: equal masses, so each level keeps the ceil(p|F|) lowest ids."""
    C, L, d = 4, 3, 8
    N = C ** L * 5
    K = np.tile(np.random.default_rng(22).standard_normal(d), (N, 1))
    _, _, refs, q = _rand(23, N, d, 2, 2)
    t = oracle.tree_definition(K, refs, C, L)
    p = 0.55
    F, Kp = oracle.route(t, N, C, L, q, p)
    for l in range(L, 0, -1):
        n = len(F[l])
        assert abs(p * n - round(p * n)) > 1e-6
        assert np.array_equal(Kp[l], F[l][:math.ceil(p * n)]), l


# --------------------------------------------------------------------- P12

def pin_single_level_nesting():
    N, C, R, d, G = 2000, 4, 4, 16, 2
    K, _, refs, q = _rand(24, N, d, R, G, kscale=1.3)
    t = oracle.tree_definition(K, refs, C, 1)
    prev = None
    for p in np.linspace(0.05, 1.0, 20):
        _, Kp = oracle.route(t, N, C, 1, q, p)
        cur = set(Kp[1].tolist())
        if prev is not None:
            assert prev <= cur
        prev = cur
    assert prev == set(range(t.counts[0]))


# --------------------------------------------------------------------- P13

def pin_growth():
    """Growing the cache leaves every node that was complete before unchanged."""
    C, L, R, d = 4, 3, 2, 8
    N1, N2 = 4 * 16 * 2 + 9, 4 * 16 * 3 + 2
    K, _, refs, _ = _rand(25, N2, d, R, 1)
    a = oracle.tree_definition(K[:N1], refs, C, L)
    b = oracle.tree_definition(K, refs, C, L)
    Nc1 = (N1 // C) * C
    for l in range(1, L + 1):
        full = Nc1 // C ** l
        assert np.array_equal(a.m[l][:full], b.m[l][:full])
        assert np.array_equal(a.b[l][:full], b.b[l][:full])


# --------------------------------------------------------------------- P14 / P1

def pin_dense_two_ways():
    import torch
    N, d, G = 777, 16, 4
    K, V, _, q = _rand(26, N, d, 1, G, kscale=1.5)
    S = np.arange(N)
    out, lse = oracle.attend(q, K, V, S)
    for blk in (1, 7, 64, 1000):
        o2, l2 = oracle.attend_blockwise(q, K, V, S, blk)
        _close(o2, out, 1e-12, "blockwise out")
        _close(l2, lse, 1e-12, "blockwise lse")
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, None, :], torch.tensor(K)[None].expand(G, N, d), torch.tensor(V)[None].expand(G, N, d),
        scale=1.0)[:, 0, :].numpy()
    _close(out, ref, 1e-12, "torch attention")


def pin_p_one_is_dense():
    N, C, L, R, d, G = 4 ** 3 * 3 + 5, 4, 3, 3, 8, 2
    K, V, refs, q = _rand(27, N, d, R, G)
    t = oracle.tree_definition(K, refs, C, L)
    F, Kp = oracle.route(t, N, C, L, q, 1.0)
    for l in range(1, L + 1):
        assert np.array_equal(Kp[l], np.arange(t.counts[l - 1]))
    S = oracle.attend_set(N, C, Kp[1])
    assert np.array_equal(S, np.arange(N))
    o1, l1 = oracle.attend(q, K, V, S)
    o2, l2 = oracle.attend(q, K, V, np.arange(N))
    _close(o1, o2, 1e-12, "p=1 out"); _close(l1, l2, 1e-12, "p=1 lse")


# --------------------------------------------------------------------- P15

def pin_attend_set():
    for N, C, kept in [(103, 4, [1, 3, 7]), (103, 4, [0, 1, 24]), (3, 4, []), (1, 4, []), (1024, 256, [2]),
                       (17, 4, [])]:
        S = oracle.attend_set(N, C, np.array(kept, dtype=np.int32))
        Nc = (N // C) * C
        want = {0} | {k * C + c for k in kept for c in range(C)} | set(range(Nc, N))
        assert S.tolist() == sorted(want), (N, C, kept)


# ------------------------------------------------- blocks of queries

def pin_block_attend_set():
    """Query t of a block after N cached tokens reads token 0, its kept chunks, the partial
    chunk and the block's rows N .. N + t: built here position by position."""
    for N, C, kept, t in [(103, 4, [1, 3, 7], 0), (103, 4, [1, 3, 7], 5), (100, 4, [0, 24], 3), (0, 4, [], 2),
                          (3, 4, [], 0), (1024, 256, [2], 300), (17, 4, [], 9)]:
        S = oracle.block_attend_set(N, C, np.array(kept, dtype=np.int32), t)
        Nc = (N // C) * C
        want = [x for x in range(N + t + 1)
                if x == 0 or x >= Nc or (x // C) in kept]
        assert S.tolist() == want, (N, C, kept, t)


def pin_block_p_one_is_causal():
    """With p = 1 every query of a block reads every earlier position and itself: the
    block's outputs are causal attention (torch's attention with the causal mask)."""
    import torch
    for N, C, L, T in [(4 ** 3 + 6, 4, 3, 7), (4 ** 3, 4, 3, 5)]:
        d, R, G = 8, 2, 2
        K, V, refs, _ = _rand(41, N + T, d, R, G)
        rng = np.random.default_rng(42)
        Q = rng.standard_normal((T, G, d)) / math.sqrt(d) * 3.0
        tree = oracle.tree_definition(K[:N], refs, C, L)
        mask = np.arange(N + T)[None, :] <= (N + np.arange(T))[:, None]          # [T][N+T]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(Q).transpose(0, 1), torch.tensor(K)[None].expand(G, N + T, d),
            torch.tensor(V)[None].expand(G, N + T, d), attn_mask=torch.tensor(mask)[None], scale=1.0)
        for t in range(T):
            _, Kp = oracle.route(tree, N, C, L, Q[t], 1.0)
            S = oracle.block_attend_set(N, C, Kp[1], t)
            assert np.array_equal(S, np.arange(N + t + 1)), (N, t)
            o, _ = oracle.attend(Q[t], K, V, S)
            _close(o, ref[:, t, :].numpy(), 1e-12, f"block query {t} at p=1")


def pin_block_first_query_is_decode():
    """Query 0 of a block after N tokens is the decode query of a cache of N + 1 tokens
    when token N does not complete a chunk: the tree is the same (it holds complete chunks
    only), so are the route and the attention set."""
    N, C, L, d, R, G, p = 4 ** 3 * 2 + 5, 4, 3, 8, 3, 2, 0.8
    assert (N + 1) % C != 0
    K, V, refs, q = _rand(43, N + 1, d, R, G)
    t_blk = oracle.tree_definition(K[:N], refs, C, L)
    t_dec = oracle.tree_definition(K[:N + 1], refs, C, L)
    _, Kb = oracle.route(t_blk, N, C, L, q, p)
    _, Kd = oracle.route(t_dec, N + 1, C, L, q, p)
    for l in range(1, L + 1):
        assert np.array_equal(Kb[l], Kd[l]), l
    Sb = oracle.block_attend_set(N, C, Kb[1], 0)
    Sd = oracle.attend_set(N + 1, C, Kd[1])
    assert np.array_equal(Sb, Sd)
    assert Sb[-1] == N


# ------------------------------------------------------- fp8 summaries

def _e4m3_grid():
    """Every finite OCP e4m3 value by its code (sign, 4-bit exponent with bias 7,
    3-bit mantissa; exponent field 0 is subnormal; code 0x7F / 0xFF is not a number)."""
    vals = {}
    for c in range(256):
        sgn, e, f = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and f == 7:
            continue
        v = f * 2.0 ** -9 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7)
        vals[c] = -v if sgn else v
    return vals


def _bruteforce_e4m3(x, grid):
    """Nearest grid value by enumeration; on a tie the code with the even mantissa bit."""
    best = None
    for c, v in grid.items():
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (d, c, v)
    return best[2]


def pin_fp8_quantizer():
    """The oracle's e4m3 rounding equals enumeration of the format's 254 finite values
    (nearest, ties to even mantissa) on grid points, midpoints, just off midpoints and
    random values over the whole range, subnormals included; 448 is the largest value."""
    grid = _e4m3_grid()
    assert max(grid.values()) == 448.0 and min(v for v in grid.values() if v > 0) == 2.0 ** -9
    pos = sorted(v for v in grid.values() if v >= 0)
    xs = []
    for a, b in zip(pos, pos[1:]):
        mid = 0.5 * (a + b)
        xs += [a, mid, mid * (1 + 1e-9), mid * (1 - 1e-9), -mid, -a]
    rng = np.random.default_rng(5)
    xs += list(rng.uniform(-448, 448, 300)) + list(rng.uniform(-1, 1, 300) * 2.0 ** rng.integers(-12, 9, 300))
    for x in xs:
        got = oracle.e4m3_round(x)
        want = _bruteforce_e4m3(x, grid)
        assert got == want or (got == 0 and want == 0), f"e4m3({x!r}) = {got!r}, nearest is {want!r}"


def pin_fp8_rows():
    """Row storage: the scale is the smallest power of two that brings the row's largest
    magnitude within 448 (checked against the neighbouring exponent), every stored value is
    a grid value times the scale, and the error is within half a grid step."""
    grid = set(abs(v) for v in _e4m3_grid().values())
    rng = np.random.default_rng(6)
    m = rng.standard_normal((40, 32)) * 10.0 ** rng.uniform(-4, 3, (40, 1))
    m[3] = 0.0
    m[5, :] = 448.0 * 2.0 ** -3          # an exact power-of-two boundary
    mq, sc = oracle.fp8_rows(m)
    for i in range(m.shape[0]):
        amax = np.max(np.abs(m[i]))
        s = math.log2(sc[i])
        assert s == int(s), "scale is a power of two"
        if amax == 0:
            assert np.all(mq[i] == 0) and sc[i] == 1.0
            continue
        assert amax / sc[i] <= 448.0 and amax / (sc[i] / 2) > 448.0, f"row {i}: scale not minimal"
        for v, x in zip(mq[i], m[i]):
            c = abs(v) / sc[i]
            assert c in grid, f"row {i}: {v} is not a grid value times the scale"
            a = abs(x) / sc[i]
            half = 2.0 ** -10 if a < 2.0 ** -6 else 2.0 ** (math.floor(math.log2(a)) - 4)
            assert abs(v - x) / sc[i] <= half * (1 + 1e-12), f"row {i}: error beyond half a step"
    # planes from fp8 means stay exact at q = r (b is formed from the stored mean)
    K, _, refs, _ = _rand(7, 40, 16, 4, 1)
    t = oracle.tree_definition(K, refs, 4, 2)
    for l in (1, 2):
        mq, b, _ = oracle.fp8_planes(t.m[l], t.lse[l], refs)
        at_r = b + np.einsum("nrd,rd->nr", mq, refs)
        _close(at_r, t.lse[l], 1e-12, f"fp8 plane at q = r, level {l}")


def _e2m1_grid():
    """Every OCP e2m1 value by its code (sign, 2-bit exponent with bias 1, 1 mantissa bit;
    exponent field 0 is subnormal)."""
    vals = {}
    for c in range(16):
        sgn, e, f = c >> 3, (c >> 1) & 3, c & 1
        v = f * 0.5 if e == 0 else (1 + f / 2) * 2.0 ** (e - 1)
        vals[c] = -v if sgn else v
    return vals


def pin_fp4_quantizer():
    """The oracle's e2m1 rounding equals enumeration of the format's 16 codes (nearest, ties
    to the even mantissa) on grid points, midpoints, just off midpoints and random values;
    the grid is 0, 0.5, 1, 1.5, 2, 3, 4, 6."""
    grid = _e2m1_grid()
    pos = sorted(set(v for v in grid.values() if v >= 0))
    assert pos == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    xs = []
    for a, b in zip(pos, pos[1:]):
        mid = 0.5 * (a + b)
        xs += [a, mid, mid * (1 + 1e-9), mid * (1 - 1e-9), b]
    rng = np.random.default_rng(8)
    xs += list(rng.uniform(-6, 6, 3000))
    for x in xs + [-v for v in xs]:
        best = None
        for c, v in grid.items():
            d = abs(v - x)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
                best = (d, c, v)
        got = oracle.e2m1_round(x)
        assert abs(got) == abs(best[2]), (x, got, best)


def pin_fp4_blocks():
    """Block storage: each block of 32 values has the smallest power-of-two scale bringing its
    largest magnitude within 6 (checked against the neighbouring exponent), every stored
    value is a grid value times its block's scale with error within half a grid step, and
    blocks do not share scales; fp4 planes stay exact at q = r."""
    grid = set(abs(v) for v in _e2m1_grid().values())
    rng = np.random.default_rng(9)
    m = rng.standard_normal((24, 128)) * 10.0 ** rng.uniform(-4, 3, (24, 1))
    m[2] = 0.0
    m[4, :32] = 6.0 * 2.0 ** -5            # an exact power-of-two boundary in one block
    m[6, 32:64] *= 1e3                     # one loud block beside quiet ones
    mq, sc = oracle.fp4_rows(m)
    assert sc.shape == (24, 4)
    for i in range(m.shape[0]):
        for blk in range(4):
            xb, qb, s = m[i, 32 * blk:32 * blk + 32], mq[i, 32 * blk:32 * blk + 32], sc[i, blk]
            amax = np.max(np.abs(xb))
            assert math.log2(s) == int(math.log2(s)), "scale is a power of two"
            if amax == 0:
                assert np.all(qb == 0) and s == 1.0
                continue
            assert amax / s <= 6.0 and amax / (s / 2) > 6.0, f"row {i} block {blk}: scale not minimal"
            for v, x in zip(qb, xb):
                assert abs(v) / s in grid, f"row {i} block {blk}: {v} is not a grid value times the scale"
                a = abs(x) / s
                half = 0.25 if a < 2.0 else (0.5 if a < 4.0 else 1.0)
                assert abs(v - x) / s <= half * (1 + 1e-12), f"row {i} block {blk}: error beyond half a step"
    assert sc[6, 1] > 100 * sc[6, 0], "each block has its own scale"
    K, _, refs, _ = _rand(10, 40, 64, 4, 1)
    t = oracle.tree_definition(K, refs, 4, 2)
    for l in (1, 2):
        mq, b, _ = oracle.fp4_planes(t.m[l], t.lse[l], refs)
        at_r = b + np.einsum("nrd,rd->nr", mq, refs)
        _close(at_r, t.lse[l], 1e-12, f"fp4 plane at q = r, level {l}")


ALL_PINS = [
    pin_geometry, pin_tangent_planes, pin_merge_equals_definition, pin_top_p_minimal,
    pin_bruteforce_tiny, pin_nucleus_single_tokens, pin_exact_reference, pin_translation_permutation,
    pin_value_closed_forms, pin_equal_masses, pin_single_level_nesting, pin_growth,
    pin_dense_two_ways, pin_p_one_is_dense, pin_attend_set, pin_fp8_quantizer, pin_fp8_rows,
    pin_block_attend_set, pin_block_p_one_is_causal, pin_block_first_query_is_decode,
    pin_fp4_quantizer, pin_fp4_blocks,
]
