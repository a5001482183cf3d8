"""HIP path against the fp64 oracle through the C ABI (needs a gfx950 GPU).

Each test prints the case it is about to run before touching the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import zha_inputs as zi
from hierarchical_tree_indexed_02_amd import zha
from parity import Case, check_attend, check_block, check_build, check_dense, check_route, full_check, route_attend

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name="deep_256k", **kw):
    return zi.get_config(name, **kw)


# --------------------------------------------------------------------------- tiny workload, everything

def test_tiny_deep_f32_every_query():
    cfg = zi.get_config("tiny_deep_f32")
    say("case tiny_deep_f32: N=4096 d=64 C=4 L=3 R=4 fp32, 8 queries")
    case = Case(cfg, n_queries=cfg.n_queries)
    tree = case.tree()
    torch.cuda.synchronize()
    say(" build", check_build(case, tree))
    for t in range(cfg.n_queries):
        r, a = full_check(case, tree, t, 0.95)
        say(f" t={t}", r, a)
    say(" dense", check_dense(case, 0))


# --------------------------------------------------------------------------- shape variants, ragged tails

VARIANTS = [
    # (label, config overrides, lengths)
    ("bf16 d128 C4 L3 R16 G8 B2", dict(batch=2, n_tokens=5000, chunk=4, levels=3, n_refs=16), [5000, 3333]),
    ("bf16 d64 C4 L2 R4 G4", dict(batch=1, n_tokens=2051, head_dim=64, n_q_heads=16, n_kv_heads=4, chunk=4, levels=2,
                                  n_refs=4), [2051]),
    ("f32 d128 C3 L3 R8 G2", dict(batch=1, n_tokens=1000, n_q_heads=8, n_kv_heads=4, chunk=3, levels=3, n_refs=8,
                                  dtype="f32"), [1000]),
    ("bf16 d128 C5 L2 R2 G16", dict(batch=1, n_tokens=777, n_q_heads=16, n_kv_heads=1, chunk=5, levels=2, n_refs=2),
     [777]),
    ("bf16 d64 C16 L2 R1 G1 B3", dict(batch=3, n_tokens=4109, head_dim=64, n_q_heads=2, n_kv_heads=2, chunk=16,
                                      levels=2, n_refs=1), [4109, 300, 17]),
    ("bf16 d128 wide C256 L1 R16", dict(batch=1, n_tokens=16484, chunk=256, levels=1, n_refs=16), [16484]),
    ("f32 d64 C4 L4 R16 G1", dict(batch=1, n_tokens=3000, head_dim=64, n_q_heads=1, n_kv_heads=1, chunk=4, levels=4,
                                  n_refs=16, dtype="f32", head_scale=False), [3000]),
    # levels of up to 8192 nodes are selected by one workgroup (two load batches in "mid flat");
    # larger levels take the multi-workgroup masses, the histogram cut and the look-back
    # compaction ("large frontier", "large flat")
    ("bf16 d64 C16 L1 R4 G4 mid flat", dict(batch=2, n_tokens=100000, head_dim=64, n_q_heads=8, n_kv_heads=2,
                                            chunk=16, levels=1, n_refs=4), [100000, 75001]),
    ("bf16 d128 C4 L2 R16 G8 large frontier", dict(batch=1, n_tokens=65539, n_q_heads=16, n_kv_heads=2, chunk=4,
                                                   levels=2, n_refs=16), [65539]),
    ("bf16 d64 C8 L1 R4 G4 large flat", dict(batch=2, n_tokens=200000, head_dim=64, n_q_heads=8, n_kv_heads=2,
                                             chunk=8, levels=1, n_refs=4), [200000, 150001]),
]


@pytest.mark.parametrize("label,kw,lens", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_variants(label, kw, lens):
    cfg = small(**kw, n_queries=4, needles_per_unit=4)
    say(f"case {label}: lens={lens}")
    case = Case(cfg, lens=lens, n_queries=2)
    tree = case.tree()
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=None if sum(lens) < 20000 else 256))
    for t in range(2):
        for p in (0.5, 0.9):
            r, a = full_check(case, tree, t, p)
            say(f" t={t} p={p}", r, a)
    if "flat" in label or "frontier" in label:  # level 1 of 6250 nodes: one workgroup; 16384, 25000: many
        assert selection_levels(tree, lambda: tree.route(case.qd[0], 0.9, 1.0)) == ([] if "mid" in label else [1])
    say(" dense", check_dense(case, 0))


# --------------------------------------------------------------------------- fp8 router summaries

FP8_VARIANTS = [v for v in VARIANTS if v[1].get("dtype", "bf16") == "bf16" and "mid flat" not in v[0]
                and "large flat" not in v[0]]


@pytest.mark.parametrize("label,kw,lens", FP8_VARIANTS, ids=[v[0] for v in FP8_VARIANTS])
def test_fp8_summaries(label, kw, lens):
    """Planes stored as e4m3 codes with a power-of-two row scale: storage checked against the
    oracle's means, routing teacher-forced on the decoded planes, attention on the kept set."""
    cfg = small(**kw, n_queries=4, needles_per_unit=4)
    say(f"case fp8 summaries {label}: lens={lens}")
    case = Case(cfg, lens=lens, n_queries=2)
    tree = case.tree(summary="fp8")
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=None if sum(lens) < 20000 else 256))
    for t in range(2):
        for p in (0.5, 0.95):
            r, a = full_check(case, tree, t, p)
            say(f" t={t} p={p}", r, a)


@pytest.mark.parametrize("summary", ["fp8", "fp4"])
def test_low_precision_per_head_routing(summary):
    """Per-head routes (union scoring of the eight heads of a KV head, union attention) over
    fp8 and fp4 planes, teacher-forced on the decoded planes like the group routes."""
    cfg = small(batch=2, n_tokens=5000, chunk=4, levels=3, n_refs=16, n_queries=4, needles_per_unit=4)
    lens = [5000, 3333]
    say(f"case per-head routes over {summary} planes: lens={lens} C=4 L=3 R=16 G=8")
    case = Case(cfg, lens=lens, n_queries=2)
    tree = case.tree(summary=summary, per_head_routes=True)
    for t, p in ((0, 0.5), (1, 0.95)):
        r, a = full_check(case, tree, t, p, mode="per_head")
        say(f" t={t} p={p}", r, a)


def _e4m3_nonnegative():
    """Every non-negative finite e4m3 value: zero, the subnormals f 2^-9 and the normals up to 448."""
    v = [f * 2.0 ** -9 for f in range(0, 8)] + [(1 + f / 8) * 2.0 ** (e - 7) for e in range(1, 16) for f in range(8)]
    return sorted(x for x in v if x <= 448.0)


def test_fp8_rounding_exact():
    """Leaves whose C keys are equal have m = that key exactly, so the stored codes can be
    compared with the oracle's rounding bit for bit: every midpoint between neighbouring e4m3
    values (ties go to the even mantissa, subnormals included), the bf16 neighbours of each
    midpoint, and rows whose largest value sits on either side of a scale boundary."""
    grid = _e4m3_nonnegative()
    mids = [0.5 * (a + b) for a, b in zip(grid, grid[1:])]
    vals = []
    for m in mids:
        lo = float(torch.tensor(m, dtype=torch.float64).to(torch.bfloat16).float())
        assert lo == m, "every e4m3 midpoint is a bf16 value"
        up = float(torch.nextafter(torch.tensor(m, dtype=torch.bfloat16), torch.tensor(1e9, dtype=torch.bfloat16)))
        dn = float(torch.nextafter(torch.tensor(m, dtype=torch.bfloat16), torch.tensor(-1e9, dtype=torch.bfloat16)))
        vals += [m, -m, up, -dn]
    d, C = 128, 4
    per_row = d - 1
    rows = []
    for i in range(0, len(vals), per_row):
        chunk = vals[i:i + per_row]
        chunk += [0.0] * (per_row - len(chunk))
        rows.append([448.0] + chunk)                      # largest value exactly 448: scale 2^0
    rows.append([450.0] + [v / 2 for v in vals[:per_row]])  # 450 needs scale 2^1
    rows.append([-0.875] + [v / 512 for v in vals[:per_row]])  # largest 0.875 = 448 * 2^-9
    keys = np.array(rows, dtype=np.float32)
    n_leaf = len(rows)
    N = n_leaf * C
    cfg = small(batch=1, n_tokens=N, n_q_heads=1, n_kv_heads=1, head_dim=d, chunk=C, levels=1, n_refs=4,
                n_queries=2, needles_per_unit=1)
    say(f"case fp8 rounding of exact midpoints: {n_leaf} leaves of {C} equal keys, d={d}")
    case = Case(cfg, lens=[N], n_queries=2)
    Kfull = np.repeat(keys, C, axis=0)
    case.Kd[0, 0, :N] = torch.from_numpy(Kfull).to(case.Kd.device, torch.bfloat16)
    assert torch.equal(case.Kd[0, 0, :N].float().cpu(), torch.from_numpy(Kfull)), "keys are bf16 values"
    tree = case.tree(summary="fp8")
    m_d, _ = tree.level(1)
    s_d = tree.scales(1)
    got_m = m_d[0, :n_leaf].double().cpu().numpy()            # [n_leaf][R][d]
    got_s = s_d[0, :n_leaf].double().cpu().numpy()            # [n_leaf][R]
    want_m, want_s = oracle.fp8_rows(np.repeat(keys[:, None, :].astype(np.float64), cfg.n_refs, axis=1))
    bad = np.argwhere(got_m != want_m)
    assert bad.size == 0, f"{len(bad)} stored values differ from the oracle's rounding, e.g. leaf/ref/k {bad[0].tolist()}: " \
                          f"gpu {got_m[tuple(bad[0])]!r} oracle {want_m[tuple(bad[0])]!r}"
    assert np.array_equal(got_s, want_s), "row scales differ"
    say(f" {got_m.size} stored values equal the oracle's rounding; scales {sorted(set(got_s.ravel().tolist()))}")


@pytest.mark.parametrize("label,kw,lens", FP8_VARIANTS, ids=[v[0] for v in FP8_VARIANTS])
def test_fp4_summaries(label, kw, lens):
    """Planes stored as e2m1 codes with a power-of-two scale per block of 32 values: storage
    checked against the oracle's means, routing teacher-forced on the decoded planes,
    attention on the kept set."""
    cfg = small(**kw, n_queries=4, needles_per_unit=4)
    say(f"case fp4 summaries {label}: lens={lens}")
    case = Case(cfg, lens=lens, n_queries=2)
    tree = case.tree(summary="fp4")
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=None if sum(lens) < 20000 else 256))
    for t in range(2):
        for p in (0.5, 0.95):
            r, a = full_check(case, tree, t, p)
            say(f" t={t} p={p}", r, a)


def test_fp4_rounding_exact():
    """Leaves whose C keys are equal have m = that key exactly, so the stored codes can be
    compared with the oracle's rounding bit for bit: every midpoint between neighbouring e2m1
    values (ties go to the even mantissa) and its bf16 neighbours, in blocks whose largest
    value sits on either side of a scale boundary."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = []
    for a_, b_ in zip(grid, grid[1:]):
        m = 0.5 * (a_ + b_)
        up = float(torch.nextafter(torch.tensor(m, dtype=torch.bfloat16), torch.tensor(1e9, dtype=torch.bfloat16)))
        dn = float(torch.nextafter(torch.tensor(m, dtype=torch.bfloat16), torch.tensor(-1e9, dtype=torch.bfloat16)))
        vals += [m, -m, up, -dn, dn, a_, -b_]
    vals = (vals * 2)[:31]
    d, C = 128, 4
    blocks = [[6.0] + vals,                                   # largest exactly 6: scale 2^0
              [12.0] + [2 * v for v in vals],                 # scale 2^1
              [6.0 * 2.0 ** -4] + [v / 16 for v in vals],     # largest 0.375 = 6 * 2^-4
              [-6.03125] + [v / 2 for v in vals]]             # just above 6: scale 2^1
    rows = [sum(blocks[k:] + blocks[:k], []) for k in range(4)]
    keys = np.array(rows, dtype=np.float32)
    assert keys.shape == (4, d)
    n_leaf = len(rows)
    N = n_leaf * C
    cfg = small(batch=1, n_tokens=N, n_q_heads=1, n_kv_heads=1, head_dim=d, chunk=C, levels=1, n_refs=4,
                n_queries=2, needles_per_unit=1)
    say(f"case fp4 rounding of exact midpoints: {n_leaf} leaves of {C} equal keys, d={d}")
    case = Case(cfg, lens=[N], n_queries=2)
    Kfull = np.repeat(keys, C, axis=0)
    case.Kd[0, 0, :N] = torch.from_numpy(Kfull).to(case.Kd.device, torch.bfloat16)
    assert torch.equal(case.Kd[0, 0, :N].float().cpu(), torch.from_numpy(Kfull)), "keys are bf16 values"
    tree = case.tree(summary="fp4")
    m_d, _ = tree.level(1)
    s_d = tree.scales(1)
    got_m = m_d[0, :n_leaf].double().cpu().numpy()            # [n_leaf][R][d]
    got_s = s_d[0, :n_leaf].double().cpu().numpy()            # [n_leaf][R][d/32]
    want_m, want_s = oracle.fp4_rows(np.repeat(keys[:, None, :].astype(np.float64), cfg.n_refs, axis=1))
    bad = np.argwhere(got_m != want_m)
    assert bad.size == 0, f"{len(bad)} stored values differ from the oracle's rounding, e.g. leaf/ref/k {bad[0].tolist()}: " \
                          f"gpu {got_m[tuple(bad[0])]!r} oracle {want_m[tuple(bad[0])]!r}"
    assert np.array_equal(got_s, want_s), "block scales differ"
    say(f" {got_m.size} stored values equal the oracle's rounding; scales {sorted(set(got_s.ravel().tolist()))}")


# --------------------------------------------------------------------------- per-query-head routing

PER_HEAD_VARIANTS = [
    ("per-head bf16 d128 C4 L3 R16 G8 B2", dict(batch=2, n_tokens=5000, chunk=4, levels=3, n_refs=16), [5000, 3333]),
    ("per-head bf16 d64 C4 L2 R4 G4", dict(batch=1, n_tokens=2051, head_dim=64, n_q_heads=16, n_kv_heads=4, chunk=4,
                                            levels=2, n_refs=4), [2051]),
    ("per-head f32 d128 C3 L3 R8 G2", dict(batch=1, n_tokens=1000, n_q_heads=8, n_kv_heads=4, chunk=3, levels=3,
                                           n_refs=8, dtype="f32"), [1000]),
    ("per-head bf16 d128 C4 L2 R16 G8 large frontier", dict(batch=1, n_tokens=65539, n_q_heads=16, n_kv_heads=2,
                                                            chunk=4, levels=2, n_refs=16), [65539]),
]


@pytest.mark.parametrize("label,kw,lens", PER_HEAD_VARIANTS, ids=[v[0] for v in PER_HEAD_VARIANTS])
def test_per_head_routing(label, kw, lens):
    """Every query head routed alone (its own frontier, softmax, cut and attention set),
    teacher-forced per (sequence, query head) against the oracle with that head's query."""
    cfg = small(**kw, n_queries=4, needles_per_unit=4)
    say(f"case {label}: lens={lens}")
    case = Case(cfg, lens=lens, n_queries=2)
    tree = case.tree(per_head_routes=True)
    for t in range(2):
        for p in (0.5, 0.9):
            r, a = full_check(case, tree, t, p, mode="per_head")
            say(f" t={t} p={p}", r, a)
    # group routes on the same tree are unchanged by the per-head ones
    out0, lse0 = route_attend(case, tree, 0, 0.9)
    _, nk0, ids0 = tree.route_level(1)
    route_attend(case, tree, 1, 0.9, mode="per_head")
    out1, lse1 = route_attend(case, tree, 0, 0.9)
    _, nk1, ids1 = tree.route_level(1)
    assert torch.equal(nk0, nk1) and torch.equal(ids0, ids1) and torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_per_head_equals_group_at_one_head():
    """With one query head per KV head the two modes are the same computation: kept sets and
    outputs are bit-identical."""
    cfg = small(batch=2, n_tokens=9000, n_q_heads=4, n_kv_heads=4, chunk=4, levels=4, n_refs=16, n_queries=2,
                needles_per_unit=4)
    say("case per-head == group at G = 1: B=2 N=9000 Hq=Hkv=4 C=4 L=4 R=16")
    case = Case(cfg, lens=[9000, 7001], n_queries=2)
    tree = case.tree(per_head_routes=True)
    for p in (0.5, 0.95):
        og, lg = route_attend(case, tree, 0, p)
        kg = [tree.route_level(l) for l in range(1, tree.L + 1)]
        oh, lh = route_attend(case, tree, 0, p, mode="per_head")
        kh = [tree.route_level(l) for l in range(1, tree.L + 1)]
        for (a1, b1, c1), (a2, b2, c2) in zip(kg, kh):
            assert torch.equal(a1, a2) and torch.equal(b1, b2) and torch.equal(c1, c2)
        assert torch.equal(og, oh) and torch.equal(lg, lh)


def test_per_head_needs_the_workspace():
    cfg = small(batch=1, n_tokens=1000, n_q_heads=8, n_kv_heads=2, chunk=4, levels=2, n_refs=4, n_queries=2,
                needles_per_unit=2)
    say("case per-head route on a tree without the per-head workspace")
    case = Case(cfg, lens=[1000], n_queries=2)
    tree = case.tree()
    with pytest.raises(zha.ZhaError):
        tree.route(case.qd[0], 0.9, mode="per_head")


# --------------------------------------------------------------------------- blocks of queries

def block_of(case: Case, Tq: int):
    """The first Tq decode queries of every sequence as one block: host [B][Tq][Hq][d] and device."""
    qb = np.ascontiguousarray(case.q[:Tq].transpose(1, 0, 2, 3))
    return qb, case.qd[:Tq].transpose(0, 1).contiguous()


MULTI_VARIANTS = [
    # lengths leave the block's rows inside the generated keys; 4990 % 4 = 2, so the tails of
    # the later queries cross a chunk boundary
    ("block bf16 d128 C4 L3 R16 G8 B2 T5", dict(batch=2, n_tokens=5000, chunk=4, levels=3, n_refs=16), [4990, 3333],
     5, "group", 5),
    ("block bf16 d128 C4 L3 R16 G8 B2 T5 per-head", dict(batch=2, n_tokens=5000, chunk=4, levels=3, n_refs=16),
     [4990, 3333], 5, "per_head", 5),
    ("block f32 d64 C3 L3 R4 G2 T7 of 9", dict(batch=1, n_tokens=1100, head_dim=64, n_q_heads=8, n_kv_heads=4,
                                               chunk=3, levels=3, n_refs=4, dtype="f32"), [1001], 7, "group", 9),
    ("block bf16 d128 C4 L2 R16 G8 T3 large frontier", dict(batch=1, n_tokens=65560, n_q_heads=16, n_kv_heads=2,
                                                            chunk=4, levels=2, n_refs=16), [65539], 3, "group", 3),
    ("block bf16 d128 C4 L3 R4 G4 B3 T4 short sequences", dict(batch=3, n_tokens=600, n_q_heads=16, chunk=4,
                                                                 levels=3, n_refs=4), [3, 1, 517], 4, "group", 4),
    ("block bf16 d64 C4 L3 R4 G1 T16", dict(batch=2, n_tokens=3000, head_dim=64, n_q_heads=2, n_kv_heads=2, chunk=4,
                                             levels=3, n_refs=4), [2950, 1234], 16, "group", 16),
    # d = 64 union attention staged in LDS: 40 columns (four tiles per group) and 24 (two)
    ("block bf16 d64 C4 L3 R8 G8 B2 T5", dict(batch=2, n_tokens=3000, head_dim=64, n_q_heads=16, n_kv_heads=2,
                                               chunk=4, levels=3, n_refs=8), [2990, 1500], 5, "group", 5),
    ("block bf16 d64 C4 L3 R8 G8 T3", dict(batch=1, n_tokens=2000, head_dim=64, n_q_heads=16, n_kv_heads=2, chunk=4,
                                            levels=3, n_refs=8), [1990], 3, "group", 3),
    # a sequence without a complete chunk beside a longer one, in union attention groups of 40
    # columns (three tiles): the short sequence's groups have empty kept-chunk lists
    ("block bf16 d128 C4 L3 R16 G8 B2 T5 empty list", dict(batch=2, n_tokens=3000, chunk=4, levels=3, n_refs=16),
     [3, 2990], 5, "group", 5),
    # f32 union scoring with four column tiles (40 columns); f32 attention groups of 16 columns
    ("block f32 d128 C4 L3 R16 G8 T5", dict(batch=1, n_tokens=2000, n_q_heads=16, n_kv_heads=2, chunk=4, levels=3,
                                            n_refs=16, dtype="f32"), [1990], 5, "group", 5),
]


@pytest.mark.parametrize("label,kw,lens,Tq,mode,maxq", MULTI_VARIANTS, ids=[v[0] for v in MULTI_VARIANTS])
def test_block_routing(label, kw, lens, Tq, mode, maxq):
    """A block of Tq queries per sequence, each routed alone over the tree of the N cached
    tokens and attending its kept chunks plus the block's rows up to its own position."""
    cfg = small(**kw, n_queries=max(Tq, 4), needles_per_unit=4)
    say(f"case {label}: lens={lens} Tq={Tq} mode={mode} max_queries={maxq}")
    case = Case(cfg, lens=lens, n_queries=Tq, max_tokens=cfg.n_tokens)
    tree = case.tree(per_head_routes=mode == "per_head", max_queries=maxq)
    qb, qbd = block_of(case, Tq)
    for p in (0.5, 0.9, 1.0):
        tree.route_multi(qbd, p, mode=mode)
        out, lse = tree.attend_multi(qbd, case.Kd, case.Vd)
        torch.cuda.synchronize()
        r, a = check_block(case, tree, qb, p, out, lse, mode=mode)
        say(f" p={p}", r, a)


def test_block_capacity_and_order():
    """A block needs a tree sized for it and its rows inside K/V; a block route is attended
    only by attend_multi of the same size, a single-query route only by attend; block routes
    leave later single-query routes unchanged."""
    cfg = small(batch=1, n_tokens=1000, n_q_heads=8, n_kv_heads=2, chunk=4, levels=2, n_refs=4, n_queries=4,
                needles_per_unit=2)
    say("case block routing errors: N=996 of max 1000, max_queries 4")
    case = Case(cfg, lens=[996], n_queries=4, max_tokens=1000)
    tree = case.tree(max_queries=4)
    out0, lse0 = route_attend(case, tree, 0, 0.9)
    qb4, qbd4 = block_of(case, 4)
    with pytest.raises(zha.ZhaError) as ei:
        tree.route_multi(torch.cat([qbd4, qbd4[:, :1]], 1).contiguous(), 0.9)
    assert ei.value.status == zha.ZHA_ERR_CAPACITY
    tree.route_multi(qbd4, 0.9)  # N + 4 = max_tokens: fits
    with pytest.raises(zha.ZhaError):
        tree.attend(case.qd[0], case.Kd, case.Vd)
    with pytest.raises(zha.ZhaError):
        tree.attend_multi(qbd4[:, :3].contiguous(), case.Kd, case.Vd)
    out, lse = tree.attend_multi(qbd4, case.Kd, case.Vd)
    torch.cuda.synchronize()
    say(" block of 4 at the capacity edge", *check_block(case, tree, qb4, 0.9, out, lse))
    out1, lse1 = route_attend(case, tree, 0, 0.9)
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
    with pytest.raises(zha.ZhaError):
        tree.attend_multi(qbd4, case.Kd, case.Vd)
    tree.append(case.Kd, [997])  # N + 4 > max_tokens now
    tree.route_multi(qbd4, 0.9)
    with pytest.raises(zha.ZhaError) as ei:
        tree.attend_multi(qbd4, case.Kd, case.Vd)
    assert ei.value.status == zha.ZHA_ERR_CAPACITY


def test_attend_needs_a_current_route():
    """A route's kept lists describe the cache it was taken on: after an append (or a
    rebuild) attention refuses them until the tree is routed again."""
    cfg = small(batch=1, n_tokens=1100, n_q_heads=8, n_kv_heads=2, chunk=4, levels=2, n_refs=4, n_queries=4,
                needles_per_unit=2, append_steps=8)
    say("case stale route: N=1090 of max 1108, append then attend")
    case = Case(cfg, lens=[1090], n_queries=4, max_tokens=1108)
    tree = case.tree(max_queries=2)
    route_attend(case, tree, 0, 0.9)
    tree.append(case.Kd, [1094])  # completes a chunk: the kept list no longer covers the cache
    with pytest.raises(zha.ZhaError) as ei:
        tree.attend(case.qd[0], case.Kd, case.Vd)
    assert ei.value.status == zha.ZHA_ERR_INVALID
    case.lens = [1094]
    r, a = full_check(case, tree, 1, 0.9)
    say(" routed again after the append:", r, a)
    qb, qbd = block_of(case, 2)
    tree.route_multi(qbd, 0.9)
    tree.build(case.Kd, case.refs_d, [1094])
    with pytest.raises(zha.ZhaError) as ei:
        tree.attend_multi(qbd, case.Kd, case.Vd)
    assert ei.value.status == zha.ZHA_ERR_INVALID
    tree.route_multi(qbd, 0.9)
    out, lse = tree.attend_multi(qbd, case.Kd, case.Vd)
    torch.cuda.synchronize()
    say(" block routed again after the rebuild:", *check_block(case, tree, qb, 0.9, out, lse))
    tree.check()


def selection_levels(tree, route):
    """Levels whose selection ran the multi-workgroup path (a mass kernel) in `route()`."""
    tree.timing(True)
    route()
    torch.cuda.synchronize()
    recs = tree.timing_read()
    tree.timing(False)
    return sorted({l for k, l, _ in recs if k == zha.ZHA_K_MASS})


# --------------------------------------------------------------------------- large-level selection paths

def test_large_level_cut_paths():
    """A 16384-node level takes the multi-workgroup selection; p from tiny to nearly 1 puts
    the cut at the heaviest node (a crossing slice of a few keys), inside the fine window
    (hundreds of keys, narrowed again in LDS) and below the window (every key's range)."""
    cfg = small(batch=1, n_tokens=65539, n_q_heads=16, n_kv_heads=2, chunk=4, levels=2, n_refs=16, n_queries=2,
                needles_per_unit=4)
    say("case large-level cut paths: N=65539 C=4 L=2 R=16 G=8, p in 1e-6 .. 0.999999")
    case = Case(cfg, n_queries=2)
    tree = case.tree()
    for p in (1e-6, 0.3, 0.9, 0.999999):
        r, a = full_check(case, tree, int(p < 0.5), p)
        say(f" p={p}", r, a)
    assert selection_levels(tree, lambda: tree.route(case.qd[0], 0.9, 1.0)) == [1]


def test_maximum_shapes():
    """The largest batch (64 sequences of ragged lengths), 16 query heads per KV head, 16
    references, and 12 levels of chunk 2."""
    cfg = small(batch=64, n_tokens=3000, n_q_heads=16, n_kv_heads=1, head_dim=64, chunk=2, levels=12, n_refs=16,
                n_queries=2, needles_per_unit=2)
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 3001, 64)]
    lens[0], lens[1] = 1, 3000
    say(f"case maximum shapes: B=64 lens {min(lens)}..{max(lens)}, G=16, C=2 L=12 R=16 d=64")
    case = Case(cfg, lens=lens, n_queries=2)
    tree = case.tree()
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=64))
    r, a = full_check(case, tree, 0, 0.9)
    say(" p=0.9", r, a)


def test_large_level_with_short_sequence():
    """A batch where one sequence has no leaf chunk while the other's level 1 takes the
    large-level path: the empty unit keeps nothing and attends its few tokens densely."""
    cfg = small(batch=3, n_tokens=65600, n_q_heads=8, n_kv_heads=2, chunk=4, levels=2, n_refs=16, n_queries=2,
                needles_per_unit=4)
    lens = [65539, 3, 1]
    say(f"case large level with short sequences: lens={lens} C=4 L=2 (16384-node level 1)")
    case = Case(cfg, lens=lens, n_queries=2)
    tree = case.tree()
    for p in (0.5, 0.95):
        r, a = full_check(case, tree, 0, p)
        _, nk, _ = tree.route_level(1)
        assert nk.cpu().tolist()[2:] == [0, 0, 0, 0]
        say(f" p={p}", r, a)


GRAPH_CASES = [
    ("bf16 d128 C4 L3 R16 G8 B2", dict(batch=2, n_tokens=5000, chunk=4, levels=3, n_refs=16)),
    ("bf16 d128 C4 L2 R16 G8 large level", dict(batch=1, n_tokens=65539, n_q_heads=16, n_kv_heads=2, chunk=4, levels=2,
                                                  n_refs=16)),
]


@pytest.mark.parametrize("label,kw", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_route_attend_graph_replays(label, kw):
    """Route + attend captured in a HIP graph (they allocate nothing, enqueue no memset and do
    not wait on the host): every replay, with another query's eager route and attention and a
    synchronisation before it, equals the eager result bit for bit -- small levels selected
    inside the next level's launch, and a 16384-node level with the mass, cut and look-back
    compaction (whose epochs advance on the device)."""
    cfg = small(**kw, n_queries=2, needles_per_unit=4)
    say(f"case graph replays, {label}")
    case = Case(cfg, n_queries=2)
    tree = case.tree()
    q0, q1 = case.qd[0], case.qd[1]

    def kept_lists():
        _, nk, ids = tree.route_level(1)
        nk = nk.cpu().tolist()
        ids = ids.cpu()
        return nk, [ids[u, :n].clone() for u, n in enumerate(nk)]

    tree.route(q0, 0.9, 1.0)
    o_ref, l_ref = tree.attend(q0, case.Kd, case.Vd, 1.0)
    torch.cuda.synchronize()
    o_ref, l_ref = o_ref.clone(), l_ref.clone()
    nk_ref, ids_ref = kept_lists()
    qs = q0.clone()
    out = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    side = torch.cuda.Stream()  # warm-up on a side stream before capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tree.route(qs, 0.9, 1.0)
        tree.attend(qs, case.Kd, case.Vd, 1.0, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tree.route(qs, 0.9, 1.0)
        tree.attend(qs, case.Kd, case.Vd, 1.0, out=out, lse=lse)
    torch.cuda.synchronize()
    for rep in range(4):
        tree.route(q1, 0.5, 1.0)  # eager work of another query between replays
        tree.attend(q1, case.Kd, case.Vd, 1.0)
        torch.cuda.synchronize()
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        nk, ids = kept_lists()
        assert nk == nk_ref, f"replay {rep}: kept counts {nk} != {nk_ref}"
        assert all(torch.equal(a, b) for a, b in zip(ids, ids_ref)), f"replay {rep}: kept ids differ"
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), f"replay {rep}: attention differs"
    tree.check()
    say(f" 4 replays bit-identical to the eager route and attention (kept {sum(nk_ref)} chunks)")


def test_small_level_p_sweep():
    """Every level of at most 1024 nodes (level 1 by its own selection launch, levels 2 and 3
    by the next level's scoring launch) across many p: the crossing slice lands on heavier and
    lighter candidates of every mass magnitude."""
    cfg = small(batch=2, n_tokens=4096, chunk=4, levels=3, n_refs=16, n_queries=4, needles_per_unit=4)
    say("case small-level p sweep: B=2 N=4096,3001 C=4 L=3 R=16 G=8, 40 values of p")
    case = Case(cfg, lens=[4096, 3001], n_queries=4)
    tree = case.tree()
    amb = 0
    for i, p in enumerate(np.linspace(0.02, 0.998, 40)):
        r, a = full_check(case, tree, i % 4, float(p))
        amb += r["ambiguous"]
    say(f" 40 routes, {amb} ambiguous nodes in all")


@pytest.mark.parametrize("N", [20000, 40000])
def test_equal_masses_large_level(N):
    """All keys zero: every node of a 5000-node level (one-workgroup selection) or a
    10000-node level (multi-workgroup selection) carries the same mass, so the crossing slice is
    one value held by every node (more than the candidate buffer) and the cut is split by
    position: exactly the first ceil(p n) ids are kept."""
    cfg = small(batch=1, n_tokens=N, n_q_heads=8, n_kv_heads=2, chunk=4, levels=1, n_refs=4, head_dim=64,
                n_queries=2, needles_per_unit=2)
    say(f"case equal masses: N={N} C=4 L=1 R=4, K = 0, p=0.33333")
    case = Case(cfg, n_queries=2)
    case.Kd.zero_()
    for key in case.K:
        case.K[key] = np.zeros_like(case.K[key])
    tree = case.tree()
    p = 0.33333
    r, a = full_check(case, tree, 0, p)
    nf, nk, ids = tree.route_level(1)
    n = N // 4
    assert selection_levels(tree, lambda: tree.route(case.qd[0], p, 1.0)) == ([1] if n > 8192 else [])
    k = int(np.ceil(p * n))
    assert nf.cpu().tolist() == [n] * case.Hkv
    assert nk.cpu().tolist() == [k] * case.Hkv, nk.cpu().tolist()
    assert torch.equal(ids[:, :k].cpu(), torch.arange(k, dtype=torch.int32).repeat(case.Hkv, 1))
    say(" ", r, a)


# --------------------------------------------------------------------------- edge cases

def test_short_sequences_no_tree():
    """N < C: no complete chunk, no tree; S = [0, N): attention equals dense."""
    cfg = small(batch=4, n_tokens=40, chunk=16, levels=2, n_refs=4, n_queries=2, needles_per_unit=2)
    lens = [1, 3, 15, 16]
    say(f"case short sequences lens={lens} C=16")
    case = Case(cfg, lens=lens)
    tree = case.tree()
    out, lse = route_attend(case, tree, 0, 0.9)
    r = check_route(case, tree, 0, 0.9)
    a = check_attend(case, tree, out, lse, 0)
    _, nk, _ = tree.route_level(1)
    assert nk.cpu().tolist()[:12] == [0] * 12  # batch entries 0..2 have no complete chunk
    say(" ", r, a)


def test_p_extremes():
    cfg = small(batch=1, n_tokens=4096 + 7, chunk=4, levels=3, n_refs=16, n_queries=2, needles_per_unit=4)
    say("case p extremes: N=4103 C=4 L=3 R=16")
    case = Case(cfg)
    tree = case.tree()
    # p = 1 keeps every node; the sparse output equals dense attention
    out, lse = route_attend(case, tree, 0, 1.0)
    for l in range(1, tree.L + 1):
        nf, nk, ids = tree.route_level(l)
        n_l = oracle.level_nodes(case.lens[0], tree.C, l)
        assert nk.cpu().tolist() == [n_l] * case.Hkv
        assert torch.equal(ids[:, :n_l].cpu(), torch.arange(n_l, dtype=torch.int32).repeat(case.Hkv, 1))
    a = check_attend(case, tree, out, lse, 0)
    assert abs(a["kappa"] - 1.0) < 1e-12
    check_dense(case, 0)
    # tiny p keeps one node per level: the heaviest
    r, a = full_check(case, tree, 1, 1e-6)
    for l, (nF, nK) in r["levels"].items():
        assert nK == case.Hkv, (l, nK)
    say(" ", r, a)


def test_determinism():
    """Two trees built and routed from the same inputs agree bit for bit."""
    cfg = small(batch=2, n_tokens=9000, chunk=4, levels=4, n_refs=16, n_queries=2, needles_per_unit=8)
    say("case determinism: B=2 N=9000 C=4 L=4 R=16")
    case = Case(cfg)
    tree = case.tree()
    o1, l1 = route_attend(case, tree, 0, 0.9)
    o1, l1 = o1.clone(), l1.clone()
    tree2 = case.tree()
    o2, l2 = route_attend(case, tree2, 0, 0.9)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for l in range(1, 5):
        m1, b1 = tree.level(l)
        m2, b2 = tree2.level(l)
        n_l = oracle.level_nodes(case.lens[0], tree.C, l)
        assert torch.equal(m1[:, :n_l].view(torch.int16), m2[:, :n_l].view(torch.int16))
        assert torch.equal(b1[:, :n_l], b2[:, :n_l])
        nf1, nk1, i1 = tree.route_level(l)
        nf2, nk2, i2 = tree2.route_level(l)
        assert torch.equal(nf1, nf2) and torch.equal(nk1, nk2)
        for u in range(case.B * case.Hkv):
            assert torch.equal(i1[u, :nk1[u]], i2[u, :nk2[u]])


# --------------------------------------------------------------------------- growth

def _valid_equal(case, t_inc, t_full):
    fp8 = t_inc.summary != "native"  # low-precision storage: scales too
    for l in range(1, t_inc.L + 1):
        m1, b1 = t_inc.level(l)
        m2, b2 = t_full.level(l)
        s1, s2 = (t_inc.scales(l), t_full.scales(l)) if fp8 else (None, None)
        for b in range(case.B):
            n_l = oracle.level_nodes(case.lens[b], t_inc.C, l)
            for g in range(case.Hkv):
                u = b * case.Hkv + g
                x1, x2 = m1[u, :n_l], m2[u, :n_l]
                if x1.dtype == torch.bfloat16:
                    x1, x2 = x1.view(torch.int16), x2.view(torch.int16)
                assert torch.equal(x1, x2), f"m level {l} unit {u}"
                assert torch.equal(b1[u, :n_l], b2[u, :n_l]), f"b level {l} unit {u}"
                if fp8:
                    assert torch.equal(s1[u, :n_l], s2[u, :n_l]), f"scale level {l} unit {u}"


@pytest.mark.parametrize("dtype,summary", [("bf16", "native"), ("f32", "native"), ("bf16", "fp8"), ("bf16", "fp4")])
def test_append_equals_rebuild(dtype, summary):
    cfg = small(batch=2, n_tokens=1200, chunk=4, levels=4, n_refs=8, n_q_heads=8, n_kv_heads=2, n_queries=2,
                needles_per_unit=4, append_steps=400, dtype=dtype)
    say(f"case append == rebuild ({dtype}, {summary} summaries): B=2 N=1200 +400 C=4 L=4 R=8")
    case = Case(cfg, lens=[1200, 1001], max_tokens=1700)
    rows = {(b, g): zi.append_rows(cfg, b, g) for b in range(2) for g in range(2)}
    tree = case.tree(summary=summary)
    lens = list(case.lens)
    schedule = [1] * 37 + [5, 64, 3, 200] + [1] * 20
    done = 0
    for k in schedule:
        for b in range(2):
            for g in range(2):
                Kr, Vr = rows[(b, g)]
                case.add_rows(b, g, lens[b], Kr[done:done + k], Vr[done:done + k])
        lens = [n + k for n in lens]
        tree.append(case.Kd, lens)
        done += k
    case.lens = lens
    full = case.tree(summary=summary)
    torch.cuda.synchronize()
    _valid_equal(case, tree, full)
    say(" bitwise equal after", len(schedule), "appends; lens", lens)
    say(" build", check_build(case, tree, sample=64))
    r, a = full_check(case, tree, 0, 0.9)
    say(" ", r, a)


# Shapes of the matrix-core build (bf16 keys, C = 4): references that fill only part of a
# lane group (R = 1, 2), both head dimensions, trees of one level and of five to seven (the
# upper-level kernel), fp8 and fp4 summaries, and lengths whose last 64-leaf workgroup is
# partial, exactly full, or the only one; appends cross leaf, level-2, level-3 and level-4
# boundaries.
C4_SHAPES = [
    ("d128 R1 L6", dict(n_refs=1, levels=6), [4100, 3072, 257], "native"),
    ("d64 R2 L5", dict(n_refs=2, levels=5, head_dim=64), [6001, 4160, 63], "native"),
    ("d128 R8 L1", dict(n_refs=8, levels=1), [1001, 6], "native"),
    ("d64 R16 L6 fp8", dict(n_refs=16, levels=6, head_dim=64), [5000], "fp8"),
    ("d128 R4 L7 fp4", dict(n_refs=4, levels=7), [20000, 16387], "fp4"),
]


@pytest.mark.parametrize("label,kw,lens,summary", C4_SHAPES, ids=[v[0] for v in C4_SHAPES])
def test_c4_build_shapes(label, kw, lens, summary):
    B = len(lens)
    cfg = small(batch=B, n_tokens=max(lens), chunk=4, n_q_heads=8, n_kv_heads=2, n_queries=2, needles_per_unit=4,
                append_steps=300, **kw)
    say(f"case C=4 build {label} ({summary} summaries): lens={lens}")
    case = Case(cfg, lens=lens, max_tokens=max(lens) + 300)
    tree = case.tree(summary=summary)
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=None if sum(lens) < 12000 else 128))
    rows = {(b, g): zi.append_rows(cfg, b, g) for b in range(B) for g in range(cfg.n_kv_heads)}
    cur = list(case.lens)
    done = 0
    for k in (1, 3, 4, 60, 1, 200, 31):
        for b in range(B):
            for g in range(cfg.n_kv_heads):
                Kr, Vr = rows[(b, g)]
                case.add_rows(b, g, cur[b], Kr[done:done + k], Vr[done:done + k])
        cur = [n + k for n in cur]
        tree.append(case.Kd, cur)
        done += k
    case.lens = cur
    full = case.tree(summary=summary)
    torch.cuda.synchronize()
    _valid_equal(case, tree, full)
    say(" appended tree bitwise equal to a rebuild; lens", cur)
    say(" build after appends", check_build(case, tree, sample=64))
    r, a = full_check(case, tree, 0, 0.9)
    say(" ", r, a)
    full.close()
    tree.close()


def test_batched_append_p_sweep():
    """Batched decode with growth, routing at several p per step (reduced sizes)."""
    cfg = small("batch8_append_512k", n_tokens=8192, append_steps=64, n_queries=64)
    say("case batched append: B=8 N=8192 +64 C=4 L=6 R=4, p in {0.7, 0.9, 0.99}")
    case = Case(cfg, n_queries=64, max_tokens=8192 + 64)
    rows = {(b, g): zi.append_rows(cfg, b, g) for b in range(cfg.batch) for g in range(cfg.n_kv_heads)}
    tree = case.tree()
    lens = list(case.lens)
    for step in range(64):
        for b in range(cfg.batch):
            for g in range(cfg.n_kv_heads):
                Kr, Vr = rows[(b, g)]
                case.add_rows(b, g, lens[b], Kr[step:step + 1], Vr[step:step + 1])
        lens = [n + 1 for n in lens]
        tree.append(case.Kd, lens)
        case.lens = lens
        for p in cfg.p:
            if step in (0, 1, 2, 3, 31, 63):
                r, a = full_check(case, tree, step, p, units={0, 5, 17, 31})
                say(f" step {step} p={p}", r["levels"].get(1), r["ambiguous"], a)
            else:
                route_attend(case, tree, step, p)
    full = case.tree()
    torch.cuda.synchronize()
    _valid_equal(case, tree, full)
    say(" bitwise equal to rebuild after 64 steps")


# --------------------------------------------------------------------------- full-size workloads

@pytest.mark.slow
def test_deep_256k_full():
    cfg = zi.get_config("deep_256k")
    say("case deep_256k full: N=262144, 32q/4kv, d=128, C=4 L=6 R=16 p=0.95")
    case = Case(cfg, n_queries=2)
    tree = case.tree()
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=24))
    for t in range(2):
        r, a = full_check(case, tree, t, 0.95)
        say(f" t={t}", r, a)
    say(" dense", check_dense(case, 0))


@pytest.mark.slow
def test_deep_256k_fp8_full():
    cfg = zi.get_config("deep_256k")
    say("case deep_256k full, fp8 summaries: N=262144, 32q/4kv, d=128, C=4 L=6 R=16 p=0.95")
    case = Case(cfg, n_queries=2)
    tree = case.tree(summary="fp8")
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=24))
    for t in range(2):
        r, a = full_check(case, tree, t, 0.95)
        say(f" t={t}", r, a)


@pytest.mark.slow
def test_deep_256k_fp4_full():
    cfg = zi.get_config("deep_256k")
    say("case deep_256k full, fp4 summaries: N=262144, 32q/4kv, d=128, C=4 L=6 R=16 p=0.95")
    case = Case(cfg, n_queries=2)
    tree = case.tree(summary="fp4")
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=24))
    for t in range(2):
        r, a = full_check(case, tree, t, 0.95)
        say(f" t={t}", r, a)


@pytest.mark.slow
def test_deep_256k_per_head_full():
    """Per-head routes at full size (the launch shapes the benchmark times): two KV heads'
    16 query heads checked against the oracle."""
    cfg = zi.get_config("deep_256k")
    say("case deep_256k full, per-head routes: N=262144, 32q/4kv, d=128, C=4 L=6 R=16 p=0.95, KV heads 0 and 3")
    case = Case(cfg, n_queries=1)
    tree = case.tree(per_head_routes=True)
    torch.cuda.synchronize()
    r, a = full_check(case, tree, 0, 0.95, units={0, 3}, mode="per_head")
    say(" t=0", r, a)


@pytest.mark.slow
def test_deep_256k_block_full():
    """A block of 8 queries over the first N - 8 tokens at full size (the benchmark's block
    leg): queries 0 and 7 of KV heads 0 and 3 checked against the oracle."""
    cfg = zi.get_config("deep_256k")
    N = cfg.n_tokens
    say(f"case deep_256k full, block of 8 queries after {N - 8} tokens: 32q/4kv, d=128, C=4 L=6 R=16 p=0.95")
    case = Case(cfg, lens=[N - 8], n_queries=8, max_tokens=N)
    tree = case.tree(max_queries=8)
    qb, qbd = block_of(case, 8)
    tree.route_multi(qbd, 0.95)
    out, lse = tree.attend_multi(qbd, case.Kd, case.Vd)
    torch.cuda.synchronize()
    units = {((0 * 8 + t) * case.Hkv + g) for t in (0, 7) for g in (0, 3)}
    r, a = check_block(case, tree, qb, 0.95, out, lse, units=units)
    say(" queries 0 and 7", r, a)


@pytest.mark.slow
def test_wide_256k_full():
    cfg = zi.get_config("wide_256k")
    say("case wide_256k full: N=262144, 32q/4kv, d=128, C=256 L=1 R=16 p=0.95")
    case = Case(cfg, n_queries=2)
    tree = case.tree()
    torch.cuda.synchronize()
    say(" build", check_build(case, tree, sample=48))
    for t in range(2):
        r, a = full_check(case, tree, t, 0.95)
        say(f" t={t}", r, a)

