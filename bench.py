"""Decode-step benchmark of the ZHA path on one MI355X.

One step = one decode step of one attention layer: route the B x Hq queries
through that layer's tree (every level) and attend over the kept chunks plus
sink and tail.  For a workload with decode-time growth (batch8_append_512k) a
step first appends one K/V row per sequence (zha_append), then routes and
attends once for each p of the workload's sweep; its step time is append +
route + attend at the first p, and `p_sweep` gives every p.  Inputs are
resident in HBM before timing; steps cycle through `--layers` replicas of
(K, V, tree) so every step reads its layer cold, and through `--queries`
different decode queries.

The headline workload (--config, default deep_256k) is measured with every
extra leg (fp8 and fp4 summaries, per-head routes, a block of queries, dense
decode on the same inputs, the CPU oracle); the other workloads of the metric
(wide_256k, deep_1m, batch8_append_512k) follow as sub-records under
`workloads`, each with its own step time, dense time and roofline.  Prints one
JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config deep_256k]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "ZHA decode µs/step/layer at 256K & 1M ctx; achieved HBM GB/s vs peak"
SUB_WORKLOADS = ("wide_256k", "deep_1m", "batch8_append_512k")
# layer replicas per workload: enough that a step never finds its layer in the 256 MB
# last-level cache (one layer of the 1M and batched workloads is several GB)
SUB_LAYERS = {"wide_256k": 4, "deep_1m": 2, "batch8_append_512k": 2}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="deep_256k")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--queries", type=int, default=8)
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--cpu-queries", type=int, default=64)
    ap.add_argument("--summary", choices=["native", "fp8", "fp4"], default="native",
                    help="storage of the planes' m for the headline measurement")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the extra passes with fp8 and fp4 summaries (reported beside the headline)")
    ap.add_argument("--block", type=int, default=8,
                    help="also route and attend blocks of this many queries per sequence (0: skip)")
    ap.add_argument("--no-per-head", action="store_true",
                    help="skip the extra pass that routes every query head alone (reported beside the headline)")
    ap.add_argument("--workloads", default=",".join(SUB_WORKLOADS),
                    help="comma-separated workloads measured after the headline as sub-records ('' for none)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip timing the headline inputs under other tree geometries (C, L, R) and p against the "
                         "step model")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


SCORE_END = b"// ------------------------------------------------------------------------ shared selection"


def score_kernel_sha() -> str:
    """First 16 hex digits of the SHA-256 of the scoring kernel's source: zha_route.hip up to
    the shared-selection section (the kernel and every helper it uses), then zha_internal.h."""
    csrc = os.path.join(ROOT, "hierarchical_tree_indexed_02_amd", "csrc")
    with open(os.path.join(csrc, "zha_route.hip"), "rb") as f:
        route = f.read()
    with open(os.path.join(csrc, "zha_internal.h"), "rb") as f:
        internal = f.read()
    end = route.find(SCORE_END)
    return hashlib.sha256(route[:end if end >= 0 else len(route)] + internal).hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM traffic per launch of the dominant kernel from the committed counter summary,
    or None when there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"score_level1_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path, encoding="utf-8").read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", txt)
    m_tr = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_tr or m_sha.group(1) != score_kernel_sha():
        return None
    return float(m_tr.group(1))


def cpu_model() -> str:
    """The host CPU's model name (lscpu's "Model name" line, read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q)) if len(xs) else None


# Tree geometries (chunk C, levels L, references R, p) over the same 256K-token inputs: every R
# and p of the pages' sweep on the deep C = 4, L = 6 tree, and trees of other C and L (C^L =
# 4096 tokens per top node, 1024 for C = 4, L = 5, the flat C = 256 tree) at R = 16, p = 0.95.
SWEEP = [(4, 6, R, p) for R in (16, 4, 2, 1) for p in (0.95, 0.7, 0.9, 0.99)] + \
    [(8, 4, 16, 0.95), (16, 3, 16, 0.95), (64, 2, 16, 0.95), (4, 5, 16, 0.95), (256, 1, 16, 0.95)]


def level_caps(N, C, L):
    """Nodes per unit at each level 1..L of a tree over N tokens."""
    Nc = (N // C) * C
    return [-(-Nc // C ** l) for l in range(1, L + 1)]


def level_kind(l, cap):
    """How the route selects a level: inside the next level's scoring launch (fused), in a
    one-workgroup launch (wave: level 1 of <= 1024 nodes; small: <= 8192), or with the
    many-workgroup mass and compaction launches (large)."""
    if cap > 8192:
        return "large"
    if cap <= 1024:
        return "fused" if l > 1 else "wave"
    return "small"


def launches(caps):
    """Launches of one group route + attend: a scoring launch per level, the selection launches
    of each level by kind, attention and merge."""
    n = len(caps) + 2
    for l in range(1, len(caps) + 1):
        n += {"fused": 0, "wave": 1, "small": 1, "large": 3}[level_kind(l, caps[l - 1])]
    return n


def model_constants(res, caps, bw):
    """Constants of the step model, measured at one geometry (res: its measure() record with
    the per-launch times of the stage-breakdown pass; bw: bytes per microsecond of dense
    decode on the same GPU and inputs) -- not fitted:
      delta     how much an event-timed launch overstates its share of the step: (sum of the
                launch times - the step time) / launches;
      t_wave    the worker-wave cost of a scoring launch, paid on top of streaming its bytes:
                the top level's launch (every workgroup one super-tile) less its bytes' time;
      c_fused   selection of a small level inside the next level's scoring launch: the time
                those launches take beyond their own scoring;
      c_small   the one-workgroup selection launch; c_large: selection, mass and compaction of a
                large level;
      c_attend  attention and merge beyond streaming the attended bytes."""
    k = {n: v["avg_us"] for n, v in res["kernels"].items()}
    L = len(caps)
    Bl = res["route_bytes_l"]
    delta = (sum(k.values()) - res["ms_step"] * 1e3) / launches(caps)
    t_wave = k[f"score_l{L}"] - delta - Bl[L] / bw
    fused = [l for l in range(1, L) if level_kind(l + 1, caps[l]) == "fused"]
    c_fused = (sum(k[f"score_l{l}"] - delta - (t_wave + Bl[l] / bw) for l in fused) / len(fused)) if fused else 0.0
    small = [l for l in range(1, L + 1) if level_kind(l, caps[l - 1]) == "small"]
    large = [l for l in range(1, L + 1) if level_kind(l, caps[l - 1]) == "large"]
    c_small = sum(k.get(f"select_l{l}", 0.0) - delta for l in small) / len(small) if small else 0.0
    c_large = (sum(k.get(f"mass_l{l}", 0.0) + k.get(f"select_l{l}", 0.0) + k.get(f"compact_l{l}", 0.0) - 3 * delta
                   for l in large) / len(large)) if large else 0.0
    c_attend = k.get("attend", 0.0) + k.get("merge", 0.0) - 2 * delta - res["attend_bytes"] / bw
    return dict(bw_gbs=round(bw * 1e-3, 1), delta_us=round(delta, 2), t_wave_us=round(t_wave, 2),
                c_fused_us=round(c_fused, 2), c_small_us=round(c_small, 2), c_large_us=round(c_large, 2),
                c_attend_us=round(c_attend, 2))


def model_step(row, m):
    """Step time of one geometry from the four segments of the pages' model: build (none in a
    decode step without growth), per-level routing (each level's scoring launch streams its
    plane bytes at the dense bandwidth and pays one worker wave on top), node scan (each
    level's selection, by kind) and attention (the attended K/V bytes at the dense bandwidth
    plus its fixed time).  Returns the total and the segments in microseconds."""
    bw = m["bw_gbs"] * 1e3  # bytes per microsecond
    caps = row["caps"]
    route = sum(m["t_wave_us"] + b / bw for b in row["route_bytes_l"].values())
    scan = 0.0
    for l in range(1, len(caps) + 1):
        kind = level_kind(l, caps[l - 1])
        scan += {"fused": m["c_fused_us"], "wave": m["t_wave_us"] + m["c_fused_us"], "small": m["c_small_us"],
                 "large": m["c_large_us"]}[kind]
    attend = row["attend_bytes"] / bw + m["c_attend_us"]
    return route + scan + attend, dict(route=round(route, 1), scan=round(scan, 1), attend=round(attend, 1))


def geometry_sweep(measure, cfg, zi, torch, np, dev, N, B, Hkv, d, es, log):
    """Times route + attend under each geometry of SWEEP on the workload's inputs; returns one
    record per geometry (the step model's prediction is added once dense decode is timed)."""
    rows = []
    for C, L, R, p in SWEEP:
        if C ** L > N:
            continue
        g = zi.get_config(cfg.name, chunk=C, levels=L, n_refs=R)
        refs = torch.from_numpy(zi.refs(g)).to(dev)
        log(f"-- geometry C={C} L={L} R={R} p={p}")
        r = measure("native", "group", C=C, L=L, R=R, refs=refs, p=p)
        caps = level_caps(N, C, L)
        rows.append(dict(C=C, L=L, R=R, p=p, us_per_step=round(r["ms_step"] * 1e3, 2),
                         median_us=round(r["median_us"], 2), step_bytes=round(r["step_bytes"]),
                         route_bytes_l={str(l): round(v) for l, v in r["route_bytes_l"].items()},
                         attend_bytes=round(r["attend_bytes"]), kappa=round(r["kappa"], 4), caps=caps,
                         levels_by_kind={kd: sum(1 for l in range(1, L + 1) if level_kind(l, caps[l - 1]) == kd)
                                         for kd in ("fused", "wave", "small", "large")},
                         kernels={k: round(v["avg_us"], 2) for k, v in r["kernels"].items()},
                         tree_bytes=r["tree_bytes"]))
    return rows


def sweep_model(rows, consts, log):
    """Adds the step model's prediction to every geometry; returns the summary record."""
    worst = 0.0
    for x in rows:
        pred, segs = model_step(x, consts)
        x["model_us"] = round(pred, 1)
        x["model_segments_us"] = segs
        x["model_err"] = round(pred / x["us_per_step"] - 1.0, 4)
        worst = max(worst, abs(x["model_err"]))
        log(f"  C={x['C']:3d} L={x['L']} R={x['R']:2d} p={x['p']}: {x['us_per_step']:8.1f} us, model {pred:8.1f} "
            f"({100 * x['model_err']:+.1f}%), kappa {x['kappa']:.3f}")
    log(f"step model: {consts}; worst error {100 * worst:.1f}%")
    return dict(constants=consts, worst_abs_err=round(worst, 4), rows=rows)


NEAR = 1e-4  # a node is near the cut when its log mass, or the cumulative mass at the cut, is this close


def near_cut_counts(tree, torch, q, p, scale, C, L, lens, Hkv, G):
    """Nodes near each level's cut in the last group route of q [B][Hq][d]: from the tree's
    stored planes, each frontier node's mass (its per-head softmax over the frontier of the
    scores max_r (b_r + q.m~_r), averaged over the group's heads) in fp64, ordered by mass
    against the route's own kept count k; counted are the nodes whose log mass lies within
    NEAR of the k-th or (k+1)-th node's, and those two when the cumulative mass there lies
    within NEAR of p.  These are the decisions that fp32 arithmetic (the kernels) and fp64
    (the oracle) may take differently.  Returns ({level: count}, frontier nodes)."""
    counts, nodes = {}, 0
    qf = q.double() * scale
    kept_prev = None
    for l in range(L, 0, -1):
        nf, nk, ids = tree.route_level(l)
        m_all, b_all = tree.level(l)
        c_l = 0
        kept_now = []
        for b, N in enumerate(lens):
            Nc = (N // C) * C
            n_l = -(-Nc // C ** l)
            for g in range(Hkv):
                u = b * Hkv + g
                if l == L:
                    F = torch.arange(n_l, device=ids.device)
                else:
                    par = kept_prev[u]
                    F = (par[:, None] * C + torch.arange(C, device=ids.device)[None, :]).reshape(-1)
                    F = F[F < n_l]
                k = int(nk[u])
                kept_now.append(ids[u, :k].long())
                nodes += len(F)
                if len(F) == 0 or k <= 0 or k >= len(F) or p >= 1.0:
                    continue
                mF = m_all[u, F].double()                      # [F][R][d]
                bF = b_all[u, F].double()                      # [F][R]
                qh = qf[b, g * G:(g + 1) * G]                  # [G][d]
                s_ = (torch.einsum("frd,hd->hfr", mF, qh) + bF[None]).amax(dim=2)  # [G][F]
                w = torch.exp(s_ - torch.logsumexp(s_, dim=1, keepdim=True)).mean(dim=0)
                order = torch.argsort(w, descending=True)
                lw = torch.log(w)
                near = (torch.abs(lw - lw[order[k - 1]]) < NEAR) | (torch.abs(lw - lw[order[k]]) < NEAR)
                cs = torch.cumsum(w[order], 0) / w.sum()
                c_prev = float(cs[k - 2]) if k >= 2 else -1.0
                extra = 2 if min(abs(c_prev - p), abs(float(cs[k - 1]) - p)) < NEAR else 0
                c_l += int(near.sum()) + extra
        counts[l] = c_l
        kept_prev = kept_now
    return counts, nodes


def union_counts(tree, L, C, hr, Tq, Hkv, lens, qtail):
    """Distinct work of the last route when all routing units of one (sequence, KV head)
    are served together, as the union kernels serve them (its query heads after a per-head
    route, its queries after a block route): per level, the distinct frontier nodes (every
    top-level node; below, the existing children of the union of the units' kept nodes one
    level up), and the distinct attended tokens (the union of kept chunks, the sink when no
    unit keeps chunk 0, and the longest tail).  Returns (frontier per level, tokens, frontier
    per level summed over units, kept per level summed over units)."""
    import numpy as np
    kept, fr_unit, kept_unit = {}, {}, {}
    for l in range(1, L + 1):
        nf, nk, ids = tree.route_level(l)
        nk, ids = nk.cpu().numpy(), ids.cpu().numpy()
        fr_unit[l], kept_unit[l] = int(nf.sum()), int(nk.sum())
        per = {}
        for u in range(len(nk)):
            per.setdefault((u // (Tq * Hkv * hr), (u // hr) % Hkv), []).append(ids[u, :nk[u]])
        kept[l] = {k: np.unique(np.concatenate(v)) for k, v in per.items()}
    fr = {}
    for l in range(1, L + 1):
        tot = 0
        for (b, g) in kept[l]:
            n_l = -(-((lens[b] // C) * C) // C ** l)
            if l == L:
                tot += n_l
            else:
                j = kept[l + 1][(b, g)].astype(np.int64)
                tot += int(np.clip(n_l - j * C, 0, C).sum())
        fr[l] = tot
    tok = 0
    for (b, g), k1 in kept[1].items():
        Nc = (lens[b] // C) * C
        sink = 1 if (Nc > 0 and (len(k1) == 0 or k1[0] != 0)) else 0
        tok += sink + (lens[b] + (Tq if qtail else 0) - Nc) + len(k1) * C
    return fr, tok, fr_unit, kept_unit


def input_key(cfg):
    """Fields that decide a workload's generated inputs (deep_256k and wide_256k share theirs)."""
    return (cfg.seed, cfg.batch, cfg.n_tokens, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_queries,
            cfg.needles_per_unit, cfg.needles_per_query, cfg.dtype, cfg.head_scale, cfg.append_steps)


def load_inputs(cfg, zi, torch, dev, nq, workers=16):
    """K, V [B][Hkv][max_tokens][d] on the device (the rows appended during decode included),
    the first nq decode queries [nq][B][Hq][d] and the references, each unit generated from its
    own stream in a parallel thread."""
    from concurrent.futures import ThreadPoolExecutor
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, Hkv, d, N, T = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.n_tokens, cfg.max_tokens
    q_all = zi.queries(cfg)
    K0 = torch.empty((B, Hkv, T, d), dtype=dt, device=dev)
    V0 = torch.empty((B, Hkv, T, d), dtype=dt, device=dev)

    def gen(bg):
        b, g = bg
        Ku, Vu = zi.unit_kv(cfg, b, g, q_all)
        app = zi.append_rows(cfg, b, g) if cfg.append_steps else None
        return bg, Ku, Vu, app

    pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(max(1, min(workers, len(pairs)))) as ex:
        for (b, g), Ku, Vu, app in ex.map(gen, pairs):
            K0[b, g, :N] = torch.from_numpy(Ku).to(dev, dt)
            V0[b, g, :N] = torch.from_numpy(Vu).to(dev, dt)
            if app is not None:  # the rows each decode step appends (written before zha_append)
                K0[b, g, N:] = torch.from_numpy(app[0]).to(dev, dt)
                V0[b, g, N:] = torch.from_numpy(app[1]).to(dev, dt)
    qd = torch.from_numpy(q_all[:nq]).to(dev, dt)
    return K0, V0, qd, q_all


def run_workload(cfg, args, env, headline, layers):
    """Measures one workload; returns its record.  env: modules, device and the input cache."""
    np, torch, zi, zha, Tree, dense_decode, dev = (env[k] for k in ("np", "torch", "zi", "zha", "Tree", "dense",
                                                                   "dev"))
    p = args.p if (args.p is not None and headline) else cfg.p[0]
    growing = cfg.append_steps > 0
    p_sweep = [p] + [x for x in cfg.p if x != p] if growing else [p]
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    es = 2 if cfg.dtype == "bf16" else 4
    B, Hkv, Hq, d, N = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim, cfg.n_tokens
    U, G, C, L, R = B * Hkv, cfg.group, cfg.chunk, cfg.levels, cfg.n_refs
    T = cfg.max_tokens  # token stride: room for the rows appended during decode
    nq = min(args.queries, cfg.n_queries)

    t0 = time.time()
    key = input_key(cfg)
    if env["inputs"].get("key") != key:
        env["inputs"].clear()
        torch.cuda.empty_cache()
        K0, V0, qd, q_all = load_inputs(cfg, zi, torch, dev, max(nq, args.block if headline else 0))
        env["inputs"].update(key=key, K0=K0, V0=V0, qd=qd, q_all=q_all)
        log(f"[{cfg.name}] inputs ready in {time.time() - t0:.1f}s")
    else:
        log(f"[{cfg.name}] inputs shared with the previous workload")
    K0, V0, qd, q_all = (env["inputs"][k] for k in ("K0", "V0", "qd", "q_all"))
    refs = torch.from_numpy(zi.refs(cfg)).to(dev)

    Ks, Vs = [K0], [V0]
    for _ in range(1, layers):
        Ks.append(K0.clone())
        Vs.append(V0.clone())
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(layers)]
    lses = [torch.empty((B, Hq), dtype=torch.float32, device=dev) for _ in range(layers)]

    def kernel_table(recs):
        per = {}
        for k, l, ms in recs:
            per.setdefault((k, l), []).append(ms)
        return {f"{zha.KERNEL_NAMES[k]}{'_l' + str(l) if l else ''}": dict(launches=len(v), avg_us=1e3 * sum(v) / len(v),
                                                                           total_ms=sum(v), code=k, level=l)
                for (k, l), v in sorted(per.items())}

    def measure_block(Tq, mode="group"):
        """A block of Tq queries per sequence (the first Tq decode queries; a speculative
        verification step or a prefill chunk) routed and attended over the tree of the N_b
        cached tokens, N_b = N - Tq when the block's rows would not fit after N."""
        Nb = N if N + Tq <= T else N - Tq
        trees = []
        for li in range(layers):
            tr = Tree(B, Hkv, Hq, d, C, L, R, T, dt, per_head_routes=mode == "per_head", max_queries=Tq)
            tr.build(Ks[li], refs, [Nb] * B)
            trees.append(tr)
        qb = torch.from_numpy(np.ascontiguousarray(q_all[:Tq].transpose(1, 0, 2, 3))).to(dev, dt)
        ob = [torch.empty((B, Tq, Hq, d), dtype=torch.float32, device=dev) for _ in range(layers)]
        lb = [torch.empty((B, Tq, Hq), dtype=torch.float32, device=dev) for _ in range(layers)]

        def step(i):
            li = i % layers
            trees[li].route_multi(qb, p, 1.0, mode=mode)
            trees[li].attend_multi(qb, Ks[li], Vs[li], 1.0, out=ob[li], lse=lb[li])

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        for tr in trees:
            tr.timing(True)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        recs = []
        for tr in trees:
            recs += tr.timing_read()
            tr.timing(False)
        kernels = kernel_table(recs)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        us = 1e3 * ev0.elapsed_time(ev1) / args.steps
        for tr in trees:
            tr.check()
        # algorithmic bytes: replay the block's route once; a KV head's queries and query heads
        # are served as one union, so each distinct node and token is counted once per KV head
        hr = G if mode == "per_head" else 1
        trees[0].route_multi(qb, p, 1.0, mode=mode)
        torch.cuda.synchronize()
        S_node = R * (d * es + 4)
        ufr, tok, _, _ = union_counts(trees[0], L, C, hr, Tq, Hkv, [Nb] * B, True)
        route_bytes = sum(ufr.values()) * S_node
        attend_bytes = tok * 2 * d * es
        nbytes = route_bytes + attend_bytes
        for tr in trees:
            tr.close()
        torch.cuda.empty_cache()
        log(f"block of {Tq} ({mode}): {us:.1f} us ({us / Tq:.1f} us per query), {nbytes / 1e6:.1f} MB "
            f"({nbytes / (us * 1e-6) / 1e9:.0f} GB/s), kappa {tok / (U * (Nb + Tq)):.3f}")
        for k, v in kernels.items():
            log(f"  {k:12s} {v['launches']:4d} launches  avg {v['avg_us']:8.2f} us")
        return dict(queries=Tq, cached_tokens=Nb, mode=mode, us_per_block=round(us, 2),
                    us_per_query=round(us / Tq, 2), block_bytes=round(nbytes),
                    block_gbs=round(nbytes / (us * 1e-6) / 1e9, 1), kappa=round(tok / (U * (Nb + Tq)), 4),
                    kernels={k: round(v["avg_us"], 2) for k, v in kernels.items()})

    def measure(summary, mode="group", C=C, L=L, R=R, refs=refs, p=p, warm=False, near_cut=False):
        """Builds one tree per layer replica with the given m storage (and geometry C, L, R),
        times the stage breakdown and the K-step region, and replays the routes for the
        byte counts.  warm: every step reads layer 0 with query 0 (its data partly cached)."""
        lens = [N] * B
        layer_lens = [[N] * B for _ in range(layers)]
        trees = []
        build_ms = []
        for li in range(layers):
            tr = Tree(B, Hkv, Hq, d, C, L, R, T, dt, summary=summary, per_head_routes=mode == "per_head")
            torch.cuda.synchronize()
            ev0.record()
            tr.build(Ks[li], refs, lens)
            ev1.record()
            torch.cuda.synchronize()
            build_ms.append(ev0.elapsed_time(ev1))
            trees.append(tr)
        tree_bytes = trees[0].bytes()
        log(f"trees built: {[round(x, 3) for x in build_ms]} ms; tree+workspace {tree_bytes / 1e9:.2f} GB per layer")

        if headline and summary == args.summary and mode == "group" and not warm:
            # a copy kernel of known size, for calibrating hardware byte counters in profiles
            cal_n16 = (256 << 20) // 16
            cal_src = torch.empty(cal_n16 * 16, dtype=torch.uint8, device=dev)
            cal_dst = torch.empty_like(cal_src)
            zha.zha_calibration_copy(cal_dst, cal_src, cal_n16)
            torch.cuda.synchronize()
            del cal_src, cal_dst

        segs = []  # per-step event pairs: the step (fixed-size workloads) or append and each p's route + attend
        # every event of the timed region is created before it (creating one is a host-side
        # allocation that can leave the GPU idle between steps)
        nseg = 1 + len(p_sweep) if growing else 1
        pool = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nseg * args.steps)]
        for e in pool:  # torch creates the device event at its first record
            e.record()
        torch.cuda.synchronize()

        def seg(name, fn, record):
            if record:
                a, b = pool.pop(), pool.pop()
                a.record()
                fn()
                b.record()
                segs[-1][name] = (a, b)
            else:
                fn()

        tmask = {}  # growing workloads: kernel timing mask, applied to the headline p's launches only

        def step(i, record=False):
            li, t = (0, 0) if warm else (i % layers, i % nq)
            tr = trees[li]
            if record:
                segs.append({})
            if growing:
                if layer_lens[li][0] < T:
                    layer_lens[li] = [n + 1 for n in layer_lens[li]]
                    if tmask:  # the append is timed in the breakdown pass only
                        tr.timing(tmask["kernels"] is None)
                    seg("append", lambda: tr.append(Ks[li], layer_lens[li]), record)
                for x in p_sweep:
                    if tmask:
                        tr.timing(x == p, **tmask)
                    seg(x, lambda x=x: (tr.route(qd[t], x, 1.0, mode=mode),
                                        tr.attend(qd[t], Ks[li], Vs[li], 1.0, out=outs[li], lse=lses[li])), record)
                if tmask:
                    tr.timing(False)
                return
            seg("step", lambda: (tr.route(qd[t], p, 1.0, mode=mode),
                                 tr.attend(qd[t], Ks[li], Vs[li], 1.0, out=outs[li], lse=lses[li])), record)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()

        # stage breakdown: every launch timed with HIP events (events between launches add
        # a little time, so this pass is not the one whose step time is reported)
        for tr in trees:
            tr.timing(True)
        if growing:
            tmask.update(kernels=None, levels=None)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        recs = []
        for tr in trees:
            recs += tr.timing_read()
            tr.timing(False)
        kernels = kernel_table(recs)
        dom_name, dom = max(kernels.items(), key=lambda kv: kv[1]["total_ms"])

        # timed region: K steps, with an event pair around the dominant kernel only (the
        # library's timing events carry no cache-flushing fence).  A growing workload's step is
        # its append plus its route + attend at the headline p, so it also times each segment;
        # a fixed-size workload's median and 90th percentile come from a separate pass with an
        # event pair around each step, so that those events stay out of the reported mean.
        for tr in trees:
            tr.timing(True, kernels=[dom["code"]], levels=[dom["level"]])
        if growing:
            tmask.update(kernels=[dom["code"]], levels=[dom["level"]])
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            step(i, record=growing)
        ev1.record()
        torch.cuda.synchronize()
        ms_total = ev0.elapsed_time(ev1)
        ms_step = ms_total / args.steps
        live = []
        for tr in trees:
            live += [ms for _, _, ms in tr.timing_read()]
            tr.timing(False)
        if not growing:  # the distribution pass
            for i in range(args.steps):
                step(i, record=True)
            torch.cuda.synchronize()
        seg_us = {}
        for sg in segs:
            for k, (a, b) in sg.items():
                seg_us.setdefault(k, []).append(1e3 * a.elapsed_time(b))
        if growing:  # a step: its append (if the layer had room) + route + attend at p
            per_step = [1e3 * sum(sg[k][0].elapsed_time(sg[k][1]) for k in ("append", p) if k in sg) for sg in segs]
            seg_mean = {k: sum(v) / len(v) for k, v in seg_us.items()}
            ms_step = (seg_mean.get("append", 0.0) + seg_mean[p]) * 1e-3  # append + route + attend at p
        else:
            per_step = seg_us["step"]
            seg_mean = {}
        for tr in trees:
            tr.check()  # no device-side wait of a route gave up
        dom_live_us = 1e3 * sum(live) / len(live)

        # algorithmic bytes of each step (routes are deterministic: replay each query once, untimed)
        S_node = {"fp8": R * (d + 8), "fp4": R * (d // 2 + d // 32 + 4)}.get(summary, R * (d * es + 4))
        hr = G if mode == "per_head" else 1        # routing units per (sequence, KV head)
        Gr = G if mode == "group" else 1           # query heads per routing unit
        fr_tot = {l: 0 for l in range(1, L + 1)}   # distinct frontier nodes per (sequence, KV head)
        fr_unit = {l: 0 for l in range(1, L + 1)}  # frontier nodes summed over routing units
        kept_tot = {l: 0 for l in range(1, L + 1)}
        attend_tok = 0
        steps_q = [0 if warm else i % nq for i in range(args.steps)]
        near = [] if near_cut and mode == "group" else None
        for t in sorted(set(steps_q)):
            w = steps_q.count(t)
            trees[0].route(qd[t], p, 1.0, mode=mode)
            torch.cuda.synchronize()
            if near is not None and len(near) < 4:  # the first four distinct queries
                cnt, nod = near_cut_counts(trees[0], torch, qd[t], p, 1.0, C, L, layer_lens[0], Hkv, G)
                near.append(dict(query=t, near_cut=sum(cnt.values()), by_level={str(k): v for k, v in cnt.items()},
                                 frontier_nodes=nod))
            ufr, utok, frs, kps = union_counts(trees[0], L, C, hr, 1, Hkv, layer_lens[0], False)
            if hr == 1 and ufr != frs:
                raise RuntimeError(f"frontier recount {ufr} disagrees with the route's counts {frs}")
            for l in range(1, L + 1):
                fr_tot[l] += w * ufr[l]
                fr_unit[l] += w * frs[l]
                kept_tot[l] += w * kps[l]
            attend_tok += w * utok
        nsteps = args.steps
        route_bytes = sum(fr_tot[l] for l in fr_tot) * S_node / nsteps
        attend_bytes = attend_tok * 2 * d * es / nsteps
        io_bytes = B * Hq * d * es + B * Hq * (d + 1) * 4 + 8 * sum(kept_tot.values()) / nsteps
        step_bytes = route_bytes + attend_bytes + io_bytes
        Ncur = layer_lens[0][0]
        kappa = attend_tok / nsteps / (U * Ncur)
        dense_bytes = U * Ncur * 2 * d * es

        # the dominant kernel: largest share of the step's time
        if dom_name.startswith("score_l"):
            l = dom["level"]
            dom_bytes = (fr_tot[l] * S_node + fr_unit[l] * Gr * 4 + (fr_unit[l] / C * 4 if l < L else 0)) / nsteps \
                + B * Hq * d * es
            traffic = committed_traffic(cfg.name) if l == 1 and summary == "native" and mode == "group" else None
        elif dom_name == "attend":
            dom_bytes = attend_bytes + B * Hq * d * es
            traffic = None
        else:
            dom_bytes = None
            traffic = None
        dom_avg_s = dom_live_us * 1e-6
        achieved = dom_bytes / dom_avg_s / 1e9 if dom_bytes else None
        roofline = dict(kernel=f"zha_score_kernel (level {dom_name.split('_l')[1]})" if dom_name.startswith("score_l")
                        else dom_name,
                        bound="hbm", achieved=round(achieved, 1) if achieved else None, peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(achieved / PEAK_HBM_GBS, 4) if achieved else None,
                        traffic=traffic, bytes_per_launch=round(dom_bytes) if dom_bytes else None,
                        avg_launch_us=round(dom_live_us, 2))
        log(f"step {ms_step * 1e3:.1f} us (median {pct(per_step, 50):.1f}, p90 {pct(per_step, 90):.1f}), "
            f"{step_bytes / 1e6:.1f} MB/step ({step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s), kappa {kappa:.3f}")
        if growing:
            log("  segments (us): " + ", ".join(f"{k}: {v:.1f}" for k, v in seg_mean.items()))
        for k, v in kernels.items():
            log(f"  {k:12s} {v['launches']:4d} launches  avg {v['avg_us']:8.2f} us")

        for tr in trees:
            tr.close()
        torch.cuda.empty_cache()
        return dict(ms_step=ms_step, step_bytes=step_bytes, kappa=kappa, kernels=kernels, roofline=roofline,
                    seg_us=seg_mean, fr_tot=fr_tot, build_ms=build_ms, tree_bytes=tree_bytes, layer_lens=layer_lens,
                    dense_bytes=dense_bytes, nsteps=nsteps, median_us=pct(per_step, 50), p90_us=pct(per_step, 90),
                    route_bytes_l={l: fr_tot[l] * S_node / nsteps for l in fr_tot}, attend_bytes=attend_bytes,
                    near_cut=near)

    sweep_rows = None
    summary = args.summary if headline else "native"
    log(f"== {cfg.name}: B={B} N={N} {Hq}q/{Hkv}kv d={d} C={C} L={L} R={R} p={p_sweep} ({layers} layer replicas)")
    res = measure(summary, near_cut=True)
    ms_step, step_bytes, kappa, kernels = res["ms_step"], res["step_bytes"], res["kappa"], res["kernels"]
    layer_lens, dense_bytes, nsteps = res["layer_lens"], res["dense_bytes"], res["nsteps"]
    rec = {
        "us_per_step": round(ms_step * 1e3, 2),
        "median_us": round(res["median_us"], 2),
        "p90_us": round(res["p90_us"], 2),
        "roofline": res["roofline"],
        "step_bytes": round(step_bytes),
        "step_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "dense_bytes": dense_bytes,
        "kappa": round(kappa, 4),
        "frontier_per_unit": {l: round(res["fr_tot"][l] / nsteps / U, 1) for l in range(L, 0, -1)},
        "build_us": round(1e3 * float(np.median(res["build_ms"])), 1),
        "near_cut_per_step": res["near_cut"],
        "tree_bytes": res["tree_bytes"],
        "kernels": {k: dict(launches=v["launches"], avg_us=round(v["avg_us"], 2)) for k, v in kernels.items()},
        "config": {"workload": cfg.name, "batch": B, "context": N, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "chunk": C, "levels": L, "refs": R, "p": p, "layers_cycled": layers, "summary": summary},
    }
    if growing:
        rec["append_us"] = round(res["seg_us"].get("append", 0.0), 2)
        rec["p_sweep"] = {str(x): round(res["seg_us"].get("append", 0.0) + res["seg_us"][x], 2) for x in p_sweep}
        rec["config"]["appended_per_step"] = 1

    if headline:
        log("-- warm: every step on the same layer and query")
        rw = measure(summary, warm=True)
        rec["warm_us_per_step"] = round(rw["ms_step"] * 1e3, 2)
        low = {}  # the same workload with low-precision summaries
        if not args.no_fp8 and args.summary == "native" and cfg.dtype == "bf16":
            for sm in ("fp8", "fp4"):
                log(f"-- the same workload with {sm} summaries")
                r8 = measure(sm)
                low[sm] = dict(us_per_step=round(r8["ms_step"] * 1e3, 2), median_us=round(r8["median_us"], 2),
                               step_bytes=round(r8["step_bytes"]),
                               step_gbs=round(r8["step_bytes"] / (r8["ms_step"] * 1e-3) / 1e9, 1),
                               kappa=round(r8["kappa"], 4), roofline=r8["roofline"],
                               build_us=round(1e3 * float(np.median(r8["build_ms"])), 1), tree_bytes=r8["tree_bytes"],
                               kernels={k: round(v["avg_us"], 2) for k, v in r8["kernels"].items()})
                if growing:
                    low[sm]["p_sweep"] = {str(x): round(r8["seg_us"].get("append", 0.0) + r8["seg_us"][x], 2)
                                          for x in p_sweep}
        for sm, v in low.items():
            rec[f"{sm}_summaries"] = v
        if not args.no_sweep and not growing:
            sweep_rows = geometry_sweep(measure, cfg, zi, torch, np, dev, N, B, Hkv, d, es, log)
        if not args.no_per_head and args.summary == "native":
            log("-- the same workload, every query head routed alone")
            rh = measure("native", mode="per_head")
            rec["per_head_routes"] = dict(us_per_step=round(rh["ms_step"] * 1e3, 2), step_bytes=round(rh["step_bytes"]),
                                          step_gbs=round(rh["step_bytes"] / (rh["ms_step"] * 1e-3) / 1e9, 1),
                                          kappa=round(rh["kappa"], 4), roofline=rh["roofline"],
                                          kernels={k: round(v["avg_us"], 2) for k, v in rh["kernels"].items()})
            if growing:
                rec["per_head_routes"]["p_sweep"] = {str(x): round(rh["seg_us"].get("append", 0.0) + rh["seg_us"][x], 2)
                                                     for x in p_sweep}
        if args.block > 0 and args.summary == "native":
            log(f"-- blocks of {args.block} queries per sequence, each routed alone")
            rec["query_block"] = measure_block(args.block)

    # dense decode on the same GPU and inputs, same protocol
    if not args.no_dense:
        nb = zha.zha_dense_workspace_bytes(B, Hq, Hkv, d, T)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        for i in range(args.warmup):
            li = i % layers
            dense_decode(qd[i % nq], Ks[li], Vs[li], layer_lens[li], Hkv, 1.0, ws, outs[li], lses[li])
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in evs:  # the events exist on the device before the timed region
            a.record()
            b.record()
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            li = i % layers
            dense_decode(qd[i % nq], Ks[li], Vs[li], layer_lens[li], Hkv, 1.0, ws, outs[li], lses[li])
        ev1.record()
        torch.cuda.synchronize()
        dense_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
        for i in range(args.steps):  # the distribution pass: an event pair around each step
            li = i % layers
            evs[i][0].record()
            dense_decode(qd[i % nq], Ks[li], Vs[li], layer_lens[li], Hkv, 1.0, ws, outs[li], lses[li])
            evs[i][1].record()
        torch.cuda.synchronize()
        dense_med = pct([1e3 * a.elapsed_time(b) for a, b in evs], 50)
        log(f"dense {dense_us:.1f} us/step (median {dense_med:.1f}; {dense_bytes / (dense_us * 1e-6) / 1e9:.0f} GB/s)")
        rec["dense_us_per_step"] = round(dense_us, 2)
        rec["dense_median_us"] = round(dense_med, 2)
        rec["speedup_vs_dense"] = round(dense_us / (ms_step * 1e3), 3)
        if sweep_rows:
            log("-- geometry sweep against the step model (bandwidth of dense decode; constants measured here)")
            bw = dense_bytes / dense_us  # bytes per microsecond
            consts = model_constants(res, level_caps(N, C, L), bw)
            rec["geometry_sweep"] = sweep_model(sweep_rows, consts, log)
    del Ks, Vs, outs, lses
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(cfg, args, env):
    """The oracle on the host cores, on a bounded sample: the decode queries of two (sequence,
    KV head) units (about 10-20 s of host work), scaled to a whole step; then the same on one
    thread for a few queries of one unit."""
    np, zi = env["np"], env["zi"]
    import oracle
    p = args.p if args.p is not None else cfg.p[0]
    B, Hkv, N, C, L, G = cfg.batch, cfg.n_kv_heads, cfg.n_tokens, cfg.chunk, cfg.levels, cfg.group
    U = B * Hkv
    ncpu = min(args.cpu_queries, cfg.n_queries)
    qc = zi.queries(cfg, n=ncpu)
    q_all = env["inputs"].get("q_all") if env["inputs"].get("key") == input_key(cfg) else None
    units = [(0, g) for g in range(min(2, Hkv))]
    trees, kv = {}, {}
    for (b0, g0) in units:
        Ku, Vu = zi.unit_kv(cfg, b0, g0, q_all)
        kv[(b0, g0)] = (Ku.astype(np.float64), Vu.astype(np.float64))
        trees[(b0, g0)] = oracle.tree_merge(Ku, zi.refs(cfg)[g0], C, L)  # untimed

    def run(pairs, nqq):
        t0 = time.time()
        for (b0, g0) in pairs:
            Ku, Vu = kv[(b0, g0)]
            for t in range(nqq):
                qu = qc[t, b0, g0 * G:(g0 + 1) * G].astype(np.float64)
                _, kept = oracle.route(trees[(b0, g0)], N, C, L, qu, p)
                S = oracle.attend_set(N, C, kept[1])
                oracle.attend(qu, Ku, Vu, S)
        return time.time() - t0

    threads = oracle.num_threads()
    sec = run(units, ncpu)
    per_unit_step = sec / (ncpu * len(units))
    n1 = min(4, ncpu)
    oracle.set_num_threads(1)
    try:
        sec1 = run(units[:1], n1)
    finally:
        oracle.set_num_threads(threads)
    one = dict(value=round(sec1 / n1 * U * 1e6, 1), unit="us/step/layer", cores=1,
               sample=f"route+attend of 1 unit for {n1} decode queries ({sec1:.1f} s), scaled by {U} units")
    cpu = dict(value=round(per_unit_step * U * 1e6, 1), unit="us/step/layer", cores=threads, kind="oracle",
               cpu_model=cpu_model(),
               sample=f"route+attend of {len(units)} (sequence, KV head) units for {ncpu} decode queries each "
                      f"({sec:.1f} s), scaled by {U} units to one full step; oracle trees built untimed",
               single_thread=one)
    log(f"cpu oracle {cpu['value']:.0f} us/step on {threads} threads, {one['value']:.0f} us/step on 1 thread "
        f"({cpu['cpu_model']})")
    return cpu


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path would shard by (sequence, KV head), with no exchange between GPUs", flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    import zha_inputs as zi
    from hierarchical_tree_indexed_02_amd import zha
    from hierarchical_tree_indexed_02_amd.runtime import Tree, dense_decode

    env = dict(np=np, torch=torch, zi=zi, zha=zha, Tree=Tree, dense=dense_decode, dev=torch.device("cuda:0"),
               inputs={})
    t_start = time.time()
    cfg = zi.get_config(args.config)
    head = run_workload(cfg, args, env, headline=True, layers=args.layers)
    subs = {}
    for name in [w for w in args.workloads.split(",") if w and w != cfg.name]:
        subs[name] = run_workload(zi.get_config(name), args, env, headline=False,
                                  layers=SUB_LAYERS.get(name, args.layers))
        log(f"[{name}] {subs[name]['us_per_step']} us/step (dense {subs[name].get('dense_us_per_step')}); "
            f"{time.time() - t_start:.0f} s so far")
    env["inputs"].clear()
    torch.cuda.empty_cache()
    cpu = None if args.no_cpu else cpu_baseline(cfg, args, env)

    ms_step = head["us_per_step"] * 1e-3
    result = {
        "metric": METRIC,
        "value": head["us_per_step"],
        "unit": "us/step/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded planted-needle keys/values, random reference queries)",
        "config": head.pop("config"),
        "roofline": head.pop("roofline"),
        "cpu_baseline": cpu,
    }
    head.pop("us_per_step")
    result.update(head)
    if subs:
        result["workloads"] = subs
    result["bench_wall_s"] = round(time.time() - t_start, 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
