"""Decode-step benchmark of the ZHA path on one MI355X.

One step = one decode step of one attention layer: route the B x Hq queries
through that layer's tree (every level) and attend over the kept chunks plus
sink and tail.  For a workload with decode-time growth (batch8_append_512k) a
step first appends one K/V row per sequence (zha_append), then routes and
attends once for each p of the workload's sweep; `value` is append + route +
attend at the first p (or --p), and `p_sweep` gives every p.  Inputs are
resident in HBM before timing; steps cycle through `--layers` replicas of
(K, V, tree) so every step reads its layer cold, and through `--queries`
different decode queries.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 40] [--warmup 5] [--config deep_256k]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "ZHA decode µs/step/layer at 256K & 1M ctx; achieved HBM GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
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
    ap.add_argument("--sweep", action="store_true",
                    help="also time the workload's inputs under other tree geometries (C, L, R) and p, and fit a "
                         "step-time model (bytes at the measured bandwidths + a fixed cost per routing level)")
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


# Tree geometries (chunk C, levels L, references R) over the same 256K-token inputs: C^L = 4096
# tokens per top node except where noted, and the flat C = 256 tree.
SWEEP = [(4, 6, 16, 0.95), (4, 6, 4, 0.95), (4, 6, 1, 0.95), (4, 6, 16, 0.7), (8, 4, 16, 0.95), (8, 4, 4, 0.95),
         (16, 3, 16, 0.95), (16, 3, 4, 0.95), (64, 2, 16, 0.95), (4, 5, 16, 0.95), (256, 1, 16, 0.95),
         (256, 1, 4, 0.95), (256, 1, 16, 0.7)]


def geometry_sweep(measure, cfg, zi, torch, np, dev, N, B, Hkv, d, es, log):
    """Times route + attend under each geometry of SWEEP and fits
        t_step = route_bytes / BW_route + attend_bytes / BW_attend + n_small * c_small + n_large * c_large + c0
    by least squares (n_small / n_large: routing levels of at most / more than 8192 nodes
    per unit); returns one record per geometry with the fitted prediction."""
    rows = []
    for C, L, R, p in SWEEP:
        if C ** L > N:
            continue
        g = zi.get_config(cfg.name, chunk=C, levels=L, n_refs=R)
        refs = torch.from_numpy(zi.refs(g)).to(dev)
        log(f"-- geometry C={C} L={L} R={R} p={p}")
        r = measure("native", "group", C=C, L=L, R=R, refs=refs, p=p)
        caps = [-(-((N // C) * C) // C ** l) for l in range(1, L + 1)]
        n_small = sum(1 for c in caps if c <= 8192)
        kern = r["kernels"]
        route_us = sum(v["avg_us"] for k, v in kern.items() if k.split("_l")[0] in ("score", "select", "mass", "compact"))
        att_us = kern.get("attend", {}).get("avg_us", 0.0)
        S_node = R * (d * es + 4)
        route_bytes = sum(r["fr_tot"].values()) * S_node / r["nsteps"]
        rows.append(dict(C=C, L=L, R=R, p=p, us_per_step=round(r["ms_step"] * 1e3, 2),
                         step_bytes=round(r["step_bytes"]), route_bytes=round(route_bytes),
                         attend_bytes=round(r["step_bytes"] - route_bytes), kappa=round(r["kappa"], 4),
                         route_us=round(route_us, 1), attend_us=round(att_us, 1), small_levels=n_small,
                         large_levels=L - n_small, tree_bytes=r["tree_bytes"]))
    X = np.array([[x["route_bytes"] / 1e9, x["attend_bytes"] / 1e9, x["small_levels"], x["large_levels"], 1.0]
                  for x in rows])
    y = np.array([x["us_per_step"] for x in rows])
    coef, *_ = np.linalg.lstsq(X, y, rcond=None)
    for x, pred in zip(rows, X @ coef):
        x["model_us"] = round(float(pred), 1)
    fit = dict(us_per_GB_route=round(float(coef[0]), 2), us_per_GB_attend=round(float(coef[1]), 2),
               us_per_small_level=round(float(coef[2]), 2), us_per_large_level=round(float(coef[3]), 2),
               us_fixed=round(float(coef[4]), 2))
    log("geometry sweep fit: " + ", ".join(f"{k} {v}" for k, v in fit.items()))
    for x in rows:
        log(f"  C={x['C']:3d} L={x['L']} R={x['R']:2d} p={x['p']}: {x['us_per_step']:8.1f} us (model {x['model_us']:8.1f}), "
            f"kappa {x['kappa']:.3f}, route {x['route_bytes'] / 1e6:7.1f} MB, attend {x['attend_bytes'] / 1e6:6.1f} MB")
    return dict(fit=fit, rows=rows)



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

    cfg = zi.get_config(args.config)
    p = args.p if args.p is not None else cfg.p[0]
    growing = cfg.append_steps > 0
    p_sweep = [p] + [x for x in cfg.p if x != p] if growing else [p]
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    es = 2 if cfg.dtype == "bf16" else 4
    B, Hkv, Hq, d, N = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim, cfg.n_tokens
    U, G, C, L, R = B * Hkv, cfg.group, cfg.chunk, cfg.levels, cfg.n_refs
    T = cfg.max_tokens  # token stride: room for the rows appended during decode
    nq = min(args.queries, cfg.n_queries)

    t0 = time.time()
    q_all = zi.queries(cfg)
    q_host = q_all[:nq]
    K0 = torch.empty((B, Hkv, T, d), dtype=dt, device=dev)
    V0 = torch.empty((B, Hkv, T, d), dtype=dt, device=dev)
    for b in range(B):
        for g in range(Hkv):
            Ku, Vu = zi.unit_kv(cfg, b, g, q_all)
            K0[b, g, :N] = torch.from_numpy(Ku).to(dev, dt)
            V0[b, g, :N] = torch.from_numpy(Vu).to(dev, dt)
            if growing:  # the rows each decode step appends (written by the caller before zha_append)
                Ka, Va = zi.append_rows(cfg, b, g)
                K0[b, g, N:] = torch.from_numpy(Ka).to(dev, dt)
                V0[b, g, N:] = torch.from_numpy(Va).to(dev, dt)
    qd = torch.from_numpy(q_host).to(dev, dt)
    refs = torch.from_numpy(zi.refs(cfg)).to(dev)
    log(f"inputs ready in {time.time() - t0:.1f}s")

    Ks, Vs = [K0], [V0]
    for _ in range(1, args.layers):
        Ks.append(K0.clone())
        Vs.append(V0.clone())
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(args.layers)]
    lses = [torch.empty((B, Hq), dtype=torch.float32, device=dev) for _ in range(args.layers)]

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
        for li in range(args.layers):
            tr = Tree(B, Hkv, Hq, d, C, L, R, T, dt, per_head_routes=mode == "per_head", max_queries=Tq)
            tr.build(Ks[li], refs, [Nb] * B)
            trees.append(tr)
        qb = torch.from_numpy(np.ascontiguousarray(q_all[:Tq].transpose(1, 0, 2, 3))).to(dev, dt)
        ob = [torch.empty((B, Tq, Hq, d), dtype=torch.float32, device=dev) for _ in range(args.layers)]
        lb = [torch.empty((B, Tq, Hq), dtype=torch.float32, device=dev) for _ in range(args.layers)]

        def step(i):
            li = i % args.layers
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

    def measure(summary, mode="group", C=C, L=L, R=R, refs=refs, p=p):
        """Builds one tree per layer replica with the given m storage (and geometry C, L, R),
        times the stage breakdown and the K-step region, and replays the routes for the
        byte counts."""
        lens = [N] * B
        layer_lens = [[N] * B for _ in range(args.layers)]
        trees = []
        build_ms = []
        for li in range(args.layers):
            tr = Tree(B, Hkv, Hq, d, C, L, R, T, dt, summary=summary, per_head_routes=mode == "per_head")
            torch.cuda.synchronize()
            ev0.record()
            tr.build(Ks[li], refs, lens)
            ev1.record()
            torch.cuda.synchronize()
            build_ms.append(ev0.elapsed_time(ev1))
            trees.append(tr)
        tree_bytes = trees[0].bytes()
        log(f"trees built: {build_ms} ms; tree+workspace {tree_bytes / 1e9:.2f} GB per layer")

        if summary == args.summary:
            # a copy kernel of known size, for calibrating hardware byte counters in profiles
            cal_n16 = (256 << 20) // 16
            cal_src = torch.empty(cal_n16 * 16, dtype=torch.uint8, device=dev)
            cal_dst = torch.empty_like(cal_src)
            zha.zha_calibration_copy(cal_dst, cal_src, cal_n16)
            torch.cuda.synchronize()
            del cal_src, cal_dst

        segs = []  # growing workloads: per-step event pairs of append and of each p's route + attend

        def seg(name, fn, record):
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                segs[-1][name] = (a, b)
            else:
                fn()

        tmask = {}  # growing workloads: kernel timing mask, applied to the headline p's launches only

        def step(i, record=False):
            li, t = i % args.layers, i % nq
            tr = trees[li]
            if growing:
                if record:
                    segs.append({})
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
            tr.route(qd[t], p, 1.0, mode=mode)
            tr.attend(qd[t], Ks[li], Vs[li], 1.0, out=outs[li], lse=lses[li])

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

        # timed region: K steps, with an event pair around the dominant kernel only
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
        seg_us = {}
        if growing:
            for sg in segs:
                for k, (a, b) in sg.items():
                    seg_us.setdefault(k, []).append(1e3 * a.elapsed_time(b))
            seg_us = {k: sum(v) / len(v) for k, v in seg_us.items()}
            ms_step = (seg_us.get("append", 0.0) + seg_us[p]) * 1e-3  # append + route + attend at p
        live = []
        for tr in trees:
            live += [ms for _, _, ms in tr.timing_read()]
            tr.timing(False)
        dom_live_us = 1e3 * sum(live) / len(live)

        # algorithmic bytes of each step (routes are deterministic: replay each query once, untimed)
        S_node = {"fp8": R * (d + 8), "fp4": R * (d // 2 + d // 32 + 4)}.get(summary, R * (d * es + 4))
        hr = G if mode == "per_head" else 1        # routing units per (sequence, KV head)
        Gr = G if mode == "group" else 1           # query heads per routing unit
        fr_tot = {l: 0 for l in range(1, L + 1)}   # distinct frontier nodes per (sequence, KV head)
        fr_unit = {l: 0 for l in range(1, L + 1)}  # frontier nodes summed over routing units
        kept_tot = {l: 0 for l in range(1, L + 1)}
        attend_tok = 0
        steps_q = [i % nq for i in range(args.steps)]
        for t in sorted(set(steps_q)):
            w = steps_q.count(t)
            trees[0].route(qd[t], p, 1.0, mode=mode)
            torch.cuda.synchronize()
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
            traffic = committed_traffic(args.config) if l == 1 and summary == "native" and mode == "group" else None
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
        log(f"step {ms_step * 1e3:.1f} us, {step_bytes / 1e6:.1f} MB/step ({step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s), "
            f"kappa {kappa:.3f}")
        if growing:
            log("  segments (us): " + ", ".join(f"{k}: {v:.1f}" for k, v in seg_us.items()))
        for k, v in kernels.items():
            log(f"  {k:12s} {v['launches']:4d} launches  avg {v['avg_us']:8.2f} us")

        for tr in trees:
            tr.close()
        torch.cuda.empty_cache()
        return dict(ms_step=ms_step, step_bytes=step_bytes, kappa=kappa, kernels=kernels, roofline=roofline,
                    seg_us=seg_us, fr_tot=fr_tot, build_ms=build_ms, tree_bytes=tree_bytes, layer_lens=layer_lens,
                    dense_bytes=dense_bytes, nsteps=nsteps)

    res = measure(args.summary)
    ms_step, step_bytes, kappa, kernels = res["ms_step"], res["step_bytes"], res["kappa"], res["kernels"]
    roofline, seg_us, fr_tot, build_ms = res["roofline"], res["seg_us"], res["fr_tot"], res["build_ms"]
    layer_lens, dense_bytes, nsteps = res["layer_lens"], res["dense_bytes"], res["nsteps"]
    low = {}  # the same workload with low-precision summaries
    if not args.no_fp8 and args.summary == "native" and cfg.dtype == "bf16":
        for sm in ("fp8", "fp4"):
            log(f"-- the same workload with {sm} summaries")
            r8 = measure(sm)
            low[sm] = dict(us_per_step=round(r8["ms_step"] * 1e3, 2), step_bytes=round(r8["step_bytes"]),
                           step_gbs=round(r8["step_bytes"] / (r8["ms_step"] * 1e-3) / 1e9, 1),
                           kappa=round(r8["kappa"], 4), roofline=r8["roofline"],
                           build_us=round(1e3 * float(np.median(r8["build_ms"])), 1), tree_bytes=r8["tree_bytes"],
                           kernels={k: round(v["avg_us"], 2) for k, v in r8["kernels"].items()})
            if growing:
                low[sm]["p_sweep"] = {str(x): round(r8["seg_us"].get("append", 0.0) + r8["seg_us"][x], 2)
                                      for x in p_sweep}
    sweep = None
    if args.sweep and not growing:
        sweep = geometry_sweep(measure, cfg, zi, torch, np, dev, N, B, Hkv, d, es, log)
    per_head = None
    if not args.no_per_head and args.summary == "native":
        log("-- the same workload, every query head routed alone")
        rh = measure("native", mode="per_head")
        per_head = dict(us_per_step=round(rh["ms_step"] * 1e3, 2), step_bytes=round(rh["step_bytes"]),
                        step_gbs=round(rh["step_bytes"] / (rh["ms_step"] * 1e-3) / 1e9, 1),
                        kappa=round(rh["kappa"], 4), roofline=rh["roofline"],
                        kernels={k: round(v["avg_us"], 2) for k, v in rh["kernels"].items()})
        if growing:
            per_head["p_sweep"] = {str(x): round(rh["seg_us"].get("append", 0.0) + rh["seg_us"][x], 2) for x in p_sweep}

    block = None
    if args.block > 0 and args.summary == "native":
        log(f"-- blocks of {args.block} queries per sequence, each routed alone")
        block = measure_block(args.block)

    # dense decode on the same GPU and inputs, same protocol
    dense_us = None
    if not args.no_dense:
        nb = zha.zha_dense_workspace_bytes(B, Hq, Hkv, d, T)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        for i in range(args.warmup):
            li = i % args.layers
            dense_decode(qd[i % nq], Ks[li], Vs[li], layer_lens[li], Hkv, 1.0, ws, outs[li], lses[li])
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            li = i % args.layers
            dense_decode(qd[i % nq], Ks[li], Vs[li], layer_lens[li], Hkv, 1.0, ws, outs[li], lses[li])
        ev1.record()
        torch.cuda.synchronize()
        dense_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
        log(f"dense {dense_us:.1f} us/step ({dense_bytes / (dense_us * 1e-6) / 1e9:.0f} GB/s)")

    # the oracle on the host cores, on a bounded sample: the decode queries of two (sequence,
    # KV head) units (about 10-20 s of host work), scaled to a whole step
    cpu = None
    if not args.no_cpu:
        import oracle
        ncpu = min(args.cpu_queries, cfg.n_queries)
        qc = zi.queries(cfg, n=ncpu)
        units = [(0, g) for g in range(min(2, Hkv))]
        sec = 0.0
        for (b0, g0) in units:
            Ku, Vu = zi.unit_kv(cfg, b0, g0, q_all)
            tree_o = oracle.tree_merge(Ku, zi.refs(cfg)[g0], C, L)  # untimed
            tc0 = time.time()
            for t in range(ncpu):
                qu = qc[t, b0, g0 * G:(g0 + 1) * G].astype(np.float64)
                _, kept = oracle.route(tree_o, N, C, L, qu, p)
                S = oracle.attend_set(N, C, kept[1])
                oracle.attend(qu, Ku, Vu, S)
            sec += time.time() - tc0
        per_unit_step = sec / (ncpu * len(units))
        cpu = dict(value=round(per_unit_step * U * 1e6, 1), unit="us/step/layer", cores=oracle.num_threads(),
                   kind="oracle",
                   sample=f"route+attend of {len(units)} (sequence, KV head) units for {ncpu} decode queries each "
                          f"({sec:.1f} s), scaled by {U} units to one full step; oracle trees built untimed")
        log(f"cpu oracle {cpu['value']:.0f} us/step on {cpu['cores']} threads")

    result = {
        "metric": METRIC,
        "value": round(ms_step * 1e3, 2),
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
        "config": {"workload": cfg.name, "batch": B, "context": N, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "chunk": C, "levels": L, "refs": R, "p": p, "layers_cycled": args.layers},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_us_per_step": round(dense_us, 2) if dense_us else None,
        "speedup_vs_dense": round(dense_us / (ms_step * 1e3), 3) if dense_us else None,
        "step_bytes": round(step_bytes),
        "step_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "dense_bytes": dense_bytes,
        "kappa": round(kappa, 4),
        "frontier_per_unit": {l: round(fr_tot[l] / nsteps / U, 1) for l in range(L, 0, -1)},
        "build_us": round(1e3 * float(np.median(build_ms)), 1),
        "kernels": {k: dict(launches=v["launches"], avg_us=round(v["avg_us"], 2)) for k, v in kernels.items()},
    }
    result["config"]["summary"] = args.summary
    for sm, v in low.items():
        result[f"{sm}_summaries"] = v
    if per_head is not None:
        result["per_head_routes"] = per_head
    if sweep is not None:
        result["geometry_sweep"] = sweep
    if block is not None:
        result["query_block"] = block
    if growing:
        result["append_us"] = round(seg_us.get("append", 0.0), 2)
        result["p_sweep"] = {str(x): round(seg_us.get("append", 0.0) + seg_us[x], 2) for x in p_sweep}
        result["config"]["appended_per_step"] = 1
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
