#!/usr/bin/env python3
"""Benchmark of one fused prefix-shared decode step on one MI355X.

A step is one launch of the fused kernel over the whole batch of the chosen
workload (default: Llama-3-8B attention shape, 8 prefix groups x 100
requests, 2048-token prefixes, distinct lengths U[64, 512], bf16), with Q and
the paged K/V pools already resident in HBM.  The plan is built and uploaded
before timing.  Each timed step is bracketed by HIP events on the launch
stream; L2 and the 256 MB MALL are flushed before every step, outside the
events, by reading a 1 GiB buffer (a read leaves no dirty lines whose
write-back would be charged to the timed launch).  Prints one JSON line.

--gpus N with N > 1 is refused: the benchmark measures one GPU; the path
shards by prefix group or kv head without any exchange between GPUs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention queries/s + effective KV GB/s (% of HBM roofline), 8×100 groups"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("decode.hip", "psa_internal.h", "layout.h", "plan.cpp"):
        with open(os.path.join(ROOT, "prefix_shared_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, launch_bytes_alg):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def describe(wl, batch):
    import numpy as np

    lp = np.asarray(batch["group_prefix_len"])
    ld = np.asarray(batch["query_distinct_len"])
    return {
        "workload": wl.name,
        "num_queries": int(len(batch["query_group"])),
        "prefix_groups": int(len(lp)),
        "prefix_tokens": sorted(set(int(x) for x in lp))[:4],
        "distinct_tokens_min_max_mean": [int(ld.min()), int(ld.max()), round(float(ld.mean()), 1)] if len(ld) else [],
        "q_heads": wl.num_q_heads,
        "kv_heads": wl.num_kv_heads,
        "head_dim": wl.head_dim,
        "page_size": wl.page_size,
        "kv_dtype": wl.dtype,
        "seed": wl.seed,
    }


def cpu_baseline(wl, batch, q, k, v, target_s, max_s):
    """The fp64 oracle on a bounded sample of the same workload, queries/s."""
    import numpy as np

    import oracle
    from workloads import subset_for_queries

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = 1
    n = len(batch["query_group"])
    rng = np.random.default_rng(123)
    order = rng.permutation(n)

    def run(count, passes=1):
        import torch

        qs = sorted(int(x) for x in order[:count])
        sub, page_ids = subset_for_queries(batch, qs)
        idx = torch.as_tensor(page_ids, device=k.device, dtype=torch.long)
        ks = k.index_select(0, idx).float().cpu().numpy()
        vs = v.index_select(0, idx).float().cpu().numpy()
        qh = q.index_select(0, torch.as_tensor(qs, device=q.device)).float().cpu().numpy()
        t0 = time.perf_counter()
        for _ in range(passes):
            oracle.decode_attention(qh, ks, vs, sub)
        return time.perf_counter() - t0

    count = 4
    el = run(count)
    while el < target_s / 4 and count < n:
        count = min(n, count * 4)
        el = run(count)
    if el < target_s and count < n:
        count = min(n, max(count + 1, int(count * target_s / max(el, 1e-3))))
        el = run(count)
    while el > max_s and count > 1:
        count = max(1, count // 2)
        el = run(count)
    passes = 1
    if count == n and el < target_s / 2:  # the whole workload is quick: time several passes over it
        passes = min(8, max(1, int(target_s / max(el, 1e-3))))
        el = run(count, passes)
    return {
        "value": count * passes / el,
        "unit": "queries/s",
        "cores": int(threads),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{count} of {n} queries of {wl.name} (all heads), {passes} pass(es), fp64 numpy oracle, "
                  f"{el:.1f} s",
        "note": "plain fp64 oracle on the host cores: a reported baseline, not the target",
    }


def host_identification(P, reps=3):
    """Host time of psa_identify_prefix_groups on 8000 token-id prompts shaped
    like the pages' industrial workload (best of `reps`)."""
    from workloads import build_token_batch

    seqs = build_token_batch()
    best, res = None, None
    for _ in range(reps):
        t0 = time.perf_counter()
        res = P.psa_identify_prefix_groups(seqs)
        el = time.perf_counter() - t0
        best = el if best is None else min(best, el)
    tokens = int(sum(len(x) for x in seqs))
    return {"requests": len(seqs), "tokens": tokens, "ms": 1e3 * best, "groups": int(len(res["group_prefix_len"])),
            "saved_tokens": res["saved_tokens"],
            "shape": "50-token system prompt, documents of 1000-2100 tokens shared by 3 requests, 1-60 "
                     "distinct tokens each",
            "context": "the pages quote 1.51 s for 8000 requests (Python, host CPU), tree build to group list"}


def trace_summary(P, plan, q, k, v, out, ws, flush, sink, info, path, wl, launches=3):
    """Traced launches (a cache flush before each): per unit its start, end
    and XCD (s_memrealtime, 100 MHz).  Reported per launch: per-kind unit
    durations, how many units of each kind run at once (10 us bins), each
    XCD's last end and summed unit time, and the mat-vec units' KV rate over
    time, estimated by spreading each unit's bytes evenly over its life (an
    estimate: good for comparing phases and runs, not an absolute rate)."""
    import numpy as np
    import torch

    units = int(info["num_items"])
    it = np.asarray(plan.items()).reshape(units, 4, 8)
    kind_of = it[:, 0, 0] & 0xFF
    tok_bytes = wl.head_dim * (2 if wl.dtype == "bf16" else 4) * 2  # K and V of one token, one kv head
    mv_tokens = np.zeros(units)
    for w in range(4):
        mv_tokens += np.where((it[:, w, 0] & 0xFF) == 1, it[:, w, 4] - it[:, w, 3], 0)
    names = {0: "nop", 1: "matvec", 2: "mfma_prefix", 3: "empty"}
    res = {"units": units, "launches": []}
    for li in range(launches):
        tr = torch.zeros(units * 4, dtype=torch.int64, device="cuda")
        if flush is not None:
            torch.sum(flush, dim=None, out=sink)
        P.psa_decode_attention(plan, q, k, v, out, ws, trace=tr)
        torch.cuda.synchronize()
        t = tr.view(units, 4).cpu().numpy()
        if li == 0:
            np.save(path + ".npy", t)  # raw records of the first launch: start, end, HW_ID | XCC_ID << 32, kind
        ok = (t[:, 0] > 0) & (t[:, 1] >= t[:, 0])
        if not ok.all():
            log(f"trace: {int((~ok).sum())} of {units} units without a valid record, e.g. {t[~ok][:3].tolist()}")
            continue
        t0 = t[:, 0].min()
        start = (t[:, 0] - t0) / 100.0  # 100 MHz clock -> us
        end = (t[:, 1] - t0) / 100.0
        kind = t[:, 3]
        span = float(end.max())
        bins = np.arange(0.0, span + 10.0, 10.0)
        rec = {"span_us": span, "kinds": {}}
        for kd in np.unique(kind):
            sel = kind == kd
            dur = end[sel] - start[sel]
            rec["kinds"][names.get(int(kd), str(kd))] = {
                "count": int(sel.sum()), "dur_us_mean": float(dur.mean()), "dur_us_p50": float(np.median(dur)),
                "dur_us_max": float(dur.max()), "first_start_us": float(start[sel].min()),
                "last_start_us": float(start[sel].max()), "last_end_us": float(end[sel].max()),
                "active_per_10us": [int(((start[sel] < b + 10.0) & (end[sel] > b)).sum()) for b in bins]}
        xcc = (t[:, 2] >> 32) & 0xF
        rec["xcd"] = [{"units": int((xcc == x).sum()), "last_end_us": float(end[xcc == x].max()),
                       "unit_us": float((end - start)[xcc == x].sum())} for x in range(8) if (xcc == x).any()]
        rate = np.zeros(len(bins))
        for u in np.where((kind_of == 1) & (end > start))[0]:
            r = mv_tokens[u] * tok_bytes / (end[u] - start[u])  # bytes per us
            lo, hi = start[u], end[u]
            for j in range(int(lo // 10), min(int(hi // 10) + 1, len(bins))):
                rate[j] += r * max(0.0, min(hi, bins[j] + 10.0) - max(lo, bins[j])) / 10.0
        rec["matvec_TBps_per_10us_estimate"] = [round(float(x) / 1e6, 3) for x in rate]
        res["launches"].append(rec)
        log(f"trace launch {li}: span {span:.1f} us; XCD last ends "
            + " ".join(f"{x['last_end_us']:.0f}" for x in rec["xcd"]))
        for name, r in rec["kinds"].items():
            log(f"  {name}: n={r['count']} dur mean {r['dur_us_mean']:.1f} us max {r['dur_us_max']:.1f}, "
                f"starts {r['first_start_us']:.1f}..{r['last_start_us']:.1f}, last end {r['last_end_us']:.1f} us")
        log("  mat-vec TB/s per 10 us (estimate): " + " ".join(f"{x:.1f}" for x in rec["matvec_TBps_per_10us_estimate"]))
    with open(path, "w") as f:
        json.dump(res, f)


def tiles_in_fused(P, plan, q, k, v, out, ws, flush, sink, info, wl, launches=3):
    """MFMA utilisation of the prefix tiles inside the fused launch: traced
    launches (psa_decode_attention_traced, caches flushed before each) give
    each MFMA tile unit's start, end and CU; the tiles' algorithmic flops
    (4 d per row and prefix token) over the time each CU is busy with tiles
    (union of its tiles' intervals) at the CU's share of the dense bf16
    peak.  Median over the launches."""
    import numpy as np
    import torch

    units = int(info["num_items"])
    it = np.asarray(plan.items()).reshape(units, 4, 8)
    tile = (it[:, 0, 0] & 0xFF) == 2
    flops_u = np.where(tile, 4.0 * wl.head_dim * it[:, 0, 7].astype(np.float64) * (it[:, 0, 4] - it[:, 0, 3]), 0.0)
    per_cu_peak = BF16_MFMA_PEAK_TFLOPS * 1e12 / 256
    fr, busy_l, cus_l, span_l = [], [], [], []
    for _ in range(launches):
        tr = torch.zeros(units * 4, dtype=torch.int64, device="cuda")
        if flush is not None:
            torch.sum(flush, dim=None, out=sink)
        P.psa_decode_attention(plan, q, k, v, out, ws, trace=tr)
        torch.cuda.synchronize()
        t = tr.view(units, 4).cpu().numpy()
        if not ((t[:, 0] > 0) & (t[:, 1] >= t[:, 0])).all():
            continue
        start, end = t[:, 0] / 100.0, t[:, 1] / 100.0  # 100 MHz clock -> us
        cu = ((t[:, 2] >> 32) & 0xF) * 256 + ((t[:, 2] >> 8) & 0xFF)  # XCC, then SE / SH / CU of HW_ID
        busy = 0.0
        ids = np.unique(cu[tile])
        for c in ids:  # union of the tile intervals on each CU
            iv = sorted(zip(start[tile & (cu == c)], end[tile & (cu == c)]))
            lo, hi = iv[0]
            for a, b in iv[1:]:
                if a > hi:
                    busy += hi - lo
                    lo, hi = a, b
                else:
                    hi = max(hi, b)
            busy += hi - lo
        fr.append(flops_u.sum() / (busy * 1e-6 * per_cu_peak))
        busy_l.append(busy)
        cus_l.append(len(ids))
        span_l.append(float(end[tile].max() - start.min()))
    if not fr:
        return None
    j = int(np.argsort(fr)[len(fr) // 2])
    return {"mfma_frac_on_their_cus": fr[j], "tile_flops": float(flops_u.sum()), "cus": cus_l[j],
            "cu_busy_us_sum": busy_l[j], "tiles_end_us": span_l[j], "launches": len(fr),
            "note": "prefix tiles' flops (4 d x rows x chunk tokens of every tile; keys masked by a prefill row's "
                    "causal limit included) over (time each CU runs tiles x the CU's 1/256 share of the 2.5 PFLOP/s "
                    "dense bf16 peak), from traced fused launches; median launch"}


def timed(fn, steps, flush, sink):
    """Mean ms of fn() over `steps` runs, HIP events around each run, caches
    flushed (by a read) before each."""
    import numpy as np
    import torch

    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            torch.sum(flush, dim=None, out=sink)
        evs[i][0].record()
        fn()
        evs[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def measured_peaks(P, buf, reps):
    """Measured ceilings of this GPU (psa_debug_read_peak / psa_debug_mfma_peak):
    the best of `reps` launches of a 1 GiB streaming read, and of a dependent
    bf16 MFMA run at eight waves per CU."""
    import torch

    sink = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    fout = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    nbytes = buf.numel() * buf.element_size()
    iters = 4096
    flops = 0.0

    def rd():
        P.psa_debug_read_peak(buf, sink)

    def mf():
        nonlocal flops
        flops = P.psa_debug_mfma_peak(fout, iters)

    best = {}
    for name, fn in (("read", rd), ("mfma", mf)):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        best[name] = min(ts)
    return {"hbm_read_GBps": nbytes / (best["read"] / 1e3) / 1e9, "read_bytes": nbytes,
            "mfma_bf16_TFLOPs": flops / (best["mfma"] / 1e3) / 1e12,
            "issue_cycles": issue_rates(P),
            "note": "best of %d launches each: a non-temporal 16-byte-load read of %d MiB (one contiguous span per workgroup), and 2048x4 waves of "
                    "%d dependent v_mfma_f32_16x16x32_bf16" % (reps, nbytes >> 20, iters)}


def issue_rates(P, iters=1024):
    """Core-clock cycles one wave (alone on its SIMD) spends per instruction of
    each issue-probe pattern (psa_debug_issue_probe; median over all waves of
    the second of two launches; pattern 7 per MFMA with its share of softmax
    work)."""
    import torch

    cyc = torch.empty(1024, dtype=torch.int64, device="cuda")
    row = {}
    for pat, (name, per_iter) in P.ISSUE_PATTERNS.items():
        P.psa_debug_issue_probe(pat, cyc, iters)
        P.psa_debug_issue_probe(pat, cyc, iters)
        torch.cuda.synchronize()
        row[name] = round(float(cyc.double().median()) / (iters * per_iter), 2)
    return row


def components(P, cfg, batch, wl, q, k, v, flush, sink, steps, fused_ms, peaks=None):
    """The fused launch's two halves alone, and the unfused structure the pages
    describe as prior work: a prefix launch, a distinct launch and a merge
    launch (three launches, partials through HBM)."""
    import torch

    n = len(batch["query_group"])
    res = {}
    parts = {}
    for name, flag in (("prefix_only", P.PREFIX_ONLY), ("distinct_only", P.DISTINCT_ONLY)):
        plan = P.psa_build_plan(cfg, batch, flags=flag)
        info = plan.info()
        ws = torch.empty(max(int(info["workspace_bytes"]), 256), dtype=torch.uint8, device="cuda")
        P.psa_plan_upload(plan, ws)
        o = torch.empty((n, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
        m = torch.empty((n, wl.num_q_heads), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        torch.cuda.synchronize()
        parts[name] = (plan, ws, o, m, l, info)
        ms = timed(lambda: P.psa_decode_attention(plan, q, k, v, o, ws, m, l), steps, flush, sink)
        rec = {"ms": ms}
        if name == "prefix_only":
            tf = info["prefix_flops"] / (ms / 1e3) / 1e12
            if peaks:
                rec["mfma_frac_of_measured"] = tf / peaks["mfma_bf16_TFLOPs"]
            rec.update({"prefix_tflops": tf, "mfma_peak_tflops": BF16_MFMA_PEAK_TFLOPS, "mfma_frac": tf / BF16_MFMA_PEAK_TFLOPS,
                        "note": "prefix flops (4 d Hq per attended prefix token) over the launch time; the launch "
                                "also writes the prefix partials"})
        else:
            gbps = info["distinct_kv_bytes"] / (ms / 1e3) / 1e9
            q_out = info["algorithmic_bytes"] - info["prefix_kv_bytes"] - info["distinct_kv_bytes"]
            alg = (info["distinct_kv_bytes"] + q_out) / (ms / 1e3) / 1e9  # distinct KV + q + out
            rec.update({"distinct_kv_GBps": gbps, "algorithmic_GBps": alg, "hbm_frac": alg / HBM_PEAK_GBPS})
            if peaks:
                rec["hbm_frac_of_measured_read"] = alg / peaks["hbm_read_GBps"]
        res[name] = rec
    (pa, wa, oa, ma, la, _), (pb, wb, ob, mb, lb, _) = parts["prefix_only"], parts["distinct_only"]
    o = torch.empty_like(oa)
    m = torch.empty_like(ma)
    l = torch.empty_like(la)
    d = wl.head_dim

    def unfused():
        P.psa_decode_attention(pa, q, k, v, oa, wa, ma, la)
        P.psa_decode_attention(pb, q, k, v, ob, wb, mb, lb)
        P.psa_merge(oa.view(-1, d), ma.view(-1), la.view(-1), ob.view(-1, d), mb.view(-1), lb.view(-1),
                    o.view(-1, d), m.view(-1), l.view(-1))

    ms = timed(unfused, steps, flush, sink)
    res["unfused_3_launches"] = {"ms": ms, "fused_speedup": ms / fused_ms}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_8x100",
                    help="a preset of workloads/synth.py, or 'all': one JSON line per preset")
    ap.add_argument("--no-flush", action="store_true", help="do not flush L2/MALL between steps")
    ap.add_argument("--write-flush", action="store_true",
                    help="flush by writing 1 GiB (leaves dirty lines) instead of reading it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--flags", type=int, default=0, help="psa_plan flags (e.g. 1 = PREFIX_ONLY)")
    ap.add_argument("--prefix-chunk", type=int, default=0)
    ap.add_argument("--distinct-chunk", type=int, default=0)
    ap.add_argument("--tile-rows", type=int, default=0)
    ap.add_argument("--json-out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--trace", default=None,
                    help="after timing, run one traced launch and write its per-unit timeline summary (JSON) here")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured read / MFMA ceilings")
    ap.add_argument("--no-identify", action="store_true",
                    help="skip timing the host prefix identification (token ids -> groups)")
    ap.add_argument("--no-components", action="store_true",
                    help="skip the prefix-only / distinct-only / unfused three-launch measurements")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the prefix-shared decode path shards by prefix group or kv head with no exchange "
              "between GPUs", file=sys.stderr)
        sys.exit(2)

    if args.workload == "all":
        from workloads import PRESETS

        for name in PRESETS:
            args.workload = name
            run_one(args)
        return
    run_one(args)


def run_one(args):
    """Time one workload and print its JSON line."""
    import numpy as np
    import torch

    import prefix_shared_decode_amd as P
    from workloads import make_values, make_workload

    torch.cuda.set_device(0)
    wl = make_workload(args.workload)
    batch = wl.batch
    if wl.tree is not None:
        t0 = time.perf_counter()
        batch, saved = P.psa_flatten_prefix_tree(wl.tree)
        log(f"flattened two-level tree in {1e3 * (time.perf_counter() - t0):.1f} ms (saved tokens {saved})")
    log(f"workload {wl.name}: generating inputs on the GPU")
    q, k, v = make_values(wl, "cuda")
    cfg = P.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.dtype, "f32")
    t0 = time.perf_counter()
    plan = P.psa_build_plan(cfg, batch, flags=args.flags, prefix_chunk_tokens=args.prefix_chunk,
                            distinct_chunk_tokens=args.distinct_chunk, mfma_tile_rows=args.tile_rows)
    plan_ms = 1e3 * (time.perf_counter() - t0)
    info = plan.info()
    ws = torch.empty(max(int(info["workspace_bytes"]), 256), dtype=torch.uint8, device="cuda")
    P.psa_plan_upload(plan, ws)
    torch.cuda.synchronize()
    n = len(batch["query_group"])
    out = torch.empty((n, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    log(f"plan: {info['num_items']} items ({info['num_prefix_items']} MFMA prefix, {info['num_matvec_items']} "
        f"mat-vec), workspace {info['workspace_bytes'] / 2**20:.1f} MiB, built in {plan_ms:.1f} ms")

    def step():
        P.psa_decode_attention(plan, q, k, v, out, ws)

    flush = None if args.no_flush else torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    if args.copy_calib_mib > 0:
        # a plain copy kernel of known size: reads and writes exactly this many bytes
        src = torch.ones(args.copy_calib_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            if args.write_flush:
                flush.fill_(float(i))
            else:
                torch.sum(flush, dim=None, out=sink)
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    times_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms = float(times_ms.mean())
    sec = ms / 1e3
    # bytes the method must stream: KV over distinct (page, slot) places, q, out.  This is the
    # single-level definition (prefix once per group) except where groups' prefixes name the same
    # pages (a flattened tree's shared root), which count once.
    kv_alg = info["prefix_kv_bytes"] + info["distinct_kv_bytes"]
    bytes_single_level = info["algorithmic_bytes"]
    bytes_alg = bytes_single_level - kv_alg + info["unique_kv_bytes"]
    if args.flags & P.DISTINCT_ONLY:  # a distinct-only plan streams the distinct KV, q and out
        bytes_alg = bytes_single_level - info["prefix_kv_bytes"]
    achieved = bytes_alg / sec / 1e9
    traffic = load_traffic(wl.name, bytes_alg)
    rec = {
        "metric": METRIC,
        "value": n / sec,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled pages)",
        "config": describe(wl, batch),
        "effective_kv_GBps": kv_alg / sec / 1e9,
        "hbm_roofline_frac": achieved / HBM_PEAK_GBPS,
        "ms_p10_p50_p90": [float(np.percentile(times_ms, p)) for p in (10, 50, 90)],
        "timing": "HIP events around each launch on its stream; L2+MALL flushed before each step"
                  if flush is not None else "HIP events around each launch; caches warm",
        "timed_region_wall_s": t_wall,
        "plan": {"build_ms": plan_ms, "items": info["num_items"], "mfma_prefix_items": info["num_prefix_items"],
                 "matvec_items": info["num_matvec_items"], "flags": args.flags,
                 "saved_tokens": info["saved_tokens"], "logical_tokens": info["logical_tokens"]},
        "roofline": {
            "kernel": "psa::decode_kernel<128,4,true> (fused prefix MFMA + distinct mat-vec + merge)"
            if wl.num_q_heads // wl.num_kv_heads == 4 else "psa::decode_kernel (fused)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": bytes_alg,
            "single_level_bytes_per_launch": bytes_single_level,
            "traffic": traffic,
        },
    }
    if info["prefix_flops"] > 0:
        rec["roofline"]["prefix_flops_per_launch"] = info["prefix_flops"]
    if args.flags & P.PREFIX_ONLY:  # the prefix tiles alone: matrix-core bound
        tf = info["prefix_flops"] / sec / 1e12
        rec["roofline"].update({"bound": "mfma", "achieved": tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": tf / BF16_MFMA_PEAK_TFLOPS})
        rec["hbm_roofline_frac"] = None
    if not args.no_peaks and flush is not None:
        rec["measured_peaks"] = measured_peaks(P, flush, max(5, args.steps // 5))
        mp = rec["measured_peaks"]
        if args.flags & P.PREFIX_ONLY:
            rec["roofline"]["frac_of_measured_mfma_peak"] = rec["roofline"]["achieved"] / mp["mfma_bf16_TFLOPs"]
        else:
            rec["roofline"]["frac_of_measured_read_peak"] = achieved / mp["hbm_read_GBps"]
    if not args.no_components and args.flags == 0 and info["num_prefix_items"] > 0:
        rec["components"] = components(P, cfg, batch, wl, q, k, v, flush, sink, max(10, args.steps // 2), ms,
                                       rec.get("measured_peaks"))
        rec["components"]["prefix_tiles_in_fused"] = tiles_in_fused(P, plan, q, k, v, out, ws, flush, sink, info, wl)
    if not args.no_identify and wl.name == "llama3_8b_8x100":
        rec["host_prefix_identification"] = host_identification(P)
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the fp64 oracle on a sample")
        rec["cpu_baseline"] = cpu_baseline(wl, batch, q, k, v, args.cpu_seconds, 30.0)
    if args.trace:
        trace_summary(P, plan, q, k, v, out, ws, flush, sink, info, args.trace, wl)
    rec["context"] = {
        "note": "figures quoted by the pages; end-to-end serving speedups on other hardware, not measurements "
                "of this kernel, so no vs_baseline is derived from them",
        "batchllm_end_to_end_vs_vllm_sglang": "1.3x-10.8x (NVIDIA A100 80GB and AMD MI200)",
        "feather_scheduler_end_to_end": "2x-10x (NVIDIA RTX 6000 Ada, A100)",
    }
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
