#!/usr/bin/env python3
"""Benchmark of the factored recurrent-state decode path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic inputs:
decode_step on every state (decay, append, read after update, delta rule
where configured) followed by the compaction of the groups the staggered
schedule makes due (Brand update, truncation, re-split, dense promotion).

Default workload: 258,048 Mamba-2-shaped states (128 requests x 21 layers x
96 heads, d_k = 128, d_v = 80, fp32), rank-8 start, 4 stagger groups, the
whole 1,024-step job.  Inputs are generated on the GPU in chunks before each
timed chunk (not timed).  W warmup steps first run on a scratch pool of the
same workload.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
# plain (non-packed) fp32 VALU ceiling of the compaction: 256 CUs x 4 SIMDs x 16 lanes x 2 flops per
# FMA x 2.4 GHz = 78.6 TFLOP/s (the published 157.3 counts packed fp32 instructions, which this
# library does not use)
FP32_VALU_PEAK_TFLOPS = 78.6
METRIC = "state-steps/sec and achieved HBM GB/s (% peak) for decode_step, 258k states"


def _pool(ss, w, init, **kw):
    return ss.state_pool_create(w.n_states, w.d_k, w.d_v, w.K, w.r, group_of_state=init["group_of_state"],
                                group_offset=init["group_offset"], rule=init["rule"], eps=init["eps"],
                                comp_off=init["comp_off"], u=init["u"], v=init["v"], sigma=init["sigma"],
                                diag_decay=w.diag_decay, **kw)


ASYNC_LOG = {}  # poll results (and launches) of the asynchronous consolidation, per step


def _run_steps(ss, torch, pool, xs, t0, o, ev=None, cons=(0, 1), side=None):
    """Run len(xs) steps starting after step t0; optional per-step events.  cons = (groups, period):
    every `period` steps, consolidate up to `groups` groups from the wait queue after the compactions.
    side: a second stream for the asynchronous consolidation (or "host" for the host-core form):
    after each step's compactions the finished result is installed (or dropped when stale) and the
    next group from the queue starts."""
    for i, x in enumerate(xs):
        t = t0 + i + 1
        if ev is not None:
            ev[i].record()
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        for g in ss.schedule_due(pool, t):
            ss.compact(pool, g)
        if side is not None:
            st = ss.consolidate_poll(pool)
            ASYNC_LOG[st] = ASYNC_LOG.get(st, 0) + 1
            if st != ss.CONS_RUNNING and (ss.consolidate_host(pool) if side == "host"
                                          else ss.consolidate_async(pool, side)) >= 0:
                ASYNC_LOG["launched"] = ASYNC_LOG.get("launched", 0) + 1
        elif cons[0] > 0 and t % cons[1] == 0:
            ss.consolidate_next(pool, cons[0])
    if ev is not None:
        ev[len(xs)].record()


def graph_replay(ss, torch, W, steps=256, warm=16):
    """Per-step wall time of whole steps (decode + due compactions) launched eagerly versus replayed
    as step graphs, at batch sizes where launch overhead matters.  Inputs sit in fixed buffers and
    are refreshed every step on the device (same work on both paths)."""
    import time as _t
    out = {}
    for name, req in (("tiny", None), ("mamba2_258k", 1)):
        w = W.get(name, n_requests=req)
        init = W.initial_state(w)
        gen = W.StepInputs(w, device="cuda")
        xs = [gen.generate(t) for t in range(1, 9)]
        buf = {k: v.clone() for k, v in xs[0].items()}
        o = torch.empty(w.n_states, w.d_v, device="cuda")
        res = {}
        for mode in ("eager", "graph"):
            pool = _pool(ss, w, init)
            g = ss.StepGraph(pool, buf["q"], buf["k"], buf["v"], buf["alpha"], buf["beta"], o) if mode == "graph" \
                else None
            t0 = None
            for t in range(1, warm + steps + 1):
                if t == warm + 1:
                    torch.cuda.synchronize()
                    t0 = _t.perf_counter()
                x = xs[t % len(xs)]
                for k in buf:
                    buf[k].copy_(x[k])
                if g is not None:
                    g.launch(t)
                else:
                    ss.decode_step(pool, buf["q"], buf["k"], buf["v"], buf["alpha"], buf["beta"], o)
                    for gg in ss.schedule_due(pool, t):
                        ss.compact(pool, gg)
            torch.cuda.synchronize()
            res[mode] = 1e6 * (_t.perf_counter() - t0) / steps
            if g is not None:
                g.close()
            pool.close()
        out[name] = {"n_states": w.n_states, "eager_us_per_step": res["eager"], "graph_us_per_step": res["graph"],
                     "speedup": res["eager"] / res["graph"]}
    return out


def rsvd_init_rate(ss, torch, n=32768, d_k=128, d_v=80, b=8, nb=7, iters=2, eps=3e-3, seed=20261202):
    """Randomized block SVD initialization of prefill-like dense states (a spectrum decaying as
    0.6^i over 24 random directions plus 1e-4 noise) on the GPU.  Algorithmic flops per block:
    (4 iters + 2) d_k d_v b for the products with the state and the subtraction, plus the QRs."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    r = 24
    A = torch.randn(n, d_k, r, device="cuda", generator=g) * (0.6 ** torch.arange(r, device="cuda"))
    B = torch.randn(n, d_v, r, device="cuda", generator=g)
    S = torch.bmm(A, B.transpose(1, 2).contiguous()) / r ** 0.5
    S += 1e-4 * torch.randn(n, d_k, d_v, device="cuda", generator=g)
    om = torch.randn(n, nb, d_k, b, device="cuda", generator=g)
    del A, B
    ss.rsvd_init(S[:64].contiguous(), om[:64].contiguous(), eps, iters=iters)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    u, v, sg, rk = ss.rsvd_init(S, om, eps, iters=iters)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    rk = rk.double()
    blocks = torch.clamp(torch.floor(rk / b) + 1, max=nb)
    per_block = (4 * iters + 2) * d_k * d_v * b + iters * 4 * d_v * b * b + 4 * d_k * b * b + 2 * (d_k + d_v) * b * b
    flops = float(blocks.sum().item()) * per_block
    return {"n_states": n, "shape": [d_k, d_v], "block": b, "iters": iters, "ms": ms,
            "states_per_s": n / (ms / 1e3), "mean_rank": float(rk.mean().item()),
            "algorithmic_TFLOPs": flops / (ms / 1e3) / 1e12, "fp32_peak_TFLOPs": 157.3}


def cpu_baseline(w, init, n_sample, n_steps, device="cpu"):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload, all host cores.
    Inputs are drawn per step for the sampled states on `device` and copied to the host (not timed);
    only the oracle calls are timed."""
    import numpy as np
    from oracle import OraclePool, schedule_due
    from oracle.oracle import OracleState, max_threads
    from rank_recurrent_state_amd import workloads as W

    rng = np.random.default_rng(7)
    ids = np.sort(rng.choice(w.n_states, size=min(n_sample, w.n_states), replace=False))
    P = OraclePool(len(ids), w.d_k, w.d_v, w.K, w.r, -1, True, diag_decay=w.diag_decay)
    off = init["comp_off"]
    for j, s in enumerate(ids):
        a, b = off[s], off[s + 1]
        P.set_state(j, OracleState(init["u"][a:b].astype(np.float64), init["v"][a:b].astype(np.float64),
                                   init["sigma"][a:b].astype(np.float64), rule=int(init["rule"][s]),
                                   eps=float(init["eps"][s])))
    gen = W.StepInputs(w, device=device)
    grp = init["group_of_state"][ids]
    nthreads = max_threads()
    t_dec = t_cmp = 0.0
    for t in range(1, n_steps + 1):
        x = {k: v.cpu().numpy().astype(np.float64) for k, v in gen.generate(t, states=ids).items()}
        a = time.perf_counter()
        P.decode(x["q"], x["k"], x["v"], x["alpha"], x["beta"], nthreads=nthreads)
        b = time.perf_counter()
        due = schedule_due(t, w.K, init["group_offset"])
        if due:
            P.compact(np.nonzero(np.isin(grp, due))[0], nthreads=nthreads)
        t_dec += b - a
        t_cmp += time.perf_counter() - b
    tot = t_dec + t_cmp
    return {"value": len(ids) * n_steps / tot, "unit": "state-steps/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{len(ids)} states drawn from the same {w.n_states}-state workload, steps 1-{n_steps} "
                      f"(decode + staggered compaction + promotion), fp64, OpenMP over states",
            "decode_state_steps_per_s": len(ids) * n_steps / t_dec, "seconds": tot,
            "cpu": _cpu_model()}


def copy_calibration(gib=4, reps=5):
    """A plain device-to-device copy of known size, for scaling HBM byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                      "reps": reps}), flush=True)


def _traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the decode
    kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in ("ss_decode.hip", "ss_internal.h", "ss_wave.h"):
        h.update(open(os.path.join(ROOT, "rank_recurrent_state_amd", "csrc", f), "rb").read())
    if rec.get("kernel") != kernel or rec.get("decode_source_sha256") != h.hexdigest():
        return None
    return rec["traffic_bytes_per_launch"]


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: the workload's job length)")
    ap.add_argument("--warmup", type=int, default=16, help="untimed steps on a scratch pool first")
    ap.add_argument("--workload", default="mamba2_258k")
    ap.add_argument("--requests", type=int, default=None, help="override the number of requests")
    ap.add_argument("--chunk", type=int, default=64, help="steps whose inputs are generated at once")
    ap.add_argument("--dense-steps", type=int, default=64, help="steps of the dense HIP baseline (0: skip)")
    ap.add_argument("--cpu-sample", type=int, default=131072)
    ap.add_argument("--cpu-steps", type=int, default=64)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 4 GiB device copy (for scaling rocprof byte counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--consolidate", type=int, default=0,
                    help="groups consolidated from the wait queue after a step's compactions (0: off)")
    ap.add_argument("--consolidate-period", type=int, default=1, help="steps between consolidation calls")
    ap.add_argument("--consolidate-host", action="store_true",
                    help="consolidate frozen parts on host cores beside the decode (download, fp64 SVD, upload)")
    ap.add_argument("--consolidate-async", action="store_true",
                    help="consolidate on a second stream, one group at a time from the wait queue, beside the decode")
    ap.add_argument("--stagger", default=None, choices=["none", "even4", "paper8", "state8"],
                    help="override the workload's compaction stagger (the per-step latency comparison)")
    ap.add_argument("--factor-fp16", action="store_true",
                    help="store the factor vectors in fp16 (pad, sigma, dense region and arithmetic stay fp32)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the eager-versus-graph step timing and the initialization timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "single-GPU implementation: --gpus must be 1 (the path shards by request "
                                   "with no exchange step between GPUs)"}))
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch
    from rank_recurrent_state_amd import sinkstate as ss
    from rank_recurrent_state_amd import workloads as W

    torch.cuda.set_device(0)
    w = W.get(args.workload, n_requests=args.requests)
    if args.stagger is not None:
        import dataclasses
        w = dataclasses.replace(w, stagger=args.stagger)
    K_steps = args.steps if args.steps is not None else w.steps
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    log(f"[bench] workload {w.name}: {w.n_states} states {w.d_k}x{w.d_v}, {K_steps} timed steps")
    t_init = time.time()
    init = W.initial_state(w)
    log(f"[bench] initial states built in {time.time() - t_init:.1f}s")
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")

    cons = (max(0, args.consolidate), max(1, args.consolidate_period))
    side = "host" if args.consolidate_host else torch.cuda.Stream() if args.consolidate_async else None  # default priority
    # warmup on a scratch pool of the same workload
    fkw = {"factor_fp16": True} if args.factor_fp16 else {}
    if args.warmup > 0:
        pool = _pool(ss, w, init, **fkw)
        wchunk = max(1, min(args.chunk, int(16e9 // (w.n_states * (2 * w.d_k + w.d_v + 2 + (w.d_k if w.diag_decay else 0)) * 4))))
        for c0 in range(0, args.warmup, wchunk):
            xs = [gen.generate(t) for t in range(c0 + 1, min(args.warmup, c0 + wchunk) + 1)]
            _run_steps(ss, torch, pool, xs, c0, o, cons=cons, side=side)
        if side is not None:
            ss.consolidate_poll(pool, wait=True)
        torch.cuda.synchronize()
        pool.close()
        del xs
        log(f"[bench] warmup {args.warmup} steps done")

    # the timed job
    ASYNC_LOG.clear()
    pool = _pool(ss, w, init, **fkw)
    st0 = ss.pool_stats(pool)
    ss.pool_timing(pool, True)
    step_ms = []
    hist_marks = {}
    t = 0
    # inputs of a chunk are generated at once: keep them within about 16 GB
    chunk = max(1, min(args.chunk, int(16e9 // (w.n_states * (2 * w.d_k + w.d_v + 2 + (w.d_k if w.diag_decay else 0)) * 4))))
    while t < K_steps:
        n = min(chunk, K_steps - t)
        xs = [gen.generate(s) for s in range(t + 1, t + n + 1)]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        _run_steps(ss, torch, pool, xs, t, o, ev, cons=cons, side=side)
        torch.cuda.synchronize()
        step_ms += [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
        t += n
        del xs
        st = ss.pool_stats(pool)
        hist_marks[t] = {"dense_fraction": st["n_dense"] / w.n_states,
                         "mean_rank_factored": (st["active_components"] + st["frozen_components"])
                         / max(1, st["n_factored"])}
        log(f"[bench] {t}/{K_steps} steps, dense fraction {hist_marks[t]['dense_fraction']:.3f}, "
            f"mean factored rank {hist_marks[t]['mean_rank_factored']:.1f}, "
            f"chunk {sum(step_ms[-n:]):.1f} ms")
    st1 = ss.pool_stats(pool)
    pool.close()
    total_ms = float(sum(step_ms))
    value = w.n_states * K_steps / (total_ms / 1e3)

    kms = {k: st1["kernel_ms"][k] - st0["kernel_ms"][k] for k in st1["kernel_ms"]}
    kn = {k: st1["kernel_launches"][k] - st0["kernel_launches"][k] for k in st1["kernel_launches"]}
    bytes_k = {"decode_factored": st1["decode_bytes_factored"] - st0["decode_bytes_factored"],
               "decode_dense": st1["decode_bytes_dense"] - st0["decode_bytes_dense"]}
    decode_ms = kms["decode_factored"] + kms["decode_dense"]
    decode_bytes = bytes_k["decode_factored"] + bytes_k["decode_dense"]
    dom = max(("decode_factored", "decode_dense"), key=lambda k: kms[k])
    ach = bytes_k[dom] / (kms[dom] / 1e3) / 1e9 if kms[dom] > 0 else 0.0
    per_kernel = {}
    for k in ("decode_factored", "decode_dense"):
        if kn[k]:
            gbs = bytes_k[k] / (kms[k] / 1e3) / 1e9
            per_kernel[k] = {"launches": kn[k], "avg_us": 1e3 * kms[k] / kn[k], "bytes_per_launch": bytes_k[k] / kn[k],
                             "achieved_GBs": gbs, "frac": gbs / HBM_PEAK_GBS}
    cflops = st1["compact_flops"] - st0["compact_flops"]
    cstates = st1["compact_states"] - st0["compact_states"]
    compaction = {"launches": kn["compact"], "ms_total": kms["compact"], "states": cstates,
                  "states_per_s": cstates / (kms["compact"] / 1e3) if kms["compact"] else None,
                  "algorithmic_TFLOPs": cflops / (kms["compact"] / 1e3) / 1e12 if kms["compact"] else None,
                  "materialize_ms_total": kms["materialize"], "promotions": st1["promotions"] - st0["promotions"]}
    consolidation = None
    if cons[0] > 0 or side is not None:
        xf = st1["consolidate_flops"] - st0["consolidate_flops"]
        alog = {"launched": ASYNC_LOG.get("launched", 0), "steps_running": ASYNC_LOG.get(ss.CONS_RUNNING, 0),
                "installed": ASYNC_LOG.get(ss.CONS_INSTALLED, 0), "discarded": ASYNC_LOG.get(ss.CONS_DISCARDED, 0)}
        consolidation = {"mode": "host cores (download, fp64 SVD, upload)" if side == "host" else
                         "async (second stream)" if side is not None else "in the step",
                         "async_polls": alog if side is not None else None,
                         "groups_per_call": cons[0], "period": cons[1], "launches": kn["consolidate"],
                         "live_bytes_end": st1["live_bytes"], "n_dense_end": st1["n_dense"],
                         "ms_total": kms["consolidate"], "states": st1["consolidate_states"] - st0["consolidate_states"],
                         "removed_components": st1["consolidate_removed"] - st0["consolidate_removed"],
                         "algorithmic_TFLOPs": xf / (kms["consolidate"] / 1e3) / 1e12 if kms["consolidate"] else None,
                         "frozen_components_end": st1["frozen_components"],
                         "active_components_end": st1["active_components"]}
    sm = np.array(step_ms)
    first = min(64, K_steps)
    phases = {"steps_1_%d_ms_per_step" % first: float(sm[:first].mean()),
              "steps_%d_%d_ms_per_step" % (first + 1, K_steps): float(sm[first:].mean()) if K_steps > first else None,
              "p50_step_ms": float(np.percentile(sm, 50)), "p99_step_ms": float(np.percentile(sm, 99)),
              "state_mix": hist_marks}

    # dense HIP baseline on the same inputs
    dense = None
    if args.dense_steps > 0:
        args.dense_steps = min(args.dense_steps, chunk)  # its inputs are generated at once too
        dp = _pool(ss, w, init, force_dense=True)
        xs = [gen.generate(s) for s in range(1, args.dense_steps + 1)]
        ss.pool_timing(dp, True)
        s0 = ss.pool_stats(dp)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for x in xs:
            ss.decode_step(dp, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        e1.record()
        torch.cuda.synchronize()
        s1 = ss.pool_stats(dp)
        dp.close()
        del xs
        dms = e0.elapsed_time(e1)
        kd = s1["kernel_ms"]["decode_dense"] - s0["kernel_ms"]["decode_dense"]
        bd = s1["decode_bytes_dense"] - s0["decode_bytes_dense"]
        dense = {"value": w.n_states * args.dense_steps / (dms / 1e3), "unit": "state-steps/s",
                 "ms_per_step": dms / args.dense_steps, "steps": args.dense_steps,
                 "achieved_GBs": bd / (kd / 1e3) / 1e9, "frac": bd / (kd / 1e3) / 1e9 / HBM_PEAK_GBS,
                 "kernel_avg_us": 1e3 * kd / args.dense_steps, "bytes_per_step": bd / args.dense_steps}
        log(f"[bench] dense baseline {dense['ms_per_step']:.3f} ms/step, {dense['achieved_GBs']:.0f} GB/s")

    graphs = graph_replay(ss, torch, W) if not args.no_graph else None
    init_rate = rsvd_init_rate(ss, torch) if not args.no_graph else None
    if init_rate:
        log(f"[bench] randomized SVD init: {init_rate['states_per_s']:.3e} states/s, "
            f"{init_rate['algorithmic_TFLOPs']:.1f} TFLOP/s, mean rank {init_rate['mean_rank']:.1f}")
    if graphs:
        log("[bench] graph replay " + ", ".join(f"{k}: {v['eager_us_per_step']:.0f} -> {v['graph_us_per_step']:.0f} us/step"
                                                for k, v in graphs.items()))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, init, args.cpu_sample, args.cpu_steps, device="cuda")
        log(f"[bench] cpu baseline {cpu['value']:.3e} state-steps/s on {cpu['cores']} threads ({cpu['seconds']:.1f}s)")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "state-steps/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / K_steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}; {w.n_requests} requests x {w.n_layers} layers x "
                               f"{w.n_heads} heads, K={w.K}, r={w.r}, stagger={w.stagger}, whole {K_steps}-step job",
                   "n_states": w.n_states, "d_k": w.d_k, "d_v": w.d_v,
                   "factor_storage": "fp16" if args.factor_fp16 else "fp32"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": _traffic(dom, w.name),
                     "algorithmic_bytes_per_launch": bytes_k[dom] / max(1, kn[dom])},
        "cpu_baseline": cpu,
        "decode_step": {"state_steps_per_s": w.n_states * K_steps / (decode_ms / 1e3) if decode_ms else None,
                        "achieved_GBs": decode_bytes / (decode_ms / 1e3) / 1e9 if decode_ms else None,
                        "kernels": per_kernel},
        "compaction": compaction,
        "compaction_roofline": {"bound": "valu", "kernel": "compact",
                                "achieved": compaction["algorithmic_TFLOPs"], "peak": FP32_VALU_PEAK_TFLOPS,
                                "unit": "TFLOP/s",
                                "frac": compaction["algorithmic_TFLOPs"] / FP32_VALU_PEAK_TFLOPS
                                if compaction["algorithmic_TFLOPs"] else None,
                                "flops_per_launch": cflops / kn["compact"] if kn["compact"] else None,
                                "share_of_step": kms["compact"] / total_ms if total_ms else None},
        "consolidation": consolidation,
        "frozen_components_end": st1["frozen_components"],
        "phases": phases,
        "dense_baseline": dense,
        "graph_replay": graphs,
        "rsvd_init": init_rate,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
