"""Throughput of the speculative verification + SAGUARO cache path on one GPU.

One step = one pass of the whole path over one batch: ssd_fanout (host),
then ssd_verify_round (the cache build on draft rows 0..K, verification
against sigma_{F,C}, the cache lookup: three launches). --separate runs the
same step as ssd_build_cache -> ssd_verify (sigma) -> ssd_cache_lookup (five
launches); both give bit-identical outputs, which the bench checks.
Default workload: B=64 sequences, K=5 drafted tokens, V=128256, bf16 logits,
tau=0.7, cache budget 64 split with a_p=0.8, r=1, C=0.5.

Inputs are resident in HBM before timing; ceil(512 MB / bytes) + 1
rotating copies (more than the 256 MB Infinity Cache holds) make each step
read its logits from HBM. The drafted tokens of the step are drawn on the GPU
from q_sigma (ssd_draft_sample) before timing, as the SAGUARO draft phase
does, so the acceptance and hit rates are those of the process the cache is
built for.
Each copy's step is captured once in a HIP graph and replayed. Timing uses
HIP events on the stream the library launches on.

Prints one JSON line (rank 0).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak, GB/s
ROTATE_BYTES = 512 << 20   # twice the 256 MB Infinity Cache


def n_copies(nbytes):
    """Rotating input copies so that consecutive steps never find their
    logits in the 256 MB Infinity Cache: ceil(512 MB / bytes) + 1."""
    return int(math.ceil(ROTATE_BYTES / nbytes)) + 1


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--workload", choices=["step", "tree", "greedy", "sample"], default="step",
                    help="step: the verification + cache step (default); tree: token-tree verification; "
                         "greedy: greedy verification; sample: sigma-aware draft sampling")
    ap.add_argument("--report", default=None,
                    help="per-workload measurement report instead of the bench line: comma-separated "
                         "workload numbers 1-5 (5 runs at tau 0.5 and 1.0), or 'all'; one JSON line each")
    ap.add_argument("--calls", type=int, default=120, help="timed calls per workload in --report")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--separate", action="store_true",
                    help="run the step as three calls (ssd_build_cache, ssd_verify, ssd_cache_lookup) instead of "
                         "the fused ssd_verify_round")
    ap.add_argument("--profile-loop", type=int, default=0,
                    help="after the bench, run this many extra eager steps (for profilers)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 256 MiB read + 256 MiB write elementwise kernel (torch.neg on "
                         "bf16) three times: the known-size reference that scales hardware byte counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every batch row is independent, so more GPUs would each run this same "
              "kernel on B/N rows)", file=sys.stderr)
        sys.exit(2)

    if args.report:
        return bench_report(args)
    if args.workload == "tree":
        return bench_tree(args)
    if args.workload in ("greedy", "sample"):
        return bench_rows(args)

    import torch
    import verify_speculation_cache_amd as S
    import workloads as W

    cfg = W.get_config(args.config)
    if not cfg.has_cache:   # the cache build reads draft row K and needs cache parameters
        raise SystemExit("bench workload needs cache parameters (use --config 2, 3 or 5)")
    B, K, V = cfg.B, cfg.K, cfg.V
    tau = cfg.taus[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy:
        src = torch.ones(128 << 20, dtype=torch.bfloat16, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    t0 = time.time()
    d = W.make_inputs(cfg, tau=tau)
    gen_s = time.time() - t0

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    tgt0, dft0 = up(d["target"]), up(d["draft"][:, :K + 1])
    step_bytes = tgt0.numel() * tgt0.element_size() + dft0.numel() * dft0.element_size()
    ncopy = n_copies(step_bytes)
    tgts = [tgt0] + [tgt0.clone() for _ in range(ncopy - 1)]
    dfts = [dft0] + [dft0.clone() for _ in range(ncopy - 1)]
    ua = torch.from_numpy(d["u_acc"]).to(dev)
    ur = torch.from_numpy(d["u_res"]).to(dev)
    F = S.ssd_fanout(cfg.n_budget, K, cfg.a_p, cfg.r)
    C = cfg.C
    # the draft phase: d_{i+1} ~ sigma_{F_i,C}(draft row i / tau), on the GPU
    u_draft_np = W.make_draft_uniforms(cfg, tau)
    cache_d = S.ssd_build_cache(dfts[0], tau, F)
    toks = S.ssd_draft_sample(dfts[0], torch.from_numpy(u_draft_np).to(dev), tau, S.sigma_from_cache(cache_d, C))
    toks_plain = torch.from_numpy(d["tokens"]).to(dev)   # softmax drafts for plain verification
    torch.cuda.synchronize()
    toks_np = toks.cpu().numpy()

    outs = []
    for j in range(ncopy):
        cache = S.ssd_build_cache(dfts[j], tau, F)
        res = S.ssd_verify(tgts[j], dfts[j], toks, ua, ur, tau, S.sigma_from_cache(cache, C))
        look = S.ssd_cache_lookup(cache["cache_tokens"], F, res["accepted"], res["out_tokens"])
        outs.append((cache, res, look))
    torch.cuda.synchronize()

    rounds = [S.ssd_verify_round(tgts[j], dfts[j], F, C, toks, ua, ur, tau) for j in range(ncopy)]
    torch.cuda.synchronize()
    # the fused round builds the same cache bit for bit; its verification sums
    # rows over other chunk partials, so an outcome may differ from the three
    # calls' only where a decision is within rounding of its threshold
    round_rows_differ = 0
    for j in range(ncopy):
        cache, res, look = outs[j]
        for k, v in (("cache_tokens", cache["cache_tokens"]), ("draft_stats", cache["draft_stats"]),
                     ("thr", cache["thr"])):
            assert torch.equal(rounds[j][k], v), k
        same = ((rounds[j]["accepted"] == res["accepted"]) & (rounds[j]["out_tokens"] == res["out_tokens"]).all(1)
                & (rounds[j]["hit"] == look["hit"]))
        round_rows_differ += int((~same).sum().item())
    sep_ref = [(o[1]["accepted"].clone(), o[1]["out_tokens"].clone(), o[2]["hit"].clone()) for o in outs]
    round_ref = [(r["accepted"].clone(), r["out_tokens"].clone(), r["hit"].clone()) for r in rounds]

    def step(j):
        if not args.separate:
            S.ssd_verify_round(tgts[j], dfts[j], F, C, toks, ua, ur, tau, out=rounds[j])
            return
        cache, res, look = outs[j]
        S.ssd_build_cache(dfts[j], tau, F, out=cache)
        S.ssd_verify(tgts[j], dfts[j], toks, ua, ur, tau, S.sigma_from_cache(cache, C), out=res)
        S.ssd_cache_lookup(cache["cache_tokens"], F, res["accepted"], res["out_tokens"], out=look)

    def host_row(j):
        F_host = S.ssd_fanout(cfg.n_budget, K, cfg.a_p, cfg.r)   # host row of the step
        assert F_host == F

    run = _replay_runner(step, ncopy, args, per_step=host_row)

    run(args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run(args.steps, args.warmup)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # replays must reproduce the eager outputs
    for j in range(ncopy):
        if args.separate:
            got = (outs[j][1]["accepted"], outs[j][1]["out_tokens"], outs[j][2]["hit"])
            want = sep_ref[j]
        else:
            got = (rounds[j]["accepted"], rounds[j]["out_tokens"], rounds[j]["hit"])
            want = round_ref[j]
        assert all(torch.equal(x, y) for x, y in zip(got, want))

    # per-entry-point durations (eager, events on the launching stream)
    def time_call(fn, n=60):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            fn(i % ncopy)
            ev[i][1].record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        return float(np.mean(ts[n // 10: n - n // 10]))   # trimmed mean, ms

    def call_build(j):
        S.ssd_build_cache(dfts[j], tau, F, out=outs[j][0])

    def call_verify(j):
        S.ssd_verify(tgts[j], dfts[j], toks, ua, ur, tau, S.sigma_from_cache(outs[j][0], C), out=outs[j][1])

    def call_plain(j):
        S.ssd_verify(tgts[j], dfts[j], toks_plain, ua, ur, tau, out=plain_out[j])

    def call_lookup(j):
        cache, res, look = outs[j]
        S.ssd_cache_lookup(cache["cache_tokens"], F, res["accepted"], res["out_tokens"], out=look)

    plain_out = [S.ssd_verify(tgts[j], dfts[j], toks_plain, ua, ur, tau) for j in range(ncopy)]
    torch.cuda.synchronize()
    for _ in range(2):
        time_call(call_build, 10), time_call(call_verify, 10), time_call(call_plain, 10)
    t_build = time_call(call_build)
    t_verify = time_call(call_verify)
    t_plain = time_call(call_plain)
    t_lookup = time_call(call_lookup)
    for j, o in enumerate(outs):
        assert torch.equal(o[1]["accepted"], sep_ref[j][0]) and torch.equal(o[1]["out_tokens"], sep_ref[j][1])
        assert torch.equal(o[2]["hit"], sep_ref[j][2])

    # the round's launches timed one by one (ssd_verify_round_marked): the
    # first launch records its own start and end events (its execution
    # time); events recorded on the launching stream after the second and
    # the third give those launches with the gap before each; back-to-back
    # calls over the rotating copies
    n_mark = 60
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_mark)]
    for i in range(n_mark):
        j = i % ncopy
        S.ssd_verify_round(tgts[j], dfts[j], F, C, toks, ua, ur, tau, out=rounds[j], marks=marks[i])
    torch.cuda.synchronize()
    launch_ms = {name: float(np.mean([m[k].elapsed_time(m[k + 1]) for m in marks[n_mark // 6:]]))
                 for k, name in enumerate(("k_round_chunks", "k_round_merge_stats", "k_round_resid"))}
    for j in range(ncopy):   # the marked calls wrote the same outputs
        assert torch.equal(rounds[j]["accepted"], round_ref[j][0]) and torch.equal(rounds[j]["hit"], round_ref[j][2])

    if args.profile_loop:
        for i in range(args.profile_loop):
            step(i % ncopy)
            call_plain(i % ncopy)
        torch.cuda.synchronize()

    acc = (outs[0][1] if args.separate else rounds[0])["accepted"].cpu().numpy()
    hit = (outs[0][2] if args.separate else rounds[0])["hit"].cpu().numpy()

    # single-read algorithmic bytes
    elem = 2 if cfg.dtype == "bf16" else 4
    row_bytes = V * elem
    bytes_build = B * (K + 1) * row_bytes            # draft rows 0..K
    bytes_verify_sigma = B * (K + 1) * row_bytes     # target rows 0..K (draft stats reused)
    bytes_plain = B * (2 * K + 1) * row_bytes        # target 0..K + draft 0..K-1
    s_step = ms_step / 1e3
    gbps = step_bytes / s_step / 1e9

    if args.separate:
        # dominant library call of the three-call step: the cache build (chunk pass + per-row merge)
        dom_ms = t_build
        dom_gbps = bytes_build / (dom_ms / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(dom_gbps, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(dom_gbps / PEAK_HBM_GBS, 4), "traffic": measured_traffic(HBM_BYTES_PROFILE),
                    "kernel": "ssd_build_cache (k_cache_chunk + k_cache_merge, bf16)",
                    "bytes_per_launch": bytes_build, "avg_launch_ms": round(dom_ms, 5)}
    else:
        # dominant kernel of the step: k_round_chunks, the launch that
        # streams draft rows 0..K for the cache and target rows 0..na-1 for
        # the row statistics (na = floor(2(K+1)/3), the split documented with
        # ssd_verify_round; the second launch streams the other target rows
        # beside the cache merges), timed by the marks
        na = 2 * (K + 1) // 3
        dom_bytes = B * (K + 1 + na) * V * tgt0.element_size()
        dom_ms = launch_ms["k_round_chunks"]
        dom_gbps = dom_bytes / (dom_ms / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(dom_gbps, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(dom_gbps / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(ROUND_BYTES_PROFILE, "k_round_chunks<1>"),
                    "kernel": f"k_round_chunks (cache chunk pass over draft rows 0..{K} + row-statistics chunk "
                              f"pass over target rows 0..{na - 1}, bf16)",
                    "bytes_per_launch": dom_bytes, "avg_launch_ms": round(dom_ms, 5),
                    "launches_timed": n_mark - n_mark // 6}

    ceil = box_ceilings(dev)
    cpu, check = None, None
    if not args.no_cpu:
        src = outs[0] if args.separate else None
        gpu = {"accepted": (src[1] if src else rounds[0])["accepted"].cpu().numpy(),
               "out_tokens": (src[1] if src else rounds[0])["out_tokens"].cpu().numpy(),
               "hit": (src[2] if src else rounds[0])["hit"].cpu().numpy(),
               "cache_tokens": (src[0] if src else rounds[0])["cache_tokens"].cpu().numpy(),
               "tokens": toks_np}
        cpu, check = cpu_baseline(args.config, tau, F, C, gpu, u_draft_np, args.cpu_seconds)

    line = {
        "metric": "verified rows/sec + logits HBM GB/s (% of peak), B=64 K=5 V=128256 bf16",
        "value": round(B / s_step, 1),
        "unit": "verified rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian + Zipf-rank logits, draft = target + noise, drafts drawn on the GPU "
                "from q_sigma)",
        "config": {"workload": ("ssd_step_fanout_buildcache_verify_sigma_lookup" if args.separate
                                else "ssd_step_fanout_verify_round"), "B": B, "K": K, "V": V,
                   "logits": cfg.dtype, "tau": tau, "cache": {"budget": cfg.n_budget, "a_p": cfg.a_p,
                                                                "r": cfg.r, "C": C, "F": F},
                   "rotating_copies": ncopy, "graph_replay": not args.eager},
        "logits_gbps": round(gbps, 1),
        "pct_peak_hbm": round(100 * gbps / PEAK_HBM_GBS, 2),
        "bytes_per_step": step_bytes,
        "roofline": roofline,
        "step_roofline": ({"achieved": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBS, 4), "unit": "GB/s",
                           "traffic": measured_traffic(ROUND_BYTES_PROFILE),
                           "what": "the whole graph-replayed step (three launches, launch gaps included)"}
                          if not args.separate else None),
        "launch_ms": ({k: round(v, 5) for k, v in launch_ms.items()} if not args.separate else None),
        "per_call_ms": {"ssd_build_cache": round(t_build, 5), "ssd_verify_sigma": round(t_verify, 5),
                        "ssd_cache_lookup": round(t_lookup, 5)},
        "verify_only": {"ms": round(t_plain, 5), "rows_per_s": round(B / (t_plain / 1e3), 1),
                        "bytes": bytes_plain,
                        "gbps": round(bytes_plain / (t_plain / 1e3) / 1e9, 1),
                        "pct_peak_hbm": round(100 * bytes_plain / (t_plain / 1e3) / 1e9 / PEAK_HBM_GBS, 2)},
        "verify_sigma_gbps": round(bytes_verify_sigma / (t_verify / 1e3) / 1e9, 1),
        "round_vs_separate_rows_differ": round_rows_differ,
        "box_ceilings": dict(ceil, dominant_kernel_vs_copy=round(dom_gbps / ceil["copy_gbps"], 4)),
        "oracle_check": check,
        "mean_accepted_plus_1": round(float(np.mean(acc + 1)), 4),
        "hit_rate": round(float(np.mean(hit)), 4),
        "cpu_baseline": cpu,
        "gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)
    if check is not None and check["rows_differ"] > 0:
        print(f"oracle parity FAILED on rows {check['differ_rows']}", file=sys.stderr)
        sys.exit(1)


def bench_report(args):
    """Per-workload report: the whole C-ABI call timed with HIP events around
    it (median, p10, p90 over --calls back-to-back calls on rotating input
    copies, ceil(512 MB / bytes) + 1 of them, so logits come from HBM), plus
    the same call on one warm copy, and the calls replayed as HIP graphs
    (t_graph_us: GPU time per call without host launch overhead, the
    latency figure for launch-bound workloads). Plain workloads time ssd_verify; cache
    workloads time ssd_verify_round (cache build, sigma verification, lookup)
    on drafts drawn on the GPU from q_sigma (ssd_draft_sample).
    Bytes: single-read logits bytes of the call, and the early-exit minimum
    (target rows 0..a and draft rows 0..min(a, K-1) per sequence; all draft
    rows 0..K when the cache is built)."""
    import torch
    import verify_speculation_cache_amd as S
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    todo = []
    ids = [1, 2, 3, 4, 5] if args.report == "all" else [int(x) for x in args.report.split(",")]
    for c in ids:
        for tau in W.get_config(c).taus:
            todo.append((c, tau))

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    for c, tau in todo:
        cfg = W.get_config(c)
        B, K, V = cfg.B, cfg.K, cfg.V
        elem = cfg.elem_bytes
        t0 = time.time()
        d = W.make_inputs(cfg, tau=tau, draw_tokens=not cfg.has_cache)
        gen_s = time.time() - t0
        cache_mode = cfg.has_cache and c != 2      # workload 2 is the plain-verify metric
        n_draft = K + 1 if cache_mode else K
        tgt0 = up(d["target"])
        dft0 = up(d["draft"][:, :n_draft])
        bytes_call = B * (K + 1 + n_draft) * V * elem
        ncopy = n_copies(bytes_call)
        tgts = [tgt0] + [tgt0.clone() for _ in range(ncopy - 1)]
        dfts = [dft0] + [dft0.clone() for _ in range(ncopy - 1)]
        ua = torch.from_numpy(d["u_acc"]).to(dev)
        ur = torch.from_numpy(d["u_res"]).to(dev)
        tau32 = d["tau"]
        if cache_mode:
            F = S.ssd_fanout(cfg.n_budget, K, cfg.a_p, cfg.r)
            cache0 = S.ssd_build_cache(dfts[0], tau32, F)   # sigma for the drafts
            u_draft = torch.from_numpy(W.make_draft_uniforms(cfg, tau)).to(dev)
            toks = S.ssd_draft_sample(dfts[0], u_draft, tau32, S.sigma_from_cache(cache0, cfg.C))
            outs = [S.ssd_verify_round(tgts[j], dfts[j], F, cfg.C, toks, ua, ur, tau32) for j in range(ncopy)]

            def call(j):
                S.ssd_verify_round(tgts[j], dfts[j], F, cfg.C, toks, ua, ur, tau32, out=outs[j])
        else:
            toks = torch.from_numpy(d["tokens"]).to(dev)
            outs = [S.ssd_verify(tgts[j], dfts[j], toks, ua, ur, tau32) for j in range(ncopy)]

            def call(j):
                S.ssd_verify(tgts[j], dfts[j], toks, ua, ur, tau32, out=outs[j])
        torch.cuda.synchronize()

        def timed(n, rotate):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for i in range(n):
                j = i % ncopy if rotate else 0
                ev[i][0].record()
                call(j)
                ev[i][1].record()
            torch.cuda.synchronize()
            return sorted(a.elapsed_time(b) for a, b in ev)

        timed(10, True)
        ts = timed(args.calls, True)
        warm = timed(max(20, args.calls // 4), False)
        # the same calls replayed as HIP graphs (one graph per cycle over the
        # copies): GPU time per call without the host's launch overhead
        run = _replay_runner(call, ncopy, argparse.Namespace(eager=False))
        n_graph = ncopy * max(1, -(-args.calls // ncopy))
        run(ncopy)
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        run(n_graph)
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) * 1e3 / n_graph
        del run
        med, p10, p90 = ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]
        acc = outs[0]["accepted"].cpu().numpy()
        ok = acc >= 0
        a = acc[ok]
        rows_min = np.sum(a + 1) + (B * n_draft if cache_mode else np.sum(np.minimum(a + 1, K)))
        bytes_min = int(rows_min) * V * elem
        alpha = [float(np.sum(a > i) / max(1, np.sum(a >= i))) for i in range(K)]
        line = {
            "report": "per_workload", "workload": cfg.name, "B": B, "K": K, "V": V, "dtype": cfg.dtype,
            "tau": tau, "call": ("ssd_verify_round (cache build, sigma verification, lookup)" if cache_mode
                                 else "ssd_verify"),
            "calls": args.calls, "rotating_copies": ncopy,
            "t_call_us": {"median": round(med * 1e3, 2), "p10": round(p10 * 1e3, 2), "p90": round(p90 * 1e3, 2)},
            "warm_single_copy_us": round(warm[len(warm) // 2] * 1e3, 2),
            "t_graph_us": round(graph_us, 2),
            "rows_per_s": round(B / (med / 1e3), 1),
            "bytes_single_read": bytes_call,
            "eff_gbps": round(bytes_call / (med / 1e3) / 1e9, 1),
            "pct_peak": round(100 * bytes_call / (med / 1e3) / 1e9 / PEAK_HBM_GBS, 2),
            "early_exit_min_bytes": bytes_min,
            "early_exit_min_gbps": round(bytes_min / (med / 1e3) / 1e9, 1),
            "alpha_empirical": [round(x, 4) for x in alpha],
            "mean_accepted_plus_1": round(float(np.mean(a + 1)), 4),
            "flagged_rows": int(np.sum(~ok)),
            "gen_s": round(gen_s, 1),
        }
        if cache_mode:
            line["hit_rate"] = round(float(outs[0]["hit"].float().mean().item()), 4)
            line["F"] = F
            line["C"] = cfg.C
        print(json.dumps(line), flush=True)
        del tgts, dfts, tgt0, dft0, outs
        torch.cuda.empty_cache()


def _replay_runner(step, ncopy, args, per_step=None):
    """Return run(n, offset) that performs n steps over the rotating copies,
    copy (offset + i) % ncopy at step i.

    Unless args.eager, the steps run as HIP graph replays: one graph holds a
    whole cycle step(0) .. step(ncopy - 1), so a launch is paid once per
    ncopy steps, and one graph per copy serves the steps that do not start
    or fill a whole cycle. Every step still runs, in order, exactly once.
    The per-shape workspaces are warmed eagerly on the capture stream first.
    per_step(j), if given, runs on the host for every step."""
    import torch
    whole, single = None, []
    if not args.eager:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for j in range(ncopy):
                step(j)
        torch.cuda.synchronize()
        whole = torch.cuda.CUDAGraph()
        with torch.cuda.graph(whole, stream=stream):
            for j in range(ncopy):
                step(j)
        for j in range(ncopy):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(j)
            single.append(g)
        torch.cuda.synchronize()

    def run(n, offset=0):
        i = 0
        while i < n:
            j = (offset + i) % ncopy
            if per_step is not None:
                per_step(j)
            if whole is None:
                step(j)
                i += 1
            elif j == 0 and n - i >= ncopy:
                if per_step is not None:
                    for jj in range(1, ncopy):
                        per_step(jj)
                whole.replay()
                i += ncopy
            else:
                single[j].replay()
                i += 1
    return run


def _graph_time(step, ncopy, args):
    """Time args.steps steps (after args.warmup untimed ones) through
    _replay_runner, HIP events around the loop. Returns ms per step."""
    import torch
    run = _replay_runner(step, ncopy, args)
    run(args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run(args.steps, args.warmup)
    e1.record()
    torch.cuda.synchronize()
    if args.profile_loop:
        for i in range(args.profile_loop):
            step(i % ncopy)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / args.steps


def bench_rows(args):
    """Greedy verification or sigma-aware draft sampling on the main workload's
    shape (B=64, K=5, V=128256, bf16, tau=0.7): one step = one library call.
    greedy: ssd_verify_greedy on target rows 0..K (drafted tokens from the
    workload); sample: ssd_draft_sample on draft rows 0..K-1 with sigma_{F,C}
    from ssd_build_cache (budget 64, a_p 0.8, r 1, C 0.5), built once before
    timing. Bytes: each row the call reads, once."""
    import torch
    import verify_speculation_cache_amd as S
    import workloads as W

    cfg = W.get_config(2)
    B, K, V, tau = cfg.B, cfg.K, cfg.V, cfg.taus[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    d = W.make_inputs(cfg, tau=tau)
    gen_s = time.time() - t0

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    greedy = args.workload == "greedy"
    src = d["target"] if greedy else d["draft"][:, :K + 1]
    x0 = up(src)
    rows_read = K + 1 if greedy else K
    bytes_call = B * rows_read * V * 2
    ncopy = n_copies(bytes_call)
    xs = [x0] + [x0.clone() for _ in range(ncopy - 1)]
    toks = torch.from_numpy(d["tokens"]).to(dev)
    if greedy:
        outs = [S.ssd_verify_greedy(xs[j], toks) for j in range(ncopy)]

        def step(j):
            S.ssd_verify_greedy(xs[j], toks, out=outs[j])
    else:
        F = S.ssd_fanout(cfg.n_budget, K, cfg.a_p, cfg.r)
        sig = [S.sigma_from_cache(S.ssd_build_cache(xs[j], tau, F), cfg.C) for j in range(ncopy)]
        u_np = W.make_draft_uniforms(cfg, tau)
        u = torch.from_numpy(u_np).to(dev)
        outs = [S.ssd_draft_sample(xs[j], u, tau, sig[j]) for j in range(ncopy)]

        def step(j):
            S.ssd_draft_sample(xs[j], u, tau, sig[j], out=outs[j])
    torch.cuda.synchronize()
    ref = [(o["out_tokens"] if greedy else o).clone() for o in outs]
    ms_step = _graph_time(step, ncopy, args)
    for j, o in enumerate(outs):
        assert torch.equal(o["out_tokens"] if greedy else o, ref[j])
    gbps = bytes_call / (ms_step / 1e3) / 1e9
    cpu = None
    if not args.no_cpu:
        import oracle as O
        t0 = time.time()
        n = 0
        while n < B and (time.time() - t0) < args.cpu_seconds:
            sl = slice(n, n + 1)
            if greedy:
                O.verify_greedy(d["target"][sl], d["tokens"][sl])
            else:
                O.draft_sample(d["draft"][sl], d["tau"], u_np[sl], F, cfg.C)
            n += 1
        dt = time.time() - t0
        cpu = {"value": round(n / dt, 3), "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n} of {B} batch rows of the same call, float64 NumPy, {dt:.1f} s"
                         + ("" if greedy else " (the oracle takes each row's top-F for sigma itself)"),
               "cpu_model": _cpu_model()}
    name = "ssd_verify_greedy" if greedy else "ssd_draft_sample"
    kern = "k_greedy<1>, one launch" if greedy else "k_sample_chunks<1, true> + k_sample_pick<1, true>"
    line = {
        "metric": ("greedy-verified rows/sec" if greedy else "sigma-drafted rows/sec") + ", B=64 K=5 V=128256 bf16",
        "value": round(B / (ms_step / 1e3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian + Zipf-rank logits, draft = target + noise)",
        "config": {"workload": name, "B": B, "K": K, "V": V, "logits": cfg.dtype, "tau": tau,
                   "rotating_copies": ncopy, "graph_replay": not args.eager},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": f"{name} ({kern})", "bytes_per_launch": bytes_call,
                     "avg_launch_ms": round(ms_step, 5)},
        "cpu_baseline": cpu,
        "gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def bench_tree(args):
    """Token-tree verification on its workload: B=32 sequences, a 29-node
    tree (4 first-token candidates, 2 continuations each, then chains to
    depth 4), V=128256, bf16, tau=0.7. One step = one ssd_verify_tree call
    (the statistics pass, then the residual rounds the topology needs)."""
    import torch
    import verify_speculation_cache_amd as S
    import workloads as W

    cfg = W.TREE_CONFIGS["tree"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    d = W.make_tree_inputs(cfg)
    gen_s = time.time() - t0
    B, N, V = cfg.B, cfg.N, cfg.V
    parent = d["parent"]
    inner = sum(1 for n in range(N) if n in set(parent[1:]))

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    tgt0 = up(d["target"])
    # only inner nodes' draft rows are read; the rest of the buffer is never touched
    dft0 = up(d["draft"])
    row_bytes = V * 2
    bytes_single = B * (N + inner) * row_bytes       # every statistics row once
    ncopy = n_copies(bytes_single)
    tgts = [tgt0] + [tgt0.clone() for _ in range(ncopy - 1)]
    dfts = [dft0] + [dft0.clone() for _ in range(ncopy - 1)]
    toks = torch.from_numpy(d["tokens"]).to(dev)
    ua = torch.from_numpy(d["u_acc"]).to(dev)
    ur = torch.from_numpy(d["u_res"]).to(dev)
    outs = [S.ssd_verify_tree(tgts[j], dfts[j], parent, toks, ua, ur, cfg.tau) for j in range(ncopy)]
    torch.cuda.synchronize()
    ref = [(o["accepted"].clone(), o["out_tokens"].clone()) for o in outs]

    def step(j):
        S.ssd_verify_tree(tgts[j], dfts[j], parent, toks, ua, ur, cfg.tau, out=outs[j])

    ms_step = _graph_time(step, ncopy, args)
    for j, o in enumerate(outs):
        assert torch.equal(o["accepted"], ref[j][0]) and torch.equal(o["out_tokens"], ref[j][1])
    acc = outs[0]["accepted"].cpu().numpy()
    gbps = bytes_single / (ms_step / 1e3) / 1e9
    cpu = None
    if not args.no_cpu:
        import oracle as O
        t0 = time.time()
        n = 0
        while n < B and (time.time() - t0) < args.cpu_seconds:
            sl = slice(n, n + 1)
            O.verify_tree(d["target"][sl], d["draft"][sl], parent, d["tokens"][sl], d["u_acc"][sl],
                          d["u_res"][sl], d["tau"])
            n += 1
        dt = time.time() - t0
        cpu = {"value": round(n / dt, 3), "unit": "verified trees/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n} of {B} batch rows of the same step, float64 NumPy, {dt:.1f} s"}
    line = {
        "metric": "verified trees/sec, B=32 N=29 V=128256 bf16",
        "value": round(B / (ms_step / 1e3), 1),
        "unit": "verified trees/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian + Zipf-rank logits, draft = target + noise, siblings drawn "
                "independently from the parent's draft distribution)",
        "config": {"workload": "ssd_verify_tree", "B": B, "N": N, "branching": list(cfg.branching), "V": V,
                   "logits": cfg.dtype, "tau": cfg.tau, "rounds": S.ssd_tree_rounds(parent),
                   "rotating_copies": ncopy, "graph_replay": not args.eager},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "ssd_verify_tree (k_tree_stats + rounds of k_tree_round, bf16)",
                     "bytes_per_launch": bytes_single, "avg_launch_ms": round(ms_step, 5)},
        "mean_accepted_plus_1": round(float(np.mean(acc + 1)), 4),
        "cpu_baseline": cpu,
        "gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


HBM_BYTES_PROFILE = os.path.join(ROOT, "profiles", "ssd_build_cache_B64_K5_V128256_bf16_hbm_bytes.md")
ROUND_BYTES_PROFILE = os.path.join(ROOT, "profiles", "ssd_verify_round_B64_K5_V128256_bf16_hbm_bytes.md")


def box_ceilings(dev):
    """What plain torch kernels reach on this machine's HBM, as context for the
    roofline fractions (8 TB/s is the published peak): a device copy of a
    512 MiB bf16 tensor (bytes read + written per second) and its float32
    sum (bytes read per second), medians of 7 runs timed with events."""
    import torch
    nbytes = 512 << 20
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)

    def med(fn, reps=7):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[reps // 2]

    t_copy = med(lambda: y.copy_(x))
    t_sum = med(lambda: x.sum(dtype=torch.float32))
    del x, y
    torch.cuda.synchronize()
    return {"copy_gbps": round(2 * nbytes / t_copy / 1e6, 1), "sum_read_gbps": round(nbytes / t_sum / 1e6, 1),
            "what": "torch copy_ (read + write) and sum (read) of a 512 MiB bf16 tensor, median of 7"}


def measured_traffic(profile, kernel=None):
    """HBM bytes per call (or, with kernel, per launch of that kernel) from a
    committed FETCH_SIZE / WRITE_SIZE counter summary, or None when the
    kernel sources changed since it was taken."""
    import hashlib
    try:
        text = open(profile).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        h = hashlib.sha256()
        for p in rec["sources"]:
            h.update(open(os.path.join(ROOT, p), "rb").read())
    except (OSError, ValueError, KeyError, IndexError):
        return None
    if h.hexdigest() != rec["source_sha256"]:
        return None
    if kernel is not None:
        return rec.get("kernel_bytes", {}).get(kernel)
    return rec["traffic_bytes_per_launch"]


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_inputs(cid, tau, b):
    import workloads as W
    return W.make_inputs(W.get_config(cid), tau=tau, draw_tokens=False, b_rows=[b])


def _oracle_step_row(d, K, F, C, b, toks_row, u_row):
    """The oracle on batch row b of the step: its sigma draws with the GPU's
    uniforms (a parity check of the draft phase, untimed), then, timed, the
    cache build, the sigma verification of the GPU's drafted tokens and the
    lookup. Returns its outputs and the seconds the step took."""
    import oracle as O
    dtoks, dmarg = O.draft_sample(d["draft"][:, :K], d["tau"], u_row[None, :], F, C)
    t1 = time.time()
    cache = O.build_cache(d["draft"][:, :K + 1], d["tau"], F, C)
    ref = O.verify(d["target"], d["draft"], toks_row[None, :], d["u_acc"], d["u_res"], d["tau"], {"F": F, "C": C})
    hit, _ = O.cache_lookup(cache["cache_tokens"], F, ref["accepted"], ref["out_tokens"])
    return {"b": b, "accepted": int(ref["accepted"][0]), "out_tokens": ref["out_tokens"][0],
            "acc_margin": ref["acc_margin"][0], "res_margin": float(ref["res_margin"][0]),
            "cache_tokens": cache["cache_tokens"][0], "hit": int(hit[0]),
            "draft_tokens": dtoks[0], "draft_margin": dmarg[0], "oracle_s": time.time() - t1}


def _oracle_worker(jobs, barrier, queue):
    """One host process of the fan-out: generate its rows' inputs, wait for
    every process, then run the oracle on them and report."""
    for v in ("OMP_NUM_THREADS", "MKL_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
        os.environ[v] = "1"
    inputs = [_oracle_inputs(j[0], j[1], j[4]) for j in jobs]
    barrier.wait()
    out = []
    for d, (cid, tau, F, C, b, toks_row, u_row, K) in zip(inputs, jobs):
        out.append(_oracle_step_row(d, K, F, C, b, toks_row, u_row))
    queue.put(out)


def _check_rows(rows, gpu, F):
    """GPU outputs of the step against the oracle rows: cache tokens exact;
    drafted tokens equal the oracle's draws unless that draw's margin is
    below 1e-6; accepted length and emitted tokens equal unless the oracle's
    margin at the first differing decision is below 1e-6; the hit bit of the
    GPU's own outcome equals the oracle lookup of that outcome."""
    import oracle as O
    differ, excused = [], []
    for r in rows:
        b = r["b"]
        ok = np.array_equal(gpu["cache_tokens"][b], r["cache_tokens"])
        dt_ok = np.all((gpu["tokens"][b] == r["draft_tokens"]) | (r["draft_margin"] < 1e-6))
        a_g, out_g = int(gpu["accepted"][b]), gpu["out_tokens"][b]
        same = a_g == r["accepted"] and np.array_equal(out_g, r["out_tokens"])
        if not same:
            if a_g != r["accepted"]:
                m = r["acc_margin"][min(a_g, r["accepted"])] if min(a_g, r["accepted"]) >= 0 else math.inf
            else:
                m = r["res_margin"]
            if m < 1e-6:
                excused.append(b)
            else:
                ok = False
        h_own, _ = O.cache_lookup(r["cache_tokens"][None, :], F, np.array([a_g]), out_g[None, :])
        ok = ok and dt_ok and int(h_own[0]) == int(gpu["hit"][b])
        if not ok:
            differ.append(b)
    return {"rows": len(rows), "rows_differ": len(differ), "differ_rows": differ, "excused_rows": excused}


def cpu_baseline(cid, tau, F, C, gpu, u_draft, budget_s):
    """The float64 oracle on the host over the same step (drafted tokens as
    the GPU drew them): (i) one process, rows in order for at most budget_s
    of oracle time; (ii) the same per-row function over every batch row,
    fanned out over all host cores the process may use (rows are
    independent; each process generates its rows' inputs first, then all
    start together and the wall time of the oracle phase is taken). The rows
    of (ii) are checked against the GPU's outputs. Returns (baseline, check)."""
    import multiprocessing as mp
    import queue as qmod
    import workloads as W
    cfg = W.get_config(cid)
    B, K = cfg.B, cfg.K
    jobs = [(cid, tau, list(F), C, b, gpu["tokens"][b], u_draft[b], K) for b in range(B)]
    single, dt1 = [], 0.0
    while len(single) < B and dt1 < budget_s:
        j = jobs[len(single)]
        single.append(_oracle_step_row(_oracle_inputs(cid, tau, j[4]), K, j[2], j[3], j[4], j[5], j[6]))
        dt1 += single[-1]["oracle_s"]
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")
    barrier, q = ctx.Barrier(cores + 1), ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(jobs[i::cores], barrier, q)) for i in range(cores)]
    for p in procs:
        p.start()
    barrier.wait(timeout=600)
    t0 = time.time()
    rows = []
    for _ in range(cores):
        try:
            rows += q.get(timeout=600)
        except qmod.Empty:
            break
    dtn = time.time() - t0
    for p in procs:
        p.join(timeout=60)
    rows.sort(key=lambda r: r["b"])
    base = {"value": round(len(rows) / dtn, 3), "unit": "verified rows/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"all {len(rows)} of {B} batch rows of the same step (cache build, sigma verify, lookup), "
                      f"float64 NumPy, the per-row oracle fanned out over {cores} processes, {dtn:.1f} s wall",
            "single_thread": {"value": round(len(single) / dt1, 3), "unit": "verified rows/s", "cores": 1,
                              "sample": f"first {len(single)} of {B} rows, {dt1:.1f} s"}}
    return base, _check_rows(rows, gpu, F)


if __name__ == "__main__":
    main()
