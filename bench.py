#!/usr/bin/env python3
"""Causal-attention throughput of one prefill-context-parallel rank share on
one MI355X.

A step is one pass of the whole hot path over the workload's inputs, already
resident in HBM: the paged context pass, the end-aligned causal new-token
pass and the LSE merge, run as one fused launch (pcp_attn_rank_share; the
host row plan and unit order are built once, a few milliseconds of host
work). The same step through the three separate calls (context pass,
new-token pass, lse_merge) is timed as well and reported per kernel. The
default workload is one rank's share of a 131072-token prompt split over 4
PCP ranks (8 Q / 1 KV heads, d = 256).

Prints one JSON line. ``value`` is useful causal TFLOP/s of the step:
4 * d * Hq FLOPs per visible (query, key) pair, masked and padded work not
counted. ``roofline`` reports the step's kernel against the MI355X dense
bf16 MFMA peak, timed with HIP events on the stream the kernels run on.
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
rank share's queries. ``fp8`` times the same step with E4M3 Q/K/V and
per-(request, KV head) descales (pcp_attn_rank_share_fp8) against its own
peak (QK^T on the FP8 MFMA, PV on the bf16 MFMA).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# 256 CUs x 2.4 GHz x 4096 bf16 FLOP/clk/CU (dense; the published 2.5 PFLOP/s)
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
# FP8 dense MFMA runs at twice the bf16 rate (the published 5.0 PFLOP/s)
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS
# The FP8 rank share runs QK^T (half of the useful FLOP) on the FP8 MFMA and
# PV (the other half) on the bf16 MFMA: its peak is the rate at which both
# halves finish, 1 / (0.5 / fp8 peak + 0.5 / bf16 peak).
PEAK_FP8_QK_BF16_PV_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0

DEFAULT_WORKLOAD = "hybrid_fullattn_128k_pcp4_r1"


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def plan_pairs(rows):
    """(new-token pairs, context pairs) of a plan, per query head.
    Row with m queries and n new keys: query t sees min(n, max(0, n - m + t + 1))."""
    new = 0
    ctx = 0
    for r in rows:
        m, n, cl = int(r[3]), int(r[6]), int(r[8])
        for_rows = 0
        if m <= n:
            for_rows = m * (n - m) + m * (m + 1) // 2
        else:  # only the last n queries see keys
            for_rows = n * (n + 1) // 2
        new += for_rows
        ctx += m * cl
    return new, ctx


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:  # pragma: no cover
        pass
    return os.cpu_count() or 1


def cpu_baseline(inp, share, budget_s: float, seed: int):
    """Time the fp64 oracle on a growing, seeded sample of this rank's queries
    until about ``budget_s`` seconds of CPU work; returns TFLOP/s of the
    sample's useful work, and the whole share's oracle time extrapolated from
    the sample's rate per visible (query, key) pair, plus the oracle's row
    plan, which is timed on its own."""
    import numpy as np
    import torch

    import oracle

    w = inp.workload
    t0 = time.perf_counter()
    plan = oracle.plan_rows(inp.cu_seqlens_new, inp.ctx_lens, w.pcp_size, share.pcp_rank,
                            w.dcp_size, share.dcp_rank, w.block_size)
    plan_s = time.perf_counter() - t0
    rows = plan.astype(np.int64)
    assert np.array_equal(rows, share.rows_host.astype(np.int64))
    q_local = share.q.float().cpu().double().numpy()
    k_new = inp.k_new.double().numpy()
    v_new = inp.v_new.double().numpy()
    k_c = inp.k_cached.double().numpy()
    v_c = inp.v_cached.double().numpy()
    order = np.random.default_rng(seed).permutation(share.total_q)
    starts = rows[:, 2]
    done = 0
    flops = 0
    pairs_done = 0
    spent = 0.0
    while spent < budget_s and done < len(order):
        ids = np.sort(order[done:done + 64])
        done += len(ids)
        t0 = time.perf_counter()
        oracle.rank_share(q_local, k_new, v_new, k_c, v_c, inp.cu_cache, rows, w.dcp_size,
                          share.dcp_rank, w.block_size, w.num_q_heads, w.num_kv_heads,
                          w.softmax_scale, query_ids=ids)
        spent += time.perf_counter() - t0
        ridx = np.searchsorted(starts, ids, side="right") - 1
        t = ids - starts[ridx]
        m, n, cl = rows[ridx, 3], rows[ridx, 6], rows[ridx, 8]
        pairs = np.clip(n - m + t + 1, 0, n) + cl
        pairs_done += int(pairs.sum())
        flops += int(4 * w.head_dim * w.num_q_heads * pairs.sum())
    del torch
    new_p, ctx_p = plan_pairs(rows)
    whole_s = plan_s + (new_p + ctx_p) / pairs_done * spent if pairs_done else None
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": "%d of %d query rows (seeded random), all %d heads, fp64 numpy; %.1f s" % (
            done, share.total_q, w.num_q_heads, spent),
        "whole_share_s": {
            "value": round(whole_s, 1) if whole_s is not None else None,
            "kind": "extrapolated",
            "basis": "the sample's seconds per visible (query, key) pair times the share's "
                     "%d pairs, plus the oracle's row plan (%.4f s, timed)" % (new_p + ctx_p,
                                                                              plan_s),
        },
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured by rocprofv3 counters (JSON)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 leg")
    ap.add_argument("--report", action="store_true",
                    help="instead of the JSON line: time every named workload (and a "
                         "decode-only context launch) and print one JSON object per workload")
    ap.add_argument("--report-decode", action="store_true",
                    help="instead of the JSON line: only the decode-only batches of --report "
                         "(context pass over decode rows, unsplit and split, warm and cold)")
    ap.add_argument("--resplit", action="store_true",
                    help="instead of the JSON line: the --workload's re-split path (cache write, "
                         "then the fused launch over re-split rows) beside its standard fused "
                         "launch, one JSON object (for the profiler)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="instead of the workload, run a plain 1 GiB device copy (torch.neg, "
                         "1 GiB read + 1 GiB written per launch) to scale FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="instead of timing: read the rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "runs of the workload and of --calibrate-copy under DIR (subfolders "
                         "pmc_FETCH_SIZE, pmc_WRITE_SIZE, copy_FETCH_SIZE, copy_WRITE_SIZE) and "
                         "write the --workload's entries into the --traffic JSON")
    args = ap.parse_args()
    if args.traffic_from:
        return write_traffic(args.traffic_from, args.workload, args.traffic)
    if args.calibrate_copy:
        return calibrate_copy()
    if args.report:
        return report(args.steps, args.warmup)
    if args.resplit:
        return resplit_line(args.workload, args.steps, args.warmup)
    if args.report_decode:
        import torch

        flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB, read to evict
        for line in report_decode_batches(args.steps, args.warmup, flush):
            print(json.dumps(line), flush=True)
        return 0

    if args.gpus != 1:
        print("bench.py runs one rank share on one GPU; --gpus %d is not supported "
              "(the path has no cross-GPU collectives in this library)" % args.gpus,
              file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is single-process; WORLD_SIZE > 1 is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from context_causal_gqa_amd.share import RankShare
    from pcp_workloads import WORKLOADS, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    w = WORKLOADS[args.workload]
    log("generating %s (seed %d)" % (w.name, w.seed))
    inp = generate(w)
    log("uploading")
    share = RankShare(inp, device="cuda:0")
    new_pairs, ctx_pairs = plan_pairs(share.rows_host)
    per_pair = 4 * w.head_dim * w.num_q_heads
    flops_new = per_pair * new_pairs
    flops_ctx = per_pair * ctx_pairs
    flops = flops_new + flops_ctx

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        share.step_fused()
        share.step()
    torch.cuda.synchronize()

    log("timing %d steps (one fused launch each)" % args.steps)
    evf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for e0, e1 in evf:
        e0.record()
        share.step_fused()
        e1.record()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    ms_fused = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evf]))
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_fused * 1e-3) / 1e12

    log("timing %d steps through the three calls" % args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        share.context_pass()
        ev[i][1].record()
        share.new_token_pass()
        ev[i][2].record()
        share.merge()
        ev[i][3].record()
    torch.cuda.synchronize()
    ms_ctx = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ms_new = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_merge = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    ms_three = float(np.mean([e[0].elapsed_time(e[3]) for e in ev]))
    log("step %.3f ms fused (%.1f TFLOP/s); three calls %.3f ms (ctx %.3f, new %.3f, merge %.3f)"
        % (ms_step, value, ms_three, ms_ctx, ms_new, ms_merge))

    traffic = traffic_entry(args.traffic, w.name)

    line = {
        "metric": "causal attn TFLOP/s + % of bf16 MFMA peak, 128k-token PCP rank share",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": w.name,
            "new_tokens": int(inp.cu_seqlens_new[-1]),
            "cached_tokens": int(inp.ctx_lens.sum()),
            "pcp_size": w.pcp_size,
            "pcp_rank": w.pcp_rank,
            "dcp_size": w.dcp_size,
            "query_rows": share.total_q,
            "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "useful_flop_per_step": flops,
        },
        "kernels_ms": {
            "rank_share_fused": round(ms_fused, 4),
            "three_calls": {"context_paged": round(ms_ctx, 4), "prefill": round(ms_new, 4),
                            "lse_merge": round(ms_merge, 4), "step": round(ms_three, 4),
                            "step_tflops": round(flops / (ms_three * 1e-3) / 1e12, 2),
                            "prefill_tflops": round(flops_new / (ms_new * 1e-3) / 1e12, 2)},
        },
        "roofline": {
            "kernel": "attn_fwd_kernel, fused rank share (pcp_attn_rank_share)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_fp8:
        line["fp8"] = bench_fp8(inp, flops, args.steps, args.warmup)
        line["fp8"]["roofline"]["traffic"] = traffic_entry(args.traffic, w.name + ":fp8")
    if args.cpu_budget > 0:
        log("cpu baseline (%.0f s budget)" % args.cpu_budget)
        line["cpu_baseline"] = cpu_baseline(inp, share, args.cpu_budget, seed=w.seed)
    print(json.dumps(line), flush=True)
    return 0


def bench_fp8(inp, flops: int, steps: int, warmup: int) -> dict:
    """The same rank share with E4M3 Q/K/V (quantised on the host before the
    timed region; per-(request, KV head) descales): one fused launch per
    step, timed with HIP events on its stream."""
    import numpy as np
    import torch

    from context_causal_gqa_amd.share import RankShare
    from pcp_workloads import quantize_fp8

    log("fp8: quantising and uploading")
    share = RankShare(inp, device="cuda:0", fp8=quantize_fp8(inp))
    for _ in range(warmup):
        share.step_fused()
    torch.cuda.synchronize()
    log("fp8: timing %d steps" % steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for e0, e1 in ev:
        e0.record()
        share.step_fused()
        e1.record()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    ms_kernel = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    log("fp8: step %.3f ms (%.1f TFLOP/s)" % (ms_step, flops / (ms_step * 1e-3) / 1e12))
    del share
    torch.cuda.empty_cache()
    return {
        "dtype": "e4m3 Q/K/V, per-(request, KV head) descales; bf16 out",
        "ms_per_step": round(ms_step, 4),
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "roofline": {
            "kernel": "attn_fwd_kernel FP8, fused rank share (pcp_attn_rank_share_fp8)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_FP8_QK_BF16_PV_TFLOPS, 1),
            "peak_note": "QK^T at the FP8 MFMA peak (%.0f), PV at the bf16 one (%.0f)"
                         % (PEAK_FP8_TFLOPS, PEAK_BF16_TFLOPS),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_QK_BF16_PV_TFLOPS, 4),
        },
    }


# A launch runs at the clock the chip holds when it starts. After a pause
# (host-side input generation or quantisation) the first few hundred ms of
# back-to-back work run slower: on the Qwen-shaped share the fused launch
# timed 0.319, then 0.284, then 0.256 ms after 300 ms of back-to-back calls
# (FP8: 0.271, 0.245, 0.213 ms). The report's timings (not the headline line,
# which does exactly the warm-up steps it is given) start after SETTLE_S
# seconds of calls of the function they time.
SETTLE_S = 0.3


def settle(fn) -> None:
    """Call ``fn`` back to back (a synchronisation every 4 calls bounds the
    queue) until SETTLE_S seconds have passed."""
    import time

    import torch

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def time_share(share, steps: int, warmup: int):
    """Average ms of (context pass, new-token pass, merge, whole step)."""
    import numpy as np
    import torch

    for _ in range(warmup):
        share.step()
    settle(share.step)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        share.context_pass()
        ev[i][1].record()
        share.new_token_pass()
        ev[i][2].record()
        share.merge()
        ev[i][3].record()
    torch.cuda.synchronize()
    t = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3]),
                   e[0].elapsed_time(e[3])] for e in ev])
    return t.mean(axis=0)


def time_fused(share, steps: int, warmup: int) -> float:
    """Average ms of the fused single-launch step."""
    import torch

    for _ in range(warmup):
        share.step_fused()
    settle(share.step_fused)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        share.step_fused()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_cold(fn, iters: int, flush) -> float:
    """Average ms of ``fn`` with the 256 MB Infinity Cache (and L2) defeated:
    a sum over a 1 GiB buffer runs on the same stream before every timed
    call. It only reads, so it leaves no dirty lines whose write-back would
    overlap the timed call (a 1 GiB fill does, and slows short HBM-bound
    launches by 15-55%)."""
    import numpy as np
    import torch

    sink = torch.empty((), dtype=flush.dtype, device=flush.device)
    settle(fn)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for e0, e1 in ev:
        torch.sum(flush, dim=0, out=sink)
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))


def report(steps: int, warmup: int) -> int:
    """Per-workload throughput table (useful TFLOP/s of each pass, merge and
    decode bandwidth). Prints one JSON object per line."""
    import numpy as np
    import torch

    from context_causal_gqa_amd.share import RankShare
    from pcp_workloads import WORKLOADS, generate, scaled_workload

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB, read to evict
    for name, w in WORKLOADS.items():
        log("report: " + name)
        inp = generate(w)
        share = RankShare(inp, device="cuda:0")
        new_pairs, ctx_pairs = plan_pairs(share.rows_host)
        per_pair = 4 * w.head_dim * w.num_q_heads
        ms_ctx, ms_new, ms_merge, ms_step = time_share(share, steps, warmup)
        ms_fused = time_fused(share, steps, warmup)
        tq, hq, d = share.total_q, w.num_q_heads, w.head_dim
        merge_bytes = 3 * tq * hq * (2 * d + 4)
        ms_merge_cold = time_cold(share.merge, steps, flush)
        line = {
            "workload": w.name,
            "rows": share.num_rows,
            "query_rows": tq,
            "useful_flop": per_pair * (new_pairs + ctx_pairs),
            "ms": {"rank_share_fused": round(ms_fused, 4), "context_paged": round(ms_ctx, 4),
                   "prefill": round(ms_new, 4), "lse_merge": round(ms_merge, 4),
                   "step_three_calls": round(ms_step, 4)},
            "tflops": {
                "fused": round(per_pair * (new_pairs + ctx_pairs) / ms_fused / 1e9, 1),
                "step_three_calls": round(per_pair * (new_pairs + ctx_pairs) / ms_step / 1e9, 1),
                "prefill": round(per_pair * new_pairs / ms_new / 1e9, 1),
                "context_paged": round(per_pair * ctx_pairs / ms_ctx / 1e9, 1) if ctx_pairs else None,
            },
            "pct_bf16_peak_fused": round(100 * per_pair * (new_pairs + ctx_pairs) / ms_fused / 1e9
                                         / PEAK_BF16_TFLOPS, 2),
            "merge_gbs": round(merge_bytes / ms_merge / 1e6, 1),
            "merge_gbs_cold": round(merge_bytes / ms_merge_cold / 1e6, 1),
        }
        dec = np.nonzero(inp.is_decode)[0]
        if len(dec):
            # decode rows alone in one context launch: bytes = local K + V of
            # every decode row's KV head streams + q/out/lse
            wd = scaled_workload(w, w.name + "_decode_only", inp.new_lens[dec], inp.ctx_lens[dec])
            dinp = generate(wd)
            entries = []
            for splits in (1, None):  # one workgroup per (row, KV head); the chosen split
                dshare = RankShare(dinp, device="cuda:0", decode_splits=splits)
                for _ in range(warmup):
                    dshare.context_pass()
                settle(dshare.context_pass)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    dshare.context_pass()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / steps
                ms_cold = time_cold(dshare.context_pass, steps, flush)
                kv = int(dshare.rows_host[:, 8].sum()) * w.num_kv_heads * d * 2 * 2
                io = dshare.total_q * hq * (4 * d + 4)
                entries.append({"rows": dshare.num_rows, "decode_splits": dshare.decode_splits,
                                "ms": round(ms, 4), "bytes": kv + io,
                                "gbs": round((kv + io) / ms / 1e6, 1),
                                "ms_cold": round(ms_cold, 4),
                                "gbs_cold": round((kv + io) / ms_cold / 1e6, 1)})
                del dshare
            line["decode_only_context"] = entries
        from pcp_workloads import quantize_fp8

        s8 = RankShare(inp, device="cuda:0", fp8=quantize_fp8(inp))
        ms8 = time_fused(s8, steps, warmup)
        fl = per_pair * (new_pairs + ctx_pairs)
        line["fp8_fused"] = {"ms": round(ms8, 4), "tflops": round(fl / ms8 / 1e9, 1),
                             "pct_of_fp8_qk_bf16_pv_peak":
                                 round(100 * fl / ms8 / 1e9 / PEAK_FP8_QK_BF16_PV_TFLOPS, 2)}
        del s8
        line["resplit"] = report_resplit(inp, steps, warmup, flush)
        print(json.dumps(line), flush=True)
        del share, inp
        torch.cuda.empty_cache()
    for line in report_decode_batches(steps, warmup, flush):
        print(json.dumps(line), flush=True)
    for line in report_large_batches(steps, warmup):
        print(json.dumps(line), flush=True)
    return 0


def report_large_batches(steps: int, warmup: int):
    """Qwen3-0.6B-shaped prefill batches (16 / 8 heads, d = 128, 4096-token
    requests, pcp2 rank 1) of 32 and 64 requests, whose K/V exceeds the
    256 MB Infinity Cache: the fused launch in the host-made order (which
    keeps each (request, KV head) group of units on one XCD there) and in the
    kernels' built-in order."""
    import torch

    from context_causal_gqa_amd.share import RankShare
    from pcp_workloads import WORKLOADS, generate, scaled_workload

    base = WORKLOADS["qwen3_0p6b_8x4096_pcp2_r1"]
    for b in (32, 64):
        w = scaled_workload(base, "qwen3_0p6b_%dx4096_pcp2_r1" % b, (4096,) * b, (0,) * b)
        log("report: " + w.name)
        inp = generate(w)
        line = {"workload": w.name, "requests": b}
        shares = {key: RankShare(inp, device="cuda:0", schedule=sched)
                  for key, sched in (("host_order", True), ("builtin_order", False))}
        new_pairs, ctx_pairs = plan_pairs(shares["host_order"].rows_host)
        fl = 4 * w.head_dim * w.num_q_heads * (new_pairs + ctx_pairs)
        line["useful_flop"] = fl
        for sh in shares.values():  # the first launches on fresh buffers run ~15% slow
            time_fused(sh, steps, warmup)
        for key, sh in shares.items():
            ms = time_fused(sh, steps, warmup)
            line[key] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                         "pct_bf16_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2)}
        del shares
        yield line
        del inp
        torch.cuda.empty_cache()


def decode_batches():
    """Decode-only batches at sizes where HBM bandwidth, not launch latency,
    decides: the long-context layer of the 256k workload (8 Q / 1 KV heads,
    d = 256, pcp4 dcp4 rank 3) with 16 decode rows at 64k tokens of context,
    and the Qwen3-0.6B-shaped layer (16 / 8 heads, d = 128, pcp2 dcp2 rank 0)
    with 32 decode rows at seeded contexts in [2048, 8192)."""
    import numpy as np

    from pcp_workloads import WORKLOADS, scaled_workload

    rng = np.random.default_rng(7)
    return [
        scaled_workload(WORKLOADS["hybrid_fullattn_256k_ctx64k_pcp4_dcp4_r3"],
                        "decode_batch_16x64k_d256_dcp4_r3", [1] * 16, [65535] * 16),
        scaled_workload(WORKLOADS["mixed_pcp2_dcp2_8prefill_4decode"],
                        "decode_batch_32x2k-8k_d128_dcp2_r0", [1] * 32,
                        rng.integers(2047, 8192, 32)),
    ]


def report_decode_batches(steps: int, warmup: int, flush):
    """HBM bandwidth of the context pass over decode-only batches (row a5),
    unsplit and with the chosen key-range splits, warm and cold, and from
    E4M3 Q/K/V with the chosen splits. Bytes: the local K and V of every
    decode row's KV head, plus q / out / lse."""
    import torch

    from context_causal_gqa_amd.share import RankShare
    from pcp_workloads import generate

    for w in decode_batches():
        log("report: " + w.name)
        inp = generate(w)
        entries = []
        for splits in (1, None):
            sh = RankShare(inp, device="cuda:0", decode_splits=splits)
            ms = time_passes(sh.context_pass, steps, warmup)
            ms_cold = time_cold(sh.context_pass, steps, flush)
            kv = int(sh.rows_host[:, 8].sum()) * w.num_kv_heads * w.head_dim * 2 * 2
            io = sh.total_q * w.num_q_heads * (4 * w.head_dim + 4)
            entries.append({"decode_splits": sh.decode_splits, "bytes": kv + io,
                            "ms": round(ms, 4), "gbs": round((kv + io) / ms / 1e6, 1),
                            "ms_cold": round(ms_cold, 4),
                            "gbs_cold": round((kv + io) / ms_cold / 1e6, 1),
                            "pct_hbm_cold": round(100 * (kv + io) / ms_cold / 1e6 / PEAK_HBM_GBS,
                                                  1)})
            del sh
        # the same batch from E4M3 Q/K/V (one byte per element), chosen splits
        from pcp_workloads import quantize_fp8

        s8 = RankShare(inp, device="cuda:0", fp8=quantize_fp8(inp))
        ms = time_passes(s8.context_pass, steps, warmup)
        ms_cold = time_cold(s8.context_pass, steps, flush)
        kv = int(s8.rows_host[:, 8].sum()) * w.num_kv_heads * w.head_dim * 2
        io = s8.total_q * w.num_q_heads * (3 * w.head_dim + 4)
        fp8 = {"decode_splits": s8.decode_splits, "bytes": kv + io, "ms": round(ms, 4),
               "gbs": round((kv + io) / ms / 1e6, 1), "ms_cold": round(ms_cold, 4),
               "gbs_cold": round((kv + io) / ms_cold / 1e6, 1),
               "pct_hbm_cold": round(100 * (kv + io) / ms_cold / 1e6 / PEAK_HBM_GBS, 1)}
        del s8
        yield {"workload": w.name, "decode_rows": len(w.new_lens), "q_heads": w.num_q_heads,
               "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "context_pass": entries,
               "context_pass_fp8": fp8}
        del inp
        torch.cuda.empty_cache()


def time_passes(fn, steps: int, warmup: int) -> float:
    """Average ms of ``fn`` over ``steps`` back-to-back calls on one stream."""
    import torch

    for _ in range(warmup):
        fn()
    settle(fn)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def resplit_line(name: str, steps: int, warmup: int) -> int:
    """The re-split path of one workload next to its standard fused launch,
    both timed in the same process (what the per-workload report does for
    every workload), printed as one JSON object."""
    import torch

    from context_causal_gqa_amd.share import RankShare
    from pcp_workloads import WORKLOADS, generate

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB, read to evict
    w = WORKLOADS[name]
    inp = generate(w)
    share = RankShare(inp, device="cuda:0")
    new_pairs, ctx_pairs = plan_pairs(share.rows_host)
    fl = 4 * w.head_dim * w.num_q_heads * (new_pairs + ctx_pairs)
    ms = time_fused(share, steps, warmup)
    del share
    torch.cuda.empty_cache()
    line = {"workload": name, "standard_fused": {"useful_flop": fl, "ms": round(ms, 4),
                                                 "tflops": round(fl / ms / 1e9, 1)},
            "resplit": report_resplit(inp, steps, warmup, flush)}
    print(json.dumps(line), flush=True)
    return 0


def report_resplit(inp, steps: int, warmup: int, flush) -> dict:
    """The re-split path on the same inputs: the paged cache write (HBM
    bytes: each written token's K and V read once and written once) and the
    attention launch (useful FLOP of its own plan)."""
    import numpy as np
    import torch

    from context_causal_gqa_amd.share import ResplitShare
    from pcp_workloads import resplit_cache

    w = inp.workload
    rs = ResplitShare(inp, resplit_cache(inp), device="cuda:0")
    written = int((rs.slots_host >= 0).sum())
    wbytes = written * w.num_kv_heads * w.head_dim * 2 * 2 * 2
    for _ in range(warmup):
        rs.step()
    settle(rs.step)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        rs.cache_write()
        e[1].record()
        rs.attend()
        e[2].record()
    torch.cuda.synchronize()
    ms_w = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ms_a = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_w_cold = time_cold(rs.cache_write, steps, flush)
    new_pairs, ctx_pairs = plan_pairs(rs.rows_host)
    fl = 4 * w.head_dim * w.num_q_heads * (new_pairs + ctx_pairs)
    out = {"cache_write": {"tokens": written, "bytes": wbytes, "ms": round(ms_w, 4),
                           "gbs": round(wbytes / ms_w / 1e6, 1) if ms_w > 0 else None,
                           "ms_cold": round(ms_w_cold, 4),
                           "gbs_cold": round(wbytes / ms_w_cold / 1e6, 1) if ms_w_cold > 0 else None},
           "attention": {"useful_flop": fl, "ms": round(ms_a, 4),
                         "tflops": round(fl / ms_a / 1e9, 1)},
           "decode_splits": rs.decode_splits}
    del rs
    torch.cuda.empty_cache()
    return out


def calibrate_copy() -> int:
    import torch

    n = 1 << 28  # float32 elements: 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 5}))
    return 0


def _pmc_means(folder: str, counter: str) -> dict:
    """Mean value of ``counter`` per kernel name over the dispatches of the
    rocprofv3 counter-collection CSV files under ``folder``."""
    import csv
    import glob

    sums, counts = {}, {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no *counter_collection.csv under " + folder)
    for path in files:
        with open(path, newline="") as f:
            for rec in csv.DictReader(f):
                if rec.get("Counter_Name") != counter:
                    continue
                name = rec["Kernel_Name"]
                sums[name] = sums.get(name, 0.0) + float(rec["Counter_Value"])
                counts[name] = counts.get(name, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def write_traffic(root: str, workload: str, out_path: str) -> int:
    """HBM bytes per launch of the attention kernels from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the
    1 GiB ``--calibrate-copy`` launch read and write 1 GiB; entries keyed by
    workload (bf16 fused launch) and workload + ':fp8', with the kernel-code
    sha they were measured on."""
    gib = float(1 << 30)
    scale = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = _pmc_means(os.path.join(root, "copy_" + counter), counter)
        neg = [v for k, v in copy.items() if "neg" in k.lower()]
        kib = max(neg) if neg else max(copy.values())
        scale[counter] = round(gib / (kib * 1024.0), 4)
    fetch = _pmc_means(os.path.join(root, "pmc_FETCH_SIZE"), "FETCH_SIZE")
    write = _pmc_means(os.path.join(root, "pmc_WRITE_SIZE"), "WRITE_SIZE")
    kernels = {k: {"fetch_bytes": int(round(fetch[k] * 1024 * scale["FETCH_SIZE"])),
                   "write_bytes": int(round(write.get(k, 0.0) * 1024 * scale["WRITE_SIZE"]))}
               for k in fetch}
    data = json.load(open(out_path)) if os.path.exists(out_path) else {}
    sha = kernel_source_sha()
    note = ("rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the "
            "factor that makes a 1 GiB torch.neg copy (bench.py --calibrate-copy) read and "
            "write 1 GiB")
    for key, pick in ((workload, lambda k: ", false>" in k and "attn_fwd_kernel<" in k
                       and ", 3, " in k),
                      (workload + ":fp8", lambda k: ", true>" in k and "attn_fwd_kernel<" in k
                       and ", 3, " in k)):
        names = [k for k in kernels if pick(k)]
        if not names:
            continue
        name = names[0]
        e = kernels[name]
        data[key] = {"kernel": name, "kernel_source_sha": sha,
                     "hbm_bytes_per_launch": e["fetch_bytes"] + e["write_bytes"],
                     "fetch_bytes": e["fetch_bytes"], "write_bytes": e["write_bytes"],
                     "calibration": scale, "note": note}
        if not key.endswith(":fp8"):
            data[key]["other_kernels"] = {k: v for k, v in kernels.items() if k != name}
    with open(out_path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps({k: data[k].get("hbm_bytes_per_launch") for k in data}))
    return 0


def traffic_entry(path, key: str):
    """HBM bytes per launch measured for ``key`` by rocprofv3 counters, or
    None when absent or taken on other kernel sources."""
    if not path or not os.path.exists(path):
        return None
    try:
        entry = json.load(open(path)).get(key)
    except Exception:  # pragma: no cover
        return None
    if entry and entry.get("kernel_source_sha") == kernel_source_sha():
        return entry.get("hbm_bytes_per_launch")
    return None


def kernel_source_sha() -> str:
    """sha256[:16] of the attention kernel's code (pcp_attn_fwd.h and
    pcp_geometry.h with comments and blank lines stripped): counters taken on
    other code are not reported, comment edits keep them."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in ("pcp_attn_fwd.h", "pcp_geometry.h"):
        with open(os.path.join(ROOT, "context_causal_gqa_amd", "csrc", name)) as f:
            src = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        lines = [re.sub(r"//.*$", "", line).rstrip() for line in src.split("\n")]
        h.update("\n".join(line for line in lines if line.strip()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
