"""Every output of a full-size rank share against the fp64 oracle, once.

The GPU tests check the named workloads at full size on sampled queries
(every row's boundaries plus random ones); this script checks all of them.
It runs one path on cuda:0 -- the fused launch (default), the three calls
(--path three) or the re-split path, cache write then the fused launch over
re-split rows (--path resplit) -- in bf16, or FP8 with --fp8, then the
oracle over every query in chunks, printing progress after each chunk, and
writes a JSON summary (max / mean |err| of out over all outputs, max |err|
of LSE, the -inf pattern) to --out. Minutes of CPU work at the 128k and 256k
shares, so it is a script, not a collected test.

    python tests/full_share_parity.py --workload hybrid_fullattn_128k_pcp4_r1 [--fp8] [--path three]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
from pcp_workloads import WORKLOADS, generate, quantize_fp8  # noqa: E402

TOL_MAX, TOL_MEAN, TOL_LSE = 2e-2, 2e-3, 1e-3


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="hybrid_fullattn_128k_pcp4_r1")
    ap.add_argument("--fp8", action="store_true")
    ap.add_argument("--path", choices=("fused", "three", "resplit"), default="fused")
    ap.add_argument("--chunk", type=int, default=2048)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    from context_causal_gqa_amd.share import RankShare, ResplitShare

    w = WORKLOADS[args.workload]
    print("generating", w.name, flush=True)
    inp = generate(w)
    f8 = quantize_fp8(inp) if args.fp8 else None
    cu, cx = inp.cu_seqlens_new, inp.ctx_lens
    if args.path == "resplit":
        from pcp_workloads import resplit_cache, resplit_cache_fp8

        cache = resplit_cache(inp)
        if args.fp8:
            cache = resplit_cache_fp8(inp, cache, f8)
        share = ResplitShare(inp, cache, device="cuda:0", fp8=f8)
        share.out.fill_(float("nan"))
        share.lse.fill_(float("nan"))
        share.step()
        plan = oracle.plan_rows_resplit(cu, cx, w.pcp_size, share.pcp_rank, w.dcp_size,
                                        share.dcp_rank, w.block_size)
        slots = oracle.slot_mapping(cu, cx, cache.block_table, w.dcp_size, share.dcp_rank,
                                    w.block_size)
        assert np.array_equal(slots, share.slots_host), "slot mapping differs"
    else:
        share = RankShare(inp, device="cuda:0", fp8=f8)
        share.out.fill_(float("nan"))
        share.lse.fill_(float("nan"))
        if args.path == "three":
            share.step()
        else:
            share.step_fused()
        plan = oracle.plan_rows(cu, cx, w.pcp_size, share.pcp_rank, w.dcp_size, share.dcp_rank,
                                w.block_size)
    torch.cuda.synchronize()
    out = share.out.float().cpu().double().numpy()
    lse = share.lse.cpu().double().numpy()
    assert np.array_equal(share.rows_host.astype(np.int64), plan), "row plan differs"
    if args.path == "resplit" and args.fp8:
        q8l = oracle.gather_local_queries(f8.q8.numpy(), cu, cx, plan)
        k8l = oracle.gather_local_queries(f8.k8_new.numpy(), cu, cx, plan)
        v8l = oracle.gather_local_queries(f8.v8_new.numpy(), cu, cx, plan)
    elif args.path == "resplit":
        def gather(x):  # exact bf16 bit patterns, gathered by the oracle, widened
            bits = oracle.gather_local_queries(x.view(torch.int16).numpy(), cu, cx, plan)
            return torch.from_numpy(bits).view(torch.bfloat16).double().numpy()

        ql, kl, vl = gather(inp.q), gather(inp.k_new), gather(inp.v_new)
        kn, vn = inp.k_new.double().numpy(), inp.v_new.double().numpy()
        kc, vc = inp.k_cached.double().numpy(), inp.v_cached.double().numpy()
    elif args.fp8:
        q_local = oracle.gather_local_queries(f8.q8.numpy(), cu, cx, plan)
        req_q = oracle.fp8.query_requests(plan)
        g = w.num_q_heads // w.num_kv_heads
        req_new, req_c = oracle.fp8.token_requests(cu), oracle.fp8.token_requests(inp.cu_cache)
        ql = oracle.fp8.dequantize(q_local, f8.q_descale, req_q, g)
        kn = oracle.fp8.dequantize(f8.k8_new, f8.k_descale, req_new, 1)
        vn = oracle.fp8.dequantize(f8.v8_new, f8.v_descale, req_new, 1)
        kc = oracle.fp8.dequantize(f8.k8_cached, f8.k_descale, req_c, 1)
        vc = oracle.fp8.dequantize(f8.v8_cached, f8.v_descale, req_c, 1)
    else:
        ql = oracle.gather_local_queries(inp.q.double().numpy(), cu, cx, plan)
        kn, vn = inp.k_new.double().numpy(), inp.v_new.double().numpy()
        kc, vc = inp.k_cached.double().numpy(), inp.v_cached.double().numpy()
    total_q = share.total_q
    err_max = lse_max = 0.0
    err_sum = 0.0
    n_out = 0
    inf_ok = True
    t0 = time.time()
    for c0 in range(0, total_q, args.chunk):
        ids = np.arange(c0, min(total_q, c0 + args.chunk))
        if args.path == "resplit" and args.fp8:
            ref = oracle.fp8.rank_share_resplit_fp8(
                q8l, k8l, v8l, f8.k8_new, f8.v8_new, cu, f8.k8_cached, f8.v8_cached, inp.cu_cache,
                cx, plan, f8.q_descale, f8.k_descale, f8.v_descale, w.dcp_size, share.dcp_rank,
                w.block_size, w.num_q_heads, w.num_kv_heads, w.softmax_scale,
                query_ids=ids)["merged"]
        elif args.path == "resplit":
            ref = oracle.rank_share_resplit(ql, kl, vl, kn, vn, cu, kc, vc, inp.cu_cache, cx,
                                            plan, w.dcp_size, share.dcp_rank, w.block_size,
                                            w.num_q_heads, w.num_kv_heads, w.softmax_scale,
                                            query_ids=ids)["merged"]
        else:
            ref = oracle.rank_share(ql, kn, vn, kc, vc, inp.cu_cache, plan, w.dcp_size,
                                    share.dcp_rank, w.block_size, w.num_q_heads,
                                    w.num_kv_heads, w.softmax_scale, query_ids=ids)["merged"]
        e = np.abs(out[ids] - ref[0])
        err_max = max(err_max, float(e.max()))
        err_sum += float(e.sum())
        n_out += e.size
        rl, gl = ref[1], lse[:, ids]
        inf_ok &= bool(np.array_equal(np.isneginf(rl), np.isneginf(gl)))
        fin = ~np.isneginf(rl)
        if fin.any():
            lse_max = max(lse_max, float(np.abs(gl[fin] - rl[fin]).max()))
        print("queries %d/%d: out max %.3e mean %.3e, lse max %.3e (%.0f s)"
              % (ids[-1] + 1, total_q, err_max, err_sum / n_out, lse_max, time.time() - t0),
              flush=True)
    from bench import kernel_source_sha

    summary = {
        "workload": w.name,
        "path": "%s %s" % ("fp8" if args.fp8 else "bf16",
                           {"fused": "fused", "three": "three calls", "resplit": "re-split"}[args.path]),
        "kernel_source_sha": kernel_source_sha(),
        "queries": total_q, "heads": w.num_q_heads, "head_dim": w.head_dim,
        "outputs_checked": n_out, "out_max_abs_err": err_max, "out_mean_abs_err": err_sum / n_out,
        "lse_max_abs_err": lse_max, "neg_inf_pattern_equal": inf_ok,
        "tolerances": {"out_max": TOL_MAX, "out_mean": TOL_MEAN, "lse": TOL_LSE},
        "oracle_seconds": round(time.time() - t0, 1),
        "pass": err_max <= TOL_MAX and err_sum / n_out <= TOL_MEAN and lse_max <= TOL_LSE
        and inf_ok and bool(np.isfinite(out).all()),
    }
    print(json.dumps(summary), flush=True)
    if args.out:
        with open(args.out, "w") as fh:
            json.dump(summary, fh, indent=1)
    return 0 if summary["pass"] else 1


if __name__ == "__main__":
    sys.exit(main())
