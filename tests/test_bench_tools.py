"""Host-side measurement helpers of bench.py: the HBM-traffic entry written
from rocprofv3 counter runs and its code-sha guard (no GPU)."""

import csv
import json
import os

import bench

BF16 = "void (anonymous namespace)::attn_fwd_kernel<256, 32, 8, 3, false>((anonymous namespace)::AttnArgs)"
FP8 = "void (anonymous namespace)::attn_fwd_kernel<256, 64, 8, 3, true>((anonymous namespace)::AttnArgs)"
NEW = "void (anonymous namespace)::attn_fwd_kernel<256, 32, 8, 0, false>((anonymous namespace)::AttnArgs)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>"


def _write(root, folder, counter, rows):
    d = os.path.join(root, folder, "host")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "123_pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, value) in enumerate(rows):
            w.writerow([i, name, counter, value])


def test_write_traffic_scales_by_the_copy_and_averages_dispatches(tmp_path):
    root = str(tmp_path)
    # the copy reads 1 GiB but FETCH_SIZE reports half of it; WRITE_SIZE reports all
    _write(root, "copy_FETCH_SIZE", "FETCH_SIZE", [(FILL, 20.0), (NEG, 524288.0)])
    _write(root, "copy_WRITE_SIZE", "WRITE_SIZE", [(FILL, 1048576.0), (NEG, 1048576.0)])
    _write(root, "pmc_FETCH_SIZE", "FETCH_SIZE",
           [(BF16, 1000.0), (BF16, 3000.0), (FP8, 500.0), (NEW, 7.0)])
    _write(root, "pmc_WRITE_SIZE", "WRITE_SIZE", [(BF16, 100.0), (FP8, 50.0), (NEW, 1.0)])
    out = os.path.join(root, "traffic.json")
    assert bench.write_traffic(root, "wl", out) == 0
    data = json.load(open(out))
    e = data["wl"]
    assert e["kernel"] == BF16
    assert e["calibration"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    assert e["fetch_bytes"] == 2000 * 1024 * 2  # mean of the two dispatches, KiB, x2
    assert e["write_bytes"] == 100 * 1024
    assert e["hbm_bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    assert e["kernel_source_sha"] == bench.kernel_source_sha()
    assert e["other_kernels"][NEW] == {"fetch_bytes": 7 * 1024 * 2, "write_bytes": 1024}
    f = data["wl:fp8"]
    assert f["kernel"] == FP8 and f["fetch_bytes"] == 500 * 2048 and f["write_bytes"] == 50 * 1024
    # bench.py reports the entry while the kernel code is the one measured ...
    assert bench.traffic_entry(out, "wl") == e["hbm_bytes_per_launch"]
    # ... and null once it is not
    data["wl"]["kernel_source_sha"] = "0" * 16
    json.dump(data, open(out, "w"))
    assert bench.traffic_entry(out, "wl") is None
    assert bench.traffic_entry(os.path.join(root, "missing.json"), "wl") is None


def test_kernel_source_sha_ignores_comments(tmp_path, monkeypatch):
    src = os.path.join(tmp_path, "context_causal_gqa_amd", "csrc")
    os.makedirs(src)
    body = "int f() {\n  return 1;\n}\n"
    for name in ("pcp_attn_fwd.h", "pcp_geometry.h"):
        open(os.path.join(src, name), "w").write(body)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_source_sha()
    open(os.path.join(src, "pcp_attn_fwd.h"), "w").write(
        "// a comment\n/* a block\n comment */\nint f() {  // trailing\n\n  return 1;\n}\n")
    assert bench.kernel_source_sha() == sha
    open(os.path.join(src, "pcp_attn_fwd.h"), "w").write("int f() {\n  return 2;\n}\n")
    assert bench.kernel_source_sha() != sha


def test_cpu_baseline_extrapolates_the_whole_share(monkeypatch):
    """The oracle's rate on the sample and its whole-share time: with every
    query sampled, the extrapolation is the sampled time plus the timed plan;
    the plan it times is the one the share runs."""
    import types

    import numpy as np
    import torch

    import oracle
    from pcp_workloads import Workload, generate

    w = Workload(name="cpu", seed=3, num_q_heads=4, num_kv_heads=2, head_dim=64, pcp_size=2,
                 pcp_rank=1, dcp_size=2, dcp_rank=0, block_size=16, new_lens=(150, 1, 90),
                 ctx_lens=(40, 70, 0))
    inp = generate(w)
    rows = oracle.plan_rows(inp.cu_seqlens_new, inp.ctx_lens, 2, 1, 2, 0, 16).astype(np.int32)
    from context_causal_gqa_amd.share import local_query_index

    qidx = local_query_index(rows, inp.cu_seqlens_new, inp.ctx_lens)
    share = types.SimpleNamespace(rows_host=rows, q=inp.q[torch.from_numpy(qidx)],
                                  total_q=len(qidx), pcp_rank=1, dcp_rank=0)
    out = bench.cpu_baseline(inp, share, budget_s=60.0, seed=1)
    assert out["kind"] == "oracle" and out["value"] > 0
    assert out["sample"].startswith("%d of %d query rows" % (len(qidx), len(qidx)))
    whole = out["whole_share_s"]
    assert whole["kind"] == "extrapolated" and whole["value"] is not None
    new_p, ctx_p = bench.plan_pairs(rows)
    assert str(new_p + ctx_p) in whole["basis"]
    spent = float(out["sample"].rsplit(";", 1)[1].strip().rstrip(" s"))
    assert abs(whole["value"] - spent) <= 0.2  # the sample is the whole share, plus the plan
