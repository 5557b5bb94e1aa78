"""GPU parity of the FP8 (E4M3) rank share: the _fp8 entry points through the
C ABI against the fp64 oracle on the dequantized inputs (oracle/fp8.py).

Tolerances are the bf16 path's (out max 2e-2, mean 2e-3, LSE 1e-3): the
kernels compute on the exact E4M3 values (QK^T on the FP8 MFMA, V widened
to bf16 exactly), keep P in bf16 like the bf16 kernels, and fold the
descales into fp32 factors, so the approximation error is the same kind as
on the bf16 path. Plans and the device's query codes are compared exactly.

Small cases cover every head dim with both paged-load paths (block_size a
multiple of the key rows per 1 KB chunk -- 1024 / head_dim for E4M3 -- or
not), GQA groups 1 to 16, decode rows with and without key-range splits, and
descales that differ per (request, KV head); the named workloads at full
size are in test_gpu_workloads.
"""

import numpy as np
import pytest
import torch

import oracle
from pcp_workloads import WORKLOADS, Workload, generate, quantize_fp8

from test_gpu_parity import _np, assert_close, sample_queries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_causal_gqa_amd as m

    return m


def fp8_inputs(inp, jitter_seed=None):
    """FP8 codes and descales of ``inp``; with ``jitter_seed`` each (request,
    KV head) descale is scaled by its own factor in [0.5, 1], so a wrong index
    shows while the dequantized values stay within the workload's N(0, 1)
    range that the absolute tolerances presume."""
    f = quantize_fp8(inp)
    if jitter_seed is not None:
        rng = np.random.default_rng(jitter_seed)
        for t in (f.q_descale, f.k_descale, f.v_descale):
            t *= rng.uniform(0.5, 1.0, size=t.shape).astype(np.float32)
    return f


def oracle_share_fp8(inp, f, share, query_ids=None):
    w = inp.workload
    plan = oracle.plan_rows(inp.cu_seqlens_new, inp.ctx_lens, w.pcp_size, share.pcp_rank,
                            w.dcp_size, share.dcp_rank, w.block_size)
    assert np.array_equal(plan, share.rows_host.astype(np.int64))
    q8 = oracle.gather_local_queries(f.q8.numpy(), inp.cu_seqlens_new, inp.ctx_lens, plan)
    ids = np.arange(len(q8)) if query_ids is None else query_ids
    dev_q = share.q if query_ids is None else share.q[torch.from_numpy(query_ids).cuda()]
    assert np.array_equal(dev_q.cpu().numpy(), q8[ids])  # the device holds the same codes
    return oracle.fp8.rank_share_fp8(q8, f.k8_new, f.v8_new, f.k8_cached, f.v8_cached,
                                     inp.cu_seqlens_new, inp.cu_cache, plan, f.q_descale,
                                     f.k_descale, f.v_descale, w.dcp_size, share.dcp_rank,
                                     w.block_size, w.num_q_heads, w.num_kv_heads,
                                     w.softmax_scale, query_ids=query_ids)


def run_share_fp8(inp, f, **kw):
    """The three FP8 calls, then the fused FP8 launch into NaN-filled buffers."""
    from context_causal_gqa_amd.share import RankShare

    share = RankShare(inp, fp8=f, **kw)
    share.step()
    share.out_fused = torch.full_like(share.out, float("nan"))
    share.lse_fused = torch.full_like(share.lse, float("nan"))
    share.step_fused(out=share.out_fused, lse=share.lse_fused)
    torch.cuda.synchronize()
    return share


def check_share_fp8(inp, f, share, query_ids=None, what=""):
    ref = oracle_share_fp8(inp, f, share, query_ids)
    sel = slice(None) if query_ids is None else torch.from_numpy(query_ids).cuda()
    for key, (o, l) in (("new", (share.out_new, share.lse_new)),
                        ("ctx", (share.out_ctx, share.lse_ctx)),
                        ("merged", (share.out, share.lse)),
                        ("fused", (share.out_fused, share.lse_fused))):
        rk = "merged" if key == "fused" else key
        assert_close(o[sel], l[:, sel], ref[rk][0], ref[rk][1], "%s fp8 %s" % (what, key))


SMALL_FP8 = [
    # name, hq, hkv, d, pcp, rank, dcp, drank, bs, new_lens, ctx_lens
    ("d64_g2_bs16", 4, 2, 64, 2, 1, 1, 0, 16, (300, 77), (0, 0)),
    ("d64_g1_bs8_ctx", 3, 3, 64, 2, 0, 2, 1, 8, (413, 1, 90), (55, 130, 17)),
    ("d128_g2_mixed", 8, 4, 128, 2, 0, 2, 0, 16, (700, 1, 333, 1), (41, 600, 0, 16)),
    ("d128_g4_bs5", 8, 2, 128, 3, 2, 3, 1, 5, (900, 65), (123, 31)),
    ("d128_g16", 16, 1, 128, 2, 0, 1, 0, 16, (200,), (0,)),
    ("d256_g8", 8, 1, 256, 4, 1, 1, 0, 16, (1500,), (0,)),
    ("d256_g8_ctx", 8, 1, 256, 4, 3, 4, 3, 16, (1200, 1), (333, 999)),
    ("d256_g2_bs6", 4, 2, 256, 2, 0, 2, 1, 6, (257, 129), (70, 1)),
    ("d64_g3", 6, 2, 64, 2, 1, 2, 0, 16, (333,), (40,)),
    ("d128_g16_decode", 16, 1, 128, 2, 1, 2, 1, 16, (1, 150, 1), (2000, 64, 500)),
    ("d256_g8_bs32", 8, 1, 256, 2, 1, 2, 0, 32, (300, 1), (250, 700)),
]


@pytest.mark.parametrize("idx", range(len(SMALL_FP8)), ids=[c[0] for c in SMALL_FP8])
def test_fp8_small_rank_share_full_parity(cc, idx):
    name, hq, hkv, d, p, r, dd, rd, bs, new, ctx = SMALL_FP8[idx]
    w = Workload(name=name, seed=5000 + idx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 pcp_size=p, pcp_rank=r, dcp_size=dd, dcp_rank=rd, block_size=bs,
                 new_lens=new, ctx_lens=ctx)
    inp = generate(w)
    f = fp8_inputs(inp, jitter_seed=idx)
    share = run_share_fp8(inp, f)
    check_share_fp8(inp, f, share, what=name)


@pytest.mark.parametrize("splits", [1, 5])
def test_fp8_decode_rows_split_and_whole(cc, splits):
    """Decode rows (one query, cached context only), their key ranges split
    over several workgroups or not, next to a prefill row."""
    w = Workload(name="fp8dec", seed=5100 + splits, num_q_heads=8, num_kv_heads=2, head_dim=128,
                 pcp_size=2, pcp_rank=1, dcp_size=2, dcp_rank=0, block_size=16,
                 new_lens=(1, 1, 260, 1), ctx_lens=(3000, 47, 100, 1200))
    inp = generate(w)
    f = fp8_inputs(inp, jitter_seed=splits)
    share = run_share_fp8(inp, f, decode_splits=splits)
    check_share_fp8(inp, f, share, what="decode splits %d" % splits)


def test_fp8_matches_bf16_path_on_the_same_values(cc):
    """With every descale 2^-7, code * descale is exactly a bf16 value (a
    power-of-two scaling of an E4M3 value) of at most 3.5 in magnitude: the
    bf16 path then sees exactly the FP8 path's values, and both must match
    the oracle."""
    from context_causal_gqa_amd.share import RankShare

    w = Workload(name="fp8eq", seed=5200, num_q_heads=8, num_kv_heads=2, head_dim=256,
                 pcp_size=2, pcp_rank=0, dcp_size=1, dcp_rank=0, block_size=16,
                 new_lens=(640, 1), ctx_lens=(96, 200))
    inp = generate(w)
    f = fp8_inputs(inp)
    ds = 2.0 ** -7
    for t in (f.q_descale, f.k_descale, f.v_descale):
        t[:] = ds
    as_bf16 = lambda c: (c.view(torch.float8_e4m3fn).float() * ds).to(torch.bfloat16)
    inp.q, inp.k_new, inp.v_new = as_bf16(f.q8), as_bf16(f.k8_new), as_bf16(f.v8_new)
    nan = torch.isnan(f.k8_pool.view(torch.float8_e4m3fn).float())
    assert torch.equal(nan, torch.isnan(f.v8_pool.view(torch.float8_e4m3fn).float()))
    inp.k_pool, inp.v_pool = as_bf16(f.k8_pool), as_bf16(f.v8_pool)
    s8 = run_share_fp8(inp, f)
    s16 = RankShare(inp)
    s16.step_fused()
    torch.cuda.synchronize()
    ref = oracle_share_fp8(inp, f, s8)["merged"]
    assert_close(s8.out_fused, s8.lse_fused, ref[0], ref[1], "fp8")
    assert_close(s16.out, s16.lse, ref[0], ref[1], "bf16 on the same values")


# ------------------------------------------------------------------ re-split path


@pytest.mark.parametrize("hkv,d", [(1, 256), (2, 128), (8, 64)])
def test_fp8_kv_cache_write_bit_exact(cc, hkv, d):
    """E4M3 codes land at their slots unchanged; negative slots and slots past
    the pool are skipped; every other byte keeps its 0x7F canary."""
    g = torch.Generator().manual_seed(hkv * 7 + d)
    t, nb, bs = 257, 37, 16
    k = torch.randint(0, 256, (t, hkv, d), generator=g, dtype=torch.uint8)
    v = torch.randint(0, 256, (t, hkv, d), generator=g, dtype=torch.uint8)
    rng = np.random.default_rng(d * 3 + hkv)
    slots = rng.permutation(nb * bs)[:t].astype(np.int64)
    slots[rng.random(t) < 0.2] = -1
    slots[3] = nb * bs + 1  # outside the pool: skipped
    kp = torch.full((nb, bs, hkv, d), 0x7F, dtype=torch.uint8)
    vp = torch.full((nb, bs, hkv, d), 0x7F, dtype=torch.uint8)
    kd, vd = kp.cuda(), vp.cuda()
    cc.pcp_kv_cache_write_fp8(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), kd, vd)
    torch.cuda.synchronize()
    s_ok = np.where(slots < nb * bs, slots, -1)
    want_k, want_v = oracle.kv_cache_write(k.numpy(), v.numpy(), s_ok, kp.numpy(), vp.numpy())
    assert np.array_equal(kd.cpu().numpy(), want_k.astype(np.uint8))
    assert np.array_equal(vd.cpu().numpy(), want_v.astype(np.uint8))


RESPLIT_FP8 = [
    # name, hq, hkv, d, pcp, rank, dcp, drank, bs, new_lens, ctx_lens
    ("d128_dcp2_mixed", 8, 4, 128, 2, 1, 2, 1, 16, (700, 1, 333, 1), (41, 600, 0, 16)),
    ("d256_g8_dcp4", 8, 1, 256, 4, 3, 4, 3, 16, (1200, 1), (333, 999)),
    ("d64_g2_bs5", 4, 2, 64, 2, 0, 3, 2, 5, (413, 1, 90), (55, 130, 17)),
]


@pytest.mark.parametrize("idx", range(len(RESPLIT_FP8)), ids=[c[0] for c in RESPLIT_FP8])
def test_fp8_resplit_share_full_parity(cc, idx):
    """FP8 cache write, then the FP8 fused launch over re-split rows, against
    the oracle's re-split share of the dequantized inputs."""
    from context_causal_gqa_amd.share import ResplitShare
    from pcp_workloads import resplit_cache, resplit_cache_fp8

    name, hq, hkv, d, p, r, dd, rd, bs, new, ctx = RESPLIT_FP8[idx]
    w = Workload(name=name, seed=5300 + idx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 pcp_size=p, pcp_rank=r, dcp_size=dd, dcp_rank=rd, block_size=bs,
                 new_lens=new, ctx_lens=ctx)
    inp = generate(w)
    f = fp8_inputs(inp, jitter_seed=idx)
    cache8 = resplit_cache_fp8(inp, resplit_cache(inp), f)
    share = ResplitShare(inp, cache8, fp8=f)
    share.out.fill_(float("nan"))
    share.step()
    torch.cuda.synchronize()
    cu, cx = inp.cu_seqlens_new, inp.ctx_lens
    plan = oracle.plan_rows_resplit(cu, cx, p, r, dd, rd, bs)
    assert np.array_equal(plan, share.rows_host.astype(np.int64))
    q8 = oracle.gather_local_queries(f.q8.numpy(), cu, cx, plan)
    assert np.array_equal(share.q.cpu().numpy(), q8)
    k8l = oracle.gather_local_queries(f.k8_new.numpy(), cu, cx, plan)
    v8l = oracle.gather_local_queries(f.v8_new.numpy(), cu, cx, plan)
    ref = oracle.fp8.rank_share_resplit_fp8(q8, k8l, v8l, f.k8_new, f.v8_new, cu, f.k8_cached,
                                            f.v8_cached, inp.cu_cache, cx, plan, f.q_descale,
                                            f.k_descale, f.v_descale, dd, rd, bs, hq, hkv,
                                            w.softmax_scale)
    assert_close(share.out, share.lse, ref["merged"][0], ref["merged"][1], name + " fp8 resplit")
