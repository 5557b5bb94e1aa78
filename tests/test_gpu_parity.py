"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: out max |err| <= 2e-2 and mean |err| <= 2e-3, LSE |err| <= 1e-3,
row plans and masks exact. Masks are checked exactly through Q = 0 probes:
every score is then 0, so exp(LSE) is the visible key count, which float32
resolves exactly at these sizes.

Every output buffer is NaN-filled before a run and must be fully written
afterwards, with -inf LSEs exactly where the plan leaves a query no key.
Small cases run the oracle on every output; the five named workloads at full
size are in test_gpu_workloads.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import F
from pcp_workloads import WORKLOADS, Workload, generate, scaled_workload

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN, TOL_LSE = 2e-2, 2e-3, 1e-3


@pytest.fixture(scope="module")
def cc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_causal_gqa_amd as m

    assert os.path.exists(m.LIB_PATH), "libpcpattn.so must be built before the GPU tests"
    return m


def _np(t):
    return t.detach().float().cpu().double().numpy()


def assert_close(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    o = _np(out_gpu) if isinstance(out_gpu, torch.Tensor) else out_gpu
    l = _np(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert o.shape == out_ref.shape and l.shape == lse_ref.shape, what
    assert np.isfinite(o).all(), what + ": non-finite output"
    err = np.abs(o - out_ref)
    assert err.max() <= TOL_MAX, "%s: out max err %.3g" % (what, err.max())
    assert err.mean() <= TOL_MEAN, "%s: out mean err %.3g" % (what, err.mean())
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), inf_ref), what + ": -inf LSE pattern differs"
    assert not np.isnan(l).any(), what + ": NaN LSE"
    if (~inf_ref).any():
        lerr = np.abs(l[~inf_ref] - lse_ref[~inf_ref]).max()
        assert lerr <= TOL_LSE, "%s: lse err %.3g" % (what, lerr)


def visible_counts(rows):
    """(new-token, context) visible key counts of every rank-local query: query
    t of a row with q_len m and k_len n sees max(0, min(n, n - m + t + 1)) new
    keys and ctx_len_local context keys."""
    total = int((rows[:, F["q_start"]] + rows[:, F["q_len"]]).max()) if len(rows) else 0
    new = np.zeros(total, dtype=np.int64)
    ctx = np.zeros(total, dtype=np.int64)
    for r in rows:
        qs, m, n = int(r[F["q_start"]]), int(r[F["q_len"]]), int(r[F["k_len"]])
        t = np.arange(m)
        new[qs:qs + m] = np.clip(n - m + t + 1, 0, n)
        ctx[qs:qs + m] = int(r[F["ctx_len_local"]])
    return new, ctx


def assert_written(out, lse, count, what):
    """All of a NaN-prefilled (out, LSE) pair was written: out finite, LSE
    never NaN, and -inf exactly for the queries with no visible key."""
    assert bool(torch.isfinite(out).all()), what + ": an output was not written (or not finite)"
    assert not bool(torch.isnan(lse).any()), what + ": an LSE was not written"
    empty = torch.from_numpy(count == 0).to(lse.device)
    got = torch.isneginf(lse)
    assert bool((got == empty[None, :]).all()), what + ": -inf LSE pattern differs from the plan"


def share_buffers(share):
    """The (name, (out, lse)) pairs a run_share call fills, with the visible
    key count that decides each pair's -inf LSE pattern."""
    new_c, ctx_c = visible_counts(share.rows_host)
    return (("new", (share.out_new, share.lse_new), new_c),
            ("ctx", (share.out_ctx, share.lse_ctx), ctx_c),
            ("merged", (share.out, share.lse), new_c + ctx_c),
            ("fused", (share.out_fused, share.lse_fused), new_c + ctx_c))


def oracle_share(inp, share, query_ids=None):
    w = inp.workload
    q_local = share.q if query_ids is None else share.q[torch.from_numpy(query_ids).cuda()]
    plan = oracle.plan_rows(inp.cu_seqlens_new, inp.ctx_lens, w.pcp_size, share.pcp_rank,
                            w.dcp_size, share.dcp_rank, w.block_size)
    assert np.array_equal(plan, share.rows_host.astype(np.int64))  # plans bit-exact
    ql = oracle.gather_local_queries(inp.q.double().numpy(), inp.cu_seqlens_new, inp.ctx_lens,
                                     plan)
    # the device's gathered query rows are the oracle's, bit for bit
    ids = np.arange(len(ql)) if query_ids is None else query_ids
    assert np.array_equal(_np(q_local), ql[ids])
    return oracle.rank_share(ql, inp.k_new, inp.v_new, inp.k_cached, inp.v_cached, inp.cu_cache,
                             plan, w.dcp_size, share.dcp_rank, w.block_size, w.num_q_heads,
                             w.num_kv_heads, w.softmax_scale, query_ids=query_ids)


def check_share(inp, share, query_ids=None, what=""):
    """Every buffer of a run_share call fully written, then the three calls'
    outputs and the fused launch's against the oracle."""
    for key, (o, l), count in share_buffers(share):
        assert_written(o, l, count, "%s %s" % (what, key))
    ref = oracle_share(inp, share, query_ids)
    sel = slice(None) if query_ids is None else torch.from_numpy(query_ids).cuda()
    for key, (o, l), _ in share_buffers(share):
        rk = "merged" if key == "fused" else key
        assert_close(o[sel], l[:, sel], ref[rk][0], ref[rk][1], "%s %s" % (what, key))


def run_share(cc, inp, **kw):
    """Runs the three-call step and the fused launch, every output buffer
    NaN-filled first, so an output no unit wrote stays NaN."""
    from context_causal_gqa_amd.share import RankShare

    share = RankShare(inp, **kw)
    for a in ("out_new", "lse_new", "out_ctx", "lse_ctx", "out", "lse"):
        getattr(share, a).fill_(float("nan"))
    share.step()
    share.out_fused = torch.full_like(share.out, float("nan"))
    share.lse_fused = torch.full_like(share.lse, float("nan"))
    share.step_fused(out=share.out_fused, lse=share.lse_fused)
    torch.cuda.synchronize()
    return share


def sample_queries(rows, n_random, seed):
    rng = np.random.default_rng(seed)
    ids = set()
    for r in rows:
        qs, ql = int(r[F["q_start"]]), int(r[F["q_len"]])
        ids.update([qs, qs + ql - 1, qs + ql // 2])
        if ql > 33:
            ids.update([qs + 31, qs + 32])
    total = int(rows[:, F["q_start"]].max() + rows[rows[:, F["q_start"]].argmax(), F["q_len"]])
    ids.update(rng.integers(0, total, size=n_random).tolist())
    return np.array(sorted(ids), dtype=np.int64)


# ------------------------------------------------------------------ small cases


SMALL = [
    # name, hq, hkv, d, pcp, rank, dcp, drank, bs, new_lens, ctx_lens
    ("d64_g2", 4, 2, 64, 2, 1, 1, 0, 16, (300, 77), (0, 0)),
    ("d64_g1_ctx", 3, 3, 64, 2, 0, 2, 1, 16, (413, 1, 90), (55, 130, 17)),
    ("d128_g2_mixed", 8, 4, 128, 2, 0, 2, 0, 16, (700, 1, 333, 1), (41, 600, 0, 16)),
    ("d128_g4_bs5", 8, 2, 128, 3, 2, 3, 1, 5, (900, 65), (123, 31)),
    ("d128_g8", 8, 1, 128, 2, 1, 1, 0, 16, (1000,), (0,)),
    ("d256_g8", 8, 1, 256, 4, 1, 1, 0, 16, (1500,), (0,)),
    ("d256_g8_ctx", 8, 1, 256, 4, 3, 4, 3, 16, (1200, 1), (333, 999)),
    ("d256_g2", 4, 2, 256, 2, 0, 2, 1, 16, (257, 129), (70, 1)),
    ("d64_g3", 6, 2, 64, 2, 1, 2, 0, 16, (333,), (40,)),
    ("d128_g16", 16, 1, 128, 2, 0, 1, 0, 16, (200,), (0,)),
    # cache blocks of one wave's rows (8), of one tile (32) and of several
    # tiles (64): every chunk of a wave in one block, full and partial tiles
    ("d256_g4_bs8", 8, 2, 256, 2, 0, 1, 0, 8, (200, 1), (97, 300)),
    ("d256_g8_bs32", 8, 1, 256, 2, 1, 2, 0, 32, (300, 1), (250, 700)),
    ("d128_g2_bs64", 4, 2, 128, 2, 0, 2, 1, 64, (400, 1, 77), (190, 1000, 64)),
]


@pytest.mark.parametrize("idx", range(len(SMALL)), ids=[c[0] for c in SMALL])
def test_small_rank_share_full_parity(cc, idx):
    name, hq, hkv, d, p, r, dd, rd, bs, new, ctx = SMALL[idx]
    w = Workload(name=name, seed=1000 + idx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 pcp_size=p, pcp_rank=r, dcp_size=dd, dcp_rank=rd, block_size=bs,
                 new_lens=new, ctx_lens=ctx)
    inp = generate(w)
    share = run_share(cc, inp)
    check_share(inp, share, what=name)


def test_tiny_workload_full_parity(cc):
    inp = generate(WORKLOADS["tiny_t512_pcp2_r0"])
    share = run_share(cc, inp)
    assert share.rows_host.tolist() == [[0, 0, 0, 128, 0, 0, 128, 0, 0],
                                        [0, 1, 128, 128, 384, 0, 512, 0, 0]]
    check_share(inp, share, what="tiny")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_zero_queries_masks_exact(cc, d):
    """Q = 0: exp(LSE) equals the visible key count exactly, out is the mean of
    the visible V rows (end-aligned causal mask and shard ownership)."""
    w = Workload(name="z", seed=7 + d, num_q_heads=4, num_kv_heads=1, head_dim=d, pcp_size=2,
                 pcp_rank=1, dcp_size=2, dcp_rank=1, block_size=16, new_lens=(611, 1, 96),
                 ctx_lens=(45, 77, 0))
    inp = generate(w)
    inp.q.zero_()
    from context_causal_gqa_amd.share import RankShare

    share = RankShare(inp)
    share.step()
    lse_f = torch.full_like(share.lse, float("nan"))
    share.step_fused(out=torch.empty_like(share.out), lse=lse_f)
    torch.cuda.synchronize()
    rows = share.rows_host
    lse_new = _np(share.lse_new)
    lse_ctx = _np(share.lse_ctx)
    lse = _np(share.lse)
    lse_fused = _np(lse_f)
    for row in rows:
        m, n = int(row[F["q_len"]]), int(row[F["k_len"]])
        for t in range(m):
            qi = int(row[F["q_start"]]) + t
            cnt_new = max(0, n - m + t + 1) if row[F["kind"]] != 2 else 0
            cnt_ctx = int(row[F["ctx_len_local"]])
            for h in range(4):
                for val, cnt in ((lse_new[h, qi], cnt_new), (lse_ctx[h, qi], cnt_ctx),
                                 (lse[h, qi], cnt_new + cnt_ctx),
                                 (lse_fused[h, qi], cnt_new + cnt_ctx)):
                    if cnt == 0:
                        assert val == -math.inf
                    else:
                        assert round(math.exp(val)) == cnt, (row.tolist(), t, h, val, cnt)
    ref = oracle_share(inp, share)
    for key, (o, l) in (("new", (share.out_new, share.lse_new)), ("ctx", (share.out_ctx,
                                                                           share.lse_ctx))):
        assert_close(o, l, ref[key][0], ref[key][1], "zero-q " + key)


def test_padding_rows_untouched_and_deterministic(cc):
    """Rows past the plan stay as they were (NaN canaries), and two runs give
    bit-identical results."""
    w = Workload(name="canary", seed=17, num_q_heads=8, num_kv_heads=2, head_dim=128, pcp_size=2,
                 pcp_rank=0, dcp_size=2, dcp_rank=0, block_size=16, new_lens=(520, 1),
                 ctx_lens=(99, 40))
    inp = generate(w)
    from context_causal_gqa_amd.share import RankShare

    share = RankShare(inp)
    pad = 37
    tq = share.total_q
    q = torch.cat([share.q, torch.randn(pad, 8, 128, device="cuda").bfloat16()])
    outs = []
    for _ in range(2):
        out = torch.full((tq + pad, 8, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((8, tq + pad), float("nan"), dtype=torch.float32, device="cuda")
        cc.pcp_attn_prefill(q, share.k, share.v, share.rows, out, lse, share.scale,
                            share.max_q_len, rows_host=share.rows_host)
        out2 = torch.full_like(out, float("nan"))
        lse2 = torch.full_like(lse, float("nan"))
        cc.pcp_attn_context_paged(q, share.k_cache, share.v_cache, share.block_tables,
                                  share.rows, out2, lse2, share.scale, share.max_q_len,
                                  rows_host=share.rows_host)
        out3 = torch.full_like(out, float("nan"))
        lse3 = torch.full_like(lse, float("nan"))
        cc.pcp_attn_rank_share(q, share.k, share.v, share.k_cache, share.v_cache,
                               share.block_tables, share.rows, out3, lse3, share.scale,
                               share.max_q_len, rows_host=share.rows_host)
        torch.cuda.synchronize()
        for o, l in ((out, lse), (out2, lse2), (out3, lse3)):
            assert torch.isnan(o[tq:].float()).all() and torch.isnan(l[:, tq:]).all()
            assert not torch.isnan(o[:tq].float()).any()
        outs.append((out[:tq].clone(), lse[:, :tq].clone(), out2[:tq].clone(), lse2[:, :tq].clone(),
                     out3[:tq].clone(), lse3[:, :tq].clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_reassembly_all_ranks_equals_full_attention(cc):
    """Every PCP rank's rows, merged on the GPU over the new-token pass and the
    context passes of all DCP shards, equal unsplit causal attention."""
    p, dd = 2, 2
    w = Workload(name="re", seed=23, num_q_heads=8, num_kv_heads=2, head_dim=128, pcp_size=p,
                 pcp_rank=0, dcp_size=dd, dcp_rank=0, block_size=16, new_lens=(437, 1, 200),
                 ctx_lens=(150, 300, 0))
    inp = generate(w)
    from context_causal_gqa_amd.share import RankShare

    tot = int(inp.cu_seqlens_new[-1])
    full_o = np.full((tot, 8, 128), np.nan)
    full_l = np.full((8, tot), np.nan)
    for r in range(p):
        share = RankShare(inp, pcp_rank=r, dcp_rank=0)
        share.new_token_pass()
        outs, lses = [share.out_new], [share.lse_new]
        for rd in range(dd):
            bt = torch.from_numpy(inp.rank_block_tables[rd]).cuda()
            rows_h = cc.pcp_plan_rows(inp.cu_seqlens_new, inp.ctx_lens, p, r, dd, rd, 16)
            rows_d = torch.from_numpy(rows_h).cuda()
            o = torch.empty_like(share.out_new)
            l = torch.empty_like(share.lse_new)
            cc.pcp_attn_context_paged(share.q, share.k_cache, share.v_cache, bt, rows_d, o, l,
                                      share.scale, share.max_q_len, rows_host=rows_h)
            outs.append(o)
            lses.append(l)
        cc.lse_merge(outs, lses, share.out, share.lse)
        torch.cuda.synchronize()
        o = _np(share.out)
        l = _np(share.lse)
        full_o[share.qidx] = o
        full_l[:, share.qidx] = l
    assert not np.isnan(full_o).any()
    ref_o, ref_l = oracle.full_causal_attention(inp.q, inp.k_new, inp.v_new, inp.k_cached,
                                                inp.v_cached, inp.cu_seqlens_new, inp.ctx_lens,
                                                inp.cu_cache, 8, 2, w.softmax_scale)
    assert_close(full_o, full_l, ref_o, ref_l, "reassembled")


def test_reassembly_with_fused_launch_equals_full_attention(cc):
    """Per PCP rank: the fused launch (new tokens + DCP shard 0's context)
    LSE-merged with the other shards' context passes equals unsplit causal
    attention over all ranks."""
    p, dd = 2, 3
    w = Workload(name="ref", seed=29, num_q_heads=8, num_kv_heads=1, head_dim=256, pcp_size=p,
                 pcp_rank=0, dcp_size=dd, dcp_rank=0, block_size=16, new_lens=(301, 1, 129, 1),
                 ctx_lens=(170, 260, 0, 33))
    inp = generate(w)
    from context_causal_gqa_amd.share import RankShare

    tot = int(inp.cu_seqlens_new[-1])
    full_o = np.full((tot, 8, 256), np.nan)
    full_l = np.full((8, tot), np.nan)
    for r in range(p):
        share = RankShare(inp, pcp_rank=r, dcp_rank=0)
        share.step_fused()
        outs, lses = [share.out], [share.lse]
        for rd in range(1, dd):
            bt = torch.from_numpy(inp.rank_block_tables[rd]).cuda()
            rows_h = cc.pcp_plan_rows(inp.cu_seqlens_new, inp.ctx_lens, p, r, dd, rd, 16)
            o = torch.empty_like(share.out)
            l = torch.empty_like(share.lse)
            cc.pcp_attn_context_paged(share.q, share.k_cache, share.v_cache, bt,
                                      torch.from_numpy(rows_h).cuda(), o, l, share.scale,
                                      share.max_q_len, rows_host=rows_h)
            outs.append(o)
            lses.append(l)
        m_o = torch.empty_like(share.out)
        m_l = torch.empty_like(share.lse)
        cc.lse_merge(outs, lses, m_o, m_l)
        torch.cuda.synchronize()
        full_o[share.qidx] = _np(m_o)
        full_l[:, share.qidx] = _np(m_l)
    assert not np.isnan(full_o).any()
    ref_o, ref_l = oracle.full_causal_attention(inp.q, inp.k_new, inp.v_new, inp.k_cached,
                                                inp.v_cached, inp.cu_seqlens_new, inp.ctx_lens,
                                                inp.cu_cache, 8, 1, w.softmax_scale)
    assert_close(full_o, full_l, ref_o, ref_l, "reassembled (fused)")


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 16])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_lse_merge_vs_oracle(cc, k, d):
    g = torch.Generator().manual_seed(k * 100 + d)
    tq, hq = 203, 6
    outs = [torch.randn(tq, hq, d, generator=g).bfloat16() for _ in range(k)]
    lses = [torch.randn(hq, tq, generator=g) * 5 for _ in range(k)]
    for i in range(k):  # some empty partials, and one (query, head) empty in all
        mask = torch.rand(hq, tq, generator=g) < 0.2
        lses[i][mask] = float("-inf")
        outs[i].transpose(0, 1)[mask] = 0
        lses[i][2, 7] = float("-inf")
        outs[i][7, 2] = 0
    ref_o, ref_l = oracle.lse_merge([(o, l) for o, l in zip(outs, lses)])
    od = [o.cuda() for o in outs]
    ld = [l.cuda() for l in lses]
    out = torch.empty_like(od[0])
    lse = torch.empty_like(ld[0])
    cc.lse_merge(od, ld, out, lse)
    torch.cuda.synchronize()
    assert_close(out, lse, ref_o, ref_l, "merge k=%d" % k)
    # in place into the first partial
    cc.lse_merge(od, ld, od[0], ld[0])
    torch.cuda.synchronize()
    assert torch.equal(od[0].view(torch.int16), out.view(torch.int16))
    assert torch.equal(ld[0], lse)


def test_empty_context_gives_neg_inf_not_skip(cc):
    """A row with no local context writes (0, -inf) -- the pass is not skipped
    (an early return once made rows silently ignore their context)."""
    w = Workload(name="e", seed=5, num_q_heads=4, num_kv_heads=2, head_dim=64, pcp_size=2,
                 pcp_rank=0, dcp_size=4, dcp_rank=3, block_size=16, new_lens=(64, 1),
                 ctx_lens=(20, 10))  # rank 3 holds none of these cached blocks
    inp = generate(w)
    from context_causal_gqa_amd.share import RankShare

    share = RankShare(inp)
    share.out_ctx.fill_(float("nan"))
    share.lse_ctx.fill_(float("nan"))
    share.step()
    share.out_fused = torch.full_like(share.out, float("nan"))
    share.lse_fused = torch.full_like(share.lse, float("nan"))
    share.step_fused(out=share.out_fused, lse=share.lse_fused)
    torch.cuda.synchronize()
    assert (share.rows_host[:, F["ctx_len_local"]] == 0).all()
    assert torch.equal(share.out_ctx.float(), torch.zeros_like(share.out_ctx.float()))
    assert torch.isneginf(share.lse_ctx).all()
    check_share(inp, share, what="empty ctx")


# ------------------------------------------------------- split decode rows


SPLIT = [
    # name, hq, hkv, d, dcp, drank, bs, new_lens, ctx_lens, splits
    ("d256_g8_bs16", 8, 1, 256, 2, 1, 16, (1, 1, 1, 200), (4000, 1500, 37, 900), (2, 7, 256)),
    ("d128_g4_bs5", 8, 2, 128, 1, 0, 5, (1, 1, 64), (3000, 0, 500), (3, 64)),
    ("d128_g2_bs16", 8, 4, 128, 2, 0, 16, (1, 300, 1, 1), (2500, 100, 6000, 16), (5, 33)),
    ("d64_g1_bs16", 4, 4, 64, 4, 2, 16, (1,) * 6, (9000, 5, 700, 0, 2100, 64), (4, 100)),
    # more heads per KV head than one unit packs: 16 -> two units of 8, 6 -> three of 2
    ("d128_g16_bs16", 16, 1, 128, 2, 1, 16, (1, 90, 1), (3100, 700, 260), (3, 17)),
    ("d64_g6_bs8", 12, 2, 64, 2, 0, 8, (1, 1, 40, 1), (1900, 33, 300, 5000), (2, 9)),
]


@pytest.mark.parametrize("idx", range(len(SPLIT)), ids=[c[0] for c in SPLIT])
def test_split_decode_rows_parity(cc, idx):
    """One-query rows cut into key ranges (empty ranges included, the
    workspace holding NaN on entry) match the oracle and the unsplit pass;
    the multi-query rows of the batch are unaffected."""
    name, hq, hkv, d, dd, rd, bs, new, ctx, splits = SPLIT[idx]
    w = Workload(name=name, seed=2000 + idx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 pcp_size=2, pcp_rank=1, dcp_size=dd, dcp_rank=rd, block_size=bs,
                 new_lens=new, ctx_lens=ctx)
    inp = generate(w)
    from context_causal_gqa_amd.share import RankShare

    base = run_share(cc, inp, decode_splits=1)
    assert base.workspace is None
    ref = oracle_share(inp, base)
    assert_close(base.out_ctx, base.lse_ctx, ref["ctx"][0], ref["ctx"][1], name + " unsplit")
    dec = base.rows_host[:, F["q_len"]] == 1
    assert dec.any()
    for s in splits:
        print("%s splits=%d" % (name, s), flush=True)
        share = RankShare(inp, decode_splits=s)
        assert share.workspace is not None
        share.workspace.fill_(float("nan"))
        share.out_ctx.fill_(float("nan"))
        share.step()
        out_f = torch.full_like(share.out, float("nan"))
        lse_f = torch.full_like(share.lse, float("nan"))
        share.workspace.fill_(float("nan"))
        share.step_fused(out=out_f, lse=lse_f)  # the same splits in the fused launch
        torch.cuda.synchronize()
        what = "%s splits=%d" % (name, s)
        assert_close(share.out_ctx, share.lse_ctx, ref["ctx"][0], ref["ctx"][1], what + " ctx")
        assert_close(share.out, share.lse, ref["merged"][0], ref["merged"][1], what + " merged")
        assert_close(out_f, lse_f, ref["merged"][0], ref["merged"][1], what + " fused")
        # rows with several queries take the unsplit code path: bit-identical
        multi = np.concatenate([np.arange(r[F["q_start"]], r[F["q_start"]] + r[F["q_len"]])
                                for r in base.rows_host[~dec]] or [np.zeros(0, np.int64)])
        if len(multi):
            sel = torch.from_numpy(multi).cuda()
            assert torch.equal(share.out_ctx[sel], base.out_ctx[sel]), what
            assert torch.equal(share.lse_ctx[:, sel], base.lse_ctx[:, sel]), what
        # one-query rows: the split result is the unsplit one up to rounding
        one = torch.from_numpy(base.rows_host[dec, F["q_start"]].astype(np.int64)).cuda()
        diff = (share.out_ctx[one].float() - base.out_ctx[one].float()).abs().max().item()
        assert diff <= 1e-2, "%s: split vs unsplit %.3g" % (what, diff)


# ------------------------------------------------------------ launch order


@pytest.mark.parametrize("name,splits", [("qwen3_0p6b_8x4096_pcp2_r1", None),
                                         ("mixed_pcp2_dcp2_8prefill_4decode", None),
                                         ("mixed_pcp2_dcp2_8prefill_4decode", 1)])
def test_scheduled_order_matches_builtin_order(cc, name, splits):
    """A unit's arithmetic does not depend on when it runs: launches in the
    host-made order (pcp_attn_schedule) and in the built-in order give
    bit-identical outputs."""
    inp = generate(WORKLOADS[name])
    a = run_share(cc, inp, schedule=False, decode_splits=splits)
    b = run_share(cc, inp, schedule=True, decode_splits=splits)
    assert b.order_new is not None and b.order_ctx is not None
    assert b.order_fused is not None
    for x, y in ((a.out_new, b.out_new), (a.lse_new, b.lse_new), (a.out_ctx, b.out_ctx),
                 (a.lse_ctx, b.lse_ctx), (a.out, b.out), (a.lse, b.lse),
                 (a.out_fused, b.out_fused), (a.lse_fused, b.lse_fused)):
        assert torch.equal(x, y), name


def test_degenerate_ranks_and_zero_size_calls(cc):
    """pcp 4 over a 3-token prompt and a one-token request with a cached
    prefix: rank 0 gets a one-query prefill row, ranks 1 and 2 one each too,
    rank 3 only the decode row, and with dcp 4 some shards hold no cached
    token. Every rank's three calls and fused launch match the oracle; a
    rank without rows, a merge of zero queries and a cache write of zero
    tokens are no-ops through the C ABI."""
    from context_causal_gqa_amd.share import RankShare

    w = Workload(name="degenerate", seed=41, num_q_heads=4, num_kv_heads=2, head_dim=64,
                 pcp_size=4, pcp_rank=0, dcp_size=4, dcp_rank=0, block_size=16,
                 new_lens=(3, 1), ctx_lens=(0, 40))
    inp = generate(w)
    for r in range(4):
        share = run_share(cc, inp, pcp_rank=r, dcp_rank=r)
        rows = share.rows_host
        assert len(rows) == (2 if r < 3 else 1)
        check_share(inp, share, what="degenerate rank %d" % r)

    # no rows at all: every pass returns at once and writes nothing
    w0 = Workload(name="no_rows", seed=42, num_q_heads=4, num_kv_heads=2, head_dim=64,
                  pcp_size=4, pcp_rank=3, dcp_size=1, dcp_rank=0, block_size=16,
                  new_lens=(3,), ctx_lens=(0,))
    share = RankShare(generate(w0))
    assert share.num_rows == 0 and share.total_q == 0
    share.step()
    share.step_fused()
    torch.cuda.synchronize()

    # zero queries to merge, zero tokens to write: untouched outputs
    o = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    l = torch.zeros((4, 0), dtype=torch.float32, device="cuda")
    cc.lse_merge([o, o], [l, l], o, l)
    kc = torch.full((2, 16, 2, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    vc = kc.clone()
    kv = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    cc.pcp_kv_cache_write(kv, kv, torch.zeros(0, dtype=torch.int64, device="cuda"), kc, vc)
    torch.cuda.synchronize()
    assert (kc == 3.0).all() and (vc == 3.0).all()


def test_kv_grouped_order_past_the_cache(cc):
    """32 Qwen-shaped requests read 403 MB of K/V, more than the Infinity
    Cache: the host-made order keeps each (request, KV head) group of units
    on one XCD, and its outputs are bit-identical to the built-in order's and
    match the oracle on sampled queries."""
    w = scaled_workload(WORKLOADS["qwen3_0p6b_8x4096_pcp2_r1"], "qwen_32x4096", (4096,) * 32,
                        (0,) * 32)
    inp = generate(w)
    a = run_share(cc, inp, schedule=False)
    b = run_share(cc, inp, schedule=True)
    order = b.order_fused.cpu().numpy()
    g = w.num_q_heads // w.num_kv_heads
    hg = next(h for h in (8, 4, 2, 1) if g % h == 0)
    groups, qt = w.num_kv_heads * (g // hg), -(-b.max_q_len // (256 // hg))
    xcd_of = {}
    for i, u in enumerate(order.tolist()):
        if u < 0:
            continue
        row, grp = u // (groups * qt), (u // qt) % groups
        key = (int(b.rows_host[row, F["req"]]), grp // (g // hg))
        assert xcd_of.setdefault(key, i % 8) == i % 8, "a K/V group spans XCDs"
    assert len(xcd_of) == 32 * w.num_kv_heads
    for x, y in ((a.out_fused, b.out_fused), (a.lse_fused, b.lse_fused), (a.out, b.out)):
        assert torch.equal(x, y)
    check_share(inp, b, query_ids=sample_queries(b.rows_host, 64, seed=32), what=w.name)


@pytest.mark.parametrize("fp8", [False, True])
def test_pool_beyond_4gib_takes_the_generic_paged_path(cc, fp8):
    """A paged pool of 4 GiB or more cannot be reached with the 32-bit offsets
    of the uniform-block loads, so the launcher must take the generic path:
    the workload's blocks are placed at the top of a >4 GiB pool (offsets past
    2^32) and the context pass must still match the oracle."""
    from context_causal_gqa_amd.share import RankShare
    from pcp_workloads import quantize_fp8

    w = Workload(name="bigpool", seed=1900, num_q_heads=4, num_kv_heads=1, head_dim=64,
                 pcp_size=2, pcp_rank=0, dcp_size=1, dcp_rank=0, block_size=16,
                 new_lens=(96, 1), ctx_lens=(300, 200))
    inp = generate(w)
    f8 = quantize_fp8(inp) if fp8 else None
    share = RankShare(inp, fp8=f8)
    elem = 1 if fp8 else 2
    block_bytes = w.block_size * w.num_kv_heads * w.head_dim * elem
    nb_small = share.k_cache.shape[0]
    nb_big = (1 << 32) // block_bytes + nb_small + 8  # pool just over 4 GiB
    shift = nb_big - nb_small  # the workload's blocks go to the top
    fill = 0x7F if fp8 else float("nan")
    dt = share.k_cache.dtype
    big_k = torch.full((nb_big,) + tuple(share.k_cache.shape[1:]), fill, dtype=dt, device="cuda")
    big_v = torch.full_like(big_k, fill)
    big_k[shift:] = share.k_cache
    big_v[shift:] = share.v_cache
    bt = share.block_tables.clone()
    bt[bt >= 0] += shift
    share.k_cache, share.v_cache, share.block_tables = big_k, big_v, bt
    share.out_ctx.fill_(float("nan"))
    share.context_pass()
    torch.cuda.synchronize()
    plan = share.rows_host.astype(np.int64)
    if fp8:
        q8 = oracle.gather_local_queries(f8.q8.numpy(), inp.cu_seqlens_new, inp.ctx_lens, plan)
        ref = oracle.fp8.rank_share_fp8(q8, f8.k8_new, f8.v8_new, f8.k8_cached, f8.v8_cached,
                                        inp.cu_seqlens_new, inp.cu_cache, plan, f8.q_descale,
                                        f8.k_descale, f8.v_descale, 1, 0, 16, 4, 1,
                                        w.softmax_scale)["ctx"]
    else:
        ref = oracle_share(inp, share)["ctx"]
    assert_close(share.out_ctx, share.lse_ctx, ref[0], ref[1], "pool > 4 GiB")
    del big_k, big_v
    torch.cuda.empty_cache()
