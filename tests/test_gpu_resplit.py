"""GPU parity of the re-split path: the paged KV-cache write, then each row
attending over [0, row_start) from this DCP rank's cache shard plus its own
tokens, square causal -- against the fp64 oracle (same tolerances as
test_gpu_parity: out max 2e-2 / mean 2e-3, LSE 1e-3; the cache write and the
slot mapping bit-exact)."""

import numpy as np
import pytest
import torch

import oracle
from pcp_workloads import WORKLOADS, Workload, generate, resplit_cache

from test_gpu_parity import _np, assert_close, sample_queries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_causal_gqa_amd as m

    return m


@pytest.mark.parametrize("hkv,d", [(1, 256), (2, 128), (8, 64)])
def test_kv_cache_write_bit_exact(cc, hkv, d):
    """Every token lands at its slot; negative slots and slots past the pool
    are skipped; nothing else changes (NaN canaries)."""
    g = torch.Generator().manual_seed(hkv * 1000 + d)
    t, nb, bs = 301, 41, 16
    k = torch.randn(t, hkv, d, generator=g).bfloat16()
    v = torch.randn(t, hkv, d, generator=g).bfloat16()
    rng = np.random.default_rng(d + hkv)
    slots = rng.permutation(nb * bs)[:t].astype(np.int64)
    slots[rng.random(t) < 0.2] = -1
    slots[5] = nb * bs + 3  # outside the pool: skipped
    kp = torch.full((nb, bs, hkv, d), float("nan")).bfloat16()
    vp = torch.full((nb, bs, hkv, d), float("nan")).bfloat16()
    kd, vd = kp.cuda(), vp.cuda()
    cc.pcp_kv_cache_write(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), kd, vd)
    torch.cuda.synchronize()
    s_ok = np.where(slots < nb * bs, slots, -1)
    want_k, want_v = oracle.kv_cache_write(k, v, s_ok, kp, vp)
    for got, want in ((kd, want_k), (vd, want_v)):
        got = _np(got)
        assert np.array_equal(np.isnan(got), np.isnan(want))
        assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])


def _gather_bf16(x, cu, ctx, plan):
    """Rank-local rows of a bf16 [T, H, d] tensor, gathered on exact int16 bit
    patterns by the oracle's own gather, then widened to float64."""
    bits = oracle.gather_local_queries(x.view(torch.int16).numpy(), cu, ctx, plan)
    return torch.from_numpy(bits).view(torch.bfloat16).double().numpy()


def _resplit_oracle(inp, share, query_ids=None):
    w = inp.workload
    plan = oracle.plan_rows_resplit(inp.cu_seqlens_new, inp.ctx_lens, w.pcp_size,
                                    share.pcp_rank, w.dcp_size, share.dcp_rank, w.block_size)
    assert np.array_equal(plan, share.rows_host.astype(np.int64))
    slots = oracle.slot_mapping(inp.cu_seqlens_new, inp.ctx_lens, share.cache_table, w.dcp_size,
                                share.dcp_rank, w.block_size)
    assert np.array_equal(slots, share.slots_host)
    cu, ctx = inp.cu_seqlens_new, inp.ctx_lens
    ql = _gather_bf16(inp.q, cu, ctx, plan)
    kl = _gather_bf16(inp.k_new, cu, ctx, plan)
    vl = _gather_bf16(inp.v_new, cu, ctx, plan)
    ids = np.arange(len(ql)) if query_ids is None else query_ids
    assert np.array_equal(_np(share.q)[ids], ql[ids])  # the device rows are the oracle's
    return oracle.rank_share_resplit(ql, kl, vl, inp.k_new, inp.v_new, cu, inp.k_cached,
                                     inp.v_cached, inp.cu_cache, ctx, plan, w.dcp_size,
                                     share.dcp_rank, w.block_size, w.num_q_heads,
                                     w.num_kv_heads, w.softmax_scale, query_ids=query_ids)


def _make_share(cc, inp, cache, **kw):
    from context_causal_gqa_amd.share import ResplitShare

    share = ResplitShare(inp, cache, **kw)
    share.cache_table = cache.block_table
    return share


RESPLIT = [
    # name, hq, hkv, d, pcp, rank, dcp, drank, bs, new_lens, ctx_lens
    ("d128_dcp2_mixed", 8, 4, 128, 2, 1, 2, 1, 16, (700, 1, 333, 1), (41, 600, 0, 16)),
    ("d256_g8_dcp4", 8, 1, 256, 4, 3, 4, 3, 16, (1200, 1), (333, 999)),
    ("d64_g2_bs5", 4, 2, 64, 2, 0, 3, 2, 5, (413, 1, 90), (55, 130, 17)),
    ("d128_g2_nocache", 4, 2, 128, 2, 1, 1, 0, 16, (300, 77), (0, 0)),
]


@pytest.mark.parametrize("idx", range(len(RESPLIT)), ids=[c[0] for c in RESPLIT])
def test_resplit_share_full_parity(cc, idx):
    name, hq, hkv, d, p, r, dd, rd, bs, new, ctx = RESPLIT[idx]
    w = Workload(name=name, seed=3000 + idx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 pcp_size=p, pcp_rank=r, dcp_size=dd, dcp_rank=rd, block_size=bs,
                 new_lens=new, ctx_lens=ctx)
    inp = generate(w)
    cache = resplit_cache(inp)
    share = _make_share(cc, inp, cache)
    share.out.fill_(float("nan"))
    share.step()
    torch.cuda.synchronize()
    ref = _resplit_oracle(inp, share)
    assert_close(share.out, share.lse, ref["merged"][0], ref["merged"][1], name)


def test_resplit_equals_standard_path_without_dcp(cc):
    """With one DCP rank both paths attend over the same keys: the re-split
    result matches the three-call path's within the tolerance."""
    w = Workload(name="eq", seed=3100, num_q_heads=8, num_kv_heads=2, head_dim=128, pcp_size=2,
                 pcp_rank=1, dcp_size=1, dcp_rank=0, block_size=16, new_lens=(900, 1, 257),
                 ctx_lens=(130, 40, 0))
    inp = generate(w)
    from context_causal_gqa_amd.share import RankShare

    std = RankShare(inp)
    std.step()
    rs = _make_share(cc, inp, resplit_cache(inp))
    rs.step()
    torch.cuda.synchronize()
    assert np.array_equal(std.qidx, rs.qidx)
    ref = _resplit_oracle(inp, rs)
    assert_close(rs.out, rs.lse, ref["merged"][0], ref["merged"][1], "resplit")
    assert_close(std.out, std.lse, ref["merged"][0], ref["merged"][1], "standard")


def test_resplit_reassembly_all_ranks_and_shards(cc):
    """Every PCP rank: each DCP rank writes its blocks into one shared pool;
    the fused launch of shard 0 (own tokens + shard 0's context) merged with
    the other shards' context passes equals unsplit causal attention."""
    p, dd = 2, 2
    w = Workload(name="rsr", seed=3200, num_q_heads=8, num_kv_heads=2, head_dim=128, pcp_size=p,
                 pcp_rank=0, dcp_size=dd, dcp_rank=0, block_size=16, new_lens=(437, 1, 200),
                 ctx_lens=(150, 300, 0))
    inp = generate(w)
    cache = resplit_cache(inp)
    kp, vp = cache.k_pool.cuda(), cache.v_pool.cuda()
    tot = int(inp.cu_seqlens_new[-1])
    full_o = np.full((tot, 8, 128), np.nan)
    full_l = np.full((8, tot), np.nan)
    for r in range(p):
        shares = [_make_share(cc, inp, cache, pcp_rank=r, dcp_rank=x, k_pool=kp, v_pool=vp)
                  for x in range(dd)]
        for sh in shares:
            sh.cache_write()
        shares[0].attend()
        outs, lses = [shares[0].out], [shares[0].lse]
        for sh in shares[1:]:
            o = torch.empty_like(sh.out)
            l = torch.empty_like(sh.lse)
            cc.pcp_attn_context_paged(sh.q, sh.k_cache, sh.v_cache, sh.block_tables, sh.rows, o,
                                      l, sh.scale, sh.max_q_len, rows_host=sh.rows_host)
            outs.append(o)
            lses.append(l)
        mo = torch.empty_like(shares[0].out)
        ml = torch.empty_like(shares[0].lse)
        cc.lse_merge(outs, lses, mo, ml)
        torch.cuda.synchronize()
        full_o[shares[0].qidx] = _np(mo)
        full_l[:, shares[0].qidx] = _np(ml)
    assert not np.isnan(full_o).any()
    ref_o, ref_l = oracle.full_causal_attention(inp.q, inp.k_new, inp.v_new, inp.k_cached,
                                                inp.v_cached, inp.cu_seqlens_new, inp.ctx_lens,
                                                inp.cu_cache, 8, 2, w.softmax_scale)
    assert_close(full_o, full_l, ref_o, ref_l, "re-split reassembled")
