"""GPU test of pcp_attn_rank_share_noalloc: the fused rank share with its
split-decode partials in the library's fixed per-device scratch array, for
callers that cannot allocate. Through the C ABI it must give exactly what
pcp_attn_rank_share gives with a caller workspace (same kernels, same
arithmetic: bit-identical), and match the oracle within the parity
tolerances (out max 2e-2, mean 2e-3, LSE 1e-3), on two calls in a row, the
second with a smaller input, the array keeping whatever the first call left.
A call whose partials exceed the array is refused before anything runs.
"""

import numpy as np
import pytest
import torch

from pcp_workloads import Workload, generate

from test_gpu_parity import assert_close, assert_written, oracle_share, visible_counts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_causal_gqa_amd as m

    return m


CALLS = [
    # name, hq, hkv, d, new_lens, ctx_lens, decode_splits (larger call first)
    ("d256_6dec", 8, 1, 256, (1, 1, 1, 700, 1, 1, 1), (9000, 4000, 33, 250, 6100, 0, 2200), 64),
    ("d128_2dec", 8, 2, 128, (1, 300, 1), (3000, 100, 700), 16),
]


def _run(cc, share, noalloc, splits):
    out = torch.full_like(share.out, float("nan"))
    lse = torch.full_like(share.lse, float("nan"))
    args = (share.q, share.k, share.v, share.k_cache, share.v_cache, share.block_tables,
            share.rows, out, lse, share.scale, share.max_q_len)
    if noalloc:
        cc.pcp_attn_rank_share_noalloc(*args, rows_host=share.rows_host, decode_splits=splits,
                                       unit_order=share.order_fused)
    else:
        cc.pcp_attn_rank_share(*args, rows_host=share.rows_host, workspace=share.workspace,
                               decode_splits=splits, unit_order=share.order_fused)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_matches_the_workspace_entry_point(cc):
    from context_causal_gqa_amd.share import RankShare

    for i, (name, hq, hkv, d, new, ctx, splits) in enumerate(CALLS):
        print("noalloc call %d: %s, %d splits" % (i, name, splits), flush=True)
        w = Workload(name=name, seed=6100 + i, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                     pcp_size=2, pcp_rank=1, dcp_size=2, dcp_rank=1, block_size=16,
                     new_lens=new, ctx_lens=ctx)
        inp = generate(w)
        share = RankShare(inp, decode_splits=splits)
        need = cc.pcp_context_workspace_bytes(share.num_rows, hq, d, splits)
        assert 0 < need <= cc.NOALLOC_SCRATCH_BYTES
        share.workspace.fill_(float("nan"))
        o_ws, l_ws = _run(cc, share, False, splits)
        o_na, l_na = _run(cc, share, True, splits)
        new_c, ctx_c = visible_counts(share.rows_host)
        assert_written(o_na, l_na, new_c + ctx_c, name + " noalloc")
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), name
        assert torch.equal(l_na, l_ws), name
        ref = oracle_share(inp, share)["merged"]
        assert_close(o_na, l_na, ref[0], ref[1], name + " noalloc")


def test_noalloc_refuses_partials_beyond_its_scratch(cc):
    """More partials than the array holds: PCP_ESCRATCH, nothing launched
    (the outputs keep their NaN fill)."""
    from context_causal_gqa_amd.share import RankShare

    w = Workload(name="big", seed=6200, num_q_heads=16, num_kv_heads=1, head_dim=256,
                 pcp_size=2, pcp_rank=0, dcp_size=1, dcp_rank=0, block_size=16,
                 new_lens=(1,) * 8, ctx_lens=(500,) * 8)
    share = RankShare(generate(w), decode_splits=1)
    splits = 256  # 8 rows x 16 heads x 256 x 257 x 4 bytes = 33.7 MB > 16 MiB
    assert cc.pcp_context_workspace_bytes(share.num_rows, 16, 256, splits) > \
        cc.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(share.out, float("nan"))
    lse = torch.full_like(share.lse, float("nan"))
    with pytest.raises(cc.PcpError) as e:
        cc.pcp_attn_rank_share_noalloc(share.q, share.k, share.v, share.k_cache, share.v_cache,
                                       share.block_tables, share.rows, out, lse, share.scale,
                                       share.max_q_len, decode_splits=splits)
    assert e.value.code == cc.PCP_ESCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()
    np.testing.assert_equal(share.num_rows, 8)
