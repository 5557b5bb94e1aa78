"""The entry points under HIP graph capture.

The calls enqueue kernels only (no allocation, no memset, no host read-back),
so a caller can capture a step into a graph and replay it. Each test
captures calls into NaN-filled buffers, then replays the graph several times
with eager work between the replays (buffers refilled with NaN, other calls
of the library on other buffers, synchronisations), and checks every replay
bit-identical to the eager result, which itself matches the oracle.
"""

import numpy as np
import pytest
import torch

from pcp_workloads import Workload, generate

from test_gpu_parity import cc, check_share, run_share  # noqa: F401 (cc is a fixture)

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _workload(d):
    if d == 128:
        return Workload(name="graph_d128", seed=9100, num_q_heads=16, num_kv_heads=8,
                        head_dim=128, pcp_size=2, pcp_rank=1, dcp_size=2, dcp_rank=0,
                        block_size=16, new_lens=(700, 1, 333, 1), ctx_lens=(41, 2600, 0, 900))
    return Workload(name="graph_d256", seed=9200, num_q_heads=8, num_kv_heads=1, head_dim=256,
                    pcp_size=4, pcp_rank=3, dcp_size=4, dcp_rank=3, block_size=16,
                    new_lens=(1200, 1), ctx_lens=(333, 5000))


def _nan_like(t):
    return torch.full_like(t, float("nan"))


def _replay_and_check(g, outs, refs, disturb, what):
    for rep in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), "%s: replay %d differs from the eager call" % (what, rep)


@pytest.mark.parametrize("d", [128, 256])
def test_fused_call_replays_from_a_graph(cc, d):
    """pcp_attn_rank_share with split decode rows (the caller's workspace)."""
    inp = generate(_workload(d))
    share = run_share(cc, inp, decode_splits=3)
    check_share(inp, share, what="graph eager d%d" % d)
    ref_o, ref_l = share.out_fused.clone(), share.lse_fused.clone()
    out, lse = _nan_like(share.out), _nan_like(share.lse)
    share.step_fused(out=out, lse=lse)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        share.step_fused(out=out, lse=lse)
    _replay_and_check(g, (out, lse), (ref_o, ref_l), lambda: share.step(),
                      "fused d%d" % d)


def test_noalloc_call_replays_from_a_graph(cc):
    """pcp_attn_rank_share_noalloc: its split partials live in the library's
    fixed scratch array, whose address is looked up on the first call."""
    inp = generate(_workload(128))
    share = run_share(cc, inp, decode_splits=3)
    ref_o, ref_l = share.out_fused.clone(), share.lse_fused.clone()
    out, lse = _nan_like(share.out), _nan_like(share.lse)

    def call():
        cc.pcp_attn_rank_share_noalloc(
            share.q, share.k, share.v, share.k_cache, share.v_cache, share.block_tables,
            share.rows, out, lse, share.scale, share.max_q_len, rows_host=share.rows_host,
            decode_splits=share.decode_splits_fused, unit_order=share.order_fused)

    call()  # first call on the device: the scratch address lookup, outside the capture
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replay_and_check(g, (out, lse), (ref_o, ref_l), lambda: share.step_fused(),
                      "noalloc")


def test_three_calls_replay_from_a_graph(cc):
    """The context pass, the new-token pass and lse_merge captured together."""
    inp = generate(_workload(256))
    share = run_share(cc, inp, decode_splits=4)
    refs = [t.clone() for t in (share.out_new, share.lse_new, share.out_ctx, share.lse_ctx,
                                share.out, share.lse)]
    share.step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        share.step()
    outs = (share.out_new, share.lse_new, share.out_ctx, share.lse_ctx, share.out, share.lse)
    tmp_o, tmp_l = _nan_like(share.out), _nan_like(share.lse)
    _replay_and_check(g, outs, refs, lambda: share.step_fused(out=tmp_o, lse=tmp_l),
                      "three calls")
    assert np.isfinite(share.lse.cpu().numpy()).any()
