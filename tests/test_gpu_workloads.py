"""GPU parity of the five named workloads at full size, in the launch
configuration bench.py times (host-made unit order, decode splits chosen by
the library), through the C ABI, against the fp64 oracle.

Every path runs on every workload:
  bf16     the three calls (context pass, new-token pass, lse_merge) and the
           fused launch (pcp_attn_rank_share);
  fp8      the same with E4M3 Q/K/V (the _fp8 entry points) against the
           oracle on the dequantized values;
  resplit  the cache write, then the fused launch over re-split rows
           ([0, row_start) from this DCP rank's cache + own tokens).

Every output buffer is NaN-filled before the calls. Afterwards, over all of
it: every output value is finite and the LSE is -inf exactly where the
definition gives a query no visible key (the counts follow from the plan:
query t of a row with q_len m and k_len n sees max(0, min(n, n - m + t + 1))
new keys and ctx_len_local context keys). A unit that was never run leaves
NaN behind and fails here, whatever the oracle comparison samples.

Oracle comparison (out max |err| <= 2e-2, mean <= 2e-3, LSE <= 1e-3):
  - the tiny, Qwen-shaped and mixed workloads: every output, every buffer;
  - the 128k and 256k shares: whole 32-query tiles x all heads (one tile
    is one work unit's queries at d = 256 with eight heads per KV head):
    each row's first, middle and last tile, then seeded random tiles until
    at least 1024 queries are checked. The end-aligned mask puts the causal
    diagonal inside every tile, so each checked tile includes its masked
    key tile.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import F
from pcp_workloads import WORKLOADS, generate, quantize_fp8, resplit_cache

from test_gpu_parity import _np, assert_close, assert_written, run_share, share_buffers, visible_counts

pytestmark = pytest.mark.gpu

FULL = ("tiny_t512_pcp2_r0", "qwen3_0p6b_8x4096_pcp2_r1", "mixed_pcp2_dcp2_8prefill_4decode")
TILED = ("hybrid_fullattn_128k_pcp4_r1", "hybrid_fullattn_256k_ctx64k_pcp4_dcp4_r3")
TILE, MIN_TILED_QUERIES = 32, 1024

CASES = [(n, p) for n in FULL + TILED for p in ("bf16", "fp8", "resplit")]


@pytest.fixture(scope="module")
def cc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_causal_gqa_amd as m

    return m


_INPUTS = {}


def workload_inputs(name):
    """Generated inputs of one workload; only the latest one is kept (the
    256k share's host tensors take several GB)."""
    if name not in _INPUTS:
        _INPUTS.clear()
        print("generating", name, flush=True)
        _INPUTS[name] = generate(WORKLOADS[name])
    return _INPUTS[name]


def tile_sample(rows, seed, tile=TILE, min_queries=MIN_TILED_QUERIES):
    """Rank-local query ids of whole ``tile``-query tiles: each row's first,
    middle and last tile, then seeded random tiles up to ``min_queries``."""
    rng = np.random.default_rng(seed)
    tiles = []  # (row, tile index)
    for i, r in enumerate(rows):
        nt = -(-int(r[F["q_len"]]) // tile)
        tiles += [(i, j) for j in sorted({0, nt // 2, nt - 1})]
    chosen = set(tiles)

    def size(t):
        r = rows[t[0]]
        return min(tile, int(r[F["q_len"]]) - t[1] * tile)

    n = sum(size(t) for t in chosen)
    ntiles = [-(-int(r[F["q_len"]]) // tile) for r in rows]
    while n < min_queries and len(chosen) < sum(ntiles):
        i = int(rng.integers(len(rows)))
        t = (i, int(rng.integers(ntiles[i])))
        if t not in chosen:
            chosen.add(t)
            n += size(t)
    ids = [np.arange(int(rows[i, F["q_start"]]) + j * tile,
                     int(rows[i, F["q_start"]]) + j * tile + size((i, j))) for i, j in sorted(chosen)]
    return np.concatenate(ids).astype(np.int64)


def _gather_bits(x, cu, ctx, plan):
    """Rank-local rows of a [T, H, d] tensor gathered on its raw bits (bf16 as
    int16, E4M3 as uint8) by the oracle's own gather."""
    if x.dtype == torch.bfloat16:
        bits = oracle.gather_local_queries(x.view(torch.int16).numpy(), cu, ctx, plan)
        return torch.from_numpy(bits).view(torch.bfloat16).double().numpy()
    return oracle.gather_local_queries(x.numpy(), cu, ctx, plan)


def _sel(ids):
    return slice(None) if ids is None else torch.from_numpy(ids).cuda()


def _check_parts(bufs, ref, ids, what):
    for key, (o, l) in bufs:
        rk = "merged" if key in ("fused", "merged") else key
        sel = _sel(ids)
        assert_close(o[sel], l[:, sel], ref[rk][0], ref[rk][1], "%s %s" % (what, key))


def check_standard(cc, name, inp, path):
    w = inp.workload
    f8 = quantize_fp8(inp) if path == "fp8" else None
    print("running", name, path, flush=True)
    share = run_share(cc, inp, fp8=f8)
    bufs = tuple((key, ol) for key, ol, _ in share_buffers(share))
    for key, (o, l), count in share_buffers(share):
        assert_written(o, l, count, "%s %s %s" % (name, path, key))
    ids = None if name in FULL else tile_sample(share.rows_host, seed=w.seed)
    plan = oracle.plan_rows(inp.cu_seqlens_new, inp.ctx_lens, w.pcp_size, share.pcp_rank,
                            w.dcp_size, share.dcp_rank, w.block_size)
    assert np.array_equal(plan, share.rows_host.astype(np.int64))  # plans bit-exact
    cu, cx = inp.cu_seqlens_new, inp.ctx_lens
    n = share.total_q if ids is None else len(ids)
    print("oracle on %d of %d queries" % (n, share.total_q), flush=True)
    if f8 is None:
        ql = _gather_bits(inp.q, cu, cx, plan)
        assert np.array_equal(_np(share.q[_sel(ids)]), ql if ids is None else ql[ids])
        ref = oracle.rank_share(ql, inp.k_new, inp.v_new, inp.k_cached, inp.v_cached,
                                inp.cu_cache, plan, w.dcp_size, share.dcp_rank, w.block_size,
                                w.num_q_heads, w.num_kv_heads, w.softmax_scale, query_ids=ids)
    else:
        q8 = _gather_bits(f8.q8, cu, cx, plan)
        assert np.array_equal(share.q[_sel(ids)].cpu().numpy(), q8 if ids is None else q8[ids])
        ref = oracle.fp8.rank_share_fp8(q8, f8.k8_new, f8.v8_new, f8.k8_cached, f8.v8_cached,
                                        cu, inp.cu_cache, plan, f8.q_descale, f8.k_descale,
                                        f8.v_descale, w.dcp_size, share.dcp_rank, w.block_size,
                                        w.num_q_heads, w.num_kv_heads, w.softmax_scale,
                                        query_ids=ids)
    _check_parts(bufs, ref, ids, "%s %s" % (name, path))


def check_resplit(name, inp):
    from context_causal_gqa_amd.share import ResplitShare

    w = inp.workload
    cache = resplit_cache(inp)
    share = ResplitShare(inp, cache)
    share.out.fill_(float("nan"))
    share.lse.fill_(float("nan"))
    print("running", name, "resplit", flush=True)
    share.step()
    torch.cuda.synchronize()
    new_c, ctx_c = visible_counts(share.rows_host)
    assert_written(share.out, share.lse, new_c + ctx_c, name + " resplit")
    cu, cx = inp.cu_seqlens_new, inp.ctx_lens
    plan = oracle.plan_rows_resplit(cu, cx, w.pcp_size, share.pcp_rank, w.dcp_size,
                                    share.dcp_rank, w.block_size)
    assert np.array_equal(plan, share.rows_host.astype(np.int64))
    slots = oracle.slot_mapping(cu, cx, cache.block_table, w.dcp_size, share.dcp_rank,
                                w.block_size)
    assert np.array_equal(slots, share.slots_host)
    ids = None if name in FULL else tile_sample(share.rows_host, seed=w.seed + 100)
    ql = _gather_bits(inp.q, cu, cx, plan)
    kl = _gather_bits(inp.k_new, cu, cx, plan)
    vl = _gather_bits(inp.v_new, cu, cx, plan)
    assert np.array_equal(_np(share.q[_sel(ids)]), ql if ids is None else ql[ids])
    n = share.total_q if ids is None else len(ids)
    print("oracle on %d of %d queries" % (n, share.total_q), flush=True)
    ref = oracle.rank_share_resplit(ql, kl, vl, inp.k_new, inp.v_new, cu, inp.k_cached,
                                    inp.v_cached, inp.cu_cache, cx, plan, w.dcp_size,
                                    share.dcp_rank, w.block_size, w.num_q_heads,
                                    w.num_kv_heads, w.softmax_scale, query_ids=ids)
    _check_parts((("merged", (share.out, share.lse)),), ref, ids, name + " resplit")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,path", CASES, ids=["%s-%s" % c for c in CASES])
def test_named_workload_parity(cc, name, path):
    inp = workload_inputs(name)
    if path == "resplit":
        check_resplit(name, inp)
    else:
        check_standard(cc, name, inp, path)


def test_tile_sample_covers_rows():
    """The tiled sample holds whole tiles, each row's first, middle and last,
    and at least the requested number of queries."""
    rows = np.zeros((2, 9), dtype=np.int64)
    rows[0, F["q_start"]], rows[0, F["q_len"]] = 0, 100
    rows[1, F["q_start"]], rows[1, F["q_len"]] = 100, 1000
    ids = tile_sample(rows, seed=1, tile=32, min_queries=300)
    assert len(ids) >= 300 and len(np.unique(ids)) == len(ids)
    for q in (0, 31, 32, 63, 96, 99, 100, 131, 100 + 16 * 32, 1099):
        assert q in ids
