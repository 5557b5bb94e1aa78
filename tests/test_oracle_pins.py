"""Pins of the fp64 oracle against things other than itself.

* Plan: hand-derived fixtures (tests/golden/plans.json, each cited), partition
  invariants over random batches, the zigzag balance closed form.
* Attention: brute-force pure-Python loops on tiny inputs, torch's
  scaled_dot_product_attention (a different library routine) on the unsplit
  square causal problem, torch.logsumexp for LSE, Q = 0 closed forms
  (mean of visible V, exp(LSE) = visible count).
* Merge: attention over a union of key sets equals the merge of the parts;
  empty parts are the identity.

A plausible slip in the oracle (a dropped scale, an off-by-one in the causal
bound, h % Hkv instead of h // g, log2 instead of ln, a wrong merge weight)
fails at least one of these.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import F
from pcp_workloads import Workload, generate, random_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plans.json")


# ---------------------------------------------------------------- plan pins


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_plan_matches_golden(case):
    a = case["args"]
    plan = oracle.plan_rows(a["cu_seqlens_new"], a["ctx_lens"], a["pcp_size"], a["pcp_rank"],
                            a["dcp_size"], a["dcp_rank"], a["block_size"])
    assert plan.tolist() == case["rows"]


def _cu(new):
    cu = np.zeros(len(new) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(new)
    return cu


def test_plan_partitions_new_tokens_over_ranks():
    rng = np.random.default_rng(11)
    for _ in range(300):
        new, ctx = random_batch(rng)
        cu = _cu(new)
        p = int(rng.integers(1, 6))
        cover = [np.zeros(int(n), dtype=np.int64) for n in new]
        for r in range(p):
            plan = oracle.plan_rows(cu, ctx, p, r, 1, 0, 16)
            n_pre = int(np.sum(new >= 2))
            n_dec = int(np.sum(new == 1))
            assert len(plan) <= 2 * n_pre + n_dec
            # q_start is the running sum of q_len
            if len(plan):
                assert plan[0, F["q_start"]] == 0
                assert np.all(plan[1:, F["q_start"]] == np.cumsum(plan[:-1, F["q_len"]]))
            for row in plan:
                b = row[F["req"]]
                off = oracle.row_new_token_offset(row, ctx)
                ql = row[F["q_len"]]
                assert ql >= 1
                if row[F["kind"]] == oracle.KIND_DECODE:
                    assert new[b] == 1 and row[F["k_len"]] == 0
                    assert row[F["ctx_len"]] == ctx[b] + 1
                else:
                    # k_len is the end of the chunk: the row's last query sees k_len new keys
                    assert row[F["k_len"]] == off + ql
                    assert row[F["pos_start"]] == ctx[b] + off
                    assert row[F["ctx_len"]] == ctx[b]
                assert row[F["k_start"]] == cu[b]
                cover[b][off:off + ql] += 1
        for b, n in enumerate(new):
            if n == 1:
                assert cover[b].tolist() == [p]  # decode rows live on every rank
            else:
                assert np.all(cover[b] == 1)  # prefill tokens exactly once


def test_dcp_shards_partition_cached_prefix():
    rng = np.random.default_rng(12)
    for _ in range(200):
        c = int(rng.integers(0, 500))
        bs = int(rng.choice([1, 3, 16, 64]))
        dd = int(rng.integers(1, 6))
        parts = [oracle.owned_cached_positions(c, dd, r, bs) for r in range(dd)]
        allp = np.sort(np.concatenate(parts))
        assert allp.tolist() == list(range(c))
        # each rank holds whole blocks, except possibly the global last one
        for r, pos in enumerate(parts):
            assert np.all((pos // bs) % dd == r)


@pytest.mark.parametrize("n,p", [(512, 2), (4096, 2), (131072, 4), (262144, 4), (96, 3)])
def test_zigzag_balance_closed_form(n, p):
    """With 2P | N every rank sees N^2/(2P) + N/(2P) causal pairs."""
    expect = n * n // (2 * p) + n // (2 * p)
    for r in range(p):
        plan = oracle.plan_rows([0, n], [0], p, r, 1, 0, 16)
        new_pairs, ctx_pairs = oracle.visible_pairs(plan)
        assert new_pairs == expect and ctx_pairs == 0
    if (n, p) == (131072, 4):
        assert expect == 2_147_500_032


# ---------------------------------------------------------- attention pins


def _brute_attention(qv, keys, vals, scale):
    """Pure-Python softmax attention of one query over a list of keys."""
    if not keys:
        return [0.0] * len(vals[0] if vals else qv), -math.inf
    scores = [scale * sum(a * b for a, b in zip(qv, k)) for k in keys]
    mx = max(scores)
    ws = [math.exp(s - mx) for s in scores]
    tot = sum(ws)
    out = [sum(w * v[i] for w, v in zip(ws, vals)) / tot for i in range(len(vals[0]))]
    return out, mx + math.log(tot)


def _tiny_inputs(seed, new_lens, ctx_lens, hq, hkv, d, dcp, bs=4):
    w = Workload(name="t", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 pcp_size=2, pcp_rank=0, dcp_size=dcp, dcp_rank=0, block_size=bs,
                 new_lens=tuple(new_lens), ctx_lens=tuple(ctx_lens))
    return w, generate(w)


def test_brute_force_rank_share_tiny():
    """Every output of one rank share, recomputed query by query in plain Python
    straight from the pages' definitions."""
    hq, hkv, d, p, dcp, bs = 4, 2, 8, 2, 2, 4
    w, inp = _tiny_inputs(21, [9, 1, 13], [6, 10, 0], hq, hkv, d, dcp, bs)
    cu = inp.cu_seqlens_new
    for r in range(p):
        for rd in range(dcp):
            plan = oracle.plan_rows(cu, inp.ctx_lens, p, r, dcp, rd, bs)
            q_local = oracle.gather_local_queries(inp.q.double().numpy(), cu, inp.ctx_lens, plan)
            res = oracle.rank_share(q_local, inp.k_new, inp.v_new, inp.k_cached, inp.v_cached,
                                    inp.cu_cache, plan, dcp, rd, bs, hq, hkv, w.softmax_scale)
            kn = inp.k_new.double().tolist()
            vn = inp.v_new.double().tolist()
            kc = inp.k_cached.double().tolist()
            vc = inp.v_cached.double().tolist()
            for row in plan:
                b = row[F["req"]]
                off = oracle.row_new_token_offset(row, inp.ctx_lens)
                for t in range(row[F["q_len"]]):
                    qi = row[F["q_start"]] + t
                    i_new = off + t  # index of this query among request b's new tokens
                    for h in range(hq):
                        kvh = h * hkv // hq
                        qv = q_local[qi, h].tolist()
                        # new-token keys: a decode row takes none; a prefill
                        # query at new index i sees new keys 0..i
                        if row[F["kind"]] == oracle.KIND_DECODE:
                            nk = []
                        else:
                            nk = list(range(int(cu[b]), int(cu[b]) + i_new + 1))
                        o_new, l_new = _brute_attention(qv, [kn[j][kvh] for j in nk],
                                                        [vn[j][kvh] for j in nk] or [[0.0] * d],
                                                        w.softmax_scale)
                        # cached keys held by this DCP rank: block j on rank j mod D
                        nvis = int(inp.ctx_lens[b]) + (1 if row[F["kind"]] == 2 else 0)
                        ck = [int(inp.cu_cache[b]) + x for x in range(nvis) if (x // bs) % dcp == rd]
                        o_ctx, l_ctx = _brute_attention(qv, [kc[j][kvh] for j in ck],
                                                        [vc[j][kvh] for j in ck] or [[0.0] * d],
                                                        w.softmax_scale)
                        # merged over both key sets directly
                        o_all, l_all = _brute_attention(
                            qv, [kn[j][kvh] for j in nk] + [kc[j][kvh] for j in ck],
                            ([vn[j][kvh] for j in nk] + [vc[j][kvh] for j in ck]) or [[0.0] * d],
                            w.softmax_scale)
                        for key, (o_ref, l_ref) in (("new", (o_new, l_new)), ("ctx", (o_ctx, l_ctx)),
                                                    ("merged", (o_all, l_all))):
                            o, l = res[key]
                            assert np.allclose(o[qi, h], o_ref, atol=1e-12, rtol=0)
                            if l_ref == -math.inf:
                                assert l[h, qi] == -np.inf
                            else:
                                assert abs(l[h, qi] - l_ref) < 1e-12


def _sdpa_full(inp, hq, hkv, scale):
    """Unsplit causal attention of every new token with torch's SDPA: the
    square problem over [cached prefix + new tokens], queries of cached
    positions are dummies, K/V heads repeated for GQA."""
    g = hq // hkv
    outs = []
    lses = []
    cu = inp.cu_seqlens_new
    for b in range(len(cu) - 1):
        c = int(inp.ctx_lens[b])
        n = int(cu[b + 1] - cu[b])
        if n == 0:
            continue
        cb = int(inp.cu_cache[b])
        k = torch.cat([inp.k_cached[cb:cb + c], inp.k_new[cu[b]:cu[b + 1]]]).double()
        v = torch.cat([inp.v_cached[cb:cb + c], inp.v_new[cu[b]:cu[b + 1]]]).double()
        q = torch.cat([torch.zeros(c, hq, k.shape[-1], dtype=torch.float64),
                       inp.q[cu[b]:cu[b + 1]].double()])
        kk = k.repeat_interleave(g, dim=1).transpose(0, 1).contiguous()  # [Hq, L, d]
        vv = v.repeat_interleave(g, dim=1).transpose(0, 1).contiguous()
        qq = q.transpose(0, 1).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True,
                                                             scale=scale)
        s = (qq @ kk.transpose(1, 2)) * scale
        L = s.shape[-1]
        mask = torch.ones(L, L, dtype=torch.bool).tril()
        lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
        outs.append(o.transpose(0, 1)[c:].numpy())
        lses.append(lse[:, c:].numpy())
    return np.concatenate(outs), np.concatenate(lses, axis=1)


@pytest.mark.parametrize("seed,hq,hkv,d,p,dcp,new,ctx", [
    (31, 4, 2, 16, 2, 1, [40, 23], [0, 0]),
    (32, 8, 2, 8, 3, 2, [37, 1, 50, 1], [10, 25, 0, 7]),
    (33, 6, 6, 8, 2, 3, [64, 5], [33, 17]),
    (34, 8, 1, 32, 4, 4, [96], [40]),
])
def test_reassembly_equals_sdpa(seed, hq, hkv, d, p, dcp, new, ctx):
    """All PCP ranks' rows, each merged over its new-token pass and every DCP
    shard's context pass, reassembled in natural order, equal unsplit causal
    attention computed by torch."""
    w, inp = _tiny_inputs(seed, new, ctx, hq, hkv, d, dcp, bs=4)
    out, lse, seen = oracle.reassemble_all_ranks(
        inp.q, inp.k_new, inp.v_new, inp.k_cached, inp.v_cached, inp.cu_seqlens_new,
        inp.ctx_lens, inp.cu_cache, p, dcp, 4, hq, hkv, w.softmax_scale)
    ref_o, ref_l = _sdpa_full(inp, hq, hkv, w.softmax_scale)
    assert np.all(seen[inp.new_lens[np.repeat(np.arange(len(new)), new)] >= 2] == 1)
    assert np.abs(out - ref_o).max() < 1e-12
    assert np.abs(lse - ref_l).max() < 1e-12
    # the oracle's own unsplit reference agrees too
    fo, fl = oracle.full_causal_attention(
        inp.q, inp.k_new, inp.v_new, inp.k_cached, inp.v_cached, inp.cu_seqlens_new,
        inp.ctx_lens, inp.cu_cache, hq, hkv, w.softmax_scale)
    assert np.abs(fo - ref_o).max() < 1e-12
    assert np.abs(fl - ref_l).max() < 1e-12


def test_zero_queries_give_mean_of_visible_v_and_counts():
    """With Q = 0 every score is 0: out is the mean of the visible V rows and
    exp(LSE) is exactly the number of visible keys."""
    hq, hkv, d, p, dcp, bs = 4, 2, 8, 2, 2, 4
    w, inp = _tiny_inputs(41, [29, 1, 16], [13, 22, 0], hq, hkv, d, dcp, bs)
    cu = inp.cu_seqlens_new
    for r in range(p):
        plan = oracle.plan_rows(cu, inp.ctx_lens, p, r, dcp, 1, bs)
        total_q = int(plan[:, F["q_len"]].sum())
        q0 = np.zeros((total_q, hq, d))
        res = oracle.rank_share(q0, inp.k_new, inp.v_new, inp.k_cached, inp.v_cached,
                                inp.cu_cache, plan, dcp, 1, bs, hq, hkv, w.softmax_scale)
        vn = inp.v_new.double().numpy()
        vc = inp.v_cached.double().numpy()
        for row in plan:
            b = row[F["req"]]
            m, n = row[F["q_len"]], row[F["k_len"]]
            pos = [x for x in range(row[F["ctx_len"]]) if (x // bs) % dcp == 1]
            assert len(pos) == row[F["ctx_len_local"]]
            for t in range(m):
                qi = row[F["q_start"]] + t
                cnt_new = n - m + t + 1 if row[F["kind"]] != 2 else 0
                for h in range(hq):
                    kvh = h // (hq // hkv)
                    o, l = res["new"]
                    if cnt_new:
                        assert round(math.exp(l[h, qi])) == cnt_new
                        ref = vn[cu[b]:cu[b] + cnt_new, kvh].mean(axis=0)
                        assert np.allclose(o[qi, h], ref, atol=1e-13)
                    else:
                        assert l[h, qi] == -np.inf and not o[qi, h].any()
                    o, l = res["ctx"]
                    if pos:
                        assert round(math.exp(l[h, qi])) == len(pos)
                        ref = vc[int(inp.cu_cache[b]) + np.asarray(pos), kvh].mean(axis=0)
                        assert np.allclose(o[qi, h], ref, atol=1e-13)
                    else:
                        assert l[h, qi] == -np.inf
                    o, l = res["merged"]
                    assert round(math.exp(l[h, qi])) == cnt_new + len(pos)


def test_boundary_one_hot_v():
    """V one-hot at the last visible key contributes exactly 1/count; at the
    first hidden key it contributes nothing (end-aligned mask)."""
    m, n, d = 5, 12, 4
    q = np.zeros((m, 1, d))
    plan = np.array([[0, 0, 0, m, 0, 0, n, 0, 0]])
    for t in range(m):
        for key, expect in ((n - m + t, 1.0 / (n - m + t + 1)), (n - m + t + 1, 0.0)):
            if key >= n:
                continue
            k = np.zeros((n, 1, d))
            v = np.zeros((n, 1, d))
            v[key, 0, 0] = 1.0
            o, _ = oracle.new_token_pass(q, k, v, plan, 1, 1, 0.5)
            assert abs(o[t, 0, 0] - expect) < 1e-15


def test_gqa_mapping_against_repeated_heads():
    """GQA with Hkv < Hq equals MHA over K/V heads repeated g times
    (query head h reads KV head h // g)."""
    rng = np.random.default_rng(51)
    hq, hkv, d = 6, 2, 8
    m = n = 20
    q = rng.standard_normal((m, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    plan = np.array([[0, 0, 0, m, 0, 0, n, 0, 0]])
    o1, l1 = oracle.new_token_pass(q, k, v, plan, hq, hkv, 0.3)
    g = hq // hkv
    o2, l2 = oracle.new_token_pass(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), plan,
                                   hq, hq, 0.3)
    assert np.abs(o1 - o2).max() == 0 and np.abs(l1 - l2).max() == 0
    # and a head-interleaved mapping would differ
    o3, _ = oracle.new_token_pass(q, np.tile(k, (1, g, 1)), np.tile(v, (1, g, 1)), plan, hq, hq, 0.3)
    assert np.abs(o1 - o3).max() > 1e-3


def test_lse_matches_torch_logsumexp():
    rng = np.random.default_rng(61)
    m, n, d = 7, 19, 16
    q = rng.standard_normal((m, 2, d))
    k = rng.standard_normal((n, 1, d))
    v = rng.standard_normal((n, 1, d))
    plan = np.array([[0, 0, 0, m, 0, 0, n, 0, 0]])
    scale = 1 / 4
    _, lse = oracle.new_token_pass(q, k, v, plan, 2, 1, scale)
    for h in range(2):
        s = torch.from_numpy(q[:, h] @ k[:, 0].T * scale)
        mask = torch.arange(n)[None, :] <= (n - m + torch.arange(m))[:, None]
        ref = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1).numpy()
        assert np.abs(lse[h] - ref).max() < 1e-13


# ---------------------------------------------------------------- merge pins


def test_merge_of_disjoint_key_sets_equals_union():
    rng = np.random.default_rng(71)
    m, d = 6, 8
    q = rng.standard_normal((m, 1, d))
    k = rng.standard_normal((30, 1, d))
    v = rng.standard_normal((30, 1, d))
    full = np.array([[0, 0, 0, m, 0, 0, 30, 0, 0]])
    # causal over 30 keys == merge(causal rows over keys [0,30) split as prefix/suffix):
    # prefix keys [0, 11) are all visible (they precede every query's bound)
    o_all, l_all = oracle.softmax_attention(q[:, 0], k[:, 0], v[:, 0],
                                            np.ones((m, 30), dtype=bool), 0.4)
    parts = []
    for lo, hi in ((0, 11), (11, 12), (12, 30)):
        o, l = oracle.softmax_attention(q[:, 0], k[lo:hi, 0], v[lo:hi, 0],
                                        np.ones((m, hi - lo), dtype=bool), 0.4)
        parts.append((o[:, None], l[None]))
    o_m, l_m = oracle.lse_merge(parts)
    assert np.abs(o_m[:, 0] - o_all).max() < 1e-13
    assert np.abs(l_m[0] - l_all).max() < 1e-13
    # order does not matter; merging in two steps is the same (associativity)
    o_r, l_r = oracle.lse_merge(parts[::-1])
    assert np.abs(o_r - o_m).max() < 1e-13
    o12, l12 = oracle.lse_merge(parts[:2])
    o_s, l_s = oracle.lse_merge([(o12, l12), parts[2]])
    assert np.abs(o_s - o_m).max() < 1e-13 and np.abs(l_s - l_m).max() < 1e-13
    del full


def test_merge_with_empty_parts():
    rng = np.random.default_rng(72)
    o = rng.standard_normal((5, 3, 4))
    l = rng.standard_normal((3, 5))
    empty = (np.zeros_like(o), np.full_like(l, -np.inf))
    o_m, l_m = oracle.lse_merge([empty, (o, l), empty])
    assert np.abs(o_m - o).max() < 1e-15 and np.abs(l_m - l).max() < 1e-15
    o_e, l_e = oracle.lse_merge([empty, empty])
    assert not o_e.any() and np.all(np.isneginf(l_e))
    # ln a (+) ln b = ln(a + b)
    a = (np.zeros((1, 1, 4)), np.log(np.full((1, 1), 3.0)))
    b = (np.zeros((1, 1, 4)), np.log(np.full((1, 1), 5.0)))
    _, l_ab = oracle.lse_merge([a, b])
    assert abs(l_ab[0, 0] - math.log(8.0)) < 1e-15


def test_decode_row_sees_its_own_cached_token():
    """A decode row (one new token) attends to C + 1 cached tokens, itself included."""
    w, inp = _tiny_inputs(81, [1], [9], 2, 1, 8, 1, bs=4)
    plan = oracle.plan_rows(inp.cu_seqlens_new, inp.ctx_lens, 2, 1, 1, 0, 4)
    assert plan.tolist() == [[0, 2, 0, 1, 9, 0, 0, 10, 10]]
    q = np.zeros((1, 2, 8))
    res = oracle.rank_share(q, inp.k_new, inp.v_new, inp.k_cached, inp.v_cached, inp.cu_cache,
                            plan, 1, 0, 4, 2, 1, w.softmax_scale)
    assert round(math.exp(res["merged"][1][0, 0])) == 10
    assert np.isneginf(res["new"][1]).all()


# ------------------------------------------------------------ re-split path


@pytest.mark.parametrize("seed,hq,hkv,d,p,dcp,new,ctx", [
    (41, 4, 2, 16, 2, 1, [40, 23], [0, 0]),
    (42, 8, 2, 8, 3, 2, [37, 1, 50, 1], [10, 25, 0, 7]),
    (43, 6, 6, 8, 2, 3, [64, 5], [33, 17]),
    (44, 8, 1, 32, 4, 4, [96, 1], [40, 9]),
])
def test_resplit_reassembly_equals_sdpa(seed, hq, hkv, d, p, dcp, new, ctx):
    """Re-split path ([0, row_start) from the cache shards + own tokens square
    causal) over all PCP ranks and DCP shards equals unsplit causal attention
    computed by torch."""
    w, inp = _tiny_inputs(seed, new, ctx, hq, hkv, d, dcp, bs=4)
    out, lse, seen = oracle.reassemble_resplit(
        inp.q, inp.k_new, inp.v_new, inp.k_cached, inp.v_cached, inp.cu_seqlens_new,
        inp.ctx_lens, inp.cu_cache, p, dcp, 4, hq, hkv, w.softmax_scale)
    ref_o, ref_l = _sdpa_full(inp, hq, hkv, w.softmax_scale)
    assert (seen >= 1).all()
    assert np.abs(out - ref_o).max() < 1e-12
    assert np.abs(lse - ref_l).max() < 1e-12


def _random_plan_args(seed):
    rng = np.random.default_rng(seed)
    new, ctx = random_batch(rng)
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int64)
    p = int(rng.integers(1, 5))
    d = int(rng.integers(1, 5))
    return cu, np.asarray(ctx), p, int(rng.integers(0, p)), d, int(rng.integers(0, d)), \
        int(rng.choice([1, 4, 16]))


def test_resplit_plan_relations():
    """Same rows as the standard plan; own tokens as keys; context [0, pos_start)
    whose DCP shares add up; decode rows keep their context."""
    for seed in range(40):
        cu, ctx, p, r, d, rd, bs = _random_plan_args(900 + seed)
        std = oracle.plan_rows(cu, ctx, p, r, d, rd, bs)
        rs = oracle.plan_rows_resplit(cu, ctx, p, r, d, rd, bs)
        same = [F[k] for k in ("req", "kind", "q_start", "q_len", "pos_start")]
        assert np.array_equal(std[:, same], rs[:, same])
        assert np.array_equal(rs[:, F["k_start"]], rs[:, F["q_start"]])
        dec = rs[:, F["kind"]] == oracle.KIND_DECODE
        assert np.array_equal(rs[~dec, F["k_len"]], rs[~dec, F["q_len"]])
        assert np.array_equal(rs[~dec, F["ctx_len"]], rs[~dec, F["pos_start"]])
        assert np.array_equal(rs[dec][:, 6:], std[dec][:, 6:])
        shares = sum(oracle.plan_rows_resplit(cu, ctx, p, r, d, x, bs)[:, F["ctx_len_local"]]
                     for x in range(d))
        assert np.array_equal(shares, rs[:, F["ctx_len"]])


def test_resplit_visible_pairs_equal_standard_over_all_shards():
    """Both paths attend over the same (query, key) pairs once every DCP shard
    is counted: the re-split path only moves earlier new tokens into context."""
    for seed in range(30):
        cu, ctx, p, r, d, rd, bs = _random_plan_args(950 + seed)
        tot_std = tot_rs = 0
        for x in range(d):
            n_s, c_s = oracle.visible_pairs(oracle.plan_rows(cu, ctx, p, r, d, x, bs))
            n_r, c_r = oracle.visible_pairs(oracle.plan_rows_resplit(cu, ctx, p, r, d, x, bs))
            tot_std += c_s + (n_s if x == 0 else 0)
            tot_rs += c_r + (n_r if x == 0 else 0)
        assert tot_std == tot_rs


def test_slot_mapping_golden():
    g = json.load(open(os.path.join(os.path.dirname(GOLDEN), "slot_mapping.json")))
    for case in g["cases"]:
        bt = np.asarray(case["block_table"], dtype=np.int64)
        for rank, want in case["slots"].items():
            got = oracle.slot_mapping(case["cu_seqlens_new"], case["ctx_lens"], bt,
                                      case["dcp_size"], int(rank), case["block_size"])
            assert got.tolist() == want


def test_slot_mapping_partitions_tokens_and_cache_write_fills_the_cache():
    """Over all DCP ranks every new token is written exactly once, at its own
    position of its own block; writing every rank's tokens into pools holding
    the prefix reproduces the natural-order cache content."""
    rng = np.random.default_rng(77)
    for trial in range(20):
        b = int(rng.integers(1, 5))
        new = rng.integers(1, 40, size=b)
        ctx = rng.integers(0, 30, size=b)
        cu = np.concatenate([[0], np.cumsum(new)])
        bs = int(rng.choice([1, 3, 4, 16]))
        dcp = int(rng.integers(1, 4))
        nblk = (ctx + new + bs - 1) // bs
        perm = rng.permutation(int(nblk.sum()) + 3)
        bt = np.full((b, int(nblk.max())), -1, dtype=np.int64)
        k = 0
        for i in range(b):
            bt[i, :nblk[i]] = perm[k:k + nblk[i]]
            k += nblk[i]
        writers = np.zeros(int(cu[-1]), dtype=np.int64)
        hkv, d = 2, 3
        k_new = rng.normal(size=(int(cu[-1]), hkv, d))
        pool = np.full((len(perm), bs, hkv, d), np.nan)
        for rd in range(dcp):
            s = oracle.slot_mapping(cu, ctx, bt, dcp, rd, bs)
            writers += s >= 0
            for i in range(b):
                for t in range(new[i]):
                    sl = s[cu[i] + t]
                    if sl >= 0:
                        pos = ctx[i] + t
                        assert (pos // bs) % dcp == rd
                        assert sl == bt[i, pos // bs] * bs + pos % bs
            pool, _ = oracle.kv_cache_write(k_new, k_new, s, pool, pool)
        assert (writers == 1).all()
        for i in range(b):
            for t in range(new[i]):
                pos = ctx[i] + t
                assert np.array_equal(pool[bt[i, pos // bs], pos % bs], k_new[cu[i] + t])
        # nothing else was written
        assert np.isnan(pool).sum() == pool.size - int(cu[-1]) * hkv * d
