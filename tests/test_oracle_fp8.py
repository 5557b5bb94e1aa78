"""Pins of the FP8 oracle (oracle/fp8.py) against what the format definition
and the mathematics fix: the E4M3 decode against the OCP definition's worked
values and torch's own float8_e4m3fn cast on all 256 codes; the (request, KV
head) descale indexing against brute force on tiny inputs; and the scaling
laws of the descales (closed forms)."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from pcp_workloads import Workload, generate, quantize_fp8


def test_e4m3_worked_values():
    """Values fixed by the E4M3 ("fn") definition: bias 7, 3 mantissa bits,
    subnormals below 2^-6, S.1111.111 NaN, largest finite 448."""
    cases = {
        0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
        0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0xC0: -2.0, 0x7E: 448.0, 0xFE: -448.0,
        0x77: 240.0, 0x30: 0.5, 0x0F: 1.875 * 2.0 ** -6,
    }
    got = ofp8.e4m3_to_float(np.array(list(cases)))
    assert np.array_equal(got, np.array(list(cases.values())))
    assert np.signbit(ofp8.e4m3_to_float(0x80))
    assert np.isnan(ofp8.e4m3_to_float(np.array([0x7F, 0xFF]))).all()


def test_e4m3_all_codes_match_torch():
    """Every code against torch's independent float8_e4m3fn widening."""
    mine = ofp8.e4m3_to_float(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_e4m3_monotone_and_exact_integers():
    """Positive codes 0x00..0x7E are strictly increasing; every integer up to
    16 is exactly representable (4 significant bits)."""
    v = ofp8.e4m3_to_float(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)
    assert set(range(17)) <= set(v.tolist())


def _tiny(seed, hq=4, hkv=2, d=8, pcp=2, rank=1, dcp=2, drank=0, bs=4,
          new=(9, 1, 6), ctx=(5, 7, 0)):
    w = Workload(name="fp8tiny", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 pcp_size=pcp, pcp_rank=rank, dcp_size=dcp, dcp_rank=drank, block_size=bs,
                 new_lens=new, ctx_lens=ctx)
    inp = generate(w)
    f = quantize_fp8(inp)
    # distinct descales per (request, kv head), so a wrong index shows
    rng = np.random.default_rng(seed)
    for t in (f.q_descale, f.k_descale, f.v_descale):
        t *= rng.uniform(0.5, 2.0, size=t.shape).astype(np.float32)
    return w, inp, f


def _brute_force(w, inp, f, plan):
    """Per local query and head, loop over the request's visible keys: the
    cached ones this DCP rank owns (block j on rank j mod D) and the new ones
    up to the end-aligned causal bound; decode with torch's cast; scale each
    value by the descale of its own (request, KV head)."""
    dec = lambda x: x.view(torch.float8_e4m3fn).double().numpy()
    g = w.num_q_heads // w.num_kv_heads
    cu, cuc = inp.cu_seqlens_new, inp.cu_cache
    q_full = dec(f.q8)
    kn, vn, kc, vc = dec(f.k8_new), dec(f.v8_new), dec(f.k8_cached), dec(f.v8_cached)
    total_q = int(plan[:, 3].sum())
    out = np.zeros((total_q, w.num_q_heads, w.head_dim))
    lse = np.full((w.num_q_heads, total_q), -np.inf)
    for row in plan:
        b, qs, ql, kl = int(row[0]), int(row[2]), int(row[3]), int(row[6])
        off = int(cu[b]) + oracle.row_new_token_offset(row, inp.ctx_lens)
        ctx_len = int(row[7])
        for t in range(ql):
            for h in range(w.num_q_heads):
                kvh = h // g
                qv = q_full[off + t, h] * float(f.q_descale[b, kvh])
                keys = []
                for p in range(ctx_len):
                    if (p // w.block_size) % w.dcp_size == w.dcp_rank:
                        keys.append((kc[int(cuc[b]) + p, kvh], vc[int(cuc[b]) + p, kvh]))
                if int(row[1]) != oracle.KIND_DECODE:
                    for j in range(kl - ql + t + 1):
                        keys.append((kn[int(cu[b]) + j, kvh], vn[int(cu[b]) + j, kvh]))
                if not keys:
                    continue
                s = [w.softmax_scale * float(np.dot(qv, kk * float(f.k_descale[b, kvh])))
                     for kk, _ in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = sum(e)
                o = sum(ei * vv * float(f.v_descale[b, kvh]) for ei, (_, vv) in zip(e, keys))
                out[qs + t, h] = o / tot
                lse[h, qs + t] = m + math.log(tot)
    return out, lse


def _oracle_fp8(w, inp, f, plan, **kw):
    ql = oracle.gather_local_queries(f.q8.numpy(), inp.cu_seqlens_new, inp.ctx_lens, plan)
    return ofp8.rank_share_fp8(ql, f.k8_new, f.v8_new, f.k8_cached, f.v8_cached,
                               inp.cu_seqlens_new, inp.cu_cache, plan,
                               kw.get("q_ds", f.q_descale), kw.get("k_ds", f.k_descale),
                               kw.get("v_ds", f.v_descale), w.dcp_size, w.dcp_rank,
                               w.block_size, w.num_q_heads, w.num_kv_heads,
                               kw.get("scale", w.softmax_scale))


@pytest.mark.parametrize("seed,hq,hkv,rank,drank", [(1, 4, 2, 1, 0), (2, 6, 3, 0, 1), (3, 4, 1, 1, 1)])
def test_rank_share_fp8_brute_force(seed, hq, hkv, rank, drank):
    w, inp, f = _tiny(seed, hq=hq, hkv=hkv, rank=rank, drank=drank)
    plan = oracle.plan_rows(inp.cu_seqlens_new, inp.ctx_lens, w.pcp_size, rank, w.dcp_size,
                            drank, w.block_size)
    ref_o, ref_l = _brute_force(w, inp, f, plan)
    got_o, got_l = _oracle_fp8(w, inp, f, plan)["merged"]
    np.testing.assert_allclose(got_o, ref_o, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(got_l))
    np.testing.assert_allclose(got_l[fin], ref_l[fin], rtol=1e-12, atol=1e-12)


def test_descale_scaling_laws():
    """v_descale * c scales out by c and leaves LSE alone; q_descale * c with
    k_descale / c changes nothing; q_descale * c equals softmax_scale * c
    (descales widened to float64 first, so the products are the exact ones)."""
    w, inp, f = _tiny(7)
    plan = oracle.plan_rows(inp.cu_seqlens_new, inp.ctx_lens, w.pcp_size, w.pcp_rank,
                            w.dcp_size, w.dcp_rank, w.block_size)
    o0, l0 = _oracle_fp8(w, inp, f, plan)["merged"]
    q64, k64, v64 = (x.astype(np.float64) for x in (f.q_descale, f.k_descale, f.v_descale))
    o1, l1 = _oracle_fp8(w, inp, f, plan, v_ds=v64 * 3.0)["merged"]
    np.testing.assert_allclose(o1, 3.0 * o0, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(l1, l0)
    o2, l2 = _oracle_fp8(w, inp, f, plan, q_ds=q64 * 3.0, k_ds=k64 / 3.0)["merged"]
    np.testing.assert_allclose(o2, o0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l0, rtol=1e-12, atol=1e-12)
    o3, l3 = _oracle_fp8(w, inp, f, plan, q_ds=q64 * 1.5)["merged"]
    o4, l4 = _oracle_fp8(w, inp, f, plan, scale=w.softmax_scale * 1.5)["merged"]
    np.testing.assert_allclose(o3, o4, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l3, l4, rtol=1e-12, atol=1e-12)


def test_fp8_quantisation_round_trip():
    """The generator's codes decode (times their descale) to within E4M3's
    half-step of the bf16 values: relative 2^-4 in the normal range, absolute
    2^-10 * descale below it; descale * 448 is each group's amax."""
    w, inp, _ = _tiny(11, d=16)
    f = quantize_fp8(inp)
    req = ofp8.token_requests(inp.cu_seqlens_new)
    kd = ofp8.dequantize(f.k8_new, f.k_descale, req, 1)
    x = inp.k_new.double().numpy()
    ds = f.k_descale[req][:, :, None].astype(np.float64)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * ds) * (1 + 1e-6)
    assert np.all(np.abs(kd - x) <= bound)
    g = w.num_q_heads // w.num_kv_heads
    qd = ofp8.dequantize(f.q8, f.q_descale, req, g)
    assert np.all(np.abs(qd) <= 448.0 * f.q_descale[req][:, np.arange(w.num_q_heads) // g][..., None] * (1 + 1e-6))


def test_resplit_fp8_takes_each_tokens_own_request_descales():
    """The re-split FP8 share equals the bf16 re-split definition on values
    decoded with torch's cast and scaled token by token, in explicit loops,
    by the descale of the token's own request and KV head (the rows' own
    tokens by their query's request)."""
    w, inp, f = _tiny(21, hq=4, hkv=2, new=(9, 1, 7), ctx=(5, 6, 3))
    plan = oracle.plan_rows_resplit(inp.cu_seqlens_new, inp.ctx_lens, w.pcp_size, w.pcp_rank,
                                    w.dcp_size, w.dcp_rank, w.block_size)
    cu, cuc = inp.cu_seqlens_new, inp.cu_cache
    dec = lambda x: x.view(torch.float8_e4m3fn).double().numpy()
    g = w.num_q_heads // w.num_kv_heads

    def scaled(codes, ds, req_of, group):
        x = dec(codes).copy()
        for t in range(x.shape[0]):
            for h in range(x.shape[1]):
                x[t, h] *= float(ds[req_of(t), h // group])
        return x

    def req_in(cu_arr):
        return lambda t: int(np.searchsorted(np.asarray(cu_arr), t, side="right") - 1)

    q8 = oracle.gather_local_queries(f.q8.numpy(), cu, inp.ctx_lens, plan)
    k8l = oracle.gather_local_queries(f.k8_new.numpy(), cu, inp.ctx_lens, plan)
    v8l = oracle.gather_local_queries(f.v8_new.numpy(), cu, inp.ctx_lens, plan)
    qs = plan[:, oracle.F["q_start"]]
    req_local = lambda t: int(plan[np.searchsorted(qs, t, side="right") - 1, oracle.F["req"]])
    t8 = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    ref = oracle.rank_share_resplit(
        scaled(t8(q8), f.q_descale, req_local, g), scaled(t8(k8l), f.k_descale, req_local, 1),
        scaled(t8(v8l), f.v_descale, req_local, 1), scaled(f.k8_new, f.k_descale, req_in(cu), 1),
        scaled(f.v8_new, f.v_descale, req_in(cu), 1), cu,
        scaled(f.k8_cached, f.k_descale, req_in(cuc), 1),
        scaled(f.v8_cached, f.v_descale, req_in(cuc), 1), cuc, inp.ctx_lens, plan, w.dcp_size,
        w.dcp_rank, w.block_size, w.num_q_heads, w.num_kv_heads, w.softmax_scale)["merged"]
    got = ofp8.rank_share_resplit_fp8(q8, k8l, v8l, f.k8_new, f.v8_new, cu, f.k8_cached,
                                      f.v8_cached, cuc, inp.ctx_lens, plan, f.q_descale,
                                      f.k_descale, f.v_descale, w.dcp_size, w.dcp_rank,
                                      w.block_size, w.num_q_heads, w.num_kv_heads,
                                      w.softmax_scale)["merged"]
    np.testing.assert_allclose(got[0], ref[0], rtol=1e-12, atol=1e-12)
    fin = np.isfinite(ref[1])
    assert np.array_equal(fin, np.isfinite(got[1]))
    np.testing.assert_allclose(got[1][fin], ref[1][fin], rtol=1e-12, atol=1e-12)
