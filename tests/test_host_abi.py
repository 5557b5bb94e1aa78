"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
and its host-only logic (the row plan, argument validation) is right.

The C++ row plan is compared bit-exactly with the oracle's plan, which is an
independent implementation (tests/test_oracle_pins.py pins the oracle).
No kernel is launched here.
"""

import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle
from pcp_workloads import random_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pcp_attn.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "plans.json")

cc = pytest.importorskip("context_causal_gqa_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cc.LIB_PATH):
        import context_causal_gqa_amd.build as b

        b.build()
    return cc.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined", "if"})


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(
        ["pcp_strerror", "pcp_plan_rows", "pcp_plan_rows_resplit", "pcp_slot_mapping",
         "pcp_kv_cache_write", "pcp_kv_cache_write_fp8", "pcp_attn_prefill",
         "pcp_attn_context_paged",
         "pcp_attn_rank_share", "pcp_attn_prefill_fp8", "pcp_attn_context_paged_fp8",
         "pcp_attn_rank_share_fp8", "pcp_context_workspace_bytes", "pcp_choose_decode_splits",
         "pcp_attn_schedule", "lse_merge", "pcp_attn_rank_share_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_strerror(lib):
    for code, text in ((0, "ok"), (-1, "invalid argument"), (-2, "unsupported configuration"),
                       (-3, "HIP runtime error"), (-4, "size does not fit 32-bit plan fields"),
                       (-5, "call needs more scratch than the library's fixed scratch array")):
        assert cc.strerror(code) == text


def test_row_struct_matches_plan_columns():
    # pcp_row_t is nine int32 fields in ROW_FIELDS order (also the oracle's column order)
    text = open(HEADER).read()
    body = re.search(r"typedef struct pcp_row \{(.*?)\} pcp_row_t;", text, re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert tuple(fields) == cc.ROW_FIELDS == oracle.ROW_FIELDS


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_cpp_plan_matches_golden(lib, case):
    a = case["args"]
    rows = cc.pcp_plan_rows(a["cu_seqlens_new"], a["ctx_lens"], a["pcp_size"], a["pcp_rank"],
                            a["dcp_size"], a["dcp_rank"], a["block_size"])
    assert rows.tolist() == case["rows"]


def test_cpp_plan_bit_exact_vs_oracle_random(lib):
    rng = np.random.default_rng(101)
    for it in range(3000):
        new, ctx = random_batch(rng, max_requests=10, max_new=200, max_ctx=300)
        cu = np.zeros(len(new) + 1, dtype=np.int64)
        cu[1:] = np.cumsum(new)
        cu += int(rng.integers(0, 3)) * (it % 2)  # a nonzero first offset is allowed
        p = int(rng.integers(1, 9))
        r = int(rng.integers(0, p))
        dd = int(rng.integers(1, 9))
        rd = int(rng.integers(0, dd))
        bs = int(rng.choice([1, 2, 7, 16, 32, 128]))
        got = cc.pcp_plan_rows(cu, ctx, p, r, dd, rd, bs)
        want = oracle.plan_rows(cu, ctx, p, r, dd, rd, bs)
        assert got.shape == want.shape
        assert np.array_equal(got.astype(np.int64), want), (new, ctx, p, r, dd, rd, bs)
        got = cc.pcp_plan_rows_resplit(cu, ctx, p, r, dd, rd, bs)
        want = oracle.plan_rows_resplit(cu, ctx, p, r, dd, rd, bs)
        assert np.array_equal(got.astype(np.int64), want), ("resplit", new, ctx, p, r, dd, rd)


def test_cpp_slot_mapping_golden_and_bit_exact_vs_oracle(lib):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "slot_mapping.json")))
    for case in g["cases"]:
        for rank, want in case["slots"].items():
            got = cc.pcp_slot_mapping(case["cu_seqlens_new"], case["ctx_lens"],
                                      np.asarray(case["block_table"]), case["dcp_size"],
                                      int(rank), case["block_size"])
            assert got.tolist() == want
    rng = np.random.default_rng(202)
    for it in range(500):
        new, ctx = random_batch(rng, max_requests=8, max_new=150, max_ctx=200)
        cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int64)
        bs = int(rng.choice([1, 3, 16, 64]))
        dd = int(rng.integers(1, 5))
        nblk = [(c + n + bs - 1) // bs for c, n in zip(ctx, new)]
        mb = max(nblk) + int(rng.integers(0, 3))
        bt = rng.integers(0, 10000, size=(len(new), mb)).astype(np.int64)
        for rd in range(dd):
            got = cc.pcp_slot_mapping(cu, ctx, bt, dd, rd, bs)
            want = oracle.slot_mapping(cu, ctx, bt, dd, rd, bs)
            assert np.array_equal(got, want), (it, rd)


def test_slot_mapping_rejects_a_short_table(lib):
    # 40 tokens at positions 0..39 need blocks 0..2 of size 16; the table has 2
    with pytest.raises(cc.PcpError):
        cc.pcp_slot_mapping([0, 40], [0], np.array([[3, 4]]), 1, 0, 16)
    # with 2 DCP ranks, rank 1 owns only block 1, which the table has
    assert cc.pcp_slot_mapping([0, 40], [0], np.array([[3, 4]]), 2, 1, 16).tolist() == \
        [-1] * 16 + list(range(64, 80)) + [-1] * 8
    with pytest.raises(cc.PcpError):
        cc.pcp_slot_mapping([0, 40], [0], np.array([[3, -1, 5]]), 1, 0, 16)  # a hole


def test_plan_capacity_contract(lib):
    """The plan never writes past the caller's capacity and reports the size
    it needs, so a caller can size its buffer (the 8-vs-14 rows crash on
    'Carry the row plan in attention metadata', fork PR #2)."""
    cu = np.array([0, 8, 9, 17, 25, 26, 34, 42, 50], dtype=np.int32)
    ctx = np.array([0, 40, 0, 5, 33, 0, 0, 0], dtype=np.int32)
    L = cc.lib()
    for cap in (0, 1, 8, 13, 14, 20):
        buf = np.full((cap + 4, 9), -7, dtype=np.int32)
        n = L.pcp_plan_rows(8, cu.ctypes.data, ctx.ctypes.data, 2, 0, 2, 0, 16,
                            buf.ctypes.data if cap else None, cap)
        assert n == 14
        assert np.all(buf[min(cap, 14):] == -7)  # nothing written past capacity
        if cap:
            want = oracle.plan_rows(cu, ctx, 2, 0, 2, 0, 16)
            assert np.array_equal(buf[:min(cap, 14)], want[:min(cap, 14)])


@pytest.mark.parametrize("args", [
    dict(pcp_size=0, pcp_rank=0), dict(pcp_size=2, pcp_rank=2), dict(pcp_size=2, pcp_rank=-1),
    dict(dcp_size=0), dict(dcp_size=2, dcp_rank=2), dict(block_size=0),
])
def test_plan_rejects_bad_ranks(lib, args):
    a = dict(pcp_size=2, pcp_rank=0, dcp_size=1, dcp_rank=0, block_size=16)
    a.update(args)
    cu = np.array([0, 10], dtype=np.int32)
    ctx = np.array([0], dtype=np.int32)
    buf = np.zeros((4, 9), dtype=np.int32)
    rc = cc.lib().pcp_plan_rows(1, cu.ctypes.data, ctx.ctypes.data, a["pcp_size"], a["pcp_rank"],
                                a["dcp_size"], a["dcp_rank"], a["block_size"], buf.ctypes.data, 4)
    assert rc == cc.PCP_EINVAL


def test_plan_rejects_bad_lengths(lib):
    L = cc.lib()
    buf = np.zeros((4, 9), dtype=np.int32)
    for cu, ctx in (([0, 10, 5], [0, 0]), ([0, 10], [-1]), ([-2, 10], [0])):
        cu = np.array(cu, dtype=np.int32)
        ctx = np.array(ctx, dtype=np.int32)
        assert L.pcp_plan_rows(len(ctx), cu.ctypes.data, ctx.ctypes.data, 2, 0, 1, 0, 16,
                               buf.ctypes.data, 4) == cc.PCP_EINVAL
    assert L.pcp_plan_rows(-1, None, None, 1, 0, 1, 0, 16, None, 0) == cc.PCP_EINVAL
    assert L.pcp_plan_rows(0, None, None, 1, 0, 1, 0, 16, None, 0) == 0
    # offsets that do not fit the int32 fields
    cu = np.array([0, 2_000_000_000], dtype=np.int32)
    ctx = np.array([1_000_000_000], dtype=np.int32)
    assert L.pcp_plan_rows(1, cu.ctypes.data, ctx.ctypes.data, 1, 0, 1, 0, 16,
                           buf.ctypes.data, 4) == cc.PCP_EOVERFLOW


def test_device_calls_validate_before_launch(lib):
    """Argument errors are reported on the host before anything is enqueued
    (these calls never reach the GPU)."""
    L = cc.lib()
    dummy = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # unsupported head_dim
    assert L.pcp_attn_prefill(dummy, dummy, dummy, dummy, 1, 8, 8, 8, 4, 2, 96, 0.1, dummy,
                              dummy, None, 0, None) == cc.PCP_EUNSUPPORTED
    # Hq not a multiple of Hkv
    assert L.pcp_attn_prefill(dummy, dummy, dummy, dummy, 1, 8, 8, 8, 6, 4, 64, 0.1, dummy,
                              dummy, None, 0, None) == cc.PCP_EINVAL
    # negative sizes, bad scale, null pointers
    assert L.pcp_attn_prefill(dummy, dummy, dummy, dummy, -1, 8, 8, 8, 4, 2, 64, 0.1, dummy,
                              dummy, None, 0, None) == cc.PCP_EINVAL
    assert L.pcp_attn_prefill(dummy, dummy, dummy, dummy, 1, 8, 8, 8, 4, 2, 64, 0.0, dummy,
                              dummy, None, 0, None) == cc.PCP_EINVAL
    assert L.pcp_attn_prefill(None, dummy, dummy, dummy, 1, 8, 8, 8, 4, 2, 64, 0.1, dummy,
                              dummy, None, 0, None) == cc.PCP_EINVAL
    # an order with a negative length
    assert L.pcp_attn_prefill(dummy, dummy, dummy, dummy, 1, 8, 8, 8, 4, 2, 64, 0.1, dummy,
                              dummy, dummy, -1, None) == cc.PCP_EINVAL
    # empty work is a valid no-op
    assert L.pcp_attn_prefill(None, None, None, None, 0, 0, 0, 0, 4, 2, 64, 0.1, None, None,
                              None, 0, None) == 0
    # context pass: block_size, missing cache pointers with blocks, bad dims
    assert L.pcp_attn_context_paged(dummy, dummy, dummy, 4, 0, dummy, 1, 1, dummy, 1, 8, 8, 4, 2,
                                    64, 0.1, dummy, dummy, None, 1, None, 0, None) == cc.PCP_EINVAL
    assert L.pcp_attn_context_paged(dummy, None, dummy, 4, 16, dummy, 1, 1, dummy, 1, 8, 8, 4, 2,
                                    64, 0.1, dummy, dummy, None, 1, None, 0, None) == cc.PCP_EINVAL
    assert L.pcp_attn_context_paged(dummy, dummy, dummy, 4, 16, dummy, 1, 1, dummy, 1, 8, 8, 4, 2,
                                    32, 0.1, dummy, dummy, None, 1, None, 0, None) == cc.PCP_EUNSUPPORTED
    # decode splits: at least one, a workspace when more than one, 16-byte aligned, <= 256
    ctx_args = (dummy, dummy, dummy, 4, 16, dummy, 1, 1, dummy, 1, 8, 8, 4, 2, 64, 0.1, dummy,
                dummy)
    assert L.pcp_attn_context_paged(*ctx_args, None, 0, None, 0, None) == cc.PCP_EINVAL
    assert L.pcp_attn_context_paged(*ctx_args, None, 4, None, 0, None) == cc.PCP_EINVAL
    assert L.pcp_attn_context_paged(*ctx_args, ctypes.c_void_p(0x1004), 4, None, 0,
                                    None) == cc.PCP_EINVAL
    assert L.pcp_attn_context_paged(*ctx_args, dummy, 257, None, 0, None) == cc.PCP_EUNSUPPORTED
    assert L.pcp_attn_context_paged(*ctx_args, None, 1, dummy, -1, None) == cc.PCP_EINVAL
    # fused call: the union of both calls' checks
    fused = (dummy, dummy, dummy, 8, dummy, dummy, 4, 16, dummy, 1, 1, dummy, 1, 8, 8, 4, 2)
    assert L.pcp_attn_rank_share(*fused, 96, 0.1, dummy, dummy, None, 1, None, 0,
                                 None) == cc.PCP_EUNSUPPORTED
    assert L.pcp_attn_rank_share(dummy, dummy, dummy, 8, dummy, dummy, 4, 0, dummy, 1, 1, dummy,
                                 1, 8, 8, 4, 2, 64, 0.1, dummy, dummy, None, 1, None, 0,
                                 None) == cc.PCP_EINVAL  # block_size 0
    assert L.pcp_attn_rank_share(dummy, None, dummy, 8, dummy, dummy, 4, 16, dummy, 1, 1, dummy,
                                 1, 8, 8, 4, 2, 64, 0.1, dummy, dummy, None, 1, None, 0,
                                 None) == cc.PCP_EINVAL  # new-token keys without k
    assert L.pcp_attn_rank_share(*fused, 64, 0.1, dummy, dummy, None, 2, None, 0,
                                 None) == cc.PCP_EINVAL  # splits without a workspace
    assert L.pcp_attn_rank_share(*fused, 64, 0.1, dummy, dummy, dummy, 300, None, 0,
                                 None) == cc.PCP_EUNSUPPORTED
    assert L.pcp_attn_rank_share(None, None, None, 0, None, None, 0, 16, None, 0, 0, None, 0, 0,
                                 0, 4, 2, 64, 0.1, None, None, None, 1, None, 0, None) == 0
    # cache write: nothing to do, bad head_dim, null or misaligned pointers
    assert L.pcp_kv_cache_write(None, None, None, 0, 1, 128, None, None, 4, 16, None) == 0
    assert L.pcp_kv_cache_write(dummy, dummy, dummy, 4, 1, 96, dummy, dummy, 4, 16,
                                None) == cc.PCP_EUNSUPPORTED
    assert L.pcp_kv_cache_write(dummy, None, dummy, 4, 1, 128, dummy, dummy, 4, 16,
                                None) == cc.PCP_EINVAL
    assert L.pcp_kv_cache_write(ctypes.c_void_p(0x1008), dummy, dummy, 4, 1, 128, dummy, dummy,
                                4, 16, None) == cc.PCP_EINVAL
    assert L.pcp_kv_cache_write(dummy, dummy, dummy, 4, 1, 128, dummy, dummy, 4, 0,
                                None) == cc.PCP_EINVAL
    # 16-byte chunks must fit 32-bit indices with one grid stride to spare:
    # 2^32 - 2^24 chunks at most (2048 chunks per token at 64 KV heads, d = 256)
    limit = (1 << 32) - 1 - (1 << 24)
    assert L.pcp_kv_cache_write(dummy, dummy, dummy, limit // 2048 + 1, 64, 256, dummy, dummy, 4,
                                16, None) == cc.PCP_EUNSUPPORTED
    # merge: too many partials, bad dims, null arrays
    arr = (ctypes.c_void_p * 17)(*([0x1000] * 17))
    assert L.lse_merge(17, arr, arr, 8, 4, 64, dummy, dummy, None) == cc.PCP_EUNSUPPORTED
    assert L.lse_merge(0, arr, arr, 8, 4, 64, dummy, dummy, None) == cc.PCP_EINVAL
    assert L.lse_merge(2, arr, arr, 8, 4, 48, dummy, dummy, None) == cc.PCP_EUNSUPPORTED
    assert L.lse_merge(2, None, arr, 8, 4, 64, dummy, dummy, None) == cc.PCP_EINVAL
    nulls = (ctypes.c_void_p * 2)(0x1000, 0)
    assert L.lse_merge(2, nulls, arr, 8, 4, 64, dummy, dummy, None) == cc.PCP_EINVAL


def test_fp8_calls_validate_before_launch(lib):
    """The FP8 entry points: the bf16 calls' checks, plus descale tables that
    must be given and 4-byte aligned, 16-byte aligned codes and at least one
    request (no kernel is launched)."""
    L = cc.lib()
    d = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1008)  # 8- but not 16-byte aligned
    # prefill: (q, k, v, rows, num_rows, total_q, total_k, max_q_len, num_reqs, hq, hkv, d,
    #           scale, q_ds, k_ds, v_ds, out, lse, order, num_units, stream)
    base = [d, d, d, d, 1, 8, 8, 8, 1, 4, 2, 64, 0.1, d, d, d, d, d, None, 0, None]

    def pre(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.pcp_attn_prefill_fp8(*a)

    assert pre(a11=96) == cc.PCP_EUNSUPPORTED
    assert pre(a9=6, a10=4) == cc.PCP_EINVAL
    assert pre(a13=None) == cc.PCP_EINVAL  # no q descale
    assert pre(a15=None) == cc.PCP_EINVAL  # no v descale
    assert pre(a14=ctypes.c_void_p(0x1002)) == cc.PCP_EINVAL  # misaligned descale
    assert pre(a0=odd) == cc.PCP_EINVAL  # misaligned codes
    assert pre(a2=odd) == cc.PCP_EINVAL
    assert pre(a8=0) == cc.PCP_EINVAL  # rows but no request
    assert pre(a4=0) == 0  # nothing to do
    # context pass and fused call: descales and alignment on top of the bf16 checks
    ctx = [d, d, d, 4, 16, d, 1, 1, d, 1, 8, 8, 4, 2, 64, 0.1, d, d, d, d, d, None, 1, None, 0,
           None]
    assert L.pcp_attn_context_paged_fp8(*ctx[:16], None, *ctx[17:]) == cc.PCP_EINVAL
    assert L.pcp_attn_context_paged_fp8(odd, *ctx[1:]) == cc.PCP_EINVAL
    assert L.pcp_attn_context_paged_fp8(*ctx[:1], odd, *ctx[2:]) == cc.PCP_EINVAL
    assert L.pcp_attn_context_paged_fp8(*ctx[:4], 0, *ctx[5:]) == cc.PCP_EINVAL  # block_size 0
    assert L.pcp_attn_context_paged_fp8(*ctx[:21], None, 2, *ctx[23:]) == cc.PCP_EINVAL
    fused = [d, d, d, 8, d, d, 4, 16, d, 1, 1, d, 1, 8, 8, 4, 2, 64, 0.1, d, d, d, d, d, None, 1,
             None, 0, None]
    assert L.pcp_attn_rank_share_fp8(*fused[:17], 32, *fused[18:]) == cc.PCP_EUNSUPPORTED
    assert L.pcp_attn_rank_share_fp8(*fused[:20], None, *fused[21:]) == cc.PCP_EINVAL
    assert L.pcp_attn_rank_share_fp8(*fused[:4], odd, *fused[5:]) == cc.PCP_EINVAL
    assert L.pcp_attn_rank_share_fp8(*fused[:9], 0, *fused[10:]) == cc.PCP_EINVAL  # no request
    assert L.pcp_attn_rank_share_fp8(*fused[:12], 0, *fused[13:]) == 0  # no rows
    # FP8 cache write: the bf16 write's checks, at one byte per value
    assert L.pcp_kv_cache_write_fp8(None, None, None, 0, 1, 128, None, None, 4, 16, None) == 0
    assert L.pcp_kv_cache_write_fp8(d, d, d, 4, 1, 96, d, d, 4, 16, None) == cc.PCP_EUNSUPPORTED
    assert L.pcp_kv_cache_write_fp8(d, None, d, 4, 1, 64, d, d, 4, 16, None) == cc.PCP_EINVAL
    assert L.pcp_kv_cache_write_fp8(odd, d, d, 4, 1, 64, d, d, 4, 16, None) == cc.PCP_EINVAL
    assert L.pcp_kv_cache_write_fp8(d, d, d, 4, 1, 64, d, d, 4, 0, None) == cc.PCP_EINVAL
    assert L.pcp_kv_cache_write_fp8(d, d, d, -1, 1, 64, d, d, 4, 16, None) == cc.PCP_EINVAL


def test_size_limits_are_reported_before_launch(lib):
    """New-token K/V are fetched with 32-bit buffer offsets (total_k * Hkv * d
    * bytes per value below 4 GiB); a row's context length must fit int32
    (max_blocks * block_size). Both are checked for both element types."""
    L = cc.lib()
    d = ctypes.c_void_p(0x1000)
    big = (1 << 31) - 1  # keys: 2^31 * 256 values exceed 4 GiB at any element size
    assert L.pcp_attn_prefill(d, d, d, d, 1, 8, big, 8, 8, 1, 256, 0.1, d, d, None, 0,
                              None) == cc.PCP_EUNSUPPORTED
    assert L.pcp_attn_prefill_fp8(d, d, d, d, 1, 8, big, 8, 1, 8, 1, 256, 0.1, d, d, d, d, d,
                                  None, 0, None) == cc.PCP_EUNSUPPORTED
    # 2^24 keys x Hkv 1 x d 128: 4 GiB in bf16 (refused), 2 GiB in E4M3 (accepted by the check;
    # no launch happens because num_rows = 0 is a no-op)
    n = 1 << 24
    assert L.pcp_attn_prefill(d, d, d, d, 1, 8, n, 8, 8, 1, 128, 0.1, d, d, None, 0,
                              None) == cc.PCP_EUNSUPPORTED
    assert L.pcp_attn_prefill_fp8(d, d, d, d, 0, 8, n, 8, 1, 8, 1, 128, 0.1, d, d, d, d, d,
                                  None, 0, None) == 0
    # a max_q_len near INT32_MAX cannot wrap the unit count into a negative grid
    assert L.pcp_attn_prefill(d, d, d, d, 256, 8, 8, big, 1, 1, 64, 0.1, d, d, None, 0,
                              None) == cc.PCP_EOVERFLOW
    assert L.pcp_attn_rank_share(d, d, d, 8, d, d, 4, 16, d, 1, 1, d, 256, 8, big, 1, 1, 64,
                                 0.1, d, d, None, 1, None, 0, None) == cc.PCP_EOVERFLOW
    # context: max_blocks * block_size beyond int32
    assert L.pcp_attn_context_paged(d, d, d, 4, 1 << 16, d, 1, 1 << 16, d, 1, 8, 8, 8, 1, 128,
                                    0.1, d, d, None, 1, None, 0, None) == cc.PCP_EOVERFLOW
    assert L.pcp_attn_context_paged_fp8(d, d, d, 4, 1 << 16, d, 1, 1 << 16, d, 1, 8, 8, 8, 1,
                                        128, 0.1, d, d, d, d, d, None, 1, None, 0,
                                        None) == cc.PCP_EOVERFLOW


def test_noalloc_refuses_partials_beyond_its_scratch_before_launch(lib):
    """pcp_attn_rank_share_noalloc: a split count whose partials exceed the
    fixed scratch array is refused on the host (nothing is enqueued), as are
    split counts past 256; one split needs no scratch."""
    L = cc.lib()
    d = ctypes.c_void_p(0x1000)
    head = (d, d, d, 8, d, d, 4, 16, d, 8, 1, d, 8, 8, 8, 16, 1, 256, 0.1, d, d)
    need = cc.pcp_context_workspace_bytes(8, 16, 256, 256)
    assert need > cc.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert L.pcp_attn_rank_share_noalloc(*head, 256, None, 0, None) == cc.PCP_ESCRATCH
    assert L.pcp_attn_rank_share_noalloc(*head, 257, None, 0, None) == cc.PCP_EUNSUPPORTED
    assert L.pcp_attn_rank_share_noalloc(*head[:17], 96, *head[18:], 2, None, 0,
                                         None) == cc.PCP_EUNSUPPORTED
    # with no rows the call is a no-op whatever the split count fits
    empty = (None, None, None, 0, None, None, 0, 16, None, 0, 0, None, 0, 0, 0, 16, 1, 256, 0.1,
             None, None)
    assert L.pcp_attn_rank_share_noalloc(*empty, 1, None, 0, None) == 0


def test_context_workspace_bytes(lib):
    """(head_dim + 1) floats per (row, query head, split): the partial output
    and its LSE; nothing for one split or invalid arguments."""
    for rows, hq, d, s in ((1, 1, 64, 2), (7, 16, 128, 3), (12, 8, 256, 256)):
        assert cc.pcp_context_workspace_bytes(rows, hq, d, s) == rows * hq * s * (d + 1) * 4
    assert cc.pcp_context_workspace_bytes(0, 8, 128, 4) == 0
    assert cc.pcp_context_workspace_bytes(5, 8, 128, 1) == 0
    assert cc.pcp_context_workspace_bytes(5, 8, 96, 4) == 0
    assert cc.pcp_context_workspace_bytes(-1, 8, 128, 4) == 0
    assert cc.pcp_context_workspace_bytes(5, 8, 128, 0) == 0


def test_choose_decode_splits():
    def rows(q_lens, ctx_local):
        r = np.zeros((len(q_lens), 9), dtype=np.int32)
        r[:, 3], r[:, 8] = q_lens, ctx_local
        return r

    # no one-query row: no split
    assert cc.pcp_choose_decode_splits(rows([128, 64], [10 ** 6, 10 ** 6]), 8) == 1
    assert cc.pcp_choose_decode_splits(np.zeros((0, 9), np.int32), 8) == 1
    # 4 decode rows x 4 KV heads at 65536 keys: a CU's share is 4 * 4 * 65536 / 256
    # = 4096 keys, so 16 ranges per row (the 300-query row adds 12 workgroups)
    assert cc.pcp_choose_decode_splits(rows([1, 1, 1, 1, 300], [65536] * 5), 4) == 16
    # 16 rows x 8 KV heads at 30000: share 15000, 2 ranges; 5 rows: share 4687.5, 7
    assert cc.pcp_choose_decode_splits(rows([1] * 16, [30000] * 16), 8) == 2
    assert cc.pcp_choose_decode_splits(rows([1] * 5, [30000] * 5), 8) == 7
    # mixed lengths: the longest row sets the count (share 12000 * 64 / 256 = 3000)
    assert cc.pcp_choose_decode_splits(rows([1] * 5, [8000] + [1000] * 4), 64) == 3
    # 64 rows x 8 KV heads already fill the GPU
    assert cc.pcp_choose_decode_splits(rows([1] * 64, [8192] * 64), 8) == 1
    # ranges keep about 256 keys at least
    assert cc.pcp_choose_decode_splits(rows([1], [2048]), 1) == 8
    assert cc.pcp_choose_decode_splits(rows([1], [100]), 1) == 1
    assert cc.pcp_choose_decode_splits(rows([1], [0]), 1) == 1
    # never more than 256
    assert cc.pcp_choose_decode_splits(rows([1], [10 ** 7]), 1) == 256
    # many decode rows already fill the GPU
    assert cc.pcp_choose_decode_splits(rows([1] * 600, [10 ** 5] * 600), 1) == 1
    # so do rows with several queries and cached context (but not ones without)
    assert cc.pcp_choose_decode_splits(rows([1] * 4 + [4096] * 8, [5000] * 4 + [2000] * 8), 8) == 1
    assert cc.pcp_choose_decode_splits(rows([1] * 4 + [4096] * 8, [5000] * 4 + [0] * 8), 8) == 8


def _former_python_rule(rows_host, num_kv_heads, fused=False, fill_units=512, num_cus=256,
                        min_keys_per_split=256, max_splits=256):
    """The split rule as the Python binding computed it before the library
    took it over: the reference the C policy must reproduce."""
    r = np.asarray(rows_host).reshape(-1, 9)
    is_dec = (r[:, 3] == 1) & (r[:, 6] <= 0)
    dec = r[is_dec]
    if not len(dec) or num_kv_heads < 1:
        return 1
    units = len(dec) * int(num_kv_heads)
    multi = r[~is_dec & (r[:, 3] > 0) & ((r[:, 8] > 0) | (fused & (r[:, 6] > 0)))]
    others = int((-(-multi[:, 3].astype(np.int64) // 128)).sum()) * int(num_kv_heads)
    if units + others >= fill_units:
        return 1
    keys = np.maximum(dec[:, 8].astype(np.int64), 0)
    longest = int(keys.max())
    if longest <= 0:
        return 1
    share = max(int(keys.sum()) * int(num_kv_heads) / int(num_cus), float(min_keys_per_split))
    return int(max(1, min(-(-longest // share), max_splits)))


def test_decode_split_policy_matches_former_python_rule():
    """pcp_choose_decode_splits (C) gives the former Python rule's answer on
    the named workloads' plans, the decode-only batches and random plans."""
    from pcp_workloads import WORKLOADS, draw_lengths

    for name, w in WORKLOADS.items():
        new, ctx, dec = draw_lengths(w, np.random.default_rng(w.seed))
        cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        for fn in (cc.pcp_plan_rows, cc.pcp_plan_rows_resplit):
            rows = fn(cu, ctx, w.pcp_size, w.pcp_rank, w.dcp_size, w.dcp_rank, w.block_size)
            for fused in (False, True):
                assert cc.pcp_choose_decode_splits(rows, w.num_kv_heads, fused) == \
                    _former_python_rule(rows, w.num_kv_heads, fused), (name, fn, fused)
    rng = np.random.default_rng(77)
    for it in range(3000):
        n = int(rng.integers(0, 40))
        r = np.zeros((n, 9), dtype=np.int32)
        r[:, 3] = np.where(rng.random(n) < 0.6, 1, rng.integers(0, 5000, n))
        r[:, 6] = np.where(rng.random(n) < 0.7, 0, rng.integers(-2, 9000, n))
        scale = int(rng.choice([10, 1000, 100000, 3000000]))
        r[:, 8] = rng.integers(-5, scale, n)
        hkv = int(rng.choice([1, 2, 4, 8, 16, 64]))
        for fused in (False, True):
            assert cc.pcp_choose_decode_splits(r, hkv, fused) == \
                _former_python_rule(r, hkv, fused), (it, r.tolist(), hkv, fused)
    with pytest.raises(cc.PcpError):
        cc.pcp_choose_decode_splits(np.zeros((1, 9), np.int32), 0)


def test_bindings_reject_a_plan_of_the_wrong_width():
    """Every attention binding checks that the plan tensor is [R, 9] before
    anything else (the kernels read rows with the pcp_row_t stride)."""
    import torch

    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    kv = torch.zeros((4, 1, 64), dtype=torch.bfloat16)
    cache = torch.zeros((2, 16, 1, 64), dtype=torch.bfloat16)
    bt = torch.zeros((1, 2), dtype=torch.int32)
    lse = torch.zeros((2, 4))
    ds = torch.ones((1, 1))
    for rows in (torch.zeros((2, 8), dtype=torch.int32), torch.zeros((2, 10), dtype=torch.int32),
                 torch.zeros(18, dtype=torch.int32)):
        calls = (
            lambda: cc.pcp_attn_prefill(q, kv, kv, rows, q, lse, 0.1, 4),
            lambda: cc.pcp_attn_context_paged(q, cache, cache, bt, rows, q, lse, 0.1, 4),
            lambda: cc.pcp_attn_rank_share(q, kv, kv, cache, cache, bt, rows, q, lse, 0.1, 4),
            lambda: cc.pcp_attn_prefill_fp8(q, kv, kv, rows, q, lse, 0.1, 4, ds, ds, ds),
            lambda: cc.pcp_attn_context_paged_fp8(q, cache, cache, bt, rows, q, lse, 0.1, 4, ds,
                                                  ds, ds),
            lambda: cc.pcp_attn_rank_share_fp8(q, kv, kv, cache, cache, bt, rows, q, lse, 0.1, 4,
                                               ds, ds, ds),
        )
        for call in calls:
            with pytest.raises(ValueError, match="rows must be"):
                call()


def test_python_plan_helpers(lib):
    rows = cc.pcp_plan_rows([0, 512], [0], 2, 0)
    assert cc.plan_max_q_len(rows) == 128 and cc.plan_total_q(rows) == 256


# ----------------------------------------------------------------- unit schedule


def _expected_units(rows, pass_, max_q_len, hq, hkv, d, splits):
    """(unit id -> key tiles) of every unit the kernels run, enumerated from
    the geometry pcp_attn_schedule documents: HG heads per workgroup (largest
    of 8, 4, 2, 1 dividing Hq/Hkv), 256/HG queries per tile, 32 keys per tile
    at d = 256 else 64, and one slot per key range of a split one-query row."""
    g = hq // hkv
    hg = next(h for h in (8, 4, 2, 1) if g % h == 0)
    groups, bq, bn = hkv * (g // hg), 256 // hg, (32 if d == 256 else 64)
    qt = -(-max_q_len // bq)
    if pass_ != 0 and splits > qt:
        qt = splits
    units = {}
    for r, row in enumerate(rows):
        ql, kl, ctx = int(row[3]), int(row[6]), int(row[8])
        split = pass_ != 0 and splits > 1 and ql == 1 and kl <= 0
        for grp in range(groups):
            for q in range(qt):
                if split:
                    if q >= splits:
                        continue
                    total = -(-ctx // bn)
                    per = -(-total // splits)
                    tiles = max(0, min(total - q * per, per))
                else:
                    if ql <= q * bq:
                        continue
                    tiles = 0
                    if pass_ != 0:  # context tiles
                        tiles += -(-ctx // bn)
                    if pass_ != 1:  # new-token tiles
                        t_last = min(q * bq + bq, ql) - 1
                        tiles += -(-max(0, min(kl, kl - ql + t_last + 1)) // bn)
                units[(r * groups + grp) * qt + q] = tiles
    return units, qt, groups


def _builtin_order(num_rows, groups, qt):
    """The kernels' own launch order: rows in reverse plan order, query tiles
    last to first, runs of 4 consecutive units dealt to the 8 XCDs."""
    n = num_rows * groups * qt
    w = 8 * 4
    full = n // w * w
    out = np.empty(n, dtype=np.int32)
    for b in range(n):
        u = b
        if b < full:
            win, within = divmod(b, w)
            u = win * w + (within % 8) * 4 + within // 8
        qt_rev, rest = u % qt, u // qt
        grp, row = rest % groups, num_rows - 1 - rest // groups
        out[b] = (row * groups + grp) * qt + qt - 1 - qt_rev
    return out


def test_schedule_prefers_longest_first_only_where_it_pays():
    # a mixed batch of unequal requests: longest first (no padding units)
    cu = np.concatenate([[0], np.cumsum([4096, 1024, 2048, 4096, 512, 3000, 1, 1])])
    rows = cc.pcp_plan_rows(cu, [0, 700, 0, 3000, 10, 0, 900, 5000], 2, 1)
    mq = cc.plan_max_q_len(rows)
    order = cc.pcp_attn_schedule(0, rows, mq, 16, 8, 128)
    want, qt, groups = _expected_units(rows, 0, mq, 16, 8, 128, 1)
    assert sorted(order[order >= 0].tolist()) == sorted(want)
    assert not np.array_equal(order, _builtin_order(len(rows), groups, qt))
    # one long prompt: the built-in order is already balanced and is kept
    rows = cc.pcp_plan_rows([0, 131072], [0], 4, 1)
    order = cc.pcp_attn_schedule(0, rows, cc.plan_max_q_len(rows), 8, 1, 256)
    assert np.array_equal(order, _builtin_order(2, 1, 512))


@pytest.mark.parametrize("case", range(8))
def test_schedule_is_a_balanced_longest_first_permutation(lib, case):
    rng = np.random.default_rng(100 + case)
    hq, hkv, d = [(16, 8, 128), (8, 1, 256), (4, 4, 64), (12, 4, 128), (32, 4, 128),
                  (8, 2, 256), (6, 2, 64), (16, 1, 128)][case]
    b = int(rng.integers(1, 12))
    new = rng.integers(0, 3000, size=b)
    new[rng.random(b) < 0.3] = 1
    ctx = rng.integers(0, 5000, size=b)
    cu = np.concatenate([[0], np.cumsum(new)])
    p = int(rng.integers(1, 5))
    dd = int(rng.integers(1, 4))
    rows = cc.pcp_plan_rows(cu, ctx, p, int(rng.integers(0, p)), dd, int(rng.integers(0, dd)), 16)
    mq = cc.plan_max_q_len(rows) + int(rng.integers(0, 300))
    for pass_, splits in ((0, 1), (1, 1), (1, int(rng.integers(2, 40))), (2, 1),
                          (2, int(rng.integers(2, 40)))):
        order = cc.pcp_attn_schedule(pass_, rows, mq, hq, hkv, d, splits)
        want, qt, groups = _expected_units(rows, pass_, mq, hq, hkv, d, splits)
        real = order[order >= 0]
        if len(real) != len(want) or np.array_equal(order, _builtin_order(len(rows), groups, qt)):
            # the built-in order: every unit slot, including ones that exit at once
            assert np.array_equal(order, _builtin_order(len(rows), groups, qt))
            assert set(want) <= set(order.tolist())
            continue
        assert len(order) % 8 == 0
        assert sorted(real.tolist()) == sorted(want), "every unit exactly once"
        loads = []
        for x in range(8):
            qx = order[x::8].tolist()
            n = sum(1 for u in qx if u >= 0)
            assert all(u >= 0 for u in qx[:n]) and all(u < 0 for u in qx[n:])
            tiles = [want[u] for u in qx[:n]]
            assert tiles == sorted(tiles, reverse=True), "longest first on each XCD"
            loads.append(sum(t + 2 for t in tiles))
        # runs of 4 neighbouring query tiles of one (row, group) share an XCD
        xcd_of = {int(u): i % 8 for i, u in enumerate(order) if u >= 0}
        runs = {}
        for u in sorted(want, reverse=True):
            runs.setdefault(u // qt, []).append(u)
        biggest_run = 0
        for us in runs.values():
            for k in range(0, len(us), 4):
                assert len({xcd_of[u] for u in us[k:k + 4]}) == 1
                biggest_run = max(biggest_run, sum(want[u] + 2 for u in us[k:k + 4]))
        if want:
            assert max(loads) - min(loads) <= biggest_run, "XCD loads balanced"
        # deterministic; a short buffer gets the prefix and the full count
        assert np.array_equal(order, cc.pcp_attn_schedule(pass_, rows, mq, hq, hkv, d, splits))
        if len(order) > 3:
            buf = np.full(len(order), -7, dtype=np.int32)
            n = lib.pcp_attn_schedule(pass_, np.ascontiguousarray(rows, np.int32).ctypes.data,
                                      len(rows), mq, hq, hkv, d, splits, 2, buf.ctypes.data, 3)
            assert n == len(order) and np.array_equal(buf[:3], order[:3]) and (buf[3:] == -7).all()


def _is_grouped(order, rows, want, qt, groups, hq, hkv):
    """True when every (request, KV head) group of units sits on one XCD,
    contiguous in its queue and longest first, the groups of each XCD in
    non-increasing total cost; asserts the order is a padded permutation."""
    g = hq // hkv
    hg = next(h for h in (8, 4, 2, 1) if g % h == 0)
    real = order[order >= 0]
    assert sorted(real.tolist()) == sorted(want), "every unit exactly once"
    kv = {u: int(rows[u // (groups * qt)][0]) * hkv + ((u // qt) % groups) // (g // hg) for u in want}
    cost = {}
    for u in want:
        cost[kv[u]] = cost.get(kv[u], 0) + want[u] + 2
    for x in range(8):
        qx = [int(u) for u in order[x::8]]
        n = sum(1 for u in qx if u >= 0)
        if not all(u >= 0 for u in qx[:n]) or any(u >= 0 for u in qx[n:]):
            return False
        seen, prev_cost = [], None
        for i, u in enumerate(qx[:n]):
            if i == 0 or kv[u] != kv[qx[i - 1]]:
                if kv[u] in seen or (prev_cost is not None and cost[kv[u]] > prev_cost):
                    return False
                seen.append(kv[u])
                prev_cost = cost[kv[u]]
            elif want[u] > want[qx[i - 1]]:
                return False
    return True


def test_schedule_keeps_kv_groups_together_beyond_the_cache():
    # 32 Qwen-shaped requests: 256 (request, KV head) groups reading 403 MB of
    # bf16 K/V, more than the 256 MB Infinity Cache, each a small share of an
    # XCD's work: whole groups per XCD
    # (E4M3 K/V: half the bytes, so 32 requests fit the cache and 64 do not)
    for b, eb, grouped in ((32, 2, True), (64, 2, True), (16, 2, False), (8, 2, False),
                           (32, 1, False), (64, 1, True)):
        rows = cc.pcp_plan_rows(np.arange(b + 1) * 4096, [0] * b, 2, 1)
        mq = cc.plan_max_q_len(rows)
        order = cc.pcp_attn_schedule(0, rows, mq, 16, 8, 128, 1, kv_elem_bytes=eb)
        want, qt, groups = _expected_units(rows, 0, mq, 16, 8, 128, 1)
        assert _is_grouped(order, rows, want, qt, groups, 16, 8) == grouped, (b, eb)
        if grouped:  # balanced to within one group
            loads = [sum(want[u] + 2 for u in order[x::8] if u >= 0) for x in range(8)]
            assert max(loads) - min(loads) <= max(want.values()) * 16
    # one prompt whose K/V (400 MB) exceeds the cache: one group, not grouped
    rows = cc.pcp_plan_rows([0, 409600], [0], 4, 1)
    mq = cc.plan_max_q_len(rows)
    order = cc.pcp_attn_schedule(0, rows, mq, 8, 1, 256)
    want, qt, groups = _expected_units(rows, 0, mq, 8, 1, 256, 1)
    assert np.array_equal(order, _builtin_order(len(rows), groups, qt))


def test_schedule_rejects_bad_arguments(lib):
    rows = cc.pcp_plan_rows([0, 512], [0], 2, 0)
    r = np.ascontiguousarray(rows, np.int32)
    L = cc.lib()
    assert L.pcp_attn_schedule(3, r.ctypes.data, len(r), 128, 4, 2, 64, 1, 2, None, 0) == cc.PCP_EINVAL
    # a row longer than max_q_len
    assert L.pcp_attn_schedule(0, r.ctypes.data, len(r), 100, 4, 2, 64, 1, 2, None, 0) == cc.PCP_EINVAL
    assert L.pcp_attn_schedule(0, r.ctypes.data, len(r), 128, 4, 3, 64, 1, 2, None, 0) == cc.PCP_EINVAL
    assert L.pcp_attn_schedule(0, r.ctypes.data, len(r), 128, 4, 2, 80, 1, 2, None,
                               0) == cc.PCP_EUNSUPPORTED
    assert L.pcp_attn_schedule(0, r.ctypes.data, len(r), 128, 4, 2, 64, 0, 2, None, 0) == cc.PCP_EINVAL
    assert L.pcp_attn_schedule(0, None, 2, 128, 4, 2, 64, 1, 2, None, 0) == cc.PCP_EINVAL
    assert L.pcp_attn_schedule(0, r.ctypes.data, len(r), 128, 4, 2, 64, 1, 2, None, 4) == cc.PCP_EINVAL
    assert L.pcp_attn_schedule(0, None, 0, 0, 4, 2, 64, 1, 2, None, 0) == 0
    # K/V element size: 2 (bf16) or 1 (E4M3)
    for eb in (0, 3, 4):
        assert L.pcp_attn_schedule(0, r.ctypes.data, len(r), 128, 4, 2, 64, 1, eb, None,
                                   0) == cc.PCP_EINVAL
    assert L.pcp_attn_schedule(0, r.ctypes.data, len(r), 128, 4, 2, 64, 1, 1, None, 0) > 0
