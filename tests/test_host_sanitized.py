"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

tests/host_sanitize_driver.cpp is compiled with the host sources of
libpcpattn -- the row plans and the slot mapping (pcp_plan.cpp), the launch
order and the decode-split rule (pcp_sched.cpp), and the attention calls'
argument checks (pcp_attn_check.h) -- by g++ with -fsanitize=address,undefined
and no recovery, so the first out-of-bounds access, overflow or other
undefined behaviour aborts the driver. Every buffer the library writes is a
heap array of exactly the capacity passed, so a write past it is caught.

The driver is fed random batches and plans plus edge cases (capacities too
small, int32 extremes in every row field and size) and its answers are
compared with the oracle (plans, slot mappings) and with the GPU library's own
entry points through ctypes (schedules, split counts, argument checks). The
entry points are only called where the checks reject the arguments or find
nothing to do, so no kernel is ever launched.

This is where the pages' crash class lives: a plan buffer sized for the
requests rather than the rows ("[MRv2][PCP] Carry the row plan in attention
metadata; fix mixed prefill+decode crash", section "Two things that fell out
of (1)": 8 requests, 14 rows).
"""

import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from pcp_workloads import random_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_causal_gqa_amd", "csrc")
DRIVER_SRC = os.path.join(ROOT, "tests", "host_sanitize_driver.cpp")

cc = pytest.importorskip("context_causal_gqa_amd")

I32_MIN, I32_MAX = -(1 << 31), (1 << 31) - 1


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    out = str(tmp_path_factory.mktemp("san") / "host_sanitize_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, DRIVER_SRC, os.path.join(CSRC, "pcp_plan.cpp"),
           os.path.join(CSRC, "pcp_sched.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return out


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cc.LIB_PATH):
        import context_causal_gqa_amd.build as b

        b.build()
    return cc.lib()


def run_driver(driver, lines):
    """Runs the sanitized driver on the command lines; returns its answer lines."""
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=97",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=98")
    res = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         env=env, timeout=300)
    assert res.returncode == 0, "sanitizer report:\n" + res.stderr[-6000:]
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr, \
        res.stderr[-6000:]
    return res.stdout.split("\n")


def ints(*xs):
    return " ".join(str(int(x)) for x in np.concatenate([np.ravel(np.asarray(x)) for x in xs]))


class Answers:
    def __init__(self, lines):
        self.lines = lines
        self.i = 0

    def int(self):
        v = int(self.lines[self.i])
        self.i += 1
        return v

    def ints(self, n, width=1):
        if n == 0:
            return np.zeros((0, width), dtype=np.int64)
        if width == 1:
            v = np.array(self.lines[self.i].split(), dtype=np.int64)
            self.i += 1
            return v
        v = np.array([l.split() for l in self.lines[self.i:self.i + n]], dtype=np.int64)
        self.i += n
        return v


def _batches(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        new, ctx = random_batch(rng)
        cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int64)
        p = int(rng.integers(1, 5))
        dd = int(rng.integers(1, 5))
        out.append((cu, np.asarray(ctx, np.int64), p, int(rng.integers(p)), dd,
                    int(rng.integers(dd)), int(rng.choice([1, 5, 16, 64]))))
    return out


def test_plans_under_sanitizers_match_the_oracle(driver):
    """Both plans for random batches, with capacities below, at and above
    the row count: the count and every written row match the oracle, and no
    row is written past the capacity."""
    cases, lines = [], []
    rng = np.random.default_rng(5)
    for cu, ctx, p, r, dd, rd, bs in _batches(11, 400):
        for resplit in (0, 1):
            fn = oracle.plan_rows_resplit if resplit else oracle.plan_rows
            want = fn(cu, ctx, p, r, dd, rd, bs)
            cap = int(rng.choice([0, max(0, len(want) - 1), len(want), len(want) + 3]))
            cases.append((want, cap))
            lines.append("PLAN " + ints(resplit, len(ctx), p, r, dd, rd, bs, cap, cu, ctx))
    ans = Answers(run_driver(driver, lines))
    for want, cap in cases:
        n = ans.int()
        assert n == len(want)
        got = ans.ints(min(n, cap), 9)
        assert np.array_equal(got, want[:min(n, cap)])


def test_plan_argument_errors_under_sanitizers(driver):
    """Bad ranks, sizes and lengths, and offsets past int32, are reported as
    errors (the same codes as the library's), without undefined behaviour."""
    cu, ctx = [0, 512, 513], [0, 40]
    bad = [
        (2, 2, 1, 0, 16), (2, -1, 1, 0, 16), (0, 0, 1, 0, 16), (2, 0, 0, 0, 16),
        (2, 0, 2, 2, 16), (2, 0, 1, 0, 0), (2, 0, 1, 0, -5),
    ]
    lines = ["PLAN " + ints(0, 2, *b, 4, cu, ctx) for b in bad]
    # decreasing cu_seqlens, a negative cached length, positions past int32
    lines.append("PLAN " + ints(0, 2, 2, 0, 1, 0, 16, 4, [0, 512, 500], ctx))
    lines.append("PLAN " + ints(0, 2, 2, 0, 1, 0, 16, 4, cu, [0, -1]))
    lines.append("PLAN " + ints(1, 1, 2, 0, 1, 0, 16, 4, [0, 1 << 30], [I32_MAX - 10]))
    lines.append("PLAN " + ints(0, 1, 2, 1, 3, 2, 7, 4, [I32_MAX - 5, I32_MAX], [I32_MAX]))
    lines.append("PLAN " + ints(0, -1, 2, 0, 1, 0, 16, 0))  # B < 0: no arrays follow
    ans = Answers(run_driver(driver, lines))
    got = [ans.int() for _ in lines]
    L = cc.lib()
    for line, g in zip(lines, got):
        f = [int(x) for x in line.split()[1:]]
        resplit, b = f[0], f[1]
        if b < 0:
            assert g == cc.PCP_EINVAL
            continue
        cu_a = np.array(f[8:9 + b], np.int32)
        ctx_a = np.array(f[9 + b:9 + 2 * b], np.int32)
        buf = np.zeros((4, 9), np.int32)
        fn = L.pcp_plan_rows_resplit if resplit else L.pcp_plan_rows
        want = fn(b, cu_a.ctypes.data, ctx_a.ctypes.data, *f[2:7], buf.ctypes.data, 4)
        assert g == want and g < 0, (line, g, want)


def test_slot_mapping_under_sanitizers(driver):
    """Slot mappings of random batches against the oracle, with tables that
    hold every block or miss one (an error), and short capacities."""
    cases, lines = [], []
    rng = np.random.default_rng(9)
    for cu, ctx, p, r, dd, rd, bs in _batches(13, 300):
        b = len(ctx)
        new = np.diff(cu)
        need = (ctx + new + bs - 1) // bs
        maxb = int(need.max()) if b else 0
        table = rng.permutation(max(1, b * maxb) + 5)[:b * maxb].reshape(b, maxb).astype(np.int64)
        short = b > 0 and maxb > 0 and rng.random() < 0.25
        if short:
            i = int(rng.integers(b))
            table[i, need[i] - 1] = -1
        n = int(cu[-1])
        cap = int(rng.choice([0, max(0, n - 7), n]))
        lines.append("SLOT " + ints(b, maxb, dd, rd, bs, cap, cu, ctx, table))
        cases.append((cu, ctx, table, dd, rd, bs, cap, n, short))
    ans = Answers(run_driver(driver, lines))
    for cu, ctx, table, dd, rd, bs, cap, n, short in cases:
        got_n = ans.int()
        if got_n < 0:
            assert got_n == cc.PCP_EINVAL
            # only a missing block this rank owns is an error
            want = cc.lib().pcp_slot_mapping(
                len(ctx), np.ascontiguousarray(cu, np.int32).ctypes.data,
                np.ascontiguousarray(ctx, np.int32).ctypes.data,
                np.ascontiguousarray(table, np.int32).ctypes.data, table.shape[1], dd, rd, bs,
                None, 0)
            assert want == cc.PCP_EINVAL
            continue
        assert got_n == n
        got = ans.ints(min(n, cap)) if min(n, cap) else np.zeros(0, np.int64)
        if not short:
            want = oracle.slot_mapping(cu, ctx, table, dd, rd, bs)
            assert np.array_equal(got, want[:min(n, cap)])


def _random_rows(rng, n, extreme):
    r = np.zeros((n, 9), dtype=np.int64)
    r[:, 0] = rng.integers(0, 6, n)
    r[:, 3] = np.where(rng.random(n) < 0.4, 1, rng.integers(0, 3000, n))
    r[:, 6] = np.where(rng.random(n) < 0.4, 0, rng.integers(0, 9000, n))
    r[:, 8] = rng.integers(0, 40000, n)
    if extreme:
        for col in (0, 6, 8):
            pick = rng.random(n) < 0.3
            r[pick, col] = rng.choice([I32_MIN, -1, I32_MAX, I32_MAX - 1], pick.sum())
    return r


def test_schedule_and_split_rule_under_sanitizers(driver, lib):
    """Launch orders and split counts for random plans, int32 extremes in the
    row fields included, equal the library's own answers through ctypes."""
    rng = np.random.default_rng(21)
    cases, lines = [], []
    for it in range(250):
        huge_q = it % 7 == 0  # max_q_len = INT32_MAX: a unit count past int32
        n = int(rng.integers(5 if huge_q else 0, 12))
        rows = _random_rows(rng, n, extreme=it % 3 == 0)
        hkv = 8 if huge_q else int(rng.choice([1, 2, 8]))
        hq = hkv * (8 if huge_q else int(rng.choice([1, 2, 3, 8])))
        d = int(rng.choice([64, 128, 256]))
        pass_ = int(rng.integers(3))
        splits = int(rng.choice([1, 2, 7, 64]))
        eb = int(rng.choice([1, 2]))
        mq = I32_MAX if huge_q else (int(rows[:, 3].max()) if n else 0)
        cap = int(rng.choice([0, 5, 100000]))
        lines.append("SCHED " + ints(pass_, n, mq, hq, hkv, d, splits, eb, cap, rows))
        fused = int(rng.integers(2))
        lines.append("SPLITS " + ints(n, hkv, fused, rows))
        cases.append((rows, pass_, mq, hq, hkv, d, splits, eb, cap, fused, huge_q))
    ans = Answers(run_driver(driver, lines))
    for rows, pass_, mq, hq, hkv, d, splits, eb, cap, fused, huge_q in cases:
        n = ans.int()
        got = ans.ints(min(n, cap)) if n > 0 and cap > 0 else np.zeros(0, np.int64)
        r32 = np.ascontiguousarray(rows, dtype=np.int32)
        order = np.zeros(max(cap, 1), np.int32)
        want = lib.pcp_attn_schedule(pass_, r32.ctypes.data if len(r32) else None, len(r32), mq,
                                     hq, hkv, d, splits, eb, order.ctypes.data, cap)
        assert n == want
        if huge_q:
            assert n == cc.PCP_EOVERFLOW
        if n > 0:
            assert np.array_equal(got, order[:min(n, cap)])
        s = ans.int()
        assert s == lib.pcp_choose_decode_splits(r32.ctypes.data if len(r32) else None,
                                                 len(r32), hkv, fused)
        assert 1 <= s <= 256


# (q, k, v, kc, vc, q_ds, k_ds, v_ds, rows, block_tables, out, lse, workspace, order)
ALL_PTRS = (1 << 14) - 1
PTR_BITS = ("q", "k", "v", "kc", "vc", "q_ds", "k_ds", "v_ds", "rows", "bt", "out", "lse",
            "ws", "order")


def _entry_point_rc(lib, pass_, fp8, f, ptrs):
    """The return code of the matching C-ABI entry point for CHECK fields f."""
    (num_rows, total_q, total_k, max_q_len, num_blocks, block_size, num_reqs, max_blocks, hq, hkv,
     d, splits, num_units, scale_x1000) = f
    base = 0x10008 if (ptrs >> 14) & 1 else 0x10000
    p = {name: (ctypes.c_void_p(base + 0x1000 * i) if (ptrs >> i) & 1 else None)
         for i, name in enumerate(PTR_BITS)}
    scale = ctypes.c_float(scale_x1000 / 1000.0)
    if pass_ == 0 and not fp8:
        return lib.pcp_attn_prefill(p["q"], p["k"], p["v"], p["rows"], num_rows, total_q, total_k,
                                    max_q_len, hq, hkv, d, scale, p["out"], p["lse"], p["order"],
                                    num_units, None)
    if pass_ == 0:
        return lib.pcp_attn_prefill_fp8(p["q"], p["k"], p["v"], p["rows"], num_rows, total_q,
                                        total_k, max_q_len, num_reqs, hq, hkv, d, scale,
                                        p["q_ds"], p["k_ds"], p["v_ds"], p["out"], p["lse"],
                                        p["order"], num_units, None)
    ctx = (p["q"], p["kc"], p["vc"], num_blocks, block_size, p["bt"], num_reqs, max_blocks,
           p["rows"], num_rows, total_q, max_q_len, hq, hkv, d, scale)
    if pass_ == 1 and not fp8:
        return lib.pcp_attn_context_paged(*ctx, p["out"], p["lse"], p["ws"], splits, p["order"],
                                          num_units, None)
    if pass_ == 1:
        return lib.pcp_attn_context_paged_fp8(*ctx, p["q_ds"], p["k_ds"], p["v_ds"], p["out"],
                                              p["lse"], p["ws"], splits, p["order"], num_units,
                                              None)
    fused = (p["q"], p["k"], p["v"], total_k, p["kc"], p["vc"], num_blocks, block_size, p["bt"],
             num_reqs, max_blocks, p["rows"], num_rows, total_q, max_q_len, hq, hkv, d, scale)
    if not fp8:
        return lib.pcp_attn_rank_share(*fused, p["out"], p["lse"], p["ws"], splits, p["order"],
                                       num_units, None)
    return lib.pcp_attn_rank_share_fp8(*fused, p["q_ds"], p["k_ds"], p["v_ds"], p["out"],
                                       p["lse"], p["ws"], splits, p["order"], num_units, None)


def test_argument_checks_under_sanitizers(driver, lib):
    """The attention calls' argument checks on hand-picked and random
    arguments, int32 extremes included: no undefined behaviour, the
    documented codes for the hand-picked ones, and the entry points return
    the same code wherever the checks reject the call (calls the checks
    accept are not made: they would launch)."""
    ok = (1, 64, 64, 64, 8, 16, 1, 8, 8, 1, 128, 1, 0, 88)
    hand = [  # (pass, fp8, fields, ptr mask, expected)
        (0, 0, ok, ALL_PTRS, 0),
        (1, 0, ok, ALL_PTRS, 0),
        (2, 1, ok, ALL_PTRS, 0),
        (2, 0, (0,) + ok[1:], ALL_PTRS, 1),  # no rows: nothing to do
        (0, 0, ok[:10] + (96,) + ok[11:], ALL_PTRS, cc.PCP_EUNSUPPORTED),
        (0, 0, ok[:8] + (6, 4) + ok[10:], ALL_PTRS, cc.PCP_EINVAL),
        (2, 0, ok[:13] + (0,), ALL_PTRS, cc.PCP_EINVAL),  # scale 0
        (1, 0, ok[:11] + (2,) + ok[12:], ALL_PTRS & ~(1 << 12), cc.PCP_EINVAL),  # no workspace
        (1, 0, ok[:11] + (257,) + ok[12:], ALL_PTRS, cc.PCP_EUNSUPPORTED),
        (2, 1, ok, ALL_PTRS | (1 << 14), cc.PCP_EINVAL),  # misaligned codes
        (2, 1, ok, ALL_PTRS & ~(1 << 6), cc.PCP_EINVAL),  # no k descale
        # unit count past int32 from a max_q_len near INT32_MAX
        (0, 0, (256, 8, 8, I32_MAX, 8, 16, 1, 8, 1, 1, 64, 1, 0, 100), ALL_PTRS,
         cc.PCP_EOVERFLOW),
        (2, 0, (1 << 20, 8, 8, 1 << 20, 8, 16, 1, 8, 8, 1, 64, 1, 0, 100), ALL_PTRS,
         cc.PCP_EOVERFLOW),
        # context length past int32
        (1, 0, (1, 8, 8, 8, 8, 1 << 16, 1, 1 << 16, 8, 1, 64, 1, 0, 100), ALL_PTRS,
         cc.PCP_EOVERFLOW),
        # new-token K/V past 32-bit offsets
        (0, 0, (1, 8, I32_MAX, 8, 8, 16, 1, 8, 8, 1, 256, 1, 0, 100), ALL_PTRS,
         cc.PCP_EUNSUPPORTED),
    ]
    rng = np.random.default_rng(3)
    fuzz = []
    vals = np.array([I32_MIN, -1, 0, 1, 2, 7, 16, 64, 128, 256, 257, 1 << 20, I32_MAX - 1,
                     I32_MAX], dtype=np.int64)
    for _ in range(3000):
        f = tuple(int(x) for x in rng.choice(vals, 14))
        f = f[:8] + (int(rng.choice([1, 2, 8, f[8]])), int(rng.choice([1, f[9]])),
                     int(rng.choice([64, 128, 256, f[10]]))) + f[11:]
        fuzz.append((int(rng.integers(3)), int(rng.integers(2)), f,
                     int(rng.integers(0, 1 << 15)), None))
    cases = hand + fuzz
    lines = ["CHECK " + ints(pa, fp8, f, ptrs) for pa, fp8, f, ptrs, _ in cases]
    ans = Answers(run_driver(driver, lines))
    for pa, fp8, f, ptrs, want in cases:
        rc = ans.int()
        if want is not None:
            assert rc == want, (pa, fp8, f, ptrs, rc, want)
        if rc != 0:  # rejected (or nothing to do): the entry point answers the same
            ep = _entry_point_rc(lib, pa, fp8, f, ptrs)
            assert ep == (0 if rc == 1 else rc), (pa, fp8, f, ptrs, rc, ep)
