"""GPU parity over a seeded random sweep of small shares.

Each case draws a head layout (d in 64/128/256, 1-4 KV heads, 1-16 query
heads per KV head), a PCP and DCP split with a rank of each, a cache block
size (5, 8, 16, 32 or 64: both paged-load paths, blocks smaller than, equal
to and larger than a key tile) and 1-5 requests mixing prefill rows of
1-700 new tokens and decode rows, with cached prefixes of 0-1500 tokens.
The three calls and the fused launch (every output buffer NaN-filled first)
are compared with the fp64 oracle on every output; every third case also
forces a decode split count and runs the E4M3 path. The draws are fixed by
the case index, so a failure names a reproducible shape.
"""

import numpy as np
import pytest

from pcp_workloads import Workload, generate

from test_gpu_parity import cc, check_share, run_share  # noqa: F401 (cc is a fixture)
from test_gpu_fp8 import check_share_fp8, fp8_inputs, run_share_fp8

N_CASES = 96


def draw_case(i):
    rng = np.random.default_rng(7700 + i)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    while hkv * group > 32:
        group //= 2
    pcp = int(rng.integers(1, 5))
    dcp = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([5, 8, 16, 32, 64]))
    n_req = int(rng.integers(1, 6))
    new, ctx = [], []
    for _ in range(n_req):
        if rng.random() < 0.35:
            new.append(1)
            ctx.append(int(rng.integers(0, 1501)))
        else:
            new.append(int(rng.integers(1, 701)))
            ctx.append(0 if rng.random() < 0.4 else int(rng.integers(1, 1501)))
    if all(n == 1 for n in new) and rng.random() < 0.5:
        new[0] = int(rng.integers(2, 400))  # keep some prefill work in most cases
    w = Workload(name="sweep%d" % i, seed=7800 + i, num_q_heads=hkv * group, num_kv_heads=hkv,
                 head_dim=d, pcp_size=pcp, pcp_rank=int(rng.integers(0, pcp)), dcp_size=dcp,
                 dcp_rank=int(rng.integers(0, dcp)), block_size=bs, new_lens=tuple(new),
                 ctx_lens=tuple(ctx))
    splits = int(rng.choice([2, 3, 7])) if i % 3 == 0 else None
    return w, splits


def _describe(w, splits):
    return ("%s: d=%d hq=%d hkv=%d pcp=%d/%d dcp=%d/%d bs=%d new=%s ctx=%s splits=%s"
            % (w.name, w.head_dim, w.num_q_heads, w.num_kv_heads, w.pcp_rank, w.pcp_size,
               w.dcp_rank, w.dcp_size, w.block_size, w.new_lens, w.ctx_lens, splits))


def test_sweep_draws_cover_the_paths():
    """The fixed draws include every head dim, both paged-load paths (block
    sizes that are and are not a multiple of a 1 KB chunk's key rows),
    decode rows, cached prefixes, DCP > 1 and forced splits."""
    cases = [draw_case(i) for i in range(N_CASES)]
    ws = [w for w, _ in cases]
    assert {w.head_dim for w in ws} == {64, 128, 256}
    assert any(w.block_size == 5 for w in ws) and any(w.block_size >= 32 for w in ws)
    assert any(1 in w.new_lens for w in ws)
    assert any(max(w.ctx_lens) > 0 for w in ws)
    assert any(w.dcp_size > 1 for w in ws) and any(w.pcp_size > 1 for w in ws)
    assert any(s is not None for _, s in cases)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case_full_parity(cc, i):
    w, splits = draw_case(i)
    what = _describe(w, splits)
    print(what, flush=True)
    inp = generate(w)
    kw = {} if splits is None else {"decode_splits": splits}
    share = run_share(cc, inp, **kw)
    check_share(inp, share, what=what)
    if i % 3 == 0:
        f = fp8_inputs(inp, jitter_seed=i)
        s8 = run_share_fp8(inp, f, **kw)
        check_share_fp8(inp, f, s8, what=what + " fp8")
