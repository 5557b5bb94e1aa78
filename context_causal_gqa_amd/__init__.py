"""Python binding of libpcpattn: one prefill-context-parallel (PCP) rank's
share of causal grouped-query attention on an MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in ``include/pcp_attn.h``; the
functions keep the C names. Every step of the computation runs in the HIP
library; this module only checks tensor shapes, dtypes and devices, passes
``data_ptr()`` values and the current HIP stream, and raises ``PcpError`` on a
negative return code. There is no fallback: if the library is not built the
calls raise.

Tensors (torch, on the GPU unless stated):
  q, out        [total_q, Hq, d]  bfloat16, contiguous
  k, v          [total_k, Hkv, d] bfloat16 (new-token pass)
  k_cache, v_cache [num_blocks, block_size, Hkv, d] bfloat16 (context pass)
  block_tables  [num_reqs, max_blocks] int32
  lse           [Hq, total_q] float32 (natural log)
  rows          [R, 9] int32, columns ROW_FIELDS (the pcp_row_t struct)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpcpattn.so")

ROW_FIELDS = ("req", "kind", "q_start", "q_len", "pos_start", "k_start", "k_len", "ctx_len",
              "ctx_len_local")
ROW_HEAD, ROW_TAIL, ROW_DECODE = 0, 1, 2

PCP_OK, PCP_EINVAL, PCP_EUNSUPPORTED, PCP_EHIP, PCP_EOVERFLOW, PCP_ESCRATCH = 0, -1, -2, -3, -4, -5
# scratch array of pcp_attn_rank_share_noalloc, per device (PCP_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20


class PcpError(RuntimeError):
    """A negative return code of libpcpattn."""

    def __init__(self, func: str, code: int):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (func, strerror(code), code))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libpcpattn.so is not built; run `python -m context_causal_gqa_amd.build` "
            "or __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_float, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    L.pcp_strerror.argtypes = [c_int]
    L.pcp_strerror.restype = ctypes.c_char_p
    L.pcp_plan_rows.argtypes = [c_int, vp, vp, c_int, c_int, c_int, c_int, c_int, vp, c_int]
    L.pcp_plan_rows.restype = c_int
    L.pcp_plan_rows_resplit.argtypes = [c_int, vp, vp, c_int, c_int, c_int, c_int, c_int, vp,
                                        c_int]
    L.pcp_plan_rows_resplit.restype = c_int
    L.pcp_slot_mapping.argtypes = [c_int, vp, vp, vp, c_int, c_int, c_int, c_int, vp, c_int]
    L.pcp_slot_mapping.restype = c_int
    L.pcp_kv_cache_write.argtypes = [vp, vp, vp, c_int, c_int, c_int, vp, vp, c_int, c_int, vp]
    L.pcp_kv_cache_write.restype = c_int
    L.pcp_attn_prefill.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                   c_int, c_float, vp, vp, vp, c_int, vp]
    L.pcp_attn_prefill.restype = c_int
    L.pcp_attn_context_paged.argtypes = [vp, vp, vp, c_int, c_int, vp, c_int, c_int, vp, c_int,
                                         c_int, c_int, c_int, c_int, c_int, c_float, vp, vp, vp,
                                         c_int, vp, c_int, vp]
    L.pcp_attn_context_paged.restype = c_int
    L.pcp_attn_rank_share.argtypes = [vp, vp, vp, c_int, vp, vp, c_int, c_int, vp, c_int, c_int,
                                      vp, c_int, c_int, c_int, c_int, c_int, c_int, c_float, vp,
                                      vp, vp, c_int, vp, c_int, vp]
    L.pcp_attn_rank_share.restype = c_int
    L.pcp_attn_rank_share_noalloc.argtypes = [vp, vp, vp, c_int, vp, vp, c_int, c_int, vp,
                                              c_int, c_int, vp, c_int, c_int, c_int, c_int,
                                              c_int, c_int, c_float, vp, vp, c_int, vp, c_int, vp]
    L.pcp_attn_rank_share_noalloc.restype = c_int
    L.pcp_attn_prefill_fp8.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                       c_int, c_int, c_float, vp, vp, vp, vp, vp, vp, c_int, vp]
    L.pcp_attn_prefill_fp8.restype = c_int
    L.pcp_attn_context_paged_fp8.argtypes = [vp, vp, vp, c_int, c_int, vp, c_int, c_int, vp,
                                             c_int, c_int, c_int, c_int, c_int, c_int, c_float,
                                             vp, vp, vp, vp, vp, vp, c_int, vp, c_int, vp]
    L.pcp_attn_context_paged_fp8.restype = c_int
    L.pcp_attn_rank_share_fp8.argtypes = [vp, vp, vp, c_int, vp, vp, c_int, c_int, vp, c_int,
                                          c_int, vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                          c_float, vp, vp, vp, vp, vp, vp, c_int, vp, c_int, vp]
    L.pcp_attn_rank_share_fp8.restype = c_int
    L.pcp_kv_cache_write_fp8.argtypes = [vp, vp, vp, c_int, c_int, c_int, vp, vp, c_int, c_int,
                                         vp]
    L.pcp_kv_cache_write_fp8.restype = c_int
    L.pcp_attn_schedule.argtypes = [c_int, vp, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                    vp, c_int]
    L.pcp_attn_schedule.restype = c_int
    L.pcp_choose_decode_splits.argtypes = [vp, c_int, c_int, c_int]
    L.pcp_choose_decode_splits.restype = c_int
    L.pcp_context_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    L.pcp_context_workspace_bytes.restype = ctypes.c_size_t
    L.lse_merge.argtypes = [c_int, vp, vp, c_int, c_int, c_int, vp, vp, vp]
    L.lse_merge.restype = c_int
    _lib = L
    return L


def strerror(code: int) -> str:
    return lib().pcp_strerror(int(code)).decode()


def _check(func: str, rc: int) -> int:
    if rc < 0:
        raise PcpError(func, rc)
    return rc


# ---------------------------------------------------------------- plan


def _plan(func: str, cu_seqlens_new, ctx_lens, pcp_size, pcp_rank, dcp_size, dcp_rank,
          block_size) -> np.ndarray:
    cu = np.ascontiguousarray(cu_seqlens_new, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    b = len(cu) - 1
    if b < 0 or len(ctx) != b:
        raise ValueError("cu_seqlens_new must have len(ctx_lens) + 1 entries")
    cap = 2 * b
    while True:
        rows = np.zeros((max(cap, 1), len(ROW_FIELDS)), dtype=np.int32)
        n = _check(func, getattr(lib(), func)(
            b, cu.ctypes.data, ctx.ctypes.data, pcp_size, pcp_rank, dcp_size, dcp_rank,
            block_size, rows.ctypes.data, cap))
        if n <= cap:
            return rows[:n].copy()
        cap = n


def pcp_plan_rows(cu_seqlens_new: Sequence[int], ctx_lens: Sequence[int], pcp_size: int,
                  pcp_rank: int, dcp_size: int = 1, dcp_rank: int = 0,
                  block_size: int = 16) -> np.ndarray:
    """This rank's row plan (host), int32 [R, 9] with columns ROW_FIELDS."""
    return _plan("pcp_plan_rows", cu_seqlens_new, ctx_lens, pcp_size, pcp_rank, dcp_size,
                 dcp_rank, block_size)


def pcp_plan_rows_resplit(cu_seqlens_new: Sequence[int], ctx_lens: Sequence[int],
                          pcp_size: int, pcp_rank: int, dcp_size: int = 1, dcp_rank: int = 0,
                          block_size: int = 16) -> np.ndarray:
    """Row plan of the re-split path (host): context [0, pos_start) from the
    cache, the row's own tokens as new-token keys (k_start = q_start)."""
    return _plan("pcp_plan_rows_resplit", cu_seqlens_new, ctx_lens, pcp_size, pcp_rank,
                 dcp_size, dcp_rank, block_size)


def pcp_slot_mapping(cu_seqlens_new: Sequence[int], ctx_lens: Sequence[int],
                     block_table: np.ndarray, dcp_size: int, dcp_rank: int,
                     block_size: int) -> np.ndarray:
    """Cache slot (int64) of every new token this DCP rank writes, -1 elsewhere.
    ``block_table`` is host int32 [num_reqs, max_blocks], all logical blocks."""
    cu = np.ascontiguousarray(cu_seqlens_new, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    b = len(cu) - 1
    if b < 0 or len(ctx) != b or (b > 0 and (bt.ndim != 2 or bt.shape[0] != b)):
        raise ValueError("cu_seqlens_new / ctx_lens / block_table shapes do not match")
    n = int(cu[-1] - cu[0]) if b > 0 else 0
    slots = np.zeros(max(n, 1), dtype=np.int64)
    m = _check("pcp_slot_mapping", lib().pcp_slot_mapping(
        b, cu.ctypes.data, ctx.ctypes.data, bt.ctypes.data if b else None,
        bt.shape[1] if b else 0, dcp_size, dcp_rank, block_size, slots.ctypes.data, n))
    assert m == n
    return slots[:n]


def pcp_kv_cache_write(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Write the tokens' K/V ([T, Hkv, d] bf16, GPU) to their slots of the paged
    cache ([blocks, block_size, Hkv, d]); negative slots are skipped."""
    torch = _torch()
    _need(k, "k", torch.bfloat16, 3)
    dev = k.device
    _need(v, "v", torch.bfloat16, 3, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    t, hkv, d = k.shape
    nb, bs, hkv_c, dc = k_cache.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or hkv_c != hkv or dc != d or slot_mapping.numel() != t:
        raise ValueError("k/v/slot_mapping/cache shapes do not match")
    _check("pcp_kv_cache_write", lib().pcp_kv_cache_write(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), t, hkv, d, k_cache.data_ptr(),
        v_cache.data_ptr(), nb, bs, _stream_ptr(k, stream)))


def pcp_kv_cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """``pcp_kv_cache_write`` for E4M3 codes (uint8 or float8_e4m3fn)."""
    torch = _torch()
    _need_codes(k, "k", 3, None)
    dev = k.device
    _need_codes(v, "v", 3, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    _need_codes(k_cache, "k_cache", 4, dev)
    _need_codes(v_cache, "v_cache", 4, dev)
    t, hkv, d = k.shape
    nb, bs, hkv_c, dc = k_cache.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or hkv_c != hkv or dc != d or slot_mapping.numel() != t:
        raise ValueError("k/v/slot_mapping/cache shapes do not match")
    _check("pcp_kv_cache_write_fp8", lib().pcp_kv_cache_write_fp8(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), t, hkv, d, k_cache.data_ptr(),
        v_cache.data_ptr(), nb, bs, _stream_ptr(k, stream)))


PASS_NEW_TOKENS, PASS_CONTEXT, PASS_FUSED = 0, 1, 2


def pcp_attn_schedule(pass_: int, rows_host: np.ndarray, max_q_len: int, num_q_heads: int,
                      num_kv_heads: int, head_dim: int, decode_splits: int = 1,
                      kv_elem_bytes: int = 2) -> np.ndarray:
    """Launch order (int32, -1 padded) of one attention call's work units:
    longest first per XCD, neighbouring query tiles of a row kept together
    (or, past the Infinity Cache, each (request, KV head) group on one XCD).
    ``pass_`` is PASS_NEW_TOKENS, PASS_CONTEXT or PASS_FUSED; ``kv_elem_bytes``
    is 2 for bf16 K/V and 1 for E4M3."""
    r = np.ascontiguousarray(np.asarray(rows_host, dtype=np.int32).reshape(-1, len(ROW_FIELDS)))
    args = (int(pass_), r.ctypes.data, len(r), int(max_q_len), int(num_q_heads),
            int(num_kv_heads), int(head_dim), int(decode_splits), int(kv_elem_bytes))
    n = _check("pcp_attn_schedule", lib().pcp_attn_schedule(*args, None, 0))
    order = np.zeros(max(n, 1), dtype=np.int32)
    m = _check("pcp_attn_schedule", lib().pcp_attn_schedule(*args, order.ctypes.data, n))
    assert m == n
    return order[:n]


def _order_args(unit_order, dev):
    torch = _torch()
    if unit_order is None:
        return None, 0
    if unit_order.dtype != torch.int32 or unit_order.dim() != 1 or not unit_order.is_cuda \
            or unit_order.device != dev or not unit_order.is_contiguous():
        raise ValueError("unit_order must be a contiguous 1-d int32 tensor on %s" % dev)
    return unit_order.data_ptr(), unit_order.numel()


def plan_max_q_len(rows: np.ndarray) -> int:
    return int(rows[:, 3].max()) if len(rows) else 0


def plan_total_q(rows: np.ndarray) -> int:
    return int((rows[:, 2] + rows[:, 3]).max()) if len(rows) else 0


# ---------------------------------------------------------------- device calls


def _torch():
    import torch

    return torch


def _stream_ptr(t, stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream)


def _need(t, name: str, dtype, ndim: int, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _rows_shape(rows):
    """A plan tensor must be [R, 9] (the pcp_row_t fields): checked before
    anything else, so a wrong width never reaches a kernel that reads rows
    with the struct's stride."""
    shape = tuple(getattr(rows, "shape", ()))
    if len(shape) != 2 or shape[1] != len(ROW_FIELDS):
        raise ValueError("rows must be [R, %d] (pcp_row_t fields), got shape %s"
                         % (len(ROW_FIELDS), shape))


def _check_rows_host(rows_host: Optional[np.ndarray], num_rows: int, total_q: int,
                     total_k: Optional[int], max_q_len: int, num_reqs: Optional[int] = None,
                     max_ctx: Optional[int] = None):
    """Host-side bounds check of a plan before any launch."""
    if rows_host is None:
        return
    r = np.asarray(rows_host, dtype=np.int64).reshape(-1, len(ROW_FIELDS))
    if len(r) != num_rows:
        raise ValueError("rows_host has %d rows, device rows %d" % (len(r), num_rows))
    if not len(r):
        return
    qs, ql = r[:, 2], r[:, 3]
    if (qs < 0).any() or (ql < 0).any() or (qs + ql > total_q).any():
        raise ValueError("plan rows exceed the query buffer")
    if (ql > max_q_len).any():
        raise ValueError("max_q_len is smaller than a row's q_len")
    if total_k is not None:
        ks, kl = r[:, 5], r[:, 6]
        if (ks < 0).any() or (kl < 0).any() or (ks + kl > total_k).any():
            raise ValueError("plan rows exceed the K/V buffers")
    if num_reqs is not None and ((r[:, 0] < 0).any() or (r[:, 0] >= num_reqs).any()):
        raise ValueError("plan rows name a request outside the block table")
    if max_ctx is not None and ((r[:, 8] < 0).any() or (r[:, 8] > max_ctx).any()):
        raise ValueError("a row's ctx_len_local exceeds its block table")


def _workspace_ptr(workspace, dev, num_rows: int, hq: int, d: int, decode_splits: int):
    """Device pointer of the decode-split workspace (None for one split)."""
    torch = _torch()
    if decode_splits <= 1:
        return None
    if workspace is None:
        raise ValueError("decode_splits > 1 needs a workspace")
    if workspace.dtype != torch.float32 or not workspace.is_cuda or \
            workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 tensor on %s" % dev)
    need = pcp_context_workspace_bytes(num_rows, hq, d, decode_splits)
    if workspace.numel() * 4 < need:
        raise ValueError("workspace holds %d bytes, the call needs %d"
                         % (workspace.numel() * 4, need))
    return workspace.data_ptr()


def _need_codes(t, name: str, ndim: int, device):
    """An E4M3 tensor: uint8 codes or torch.float8_e4m3fn, 16-byte aligned."""
    torch = _torch()
    dt = t.dtype if isinstance(t, torch.Tensor) else None
    _need(t, name, dt if dt in (torch.uint8, torch.float8_e4m3fn) else torch.uint8, ndim, device)
    if t.data_ptr() % 16:
        raise ValueError("%s must be 16-byte aligned" % name)


def _need_descales(descales, num_kv_heads: int, device) -> int:
    """(q, k, v) descale tables, float32 [num_reqs, num_kv_heads]; returns num_reqs."""
    torch = _torch()
    shape = None
    for t, nm in zip(descales, ("q_descale", "k_descale", "v_descale")):
        _need(t, nm, torch.float32, 2, device)
        if t.shape[1] != num_kv_heads or (shape is not None and tuple(t.shape) != shape):
            raise ValueError("descales must all be [num_reqs, %d], got %s"
                             % (num_kv_heads, tuple(t.shape)))
        shape = tuple(t.shape)
    return shape[0]


def pcp_attn_prefill(q, k, v, rows, out, lse, softmax_scale: float, max_q_len: int,
                     rows_host: Optional[np.ndarray] = None, stream=None,
                     unit_order=None) -> None:
    """New-token pass (end-aligned causal) into ``out`` / ``lse``. ``unit_order``
    is an optional GPU int32 tensor from ``pcp_attn_schedule(PASS_NEW_TOKENS, ...)``."""
    torch = _torch()
    _rows_shape(rows)
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(k, "k", torch.bfloat16, 3, dev)
    _need(v, "v", torch.bfloat16, 3, dev)
    _need(rows, "rows", torch.int32, 2, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    total_q, hq, d = q.shape
    total_k, hkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or dk != d:
        raise ValueError("k/v shapes %s %s do not match q %s" % (k.shape, v.shape, q.shape))
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (hq, total_q):
        raise ValueError("out/lse shapes do not match q")
    _check_rows_host(rows_host, rows.shape[0], total_q, total_k, max_q_len)
    ord_ptr, ord_n = _order_args(unit_order, dev)
    _check("pcp_attn_prefill", lib().pcp_attn_prefill(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), rows.data_ptr(), rows.shape[0], total_q,
        total_k, int(max_q_len), hq, hkv, d, float(softmax_scale), out.data_ptr(),
        lse.data_ptr(), ord_ptr, ord_n, _stream_ptr(q, stream)))


def pcp_context_workspace_bytes(num_rows: int, num_q_heads: int, head_dim: int,
                                decode_splits: int) -> int:
    """Bytes of float32 workspace ``pcp_attn_context_paged`` needs (0 for one split)."""
    return int(lib().pcp_context_workspace_bytes(int(num_rows), int(num_q_heads),
                                                 int(head_dim), int(decode_splits)))


def pcp_choose_decode_splits(rows_host: np.ndarray, num_kv_heads: int,
                             fused: bool = False) -> int:
    """Key-range splits for the decode rows (one query, no new-token keys) of
    a context pass (``fused``: of a pcp_attn_rank_share launch), chosen by
    the library from the host plan (see ``pcp_choose_decode_splits`` in
    include/pcp_attn.h). 1 when the plan has no decode row or the launch
    already fills the GPU."""
    r = np.ascontiguousarray(np.asarray(rows_host, dtype=np.int32).reshape(-1, len(ROW_FIELDS)))
    return _check("pcp_choose_decode_splits", lib().pcp_choose_decode_splits(
        r.ctypes.data if len(r) else None, len(r), int(num_kv_heads), 1 if fused else 0))


def pcp_attn_context_paged(q, k_cache, v_cache, block_tables, rows, out, lse,
                           softmax_scale: float, max_q_len: int,
                           rows_host: Optional[np.ndarray] = None, stream=None,
                           workspace=None, decode_splits: int = 1, unit_order=None) -> None:
    """Context pass over this DCP rank's paged cache shard into ``out`` / ``lse``.

    With ``decode_splits`` > 1, one-query rows are split over their key range;
    ``workspace`` is then a float32 GPU tensor of at least
    ``pcp_context_workspace_bytes(...)`` bytes, not shared with a call still
    in flight. ``unit_order`` as in ``pcp_attn_prefill`` (``PASS_CONTEXT``)."""
    torch = _torch()
    _rows_shape(rows)
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(rows, "rows", torch.int32, 2, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    total_q, hq, d = q.shape
    num_blocks, block_size, hkv, dk = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or dk != d:
        raise ValueError("cache shapes do not match q")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (hq, total_q):
        raise ValueError("out/lse shapes do not match q")
    num_reqs, max_blocks = block_tables.shape
    _check_rows_host(rows_host, rows.shape[0], total_q, None, max_q_len, num_reqs,
                     max_blocks * block_size)
    decode_splits = int(decode_splits)
    ws_ptr = _workspace_ptr(workspace, dev, rows.shape[0], hq, d, decode_splits)
    ord_ptr, ord_n = _order_args(unit_order, dev)
    _check("pcp_attn_context_paged", lib().pcp_attn_context_paged(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), num_blocks, block_size,
        block_tables.data_ptr(), num_reqs, max_blocks, rows.data_ptr(), rows.shape[0], total_q,
        int(max_q_len), hq, hkv, d, float(softmax_scale), out.data_ptr(), lse.data_ptr(),
        ws_ptr, decode_splits, ord_ptr, ord_n, _stream_ptr(q, stream)))


def _rank_share_args(q, k, v, k_cache, v_cache, block_tables, rows, out, lse, softmax_scale,
                     max_q_len, rows_host, stream, decode_splits, unit_order):
    """Checks the bf16 fused call's tensors; returns its C arguments before
    and after the workspace pointer, and the device."""
    torch = _torch()
    _rows_shape(rows)
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    for t, nm, nd in ((k, "k", 3), (v, "v", 3), (k_cache, "k_cache", 4), (v_cache, "v_cache", 4),
                      (out, "out", 3)):
        _need(t, nm, torch.bfloat16, nd, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(rows, "rows", torch.int32, 2, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    total_q, hq, d = q.shape
    total_k, hkv, dk = k.shape
    num_blocks, block_size, hkv_c, dc = k_cache.shape
    if tuple(v.shape) != tuple(k.shape) or dk != d:
        raise ValueError("k/v shapes %s %s do not match q %s" % (k.shape, v.shape, q.shape))
    if tuple(v_cache.shape) != tuple(k_cache.shape) or dc != d or hkv_c != hkv:
        raise ValueError("cache shapes do not match q / k")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (hq, total_q):
        raise ValueError("out/lse shapes do not match q")
    num_reqs, max_blocks = block_tables.shape
    _check_rows_host(rows_host, rows.shape[0], total_q, total_k, max_q_len, num_reqs,
                     max_blocks * block_size)
    ord_ptr, ord_n = _order_args(unit_order, dev)
    before = (q.data_ptr(), k.data_ptr(), v.data_ptr(), total_k, k_cache.data_ptr(),
              v_cache.data_ptr(), num_blocks, block_size, block_tables.data_ptr(), num_reqs,
              max_blocks, rows.data_ptr(), rows.shape[0], total_q, int(max_q_len), hq, hkv, d,
              float(softmax_scale), out.data_ptr(), lse.data_ptr())
    after = (int(decode_splits), ord_ptr, ord_n, _stream_ptr(q, stream))
    return before, after, dev


def pcp_attn_rank_share(q, k, v, k_cache, v_cache, block_tables, rows, out, lse,
                        softmax_scale: float, max_q_len: int,
                        rows_host: Optional[np.ndarray] = None, stream=None, workspace=None,
                        decode_splits: int = 1, unit_order=None) -> None:
    """The whole rank share in one launch: context tiles, then new-token
    tiles, one softmax, the merged result into ``out`` / ``lse``. Arguments
    as in ``pcp_attn_prefill`` and ``pcp_attn_context_paged``;
    ``unit_order`` from ``pcp_attn_schedule(PASS_FUSED, ...)``."""
    before, after, dev = _rank_share_args(q, k, v, k_cache, v_cache, block_tables, rows, out,
                                          lse, softmax_scale, max_q_len, rows_host, stream,
                                          decode_splits, unit_order)
    ws_ptr = _workspace_ptr(workspace, dev, rows.shape[0], q.shape[1], q.shape[2],
                            int(decode_splits))
    _check("pcp_attn_rank_share", lib().pcp_attn_rank_share(*before, ws_ptr, *after))


def pcp_attn_rank_share_noalloc(q, k, v, k_cache, v_cache, block_tables, rows, out, lse,
                                softmax_scale: float, max_q_len: int,
                                rows_host: Optional[np.ndarray] = None, stream=None,
                                decode_splits: int = 1, unit_order=None) -> None:
    """``pcp_attn_rank_share`` without a workspace, for callers that cannot
    allocate: the split-decode partials go to the library's fixed per-device
    scratch array of NOALLOC_SCRATCH_BYTES (PcpError PCP_ESCRATCH beyond
    it). Calls that overlap on one device share that array and race."""
    before, after, _ = _rank_share_args(q, k, v, k_cache, v_cache, block_tables, rows, out, lse,
                                        softmax_scale, max_q_len, rows_host, stream,
                                        decode_splits, unit_order)
    _check("pcp_attn_rank_share_noalloc", lib().pcp_attn_rank_share_noalloc(*before, *after))


def pcp_attn_prefill_fp8(q, k, v, rows, out, lse, softmax_scale: float, max_q_len: int,
                         q_descale, k_descale, v_descale,
                         rows_host: Optional[np.ndarray] = None, stream=None,
                         unit_order=None) -> None:
    """``pcp_attn_prefill`` with E4M3 q/k/v (uint8 or float8_e4m3fn) and float32
    descales [num_reqs, Hkv] indexed by (request, KV head)."""
    torch = _torch()
    _rows_shape(rows)
    _need_codes(q, "q", 3, None)
    dev = q.device
    _need_codes(k, "k", 3, dev)
    _need_codes(v, "v", 3, dev)
    _need(rows, "rows", torch.int32, 2, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    total_q, hq, d = q.shape
    total_k, hkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or dk != d:
        raise ValueError("k/v shapes %s %s do not match q %s" % (k.shape, v.shape, q.shape))
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (hq, total_q):
        raise ValueError("out/lse shapes do not match q")
    num_reqs = _need_descales((q_descale, k_descale, v_descale), hkv, dev)
    _check_rows_host(rows_host, rows.shape[0], total_q, total_k, max_q_len, num_reqs)
    ord_ptr, ord_n = _order_args(unit_order, dev)
    _check("pcp_attn_prefill_fp8", lib().pcp_attn_prefill_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), rows.data_ptr(), rows.shape[0], total_q,
        total_k, int(max_q_len), num_reqs, hq, hkv, d, float(softmax_scale),
        q_descale.data_ptr(), k_descale.data_ptr(), v_descale.data_ptr(), out.data_ptr(),
        lse.data_ptr(), ord_ptr, ord_n, _stream_ptr(q, stream)))


def pcp_attn_context_paged_fp8(q, k_cache, v_cache, block_tables, rows, out, lse,
                               softmax_scale: float, max_q_len: int, q_descale, k_descale,
                               v_descale, rows_host: Optional[np.ndarray] = None, stream=None,
                               workspace=None, decode_splits: int = 1, unit_order=None) -> None:
    """``pcp_attn_context_paged`` with E4M3 q and caches and descales as in
    ``pcp_attn_prefill_fp8``; the block table's rows are the descales' rows."""
    torch = _torch()
    _rows_shape(rows)
    _need_codes(q, "q", 3, None)
    dev = q.device
    _need_codes(k_cache, "k_cache", 4, dev)
    _need_codes(v_cache, "v_cache", 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(rows, "rows", torch.int32, 2, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    total_q, hq, d = q.shape
    num_blocks, block_size, hkv, dk = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or dk != d:
        raise ValueError("cache shapes do not match q")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (hq, total_q):
        raise ValueError("out/lse shapes do not match q")
    num_reqs, max_blocks = block_tables.shape
    if _need_descales((q_descale, k_descale, v_descale), hkv, dev) != num_reqs:
        raise ValueError("descales and block_tables disagree on the number of requests")
    _check_rows_host(rows_host, rows.shape[0], total_q, None, max_q_len, num_reqs,
                     max_blocks * block_size)
    decode_splits = int(decode_splits)
    ws_ptr = _workspace_ptr(workspace, dev, rows.shape[0], hq, d, decode_splits)
    ord_ptr, ord_n = _order_args(unit_order, dev)
    _check("pcp_attn_context_paged_fp8", lib().pcp_attn_context_paged_fp8(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), num_blocks, block_size,
        block_tables.data_ptr(), num_reqs, max_blocks, rows.data_ptr(), rows.shape[0], total_q,
        int(max_q_len), hq, hkv, d, float(softmax_scale), q_descale.data_ptr(),
        k_descale.data_ptr(), v_descale.data_ptr(), out.data_ptr(), lse.data_ptr(), ws_ptr,
        decode_splits, ord_ptr, ord_n, _stream_ptr(q, stream)))


def pcp_attn_rank_share_fp8(q, k, v, k_cache, v_cache, block_tables, rows, out, lse,
                            softmax_scale: float, max_q_len: int, q_descale, k_descale,
                            v_descale, rows_host: Optional[np.ndarray] = None, stream=None,
                            workspace=None, decode_splits: int = 1, unit_order=None) -> None:
    """``pcp_attn_rank_share`` with E4M3 q/k/v/caches and descales as in
    ``pcp_attn_prefill_fp8``."""
    torch = _torch()
    _rows_shape(rows)
    _need_codes(q, "q", 3, None)
    dev = q.device
    for t, nm, nd in ((k, "k", 3), (v, "v", 3), (k_cache, "k_cache", 4),
                      (v_cache, "v_cache", 4)):
        _need_codes(t, nm, nd, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(rows, "rows", torch.int32, 2, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    total_q, hq, d = q.shape
    total_k, hkv, dk = k.shape
    num_blocks, block_size, hkv_c, dc = k_cache.shape
    if tuple(v.shape) != tuple(k.shape) or dk != d:
        raise ValueError("k/v shapes %s %s do not match q %s" % (k.shape, v.shape, q.shape))
    if tuple(v_cache.shape) != tuple(k_cache.shape) or dc != d or hkv_c != hkv:
        raise ValueError("cache shapes do not match q / k")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (hq, total_q):
        raise ValueError("out/lse shapes do not match q")
    num_reqs, max_blocks = block_tables.shape
    if _need_descales((q_descale, k_descale, v_descale), hkv, dev) != num_reqs:
        raise ValueError("descales and block_tables disagree on the number of requests")
    _check_rows_host(rows_host, rows.shape[0], total_q, total_k, max_q_len, num_reqs,
                     max_blocks * block_size)
    decode_splits = int(decode_splits)
    ws_ptr = _workspace_ptr(workspace, dev, rows.shape[0], hq, d, decode_splits)
    ord_ptr, ord_n = _order_args(unit_order, dev)
    _check("pcp_attn_rank_share_fp8", lib().pcp_attn_rank_share_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), total_k, k_cache.data_ptr(),
        v_cache.data_ptr(), num_blocks, block_size, block_tables.data_ptr(), num_reqs,
        max_blocks, rows.data_ptr(), rows.shape[0], total_q, int(max_q_len), hq, hkv, d,
        float(softmax_scale), q_descale.data_ptr(), k_descale.data_ptr(), v_descale.data_ptr(),
        out.data_ptr(), lse.data_ptr(), ws_ptr, decode_splits, ord_ptr, ord_n,
        _stream_ptr(q, stream)))


def lse_merge(outs: Sequence, lses: Sequence, out, lse_out, stream=None) -> None:
    """Merge partial (out, lse) pairs over disjoint key sets into ``out`` / ``lse_out``
    (which may alias outs[0] / lses[0])."""
    torch = _torch()
    if len(outs) != len(lses) or not outs:
        raise ValueError("need one lse per partial output, at least one")
    _need(out, "out", torch.bfloat16, 3)
    dev = out.device
    _need(lse_out, "lse_out", torch.float32, 2, dev)
    total_q, hq, d = out.shape
    for i, (o, l) in enumerate(zip(outs, lses)):
        _need(o, "outs[%d]" % i, torch.bfloat16, 3, dev)
        _need(l, "lses[%d]" % i, torch.float32, 2, dev)
        if tuple(o.shape) != tuple(out.shape) or tuple(l.shape) != (hq, total_q):
            raise ValueError("partial %d has the wrong shape" % i)
    if tuple(lse_out.shape) != (hq, total_q):
        raise ValueError("lse_out shape")
    k = len(outs)
    optr = (ctypes.c_void_p * k)(*[o.data_ptr() for o in outs])
    lptr = (ctypes.c_void_p * k)(*[l.data_ptr() for l in lses])
    _check("lse_merge", lib().lse_merge(
        k, ctypes.cast(optr, ctypes.c_void_p), ctypes.cast(lptr, ctypes.c_void_p), total_q, hq, d,
        out.data_ptr(), lse_out.data_ptr(), _stream_ptr(out, stream)))
