"""Grouped shared-prefix attention for MI355X (gfx950): Python binding of libpg_attn.

A thin ctypes layer over the C ABI declared in include/pg_attn.h.  It only
marshals arguments: every step of the computation runs in the HIP kernels of
libpg_attn.so.  PyTorch supplies device memory and the current stream.  If
the library is not built, importing works but every call raises
LibraryNotBuilt; there is no fallback.

Functions keep the C names:
  pg_pack(groups, num_q_heads, num_kv_heads, head_dim, device) -> PackedBatch
  pg_pack_host(groups, num_q_heads, num_kv_heads, head_dim)  -> dict of numpy arrays
  pg_attn_fwd(batch, q, k, v, softmax_scale=None) -> (o, lse)
  pg_attn_bwd(batch, q, k, v, o, lse, dout, softmax_scale=None) -> (dq, dk, dv)
  pg_rope(batch, x, theta=10000.0, inverse=False)  (in place)
plus GroupedAttention, a torch.autograd.Function over pg_attn_fwd/pg_attn_bwd.

`groups` is a sequence of (prefix_len, [resp_len_1, ..., resp_len_G]); the
packed row order is [P; R_1; ...; R_G] per group, groups concatenated.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpg_attn.so")

PG_OK, PG_ERR_INVALID_ARG, PG_ERR_UNSUPPORTED, PG_ERR_WORKSPACE, PG_ERR_HIP = range(5)
PG_F32, PG_BF16 = 0, 1
PG_TILE_Q = 128
PG_TILE_KV = 128

EXPORTED = ("pg_pack_buffer_size", "pg_pack", "pg_pack_host", "pg_attn_fwd",
            "pg_attn_bwd_workspace_size", "pg_attn_bwd", "pg_attn_bwd_noalloc", "pg_rope",
            "pg_pack_rows",
            "pg_unpack_rows", "pg_logprob_workspace_size", "pg_logprob_fwd", "pg_grpo_loss",
            "pg_logprob_bwd", "pg_kernel_timing",
            "pg_kernel_times", "pg_kernel_name", "pg_last_error", "pg_version")
KERNELS = ("fwd", "bwd_pre", "bwd_dkdv", "bwd_dq", "rope", "rows", "head_fwd", "head_bwd",
           "grpo_loss")


class LibraryNotBuilt(RuntimeError):
    pass


class PgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pg status {status}: {msg}")
        self.status = status


_i32p = ctypes.POINTER(ctypes.c_int32)


class PgGroups(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("prefix_len", _i32p), ("num_resp", _i32p),
                ("resp_len", _i32p), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class PgDesc(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("num_resp", ctypes.c_int32),
                ("total_rows", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_q_tiles", ctypes.c_int32), ("num_kv_tiles", ctypes.c_int32),
                ("num_kv_items", ctypes.c_int32), ("num_kv_sums", ctypes.c_int32),
                ("num_kv_parts", ctypes.c_int32), ("total_prefix_rows", ctypes.c_int32),
                ("num_scored", ctypes.c_int32), ("max_walk_rows", ctypes.c_int32),
                ("pairs", ctypes.c_int64), ("baseline_pairs", ctypes.c_int64),
                ("row_lo", _i32p), ("row_hi", _i32p), ("q_tiles", _i32p), ("kv_tiles", _i32p),
                ("kv_items", _i32p), ("kv_sums", _i32p),
                ("group_start", _i32p), ("prefix_end", _i32p), ("prefix_before", _i32p),
                ("resp_start", _i32p),
                ("resp_len", _i32p), ("resp_group", _i32p), ("scored_row", _i32p),
                ("scored_pred", _i32p), ("scored_resp", _i32p), ("pred_start", _i32p),
                ("pred_list", _i32p), ("buf_bytes", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpg_attn.so; raises LibraryNotBuilt if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(
            f"{LIB_PATH} is missing: build it with `python -m shared_prefix_grouped_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    G, Dp = ctypes.POINTER(PgGroups), ctypes.POINTER(PgDesc)
    L.pg_pack_buffer_size.argtypes = [G]
    L.pg_pack_buffer_size.restype = sz
    L.pg_pack.argtypes = [G, vp, sz, vp, Dp, vp]
    L.pg_pack.restype = ctypes.c_int
    L.pg_pack_host.argtypes = [G, vp, sz, vp, Dp]
    L.pg_pack_host.restype = ctypes.c_int
    L.pg_attn_fwd.argtypes = [Dp, ctypes.c_int, f32, vp, vp, vp, vp, vp, vp]
    L.pg_attn_fwd.restype = ctypes.c_int
    L.pg_attn_bwd_workspace_size.argtypes = [Dp, ctypes.c_int]
    L.pg_attn_bwd_workspace_size.restype = sz
    L.pg_attn_bwd.argtypes = [Dp, ctypes.c_int, f32] + [vp] * 10 + [sz, vp]
    L.pg_attn_bwd.restype = ctypes.c_int
    L.pg_attn_bwd_noalloc.argtypes = [Dp, ctypes.c_int, f32] + [vp] * 9 + [vp]
    L.pg_attn_bwd_noalloc.restype = ctypes.c_int
    L.pg_rope.argtypes = [Dp, ctypes.c_int, vp, i32, i32, vp, f32, i32, vp]
    L.pg_rope.restype = ctypes.c_int
    L.pg_pack_rows.argtypes = [Dp, vp, vp, vp, sz, vp]
    L.pg_pack_rows.restype = ctypes.c_int
    L.pg_unpack_rows.argtypes = [Dp, vp, vp, vp, sz, vp]
    L.pg_unpack_rows.restype = ctypes.c_int
    L.pg_logprob_workspace_size.argtypes = [Dp, i32, i32]
    L.pg_logprob_workspace_size.restype = sz
    L.pg_logprob_fwd.argtypes = [Dp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    L.pg_logprob_fwd.restype = ctypes.c_int
    L.pg_grpo_loss.argtypes = [Dp, vp, vp, vp, vp, vp]
    L.pg_grpo_loss.restype = ctypes.c_int
    L.pg_logprob_bwd.argtypes = [Dp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.pg_logprob_bwd.restype = ctypes.c_int
    L.pg_kernel_timing.argtypes = [i32]
    L.pg_kernel_timing.restype = ctypes.c_int
    L.pg_kernel_times.argtypes = [i32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    L.pg_kernel_times.restype = ctypes.c_int
    L.pg_kernel_name.argtypes = [i32]
    L.pg_kernel_name.restype = ctypes.c_char_p
    L.pg_last_error.argtypes = []
    L.pg_last_error.restype = ctypes.c_char_p
    L.pg_version.argtypes = []
    L.pg_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int) -> None:
    if status != PG_OK:
        raise PgError(status, lib().pg_last_error().decode())


def _groups_struct(groups, hq, hkv, d):
    prefix = [int(p) for p, _ in groups]
    nresp = [len(rs) for _, rs in groups]
    rlen = [int(r) for _, rs in groups for r in rs]
    # one int32 array holding the three lists (values outside int32 raise);
    # it must outlive the struct's use
    keep = np.array(prefix + nresp + rlen, dtype=np.int32)
    base = keep.ctypes.data
    ng, nr = len(prefix), len(rlen)
    ptr = lambda off, n: ctypes.cast(base + 4 * off, _i32p) if n else _i32p()
    g = PgGroups(ng, ptr(0, ng), ptr(ng, ng), ptr(2 * ng, nr), int(hq), int(hkv), int(d))
    return g, keep


def _torch():
    import torch
    return torch


def _stream_ptr(device) -> ctypes.c_void_p:
    """The current stream of `device` (what torch would launch on) as a raw handle.

    torch's own raw-stream query when it has one: the public current_stream()
    builds a Stream object per call, which costs more than the kernel launch
    for small batches."""
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    idx = device.index if device.index is not None else torch.cuda.current_device()
    return ctypes.c_void_p(raw(idx))


@dataclass
class PackedBatch:
    """A planned packed batch resident on one GPU (descriptor + position ids)."""
    desc: PgDesc
    buffer: object          # torch uint8 tensor holding the device arrays of desc
    pos_ids: object         # torch int32 [T]: baseline position ids
    groups: Tuple[Tuple[int, Tuple[int, ...]], ...]

    @property
    def total_rows(self) -> int:
        return self.desc.total_rows

    @property
    def pairs(self) -> int:
        return self.desc.pairs

    @property
    def baseline_pairs(self) -> int:
        return self.desc.baseline_pairs


def pg_pack(groups: Sequence, num_q_heads: int, num_kv_heads: int, head_dim: int,
            device="cuda") -> PackedBatch:
    torch = _torch()
    L = lib()
    g, keep = _groups_struct(groups, num_q_heads, num_kv_heads, head_dim)
    nbytes = L.pg_pack_buffer_size(ctypes.byref(g))
    if nbytes == 0:
        raise PgError(PG_ERR_INVALID_ARG, L.pg_last_error().decode())
    device = torch.device(device)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    T = sum(int(p) + sum(int(r) for r in rs) for p, rs in groups)
    pos = torch.empty(max(T, 1), dtype=torch.int32, device=device)
    desc = PgDesc()
    _check(L.pg_pack(ctypes.byref(g), ctypes.c_void_p(buf.data_ptr()), nbytes,
                     ctypes.c_void_p(pos.data_ptr()), ctypes.byref(desc), _stream_ptr(device)))
    del keep
    frozen = tuple((int(p), tuple(int(r) for r in rs)) for p, rs in groups)
    return PackedBatch(desc, buf, pos[:T], frozen)


def pg_pack_host(groups: Sequence, num_q_heads: int, num_kv_heads: int, head_dim: int) -> dict:
    """The plan pg_pack would upload, built in host memory (no GPU), as numpy arrays."""
    L = lib()
    g, keep = _groups_struct(groups, num_q_heads, num_kv_heads, head_dim)
    nbytes = L.pg_pack_buffer_size(ctypes.byref(g))
    if nbytes == 0:
        raise PgError(PG_ERR_INVALID_ARG, L.pg_last_error().decode())
    buf = np.zeros(nbytes // 4 + 4, dtype=np.int32)
    T = sum(int(p) + sum(int(r) for r in rs) for p, rs in groups)
    pos = np.zeros(max(T, 1), dtype=np.int32)
    d = PgDesc()
    _check(L.pg_pack_host(ctypes.byref(g), buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes,
                          pos.ctypes.data_as(ctypes.c_void_p), ctypes.byref(d)))
    base = buf.ctypes.data

    def arr(p, n, cols=1):
        if n == 0:
            return np.zeros((0, cols) if cols > 1 else 0, dtype=np.int32)
        off = (ctypes.cast(p, ctypes.c_void_p).value - base) // 4
        a = buf[off:off + n * cols].copy()
        return a.reshape(n, cols) if cols > 1 else a

    return {
        "total_rows": d.total_rows, "pairs": d.pairs, "baseline_pairs": d.baseline_pairs,
        "num_q_tiles": d.num_q_tiles, "num_kv_tiles": d.num_kv_tiles,
        "row_lo": arr(d.row_lo, T), "row_hi": arr(d.row_hi, T),
        "q_tiles": arr(d.q_tiles, d.num_q_tiles, 4), "kv_tiles": arr(d.kv_tiles, d.num_kv_tiles, 4),
        "kv_items": arr(d.kv_items, d.num_kv_items, 8), "kv_sums": arr(d.kv_sums, d.num_kv_sums, 4),
        "num_kv_parts": d.num_kv_parts, "max_walk_rows": d.max_walk_rows,
        "scored_row": arr(d.scored_row, d.num_scored), "scored_pred": arr(d.scored_pred, d.num_scored),
        "scored_resp": arr(d.scored_resp, d.num_scored), "pred_start": arr(d.pred_start, T + 1),
        "pred_list": arr(d.pred_list, d.num_scored),
        "group_start": arr(d.group_start, d.num_groups + 1), "prefix_end": arr(d.prefix_end, d.num_groups),
        "prefix_before": arr(d.prefix_before, d.num_groups + 1), "total_prefix_rows": d.total_prefix_rows,
        "resp_start": arr(d.resp_start, d.num_resp), "resp_len": arr(d.resp_len, d.num_resp),
        "resp_group": arr(d.resp_group, d.num_resp), "pos_ids": pos[:T].copy(),
        "buf_bytes": d.buf_bytes,
    }


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.bfloat16:
        return PG_BF16
    if t == torch.float32:
        return PG_F32
    raise PgError(PG_ERR_UNSUPPORTED, f"unsupported dtype {t}")


def _check_tensor(name, x, shape, dtype, device):
    if tuple(x.shape) != tuple(shape):
        raise PgError(PG_ERR_INVALID_ARG, f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
    if x.dtype != dtype:
        raise PgError(PG_ERR_INVALID_ARG, f"{name} has dtype {x.dtype}, expected {dtype}")
    if not x.is_contiguous():
        raise PgError(PG_ERR_INVALID_ARG, f"{name} must be contiguous")
    if x.device != device:
        raise PgError(PG_ERR_INVALID_ARG, f"{name} is on {x.device}, expected {device}")


def _vp(x):
    return ctypes.c_void_p(x.data_ptr())


def _scale(s) -> float:
    return 0.0 if s is None else float(s)


def pg_attn_fwd(batch: PackedBatch, q, k, v, softmax_scale: Optional[float] = None, out=None,
                lse=None, store_lse: bool = True):
    """O (and LSE unless store_lse is False: forward-only scoring, lse is None)."""
    torch = _torch()
    d = batch.desc
    T, hq, hkv, D = d.total_rows, d.num_q_heads, d.num_kv_heads, d.head_dim
    dev = q.device
    _check_tensor("q", q, (T, hq, D), q.dtype, dev)
    _check_tensor("k", k, (T, hkv, D), q.dtype, dev)
    _check_tensor("v", v, (T, hkv, D), q.dtype, dev)
    o = torch.empty_like(q) if out is None else out
    _check_tensor("o", o, (T, hq, D), q.dtype, dev)
    l = None
    if store_lse:
        l = torch.empty((hq, T), dtype=torch.float32, device=dev) if lse is None else lse
        _check_tensor("lse", l, (hq, T), torch.float32, dev)
    _check(lib().pg_attn_fwd(ctypes.byref(d), _dtype_code(q.dtype), _scale(softmax_scale),
                             _vp(q), _vp(k), _vp(v), _vp(o), _vp(l) if l is not None else None,
                             _stream_ptr(dev)))
    return o, l


def pg_attn_bwd(batch: PackedBatch, q, k, v, o, lse, dout, softmax_scale: Optional[float] = None,
                dq=None, dk=None, dv=None, workspace=None):
    torch = _torch()
    d = batch.desc
    T, hq, hkv, D = d.total_rows, d.num_q_heads, d.num_kv_heads, d.head_dim
    dev = q.device
    for name, x, shp in (("q", q, (T, hq, D)), ("k", k, (T, hkv, D)), ("v", v, (T, hkv, D)),
                         ("o", o, (T, hq, D)), ("dout", dout, (T, hq, D))):
        _check_tensor(name, x, shp, q.dtype, dev)
    _check_tensor("lse", lse, (hq, T), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    # the kernels write through raw pointers: caller-supplied outputs must be
    # exactly the shape, type and layout they assume
    for name, x, shp in (("dq", dq, (T, hq, D)), ("dk", dk, (T, hkv, D)), ("dv", dv, (T, hkv, D))):
        _check_tensor(name, x, shp, q.dtype, dev)
    code = _dtype_code(q.dtype)
    L = lib()
    ws_bytes = L.pg_attn_bwd_workspace_size(ctypes.byref(d), code)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif (workspace.device != dev or not workspace.is_contiguous()
          or workspace.numel() * workspace.element_size() < ws_bytes):
        raise PgError(PG_ERR_WORKSPACE, f"workspace must be a contiguous buffer of at least "
                                        f"{ws_bytes} bytes on {dev}")
    _check(L.pg_attn_bwd(ctypes.byref(d), code, _scale(softmax_scale), _vp(q), _vp(k), _vp(v),
                         _vp(o), _vp(lse), _vp(dout), _vp(dq), _vp(dk), _vp(dv), _vp(workspace),
                         workspace.numel() * workspace.element_size(), _stream_ptr(dev)))
    return dq, dk, dv


NOALLOC_SCRATCH_BYTES = 64 << 20  # PG_NOALLOC_SCRATCH_BYTES


def pg_attn_bwd_noalloc(batch: PackedBatch, q, k, v, o, lse, dout, dq, dk, dv,
                        softmax_scale: Optional[float] = None):
    """pg_attn_bwd into caller-allocated dq, dk, dv with the library's own
    fixed device scratch (no allocation inside the call)."""
    torch = _torch()
    d = batch.desc
    T, hq, hkv, D = d.total_rows, d.num_q_heads, d.num_kv_heads, d.head_dim
    dev = q.device
    for name, x, shp in (("q", q, (T, hq, D)), ("k", k, (T, hkv, D)), ("v", v, (T, hkv, D)),
                         ("o", o, (T, hq, D)), ("dout", dout, (T, hq, D)),
                         ("dq", dq, (T, hq, D)), ("dk", dk, (T, hkv, D)), ("dv", dv, (T, hkv, D))):
        _check_tensor(name, x, shp, q.dtype, dev)
    _check_tensor("lse", lse, (hq, T), torch.float32, dev)
    _check(lib().pg_attn_bwd_noalloc(ctypes.byref(d), _dtype_code(q.dtype), _scale(softmax_scale),
                                     _vp(q), _vp(k), _vp(v), _vp(o), _vp(lse), _vp(dout), _vp(dq),
                                     _vp(dk), _vp(dv), _stream_ptr(dev)))
    return dq, dk, dv


def pg_rope(batch: PackedBatch, x, theta: float = 10000.0, inverse: bool = False):
    d = batch.desc
    if x.dim() != 3 or x.shape[0] != d.total_rows or not x.is_contiguous():
        raise PgError(PG_ERR_INVALID_ARG, "x must be contiguous [T, heads, head_dim]")
    _check(lib().pg_rope(ctypes.byref(d), _dtype_code(x.dtype), _vp(x), int(x.shape[1]),
                         int(x.shape[2]), _vp(batch.pos_ids), float(theta), int(bool(inverse)),
                         _stream_ptr(x.device)))
    return x


def _rows_check(x, rows: int, tail, dtype, name: str) -> None:
    if x.dim() < 1 or x.shape[0] != rows or tuple(x.shape[1:]) != tuple(tail) or \
            x.dtype != dtype or not x.is_contiguous():
        raise PgError(PG_ERR_INVALID_ARG, f"{name} must be contiguous [{rows}, *{tuple(tail)}] {dtype}")


def pg_pack_rows(batch: PackedBatch, prefix_rows, resp_rows, out=None):
    """Packed [T, ...] rows from the groups' prefix rows [sum P, ...] and the
    responses' rows [sum R, ...] (same trailing shape and dtype)."""
    torch = _torch()
    d = batch.desc
    n_pre, tail, dt = d.total_prefix_rows, tuple(prefix_rows.shape[1:]), prefix_rows.dtype
    _rows_check(prefix_rows, n_pre, tail, dt, "prefix_rows")
    _rows_check(resp_rows, d.total_rows - n_pre, tail, dt, "resp_rows")
    if out is None:
        out = torch.empty((d.total_rows,) + tail, dtype=dt, device=prefix_rows.device)
    _rows_check(out, d.total_rows, tail, dt, "out")
    row_bytes = int(np.prod(tail, dtype=np.int64)) * prefix_rows.element_size()
    _check(lib().pg_pack_rows(ctypes.byref(d), _vp(prefix_rows), _vp(resp_rows), _vp(out),
                              row_bytes, _stream_ptr(out.device)))
    return out


def pg_unpack_rows(batch: PackedBatch, packed_rows):
    """(prefix rows [sum P, ...], response rows [sum R, ...]) of packed [T, ...] rows."""
    torch = _torch()
    d = batch.desc
    n_pre, tail, dt = d.total_prefix_rows, tuple(packed_rows.shape[1:]), packed_rows.dtype
    _rows_check(packed_rows, d.total_rows, tail, dt, "packed_rows")
    pre = torch.empty((n_pre,) + tail, dtype=dt, device=packed_rows.device)
    resp = torch.empty((d.total_rows - n_pre,) + tail, dtype=dt, device=packed_rows.device)
    row_bytes = int(np.prod(tail, dtype=np.int64)) * packed_rows.element_size()
    _check(lib().pg_unpack_rows(ctypes.byref(d), _vp(packed_rows), _vp(pre), _vp(resp), row_bytes,
                                _stream_ptr(packed_rows.device)))
    return pre, resp


def _head_args(batch, hidden, weight, tokens):
    torch = _torch()
    d = batch.desc
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise PgError(PG_ERR_INVALID_ARG, "hidden and weight must be bfloat16")
    if hidden.dim() != 2 or hidden.shape[0] != d.total_rows or not hidden.is_contiguous():
        raise PgError(PG_ERR_INVALID_ARG, "hidden must be contiguous [T, d_model]")
    if weight.dim() != 2 or weight.shape[1] != hidden.shape[1] or not weight.is_contiguous():
        raise PgError(PG_ERR_INVALID_ARG, "weight must be contiguous [vocab, d_model]")
    if tokens.dtype != torch.int32 or tokens.shape != (d.total_rows,) or not tokens.is_contiguous():
        raise PgError(PG_ERR_INVALID_ARG, "tokens must be contiguous int32 [T]")
    if weight.device != hidden.device or tokens.device != hidden.device:
        raise PgError(PG_ERR_INVALID_ARG, "hidden, weight and tokens must be on one device")
    return d, int(weight.shape[0]), int(hidden.shape[1])


def _head_workspace(d, vocab, d_model, device, workspace):
    torch = _torch()
    need = lib().pg_logprob_workspace_size(ctypes.byref(d), vocab, d_model)
    if need == 0:
        raise PgError(PG_ERR_INVALID_ARG, lib().pg_last_error().decode())
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, need


def pg_logprob_fwd(batch: PackedBatch, hidden, weight, tokens, workspace=None):
    """(logp, lse), float [num_scored] each: log-probability of every scored
    response token and the logsumexp of the logits that score it."""
    torch = _torch()
    d, vocab, d_model = _head_args(batch, hidden, weight, tokens)
    n = d.num_scored
    logp = torch.empty(max(n, 1), dtype=torch.float32, device=hidden.device)
    lse = torch.empty(max(n, 1), dtype=torch.float32, device=hidden.device)
    ws, need = _head_workspace(d, vocab, d_model, hidden.device, workspace)
    _check(lib().pg_logprob_fwd(ctypes.byref(d), _vp(hidden), _vp(weight), vocab, d_model,
                                _vp(tokens), _vp(logp), _vp(lse), _vp(ws), need,
                                _stream_ptr(hidden.device)))
    return logp[:n], lse[:n]


def _f32_vector(name, x, n, device):
    """Refuse (before any launch) a float32 vector input shorter than n entries,
    strided, or on another device: the kernels read n entries."""
    torch = _torch()
    if x.dtype != torch.float32 or x.dim() != 1 or x.shape[0] < n or not x.is_contiguous():
        raise PgError(PG_ERR_INVALID_ARG, f"{name} must be a contiguous float32 vector of {n} entries")
    if x.device != device:
        raise PgError(PG_ERR_INVALID_ARG, f"{name} is on {x.device}, expected {device}")


def pg_grpo_loss(batch: PackedBatch, logp, advantages):
    """(loss [1], dlogp [num_scored]) of -mean_i(A_i * sum of response i's logp)."""
    torch = _torch()
    d = batch.desc
    _f32_vector("advantages", advantages, d.num_resp, advantages.device)
    _f32_vector("logp", logp, d.num_scored, advantages.device)
    loss = torch.empty(1, dtype=torch.float32, device=advantages.device)
    dlogp = torch.empty(max(d.num_scored, 1), dtype=torch.float32, device=advantages.device)
    _check(lib().pg_grpo_loss(ctypes.byref(d), _vp(logp), _vp(advantages), _vp(loss), _vp(dlogp),
                              _stream_ptr(advantages.device)))
    return loss, dlogp[:d.num_scored]


def pg_logprob_bwd(batch: PackedBatch, hidden, weight, tokens, lse, dlogp, workspace=None):
    """(dhidden fp32 [T, d_model], dweight fp32 [vocab, d_model])."""
    torch = _torch()
    d, vocab, d_model = _head_args(batch, hidden, weight, tokens)
    _f32_vector("lse", lse, d.num_scored, hidden.device)
    _f32_vector("dlogp", dlogp, d.num_scored, hidden.device)
    dh = torch.empty((max(d.total_rows, 1), d_model), dtype=torch.float32, device=hidden.device)
    dw = torch.empty((vocab, d_model), dtype=torch.float32, device=hidden.device)
    ws, need = _head_workspace(d, vocab, d_model, hidden.device, workspace)
    _check(lib().pg_logprob_bwd(ctypes.byref(d), _vp(hidden), _vp(weight), vocab, d_model,
                                _vp(tokens), _vp(lse), _vp(dlogp), _vp(dh), _vp(dw), _vp(ws), need,
                                _stream_ptr(hidden.device)))
    return dh[:d.total_rows], dw


def pg_kernel_timing(enable: bool) -> None:
    """Enable (and clear) or disable per-kernel HIP-event timing inside the library."""
    _check(lib().pg_kernel_timing(int(bool(enable))))


def pg_kernel_times() -> dict:
    """{kernel name: (launches, total milliseconds)} since timing was last enabled."""
    L = lib()
    out = {}
    for i, name in enumerate(KERNELS):
        n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
        _check(L.pg_kernel_times(i, ctypes.byref(n), ctypes.byref(ms)))
        out[name] = (int(n.value), float(ms.value))
    return out


def version() -> str:
    return lib().pg_version().decode()


def _make_autograd():
    torch = _torch()

    class GroupedAttention(torch.autograd.Function):
        """Grouped shared-prefix attention with the library's backward."""

        @staticmethod
        def forward(ctx, q, k, v, batch, softmax_scale=None):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            o, lse = pg_attn_fwd(batch, q, k, v, softmax_scale)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.batch = batch
            ctx.softmax_scale = softmax_scale
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = pg_attn_bwd(ctx.batch, q, k, v, o, lse, do.contiguous(), ctx.softmax_scale)
            return dq, dk, dv, None, None

    return GroupedAttention


class _Lazy:
    def __init__(self):
        self._cls = None

    def apply(self, *args):
        if self._cls is None:
            self._cls = _make_autograd()
        return self._cls.apply(*args)


GroupedAttention = _Lazy()


def grouped_attention(q, k, v, batch: PackedBatch, softmax_scale: Optional[float] = None):
    """Autograd-aware grouped attention on packed rows."""
    return GroupedAttention.apply(q, k, v, batch, softmax_scale)
