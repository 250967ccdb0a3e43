"""MI355X (gfx950) exact attention over packed variable-length sequences.

Thin Python binding over the C ABI of ``libattn_varlen.so`` (declared in
``include/attn_varlen.h``): it checks tensor shapes, dtypes and devices, allocates
outputs with PyTorch and passes raw pointers plus the current HIP stream. Every
step of the computation runs in the library's HIP kernels; there is no other
code path.

Entry points (same names as the C functions):
  * ``attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
    softmax_scale=None, causal=False, return_lse=False, out=None, lse=None,
    window_size=(-1, -1), num_splits=1)``
  * ``attn_varlen_bwd(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k,
    max_seqlen_q, max_seqlen_k, softmax_scale=None, causal=False, ...)``
  * ``attn_varlen_func(...)``: autograd wrapper (forward, then ``.backward(dout)``).

Shapes: q ``(total_q, Hq, D)``, k and v ``(total_k, Hkv, D)``, bf16, contiguous;
cu_seqlens int32 on the same device; lse fp32 ``(Hq, total_q)``. The reference
call shape is the varlen attention call of the "FA2 vs NATTEN on A100" issue's
benchmark script and the varlen entry point in the FlashAttention repository
guide's Public API.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Tuple

import torch

from ._lib import LibraryMissing, lib

__all__ = [
    "attn_varlen_fwd",
    "attn_varlen_bwd",
    "attn_varlen_fwd_window",
    "attn_varlen_bwd_window",
    "attn_varlen_bwd_workspace_size",
    "attn_varlen_bwd_ds_workspace_size",
    "bwd_workspace_bytes",
    "attn_varlen_bwd_stored_ds",
    "attn_varlen_bwd_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "attn_varlen_fwd_splitkv",
    "attn_varlen_fwd_splitkv_workspace_size",
    "attn_varlen_fwd_num_splits",
    "attn_varlen_fwd_persistent",
    "SCHED_BYTES",
    "attn_varlen_error_string",
    "attn_varlen_validate_seqlens",
    "attn_varlen_version",
    "attn_varlen_schedule_host",
    "attn_varlen_schedule_device",
    "attn_varlen_tile_plan_host",
    "attn_varlen_func",
    "attn_varlen_profile_enable",
    "attn_varlen_profile_records",
    "AttnVarlenError",
    "LibraryMissing",
]


class AttnVarlenError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where} failed with code {code}: {attn_varlen_error_string(code)}")


def attn_varlen_error_string(code: int) -> str:
    return lib().attn_varlen_error_string(int(code)).decode()


def attn_varlen_version() -> Tuple[int, int]:
    v = lib().attn_varlen_version()
    return v >> 16, v & 0xFFFF


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _on_input_device(fn):
    """Run fn with its first device tensor argument's device current: the library
    launches on the current HIP device, and its stream argument is that device's
    current stream."""

    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        for a in args:
            if isinstance(a, torch.Tensor) and a.is_cuda:
                with torch.cuda.device(a.device):
                    return fn(*args, **kwargs)
        return fn(*args, **kwargs)

    return wrapped


def _check_bf16(name: str, t: torch.Tensor, dev: torch.device):
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != 3:
        raise ValueError(f"{name} must be 3-D (tokens, heads, head_dim), got {tuple(t.shape)}")


SEQLEN_BITS = {1: "a first cu_seqlens entry is not 0", 2: "cu_seqlens decreases",
               4: "a last cu_seqlens entry differs from the token count",
               8: "a sequence is longer than its max_seqlen"}


@_on_input_device
def attn_varlen_validate_seqlens(cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, total_q: int, total_k: int,
                                 max_seqlen_q: int, max_seqlen_k: int) -> int:
    """Check the packing arrays on the device (waits for the result): returns 0 when valid, else the
    ATTN_VARLEN_SEQLEN_* bit mask."""
    dev = cu_seqlens_q.device
    res = torch.empty(1, dtype=torch.int32, device=dev)
    rc = lib().attn_varlen_validate_seqlens(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1,
                                            int(total_q), int(total_k), int(max_seqlen_q), int(max_seqlen_k),
                                            _ptr(res), _stream(dev))
    if rc != 0:
        raise AttnVarlenError(rc, "attn_varlen_validate_seqlens")
    return int(res.item())


def _maybe_validate(cu_q, cu_k, total_q, total_k, max_q, max_k):
    if os.environ.get("ATTN_VARLEN_VALIDATE") != "1":
        return
    bits = attn_varlen_validate_seqlens(cu_q, cu_k, total_q, total_k, max_q, max_k)
    if bits:
        why = "; ".join(t for b, t in SEQLEN_BITS.items() if bits & b)
        raise ValueError(f"invalid cu_seqlens / max_seqlen (mask {bits}): {why}")


def _check_inputs(q, k, v, cu_q, cu_k):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(n, t, dev)
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must have the same shape")
    if q.shape[2] != k.shape[2]:
        raise ValueError("q and k must have the same head_dim")
    for n, t in (("cu_seqlens_q", cu_q), ("cu_seqlens_k", cu_k)):
        if t.dtype != torch.int32 or t.device != dev or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous 1-D int32 tensor on {dev}")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length >= 2")
    return dev


@_on_input_device
def attn_varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                    softmax_scale: Optional[float] = None, causal: bool = False, return_lse: bool = False,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    window_size: Tuple[int, int] = (-1, -1), num_splits: int = 1,
                    workspace: Optional[torch.Tensor] = None, persistent: bool = False,
                    sched: Optional[torch.Tensor] = None):
    """Forward pass. Returns ``out`` or ``(out, lse)`` when ``return_lse`` (or ``lse`` is given).

    ``window_size = (left, right)`` restricts each query to a local band of keys
    (``attn_varlen_fwd_window``); ``(-1, -1)`` is no window. ``num_splits > 1``
    splits every item's keys over that many workgroups and merges the partial
    results (``attn_varlen_fwd_splitkv``); ``0`` lets the library choose.
    ``persistent=True`` runs the persistent scheduler (``attn_varlen_fwd_persistent``,
    one split only); ``sched`` is its zeroed scratch (``SCHED_BYTES`` bytes),
    allocated per call when not given."""
    if persistent and num_splits != 1:  # num_splits = 0 (library choice) may pick several
        raise ValueError("the persistent scheduler runs the one-pass forward: num_splits must be 1")
    dev = _check_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    total_q, Hq, D = q.shape
    total_k, Hkv, _ = k.shape
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    if lse is not None:
        if lse.dtype != torch.float32 or lse.shape != (Hq, total_q) or not lse.is_contiguous() or lse.device != dev:
            raise ValueError(f"lse must be contiguous float32 ({Hq}, {total_q}) on {dev}")
    wl, wr = (int(window_size[0]), int(window_size[1]))
    num_seqs = cu_seqlens_q.numel() - 1
    _maybe_validate(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k)
    if num_splits == 0:
        num_splits = attn_varlen_fwd_num_splits(num_seqs, total_q, max_seqlen_q, max_seqlen_k, Hq, Hkv, D)
    if num_splits != 1:
        ws_bytes = attn_varlen_fwd_splitkv_workspace_size(total_q, Hq, D, num_splits)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        rc = lib().attn_varlen_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                           num_seqs, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv,
                                           D, float(softmax_scale), int(bool(causal)), wl, wr, int(num_splits),
                                           _ptr(out), _ptr(lse), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(dev))
        if rc != 0:
            raise AttnVarlenError(rc, "attn_varlen_fwd_splitkv")
        return (out, lse) if lse is not None else out
    if persistent:
        if sched is None:
            sched = torch.zeros(SCHED_BYTES, dtype=torch.uint8, device=dev)
        elif sched.device != dev or sched.numel() * sched.element_size() < SCHED_BYTES:
            raise ValueError(f"sched must hold {SCHED_BYTES} bytes on {dev}")
        rc = lib().attn_varlen_fwd_persistent(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                              num_seqs, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), Hq,
                                              Hkv, D, float(softmax_scale), int(bool(causal)), wl, wr, _ptr(out),
                                              _ptr(lse), _ptr(sched), _stream(dev))
        if rc != 0:
            raise AttnVarlenError(rc, "attn_varlen_fwd_persistent")
        return (out, lse) if lse is not None else out
    if wl < 0 and wr < 0:  # no window: the plain entry point
        rc = lib().attn_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs,
                                   total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D,
                                   float(softmax_scale), int(bool(causal)), _ptr(out), _ptr(lse), _stream(dev))
        if rc != 0:
            raise AttnVarlenError(rc, "attn_varlen_fwd")
        return (out, lse) if lse is not None else out
    rc = lib().attn_varlen_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs,
                                      total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D,
                                      float(softmax_scale), int(bool(causal)), wl, wr, _ptr(out), _ptr(lse),
                                      _stream(dev))
    if rc != 0:
        raise AttnVarlenError(rc, "attn_varlen_fwd_window")
    return (out, lse) if lse is not None else out


SCHED_BYTES = 64  # ATTN_VARLEN_SCHED_BYTES


def attn_varlen_fwd_persistent(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
                               causal=False, window_left=-1, window_right=-1, sched=None, **kw):
    """``attn_varlen_fwd`` with the persistent scheduler (the C entry point of the same name)."""
    return attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                           window_size=(window_left, window_right), persistent=True, sched=sched, **kw)


def attn_varlen_fwd_splitkv_workspace_size(total_q: int, n_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(lib().attn_varlen_fwd_splitkv_workspace_size(total_q, n_q_heads, head_dim, num_splits))


def attn_varlen_fwd_num_splits(num_seqs: int, total_q: int, max_seqlen_q: int, max_seqlen_k: int, n_q_heads: int,
                               n_kv_heads: int, head_dim: int) -> int:
    """The library's split count for these sizes (host-only)."""
    n = int(lib().attn_varlen_fwd_num_splits(num_seqs, total_q, int(max_seqlen_q), int(max_seqlen_k), n_q_heads,
                                             n_kv_heads, head_dim))
    if n < 0:
        raise AttnVarlenError(n, "attn_varlen_fwd_num_splits")
    return n


def attn_varlen_fwd_splitkv(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
                            causal=False, window_left=-1, window_right=-1, num_splits=0, **kw):
    """``attn_varlen_fwd`` with split-KV (the C entry point of the same name); ``num_splits=0``: library choice."""
    return attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                           window_size=(window_left, window_right), num_splits=num_splits, **kw)


def attn_varlen_bwd_workspace_size(num_seqs: int, total_q: int, total_k: int, n_q_heads: int, n_kv_heads: int,
                                   head_dim: int) -> int:
    return int(lib().attn_varlen_bwd_workspace_size(num_seqs, total_q, total_k, n_q_heads, n_kv_heads, head_dim))


def attn_varlen_bwd_ds_workspace_size(num_seqs: int, total_q: int, total_k: int, max_seqlen_q: int,
                                      max_seqlen_k: int, n_q_heads: int, n_kv_heads: int, head_dim: int) -> int:
    """Workspace bytes with which the backward stores dS for dQ (0: not available)."""
    return int(lib().attn_varlen_bwd_ds_workspace_size(num_seqs, total_q, total_k, int(max_seqlen_q),
                                                       int(max_seqlen_k), n_q_heads, n_kv_heads, head_dim))


def bwd_workspace_bytes(num_seqs: int, total_q: int, total_k: int, max_seqlen_q: int, max_seqlen_k: int,
                        n_q_heads: int, n_kv_heads: int, head_dim: int, stored_ds: bool = False) -> int:
    """Workspace bytes of the backward: the recomputing one's, or with ``stored_ds``
    the stored-dS one's (``attn_varlen_bwd_stored_ds``)."""
    if stored_ds:
        ds = attn_varlen_bwd_ds_workspace_size(num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k, n_q_heads,
                                               n_kv_heads, head_dim)
        if ds == 0 and total_q > 0 and total_k > 0:
            raise ValueError("the stored-dS backward is not available for this problem")
        if ds:
            return ds
    return attn_varlen_bwd_workspace_size(num_seqs, total_q, total_k, n_q_heads, n_kv_heads, head_dim)


@_on_input_device
def attn_varlen_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                    lse: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                    max_seqlen_k: int, softmax_scale: Optional[float] = None, causal: bool = False,
                    dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                    dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    window_size: Tuple[int, int] = (-1, -1), stored_ds: bool = False):
    """Backward pass: returns ``(dq, dk, dv)`` for the loss ``sum(dout * out)``.

    ``window_size`` must be the forward's (``attn_varlen_bwd_window``).
    ``stored_ds=True`` runs ``attn_varlen_bwd_stored_ds`` (dS written by the
    dK / dV kernel and read by dQ instead of recomputed; head dims 64 / 128,
    slower on MI355X at every measured shape)."""
    dev = _check_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    _check_bf16("dout", dout, dev)
    _check_bf16("out", out, dev)
    if dout.shape != q.shape or out.shape != q.shape:
        raise ValueError("dout and out must have the shape of q")
    total_q, Hq, D = q.shape
    total_k, Hkv, _ = k.shape
    if lse.dtype != torch.float32 or lse.shape != (Hq, total_q) or not lse.is_contiguous() or lse.device != dev:
        raise ValueError(f"lse must be contiguous float32 ({Hq}, {total_q}) on {dev}")
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_bf16(n, t, dev)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have shape {tuple(ref.shape)}")
    num_seqs = cu_seqlens_q.numel() - 1
    _maybe_validate(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k)
    if workspace is None:
        ws_bytes = bwd_workspace_bytes(num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, stored_ds)
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    ws_given = workspace.numel() * workspace.element_size()
    wl, wr = (int(window_size[0]), int(window_size[1]))
    if stored_ds:
        rc = lib().attn_varlen_bwd_stored_ds(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                             num_seqs, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), Hq,
                                             Hkv, D, float(softmax_scale), int(bool(causal)), wl, wr, _ptr(dout),
                                             _ptr(out), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                             ws_given, _stream(dev))
        if rc != 0:
            raise AttnVarlenError(rc, "attn_varlen_bwd_stored_ds")
        return dq, dk, dv
    if wl < 0 and wr < 0:  # no window: the plain entry point
        rc = lib().attn_varlen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs,
                                   total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D,
                                   float(softmax_scale), int(bool(causal)), _ptr(dout), _ptr(out), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_given, _stream(dev))
        if rc != 0:
            raise AttnVarlenError(rc, "attn_varlen_bwd")
        return dq, dk, dv
    rc = lib().attn_varlen_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs,
                                      total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D,
                                      float(softmax_scale), int(bool(causal)), wl, wr, _ptr(dout), _ptr(out),
                                      _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_given,
                                      _stream(dev))
    if rc != 0:
        raise AttnVarlenError(rc, "attn_varlen_bwd_window")
    return dq, dk, dv


NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_VARLEN_NOALLOC_SCRATCH_BYTES


@_on_input_device
def attn_varlen_bwd_noalloc(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            out: torch.Tensor, lse: torch.Tensor, cu_seqlens_q: torch.Tensor,
                            cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                            softmax_scale: Optional[float] = None, causal: bool = False,
                            dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                            dv: Optional[torch.Tensor] = None):
    """``attn_varlen_bwd`` through the allocation-free C entry point: the library's
    static device scratch holds the workspace (calls on one GPU must not overlap).
    Pass ``dq``, ``dk``, ``dv`` to allocate nothing here either."""
    dev = _check_inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    _check_bf16("dout", dout, dev)
    _check_bf16("out", out, dev)
    if dout.shape != q.shape or out.shape != q.shape:
        raise ValueError("dout and out must have the shape of q")
    total_q, Hq, D = q.shape
    total_k, Hkv, _ = k.shape
    if lse.dtype != torch.float32 or lse.shape != (Hq, total_q) or not lse.is_contiguous() or lse.device != dev:
        raise ValueError(f"lse must be contiguous float32 ({Hq}, {total_q}) on {dev}")
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_bf16(n, t, dev)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have shape {tuple(ref.shape)}")
    num_seqs = cu_seqlens_q.numel() - 1
    _maybe_validate(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k)
    rc = lib().attn_varlen_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs,
                                       total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D,
                                       float(softmax_scale), int(bool(causal)), _ptr(dout), _ptr(out), _ptr(lse),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _stream(dev))
    if rc != 0:
        raise AttnVarlenError(rc, "attn_varlen_bwd_noalloc")
    return dq, dk, dv


def attn_varlen_schedule_host(cu_seqlens_q, block_m: int):
    """Host ranking of query blocks: list of (sequence, block) in the order the kernels visit them."""
    import numpy as np

    cu = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int32))
    n = lib().attn_varlen_schedule_host(cu.ctypes.data_as(ctypes.c_void_p), len(cu) - 1, block_m, None, None, 0)
    if n < 0:
        raise AttnVarlenError(int(n), "attn_varlen_schedule_host")
    seq = np.zeros(max(n, 1), dtype=np.int32)
    blk = np.zeros(max(n, 1), dtype=np.int32)
    n2 = lib().attn_varlen_schedule_host(cu.ctypes.data_as(ctypes.c_void_p), len(cu) - 1, block_m,
                                         seq.ctypes.data_as(ctypes.c_void_p), blk.ctypes.data_as(ctypes.c_void_p), n)
    assert n2 == n
    return list(zip(seq[:n].tolist(), blk[:n].tolist()))


PLAN_FWD, PLAN_DQ, PLAN_DKDV = 0, 1, 2  # ATTN_VARLEN_PLAN_*
PLAN_GROUP2, PLAN_GROUP4 = 0x10, 0x20  # or-ed into FWD / DQ: blocks of 2 / 4 heads x 64 / 32 rows


def attn_varlen_tile_plan_host(kind: int, head_dim: int, seqlen_q: int, seqlen_k: int, causal: bool,
                               window_left: int, window_right: int, block: int):
    """Tile plan of one work item (host only): dict with the block's first row or
    key, its size, the tile size, the visited tiles [lo, hi), the unmasked tiles
    [full_lo, full_hi) and, for the forward with a left bound, the left-edge tiles."""
    plan = (ctypes.c_int32 * 8)()
    rc = lib().attn_varlen_tile_plan_host(int(kind), int(head_dim), int(seqlen_q), int(seqlen_k), int(bool(causal)),
                                          int(window_left), int(window_right), int(block), plan)
    if rc != 0:
        raise AttnVarlenError(rc, "attn_varlen_tile_plan_host")
    keys = ("start", "size", "tile", "lo", "hi", "full_lo", "full_hi", "left_edge")
    return dict(zip(keys, list(plan)))


@_on_input_device
def attn_varlen_schedule_device(cu_seqlens_q: torch.Tensor, max_seqlen_q: int, block_m: int, count: int):
    """Device ranking of the first ``count`` ranks (the decode the kernels run)."""
    dev = cu_seqlens_q.device
    seq = torch.full((count,), -2, dtype=torch.int32, device=dev)
    blk = torch.full((count,), -2, dtype=torch.int32, device=dev)
    rc = lib().attn_varlen_schedule_device(_ptr(cu_seqlens_q), cu_seqlens_q.numel() - 1, int(max_seqlen_q), block_m,
                                           _ptr(seq), _ptr(blk), count, _stream(dev))
    if rc != 0:
        raise AttnVarlenError(rc, "attn_varlen_schedule_device")
    return seq, blk


class _AttnVarlenFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_q, cu_k, max_q, max_k, softmax_scale, causal, window_size, num_splits):
        out, lse = attn_varlen_fwd(q, k, v, cu_q, cu_k, max_q, max_k, softmax_scale, causal, return_lse=True,
                                   window_size=window_size, num_splits=num_splits)
        ctx.save_for_backward(q, k, v, out, lse, cu_q, cu_k)
        ctx.args = (max_q, max_k, softmax_scale, causal, window_size)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, cu_q, cu_k = ctx.saved_tensors
        max_q, max_k, softmax_scale, causal, window_size = ctx.args
        dq, dk, dv = attn_varlen_bwd(dout.contiguous(), q, k, v, out, lse, cu_q, cu_k, max_q, max_k, softmax_scale,
                                     causal, window_size=window_size)
        return dq, dk, dv, None, None, None, None, None, None, None, None


def attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
                     causal=False, window_size=(-1, -1), num_splits=1):
    """Differentiable varlen attention (forward kernel, then the backward kernels on ``.backward``)."""
    return _AttnVarlenFunction.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale,
                                     causal, tuple(window_size), int(num_splits))


def attn_varlen_fwd_window(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
                           causal=False, window_left=-1, window_right=-1, **kw):
    """``attn_varlen_fwd`` with a local window (the C entry point of the same name)."""
    return attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                           window_size=(window_left, window_right), **kw)


def attn_varlen_bwd_stored_ds(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                              softmax_scale=None, causal=False, window_left=-1, window_right=-1, **kw):
    """``attn_varlen_bwd`` with dS stored for dQ (the C entry point of the same name)."""
    return attn_varlen_bwd(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                           softmax_scale, causal, window_size=(window_left, window_right), stored_ds=True, **kw)


def attn_varlen_bwd_window(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                           softmax_scale=None, causal=False, window_left=-1, window_right=-1, **kw):
    """``attn_varlen_bwd`` with a local window (the C entry point of the same name)."""
    return attn_varlen_bwd(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                           softmax_scale, causal, window_size=(window_left, window_right), **kw)


def attn_varlen_profile_enable(enable: bool = True) -> None:
    """Start (drop earlier records) or stop per-launch event timing inside the library."""
    lib().attn_varlen_profile_enable(1 if enable else 0)


def attn_varlen_profile_records():
    """List of (kernel name, ms) for the launches recorded in the current session (waits for them)."""
    l = lib()
    n = l.attn_varlen_profile_count()
    out = []
    buf = ctypes.create_string_buffer(64)
    ms = ctypes.c_float()
    for i in range(n):
        rc = l.attn_varlen_profile_get(i, buf, 64, ctypes.byref(ms))
        if rc != 0:
            raise AttnVarlenError(rc, "attn_varlen_profile_get")
        out.append((buf.value.decode(), float(ms.value)))
    return out
