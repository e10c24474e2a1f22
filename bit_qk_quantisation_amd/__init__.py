"""BinaryAttention forward on MI355X (gfx950): Python binding.

The binding only marshals arguments: torch supplies device memory and the
current HIP stream, and every step of the computation runs in the HIP
kernels of libbinattn.so (built by ``python -m bit_qk_quantisation_amd.build``).
If the library is missing the calls raise; there is no CPU fallback.

    pack_signs(x)                          -> (bits uint32-as-int32, alpha f32)
    attention_fwd(q, k, v, table, gh, gw)  -> O (bf16); q, k, v and out may be
                                              strided [B,H,N,d] views (e.g.
                                              a [B,N,H,d] tensor transposed)
    attention_fwd_dense_bias(q, k, v, bias) -> O (bf16); bias [1 or B, H, N, N]
    attention_fwd_int8pv(q, k, v, table, gh, gw) -> O (bf16), 8-bit P.V
    attention_bwd(q, k, v, dO, table, gh, gw) -> (dq, dk, dv, dtable), float32
    qk_int_dot(qbits, kbits, d, route)     -> D (int32)
    workspace_bytes(B, H, N, d, gh, gw)    -> int
"""

from __future__ import annotations

import ctypes
import math

import torch

from ._lib import (BinAttnError, EXPORTS, QK_ROWSUM, ROUTE_MFMA_FP4,  # noqa: F401
                   ROUTE_MFMA_INT8, ROUTE_VALU_POPCOUNT, check, load)

__all__ = ["pack_signs", "attention_fwd", "attention_fwd_dense_bias", "attention_fwd_int8pv", "attention_fwd_train",
           "attention_bwd",
           "qk_int_dot", "workspace_bytes",
           "pack_words", "BinAttnError", "ROUTE_MFMA_FP4", "ROUTE_VALU_POPCOUNT", "ROUTE_MFMA_INT8",
           "QK_ROWSUM",
           "Workspace"]


def _stream(device: torch.device):
    return ctypes_ptr(torch.cuda.current_stream(device).cuda_stream)


def ctypes_ptr(x):
    return None if x in (None, 0) else int(x)


def _need(t: torch.Tensor, name: str, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _need_view(t: torch.Tensor, name: str):
    """A bf16 [B,H,N,d] view on a HIP device whose channels are contiguous."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must have 4 dims, got {tuple(t.shape)}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name} must have contiguous channels (stride 1 in the last dim)")


def pack_words(d: int) -> int:
    return load().ba_pack_words(int(d))


def workspace_bytes(B, H, N, d, gh=0, gw=0) -> int:
    return int(load().ba_workspace_bytes(int(B), int(H), int(N), int(d), int(gh), int(gw)))


def pack_signs(x: torch.Tensor):
    """Packed signs and per-token scale of a bf16 [B,H,N,d] tensor.

    Returns (bits int32 [B,H,N,W] holding the uint32 words, alpha f32 [B,H,N])."""
    lib = load()
    _need(x, "x", torch.bfloat16, 4)
    B, H, N, d = x.shape
    W = lib.ba_pack_words(d)
    bits = torch.empty((B, H, N, max(W, 1)), dtype=torch.int32, device=x.device)
    alpha = torch.empty((B, H, N), dtype=torch.float32, device=x.device)
    check(lib, lib.ba_pack_signs(x.data_ptr(), B, H, N, d, bits.data_ptr(),
                                 alpha.data_ptr(), _stream(x.device)))
    return bits, alpha


class Workspace:
    """A reusable device workspace, grown on demand: one buffer per (device,
    stream).  Calls on one stream run in order, so they may share a buffer;
    calls on two streams get two buffers and cannot race on it.  A buffer is
    allocated while its stream is current, so when a larger one replaces it,
    torch's allocator hands the old memory out again only in that stream's
    order, after the kernels that used it."""

    def __init__(self):
        self._buf = {}

    def get(self, device: torch.device, nbytes: int, stream=None) -> torch.Tensor:
        key = (str(device), stream)
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
            self._buf[key] = buf
        return buf


_default_ws = Workspace()


def attention_fwd(q, k, v, table=None, gh: int = 0, gw: int = 0, scale=None,
                  out=None, workspace: Workspace | None = None):
    """BinaryAttention forward: bf16 q, k, v [B,H,N,d] (+ bf16 table
    [H, 2gh-1, 2gw-1]) -> bf16 O [B,H,N,d]."""
    lib = load()
    _need_view(q, "q")
    _need_view(k, "k")
    _need_view(v, "v")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have the same shape")
    B, H, N, d = q.shape
    if table is not None:
        _need(table, "table", torch.bfloat16, 3)
        if tuple(table.shape) != (H, 2 * gh - 1, 2 * gw - 1):
            raise ValueError(f"table must be [H, 2gh-1, 2gw-1] = {(H, 2*gh-1, 2*gw-1)}")
    else:
        gh = gw = 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_view(out, "out")
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    nbytes = lib.ba_workspace_bytes(B, H, N, d, gh, gw)
    if nbytes == 0:
        raise BinAttnError(2, f"unsupported problem B={B} H={H} N={N} d={d} grid={gh}x{gw}")
    ws = (workspace or _default_ws).get(q.device, nbytes, _stream(q.device))
    base = ws.data_ptr()
    aligned = (base + 255) // 256 * 256
    tp = None if table is None else table.data_ptr()
    ws_len = ws.numel() - (aligned - base)
    views = (q, k, v, out)
    if all(t.is_contiguous() for t in views):
        check(lib, lib.ba_attention_fwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, int(gh), int(gw),
            B, H, N, d, float(scale), out.data_ptr(), aligned, ws_len, _stream(q.device)))
    else:
        strides = (ctypes.c_int64 * 12)(*[t.stride(i) for t in views for i in range(3)])
        check(lib, lib.ba_attention_fwd_strided(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, int(gh), int(gw),
            B, H, N, d, float(scale), out.data_ptr(), strides, aligned, ws_len,
            _stream(q.device)))
    return out


def attention_fwd_dense_bias(q, k, v, bias, scale=None, out=None,
                             workspace: Workspace | None = None):
    """BinaryAttention forward with a dense bias: bf16 q, k, v [B,H,N,d]
    views (channels contiguous) and a bf16 bias [1 or B, H, N, N] whose rows
    are contiguous and whose strides are multiples of 8 elements (size-1
    batch: shared by the whole batch) -> bf16 O [B,H,N,d]."""
    lib = load()
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need_view(t, name)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have the same shape")
    B, H, N, d = q.shape
    _need_view(bias, "bias")
    if bias.shape[1:] != (H, N, N) or bias.shape[0] not in (1, B):
        raise ValueError(f"bias must be [1 or {B}, {H}, {N}, {N}], got {tuple(bias.shape)}")
    sb = 0 if bias.shape[0] == 1 else bias.stride(0)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_view(out, "out")
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    nbytes = lib.ba_workspace_bytes(B, H, N, d, 0, 0)
    if nbytes == 0:
        raise BinAttnError(2, f"unsupported problem B={B} H={H} N={N} d={d}")
    ws = (workspace or _default_ws).get(q.device, nbytes, _stream(q.device))
    base = ws.data_ptr()
    aligned = (base + 255) // 256 * 256
    views = (q, k, v, out)
    strides = (ctypes.c_int64 * 12)(*[t.stride(i) for t in views for i in range(3)])
    check(lib, lib.ba_attention_fwd_dense_bias(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), bias.data_ptr(), sb, bias.stride(1),
        bias.stride(2), B, H, N, d, float(scale), out.data_ptr(), strides, aligned,
        ws.numel() - (aligned - base), _stream(q.device)))
    return out


def attention_fwd_int8pv(q, k, v, table=None, gh: int = 0, gw: int = 0, scale=None,
                         out=None, workspace: Workspace | None = None):
    """BinaryAttention forward with the 8-bit P.V (8-bit attention
    coefficients and per-channel 8-bit values): contiguous bf16 q, k, v
    [B,H,N,d] (+ bf16 table [H, 2gh-1, 2gw-1]) -> bf16 O [B,H,N,d]."""
    lib = load()
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, 4)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have the same shape")
    B, H, N, d = q.shape
    if table is not None:
        _need(table, "table", torch.bfloat16, 3)
        if tuple(table.shape) != (H, 2 * gh - 1, 2 * gw - 1):
            raise ValueError(f"table must be [H, 2gh-1, 2gw-1] = {(H, 2*gh-1, 2*gw-1)}")
    else:
        gh = gw = 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 4)
    nbytes = lib.ba_workspace_bytes_int8pv(B, H, N, d, gh, gw)
    if nbytes == 0:
        raise BinAttnError(3, f"unsupported problem B={B} H={H} N={N} d={d} grid={gh}x{gw}")
    ws = (workspace or _default_ws).get(q.device, nbytes, _stream(q.device))
    base = ws.data_ptr()
    aligned = (base + 255) // 256 * 256
    check(lib, lib.ba_attention_fwd_int8pv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), None if table is None else table.data_ptr(),
        int(gh), int(gw), B, H, N, d, float(scale), out.data_ptr(), aligned,
        ws.numel() - (aligned - base), _stream(q.device)))
    return out


def attention_fwd_train(q, k, v, table=None, gh: int = 0, gw: int = 0, scale=None,
                        workspace: Workspace | None = None):
    """attention_fwd for a training step: contiguous bf16 q, k, v [B,H,N,d]
    (+ bf16 table) -> (bf16 O [B,H,N,d], float32 lse [B,H,N]) with
    lse[b,h,i] = ln sum_j exp(S_ij); pass both to attention_bwd."""
    lib = load()
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, 4)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape")
    B, H, N, d = q.shape
    if table is not None:
        _need(table, "table", torch.bfloat16, 3)
        if tuple(table.shape) != (H, 2 * gh - 1, 2 * gw - 1):
            raise ValueError(f"table must be [H, 2gh-1, 2gw-1] = {(H, 2*gh-1, 2*gw-1)}")
    else:
        gh = gw = 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = lib.ba_workspace_bytes(B, H, N, d, gh, gw)
    if nbytes == 0:
        raise BinAttnError(2, f"unsupported problem B={B} H={H} N={N} d={d} grid={gh}x{gw}")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = (workspace or _default_ws).get(q.device, nbytes, _stream(q.device))
    base = ws.data_ptr()
    aligned = (base + 255) // 256 * 256
    check(lib, lib.ba_attention_fwd_train(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), None if table is None else table.data_ptr(), int(gh), int(gw),
        B, H, N, d, float(scale), out.data_ptr(), lse.data_ptr(), aligned, ws.numel() - (aligned - base),
        _stream(q.device)))
    return out, lse


def attention_bwd(q, k, v, dout, table=None, gh: int = 0, gw: int = 0, scale=None,
                  workspace: Workspace | None = None, o=None, lse=None):
    """Gradients of attention_fwd for the output gradient dout: contiguous
    bf16 q, k, v, dout [B,H,N,d] (+ bf16 table [H, 2gh-1, 2gw-1]) ->
    float32 dq, dk, dv [B,H,N,d] and dtable [H, 2gh-1, 2gw-1] (None without a
    table).  The sign function takes the clipped straight-through estimator
    and alpha = mean |x| its exact derivative.  With o and lse from
    attention_fwd_train the forward is not recomputed."""
    lib = load()
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, name, torch.bfloat16, 4)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v and dout must have the same shape")
    if (o is None) != (lse is None):
        raise ValueError("pass both o and lse, or neither")
    B, H, N, d = q.shape
    if o is not None:
        _need(o, "o", torch.bfloat16, 4)
        _need(lse, "lse", torch.float32, 3)
        if o.shape != q.shape or tuple(lse.shape) != (B, H, N):
            raise ValueError("o must be [B,H,N,d] and lse [B,H,N]")
    if table is not None:
        _need(table, "table", torch.bfloat16, 3)
        if tuple(table.shape) != (H, 2 * gh - 1, 2 * gw - 1):
            raise ValueError(f"table must be [H, 2gh-1, 2gw-1] = {(H, 2*gh-1, 2*gw-1)}")
    else:
        gh = gw = 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = lib.ba_workspace_bytes_bwd(B, H, N, d, gh, gw)
    if nbytes == 0:
        raise BinAttnError(3, f"unsupported problem B={B} H={H} N={N} d={d} grid={gh}x{gw}")
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    dtable = None if table is None else torch.empty(table.shape, dtype=torch.float32, device=q.device)
    ws = (workspace or _default_ws).get(q.device, nbytes, _stream(q.device))
    base = ws.data_ptr()
    aligned = (base + 255) // 256 * 256
    tp = None if table is None else table.data_ptr()
    dtp = None if dtable is None else dtable.data_ptr()
    ws_len = ws.numel() - (aligned - base)
    if o is None:
        check(lib, lib.ba_attention_bwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, int(gh), int(gw), B, H, N, d, float(scale),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dtp, aligned, ws_len,
            _stream(q.device)))
    else:
        check(lib, lib.ba_attention_bwd_saved(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), tp, int(gh), int(gw), B, H, N, d, float(scale),
            o.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dtp,
            aligned, ws_len, _stream(q.device)))
    return dq, dk, dv, dtable


def qk_int_dot(qbits, kbits, d: int, route: int = ROUTE_MFMA_FP4, rowsum: bool = False):
    """All-pairs integer dots <sign q_i, sign k_j> from packed bits, or
    with rowsum=True their sums over the keys, int32 [B,H,N]."""
    lib = load()
    _need(qbits, "qbits", torch.int32, 4)
    _need(kbits, "kbits", torch.int32, 4)
    if qbits.shape != kbits.shape:
        raise ValueError("qbits and kbits must have the same shape")
    B, H, N, W = qbits.shape
    if W != lib.ba_pack_words(d):
        raise ValueError("word count does not match d")
    shape = (B, H, N) if rowsum else (B, H, N, N)
    dots = torch.empty(shape, dtype=torch.int32, device=qbits.device)
    route = int(route) | (QK_ROWSUM if rowsum else 0)
    check(lib, lib.ba_qk_int_dot(qbits.data_ptr(), kbits.data_ptr(), B, H, N, int(d),
                                 int(route), dots.data_ptr(), _stream(qbits.device)))
    return dots
