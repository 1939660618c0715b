"""Python binding of libsdpa_mi355x.so (fused SDPA forward for MI355X / gfx950).

Argument marshalling only: every step of the attention runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.  When
the library is missing, every entry point raises -- there is no CPU path.

    prefill(q, k, v, scale=None, causal=False, mask=None, sinks=None, return_lse=False,
            seqlens_q=None, seqlens_k=None)
    decode(q, k, v, scale=None, causal=False, mask=None, sinks=None, return_lse=False,
           num_splits=0, seqlens_q=None, seqlens_k=None)

    prefill_backward(q, k, v, o, lse, dout, scale=None, causal=False, mask=None, sinks=None,
                     seqlens_q=None, seqlens_k=None, want_dsinks=False)
    attention(q, k, v, ...)   autograd-aware prefill (forward + backward kernels)

q: [B, Hq, Lq, D], k / v: [B, Hkv, Lk, D] (float32, float16 or bfloat16),
mask: broadcastable to [B, Hq, Lq, Lk], additive float or bool (True = the
key takes part), sinks: [Hq],
seqlens_q / seqlens_k: per-batch real query rows / keys [B] (padding masks).
Returns O ([B, Hq, Lq, D], dtype of q) or (O, LSE) with LSE fp32 [B, Hq, Lq].
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["prefill", "decode", "decode_noalloc", "DECODE_SCRATCH_BYTES", "decode_num_splits",
           "decode_workspace_bytes", "prefill_workspace_bytes", "prefill_backward", "attention", "SdpaArgs", "SdpaBwdArgs", "library",
           "library_path", "Status", "SdpaError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "lib", "libsdpa_mi355x.so")

F32, F16, BF16 = 0, 1, 2
MASK_ADD_F32, MASK_BOOL = 0, 1
_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}


class Status:
    OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_ARG, ERR_HIP = range(8)


class SdpaError(ValueError):
    """A request the library rejected (status code in ``.status``)."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"sdpa status {status}: {msg}")
        self.status = status


class SdpaArgs(ctypes.Structure):
    """Mirror of ``struct sdpa_args`` (include/sdpa_mi355x.h)."""
    _fields_ = [
        ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("Lq", ctypes.c_int64), ("Lk", ctypes.c_int64), ("D", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float), ("mask_kind", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_stride", ctypes.c_int64 * 3),
        ("k", ctypes.c_void_p), ("k_stride", ctypes.c_int64 * 3),
        ("v", ctypes.c_void_p), ("v_stride", ctypes.c_int64 * 3),
        ("o", ctypes.c_void_p), ("o_stride", ctypes.c_int64 * 3),
        ("mask", ctypes.c_void_p), ("mask_stride", ctypes.c_int64 * 4),
        ("sinks", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("seqlens_q", ctypes.c_void_p),
        ("seqlens_k", ctypes.c_void_p),
        ("Dv", ctypes.c_int64),
    ]


class SdpaBwdArgs(ctypes.Structure):
    """Mirror of ``struct sdpa_bwd_args`` (include/sdpa_mi355x.h)."""
    _fields_ = [
        ("dout", ctypes.c_void_p), ("dout_stride", ctypes.c_int64 * 3),
        ("dq", ctypes.c_void_p), ("dq_stride", ctypes.c_int64 * 3),
        ("dk", ctypes.c_void_p), ("dk_stride", ctypes.c_int64 * 3),
        ("dv", ctypes.c_void_p), ("dv_stride", ctypes.c_int64 * 3),
        ("dsinks", ctypes.c_void_p),
    ]


_lib = None


def library():
    """Load the HIP library (raises RuntimeError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"{library_path} is missing: build it with "
            "`python -m scaled_dot_product_prefill_amd.build_lib` (there is no CPU fallback)")
    lib = ctypes.CDLL(library_path)
    P = ctypes.POINTER(SdpaArgs)
    lib.sdpa_prefill.argtypes = [P, ctypes.c_void_p]
    lib.sdpa_prefill.restype = ctypes.c_int
    lib.sdpa_prefill_check.argtypes = [P]
    lib.sdpa_prefill_check.restype = ctypes.c_int
    lib.sdpa_prefill_ws.argtypes = [P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.sdpa_prefill_ws.restype = ctypes.c_int
    lib.sdpa_prefill_workspace_bytes.argtypes = [P]
    lib.sdpa_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.sdpa_decode.argtypes = [P, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.sdpa_decode.restype = ctypes.c_int
    lib.sdpa_decode_check.argtypes = [P, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t]
    lib.sdpa_decode_check.restype = ctypes.c_int
    lib.sdpa_decode_noalloc.argtypes = [P, ctypes.c_int, ctypes.c_void_p]
    lib.sdpa_decode_noalloc.restype = ctypes.c_int
    lib.sdpa_decode_num_splits.argtypes = [P, ctypes.c_int]
    lib.sdpa_decode_num_splits.restype = ctypes.c_int
    lib.sdpa_decode_workspace_bytes.argtypes = [P, ctypes.c_int]
    lib.sdpa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_version.argtypes = []
    lib.sdpa_version.restype = ctypes.c_char_p
    G = ctypes.POINTER(SdpaBwdArgs)
    lib.sdpa_prefill_backward.argtypes = [P, G, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.sdpa_prefill_backward.restype = ctypes.c_int
    lib.sdpa_prefill_backward_check.argtypes = [P, G, ctypes.c_void_p, ctypes.c_size_t]
    lib.sdpa_prefill_backward_check.restype = ctypes.c_int
    lib.sdpa_prefill_backward_workspace_bytes.argtypes = [P]
    lib.sdpa_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def _raise(status: int):
    lib = library()
    msg = lib.sdpa_last_error().decode() or lib.sdpa_status_string(status).decode()
    if status == Status.ERR_HIP:
        raise RuntimeError(f"sdpa HIP error: {msg}")
    raise SdpaError(status, msg)


def _aligned(x: torch.Tensor) -> bool:
    """Unit last-dim stride and 16-byte aligned pointer and strides (the rule
    of prepare_sdpa_input on the mlx 0.30.7 page)."""
    es = x.element_size()
    return (x.stride(-1) == 1 and x.data_ptr() % 16 == 0
            and all((s * es) % 16 == 0 for s in x.stride()[:3]))


def _prep(x: torch.Tensor, name: str) -> torch.Tensor:
    """x itself if it meets the layout rule of _aligned, else a contiguous copy."""
    if x.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, L, D], got {tuple(x.shape)}")
    return x if _aligned(x) else x.contiguous()


def _on_device(t: torch.Tensor, name: str, device) -> None:
    """The kernels dereference every pointer on the GPU: a tensor elsewhere is
    an error here, before any launch."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _out_tensor(out: Optional[torch.Tensor], shape, dtype, device, name: str) -> torch.Tensor:
    """A new output, or the caller's: on the device, of this dtype and shape,
    and (being written in place) already in the layout of _aligned."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _on_device(out, name, device)
    if out.dtype != dtype or tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {out.dtype} {tuple(out.shape)}")
    if not _aligned(out):
        raise ValueError(f"{name} needs a unit last-dim stride and 16-byte aligned pointer and strides")
    return out


def _lse_tensor(lse: Optional[torch.Tensor], shape, device) -> torch.Tensor:
    """A new LSE output, or the caller's: written as a dense float32 [B, Hq, Lq]
    array, so it must be one on the device."""
    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    _on_device(lse, "lse", device)
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape) or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 {tuple(shape)} tensor")
    return lse


def _workspace(ws: Optional[torch.Tensor], need: int, device, min_bytes: int = 0) -> torch.Tensor:
    """The caller's workspace if it holds `need` bytes, else a new one.  A
    given workspace must be a contiguous tensor on the device."""
    if ws is not None:
        _on_device(ws, "workspace", device)
        if not ws.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if ws.numel() * ws.element_size() >= need:
            return ws
    return torch.empty(max(need, min_bytes), dtype=torch.uint8, device=device)


def _fill(a: SdpaArgs, name: str, t: Optional[torch.Tensor]):
    setattr(a, name, t.data_ptr() if t is not None else None)
    if t is not None:
        st = getattr(a, name + "_stride")
        for i in range(3):
            st[i] = t.stride(i)


def _make_args(q, k, v, o, scale, causal, mask, sinks, lse, seqlens_q=None, seqlens_k=None) -> SdpaArgs:
    B, Hq, Lq, D = q.shape
    a = SdpaArgs()
    a.B, a.Hq, a.Lq, a.D = B, Hq, Lq, D
    a.Hkv, a.Lk = k.shape[1], k.shape[2]
    a.Dv = v.shape[3]
    a.dtype = _DTYPE_CODE[q.dtype]
    a.causal = 1 if causal else 0
    a.scale = float(scale)
    a.mask_kind = MASK_BOOL if (mask is not None and mask.dtype == torch.bool) else MASK_ADD_F32
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _fill(a, n, t)
    if mask is not None:
        a.mask = mask.data_ptr()
        for i in range(4):
            a.mask_stride[i] = mask.stride(i)
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.lse = lse.data_ptr() if lse is not None else None
    a.seqlens_q = seqlens_q.data_ptr() if seqlens_q is not None else None
    a.seqlens_k = seqlens_k.data_ptr() if seqlens_k is not None else None
    return a


def _lengths(x, B: int, device, name: str):
    """Per-batch lengths as a contiguous int32 [B] tensor on the device."""
    if x is None:
        return None
    t = torch.as_tensor(x).to(device=device, dtype=torch.int32).reshape(-1).contiguous()
    if t.numel() != B:
        raise ValueError(f"{name} must have B = {B} entries, got {t.numel()}")
    return t


def _common(q, k, v, scale, mask, sinks, Lq_expected=None):
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share a dtype")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k and v must be GPU tensors (there is no CPU path)")
    if k.device != q.device or v.device != q.device:
        raise ValueError(f"q, k and v must be on one device, got {q.device}, {k.device}, {v.device}")
    q, k, v = _prep(q, "q"), _prep(k, "k"), _prep(v, "v")
    B, Hq, Lq, D = q.shape
    if k.shape[:3] != v.shape[:3] or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    Lk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if mask is not None:
        if mask.dtype != torch.float32 and mask.dtype != torch.bool:
            mask = mask.to(torch.float32)                   # additive; bool masks stay one byte
        mask = mask.to(q.device).expand(B, Hq, Lq, Lk)     # broadcast dims get stride 0
    if sinks is not None:
        sinks = sinks.to(device=q.device, dtype=torch.float32).reshape(Hq).contiguous()
    return q, k, v, scale, mask, sinks


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
            causal: bool = False, mask: Optional[torch.Tensor] = None,
            sinks: Optional[torch.Tensor] = None, return_lse: bool = False,
            out: Optional[torch.Tensor] = None, seqlens_q=None, seqlens_k=None,
            split_tail: bool = True, workspace: Optional[torch.Tensor] = None):
    """Fused attention forward over a whole query block (prefill / full
    self-attention).  seqlens_q / seqlens_k: real query rows / keys of each
    batch (the rest is padding; padding rows come out as rows with no key).
    split_tail: call sdpa_prefill_ws, which runs the query tiles past the last
    multiple of the compute units as key pieces (with a workspace, allocated
    here unless one is given) where that applies; False: sdpa_prefill."""
    lib = library()
    q, k, v, scale, mask, sinks = _common(q, k, v, scale, mask, sinks)
    B, Hq, Lq, D = q.shape
    o = _out_tensor(out, (B, Hq, Lq, v.shape[3]), q.dtype, q.device, "out")
    lse = _lse_tensor(None, (B, Hq, Lq), q.device) if return_lse else None
    sq = _lengths(seqlens_q, B, q.device, "seqlens_q")
    sk = _lengths(seqlens_k, B, q.device, "seqlens_k")
    a = _make_args(q, k, v, o, scale, causal, mask, sinks, lse, sq, sk)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    need = int(lib.sdpa_prefill_workspace_bytes(ctypes.byref(a))) if split_tail else 0
    if need > 0:
        workspace = _workspace(workspace, need, q.device)
        st = lib.sdpa_prefill_ws(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                                 workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream))
    else:
        st = lib.sdpa_prefill(ctypes.byref(a), ctypes.c_void_p(stream))
    if st != 0:
        _raise(st)
    return (o, lse) if return_lse else o


def prefill_workspace_bytes(q, k, v, *, causal: bool = False, mask=None, seqlens=False) -> int:
    """Workspace bytes sdpa_prefill_ws needs (0: none) for these shapes; a
    mask or per-batch lengths (seqlens=True) rule the tail split out."""
    lib = library()
    a = _size_args(q, k, v)
    a.causal = int(bool(causal))
    if mask is not None or seqlens:
        return 0
    return int(lib.sdpa_prefill_workspace_bytes(ctypes.byref(a)))


def _decode_args(q, k, v, scale, mask, sinks):
    q, k, v, scale, mask, sinks = _common(q, k, v, scale, mask, sinks)
    return q, k, v, scale, mask, sinks


def decode_num_splits(q, k, v, *, num_splits: int = 0) -> int:
    """Splits of the key range sdpa_decode would use (1 = single pass)."""
    lib = library()
    return int(lib.sdpa_decode_num_splits(ctypes.byref(_size_args(q, k, v)), int(num_splits)))


def decode_workspace_bytes(q, k, v, *, num_splits: int = 0) -> int:
    lib = library()
    return int(lib.sdpa_decode_workspace_bytes(ctypes.byref(_size_args(q, k, v)), int(num_splits)))


def _size_args(q, k, v=None) -> SdpaArgs:
    """Sizes-only argument block for the split / workspace queries."""
    a = SdpaArgs()
    a.B, a.Hq, a.Lq, a.D = q.shape
    a.Hkv, a.Lk = k.shape[1], k.shape[2]
    a.Dv = v.shape[3] if v is not None else 0
    a.dtype = _DTYPE_CODE[q.dtype]
    a.scale = 1.0
    return a


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
           causal: bool = False, mask: Optional[torch.Tensor] = None,
           sinks: Optional[torch.Tensor] = None, return_lse: bool = False, num_splits: int = 0,
           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           seqlens_q=None, seqlens_k=None):
    """Decode attention: one query row (Lq == 1) or a few (Lq <= 16, bottom-right
    causal within the block when ``causal``).  num_splits: 0 automatic,
    1 single-pass kernel, n >= 2 two-pass split-K with n key ranges.
    seqlens_k: fill level of each batch's KV cache (k, v may be the whole
    fixed-capacity cache); seqlens_q: real query rows of each batch."""
    lib = library()
    q, k, v, scale, mask, sinks = _decode_args(q, k, v, scale, mask, sinks)
    B, Hq, Lq, D = q.shape
    o = _out_tensor(out, (B, Hq, Lq, v.shape[3]), q.dtype, q.device, "out")
    lse = _lse_tensor(None, (B, Hq, Lq), q.device) if return_lse else None
    sq = _lengths(seqlens_q, B, q.device, "seqlens_q")
    sk = _lengths(seqlens_k, B, q.device, "seqlens_k")
    a = _make_args(q, k, v, o, scale, causal, mask, sinks, lse, sq, sk)
    need = int(lib.sdpa_decode_workspace_bytes(ctypes.byref(a), int(num_splits)))
    workspace = _workspace(workspace, need, q.device) if need > 0 else None
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if ws_ptr else 0
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.sdpa_decode(ctypes.byref(a), int(num_splits), ws_ptr, ws_bytes, ctypes.c_void_p(stream))
    if st != 0:
        _raise(st)
    return (o, lse) if return_lse else o


# bytes of the library's static per-GPU scratch that decode_noalloc uses
DECODE_SCRATCH_BYTES = 16 << 20


def decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
                   causal: bool = False, mask: Optional[torch.Tensor] = None,
                   sinks: Optional[torch.Tensor] = None, return_lse: bool = False, num_splits: int = 0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   seqlens_q=None, seqlens_k=None):
    """decode() through sdpa_decode_noalloc: the split partials live in the
    library's static per-GPU scratch, so the library call allocates nothing
    (pass ``out`` -- and ``lse`` with return_lse -- to allocate nothing here
    either).  Calls that overlap on one GPU share that scratch and race."""
    lib = library()
    q, k, v, scale, mask, sinks = _decode_args(q, k, v, scale, mask, sinks)
    B, Hq, Lq, D = q.shape
    o = _out_tensor(out, (B, Hq, Lq, v.shape[3]), q.dtype, q.device, "out")
    lse = _lse_tensor(lse, (B, Hq, Lq), q.device) if return_lse else None
    sq = _lengths(seqlens_q, B, q.device, "seqlens_q")
    sk = _lengths(seqlens_k, B, q.device, "seqlens_k")
    a = _make_args(q, k, v, o, scale, causal, mask, sinks, lse, sq, sk)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.sdpa_decode_noalloc(ctypes.byref(a), int(num_splits), ctypes.c_void_p(stream))
    if st != 0:
        _raise(st)
    return (o, lse) if return_lse else o


def prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     lse: torch.Tensor, dout: torch.Tensor, *, scale: Optional[float] = None,
                     causal: bool = False, mask: Optional[torch.Tensor] = None,
                     sinks: Optional[torch.Tensor] = None, seqlens_q=None, seqlens_k=None,
                     want_dsinks: bool = False, workspace: Optional[torch.Tensor] = None):
    """Gradients of prefill(q, k, v, ...) = o (with log-sum-exp ``lse``) for the
    upstream gradient ``dout``: returns (dq, dk, dv) or, with ``want_dsinks``,
    (dq, dk, dv, dsinks).  fp32 / fp16 / bf16 inputs, head dims (D of q, k; Dv of v)
    multiples of 8 up to 128."""
    lib = library()
    q, k, v, scale, mask, sinks = _common(q, k, v, scale, mask, sinks)
    for t, n in ((o, "o"), (dout, "dout"), (lse, "lse")):
        _on_device(t, n, q.device)
    o, dout = _prep(o, "o"), _prep(dout, "dout")
    B, Hq, Lq, D = q.shape
    oshape = (B, Hq, Lq, v.shape[3])
    if tuple(o.shape) != oshape or tuple(dout.shape) != oshape:
        raise ValueError(f"o and dout must be [B, Hq, Lq, Dv] = {oshape}")
    lse = lse.to(torch.float32).contiguous()
    if lse.shape != (B, Hq, Lq):
        raise ValueError(f"lse must be [B, Hq, Lq] = {(B, Hq, Lq)}, got {tuple(lse.shape)}")
    sq = _lengths(seqlens_q, B, q.device, "seqlens_q")
    sk = _lengths(seqlens_k, B, q.device, "seqlens_k")
    a = _make_args(q, k, v, o, scale, causal, mask, sinks, lse, sq, sk)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    ds = torch.empty(Hq, dtype=torch.float32, device=q.device) if (want_dsinks and sinks is not None) else None
    g = SdpaBwdArgs()
    for n, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(g, n, t.data_ptr())
        st = getattr(g, n + "_stride")
        for i in range(3):
            st[i] = t.stride(i)
    g.dsinks = ds.data_ptr() if ds is not None else None
    need = int(lib.sdpa_prefill_backward_workspace_bytes(ctypes.byref(a)))
    workspace = _workspace(workspace, need, q.device, min_bytes=16)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.sdpa_prefill_backward(ctypes.byref(a), ctypes.byref(g), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream))
    if st != 0:
        _raise(st)
    if want_dsinks:
        return dq, dk, dv, (ds if ds is not None else None)
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """prefill forward and its backward kernels as one autograd node."""

    @staticmethod
    def forward(ctx, q, k, v, sinks, scale, causal, mask, seqlens_q, seqlens_k):
        o, lse = prefill(q, k, v, scale=scale, causal=causal, mask=mask, sinks=sinks, return_lse=True,
                         seqlens_q=seqlens_q, seqlens_k=seqlens_k)
        ctx.save_for_backward(q, k, v, o, lse, sinks)
        ctx.opts = (scale, causal, mask, seqlens_q, seqlens_k)
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse, sinks = ctx.saved_tensors
        scale, causal, mask, sq, sk = ctx.opts
        want = sinks is not None and ctx.needs_input_grad[3]
        res = prefill_backward(q, k, v, o, lse, dout.contiguous(), scale=scale, causal=causal, mask=mask,
                               sinks=sinks, seqlens_q=sq, seqlens_k=sk, want_dsinks=want)
        dq, dk, dv = res[:3]
        ds = res[3] if want else None
        return dq, dk, dv, ds, None, None, None, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
              causal: bool = False, mask: Optional[torch.Tensor] = None,
              sinks: Optional[torch.Tensor] = None, seqlens_q=None, seqlens_k=None) -> torch.Tensor:
    """Differentiable fused attention: prefill() forward, prefill_backward()
    gradients for q, k, v and (fp32) sinks.  The mask is a constant."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _Attention.apply(q, k, v, sinks, scale, causal, mask, seqlens_q, seqlens_k)
