"""gfx950 FlashAttention forward -- Python binding of libattn.so.

The binding only marshals arguments: it takes device pointers and the current
torch stream from torch tensors and calls the C ABI declared in
``include/attn.h``.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  When libattn.so is missing (not built) any call
raises, naming the build command.

    from attention_forward_amd import attn_fwd
    o, lse = attn_fwd(q, k, v, causal=True)          # q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d]
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

# status codes (include/attn.h)
ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_UNSUPPORTED = 3
ATTN_ERR_ALIGN = 4
ATTN_ERR_WORKSPACE = 5
ATTN_ERR_NO_DEVICE = 6
ATTN_ERR_HIP = 7
ATTN_ERR_VALUE = 8
ATTN_F16 = 0
ATTN_BF16 = 1

EXPORTED = ("attn_fwd", "attn_fwd_fp8", "attn_fwd_split", "attn_fwd_split_workspace_bytes", "attn_fwd_num_splits",
            "attn_decode_workspace_bytes", "attn_fwd_decode", "attn_fwd_decode_noalloc",
            "attn_decode_scratch_bytes", "attn_splitkv_combine", "attn_last_error")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("attn status %d: %s" % (status, message))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libattn.so (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libattn.so is not built; run `python -m attention_forward_amd.build` "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, f, f, f, i, vp]
    L.attn_fwd_fp8.restype = i
    L.attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.attn_fwd_split.restype = i
    L.attn_fwd_split_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_fwd_split_workspace_bytes.restype = sz
    L.attn_fwd_num_splits.argtypes = [i, i, i, i, i]
    L.attn_fwd_num_splits.restype = i
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.attn_fwd_decode.restype = i
    L.attn_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd_decode_noalloc.restype = i
    L.attn_decode_scratch_bytes.argtypes = []
    L.attn_decode_scratch_bytes.restype = sz
    L.attn_splitkv_combine.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    L.attn_splitkv_combine.restype = i
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def last_error() -> str:
    return lib().attn_last_error().decode()


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, last_error())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise AttnError(ATTN_ERR_UNSUPPORTED, "dtype %s (fp16 or bf16 only)" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _validate(*specs):
    """Check tensor arguments before anything is launched.  Each spec is
    (tensor or None, name, shape or None, dtypes or None).  First every shape
    and dtype, then that all tensors sit on the first one's GPU and are
    contiguous; so host tensors are also rejected with the precise reason.  The
    C ABI only sees pointers, so this is the only guard against a wrongly sized
    buffer."""
    specs = [s for s in specs if s[0] is not None]
    for t, name, shape, dtypes in specs:
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise AttnError(ATTN_ERR_SHAPE, "%s has shape %s, expected %s"
                            % (name, tuple(t.shape), tuple(shape)))
        if dtypes is not None and t.dtype not in dtypes:
            raise AttnError(ATTN_ERR_UNSUPPORTED, "%s has dtype %s, expected %s"
                            % (name, t.dtype, " or ".join(str(x) for x in dtypes)))
    dev = specs[0][0].device
    for t, name, _, _ in specs:
        if t.device != dev:
            raise AttnError(ATTN_ERR_VALUE, "%s is on %s, expected %s" % (name, t.device, dev))
        if not t.is_cuda:
            raise AttnError(ATTN_ERR_VALUE, "%s must be a device tensor" % name)
        if not t.is_contiguous():
            raise AttnError(ATTN_ERR_VALUE, "%s must be contiguous" % name)


def _rank(t, name, n):
    if t.dim() != n:
        raise AttnError(ATTN_ERR_SHAPE, "%s must have %d dimensions, has shape %s"
                        % (name, n, tuple(t.shape)))


def _qkv_shapes(q, k, v):
    """q [B,Hq,Sq,d], k and v [B,Hkv,Sk,d] with one B and d; returns
    (B, Hq, Sq, d, Hkv, Sk)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _rank(t, nm, 4)
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise AttnError(ATTN_ERR_SHAPE, "q %s / k %s / v %s shapes disagree"
                        % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    return B, Hq, Sq, d, Hkv, Sk


def _workspace_size(ws, need):
    if ws is not None and ws.numel() * ws.element_size() < need:
        raise AttnError(ATTN_ERR_WORKSPACE, "workspace of %d bytes needed, %d given"
                        % (need, ws.numel() * ws.element_size()))


def _torch_dtypes():
    import torch

    return (torch.float16, torch.bfloat16)


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
             want_lse: bool = True):
    """O = softmax(scale * Q K^T [causal]) V per (batch, head); returns (o, lse).

    q [B,Hq,Sq,d], k and v [B,Hkv,Sk,d], contiguous fp16/bf16 device tensors.
    lse is fp32 [B,Hq,Sq] (None when want_lse is False).  Runs on the current
    torch stream; returns without waiting for the kernel.  A caller-supplied
    out must match q in shape, dtype and device, lse be fp32 [B,Hq,Sq].
    """
    import torch

    B, Hq, Sq, d, Hkv, Sk = _qkv_shapes(q, k, v)
    _validate((q, "q", None, _torch_dtypes()), (k, "k", None, (q.dtype,)),
              (v, "v", None, (q.dtype,)), (out, "out", q.shape, (q.dtype,)),
              (lse, "lse", (B, Hq, Sq), (torch.float32,)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, d,
                        1 if causal else 0, float(scale), _dtype_code(q), _stream(q.device))
    _check(st)
    return out, lse


def attn_fwd_fp8(q, k, v, causal: bool = False, scale: float | None = None,
                 q_descale: float = 1.0, k_descale: float = 1.0, v_descale: float = 1.0,
                 out_dtype=None, out=None, lse=None, want_lse: bool = True):
    """FP8 prefill: q [B,Hq,Sq,128], k and v [B,Hkv,Sk,128] contiguous E4M3 device
    tensors (torch.float8_e4m3fn or uint8 bytes) holding the inputs divided by
    their per-tensor descales.  Returns (o in out_dtype (bf16 default), lse fp32)."""
    import torch

    B, Hq, Sq, d, Hkv, Sk = _qkv_shapes(q, k, v)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in _torch_dtypes():
        raise AttnError(ATTN_ERR_UNSUPPORTED, "output dtype %s (fp16 or bf16 only)" % out_dtype)
    e4m3 = (torch.float8_e4m3fn, torch.uint8)
    _validate((q, "q", None, e4m3), (k, "k", None, e4m3), (v, "v", None, e4m3),
              (out, "out", (B, Hq, Sq, d), (out_dtype,)),
              (lse, "lse", (B, Hq, Sq), (torch.float32,)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = ATTN_F16 if out_dtype == torch.float16 else ATTN_BF16
    if out is None:
        out = torch.empty((B, Hq, Sq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    st = lib().attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk,
                            d, 1 if causal else 0, float(scale), float(q_descale),
                            float(k_descale), float(v_descale), code, _stream(q.device))
    _check(st)
    return out, lse


def attn_fwd_num_splits(B: int, Hq: int, Sq: int, Sk: int, d: int) -> int:
    return int(lib().attn_fwd_num_splits(B, Hq, Sq, Sk, d))


def attn_fwd_split_workspace_bytes(B: int, Hq: int, Sq: int, d: int, num_splits: int) -> int:
    return int(lib().attn_fwd_split_workspace_bytes(B, Hq, Sq, d, num_splits))


def attn_fwd_split(q, k, v, num_splits: int | None = None, causal: bool = False,
                   scale: float | None = None, out=None, lse=None, workspace=None,
                   want_lse: bool = True):
    """Split-KV prefill: attn_fwd's result from num_splits key ranges merged by LSE.

    num_splits defaults to attn_fwd_num_splits(...).  `workspace` (a device
    tensor of at least attn_fwd_split_workspace_bytes bytes) is allocated when
    omitted.  Returns (o, lse) like attn_fwd.
    """
    import torch

    B, Hq, Sq, d, Hkv, Sk = _qkv_shapes(q, k, v)
    _validate((q, "q", None, _torch_dtypes()), (k, "k", None, (q.dtype,)),
              (v, "v", None, (q.dtype,)), (out, "out", q.shape, (q.dtype,)),
              (lse, "lse", (B, Hq, Sq), (torch.float32,)), (workspace, "workspace", None, None))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = attn_fwd_num_splits(B, Hq, Sq, Sk, d)
    need = attn_fwd_split_workspace_bytes(B, Hq, Sq, d, num_splits)
    _workspace_size(workspace, need)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    st = lib().attn_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk,
                              d, 1 if causal else 0, float(scale), _dtype_code(q), int(num_splits),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(q.device))
    _check(st)
    return out, lse


def attn_decode_workspace_bytes(B: int, Hq: int, d: int, num_splits: int) -> int:
    return int(lib().attn_decode_workspace_bytes(B, Hq, d, num_splits))


def attn_fwd_decode(q, k, v, num_splits: int, scale: float | None = None, out=None, lse=None,
                    workspace=None, want_lse: bool = True):
    """Single-token decode with split-KV; q [B,Hq,1,d], k/v [B,Hkv,Sk,d].

    Returns (o [B,Hq,1,d], lse [B,Hq] fp32).  `workspace` (a device tensor of
    at least attn_decode_workspace_bytes bytes) is allocated when omitted.
    """
    import torch

    B, Hq, Sq, d, Hkv, Sk = _qkv_shapes(q, k, v)
    if Sq != 1:
        raise AttnError(ATTN_ERR_SHAPE, "decode takes one query row (Sq = 1), got %d" % Sq)
    _validate((q, "q", None, _torch_dtypes()), (k, "k", None, (q.dtype,)),
              (v, "v", None, (q.dtype,)), (out, "out", q.shape, (q.dtype,)),
              (lse, "lse", (B, Hq), (torch.float32,)), (workspace, "workspace", None, None))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_decode_workspace_bytes(B, Hq, d, num_splits)
    _workspace_size(workspace, need)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib().attn_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sk, d,
                               float(scale), _dtype_code(q), int(num_splits), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st)
    return out, lse


def attn_decode_scratch_bytes() -> int:
    return int(lib().attn_decode_scratch_bytes())


def attn_fwd_decode_noalloc(q, k, v, num_splits: int, out, lse=None, scale: float | None = None):
    """attn_fwd_decode with the split partials in the library's own per-GPU
    scratch: no workspace and no allocation, for callers that cannot allocate
    (graph capture, allocation-free loops).  `out` ([B,Hq,1,d], q's dtype) is
    required and `lse` (fp32 [B,Hq]) optional, both supplied by the caller.
    Calls that overlap on one GPU share the scratch and race."""
    import torch

    B, Hq, Sq, d, Hkv, Sk = _qkv_shapes(q, k, v)
    if Sq != 1:
        raise AttnError(ATTN_ERR_SHAPE, "decode takes one query row (Sq = 1), got %d" % Sq)
    if out is None:
        raise AttnError(ATTN_ERR_NULL, "attn_fwd_decode_noalloc needs the output buffer")
    _validate((q, "q", None, _torch_dtypes()), (k, "k", None, (q.dtype,)),
              (v, "v", None, (q.dtype,)), (out, "out", q.shape, (q.dtype,)),
              (lse, "lse", (B, Hq), (torch.float32,)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().attn_fwd_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq,
                                       Hkv, Sk, d, float(scale), _dtype_code(q), int(num_splits),
                                       _stream(q.device))
    _check(st)
    return out, lse


def attn_splitkv_combine(o_part, lse_part, dtype, out=None, lse=None, want_lse: bool = True):
    """Merge fp32 partials o_part [B,Hq,S,d] / lse_part [B,Hq,S] -> (o [B,Hq,d], lse [B,Hq])."""
    import torch

    _rank(o_part, "o_part", 4)
    B, Hq, S, d = o_part.shape
    if dtype not in _torch_dtypes():
        raise AttnError(ATTN_ERR_UNSUPPORTED, "output dtype %s (fp16 or bf16 only)" % dtype)
    _validate((o_part, "o_part", None, (torch.float32,)),
              (lse_part, "lse_part", (B, Hq, S), (torch.float32,)),
              (out, "out", (B, Hq, d), (dtype,)), (lse, "lse", (B, Hq), (torch.float32,)))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=dtype, device=o_part.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=o_part.device)
    code = ATTN_F16 if dtype == torch.float16 else ATTN_BF16
    st = lib().attn_splitkv_combine(_ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse), B, Hq, d,
                                    S, code, _stream(o_part.device))
    _check(st)
    return out, lse
