"""ctypes binding over ``libw4a16.so`` (the C ABI in ``include/w4a16.h``).

Argument marshalling only: tensors are passed as device pointers with the caller's
current HIP stream; every step of the computation runs in the library's HIP kernels.
The library is loaded on first use and a missing or unloadable library raises
:class:`W4A16Error`; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")

F16, BF16, F32 = 0, 1, 2
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, 1, 2, 3, 4

_lib = None
_workspaces = {}   # device index -> uint8 scratch tensor


class W4A16Error(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load ``libw4a16.so`` once; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise W4A16Error(f"{LIB_PATH} is missing: build it with "
                         "`python -m weight_only_int4_w4a16_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.w4a16_packed_bytes.argtypes = [i32, i32]
    L.w4a16_packed_bytes.restype = sz
    L.w4a16_pack.argtypes = [vp, i32, i32, vp, vp]
    L.w4a16_pack.restype = i32
    L.w4a16_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.w4a16_workspace_bytes.restype = sz
    L.w4a16_gemm.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, i32, vp, sz, vp]
    L.w4a16_gemm.restype = i32
    L.w4a16_gemm_nf4.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, i32, vp, sz, vp]
    L.w4a16_gemm_nf4.restype = i32
    L.w4a16_awq_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.w4a16_awq_workspace_bytes.restype = sz
    L.w4a16_gemm_awq.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, i32, vp, sz, vp]
    L.w4a16_gemm_awq.restype = i32
    L.w4a16_w4a8_workspace_bytes.argtypes = [i32, i32, i32]
    L.w4a16_w4a8_workspace_bytes.restype = sz
    L.w4a16_gemm_w4a8.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp]
    L.w4a16_gemm_w4a8.restype = i32
    L.w4a16_w4a8_kernel_name.argtypes = [i32, i32, i32]
    L.w4a16_w4a8_kernel_name.restype = ctypes.c_char_p
    L.w4a16_quantize_act_int8.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    L.w4a16_quantize_act_int8.restype = i32
    L.w4a16_gemm_swiglu.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, i32, vp, sz, vp]
    L.w4a16_gemm_swiglu.restype = i32
    L.w4a16_gemm_nf4_swiglu.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, i32, vp, sz, vp]
    L.w4a16_gemm_nf4_swiglu.restype = i32
    L.w4a16_dequant.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
    L.w4a16_dequant.restype = i32
    L.w4a16_dequant_nf4.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
    L.w4a16_dequant_nf4.restype = i32
    L.w4a16_kernel_name.argtypes = [i32, i32, i32, i32]
    L.w4a16_kernel_name.restype = ctypes.c_char_p
    L.w4a16_status_string.argtypes = [i32]
    L.w4a16_status_string.restype = ctypes.c_char_p
    L.w4a16_version.argtypes = []
    L.w4a16_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != OK:
        msg = lib().w4a16_status_string(status).decode()
        raise W4A16Error(f"{what}: {msg} (status {status})", status)


def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    m = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    if t not in m:
        raise W4A16Error(f"unsupported dtype {t}")
    return m[t]


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise W4A16Error("tensors must be contiguous device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def packed_bytes(K: int, N: int) -> int:
    return int(lib().w4a16_packed_bytes(K, N))


def workspace_bytes(M: int, K: int, N: int, group_size: int) -> int:
    return int(lib().w4a16_workspace_bytes(M, K, N, group_size))


def awq_workspace_bytes(M: int, K: int, N: int, group_size: int) -> int:
    return int(lib().w4a16_awq_workspace_bytes(M, K, N, group_size))


def _workspace(device, nbytes: int, workspace=None):
    """The caller's workspace, or a cached scratch buffer for the device.

    The library keeps nothing in a workspace between calls, so one buffer serves all calls
    that do not run concurrently; callers that launch GEMMs on several streams at
    once pass their own ``workspace`` per stream. It is never allocated while a HIP graph
    is being captured (warm up eagerly first).
    """
    torch = _torch()
    if workspace is not None:
        return workspace
    if nbytes == 0:
        return None
    key = device.index if device.index is not None else torch.cuda.current_device()
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise W4A16Error("workspace must be allocated before graph capture: run the same "
                             "calls once eagerly on this stream first", ERR_WORKSPACE)
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def pack(qweight):
    """Canonical ``qweight[K/8, N]`` int32 -> the library's device layout (int32 tensor)."""
    torch = _torch()
    if qweight.dtype != torch.int32 or qweight.dim() != 2:
        raise W4A16Error("qweight must be a 2-D int32 tensor [K/8, N]")
    K, N = qweight.shape[0] * 8, qweight.shape[1]
    nb = packed_bytes(K, N)
    if nb == 0:
        raise W4A16Error(f"unsupported shape K={K} N={N}", ERR_UNSUPPORTED)
    out = torch.empty(nb // 4, dtype=torch.int32, device=qweight.device)
    _check(lib().w4a16_pack(_ptr(qweight), K, N, _ptr(out), _stream(qweight)), "w4a16_pack")
    return out


def gemm(x, packed, scales, qzeros, group_size: int, out_dtype=None, out=None, workspace=None):
    """``y = x @ W_hat`` with affine (``qzeros`` given) or symmetric (``qzeros=None``) INT4.

    ``x[M, K]`` fp16/bf16, ``scales[K/g, N]`` in x's dtype, ``qzeros[K/g, N/8]`` int32.
    ``workspace``: optional uint8 device tensor of ``workspace_bytes(M, K, N, group_size)``.
    """
    torch = _torch()
    M, K = x.shape
    N = scales.shape[1]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if scales.dtype != x.dtype:
        raise W4A16Error("scales must have the activation dtype")
    ws = _workspace(x.device, workspace_bytes(M, K, N, group_size) if M else 0, workspace)
    st = lib().w4a16_gemm(_ptr(x), M, K, N, _dt(x.dtype), _ptr(packed), _ptr(scales),
                          _ptr(qzeros), group_size, _ptr(out), _dt(out.dtype), _ptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size(), _stream(x))
    _check(st, "w4a16_gemm")
    return out


def gemm_nf4(x, packed, absmax, codebook, block_size: int = 64, out_dtype=None, out=None,
             workspace=None):
    """``y = x @ W_hat`` with NF4 weights: fp16 ``absmax[K/b, N]``, fp16 ``codebook[16]``."""
    torch = _torch()
    M, K = x.shape
    N = absmax.shape[1]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if absmax.dtype != torch.float16 or codebook.dtype != torch.float16:
        raise W4A16Error("NF4 absmax and codebook are fp16")
    ws = _workspace(x.device, workspace_bytes(M, K, N, block_size) if M else 0, workspace)
    st = lib().w4a16_gemm_nf4(_ptr(x), M, K, N, _dt(x.dtype), _ptr(packed), _ptr(absmax),
                              _ptr(codebook), block_size, _ptr(out), _dt(out.dtype), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), _stream(x))
    _check(st, "w4a16_gemm_nf4")
    return out


def gemm_awq(x, s_inv, packed, scales, qzeros, group_size: int, out_dtype=None, out=None,
             workspace=None):
    """``y = RN(x * s_inv) @ W_hat``: the GEMM of AWQ-scaled activations, ``s_inv[K]`` the
    per-input-channel S^-1 in x's dtype, the weight the INT4 format of S W (as for
    :func:`gemm`). ``workspace``: optional, ``awq_workspace_bytes(M, K, N, group_size)``."""
    torch = _torch()
    M, K = x.shape
    N = scales.shape[1]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if scales.dtype != x.dtype or s_inv.dtype != x.dtype:
        raise W4A16Error("scales and s_inv must have the activation dtype")
    if s_inv.shape != (K,) or not s_inv.is_contiguous():
        raise W4A16Error("s_inv must be a contiguous (K,) tensor")
    ws = _workspace(x.device, awq_workspace_bytes(M, K, N, group_size) if M else 0, workspace)
    st = lib().w4a16_gemm_awq(_ptr(x), _ptr(s_inv), M, K, N, _dt(x.dtype), _ptr(packed),
                              _ptr(scales), _ptr(qzeros), group_size, _ptr(out), _dt(out.dtype),
                              _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(x))
    _check(st, "w4a16_gemm_awq")
    return out


def w4a8_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().w4a16_w4a8_workspace_bytes(M, K, N))


def gemm_w4a8(x, packed, wscale, out_dtype=None, out=None, workspace=None):
    """W4A8: ``y = sx * sw * (xq @ q)`` with x quantized per token to INT8 inside the call,
    symmetric INT4 codes (packed as for :func:`gemm` with ``qzeros=None``) and one scale per
    output channel ``wscale[N]`` in x's dtype."""
    torch = _torch()
    M, K = x.shape
    N = wscale.shape[-1]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if wscale.dtype != x.dtype or wscale.numel() != N or not wscale.is_contiguous():
        raise W4A16Error("wscale must be a contiguous (N,) tensor of the activation dtype")
    ws = _workspace(x.device, w4a8_workspace_bytes(M, K, N) if M else 0, workspace)
    st = lib().w4a16_gemm_w4a8(_ptr(x), M, K, N, _dt(x.dtype), _ptr(packed), _ptr(wscale),
                               _ptr(out), _dt(out.dtype), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream(x))
    _check(st, "w4a16_gemm_w4a8")
    return out


def w4a8_kernel_name(M: int, K: int, N: int) -> str:
    return lib().w4a16_w4a8_kernel_name(M, K, N).decode()


def quantize_act_int8(x):
    """The per-token INT8 quantization of the W4A8 path: ``(xq[M, K] int8, sx[M] float32)``."""
    torch = _torch()
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    sx = torch.empty((M,), dtype=torch.float32, device=x.device)
    st = lib().w4a16_quantize_act_int8(_ptr(x), M, K, _dt(x.dtype), _ptr(xq), _ptr(sx), _stream(x))
    _check(st, "w4a16_quantize_act_int8")
    return xq, sx


def gemm_swiglu(x, packed, scales, qzeros, group_size: int, out_dtype=None, out=None,
                workspace=None):
    """``h = SiLU(x @ W_gate) * (x @ W_up)`` for a fused gate+up weight ``[K, N2]`` (gate
    columns first; ``scales[K/g, N2]``, ``qzeros[K/g, N2/8]`` or None); ``h[M, N2/2]``."""
    torch = _torch()
    M, K = x.shape
    N2 = scales.shape[1]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((M, N2 // 2), dtype=out_dtype, device=x.device)
    if scales.dtype != x.dtype:
        raise W4A16Error("scales must have the activation dtype")
    ws = _workspace(x.device, workspace_bytes(M, K, N2, group_size) if M else 0, workspace)
    st = lib().w4a16_gemm_swiglu(_ptr(x), M, K, N2, _dt(x.dtype), _ptr(packed), _ptr(scales),
                                 _ptr(qzeros), group_size, _ptr(out), _dt(out.dtype), _ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(), _stream(x))
    _check(st, "w4a16_gemm_swiglu")
    return out


def gemm_nf4_swiglu(x, packed, absmax, codebook, block_size: int = 64, out_dtype=None, out=None,
                    workspace=None):
    """NF4 counterpart of :func:`gemm_swiglu`."""
    torch = _torch()
    M, K = x.shape
    N2 = absmax.shape[1]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((M, N2 // 2), dtype=out_dtype, device=x.device)
    if absmax.dtype != torch.float16 or codebook.dtype != torch.float16:
        raise W4A16Error("NF4 absmax and codebook are fp16")
    ws = _workspace(x.device, workspace_bytes(M, K, N2, block_size) if M else 0, workspace)
    st = lib().w4a16_gemm_nf4_swiglu(_ptr(x), M, K, N2, _dt(x.dtype), _ptr(packed), _ptr(absmax),
                                     _ptr(codebook), block_size, _ptr(out), _dt(out.dtype),
                                     _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(x))
    _check(st, "w4a16_gemm_nf4_swiglu")
    return out


def dequant(packed, scales, qzeros, K: int, group_size: int):
    """Test hook: W_hat[K, N] in the scales' dtype, from the GEMM's own dequant routine."""
    torch = _torch()
    N = scales.shape[1]
    w = torch.empty((K, N), dtype=scales.dtype, device=scales.device)
    st = lib().w4a16_dequant(_ptr(packed), _ptr(scales), _ptr(qzeros), K, N, group_size,
                             _dt(scales.dtype), _ptr(w), _stream(scales))
    _check(st, "w4a16_dequant")
    return w


def dequant_nf4(packed, absmax, codebook, K: int, block_size: int = 64, wdtype=None):
    """Test hook: NF4 W_hat[K, N] (fp16 by default, or bf16)."""
    torch = _torch()
    N = absmax.shape[1]
    wdtype = torch.float16 if wdtype is None else wdtype
    w = torch.empty((K, N), dtype=wdtype, device=absmax.device)
    st = lib().w4a16_dequant_nf4(_ptr(packed), _ptr(absmax), _ptr(codebook), K, N, block_size,
                                 _dt(wdtype), _ptr(w), _stream(absmax))
    _check(st, "w4a16_dequant_nf4")
    return w


def kernel_name(M: int, K: int, N: int, group_size: int) -> str:
    return lib().w4a16_kernel_name(M, K, N, group_size).decode()


def version() -> str:
    return lib().w4a16_version().decode()
