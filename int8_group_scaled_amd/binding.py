"""ctypes binding of libi8gs (include/i8gs.h): argument marshalling only.

Each function takes torch tensors that live on the current HIP device, checks
dtype / device / contiguity, passes raw pointers and the current stream to the
C ABI entry point of the same name, and maps status codes to exceptions
(ValueError for argument and shape errors, RuntimeError for HIP / device errors,
carrying i8gs_last_error()).  Every step of the computation runs in the HIP
kernels; there is no CPU or PyTorch fallback.  Workspaces are allocated here,
through PyTorch, zero-filled once as the library requires, and cached per
(device, stream).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libi8gs.so")

I8GS_OK = 0
I8GS_ERR_INVALID_ARG = 1
I8GS_ERR_UNSUPPORTED_SHAPE = 2
I8GS_ERR_MISALIGNED = 3
I8GS_ERR_WORKSPACE = 4
I8GS_ERR_HIP = 5
I8GS_ERR_UNSUPPORTED_DEVICE = 6
OP_W8A8 = 0
OP_W4A16 = 1
OP_WEIGHT_ONLY = 2
KERNEL_AUTO = 0
KERNEL_DECODE = 1
KERNEL_TILED = 2

# Every symbol include/i8gs.h declares.
EXPORTS = (
    "i8gs_abi_version", "i8gs_last_error", "i8gs_status_string", "quant_act_per_token",
    "i8gs_workspace_bytes", "i8gs_workspace_bytes_ex", "gemm_w8a8_g128", "gemm_w8a8_g128_ex",
    "gemm_w8a8_g128_group_partials", "gemm_w8a8_g128_group_partials_ex", "gemm_w4a16_g128", "gptq_unpack",
    "gptq_quantize_rtn", "gemm_w8a8_g128_noalloc", "i8gs_noalloc_scratch_bytes", "gemm_weight_only",
    "gptq_quantize_rtn_group", "rmsnorm_quant_per_token", "kv_quant_int8_block128", "attn_qk_int8",
    "attn_pv_int8", "attn_pv_int8_workspace_bytes",
)

_lib = None


class I8GSError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class I8GSValueError(ValueError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libi8gs.so (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                          "(hipcc, gfx950). The HIP library is required; there is no fallback path.")
    lib = ctypes.CDLL(path)
    P, I64, I, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.i8gs_abi_version.restype = I
    lib.i8gs_last_error.restype = ctypes.c_char_p
    lib.i8gs_status_string.restype = ctypes.c_char_p
    lib.i8gs_status_string.argtypes = [I]
    lib.quant_act_per_token.argtypes = [P, I64, I64, I64, P, P, P]
    lib.i8gs_workspace_bytes.argtypes = [I, I64, I64, I64]
    lib.i8gs_workspace_bytes.restype = S
    lib.i8gs_workspace_bytes_ex.argtypes = [I, I64, I64, I64, I, I]
    lib.i8gs_workspace_bytes_ex.restype = S
    lib.gemm_w8a8_g128.argtypes = [P, I64, P, P, P, P, P, I64, I64, I64, I64, P, S, P]
    lib.gemm_w8a8_g128_ex.argtypes = [P, I64, P, P, P, P, P, I64, I64, I64, I64, I, I, P, S, P]
    lib.gemm_w8a8_g128_group_partials.argtypes = [P, P, P, I64, I64, I64, P]
    lib.gemm_w8a8_g128_group_partials_ex.argtypes = [P, P, P, I64, I64, I64, I, I, P]
    lib.gemm_w4a16_g128.argtypes = [P, I64, P, P, P, I64, I64, I64, I64, P, S, P]
    lib.gemm_w8a8_g128_noalloc.argtypes = [P, I64, P, P, P, P, P, I64, I64, I64, I64, P]
    lib.gemm_weight_only.argtypes = [P, I64, P, I, P, I, P, I64, I64, I64, I64, P, S, P]
    lib.gptq_quantize_rtn_group.argtypes = [P, I, I, I64, I64, P, P, P]
    lib.rmsnorm_quant_per_token.argtypes = [P, I64, P, ctypes.c_float, I64, I64, P, P, P, P]
    lib.i8gs_noalloc_scratch_bytes.restype = S
    lib.kv_quant_int8_block128.argtypes = [P, I64, I64, I64, P, P, P]
    lib.attn_qk_int8.argtypes = [P, P, P, P, ctypes.c_float, I64, I64, I64, I64, P, P, P]
    lib.attn_pv_int8.argtypes = [P, P, P, I64, I64, I64, I64, P, P, P, P, S, P]
    lib.attn_pv_int8_workspace_bytes.argtypes = [I64, I64, I64, I64]
    lib.attn_pv_int8_workspace_bytes.restype = S
    lib.gptq_unpack.argtypes = [P, P, I, I64, I64, P, P, P]
    lib.gptq_quantize_rtn.argtypes = [P, I, I64, I64, P, P, P]
    for name in ("quant_act_per_token", "gemm_w8a8_g128", "gemm_w8a8_g128_ex", "gemm_w8a8_g128_group_partials",
                 "gemm_w8a8_g128_group_partials_ex", "gemm_w4a16_g128", "gptq_unpack", "gptq_quantize_rtn",
                 "gemm_w8a8_g128_noalloc", "gemm_weight_only", "gptq_quantize_rtn_group",
                 "rmsnorm_quant_per_token", "kv_quant_int8_block128", "attn_qk_int8", "attn_pv_int8"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().i8gs_abi_version())


def last_error() -> str:
    return load_library().i8gs_last_error().decode()


def _raise(status: int) -> None:
    if status == I8GS_OK:
        return
    msg = last_error()
    if status in (I8GS_ERR_HIP, I8GS_ERR_UNSUPPORTED_DEVICE):
        raise I8GSError(status, msg)
    raise I8GSValueError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, dims: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {tuple(t.shape)}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} rows must be contiguous")


_workspaces: dict = {}


def _workspace(device: torch.device, nbytes: int) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def workspace_bytes(op: int, M: int, N: int, K: int, kernel: int = KERNEL_AUTO, decode_workgroups: int = 0) -> int:
    n = load_library().i8gs_workspace_bytes_ex(op, M, N, K, kernel, decode_workgroups)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError(f"invalid workspace query op={op} M={M} N={N} K={K} kernel={kernel} "
                         f"decode_workgroups={decode_workgroups}")
    return int(n)


def quant_act_per_token(x: torch.Tensor, qa: Optional[torch.Tensor] = None,
                        a_scale: Optional[torch.Tensor] = None):
    """Per-token INT8 quantisation of bf16 x [M, K] -> (qa int8 [M, K], a_scale fp32 [M])."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if qa is None:
        qa = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if a_scale is None:
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _need(qa, "qa", torch.int8, 2)
    if not qa.is_contiguous() or tuple(qa.shape) != (M, K):
        raise ValueError("qa must be a contiguous [M, K] int8 tensor")
    if not a_scale.is_contiguous() or tuple(a_scale.shape) != (M,) or a_scale.dtype != torch.float32:
        raise ValueError("a_scale must be a contiguous [M] float32 tensor")
    _raise(load_library().quant_act_per_token(_ptr(x), x.stride(0), M, K, _ptr(qa), _ptr(a_scale),
                                              _stream(x.device)))
    return qa, a_scale


def gemm_w8a8_g128_ex(qweight: torch.Tensor, w_scale: torch.Tensor, x: Optional[torch.Tensor] = None,
                      qa: Optional[torch.Tensor] = None, a_scale: Optional[torch.Tensor] = None,
                      y: Optional[torch.Tensor] = None, kernel: int = KERNEL_AUTO,
                      decode_workgroups: int = 0) -> torch.Tensor:
    """W8A8 G128 linear from bf16 x [M, K] or from (qa, a_scale); qweight int32 [K/4, N],
    w_scale fp32 [K/128, N] -> y bf16 [M, N]."""
    _need(qweight, "qweight", torch.int32, 2)
    _need(w_scale, "w_scale", torch.float32, 2)
    if not qweight.is_contiguous() or not w_scale.is_contiguous():
        raise ValueError("qweight and w_scale must be contiguous")
    K = qweight.shape[0] * 4
    N = qweight.shape[1]
    if tuple(w_scale.shape) != (K // 128, N):
        raise ValueError(f"w_scale must be [{K // 128}, {N}], got {tuple(w_scale.shape)}")
    if x is not None:
        _need(x, "x", torch.bfloat16, 2)
        M = x.shape[0]
        if x.shape[1] != K:
            raise ValueError(f"x must have K={K} columns, got {x.shape[1]}")
        ldx = x.stride(0)
        dev = x.device
    else:
        if qa is None or a_scale is None:
            raise ValueError("give x, or both qa and a_scale")
        _need(qa, "qa", torch.int8, 2)
        if not qa.is_contiguous() or qa.shape[1] != K:
            raise ValueError(f"qa must be contiguous [M, {K}]")
        M = qa.shape[0]
        if a_scale.dtype != torch.float32 or tuple(a_scale.shape) != (M,) or not a_scale.is_contiguous():
            raise ValueError("a_scale must be a contiguous [M] float32 tensor")
        ldx = 0
        dev = qa.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be [{M}, {N}]")
    nbytes = workspace_bytes(OP_W8A8, M, N, K, kernel, decode_workgroups)
    ws = _workspace(dev, nbytes)
    _raise(load_library().gemm_w8a8_g128_ex(_ptr(x), ldx, _ptr(qa), _ptr(a_scale), _ptr(qweight), _ptr(w_scale),
                                            _ptr(y), y.stride(0), M, N, K, kernel, decode_workgroups, _ptr(ws),
                                            0 if ws is None else ws.numel(), _stream(dev)))
    return y


def gemm_w8a8_g128_noalloc(qweight: torch.Tensor, w_scale: torch.Tensor, y: torch.Tensor,
                           x: Optional[torch.Tensor] = None, qa: Optional[torch.Tensor] = None,
                           a_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gemm_w8a8_g128 through the entry point that allocates nothing (its scratch memory is a
    static device array of the library); y must be given."""
    _need(qweight, "qweight", torch.int32, 2)
    _need(w_scale, "w_scale", torch.float32, 2)
    _need(y, "y", torch.bfloat16, 2)
    K = qweight.shape[0] * 4
    N = qweight.shape[1]
    if x is not None:
        _need(x, "x", torch.bfloat16, 2)
        M, ldx, dev = x.shape[0], x.stride(0), x.device
    else:
        if qa is None or a_scale is None:
            raise ValueError("give x, or both qa and a_scale")
        _need(qa, "qa", torch.int8, 2)
        M, ldx, dev = qa.shape[0], 0, qa.device
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be [{M}, {N}]")
    _raise(load_library().gemm_w8a8_g128_noalloc(_ptr(x), ldx, _ptr(qa), _ptr(a_scale), _ptr(qweight),
                                                 _ptr(w_scale), _ptr(y), y.stride(0), M, N, K, _stream(dev)))
    return y


def noalloc_scratch_bytes() -> int:
    return int(load_library().i8gs_noalloc_scratch_bytes())


def gemm_w8a8_g128(qweight, w_scale, x=None, qa=None, a_scale=None, y=None) -> torch.Tensor:
    """W8A8 G128 linear with the library's own kernel choice (see gemm_w8a8_g128_ex)."""
    return gemm_w8a8_g128_ex(qweight, w_scale, x=x, qa=qa, a_scale=a_scale, y=y)


def gemm_w8a8_g128_group_partials(qa: torch.Tensor, qweight: torch.Tensor, kernel: int = KERNEL_AUTO,
                                  decode_workgroups: int = 0) -> torch.Tensor:
    """int32 P [M, K/128, N] of per-group integer dot products, from the kernel and plan
    gemm_w8a8_g128_ex would use with the same kernel / workgroup choice."""
    _need(qa, "qa", torch.int8, 2)
    _need(qweight, "qweight", torch.int32, 2)
    if not qa.is_contiguous() or not qweight.is_contiguous():
        raise ValueError("qa and qweight must be contiguous")
    M, K = qa.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 4 != K:
        raise ValueError("qweight rows must be K/4")
    P = torch.empty((M, K // 128, N), dtype=torch.int32, device=qa.device)
    _raise(load_library().gemm_w8a8_g128_group_partials_ex(_ptr(qa), _ptr(qweight), _ptr(P), M, N, K, kernel,
                                                           decode_workgroups, _stream(qa.device)))
    return P


def gemm_w4a16_g128(x: torch.Tensor, qweight: torch.Tensor, w_scale: torch.Tensor,
                    y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W4A16 g128 linear: bf16 x [M, K], qweight int32 [K/8, N], w_scale fp32 [K/128, N] -> bf16 [M, N]."""
    _need(x, "x", torch.bfloat16, 2)
    _need(qweight, "qweight", torch.int32, 2)
    _need(w_scale, "w_scale", torch.float32, 2)
    if not qweight.is_contiguous() or not w_scale.is_contiguous():
        raise ValueError("qweight and w_scale must be contiguous")
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K or tuple(w_scale.shape) != (K // 128, N):
        raise ValueError("qweight must be [K/8, N] and w_scale [K/128, N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, 2)
    ws = _workspace(x.device, workspace_bytes(OP_W4A16, M, N, K))
    _raise(load_library().gemm_w4a16_g128(_ptr(x), x.stride(0), _ptr(qweight), _ptr(w_scale), _ptr(y), y.stride(0),
                                          M, N, K, _ptr(ws), 0 if ws is None else ws.numel(), _stream(x.device)))
    return y


def gptq_unpack(qweight: torch.Tensor, bits: int, w_scale: Optional[torch.Tensor] = None,
                want_codes: bool = True, want_dequant: bool = False):
    """Codes int8 [K, N] and/or dequantised fp32 [K, N] from GPTQ int32 words."""
    _need(qweight, "qweight", torch.int32, 2)
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    K = qweight.shape[0] * (32 // bits)
    N = qweight.shape[1]
    q = torch.empty((K, N), dtype=torch.int8, device=qweight.device) if want_codes else None
    w = torch.empty((K, N), dtype=torch.float32, device=qweight.device) if want_dequant else None
    if want_dequant:
        _need(w_scale, "w_scale", torch.float32, 2)
    _raise(load_library().gptq_unpack(_ptr(qweight), _ptr(w_scale), bits, K, N, _ptr(q), _ptr(w),
                                      _stream(qweight.device)))
    return q, w


def gptq_quantize_rtn(w: torch.Tensor, bits: int):
    """RTN G128 symmetric quantisation of fp32 w [K, N] -> (qweight int32, w_scale fp32)."""
    _need(w, "w", torch.float32, 2)
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    K, N = w.shape
    qw = torch.empty((K // (32 // bits), N), dtype=torch.int32, device=w.device)
    ws = torch.empty((K // 128, N), dtype=torch.float32, device=w.device)
    _raise(load_library().gptq_quantize_rtn(_ptr(w), bits, K, N, _ptr(qw), _ptr(ws), _stream(w.device)))
    return qw, ws


def gemm_weight_only(x: torch.Tensor, qweight: torch.Tensor, w_scale: torch.Tensor, bits: int, group: int,
                     y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Weight-only linear: bf16 x [M, K], qweight int32 [K/(32/bits), N], w_scale fp32 [K/group, N]
    -> bf16 [M, N] (4-bit group 128, 8-bit group 32 or 128)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(qweight, "qweight", torch.int32, 2)
    _need(w_scale, "w_scale", torch.float32, 2)
    if not qweight.is_contiguous() or not w_scale.is_contiguous():
        raise ValueError("qweight and w_scale must be contiguous")
    M, K = x.shape
    N = qweight.shape[1]
    if bits not in (4, 8) or qweight.shape[0] * (32 // bits) != K or tuple(w_scale.shape) != (K // group, N):
        raise ValueError(f"qweight must be [K/{32 // max(bits, 1)}, N] and w_scale [K/{group}, N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, 2)
    ws = _workspace(x.device, workspace_bytes(OP_WEIGHT_ONLY, M, N, K))
    _raise(load_library().gemm_weight_only(_ptr(x), x.stride(0), _ptr(qweight), bits, _ptr(w_scale), group, _ptr(y),
                                           y.stride(0), M, N, K, _ptr(ws), 0 if ws is None else ws.numel(),
                                           _stream(x.device)))
    return y


def gptq_quantize_rtn_group(w: torch.Tensor, bits: int, group: int):
    """RTN symmetric quantisation of fp32 w [K, N] with `group` K values per scale ->
    (qweight int32 [K/(32/bits), N], w_scale fp32 [K/group, N])."""
    _need(w, "w", torch.float32, 2)
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    K, N = w.shape
    qw = torch.empty((K // (32 // bits), N), dtype=torch.int32, device=w.device)
    ws = torch.empty((K // group, N), dtype=torch.float32, device=w.device)
    _raise(load_library().gptq_quantize_rtn_group(_ptr(w), bits, group, K, N, _ptr(qw), _ptr(ws),
                                                  _stream(w.device)))
    return qw, ws


def rmsnorm_quant_per_token(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, want_h: bool = False,
                            qa: Optional[torch.Tensor] = None, a_scale: Optional[torch.Tensor] = None):
    """RMS normalisation of bf16 x [M, K] with bf16 gamma [K], fused with the per-token INT8
    quantisation of its output -> (qa int8 [M, K], a_scale fp32 [M], h bf16 [M, K] or None)."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if gamma.dtype != torch.bfloat16 or tuple(gamma.shape) != (K,) or not gamma.is_contiguous() or not gamma.is_cuda:
        raise ValueError("gamma must be a contiguous bf16 [K] tensor on the GPU")
    if qa is None:
        qa = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if a_scale is None:
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    h = torch.empty((M, K), dtype=torch.bfloat16, device=x.device) if want_h else None
    _raise(load_library().rmsnorm_quant_per_token(_ptr(x), x.stride(0), _ptr(gamma), float(eps), M, K, _ptr(h),
                                                  _ptr(qa), _ptr(a_scale), _stream(x.device)))
    return qa, a_scale, h


def _need_c(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous() \
            or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on the GPU")


def kv_quant_int8_block128(kv: torch.Tensor, heads: Optional[int] = None, codes: Optional[torch.Tensor] = None,
                           scales: Optional[torch.Tensor] = None):
    """INT8 block-g128 codec of a KV slice: bf16 kv [T, H, 128] (contiguous), or bf16
    [T, >= 128*heads] whose first 128*heads values per row are the H head vectors (e.g.
    a column slice of a fused qkv output) -> (codes int8 [T, H, 128], scales fp32 [T, H])."""
    if not isinstance(kv, torch.Tensor) or kv.dtype != torch.bfloat16 or not kv.is_cuda:
        raise ValueError("kv must be a bf16 tensor on the GPU")
    if kv.dim() == 3:
        if kv.shape[2] != 128 or kv.stride(2) != 1 or kv.stride(1) != 128:
            raise ValueError("kv [T, H, 128] must have contiguous head vectors")
        T, H, ld = kv.shape[0], kv.shape[1], kv.stride(0)
    elif kv.dim() == 2:
        if heads is None or kv.stride(1) != 1 or kv.shape[1] < 128 * heads:
            raise ValueError("a 2-D kv needs heads and rows of at least 128*heads contiguous values")
        T, H, ld = kv.shape[0], int(heads), kv.stride(0)
    else:
        raise ValueError("kv must be [T, H, 128] or [T, 128*H]")
    if codes is None:
        codes = torch.empty((T, H, 128), dtype=torch.int8, device=kv.device)
    if scales is None:
        scales = torch.empty((T, H), dtype=torch.float32, device=kv.device)
    _need_c(codes, "codes", torch.int8, (T, H, 128))
    _need_c(scales, "scales", torch.float32, (T, H))
    _raise(load_library().kv_quant_int8_block128(_ptr(kv), ld, T, H, _ptr(codes), _ptr(scales), _stream(kv.device)))
    return codes, scales


def attn_qk_int8(qq: torch.Tensor, qs: torch.Tensor, kq: torch.Tensor, ks: torch.Tensor, scale: float,
                 want_dots: bool = False, s: Optional[torch.Tensor] = None):
    """INT8 QK scores on the block-g128 cache: qq int8 [Mq, Hq, 128], qs fp32 [Mq, Hq],
    kq int8 [T, Hkv, 128], ks fp32 [T, Hkv] -> (s fp32 [Hq, Mq, T], dots int32 or None)."""
    if qq.dim() != 3 or kq.dim() != 3:
        raise ValueError("qq and kq must be [rows, heads, 128]")
    Mq, Hq, T, Hkv = qq.shape[0], qq.shape[1], kq.shape[0], kq.shape[1]
    _need_c(qq, "qq", torch.int8, (Mq, Hq, 128))
    _need_c(qs, "qs", torch.float32, (Mq, Hq))
    _need_c(kq, "kq", torch.int8, (T, Hkv, 128))
    _need_c(ks, "ks", torch.float32, (T, Hkv))
    if s is None:
        s = torch.empty((Hq, Mq, T), dtype=torch.float32, device=qq.device)
    _need_c(s, "s", torch.float32, (Hq, Mq, T))
    dots = torch.empty((Hq, Mq, T), dtype=torch.int32, device=qq.device) if want_dots else None
    _raise(load_library().attn_qk_int8(_ptr(qq), _ptr(qs), _ptr(kq), _ptr(ks), float(scale), Mq, T, Hq, Hkv,
                                       _ptr(s), _ptr(dots), _stream(qq.device)))
    return s, dots


def attn_pv_int8(p: torch.Tensor, vq: torch.Tensor, vs: torch.Tensor, want_codes: bool = False,
                 out: Optional[torch.Tensor] = None):
    """INT8 PV on the block-g128 cache: p fp32 [Hq, Mq, T], vq int8 [T, Hkv, 128], vs fp32
    [T, Hkv] -> (out fp32 [Hq, Mq, 128], pq int8 [Hq, Mq, T] or None, ps fp32 [Hq, Mq, B] or None)."""
    if p.dim() != 3 or vq.dim() != 3:
        raise ValueError("p must be [Hq, Mq, T] and vq [T, Hkv, 128]")
    Hq, Mq, T = p.shape
    Hkv = vq.shape[1]
    _need_c(p, "p", torch.float32, (Hq, Mq, T))
    _need_c(vq, "vq", torch.int8, (T, Hkv, 128))
    _need_c(vs, "vs", torch.float32, (T, Hkv))
    if out is None:
        out = torch.empty((Hq, Mq, 128), dtype=torch.float32, device=p.device)
    _need_c(out, "out", torch.float32, (Hq, Mq, 128))
    B = (T + 127) // 128
    pq = torch.empty((Hq, Mq, T), dtype=torch.int8, device=p.device) if want_codes else None
    ps = torch.empty((Hq, Mq, B), dtype=torch.float32, device=p.device) if want_codes else None
    nbytes = load_library().attn_pv_int8_workspace_bytes(Mq, T, Hq, Hkv)
    if nbytes == ctypes.c_size_t(-1).value:
        raise ValueError(f"invalid attention sizes Mq={Mq} T={T} Hq={Hq} Hkv={Hkv}")
    ws = _workspace(p.device, int(nbytes))
    _raise(load_library().attn_pv_int8(_ptr(p), _ptr(vq), _ptr(vs), Mq, T, Hq, Hkv, _ptr(out), _ptr(pq), _ptr(ps),
                                       _ptr(ws), int(nbytes), _stream(p.device)))
    return out, pq, ps
