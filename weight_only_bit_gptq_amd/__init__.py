"""GPTQ weight-only GEMM for AMD MI355X (gfx950): Python binding of libgptq.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gptq.h``.  PyTorch supplies
device memory and the current stream.  If the compiled library is missing the
functions raise ``RuntimeError``; there is no CPU fallback.

    out = gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2)
    w   = dequant(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, K)
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

__all__ = ["gemm", "gemm_noalloc", "describe", "dequant", "quantize", "convert_zeros", "repack_tiled", "unrepack_tiled", "moe_gemm",
           "sort_act_order", "gemm_sorted", "read_ceiling", "release", "library", "library_path", "GptqError",
           "STATUS", "PATH_AUTO", "PATH_DECODE", "PATH_PREFILL"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "_lib", "libgptq.so")
_lock = threading.Lock()
_lib = None

PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2

STATUS = {
    0: "GPTQ_OK", -1: "GPTQ_ERR_NULL_PTR", -2: "GPTQ_ERR_BAD_BITS", -3: "GPTQ_ERR_BAD_SHAPE",
    -4: "GPTQ_ERR_BAD_GROUP", -5: "GPTQ_ERR_MISALIGNED", -6: "GPTQ_ERR_NO_MEM",
    -7: "GPTQ_ERR_LAUNCH", -8: "GPTQ_ERR_DEVICE", -9: "GPTQ_ERR_BAD_ARG",
}


class GptqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """Load libgptq.so (built in-tree by ``weight_only_bit_gptq_amd.build_lib``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libgptq.so is not built ({_LIB_PATH}); run "
                               "`python -m weight_only_bit_gptq_amd.build_lib`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32p, i64, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        gemm_args = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp, vp]
        lib.gptq_gemm.argtypes = gemm_args
        lib.gptq_gemm.restype = i32
        lib.gptq_gemm_ex.argtypes = gemm_args + [i32, i32]
        lib.gptq_gemm_noalloc.argtypes = gemm_args
        lib.gptq_gemm_noalloc.restype = i32
        lib.gptq_gemm_ex.restype = i32
        lib.gptq_dequant.argtypes = [i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, vp, vp]
        for name in ("gptq_gemm_bf16", "gptq_gemm_bf16_ex", "gptq_gemm_bf16_describe", "gptq_dequant_bf16"):
            getattr(lib, name).restype = i32
        lib.gptq_gemm_bf16.argtypes = gemm_args
        lib.gptq_gemm_bf16_ex.argtypes = gemm_args + [i32, i32]
        lib.gptq_gemm_bf16_describe.argtypes = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp, i32,
                                                i32, ctypes.c_char_p, i64]
        lib.gptq_dequant_bf16.argtypes = [i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, vp, vp]
        for name in ("gptq_gemm_tiled_bf16", "gptq_gemm_tiled_bf16_ex", "gptq_gemm_tiled_bf16_describe"):
            getattr(lib, name).restype = i32
        lib.gptq_gemm_tiled_bf16.argtypes = gemm_args
        lib.gptq_gemm_tiled_bf16_ex.argtypes = gemm_args + [i32, i32]
        lib.gptq_gemm_tiled_bf16_describe.argtypes = lib.gptq_gemm_bf16_describe.argtypes
        lib.gptq_dequant.restype = i32
        lib.gptq_gemm_check.argtypes = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp]
        lib.gptq_gemm_check.restype = i32
        lib.gptq_gemm_ex_check.argtypes = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp, i32, i32]
        lib.gptq_gemm_ex_check.restype = i32
        lib.gptq_gemm_describe.argtypes = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp, i32, i32,
                                           ctypes.c_char_p, i64]
        lib.gptq_gemm_describe.restype = i32
        lib.gptq_dequant_check.argtypes = [i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, vp]
        lib.gptq_dequant_check.restype = i32
        lib.gptq_quantize.argtypes = [vp, i32p, i32, i32, i32, i32, i64, i64, i32p, i32p, vp, vp]
        lib.gptq_quantize.restype = i32
        lib.gptq_gemm_tiled_ex.argtypes = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp, vp, i32, i32]
        lib.gptq_gemm_tiled_ex.restype = i32
        lib.gptq_gemm_tiled.argtypes = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp, vp]
        lib.gptq_gemm_tiled.restype = i32
        lib.gptq_gemm_tiled_describe.argtypes = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp, i32,
                                                 i32, ctypes.c_char_p, i64]
        lib.gptq_gemm_tiled_describe.restype = i32
        lib.gptq_sort_act_order.argtypes = [i32p, i32p, i32, i32, i64, i64, i32p, i32p, vp]
        lib.gptq_sort_act_order.restype = i32
        lib.gptq_gemm_sorted.argtypes = [vp, i32p, i32p, vp, i32p, i32, i32, i32, i64, i64, i64, vp, vp, i32, i32, i32]
        lib.gptq_gemm_sorted.restype = i32
        lib.gptq_moe_gemm.argtypes = [vp, i32p, i32p, vp, i32p, i32p, i32, i32, i32, i32, i32, i64, i64, i64, vp, vp]
        lib.gptq_moe_gemm.restype = i32
        lib.gptq_moe_gemm_ex.argtypes = lib.gptq_moe_gemm.argtypes + [i32]
        lib.gptq_moe_gemm_ex.restype = i32
        lib.gptq_repack_tiled.argtypes = [i32p, i32p, i32, i64, i64, vp]
        lib.gptq_repack_tiled.restype = i32
        lib.gptq_unrepack_tiled.argtypes = [i32p, i32p, i32, i64, i64, vp]
        lib.gptq_unrepack_tiled.restype = i32
        lib.gptq_convert_zeros.argtypes = [i32p, i32p, i32, i64, i64, i32, i32p, vp]
        lib.gptq_convert_zeros.restype = i32
        lib.gptq_convert_zeros_check.argtypes = [i32p, i32p, i32, i64, i64, i32, i32p]
        lib.gptq_convert_zeros_check.restype = i32
        lib.gptq_strerror.argtypes = [i32]
        lib.gptq_strerror.restype = ctypes.c_char_p
        lib.gptq_release.argtypes = []
        lib.gptq_release.restype = None
        lib.gptq_read_ceiling.argtypes = [vp, i64, vp, vp]
        lib.gptq_read_ceiling.restype = i32
        lib.gptq_abi_version.argtypes = []
        lib.gptq_abi_version.restype = i32
        if lib.gptq_abi_version() != 1:
            raise RuntimeError("libgptq.so ABI version mismatch")
        _lib = lib
        return lib


def _raise(code: int):
    if code != 0:
        msg = library().gptq_strerror(code).decode()
        raise GptqError(code, msg)


def _check_tensor(name, t, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _weights(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, K=None, sdtype=None):
    import torch
    sdtype = torch.float16 if sdtype is None else sdtype
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    if is_v2 not in (0, 1, True, False):
        raise ValueError("is_v2 must be a bool")
    dev = qweight.device if isinstance(qweight, torch.Tensor) else None
    _check_tensor("qweight", qweight, torch.int32, dev)
    _check_tensor("qzeros", qzeros, torch.int32, dev)
    _check_tensor("scales", scales, sdtype, dev)
    if g_idx is not None:
        _check_tensor("g_idx", g_idx, torch.int32, dev)
    if qzeros.dim() != 2 or scales.dim() != 2:
        raise ValueError("qzeros and scales must be 2-D")
    if qweight.dim() == 4:                 # tiled layout [N/16, K/32, bits, 16]
        if qweight.shape[2] != bits or qweight.shape[3] != 16:
            raise ValueError(f"tiled qweight must be [N/16, K/32, {bits}, 16], got {tuple(qweight.shape)}")
        N = qweight.shape[0] * 16
        if K is None:
            K = qweight.shape[1] * 32
        if qweight.shape[1] * 32 != K:
            raise ValueError(f"tiled qweight covers K = {qweight.shape[1] * 32}, expected {K}")
    elif qweight.dim() == 2:               # checkpoint layout [K*bits/32, N]
        N = qweight.shape[1]
        if K is None:
            K = qweight.shape[0] * 32 // bits
        if qweight.shape[0] * 32 != K * bits:
            raise ValueError(f"qweight has {qweight.shape[0]} rows, expected K*bits/32 = {K * bits / 32}")
    else:
        raise ValueError("qweight must be 2-D (checkpoint layout) or 4-D (tiled layout)")
    if group_size <= 0 or K % group_size:
        raise ValueError("group_size must divide K")
    G = K // group_size
    if tuple(scales.shape) != (G, N):
        raise ValueError(f"scales must be [{G}, {N}], got {tuple(scales.shape)}")
    if tuple(qzeros.shape) != (G, N * bits // 32) or (N * bits) % 32:
        raise ValueError(f"qzeros must be [{G}, {N * bits // 32}], got {tuple(qzeros.shape)}")
    if g_idx is not None and tuple(g_idx.shape) != (K,):
        raise ValueError(f"g_idx must be [{K}]")
    return dev, N, K


def _act_dtype(x, qweight):
    """Activation type of a call: x's dtype, fp16 or bf16."""
    import torch
    return torch.bfloat16 if getattr(x, "dtype", None) == torch.bfloat16 else torch.float16


def gemm(x, qweight, qzeros, scales, g_idx: Optional[object], bits: int, group_size: int,
         is_v2: bool, *, out=None, path: int = PATH_AUTO, decode_waves: int = 0):
    """out[M, N] = x[M, K] . dequant(qweight, qzeros, scales, g_idx).

    x, scales and out are all fp16, or all bfloat16 (gptq_gemm_bf16,
    gptq_gemm_tiled_bf16).  qweight is the checkpoint layout [K*bits/32, N]
    or, 4-D, the tiled layout made by `repack_tiled`.  Enqueued on the current
    HIP stream of x's device (asynchronous)."""
    import torch
    act = _act_dtype(x, qweight)
    dev, N, K = _weights(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, sdtype=act)
    _check_tensor("x", x, act, dev)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M, {K}], got {tuple(x.shape)}")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=act, device=dev)
    else:
        _check_tensor("out", out, act, dev)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be [{M}, {N}]")
    lib = library()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        if act == torch.bfloat16:
            fn = lib.gptq_gemm_tiled_bf16_ex if qweight.dim() == 4 else lib.gptq_gemm_bf16_ex
        else:
            fn = lib.gptq_gemm_tiled_ex if qweight.dim() == 4 else lib.gptq_gemm_ex
        code = fn(x.data_ptr(), qweight.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
                  None if g_idx is None else g_idx.data_ptr(), int(bits), int(group_size),
                  int(bool(is_v2)), M, N, K, out.data_ptr(), stream, int(path), int(decode_waves))
    _raise(code)
    return out


def gemm_noalloc(x, qweight, qzeros, scales, g_idx: Optional[object], bits: int, group_size: int, is_v2: bool, *,
                 out):
    """gemm through gptq_gemm_noalloc: the library allocates nothing (split-K
    scratch in a static per-device array); `out` must be given, fp16 [M, N],
    checkpoint qweight layout."""
    import torch
    dev, N, K = _weights(qweight, qzeros, scales, g_idx, bits, group_size, is_v2)
    if qweight.dim() != 2:
        raise ValueError("gemm_noalloc takes the checkpoint qweight layout")
    _check_tensor("x", x, torch.float16, dev)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M, {K}], got {tuple(x.shape)}")
    M = x.shape[0]
    _check_tensor("out", out, torch.float16, dev)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}, {N}]")
    lib = library()
    with torch.cuda.device(dev):
        code = lib.gptq_gemm_noalloc(x.data_ptr(), qweight.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
                                     None if g_idx is None else g_idx.data_ptr(), int(bits), int(group_size),
                                     int(bool(is_v2)), M, N, K, out.data_ptr(),
                                     torch.cuda.current_stream(dev).cuda_stream)
    _raise(code)
    return out


def describe(x, qweight, qzeros, scales, g_idx: Optional[object], bits: int, group_size: int,
             is_v2: bool, *, out=None, path: int = PATH_AUTO, decode_waves: int = 0) -> str:
    """Kernel instantiation and launch shape `gemm` with these arguments uses."""
    import torch
    act = _act_dtype(x, qweight)
    dev, N, K = _weights(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, sdtype=act)
    _check_tensor("x", x, act, dev)
    M = x.shape[0]
    out_ptr = out.data_ptr() if out is not None else x.data_ptr()
    buf = ctypes.create_string_buffer(256)
    lib = library()
    if act == torch.bfloat16:
        fn = lib.gptq_gemm_tiled_bf16_describe if qweight.dim() == 4 else lib.gptq_gemm_bf16_describe
    else:
        fn = lib.gptq_gemm_tiled_describe if qweight.dim() == 4 else lib.gptq_gemm_describe
    code = fn(x.data_ptr(), qweight.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
              None if g_idx is None else g_idx.data_ptr(), int(bits), int(group_size),
              int(bool(is_v2)), M, N, K, out_ptr, int(path), int(decode_waves), buf, 256)
    _raise(code)
    return buf.value.decode()


def dequant(qweight, qzeros, scales, g_idx: Optional[object], bits: int, group_size: int,
            is_v2: bool, *, out=None):
    """W^ [K, N], bit-exact dequantization of the packed weights (checkpoint layout),
    in the scales' type: fp16, or bfloat16 (gptq_dequant_bf16)."""
    import torch
    if isinstance(qweight, torch.Tensor) and qweight.dim() == 4:
        raise ValueError("dequant takes the checkpoint qweight layout (unrepack_tiled the tiled one)")
    act = torch.bfloat16 if getattr(scales, "dtype", None) == torch.bfloat16 else torch.float16
    dev, N, K = _weights(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, sdtype=act)
    if out is None:
        out = torch.empty((K, N), dtype=act, device=dev)
    else:
        _check_tensor("out", out, act, dev)
        if tuple(out.shape) != (K, N):
            raise ValueError(f"out must be [{K}, {N}]")
    lib = library()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        fn = lib.gptq_dequant_bf16 if act == torch.bfloat16 else lib.gptq_dequant
        code = fn(qweight.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
                                None if g_idx is None else g_idx.data_ptr(), int(bits), int(group_size),
                                int(bool(is_v2)), N, K, out.data_ptr(), stream)
    _raise(code)
    return out


def quantize(w, g_idx: Optional[object], bits: int, group_size: int, sym: bool, is_v2: bool):
    """Min/max round-to-nearest quantization of W [K, N] (fp32, GPU) into
    (qweight int32 [K*b/32, N], qzeros int32 [G, N*b/32], scales fp16 [G, N])."""
    import torch
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    dev = w.device if isinstance(w, torch.Tensor) else None
    _check_tensor("w", w, torch.float32, dev)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [K, N]")
    K, N = w.shape
    if K % 32 or N % 32 or group_size <= 0 or K % group_size:
        raise ValueError("need K % 32 == 0, N % 32 == 0 and group_size dividing K")
    if g_idx is not None:
        _check_tensor("g_idx", g_idx, torch.int32, dev)
        if tuple(g_idx.shape) != (K,):
            raise ValueError(f"g_idx must be [{K}]")
    G = K // group_size
    qweight = torch.empty((K * bits // 32, N), dtype=torch.int32, device=dev)
    qzeros = torch.empty((G, N * bits // 32), dtype=torch.int32, device=dev)
    scales = torch.empty((G, N), dtype=torch.float16, device=dev)
    lib = library()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        code = lib.gptq_quantize(w.data_ptr(), None if g_idx is None else g_idx.data_ptr(), int(bits),
                                 int(group_size), int(bool(sym)), int(bool(is_v2)), N, K, qweight.data_ptr(),
                                 qzeros.data_ptr(), scales.data_ptr(), stream)
    _raise(code)
    return qweight, qzeros, scales


def convert_zeros(qzeros, bits: int, N: int, to_v2: bool, out=None, lossy_count=None):
    """GPTQv1 <-> GPTQv2 conversion of packed zeros qzeros [G, N*b/32] (int32, GPU).

    Returns ``out`` (a new tensor unless given; may be ``qzeros`` itself for an
    in-place conversion).  ``lossy_count``, an int32 tensor of one element on
    the same device, if given, is incremented by the number of fields that the
    target format cannot hold exactly."""
    import torch
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    dev = qzeros.device if isinstance(qzeros, torch.Tensor) else None
    _check_tensor("qzeros", qzeros, torch.int32, dev)
    if N <= 0 or N % 32 or qzeros.dim() != 2 or qzeros.shape[1] != N * bits // 32 or qzeros.shape[0] < 1:
        raise ValueError(f"qzeros must be [G >= 1, {N * bits // 32}] with N % 32 == 0")
    G = qzeros.shape[0]
    if out is None:
        out = torch.empty_like(qzeros)
    _check_tensor("out", out, torch.int32, dev)
    if tuple(out.shape) != tuple(qzeros.shape):
        raise ValueError("out must have the shape of qzeros")
    if lossy_count is not None:
        _check_tensor("lossy_count", lossy_count, torch.int32, dev)
        if lossy_count.numel() != 1:
            raise ValueError("lossy_count must hold one element")
    lib = library()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        code = lib.gptq_convert_zeros(qzeros.data_ptr(), out.data_ptr(), int(bits), G, int(N), int(bool(to_v2)),
                                      None if lossy_count is None else lossy_count.data_ptr(), stream)
    _raise(code)
    return out


def sort_act_order(qweight, g_idx, bits: int, group_size: int):
    """Act-order layer -> (qweight_sorted [K*bits/32, N], perm int32 [K]): rows
    sorted by group (stable), for `gemm_sorted`.  Synchronizes the stream."""
    import torch
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    dev = qweight.device if isinstance(qweight, torch.Tensor) else None
    _check_tensor("qweight", qweight, torch.int32, dev)
    _check_tensor("g_idx", g_idx, torch.int32, dev)
    if qweight.dim() != 2:
        raise ValueError("qweight must be the checkpoint layout [K*bits/32, N]")
    N, K = qweight.shape[1], qweight.shape[0] * 32 // bits
    if tuple(g_idx.shape) != (K,):
        raise ValueError(f"g_idx must be [{K}]")
    qs = torch.empty_like(qweight)
    perm = torch.empty((K,), dtype=torch.int32, device=dev)
    lib = library()
    with torch.cuda.device(dev):
        _raise(lib.gptq_sort_act_order(qweight.data_ptr(), g_idx.data_ptr(), int(bits), int(group_size), N, K,
                                       qs.data_ptr(), perm.data_ptr(), torch.cuda.current_stream(dev).cuda_stream))
    return qs, perm


def gemm_sorted(x, qweight_sorted, qzeros, scales, perm, bits: int, group_size: int, is_v2: bool, *, out=None,
                path: int = PATH_AUTO, decode_waves: int = 0):
    """gemm for an act-order layer whose rows were sorted by `sort_act_order`
    (qweight_sorted in the checkpoint layout, or 4-D tiled by repack_tiled)."""
    import torch
    dev, N, K = _weights(qweight_sorted, qzeros, scales, None, bits, group_size, is_v2)
    _check_tensor("x", x, torch.float16, dev)
    _check_tensor("perm", perm, torch.int32, dev)
    if tuple(perm.shape) != (K,):
        raise ValueError(f"perm must be [{K}]")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M, {K}]")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    else:
        _check_tensor("out", out, torch.float16, dev)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be [{M}, {N}]")
    lib = library()
    with torch.cuda.device(dev):
        code = lib.gptq_gemm_sorted(x.data_ptr(), qweight_sorted.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
                                    perm.data_ptr(), int(bits), int(group_size), int(bool(is_v2)), M, N, K,
                                    out.data_ptr(), torch.cuda.current_stream(dev).cuda_stream,
                                    1 if qweight_sorted.dim() == 4 else 0, int(path), int(decode_waves))
    _raise(code)
    return out


def moe_gemm(x, qweight, qzeros, scales, g_idx: Optional[object], expert_offsets, max_tokens_per_expert: int,
             bits: int, group_size: int, is_v2: bool, *, out=None, path: int = 0):
    """Grouped GEMM: rows [off[e], off[e+1]) of x (tokens sorted by expert)
    times expert e's weights.  qweight [E, K*bits/32, N], qzeros
    [E, G, N*bits/32], scales [E, G, N], g_idx [E, K] or None, expert_offsets
    int32 [E+1] on the GPU.  Rows of no expert keep out's previous contents.
    path: 0 = by batch size (gptq_moe_gemm), 1 = decode kernel, 2 = prefill
    kernel (gptq_moe_gemm_ex)."""
    import torch
    if qweight.dim() != 3 or qzeros.dim() != 3 or scales.dim() != 3:
        raise ValueError("qweight, qzeros, scales must be [E, ...] stacks")
    E = qweight.shape[0]
    dev, N, K = _weights(qweight[0], qzeros[0], scales[0], None if g_idx is None else g_idx[0], bits,
                         group_size, is_v2)
    for name, t in (("qweight", qweight), ("qzeros", qzeros), ("scales", scales)):
        if t.shape[0] != E or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [E={E}, ...] stack")
    if g_idx is not None and (tuple(g_idx.shape) != (E, K) or not g_idx.is_contiguous()):
        raise ValueError(f"g_idx must be [{E}, {K}]")
    _check_tensor("x", x, torch.float16, dev)
    _check_tensor("expert_offsets", expert_offsets, torch.int32, dev)
    if tuple(expert_offsets.shape) != (E + 1,):
        raise ValueError(f"expert_offsets must be [{E + 1}]")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [T, {K}]")
    T = x.shape[0]
    if out is None:
        out = torch.zeros((T, N), dtype=torch.float16, device=dev)
    else:
        _check_tensor("out", out, torch.float16, dev)
        if tuple(out.shape) != (T, N):
            raise ValueError(f"out must be [{T}, {N}]")
    lib = library()
    with torch.cuda.device(dev):
        code = lib.gptq_moe_gemm_ex(x.data_ptr(), qweight.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
                                    None if g_idx is None else g_idx.data_ptr(), expert_offsets.data_ptr(), E,
                                    int(max_tokens_per_expert), int(bits), int(group_size), int(bool(is_v2)), T, N,
                                    K, out.data_ptr(), torch.cuda.current_stream(dev).cuda_stream, int(path))
    _raise(code)
    return out


def repack_tiled(qweight, bits: int):
    """Checkpoint qweight [K*bits/32, N] (int32, GPU) -> tiled layout [N/16, K/32, bits, 16]
    (4-bit words with their fields in pair order; see gptq_repack_tiled)."""
    import torch
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    dev = qweight.device if isinstance(qweight, torch.Tensor) else None
    _check_tensor("qweight", qweight, torch.int32, dev)
    if qweight.dim() != 2 or (qweight.shape[0] * 32) % bits:
        raise ValueError("qweight must be [K*bits/32, N]")
    N, K = qweight.shape[1], qweight.shape[0] * 32 // bits
    if N % 32 or K % 32:
        raise ValueError("need N % 32 == 0 and K % 32 == 0")
    out = torch.empty((N // 16, K // 32, bits, 16), dtype=torch.int32, device=dev)
    lib = library()
    with torch.cuda.device(dev):
        _raise(lib.gptq_repack_tiled(qweight.data_ptr(), out.data_ptr(), int(bits), N, K,
                                     torch.cuda.current_stream(dev).cuda_stream))
    return out


def unrepack_tiled(qweight_tiled, bits: int):
    """Tiled layout [N/16, K/32, bits, 16] -> checkpoint qweight [K*bits/32, N]."""
    import torch
    dev = qweight_tiled.device if isinstance(qweight_tiled, torch.Tensor) else None
    _check_tensor("qweight_tiled", qweight_tiled, torch.int32, dev)
    if qweight_tiled.dim() != 4 or qweight_tiled.shape[2] != bits or qweight_tiled.shape[3] != 16:
        raise ValueError(f"qweight_tiled must be [N/16, K/32, {bits}, 16]")
    N, K = qweight_tiled.shape[0] * 16, qweight_tiled.shape[1] * 32
    out = torch.empty((K * bits // 32, N), dtype=torch.int32, device=dev)
    lib = library()
    with torch.cuda.device(dev):
        _raise(lib.gptq_unrepack_tiled(qweight_tiled.data_ptr(), out.data_ptr(), int(bits), N, K,
                                       torch.cuda.current_stream(dev).cuda_stream))
    return out


def release():
    """Release library-owned device memory (the split-K workspaces), after synchronising the devices."""
    library().gptq_release()


def read_ceiling(buf, nbytes: Optional[int] = None, *, sink=None):
    """Read the first `nbytes` bytes of the contiguous GPU tensor `buf` once
    (gptq_read_ceiling: 16-byte nontemporal loads, nothing else), on the
    current stream: the memory-read reference the decode launches are measured
    against.  `sink` is an int32 GPU tensor the kernel may write (allocated if
    omitted)."""
    import torch
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    total = buf.numel() * buf.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if nbytes < 0 or nbytes > total:
        raise ValueError(f"nbytes must lie in [0, {total}]")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check_tensor("sink", sink, torch.int32, buf.device)
    lib = library()
    with torch.cuda.device(buf.device):
        code = lib.gptq_read_ceiling(buf.data_ptr(), nbytes, sink.data_ptr(),
                                     torch.cuda.current_stream(buf.device).cuda_stream)
    _raise(code)
    return sink
