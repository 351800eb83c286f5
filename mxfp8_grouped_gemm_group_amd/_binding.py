"""ctypes binding of libgfr.so (include/gfr.h).

Argument marshalling only: shapes and dtypes of torch tensors are read here,
device pointers and sizes go to the C ABI, and every step of the operator runs
in the library's HIP kernels.  torch provides device memory and the stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgfr.so")

GFR_OK = 0
DEV_BAD_GROUP_LIST = 0x1
DEV_BAD_ROW_INDEX = 0x2

_FP8_KIND = {torch.float8_e4m3fn: 0, torch.float8_e5m2: 1, torch.float4_e2m1fn_x2: 2}
_PACKED = torch.float4_e2m1fn_x2   # two E2M1 elements per byte along the last axis
_E8M0 = (torch.uint8, torch.float8_e8m0fnu)


class GfrError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gfr error {code}: {msg}")
        self.code = code


class GfrOptions(ctypes.Structure):
    _fields_ = [("deterministic", ctypes.c_int), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("status_dev", ctypes.c_void_p),
                ("split_k", ctypes.c_int), ("scale_per_expert", ctypes.c_int)]


_lib: Optional[ctypes.CDLL] = None

_MAIN_ARGS = [ctypes.c_void_p] * 5 + [ctypes.c_int] + [ctypes.c_void_p] * 3 + [
    ctypes.c_float, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [
    ctypes.c_int64] * 6 + [ctypes.c_void_p]


def load_library() -> ctypes.CDLL:
    """Load libgfr.so; raises if it has not been built (no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "mxfp8_grouped_gemm_group_amd.build_lib.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.gmm_finalize_routing.argtypes = _MAIN_ARGS
        lib.gmm_finalize_routing.restype = ctypes.c_int
        lib.gmm_finalize_routing_ex.argtypes = _MAIN_ARGS + [ctypes.POINTER(GfrOptions)]
        lib.gmm_finalize_routing_ex.restype = ctypes.c_int
        lib.gfr_workspace_size.argtypes = [ctypes.c_int64] * 5 + [
            ctypes.POINTER(GfrOptions), ctypes.POINTER(ctypes.c_size_t)]
        lib.gfr_workspace_size.restype = ctypes.c_int
        lib.gfr_gemm1_swiglu_quant.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] + [
            ctypes.c_void_p] * 2 + [ctypes.c_int] * 3 + [ctypes.c_int64] * 4 + [
            ctypes.c_void_p, ctypes.POINTER(GfrOptions)]
        lib.gfr_gemm1_swiglu_quant.restype = ctypes.c_int
        lib.gfr_w4a8_finalize_routing.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] + [
            ctypes.c_void_p] * 3 + [ctypes.c_float, ctypes.c_int64, ctypes.c_void_p] + [
            ctypes.c_int64] * 6 + [ctypes.c_void_p, ctypes.POINTER(GfrOptions)]
        lib.gfr_w4a8_finalize_routing.restype = ctypes.c_int
        lib.gfr_status_string.argtypes = [ctypes.c_int]
        lib.gfr_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(code: int) -> str:
    return load_library().gfr_status_string(code).decode()


def workspace_size(M: int, K: int, N: int, E: int, batch: int, deterministic: bool = False) -> int:
    opts = GfrOptions(int(deterministic), None, 0, None, 0, 0)
    n = ctypes.c_size_t(0)
    rc = load_library().gfr_workspace_size(M, K, N, E, batch, ctypes.byref(opts), ctypes.byref(n))
    if rc:
        raise GfrError(rc, status_string(rc))
    return n.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def gmm_finalize_routing(x1, x2, scale, pertoken_scale, group_list, group_list_type, logit,
                         row_index, shared_input, shared_input_weight, shared_input_offset,
                         out, transpose_x2=False, *, deterministic=False, workspace=None,
                         status=None, split_k=0, stream=None):
    """out += routed expert rows + shared term, in place; returns out.

    x1 [M,K] / x2 [E,K,N] (or [E,N,K] when transpose_x2) are float8_e4m3fn or
    float8_e5m2, or float4_e2m1fn_x2 (MXFP4: the last axis holds half as many
    bytes as elements); scale / pertoken_scale hold E8M0 codes (uint8 or
    float8_e8m0fnu); a 4-D scale (leading expert axis) is per expert; group_list int64 [E]; logit float32 [M] or None;
    row_index int64 [M]; shared_input bfloat16 [R,N] or None; out float32
    [batch,N].  ``status`` (int32 CUDA tensor, 1 element) receives device-side
    data-error bits.  ``workspace`` (uint8 CUDA tensor) is allocated here when
    the deterministic mode needs one and none is given.
    """
    lib = load_library()
    _need(x1.dtype in _FP8_KIND and x2.dtype == x1.dtype, "x1/x2 must share an FP8 / FP4 dtype")
    _need(x1.dim() == 2 and x2.dim() == 3, "x1 must be 2-D and x2 3-D")
    per = 2 if x1.dtype == _PACKED else 1     # elements per stored byte along the last axis
    M, K = x1.shape[0], x1.shape[1] * per
    E = x2.shape[0]
    if transpose_x2:
        N = x2.shape[1]
        _need(x2.shape[2] * per == K, "x2 [E,N,K] does not match K")
    else:
        N = x2.shape[2] * per
        _need(x2.shape[1] == K, "x2 [E,K,N] does not match K")
    KB = (K + 63) // 64
    _need(scale.dtype in _E8M0 and pertoken_scale.dtype in _E8M0, "scales must be E8M0 bytes")
    s3 = (N, KB, 2) if transpose_x2 else (KB, N, 2)
    per_expert = scale.dim() == 4
    _need(tuple(scale.shape) == ((E,) + s3 if per_expert else s3),
          "bad scale shape (3-D shared, or 4-D with a leading expert axis)")
    _need(tuple(pertoken_scale.shape) == (M, KB, 2), "bad pertoken_scale shape")
    _need(group_list.dtype == torch.int64 and tuple(group_list.shape) == (E,), "bad group_list")
    _need(row_index.dtype == torch.int64 and tuple(row_index.shape) == (M,), "bad row_index")
    if logit is not None:
        _need(logit.dtype == torch.float32 and tuple(logit.shape) == (M,), "bad logit")
    _need(out.dtype == torch.float32 and out.dim() == 2 and out.shape[1] == N, "bad out")
    batch = out.shape[0]
    R = 0
    if shared_input is not None:
        _need(shared_input.dtype == torch.bfloat16 and shared_input.dim() == 2
              and shared_input.shape[1] == N, "bad shared_input")
        R = shared_input.shape[0]
    tensors = [x1, x2, scale, pertoken_scale, group_list, row_index, out, logit, shared_input,
               workspace, status]
    dev = out.device
    for t in tensors:
        if t is not None:
            _need(t.is_cuda and t.device == dev, "all tensors must be on out's CUDA device")
            _need(t.is_contiguous(), "all tensors must be contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ws_bytes = 0
    if deterministic:
        need = workspace_size(M, K, N, E, batch, True)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    opts = GfrOptions(int(bool(deterministic)), _ptr(workspace), ws_bytes, _ptr(status),
                      int(split_k), int(per_expert))
    with torch.cuda.device(dev):
        rc = lib.gmm_finalize_routing_ex(
            _ptr(x1), _ptr(x2), _ptr(scale), _ptr(pertoken_scale), _ptr(group_list),
            int(group_list_type), _ptr(logit), _ptr(row_index), _ptr(shared_input),
            float(shared_input_weight), int(shared_input_offset), _ptr(out),
            int(bool(transpose_x2)), _FP8_KIND[x1.dtype], M, K, N, E, batch, R,
            ctypes.c_void_p(stream), ctypes.byref(opts))
    if rc:
        raise GfrError(rc, status_string(rc))
    return out


def gemm1_swiglu_quant(xin, w13, scale, xin_scale, group_list, group_list_type,
                       transpose_w13=False, out_dtype=torch.float8_e4m3fn, *, x1_out=None,
                       x1_scale_out=None, status=None, stream=None):
    """Upstream step of the MoE FFN: gate||up grouped matmul, SwiGLU, MX
    quantisation (include/gfr.h, gfr_gemm1_swiglu_quant).

    xin float8 [M, H]; w13 [E, H, 2I] (or [E, 2I, H] with transpose_w13) of
    xin's dtype; scale E8M0 [ceil(H/64), 2I, 2] (or [2I, ceil(H/64), 2]; 4-D
    with a leading expert axis for per-expert scales); xin_scale E8M0
    [M, ceil(H/64), 2]; group_list int64 [E].  Returns (x1, x1_scale): out_dtype
    [M, I] and uint8 [M, I/64, 2], ready to be gmm_finalize_routing's x1 and
    pertoken_scale.  Rows of tokens in no expert's range are left as they were
    in x1_out / x1_scale_out (zeros when the call allocates them)."""
    lib = load_library()
    _need(xin.dtype in (torch.float8_e4m3fn, torch.float8_e5m2) and w13.dtype == xin.dtype,
          "xin/w13 must share an FP8 dtype")
    _need(out_dtype in (torch.float8_e4m3fn, torch.float8_e5m2), "out_dtype must be FP8")
    _need(xin.dim() == 2 and w13.dim() == 3, "xin must be 2-D and w13 3-D")
    M, H = xin.shape
    E = w13.shape[0]
    if transpose_w13:
        _need(w13.shape[2] == H, "w13 [E,2I,H] does not match H")
        N2 = w13.shape[1]
    else:
        _need(w13.shape[1] == H, "w13 [E,H,2I] does not match H")
        N2 = w13.shape[2]
    _need(N2 % 2 == 0, "w13 must have an even number (2I) of columns")
    I = N2 // 2
    KB = (H + 63) // 64
    s3 = (N2, KB, 2) if transpose_w13 else (KB, N2, 2)
    _need(scale.dtype in _E8M0 and xin_scale.dtype in _E8M0, "scales must be E8M0 bytes")
    per_expert = scale.dim() == 4
    _need(tuple(scale.shape) == ((E,) + s3 if per_expert else s3), "bad scale shape")
    _need(tuple(xin_scale.shape) == (M, KB, 2), "bad xin_scale shape")
    _need(group_list.dtype == torch.int64 and tuple(group_list.shape) == (E,), "bad group_list")
    dev = xin.device
    if x1_out is None:
        x1_out = torch.zeros((M, I), dtype=torch.uint8, device=dev).view(out_dtype)
    if x1_scale_out is None:
        x1_scale_out = torch.zeros((M, (I + 63) // 64, 2), dtype=torch.uint8, device=dev)
    _need(x1_out.dtype == out_dtype and tuple(x1_out.shape) == (M, I), "bad x1_out")
    _need(x1_scale_out.dtype in _E8M0 and tuple(x1_scale_out.shape) == (M, (I + 63) // 64, 2),
          "bad x1_scale_out")
    for t in (xin, w13, scale, xin_scale, group_list, x1_out, x1_scale_out, status):
        if t is not None:
            _need(t.is_cuda and t.device == dev, "all tensors must be on xin's CUDA device")
            _need(t.is_contiguous(), "all tensors must be contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    opts = GfrOptions(0, None, 0, _ptr(status), 0, int(per_expert))
    with torch.cuda.device(dev):
        rc = lib.gfr_gemm1_swiglu_quant(
            _ptr(xin), _ptr(w13), _ptr(scale), _ptr(xin_scale), _ptr(group_list),
            int(group_list_type), _ptr(x1_out), _ptr(x1_scale_out), int(bool(transpose_w13)),
            _FP8_KIND[xin.dtype], _FP8_KIND[out_dtype], M, H, I, E, ctypes.c_void_p(stream),
            ctypes.byref(opts))
    if rc:
        raise GfrError(rc, status_string(rc))
    return x1_out, x1_scale_out


def w4a8_finalize_routing(x1, x2, scale, offset, pertoken_scale, group_list, group_list_type,
                          logit, row_index, shared_input, shared_input_weight,
                          shared_input_offset, out, *, deterministic=False, workspace=None,
                          status=None, split_k=0, stream=None):
    """The W4A8 variant (include/gfr.h, gfr_w4a8_finalize_routing): x1 int8
    [M, K]; x2 uint8 [E, K, N/2] (two signed 4-bit weights per byte along n,
    element 2j in the low nibble); scale and offset (or None) float32
    [E, 1, N]; pertoken_scale float32 [M]; the rest as gmm_finalize_routing.
    Updates out in place and returns it."""
    lib = load_library()
    _need(x1.dtype == torch.int8 and x1.dim() == 2, "x1 must be int8 [M, K]")
    _need(x2.dtype == torch.uint8 and x2.dim() == 3, "x2 must be uint8 [E, K, N/2]")
    M, K = x1.shape
    E = x2.shape[0]
    _need(x2.shape[1] == K, "x2 [E, K, N/2] does not match K")
    N = 2 * x2.shape[2]
    _need(scale.dtype == torch.float32 and tuple(scale.shape) == (E, 1, N), "bad scale")
    _need(offset is None or (offset.dtype == torch.float32 and tuple(offset.shape) == (E, 1, N)),
          "bad offset")
    _need(pertoken_scale.dtype == torch.float32 and tuple(pertoken_scale.shape) == (M,),
          "bad pertoken_scale")
    _need(group_list.dtype == torch.int64 and tuple(group_list.shape) == (E,), "bad group_list")
    _need(row_index.dtype == torch.int64 and tuple(row_index.shape) == (M,), "bad row_index")
    if logit is not None:
        _need(logit.dtype == torch.float32 and tuple(logit.shape) == (M,), "bad logit")
    _need(out.dtype == torch.float32 and out.dim() == 2 and out.shape[1] == N, "bad out")
    batch = out.shape[0]
    R = 0
    if shared_input is not None:
        _need(shared_input.dtype == torch.bfloat16 and shared_input.dim() == 2
              and shared_input.shape[1] == N, "bad shared_input")
        R = shared_input.shape[0]
    dev = out.device
    for t in (x1, x2, scale, offset, pertoken_scale, group_list, row_index, out, logit,
              shared_input, workspace, status):
        if t is not None:
            _need(t.is_cuda and t.device == dev, "all tensors must be on out's CUDA device")
            _need(t.is_contiguous(), "all tensors must be contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ws_bytes = 0
    if deterministic:
        need = workspace_size(M, K, N, E, batch, True)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    opts = GfrOptions(int(bool(deterministic)), _ptr(workspace), ws_bytes, _ptr(status),
                      int(split_k), 0)
    with torch.cuda.device(dev):
        rc = lib.gfr_w4a8_finalize_routing(
            _ptr(x1), _ptr(x2), _ptr(scale), _ptr(offset), _ptr(pertoken_scale),
            _ptr(group_list), int(group_list_type), _ptr(logit), _ptr(row_index),
            _ptr(shared_input), float(shared_input_weight), int(shared_input_offset), _ptr(out),
            M, K, N, E, batch, R, ctypes.c_void_p(stream), ctypes.byref(opts))
    if rc:
        raise GfrError(rc, status_string(rc))
    return out
