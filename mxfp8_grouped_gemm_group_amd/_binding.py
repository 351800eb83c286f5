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


class GfrTensor(ctypes.Structure):
    """gfr_tensor: device pointer, gfr_dtype, rank, extents."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4)]


# torch dtype -> gfr_dtype (include/gfr.h)
DTYPES = {torch.float8_e4m3fn: 0, torch.float8_e5m2: 1, torch.float4_e2m1fn_x2: 2,
          torch.float8_e8m0fnu: 3, torch.uint8: 4, torch.bfloat16: 5, torch.float32: 6,
          torch.int64: 7, torch.int32: 8, torch.int8: 9}


def tensor_desc(t: Optional[torch.Tensor]):
    """A gfr_tensor describing t (None for an absent optional tensor)."""
    if t is None:
        return None
    _need(t.dtype in DTYPES, f"dtype {t.dtype} has no gfr_dtype")
    _need(1 <= t.dim() <= 4, f"rank {t.dim()} is outside 1..4")
    d = GfrTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = DTYPES[t.dtype]
    d.ndim = t.dim()
    for i, n in enumerate(t.shape):
        d.shape[i] = n
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_T = ctypes.POINTER(GfrTensor)
_O = ctypes.POINTER(GfrOptions)
_RAW_MAIN_ARGS = [_P] * 5 + [ctypes.c_int] + [_P] * 3 + [
    ctypes.c_float, ctypes.c_int64, _P, ctypes.c_int, ctypes.c_int] + [ctypes.c_int64] * 6 + [_P]
# descriptor finalize: x1 x2 scale pts group_list, type, logit row_index shared, weight,
# offset, out, transpose, kind
_DESC_MAIN_ARGS = [_T] * 5 + [ctypes.c_int] + [_T] * 3 + [ctypes.c_float, ctypes.c_int64, _T,
                                                          ctypes.c_int, ctypes.c_int]


def load_library() -> ctypes.CDLL:
    """Load libgfr.so; raises if it has not been built (no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "mxfp8_grouped_gemm_group_amd.build_lib.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.gmm_finalize_routing.argtypes = _DESC_MAIN_ARGS + [_P]
        lib.gmm_finalize_routing_ex.argtypes = _DESC_MAIN_ARGS + [_P, _O]
        lib.gfr_workspace_size.argtypes = _DESC_MAIN_ARGS + [_O, ctypes.POINTER(ctypes.c_size_t)]
        lib.gfr_gemm1_swiglu_quant.argtypes = [_T] * 5 + [ctypes.c_int] + [_T] * 2 + [
            ctypes.c_int, _P, _O]
        lib.gfr_w4a8_finalize_routing.argtypes = [_T] * 6 + [ctypes.c_int] + [_T] * 3 + [
            ctypes.c_float, ctypes.c_int64, _T, _P, _O]
        lib.gmm_finalize_routing_det_noalloc.argtypes = _DESC_MAIN_ARGS + [_P, _P]
        lib.gmm_finalize_routing_raw.argtypes = _RAW_MAIN_ARGS
        lib.gmm_finalize_routing_raw_ex.argtypes = _RAW_MAIN_ARGS + [_O]
        lib.gfr_workspace_size_raw.argtypes = [ctypes.c_int64] * 5 + [
            _O, ctypes.POINTER(ctypes.c_size_t)]
        lib.gfr_gemm1_swiglu_quant_raw.argtypes = [_P] * 5 + [ctypes.c_int] + [_P] * 2 + [
            ctypes.c_int] * 3 + [ctypes.c_int64] * 4 + [_P, _O]
        lib.gfr_w4a8_finalize_routing_raw.argtypes = [_P] * 6 + [ctypes.c_int] + [_P] * 3 + [
            ctypes.c_float, ctypes.c_int64, _P] + [ctypes.c_int64] * 6 + [_P, _O]
        for name in ("gmm_finalize_routing", "gmm_finalize_routing_ex", "gfr_workspace_size",
                     "gmm_finalize_routing_det_noalloc",
                     "gfr_gemm1_swiglu_quant", "gfr_w4a8_finalize_routing",
                     "gmm_finalize_routing_raw", "gmm_finalize_routing_raw_ex",
                     "gfr_workspace_size_raw", "gfr_gemm1_swiglu_quant_raw",
                     "gfr_w4a8_finalize_routing_raw"):
            getattr(lib, name).restype = ctypes.c_int
        lib.gfr_status_string.argtypes = [ctypes.c_int]
        lib.gfr_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(code: int) -> str:
    return load_library().gfr_status_string(code).decode()


def workspace_size(M: int, K: int, N: int, E: int, batch: int, deterministic: bool = False) -> int:
    """Workspace bytes of a call of these sizes (gfr_workspace_size_raw)."""
    opts = GfrOptions(int(deterministic), None, 0, None, 0, 0)
    n = ctypes.c_size_t(0)
    rc = load_library().gfr_workspace_size_raw(M, K, N, E, batch, ctypes.byref(opts),
                                               ctypes.byref(n))
    if rc:
        raise GfrError(rc, status_string(rc))
    return n.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _on_device(tensors, dev):
    """Device and layout checks the descriptors cannot carry."""
    for t in tensors:
        if t is not None:
            _need(t.is_cuda and t.device == dev, "all tensors must be on out's CUDA device")
            _need(t.is_contiguous(), "all tensors must be contiguous")


def gmm_finalize_routing(x1, x2, scale, pertoken_scale, group_list, group_list_type, logit,
                         row_index, shared_input, shared_input_weight, shared_input_offset,
                         out, transpose_x2=False, *, deterministic=False, workspace=None,
                         status=None, split_k=0, stream=None):
    """out += routed expert rows + shared term, in place; returns out.

    x1 [M,K] / x2 [E,K,N] (or [E,N,K] when transpose_x2) are float8_e4m3fn or
    float8_e5m2, or float4_e2m1fn_x2 (MXFP4: the last axis holds half as many
    bytes as elements); scale / pertoken_scale hold E8M0 codes (uint8 or
    float8_e8m0fnu); a 4-D scale (leading expert axis) is per expert;
    group_list int64 [E]; logit float32 [M] or None; row_index int64 or int32
    [M]; shared_input bfloat16 [R,N] or None; out float32 [batch,N].
    ``status`` (int32 CUDA tensor, 1 element) receives device-side data-error
    bits.  ``workspace`` (uint8 CUDA tensor) is allocated here when the
    deterministic mode needs one and none is given.  Dtypes, ranks and shapes
    are checked by the library (gmm_finalize_routing_ex), which raises
    GfrError here.
    """
    lib = load_library()
    dev = out.device
    _on_device([x1, x2, scale, pertoken_scale, group_list, row_index, out, logit, shared_input,
                workspace, status], dev)
    kind = {torch.float8_e4m3fn: 0, torch.float8_e5m2: 1, torch.float4_e2m1fn_x2: 2}.get(x1.dtype, -1)
    descs = [tensor_desc(t) for t in (x1, x2, scale, pertoken_scale, group_list)]
    lg, ri, sh, od = (tensor_desc(t) for t in (logit, row_index, shared_input, out))
    args = [_ref(d) for d in descs] + [int(group_list_type), _ref(lg), _ref(ri), _ref(sh),
                                       float(shared_input_weight), int(shared_input_offset),
                                       _ref(od), int(bool(transpose_x2)), kind]
    opts = GfrOptions(int(bool(deterministic)), None, 0, _ptr(status), int(split_k), 0)
    if deterministic:
        need = ctypes.c_size_t(0)
        rc = lib.gfr_workspace_size(*args, ctypes.byref(opts), ctypes.byref(need))
        if rc:
            raise GfrError(rc, status_string(rc))
        if workspace is None:
            workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = lib.gmm_finalize_routing_ex(*args, ctypes.c_void_p(stream), ctypes.byref(opts))
    if rc:
        raise GfrError(rc, status_string(rc))
    return out


def gmm_finalize_routing_det_noalloc(x1, x2, scale, pertoken_scale, group_list,
                                     group_list_type, logit, row_index, shared_input,
                                     shared_input_weight, shared_input_offset, out,
                                     transpose_x2=False, *, status=None, stream=None):
    """Deterministic gmm_finalize_routing whose workspace is the library's
    static per-GPU scratch (include/gfr.h, gmm_finalize_routing_det_noalloc):
    allocates nothing, so it may run where allocation is not allowed.  Calls
    that overlap in time on one GPU race on that scratch.  Arguments as
    gmm_finalize_routing; returns out."""
    lib = load_library()
    dev = out.device
    _on_device([x1, x2, scale, pertoken_scale, group_list, row_index, out, logit, shared_input,
                status], dev)
    kind = {torch.float8_e4m3fn: 0, torch.float8_e5m2: 1, torch.float4_e2m1fn_x2: 2}.get(x1.dtype, -1)
    descs = [tensor_desc(t) for t in (x1, x2, scale, pertoken_scale, group_list)]
    lg, ri, sh, od = (tensor_desc(t) for t in (logit, row_index, shared_input, out))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = lib.gmm_finalize_routing_det_noalloc(
            *[_ref(d) for d in descs], int(group_list_type), _ref(lg), _ref(ri), _ref(sh),
            float(shared_input_weight), int(shared_input_offset), _ref(od),
            int(bool(transpose_x2)), kind, ctypes.c_void_p(stream), _ptr(status))
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
    dev = xin.device
    _need(xin.dim() == 2 and w13.dim() == 3, "xin must be 2-D and w13 3-D")
    M = xin.shape[0]
    N2 = w13.shape[1] if transpose_w13 else w13.shape[2]
    I = N2 // 2
    if x1_out is None:
        x1_out = torch.zeros((M, I), dtype=torch.uint8, device=dev).view(out_dtype)
    if x1_scale_out is None:
        x1_scale_out = torch.zeros((M, (I + 63) // 64, 2), dtype=torch.uint8, device=dev)
    _need(x1_out.dtype == out_dtype, "x1_out must have out_dtype")
    _on_device([xin, w13, scale, xin_scale, group_list, x1_out, x1_scale_out, status], dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    opts = GfrOptions(0, None, 0, _ptr(status), 0, 0)
    d = [tensor_desc(t) for t in (xin, w13, scale, xin_scale, group_list)]
    dq, dqs = tensor_desc(x1_out), tensor_desc(x1_scale_out)
    with torch.cuda.device(dev):
        rc = lib.gfr_gemm1_swiglu_quant(
            *[_ref(x) for x in d], int(group_list_type), _ref(dq), _ref(dqs),
            int(bool(transpose_w13)), ctypes.c_void_p(stream), ctypes.byref(opts))
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
    dev = out.device
    _on_device([x1, x2, scale, offset, pertoken_scale, group_list, row_index, out, logit,
                shared_input, workspace, status], dev)
    _need(x1.dim() == 2 and x2.dim() == 3 and out.dim() == 2, "x1 [M, K], x2 [E, K, N/2], out 2-D")
    ws_bytes = 0
    if deterministic:
        M, K, E, N = x1.shape[0], x1.shape[1], x2.shape[0], 2 * x2.shape[2]
        need = workspace_size(M, K, N, E, out.shape[0], True)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    opts = GfrOptions(int(bool(deterministic)), _ptr(workspace), ws_bytes, _ptr(status),
                      int(split_k), 0)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    d = [tensor_desc(t) for t in (x1, x2, scale, offset, pertoken_scale, group_list)]
    lg, ri, sh, od = (tensor_desc(t) for t in (logit, row_index, shared_input, out))
    with torch.cuda.device(dev):
        rc = lib.gfr_w4a8_finalize_routing(
            *[_ref(x) for x in d], int(group_list_type), _ref(lg), _ref(ri), _ref(sh),
            float(shared_input_weight), int(shared_input_offset), _ref(od),
            ctypes.c_void_p(stream), ctypes.byref(opts))
    if rc:
        raise GfrError(rc, status_string(rc))
    return out
