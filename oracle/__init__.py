"""CPU oracle for the fused MXFP8 grouped-matmul + finalize-routing operator.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the GPU library (``mxfp8_grouped_gemm_group_amd``) and never imports it.

The arithmetic lives in ``gfr_oracle.c`` (plain C, double precision, built with
gcc into ``liboracle.so``); this module only marshals numpy arrays to it.  See
the header of ``gfr_oracle.c`` for the operator's definition and the pages each
step follows.  ``oracle.gemm1`` adds the upstream step of the MoE FFN (gate||up
matmul through the same C definition, SwiGLU and MX block quantisation in
float64 numpy).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gfr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ERRORS = {
    0: "ok",
    -1: "bad argument",
    -2: "bad group_list",
    -3: "row_index out of range",
    -4: "shared range out of bounds",
    -5: "out of memory",
}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle error {code}: {ERRORS.get(code, 'unknown')}")
        self.code = code


def build() -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math; OpenMP spreads
    independent output rows over threads, each row computed whole by one)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
         "-fno-fast-math", "-fopenmp", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib_handle: Optional[ctypes.CDLL] = None


def _lib() -> ctypes.CDLL:
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        for name in ("oracle_decode_e4m3fn", "oracle_decode_e5m2", "oracle_decode_e8m0",
                     "oracle_decode_e2m1"):
            f = getattr(lib, name)
            f.argtypes = [ctypes.c_uint8]
            f.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_expert_ranges.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_expert_ranges.restype = ctypes.c_int
        p, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_gmm_finalize_routing.argtypes = [
            p, p, p, i32, p,          # x1 x2 scale scale_per_expert pertoken_scale
            p, i32, p, p, p,          # group_list type logit row_index shared_input
            dbl, i64, i64, p,         # shared weight, offset, rows, out_init
            i32, i32,                 # transpose_x2 fp8_kind
            i64, i64, i64, i64, i64,  # M K N E batch
            p, i64, p, p]             # rows n_rows res mag
        lib.oracle_gmm_finalize_routing.restype = ctypes.c_int
        lib.oracle_mx_group_slack.argtypes = [
            p, p, p, i32, p, p, i32, p, p, i32, i32, i64, i64, i64, i64, i64, p, i64, p]
        lib.oracle_mx_group_slack.restype = ctypes.c_int
        lib.oracle_w4a8_finalize_routing.argtypes = [
            p, p, p, p, p,            # x1 x2 scale offset pertoken_scale
            p, i32, p, p, p,          # group_list type logit row_index shared_input
            dbl, i64, i64, p,         # shared weight, offset, rows, out_init
            i64, i64, i64, i64, i64,  # M K N E batch
            p, i64, p, p]             # rows n_rows res mag
        lib.oracle_w4a8_finalize_routing.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib_handle = lib
    return _lib_handle


def num_threads() -> int:
    """Threads the oracle's output-row loop runs on (OMP_NUM_THREADS, else all cores)."""
    return int(_lib().oracle_num_threads())


def decode(kind: str, code: int) -> float:
    """Decode one code; kind in {'e4m3fn', 'e5m2', 'e2m1', 'e8m0', 'bf16'}."""
    lib = _lib()
    return {
        "e4m3fn": lib.oracle_decode_e4m3fn,
        "e5m2": lib.oracle_decode_e5m2,
        "e2m1": lib.oracle_decode_e2m1,
        "e8m0": lib.oracle_decode_e8m0,
        "bf16": lib.oracle_decode_bf16,
    }[kind](code)


E2M1 = 2   # element kind of the MXFP4 variant: two E2M1 codes per byte


def _logical_sizes(x1, x2, transpose_x2, fp8_kind):
    """(M, K, N, E) from the stored arrays; E2M1 rows hold two elements per byte."""
    per = 2 if fp8_kind == E2M1 else 1
    M, K = x1.shape[0], x1.shape[1] * per
    E = x2.shape[0]
    N = x2.shape[1] if transpose_x2 else x2.shape[2] * per
    return M, K, N, E


def expert_ranges(group_list, group_list_type: int, M: int):
    """(start, end) int64 arrays of each expert's token range; raises on bad input."""
    g = np.ascontiguousarray(group_list, dtype=np.int64)
    E = g.shape[0]
    start = np.zeros(E, np.int64)
    end = np.zeros(E, np.int64)
    rc = _lib().oracle_expert_ranges(g.ctypes.data, E, group_list_type, M,
                                     start.ctypes.data, end.ctypes.data)
    if rc:
        raise OracleError(rc)
    return start, end


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError(f"expected raw uint8 codes, got {a.dtype}")
    return a


def gmm_finalize_routing(x1, x2, scale, pertoken_scale, group_list, group_list_type,
                         logit, row_index, shared_input, shared_input_weight,
                         shared_input_offset, out_init, transpose_x2, fp8_kind,
                         rows=None):
    """Run the oracle on host numpy arrays.

    x1, x2, scale, pertoken_scale: uint8 codes (FP8 / E8M0; with fp8_kind 2
    x1 and x2 hold two E2M1 codes per byte along their last axis); shared_input:
    uint16 bf16 bit patterns or None; logit: float32 or None; group_list and
    row_index: int64; out_init: float32 [batch, N].  ``scale`` may carry a
    leading expert axis (4-D).  ``rows`` selects output rows (default: all).

    Returns (out, mag), float64 arrays of shape [len(rows), N].
    """
    x1 = _u8(x1)
    x2 = _u8(x2)
    scale = _u8(scale)
    pts = _u8(pertoken_scale)
    g = np.ascontiguousarray(group_list, dtype=np.int64)
    ri = np.ascontiguousarray(row_index, dtype=np.int64)
    init = np.ascontiguousarray(out_init, dtype=np.float32)
    M, K, N, E = _logical_sizes(x1, x2, transpose_x2, fp8_kind)
    batch = init.shape[0]
    assert init.shape == (batch, N)
    scale_per_expert = 1 if scale.ndim == 4 else 0
    lg = None if logit is None else np.ascontiguousarray(logit, dtype=np.float32)
    sh = None if shared_input is None else np.ascontiguousarray(shared_input, dtype=np.uint16)
    R = 0 if sh is None else sh.shape[0]
    if rows is None:
        rows_arr = None
        n_rows = batch
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows_arr.shape[0]
    res = np.zeros((n_rows, N), np.float64)
    mag = np.zeros((n_rows, N), np.float64)
    rc = _lib().oracle_gmm_finalize_routing(
        x1.ctypes.data, x2.ctypes.data, scale.ctypes.data, scale_per_expert, pts.ctypes.data,
        g.ctypes.data, int(group_list_type),
        None if lg is None else lg.ctypes.data, ri.ctypes.data,
        None if sh is None else sh.ctypes.data,
        float(shared_input_weight), int(shared_input_offset), R, init.ctypes.data,
        int(bool(transpose_x2)), int(fp8_kind), M, K, N, E, batch,
        None if rows_arr is None else rows_arr.ctypes.data, n_rows,
        res.ctypes.data, mag.ctypes.data)
    if rc:
        raise OracleError(rc)
    return res, mag


def mx_group_slack(x1, x2, scale, pertoken_scale, group_list, group_list_type, logit,
                   row_index, transpose_x2, fp8_kind, batch, rows=None):
    """Per-element bound on the extra error of a dot-product unit that sums
    runs of 8 consecutive K products aligned to the largest one and truncated
    13 bits below it (see oracle_mx_group_slack in gfr_oracle.c).  Not part
    of the operator: a tolerance term.  Returns float64 [len(rows), N]."""
    x1 = _u8(x1)
    x2 = _u8(x2)
    scale = _u8(scale)
    pts = _u8(pertoken_scale)
    g = np.ascontiguousarray(group_list, dtype=np.int64)
    ri = np.ascontiguousarray(row_index, dtype=np.int64)
    M, K, N, E = _logical_sizes(x1, x2, transpose_x2, fp8_kind)
    lg = None if logit is None else np.ascontiguousarray(logit, dtype=np.float32)
    if rows is None:
        rows_arr, n_rows = None, batch
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows_arr.shape[0]
    out = np.zeros((n_rows, N), np.float64)
    rc = _lib().oracle_mx_group_slack(
        x1.ctypes.data, x2.ctypes.data, scale.ctypes.data, 1 if scale.ndim == 4 else 0,
        pts.ctypes.data, g.ctypes.data, int(group_list_type),
        None if lg is None else lg.ctypes.data, ri.ctypes.data, int(bool(transpose_x2)),
        int(fp8_kind), M, K, N, E, batch,
        None if rows_arr is None else rows_arr.ctypes.data, n_rows, out.ctypes.data)
    if rc:
        raise OracleError(rc)
    return out


def within_tolerance(got, ref, mag, rel=2e-5, abs_=1e-6):
    """Per-element acceptance |got - ref| <= rel * mag + abs_; returns (ok, worst ratio)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = rel * mag + abs_
    ratio = float(np.max(err / bound)) if err.size else 0.0
    return bool(np.all(err <= bound)), ratio


def w4a8_finalize_routing(x1, x2, scale, offset, pertoken_scale, group_list, group_list_type,
                          logit, row_index, shared_input, shared_input_weight,
                          shared_input_offset, out_init, rows=None):
    """The A2/A3 W4A8 variant (oracle_w4a8_finalize_routing in gfr_oracle.c).

    x1 int8 [M, K]; x2 uint8 [E, K, N/2] (two signed 4-bit values per byte
    along n, element 2j in the low nibble); scale and offset (or None)
    float32 [E, 1, N]; pertoken_scale float32 [M]; the rest as
    gmm_finalize_routing.  Returns (out, mag) float64 [len(rows), N]."""
    x1 = np.ascontiguousarray(x1)
    if x1.dtype != np.int8:
        raise TypeError(f"x1 must be int8, got {x1.dtype}")
    x2 = _u8(x2)
    sc = np.ascontiguousarray(scale, dtype=np.float32)
    of = None if offset is None else np.ascontiguousarray(offset, dtype=np.float32)
    pts = np.ascontiguousarray(pertoken_scale, dtype=np.float32)
    g = np.ascontiguousarray(group_list, dtype=np.int64)
    ri = np.ascontiguousarray(row_index, dtype=np.int64)
    init = np.ascontiguousarray(out_init, dtype=np.float32)
    M, K = x1.shape
    E, N = x2.shape[0], x2.shape[2] * 2
    assert x2.shape[1] == K and sc.shape == (E, 1, N) and pts.shape == (M,)
    assert of is None or of.shape == (E, 1, N)
    batch = init.shape[0]
    lg = None if logit is None else np.ascontiguousarray(logit, dtype=np.float32)
    sh = None if shared_input is None else np.ascontiguousarray(shared_input, dtype=np.uint16)
    R = 0 if sh is None else sh.shape[0]
    if rows is None:
        rows_arr, n_rows = None, batch
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows_arr.shape[0]
    res = np.zeros((n_rows, N), np.float64)
    mag = np.zeros((n_rows, N), np.float64)
    rc = _lib().oracle_w4a8_finalize_routing(
        x1.ctypes.data, x2.ctypes.data, sc.ctypes.data, None if of is None else of.ctypes.data,
        pts.ctypes.data, g.ctypes.data, int(group_list_type),
        None if lg is None else lg.ctypes.data, ri.ctypes.data,
        None if sh is None else sh.ctypes.data, float(shared_input_weight),
        int(shared_input_offset), R, init.ctypes.data, M, K, N, E, batch,
        None if rows_arr is None else rows_arr.ctypes.data, n_rows,
        res.ctypes.data, mag.ctypes.data)
    if rc:
        raise OracleError(rc)
    return res, mag
