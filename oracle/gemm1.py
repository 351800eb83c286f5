"""CPU oracle for the upstream step of the MoE FFN: grouped gate||up matmul,
SwiGLU, and MX block quantisation of the result into the FP8 codes + E8M0
scales that the finalize-routing operator takes as x1 / pertoken_scale.

TEST INFRASTRUCTURE ONLY (like the rest of this package): the tests, the smoke
check and the benchmark's CPU-baseline leg use it; the GPU library never does.

Sources:
  [P1] "基于 PyPTO 的 MoE 融合算子实践：grouped_matmul_finalize_routing 的 MXFP8
       实现与精度验证": the MXFP8 operand format (FP8 codes, one E8M0 scale per
       32 K elements in [.., ceil(K/64), 2] layouts) and its dequantisation.
  [P2] "LLaDA2.0-mini MoE 融合算子实战：基于 PyPTO 的 Grouped GEMM 单内核实现"
       §3.1 (w13 holds each expert's gate and up projections side by side,
       width 2I), §3.2 (gate_up = x @ w13_e accumulated in FP32, then
       SwiGLU), §3.3 (the first I columns are gate, the last I are up;
       SiLU(g) = g / (1 + exp(-g)); result SiLU(gate) * up).

Everything is double precision.  The matmul is the finalize-routing oracle's
own definition (gfr_oracle.c) evaluated with identity routing: row t of the
output is token t, weight 1, zero initial value, no shared term; N = 2I.

MX quantisation (the pages define only the dequantisation, value * 2^(s-127)
per 32-element block; the encoding side is read as the OCP Microscaling
format's conversion):
  * blocks of 32 consecutive elements along the row (the K axis of the next
    matmul), block j covering [32j, 32j + 32); its scale byte goes to
    [t, j // 2, j % 2] of a [M, ceil(I/64), 2] array (the layout of
    pertoken_scale);
  * block exponent X = floor(log2(amax)) - emax, where amax is the block's
    largest magnitude and emax the exponent of the element format's largest
    normal (E4M3FN 8: 448 = 1.75 * 2^8; E5M2 15: 57344 = 1.75 * 2^15),
    clamped to [-127, 127]; an all-zero block gets X = -127; scale byte X + 127;
  * each element v is encoded as the FP8 code nearest to v / 2^X, ties to the
    even code, magnitudes above the largest finite value saturating to it.
"""
from __future__ import annotations

import numpy as np

from . import expert_ranges, gmm_finalize_routing, mx_group_slack

# Element formats: (exponent bias, mantissa bits, largest finite code, emax)
_FMT = {
    0: (7, 3, 0x7E, 8),    # E4M3FN: largest finite 448 = 0 1111 110
    1: (15, 2, 0x7B, 15),  # E5M2: largest finite 57344 = 0 11110 11
}


def silu(g):
    """SiLU as [P2] §3.3 composes it: g / (1 + exp(-g)), float64.  Large
    negative g overflow exp to inf and give -0.0, the limit."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def fp8_encode(y, kind: int) -> np.ndarray:
    """FP8 code nearest to y (float64 array), ties to even, saturating.

    With e = max(floor(log2|y|), emin) (emin = 1 - bias, the smallest normal
    exponent) the representable magnitudes near |y| are multiples of
    2^(e - mbits); r = round_half_even(|y| / 2^(e - mbits)) lies in
    [2^mbits, 2^(mbits+1)] for normal e (or [0, 2^mbits] below the smallest
    normal), and the code is ((e + bias) << mbits) + r - 2^mbits, which also
    carries r = 2^(mbits+1) into the next exponent.  The sign bit is the
    sign of y (a negative value that rounds to zero gives the negative zero
    code)."""
    bias, mbits, maxcode, _ = _FMT[kind]
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    emin = 1 - bias
    _, ex = np.frexp(a)                      # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, emin)
    r = np.rint(np.ldexp(a, (mbits - e).astype(np.int64)))   # numpy rint: ties to even
    code = ((e + bias) << mbits) + r.astype(np.int64) - (1 << mbits)
    code = np.where(a == 0, 0, code)
    code = np.minimum(code, maxcode)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def fp8_decode(codes, kind: int) -> np.ndarray:
    """Value of each FP8 code (finite codes only), float64."""
    bias, mbits, _, _ = _FMT[kind]
    c = np.asarray(codes, np.int64)
    ef = (c >> mbits) & ((1 << (7 - mbits)) - 1)
    mf = c & ((1 << mbits) - 1)
    mag = np.where(ef == 0, np.ldexp(mf.astype(np.float64), 1 - bias - mbits),
                   np.ldexp((mf + (1 << mbits)).astype(np.float64), ef - bias - mbits))
    return np.where(c & 0x80, -mag, mag)


def block_exponent(amax, kind: int) -> np.ndarray:
    """X = clamp(floor(log2(amax)) - emax, -127, 127); -127 for amax = 0."""
    emax = _FMT[kind][3]
    amax = np.asarray(amax, np.float64)
    _, ex = np.frexp(amax)
    x = np.where(amax > 0, ex - 1 - emax, -127)
    return np.clip(x, -127, 127).astype(np.int64)


def mx_quantize(v, kind: int):
    """MX-quantise rows of v (float64 [R, I]) in 32-element blocks.

    Returns (codes uint8 [R, I], scales uint8 [R, ceil(I/64), 2], X int64
    [R, ceil(I/32)]).  Scale entries past the last block (I % 64 in (0, 32])
    are 0."""
    v = np.asarray(v, np.float64)
    R, I = v.shape
    nb = (I + 31) // 32
    X = np.zeros((R, nb), np.int64)
    codes = np.zeros((R, I), np.uint8)
    for j in range(nb):
        blk = v[:, 32 * j: 32 * j + 32]
        X[:, j] = block_exponent(np.max(np.abs(blk), axis=1), kind)
        codes[:, 32 * j: 32 * j + 32] = fp8_encode(np.ldexp(blk, -X[:, j:j + 1]), kind)
    scales = np.zeros((R, (I + 63) // 64 * 2), np.uint8)
    scales[:, :nb] = (X + 127).astype(np.uint8)
    return codes, scales.reshape(R, (I + 63) // 64, 2), X


def routed_tokens(group_list, group_list_type: int, M: int) -> np.ndarray:
    """Boolean [M]: token t lies in some expert's range ([P1] §4.3)."""
    start, end = expert_ranges(group_list, group_list_type, M)
    mask = np.zeros(M, bool)
    for s, e in zip(start, end):
        mask[s:e] = True
    return mask


def gemm1_swiglu_quant(xin, w13, scale, xin_scale, group_list, group_list_type,
                       transpose_w13, fp8_kind, out_kind, rows=None, with_slack=False):
    """The upstream step on host arrays.

    xin [M, H], w13 [E, H, 2I] (or [E, 2I, H] with transpose_w13), scale
    [ceil(H/64), 2I, 2] (or [2I, ceil(H/64), 2]; a leading [E] axis for
    per-expert scales), xin_scale [M, ceil(H/64), 2]: uint8 codes.  rows:
    token indices to evaluate (default: all).

    Returns a dict of float64 arrays over the selected tokens: gate, up (the
    two halves of gate_up), gmag, umag (sums of term magnitudes, for
    tolerances), sw = SiLU(gate) * up; codes / scales / X from mx_quantize of
    sw in out_kind; routed (bool: the token belongs to an expert; other
    tokens are not produced); and, with with_slack, gslack / uslack, the
    MFMA group-truncation bound of gate and up (mx_group_slack)."""
    M = xin.shape[0]
    N2 = w13.shape[1] if transpose_w13 else w13.shape[2]
    assert N2 % 2 == 0
    I = N2 // 2
    ident = np.arange(M, dtype=np.int64)
    sel = ident if rows is None else np.asarray(rows, np.int64)
    gu, mag = gmm_finalize_routing(xin, w13, scale, xin_scale, group_list, group_list_type,
                                   None, ident, None, 0.0, 0, np.zeros((M, N2), np.float32),
                                   transpose_w13, fp8_kind, rows=sel)
    gate, up = gu[:, :I], gu[:, I:]
    sw = silu(gate) * up
    codes, scales, X = mx_quantize(sw, out_kind)
    res = dict(gate=gate, up=up, gmag=mag[:, :I], umag=mag[:, I:], sw=sw, codes=codes,
               scales=scales, X=X, routed=routed_tokens(group_list, group_list_type, M)[sel])
    if with_slack:
        sl = mx_group_slack(xin, w13, scale, xin_scale, group_list, group_list_type, None,
                            ident, transpose_w13, fp8_kind, M, rows=sel)
        res["gslack"], res["uslack"] = sl[:, :I], sl[:, I:]
    return res
