"""Pins of the upstream-step oracle (oracle.gemm1): gate||up grouped matmul,
SwiGLU, MX block quantisation.  CPU only.

Each pin checks the oracle against something other than itself: torch's own
float8 casts and decoders, scipy's logistic function, closed forms of the MX
block exponent, and an independent numpy/torch formulation of the whole step
(tests/tiny_inputs.numpy_reference for the matmul, scipy.special.expit for
SiLU, torch casts for the element encoding).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import gemm1 as g1
from tests.tiny_inputs import decode_np, numpy_reference, tiny_case

_F8 = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}
_MAX = {0: 448.0, 1: 57344.0}
_EMAX = {0: 8, 1: 15}
_MAXCODE = {0: 0x7E, 1: 0x7B}


def _finite(kind):
    c = np.arange(256, dtype=np.uint8)
    v = decode_np(c, kind)
    return c[np.isfinite(v)], v[np.isfinite(v)]


def _torch_encode(v, kind):
    """Independent encoding: clamp into range, float32, torch's RNE cast."""
    v = np.clip(np.asarray(v, np.float64), -_MAX[kind], _MAX[kind]).astype(np.float32)
    return torch.from_numpy(v).to(_F8[kind]).view(torch.uint8).numpy()


@pytest.mark.parametrize("kind", [0, 1])
def test_encode_decode_round_trip_every_code(kind):
    codes, vals = _finite(kind)
    assert np.array_equal(g1.fp8_encode(vals, kind), codes)
    assert np.array_equal(g1.fp8_decode(codes, kind), vals)


@pytest.mark.parametrize("kind", [0, 1])
def test_encode_matches_torch_cast_including_ties(kind):
    codes, vals = _finite(kind)
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2          # exact ties: to the even code
    rng = np.random.default_rng(5)
    lo = math.log2(pos[1]) - 2
    rnd = np.exp2(rng.uniform(lo, math.log2(_MAX[kind]), 4000)) * rng.choice([-1, 1], 4000)
    for v in (mids, -mids, rnd.astype(np.float32).astype(np.float64)):
        assert np.array_equal(g1.fp8_encode(v, kind), _torch_encode(v, kind))


@pytest.mark.parametrize("kind", [0, 1])
def test_encode_saturates(kind):
    big = np.array([_MAX[kind] * 1.0625, _MAX[kind] * 1.5, 1e30, -1e30, -_MAX[kind] * 2])
    assert list(g1.fp8_encode(big, kind)) == [_MAXCODE[kind]] * 3 + [0x80 | _MAXCODE[kind]] * 2


@pytest.mark.parametrize("kind", [0, 1])
def test_block_exponent_closed_forms(kind):
    em = _EMAX[kind]
    for k in (-20, -3, 0, 1, 7):
        assert g1.block_exponent(_MAX[kind] * 2.0 ** k, kind) == k          # largest finite
        assert g1.block_exponent(2.0 ** (em + k), kind) == k
        assert g1.block_exponent(np.nextafter(2.0 ** (em + k + 1), 0), kind) == k
    assert g1.block_exponent(0.0, kind) == -127
    assert g1.block_exponent(1e-300, kind) == -127
    assert g1.block_exponent(2.0 ** 200, kind) == 127


@pytest.mark.parametrize("kind", [0, 1])
def test_mx_quantize_blocks_layout_and_error(kind):
    rng = np.random.default_rng(7)
    I = 96                                           # three 32-blocks, last 64-pair half empty
    v = rng.standard_normal((4, I))
    v[:, 32:64] *= 2.0 ** 20                         # a block with much larger values
    v[1, 64:] = 0.0                                  # an all-zero block
    codes, scales, X = g1.mx_quantize(v, kind)
    assert scales.shape == (4, 2, 2)
    for j in range(3):
        amax = np.abs(v[:, 32 * j: 32 * j + 32]).max(axis=1)
        want = [math.floor(math.log2(a)) - _EMAX[kind] if a > 0 else -127 for a in amax]
        assert list(X[:, j]) == want
        assert list(scales.reshape(4, 4)[:, j]) == [x + 127 for x in want]
    assert (scales.reshape(4, 4)[:, 3] == 0).all()
    # dequantised values are within half a unit in the last place of the code,
    # except that scaled magnitudes above the largest finite value (possible:
    # the block maximum scales into [2^emax, 2^(emax+1)), past 448 for E4M3)
    # saturate to it
    Xe = np.repeat(X, 32, axis=1)[:, :I]
    y = v / np.exp2(Xe)
    dq = decode_np(codes, kind) * np.exp2(Xe)
    mbits = 3 if kind == 0 else 2
    _, ex = np.frexp(np.abs(y))
    emin = -6 if kind == 0 else -14
    half_ulp = np.exp2(np.maximum(ex - 1, emin) - mbits - 1 + Xe)
    sat = np.abs(y) >= _MAX[kind] + 2.0 ** (_EMAX[kind] - mbits - 1)
    assert np.all(np.abs(dq - v)[~sat] <= half_ulp[~sat])
    assert np.all((codes[sat] & 0x7F) == _MAXCODE[kind])
    assert np.all(np.abs(y) < 2.0 ** (_EMAX[kind] + 1))
    assert np.all(codes[1, 64:] == 0)


def test_silu_identities_and_scipy():
    x = np.linspace(-30, 30, 2001)
    assert np.allclose(g1.silu(x), x * scipy.special.expit(x), rtol=1e-14, atol=1e-300)
    assert np.allclose(g1.silu(x) - g1.silu(-x), x, rtol=1e-13, atol=1e-13)
    assert g1.silu(0.0) == 0.0 and g1.silu(1000.0) == 1000.0
    s = g1.silu(-1000.0)
    assert s == 0.0 and not np.isnan(s)


@pytest.mark.parametrize("transpose", [False, True])
def test_gate_up_order_one_hot(transpose):
    """One token, unit scales, x = e_0: gate_up row = row 0 of w13, so
    sw[i] = SiLU(w13[0, i]) * w13[0, I + i]; swapping the halves would give
    SiLU(up) * gate instead."""
    kind, H, I = 0, 64, 32
    gate_vals = np.linspace(-3, 3, I)
    up_vals = np.linspace(0.5, 2, I)
    xin = np.zeros((1, H), np.uint8)
    xin[0, 0] = _torch_encode([1.0], kind)[0]
    row = _torch_encode(np.concatenate([gate_vals, up_vals]), kind)
    w = np.zeros((1, H, 2 * I), np.uint8)
    w[0, 0] = row
    scale = np.full((1, 2 * I, 2), 127, np.uint8)
    if transpose:
        w = np.ascontiguousarray(w.transpose(0, 2, 1))
        scale = np.full((2 * I, 1, 2), 127, np.uint8)
    r = g1.gemm1_swiglu_quant(xin, w, scale, np.full((1, 1, 2), 127, np.uint8),
                              np.array([1]), 1, transpose, kind, kind)
    gq, uq = decode_np(row[:I], kind), decode_np(row[I:], kind)
    assert np.allclose(r["sw"][0], gq * scipy.special.expit(gq) * uq, rtol=1e-14)


CASES = [dict(seed=200 + i, E=E, M=M, K=H, N=2 * I, transpose=tr, kind=kd, gtype=gt)
         for i, (E, M, H, I, tr, kd, gt) in enumerate([
             (1, 4, 64, 32, False, 0, 1), (3, 9, 128, 64, True, 1, 0),
             (4, 12, 96, 48, False, 1, 1), (2, 7, 192, 96, True, 0, 0),
             (5, 20, 256, 40, False, 0, 0)])]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
@pytest.mark.parametrize("out_kind", [0, 1])
def test_gemm1_tiny_matches_independent(case, out_kind):
    c = tiny_case(**case, routing="identity", logit="ones", shared=False)
    c["out_init"] = np.zeros_like(c["out_init"])
    r = g1.gemm1_swiglu_quant(c["x1"], c["x2"], c["scale"], c["pertoken_scale"],
                              c["group_list"], c["group_list_type"], c["transpose_x2"],
                              c["fp8_kind"], out_kind)
    gu = numpy_reference(c)                       # np.matmul per expert, identity routing
    I = case["N"] // 2
    mag = np.concatenate([r["gmag"], r["umag"]], axis=1)
    assert np.all(np.abs(np.concatenate([r["gate"], r["up"]], axis=1) - gu) <= 1e-13 * mag)
    sw = gu[:, :I] * scipy.special.expit(gu[:, :I]) * gu[:, I:]
    assert np.allclose(r["sw"], sw, rtol=1e-12, atol=1e-300)
    # independent quantisation: math.log2 for the block exponent, torch's cast
    for t in range(sw.shape[0]):
        for j in range((I + 31) // 32):
            blk = sw[t, 32 * j: 32 * j + 32]
            a = np.abs(blk).max()
            x = max(math.floor(math.log2(a)) - _EMAX[out_kind], -127) if a > 0 else -127
            assert r["X"][t, j] == x
            assert r["scales"].reshape(sw.shape[0], -1)[t, j] == x + 127
            want = _torch_encode(blk / 2.0 ** x, out_kind)
            got = r["codes"][t, 32 * j: 32 * j + 32]
            # zero results may carry either sign bit; compare values there
            assert np.array_equal(decode_np(got, out_kind), decode_np(want, out_kind))
    start, counts = 0, (np.diff(np.concatenate([[0], c["group_list"]])) if case["gtype"] == 0
                        else c["group_list"])
    assert r["routed"].sum() == counts.sum() and r["routed"][:counts.sum()].all()


def test_rows_selection_matches_full():
    c = tiny_case(seed=9, E=3, M=10, K=128, N=64, transpose=False, kind=0, gtype=1,
                  routing="identity", logit="ones", shared=False)
    args = (c["x1"], c["x2"], c["scale"], c["pertoken_scale"], c["group_list"], 1, False, 0, 0)
    full = g1.gemm1_swiglu_quant(*args)
    part = g1.gemm1_swiglu_quant(*args, rows=[7, 2])
    for k in ("sw", "codes", "X"):
        assert np.array_equal(part[k], full[k][[7, 2]])
