"""Pins of the W4A8 oracle (oracle.w4a8_finalize_routing): INT8 x INT4 with a
fused per-channel FP32 scale, FP32 per-token scale, optional asymmetric offset,
then the finalize routing.  CPU only.

The independent reference unpacks the nibbles with numpy bit operations,
does the products with numpy's int64 matmul per expert, applies the scales in
float64 and routes with np.add.at; the shared rows are decoded by torch.
"""
import numpy as np
import pytest

import oracle
from tests.tiny_inputs import decode_np


def unpack_int4(packed):
    """[..., N/2] bytes -> [..., N] signed values, element 2j from the low nibble."""
    lo = (packed & 15).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.int64)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out


def case(seed, E, M, K, N, gtype, offset=True, shared=True, groups=None, batch=None):
    rng = np.random.default_rng(seed)
    x1 = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    x2 = rng.integers(0, 256, size=(E, K, N // 2)).astype(np.uint8)
    scale = rng.uniform(0.001, 0.01, size=(E, 1, N)).astype(np.float32)
    off = rng.uniform(-0.01, 0.01, size=(E, 1, N)).astype(np.float32) if offset else None
    pts = rng.uniform(0.5, 2.0, size=M).astype(np.float32)
    if groups is None:
        cuts = np.sort(rng.integers(0, M + 1, size=E - 1))
        counts = np.diff(np.concatenate([[0], cuts, [M]])).astype(np.int64)
    else:
        counts = np.asarray(groups, np.int64)
    gl = np.cumsum(counts) if gtype == 0 else counts
    batch = batch or max(2, M // 2)
    ri = rng.integers(0, batch, size=M).astype(np.int64)
    lg = rng.random(M, dtype=np.float32)
    if shared:
        R = int(rng.integers(1, batch + 1))
        soff = int(rng.integers(0, batch - R + 1))
        import torch
        sh = torch.from_numpy(rng.standard_normal((R, N)).astype(np.float32)).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        sh, soff = None, 0
    init = rng.standard_normal((batch, N)).astype(np.float32)
    return dict(x1=x1, x2=x2, scale=scale, offset=off, pertoken_scale=pts, group_list=gl,
                group_list_type=gtype, logit=lg, row_index=ri, shared_input=sh,
                shared_input_weight=0.75, shared_input_offset=soff, out_init=init)


def run(c, **over):
    d = dict(c, **over)
    return oracle.w4a8_finalize_routing(
        d["x1"], d["x2"], d["scale"], d["offset"], d["pertoken_scale"], d["group_list"],
        d["group_list_type"], d["logit"], d["row_index"], d["shared_input"],
        d["shared_input_weight"], d["shared_input_offset"], d["out_init"])


def reference(c):
    x = c["x1"].astype(np.int64)
    w = unpack_int4(c["x2"])
    counts = (np.diff(np.concatenate([[0], c["group_list"]])) if c["group_list_type"] == 0
              else c["group_list"])
    out = c["out_init"].astype(np.float64).copy()
    start = 0
    for e, n in enumerate(counts):
        r = slice(start, start + int(n))
        P = (x[r] @ w[e]).astype(np.float64)                 # exact int64 products
        S = x[r].sum(axis=1, keepdims=True).astype(np.float64)
        y = P * c["scale"][e, 0].astype(np.float64)
        if c["offset"] is not None:
            y = y + S * c["offset"][e, 0].astype(np.float64)
        y *= (c["pertoken_scale"][r] * 1.0).astype(np.float64)[:, None]
        y *= c["logit"][r].astype(np.float64)[:, None]
        np.add.at(out, c["row_index"][r], y)
        start += int(n)
    if c["shared_input"] is not None:
        sh = decode_np(c["shared_input"], "bf16")
        o = c["shared_input_offset"]
        out[o:o + sh.shape[0]] += c["shared_input_weight"] * sh
    return out


CASES = [(1, 4, 64, 8, 1, True), (3, 11, 128, 32, 0, True), (4, 20, 192, 64, 1, False),
         (2, 9, 64, 512, 0, True), (5, 30, 320, 40, 1, False)]


@pytest.mark.parametrize("E,M,K,N,gtype,offset", CASES)
def test_matches_independent_numpy(E, M, K, N, gtype, offset):
    c = case(7 + E * M, E, M, K, N, gtype, offset=offset)
    got, mag = run(c)
    ref = reference(c)
    assert np.all(np.abs(got - ref) <= 1e-13 * mag + 1e-300)


def test_every_byte_value_decodes():
    """x1 = e_k, unit scales, identity routing: the output row is weight row k,
    so all 256 byte values placed in one row read back as their two nibbles."""
    N, K = 512, 64
    c = case(3, 1, 1, K, N, 1, offset=False, shared=False, groups=[1], batch=1)
    c["x1"] = np.zeros((1, K), np.int8)
    c["x1"][0, 5] = 1
    c["x2"][0, 5] = np.arange(256, dtype=np.uint8)
    c.update(scale=np.ones((1, 1, N), np.float32), pertoken_scale=np.ones(1, np.float32),
             logit=np.ones(1, np.float32), row_index=np.zeros(1, np.int64),
             out_init=np.zeros((1, N), np.float32))
    got, _ = run(c)
    b = np.arange(256)
    want = np.empty(N)
    want[0::2] = ((b & 15) ^ 8) - 8
    want[1::2] = ((b >> 4) ^ 8) - 8
    assert np.array_equal(got[0], want)


def test_closed_forms_weights_one_and_zero():
    c = case(11, 2, 6, 128, 16, 1, offset=True, shared=False, groups=[3, 3], batch=6)
    c.update(row_index=np.arange(6, dtype=np.int64), out_init=np.zeros((6, 16), np.float32))
    S = c["x1"].astype(np.float64).sum(axis=1)
    e_of = np.array([0, 0, 0, 1, 1, 1])
    wfac = c["pertoken_scale"].astype(np.float64) * c["logit"].astype(np.float64)
    # every weight 1 (byte 0x11): y = pts * (scale + offset) * sum x
    got, _ = run(c, x2=np.full_like(c["x2"], 0x11))
    want = (wfac * S)[:, None] * (c["scale"][e_of, 0].astype(np.float64) +
                                  c["offset"][e_of, 0].astype(np.float64))
    assert np.allclose(got, want, rtol=1e-14, atol=0)
    # every weight 0: only the asymmetric term remains
    got, _ = run(c, x2=np.zeros_like(c["x2"]))
    assert np.allclose(got, (wfac * S)[:, None] * c["offset"][e_of, 0], rtol=1e-14, atol=0)
    got, _ = run(c, x2=np.zeros_like(c["x2"]), offset=None)
    assert np.array_equal(got, np.zeros_like(got))


def test_pertoken_scale_linearity_and_invariants():
    c = case(13, 3, 12, 128, 32, 0, offset=True)
    base, _ = run(c)
    init_sh, _ = run(c, logit=np.zeros_like(c["logit"]))
    routed = base - init_sh
    two, _ = run(c, pertoken_scale=2 * c["pertoken_scale"])
    assert np.allclose(two - init_sh, 2 * routed, rtol=1e-13, atol=1e-12)
    # logit 0: init + shared only
    ref = c["out_init"].astype(np.float64).copy()
    sh = decode_np(c["shared_input"], "bf16")
    o = c["shared_input_offset"]
    ref[o:o + sh.shape[0]] += 0.75 * sh
    assert np.allclose(init_sh, ref, rtol=0, atol=1e-12)
    # an empty expert contributes nothing: moving all tokens to one expert
    # with a zeroed copy of the others' weights changes nothing else
    gl = np.array([0, 12, 12])
    got, _ = run(c, group_list=gl)
    ref2 = reference(dict(c, group_list=gl))
    _, mag = run(c, group_list=gl)
    assert np.all(np.abs(got - ref2) <= 1e-13 * mag + 1e-300)
