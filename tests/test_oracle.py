"""Pins of the CPU oracle against things other than itself.

* decoders: every code against torch's independent float8/bfloat16 casts, plus
  the closed-form extremes of each format;
* contraction + routing: an independent float64 formulation built from library
  primitives (torch decoding, ``np.repeat`` of the scales over 32 K elements as
  the golden description in §6.3 of the grouped_matmul_finalize_routing MXFP8
  page does, ``numpy.matmul``, ``np.add.at``) on tiny brute-force inputs;
* a textbook special case (one expert, unit scales, unit logits, identity
  routing) that is a plain matrix product;
* exact integer arithmetic (int64 einsum) on the integer-valued variant;
* analytic one-hot cases that pin the scale-layout reading;
* invariants: logit = 0, empty experts, group_list formats, transposition,
  shared input absent, scale-exponent linearity.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.tiny_inputs import E2M1_VALUES, decode_np, numpy_reference, tiny_case, unpack_e2m1


# ----------------------------------------------------------------------------
# Decoders
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind,tdt", [("e4m3fn", torch.float8_e4m3fn),
                                      ("e5m2", torch.float8_e5m2),
                                      ("e8m0", torch.float8_e8m0fnu)])
def test_decode_all_codes_match_torch(kind, tdt):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(tdt).to(torch.float64).numpy()
    got = np.array([oracle.decode(kind, int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_decode_bf16_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode("bf16", int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_decode_closed_forms():
    d = oracle.decode
    # E4M3FN: max finite 448 = 1.75 * 2^8 at 0x7E, NaN at 0x7F/0xFF, no inf,
    # smallest subnormal 2^-9, smallest normal 2^-6, one = 0x38.
    assert d("e4m3fn", 0x7E) == 448.0 and d("e4m3fn", 0xFE) == -448.0
    assert math.isnan(d("e4m3fn", 0x7F)) and math.isnan(d("e4m3fn", 0xFF))
    assert d("e4m3fn", 0x01) == 2.0 ** -9 and d("e4m3fn", 0x08) == 2.0 ** -6
    assert d("e4m3fn", 0x38) == 1.0 and d("e4m3fn", 0x80) == 0.0
    # E5M2: max finite 57344 = 1.75 * 2^15 at 0x7B, +inf 0x7C, NaN 0x7D..0x7F,
    # smallest subnormal 2^-16, one = 0x3C.
    assert d("e5m2", 0x7B) == 57344.0 and d("e5m2", 0x7C) == math.inf
    assert d("e5m2", 0xFC) == -math.inf
    assert all(math.isnan(d("e5m2", c)) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert d("e5m2", 0x01) == 2.0 ** -16 and d("e5m2", 0x3C) == 1.0
    # E8M0: 2^(b-127), 0xFF NaN.
    assert d("e8m0", 127) == 1.0 and d("e8m0", 0) == 2.0 ** -127
    assert d("e8m0", 254) == 2.0 ** 127 and math.isnan(d("e8m0", 255))
    # bf16: one = 0x3F80, -2 = 0xC000.
    assert d("bf16", 0x3F80) == 1.0 and d("bf16", 0xC000) == -2.0


# ----------------------------------------------------------------------------
# group_list
# ----------------------------------------------------------------------------
def test_expert_ranges_formats():
    counts = np.array([3, 0, 2, 5, 0], np.int64)
    s1, e1 = oracle.expert_ranges(counts, 1, 10)
    s0, e0 = oracle.expert_ranges(np.cumsum(counts), 0, 10)
    assert s1.tolist() == [0, 3, 3, 5, 10] and e1.tolist() == [3, 3, 5, 10, 10]
    assert np.array_equal(s0, s1) and np.array_equal(e0, e1)


@pytest.mark.parametrize("g,t,M", [([2, -1, 3], 1, 10), ([2, 1, 3], 0, 10),
                                   ([4, 4, 4], 1, 11), ([3, 12], 0, 11)])
def test_expert_ranges_reject_invalid(g, t, M):
    with pytest.raises(oracle.OracleError) as ei:
        oracle.expert_ranges(np.array(g, np.int64), t, M)
    assert ei.value.code == -2


# ----------------------------------------------------------------------------
# Contraction and routing
# ----------------------------------------------------------------------------
def _run(c, **over):
    a = dict(c)
    a.update(over)
    return oracle.gmm_finalize_routing(
        a["x1"], a["x2"], a["scale"], a["pertoken_scale"], a["group_list"],
        a["group_list_type"], a["logit"], a["row_index"], a["shared_input"],
        a["shared_input_weight"], a["shared_input_offset"], a["out_init"],
        a["transpose_x2"], a["fp8_kind"], rows=a.get("rows"))


CASES = [dict(seed=s, E=E, M=M, K=K, N=N, transpose=tr, kind=kd, gtype=gt)
         for s, (E, M, K, N, tr, kd, gt) in enumerate([
             (1, 3, 32, 2, False, 0, 1), (2, 5, 64, 3, True, 1, 0),
             (3, 8, 96, 5, False, 1, 1), (3, 7, 128, 4, True, 0, 0),
             (2, 6, 160, 5, False, 0, 0), (3, 8, 128, 5, True, 1, 1)])]


def test_decode_e2m1_value_set():
    assert [oracle.decode("e2m1", c) for c in range(16)] == list(E2M1_VALUES)
    assert math.copysign(1.0, oracle.decode("e2m1", 8)) == -1.0


# MXFP4 ([P3] Atlas 350 MX notes): x1 / x2 hold two E2M1 codes per byte along
# their contiguous axis (element 2j in the low nibble, the reading of the
# packing); K even, N even when x2 is not transposed.
FP4_CASES = [dict(seed=100 + s, E=E, M=M, K=K, N=N, transpose=tr, kind=2, gtype=gt)
             for s, (E, M, K, N, tr, gt) in enumerate([
                 (1, 3, 32, 2, False, 1), (2, 5, 64, 3, True, 0), (3, 8, 96, 6, False, 1),
                 (3, 7, 128, 4, True, 0), (2, 6, 192, 8, False, 0)])]


@pytest.mark.parametrize("case", FP4_CASES, ids=lambda c: f"s{c['seed']}")
def test_tiny_fp4_matches_independent_numpy(case):
    c = tiny_case(**case)
    got, mag = _run(c)
    ref = numpy_reference(c)
    assert np.all(np.abs(got - ref) <= 1e-13 * mag + 1e-300)


@pytest.mark.parametrize("transpose", [False, True])
def test_fp4_textbook_plain_matmul(transpose):
    c = tiny_case(seed=43, E=1, M=6, K=128, N=6, transpose=transpose, kind=2, gtype=1,
                  groups=[6], batch=6, routing="identity", unit_scales=True,
                  logit="ones", shared=False)
    got, _ = _run(c, out_init=np.zeros_like(c["out_init"]))
    a = E2M1_VALUES[unpack_e2m1(c["x1"])]
    b = E2M1_VALUES[unpack_e2m1(c["x2"][0])]
    if transpose:
        b = b.T
    assert np.array_equal(got, a @ b)


@pytest.mark.parametrize("K,N,transpose,ok", [(64, 3, False, False), (64, 3, True, True),
                                              (63, 4, True, False), (64, 4, False, True)])
def test_fp4_packing_needs_even_sizes(K, N, transpose, ok):
    """The C entry point takes logical sizes: an odd N (non-transposed) or an
    odd K cannot be packed two per byte and is rejected (-1)."""
    import ctypes
    lib = oracle._lib()
    KB = (K + 63) // 64
    x1 = np.zeros((1, K), np.uint8)
    x2 = np.zeros((1, K, N), np.uint8)
    sc = np.full((KB * N * 2,), 127, np.uint8)
    pts = np.full((KB * 2,), 127, np.uint8)
    g = np.array([1], np.int64)
    ri = np.zeros(1, np.int64)
    init = np.zeros((1, N), np.float32)
    res = np.zeros((1, N))
    mag = np.zeros((1, N))
    rc = lib.oracle_gmm_finalize_routing(
        x1.ctypes.data, x2.ctypes.data, sc.ctypes.data, 0, pts.ctypes.data, g.ctypes.data, 1,
        None, ri.ctypes.data, None, 1.0, 0, 0, init.ctypes.data, int(transpose), 2,
        1, K, N, 1, 1, None, 1, res.ctypes.data, mag.ctypes.data)
    assert (rc == 0) == ok and (ok or rc == -1)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_tiny_matches_independent_numpy(case):
    c = tiny_case(**case)
    got, mag = _run(c)
    ref = numpy_reference(c)
    assert np.all(np.abs(got - ref) <= 1e-13 * mag + 1e-300)


# Per-expert weight scales: a leading expert axis, (e, n, ceil(k/64), 2) when
# x2 is transposed (CANN aclnnGroupedMatmulFinalizeRoutingV3, Atlas 350 scale
# notes) and (e, ceil(k/64), n, 2) otherwise (the 3-D layout's reading).
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_tiny_per_expert_scales_match_independent_numpy(case):
    c = tiny_case(**case, per_expert=True)
    assert c["scale"].ndim == 4 and c["scale"].shape[0] == case["E"]
    got, mag = _run(c)
    ref = numpy_reference(c)
    assert np.all(np.abs(got - ref) <= 1e-13 * mag + 1e-300)


@pytest.mark.parametrize("transpose", [False, True])
def test_per_expert_scales_identical_copies_equal_shared(transpose):
    c = tiny_case(seed=7, E=3, M=9, K=128, N=5, transpose=transpose, kind=0, gtype=1)
    a, _ = _run(c)
    b, _ = _run(c, scale=np.ascontiguousarray(np.broadcast_to(c["scale"], (3,) + c["scale"].shape)))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("transpose", [False, True])
def test_per_expert_scales_select_the_experts_slice(transpose):
    """Each expert's rows use only its own slice: running one expert at a time
    (the others' tokens given logit 0) with that slice as a 3-D scale, and
    summing the routed parts, reproduces the 4-D run."""
    c = tiny_case(seed=11, E=3, M=10, K=192, N=4, transpose=transpose, kind=1, gtype=1,
                  groups=[4, 3, 3], per_expert=True, shared=False)
    full, mag = _run(c)
    init = c["out_init"].astype(np.float64)
    total = init.copy()
    start = 0
    for e, cnt in enumerate(c["group_list"]):
        lg = np.zeros_like(c["logit"])
        lg[start:start + cnt] = c["logit"][start:start + cnt]
        part, _ = _run(c, scale=np.ascontiguousarray(c["scale"][e]), logit=lg,
                       out_init=np.zeros_like(c["out_init"]))
        total += part
        start += cnt
    assert np.all(np.abs(full - total) <= 1e-13 * mag + 1e-300)


@pytest.mark.parametrize("transpose", [False, True])
def test_textbook_plain_matmul(transpose):
    """One expert, unit scales, unit logits, identity routing, zero init, no
    shared input: out is exactly the decoded FP8 product x1 @ x2[0]."""
    c = tiny_case(seed=42, E=1, M=6, K=128, N=5, transpose=transpose, kind=0, gtype=1,
                  groups=[6], batch=6, routing="identity", unit_scales=True,
                  logit="ones", shared=False)
    got, _ = _run(c, out_init=np.zeros_like(c["out_init"]))
    a = decode_np(c["x1"], 0)
    b = decode_np(c["x2"][0], 0)
    if transpose:
        b = b.T
    # Products span < 40 bits and 128 terms add < 8 more: exact in float64 in
    # any summation order, so the comparison is exact.
    assert np.array_equal(got, a @ b)


def test_exact_integer_arithmetic():
    """Integer FP8 values in [-2, 2], exponents {0, 1}, logits {1, 1/2, 1/4}:
    compare against int64 arithmetic."""
    for seed in range(3):
        c = tiny_case(seed=100 + seed, E=3, M=8, K=256, N=5, transpose=bool(seed % 2),
                      kind=seed % 2, gtype=seed % 2, exact=True)
        got, _ = _run(c)
        kind = c["fp8_kind"]
        a = decode_np(c["x1"], kind).astype(np.int64)
        b = decode_np(c["x2"], kind).astype(np.int64)
        if c["transpose_x2"]:
            b = np.transpose(b, (0, 2, 1))
        M, K = a.shape
        pe = (c["pertoken_scale"].astype(np.int64) - 127).reshape(M, -1)[:, np.arange(K) // 32]
        if c["transpose_x2"]:
            se = (c["scale"].astype(np.int64) - 127).reshape(b.shape[2], -1)[:, np.arange(K) // 32].T
        else:
            s3 = c["scale"].astype(np.int64) - 127  # [KB, N, 2]
            se = np.moveaxis(s3, 2, 1).reshape(-1, s3.shape[1])[np.arange(K) // 32]
        a_s = a << pe                     # exact integers
        b_s = b << se[None]
        g = c["group_list"]
        counts = np.diff(np.concatenate([[0], g])) if c["group_list_type"] == 0 else g
        end = np.cumsum(counts)
        start = end - counts
        out = c["out_init"].astype(np.float64).copy()
        for e in range(len(start)):
            for t in range(start[e], end[e]):
                row = np.einsum("k,kn->n", a_s[t], b_s[e])  # int64
                out[c["row_index"][t]] += float(c["logit"][t]) * row.astype(np.float64)
        sh = decode_np(c["shared_input"], "bf16")
        off = c["shared_input_offset"]
        out[off:off + sh.shape[0]] += c["shared_input_weight"] * sh
        assert np.array_equal(got, out)


@pytest.mark.parametrize("transpose", [False, True])
def test_one_hot_pins_scale_layout(transpose):
    """A single non-zero in x1 at (t, k) and in x2 at (e, k, n): the only
    changed output element is (row_index[t], n) and its change is
    logit[t] * x1 * x2 * 2^(pertoken_scale[t, k//64, (k//32)%2] - 127)
    * 2^(scale[k//64, n, (k//32)%2] - 127) (scale[n, k//64, ...] if transposed)."""
    rng = np.random.default_rng(7)
    for _ in range(12):
        c = tiny_case(seed=int(rng.integers(1 << 30)), E=2, M=5, K=192, N=4,
                      transpose=transpose, kind=0, gtype=1, groups=[2, 3], batch=3)
        t = int(rng.integers(5))
        k = int(rng.integers(192))
        n = int(rng.integers(4))
        e = 0 if t < 2 else 1
        x1 = np.zeros_like(c["x1"])
        x2 = np.zeros_like(c["x2"])
        x1[t, k] = 0x38            # 1.0
        if transpose:
            x2[e, n, k] = 0x40     # 2.0
        else:
            x2[e, k, n] = 0x40
        got, _ = _run(c, x1=x1, x2=x2, shared_input=None)
        pe = int(c["pertoken_scale"][t, k // 64, (k // 32) % 2]) - 127
        se = int((c["scale"][n, k // 64, (k // 32) % 2] if transpose
                  else c["scale"][k // 64, n, (k // 32) % 2])) - 127
        want = c["out_init"].astype(np.float64).copy()
        want[c["row_index"][t], n] += float(c["logit"][t]) * 2.0 * 2.0 ** (pe + se)
        assert np.array_equal(got, want)


# ----------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------
def test_logit_zero_leaves_init_plus_shared():
    c = tiny_case(seed=5, E=3, M=8, K=128, N=5, transpose=False, kind=0, gtype=1)
    got, _ = _run(c, logit=np.zeros_like(c["logit"]))
    want = c["out_init"].astype(np.float64).copy()
    sh = decode_np(c["shared_input"], "bf16")
    off = c["shared_input_offset"]
    want[off:off + sh.shape[0]] += c["shared_input_weight"] * sh
    assert np.array_equal(got, want)


def test_empty_expert_contributes_nothing():
    c = tiny_case(seed=6, E=3, M=6, K=128, N=4, transpose=True, kind=1, gtype=1,
                  groups=[2, 0, 4])
    base, _ = _run(c)
    x2 = c["x2"].copy()
    x2[1] = np.random.default_rng(0).integers(0, 0x7B, size=x2[1].shape, dtype=np.uint8)
    got, _ = _run(c, x2=x2)
    assert np.array_equal(base, got)


def test_tokens_past_last_group_contribute_nothing():
    c = tiny_case(seed=8, E=2, M=8, K=64, N=3, transpose=False, kind=0, gtype=1,
                  groups=[2, 3])
    base, _ = _run(c)
    x1 = c["x1"].copy()
    x1[5:] = 0x38
    ri = c["row_index"].copy()
    ri[5:] = 10 ** 6   # never read
    got, _ = _run(c, x1=x1, row_index=ri)
    assert np.array_equal(base, got)


def test_group_list_type_equivalence():
    c = tiny_case(seed=9, E=3, M=8, K=96, N=4, transpose=False, kind=0, gtype=1,
                  groups=[3, 0, 4])
    a, _ = _run(c)
    b, _ = _run(c, group_list=np.cumsum(c["group_list"]), group_list_type=0)
    assert np.array_equal(a, b)


def test_transpose_equivalence():
    c = tiny_case(seed=10, E=2, M=6, K=160, N=5, transpose=False, kind=1, gtype=1)
    a, _ = _run(c)
    x2t = np.ascontiguousarray(np.transpose(c["x2"], (0, 2, 1)))
    st = np.ascontiguousarray(np.transpose(c["scale"], (1, 0, 2)))   # [KB,N,2] -> [N,KB,2]
    b, _ = _run(c, x2=x2t, scale=st, transpose_x2=True)
    assert np.array_equal(a, b)


def test_shared_absent_equals_zero_weight():
    c = tiny_case(seed=11, E=2, M=6, K=64, N=3, transpose=False, kind=0, gtype=1)
    a, _ = _run(c, shared_input=None)
    b, _ = _run(c, shared_input_weight=0.0)
    assert np.array_equal(a, b)


def test_logit_absent_equals_unit_logit():
    c = tiny_case(seed=12, E=2, M=6, K=64, N=3, transpose=True, kind=0, gtype=0)
    a, _ = _run(c, logit=None)
    b, _ = _run(c, logit=np.ones_like(c["logit"]))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("which", ["pertoken", "weight"])
def test_scale_exponent_linearity(which):
    """Raising one E8M0 exponent by 1 adds exactly that 32-element sub-block's
    contribution once more; the sub-block's contribution is measured by
    zeroing x1 outside it (integer data, so everything is exact)."""
    rng = np.random.default_rng(13)
    for trial in range(8):
        tr = bool(trial % 2)
        c = tiny_case(seed=200 + trial, E=2, M=6, K=256, N=4, transpose=tr, kind=0,
                      gtype=1, groups=[3, 3], batch=6, routing="identity", exact=True,
                      shared=False)
        base, _ = _run(c)
        kb = int(rng.integers(8))            # 32-element sub-block
        b, j = kb // 2, kb % 2
        mask = np.zeros_like(c["x1"])
        mask[:, 32 * kb:32 * kb + 32] = 1
        x1_sub = np.where(mask == 1, c["x1"], 0).astype(np.uint8)
        init0 = np.zeros_like(c["out_init"])
        if which == "pertoken":
            t = int(rng.integers(6))
            pts = c["pertoken_scale"].copy()
            pts[t, b, j] += 1
            bumped, _ = _run(c, pertoken_scale=pts)
            contrib, _ = _run(c, x1=x1_sub, out_init=init0)
            want = base.copy()
            r = c["row_index"][t]
            want[r] += contrib[r]
        else:
            n = int(rng.integers(4))
            sc = c["scale"].copy()
            if tr:
                sc[n, b, j] += 1
            else:
                sc[b, n, j] += 1
            bumped, _ = _run(c, scale=sc)
            contrib, _ = _run(c, x1=x1_sub, out_init=init0)
            want = base.copy()
            want[:, n] += contrib[:, n]
        assert np.array_equal(bumped, want)


def test_row_selection_matches_full():
    c = tiny_case(seed=14, E=3, M=8, K=64, N=4, transpose=True, kind=1, gtype=0, batch=5)
    full, fmag = _run(c)
    rows = np.array([4, 1, 3], np.int64)
    part, pmag = _run(c, rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(pmag, fmag[rows])


def test_duplicate_rows_accumulate():
    c = tiny_case(seed=15, E=1, M=4, K=64, N=3, transpose=False, kind=0, gtype=1,
                  groups=[4], batch=2, shared=False)
    ri = np.array([1, 1, 1, 1], np.int64)
    got, _ = _run(c, row_index=ri)
    # row 1 collects all four tokens; row 0 keeps its initial value
    parts = []
    for t in range(4):
        lg = np.zeros_like(c["logit"])
        lg[t] = c["logit"][t]
        p, _ = _run(c, row_index=ri, logit=lg, out_init=np.zeros_like(c["out_init"]))
        parts.append(p[1])
    assert np.array_equal(got[0], c["out_init"][0].astype(np.float64))
    assert np.allclose(got[1], c["out_init"][1] + sum(parts), rtol=1e-15, atol=0)


def test_errors():
    c = tiny_case(seed=16, E=2, M=4, K=64, N=3, transpose=False, kind=0, gtype=1,
                  groups=[2, 2], batch=2)
    with pytest.raises(oracle.OracleError) as ei:
        _run(c, row_index=np.array([0, 1, 2, 0], np.int64))
    assert ei.value.code == -3
    with pytest.raises(oracle.OracleError) as ei:
        _run(c, shared_input_offset=1)
    assert ei.value.code == -4
    with pytest.raises(oracle.OracleError) as ei:
        _run(c, group_list=np.array([3, 2], np.int64))
    assert ei.value.code == -2


def test_tolerance_helper():
    ok, r = oracle.within_tolerance([1.0, 2.0], np.array([1.0, 2.0 + 1e-4]), np.array([1.0, 1.0]))
    assert not ok and r > 1
    ok, r = oracle.within_tolerance([1.0], np.array([1.0 + 1e-5]), np.array([1.0]))
    assert ok and r < 1


# ----------------------------------------------------------------------------
# Hand-derived worked example (tests/golden/worked_example_1.json)
# ----------------------------------------------------------------------------
def _load_worked_example(kind, transpose):
    import json
    import os
    d = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "worked_example_1.json")))
    f8 = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}[kind]
    enc = lambda v: torch.tensor(v, dtype=torch.float32).to(f8).view(torch.uint8).numpy()
    x2 = enc(d["x2_values_EKN"])
    sc = (127 + np.array(d["scale_exponents_KB_N_2"])).astype(np.uint8)
    if transpose:
        x2 = np.ascontiguousarray(np.transpose(x2, (0, 2, 1)))
        sc = np.ascontiguousarray(np.transpose(sc, (1, 0, 2)))
    sh = torch.tensor(d["shared_input"], dtype=torch.float32).to(torch.bfloat16)
    c = dict(x1=enc(d["x1_values"]), x2=x2, scale=sc,
             pertoken_scale=(127 + np.array(d["pertoken_scale_exponents_M_KB_2"])).astype(np.uint8),
             group_list=np.array(d["group_list"], np.int64), group_list_type=d["group_list_type"],
             logit=np.array(d["logit"], np.float32), row_index=np.array(d["row_index"], np.int64),
             shared_input=sh.view(torch.int16).numpy().view(np.uint16),
             shared_input_weight=d["shared_input_weight"],
             shared_input_offset=d["shared_input_offset"],
             out_init=np.array(d["out_init"], np.float32), transpose_x2=transpose, fp8_kind=kind)
    return c, np.array(d["expected_out"], np.float64)


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("transpose", [False, True])
def test_worked_example(kind, transpose):
    c, want = _load_worked_example(kind, transpose)
    got, _ = _run(c)
    assert np.array_equal(got, want)


def test_mx_group_slack_analytic():
    """Group-truncation slack: groups are 8 consecutive K; each term adds
    min(|term|, 2^(E-13)) with E the exponent of the group's largest term."""
    one, sub = 0x38, 0x01          # E4M3 1.0 and 2^-9
    K, N = 16, 1
    x1 = np.full((1, K), one, np.uint8)
    x1[0, 1] = sub
    x2 = np.zeros((1, K, N), np.uint8)
    x2[0, 0:3, 0] = [one, sub, 0x30]      # group 0 terms: 1, 2^-18, 0.5 (x1[1] = 2^-9)
    x2[0, 8:11, 0] = [sub, sub, sub]      # group 1 terms: 2^-9 each
    pts = np.full((1, 1, 2), 127, np.uint8)
    sc = np.full((1, N, 2), 127, np.uint8)
    lg = np.array([0.5], np.float32)
    got = oracle.mx_group_slack(x1, x2, sc, pts, np.array([1]), 1, lg, np.array([0]),
                                False, 0, 1)
    # group 0: E = 0, q = 2^-13; terms 1, 2^-9 * 2^-9 = 2^-18, 0.5
    want_g0 = 2.0 ** -13 + 2.0 ** -18 + 2.0 ** -13
    want_g1 = 3 * 2.0 ** -22            # E = -9, q = 2^-22, each term 2^-9 > q
    assert got.shape == (1, 1)
    assert got[0, 0] == 0.5 * (want_g0 + want_g1)


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("kind", [0, 1])
def test_truncation_patterns_oracle_side(kind, transpose):
    """The crafted sums of tests/test_mfma_truncation_gpu.py on the CPU: the
    oracle gives each exact sum (powers of two: exact in double), and its
    truncation bound covers the value a run-truncating unit returns, while the
    plain bar does not for the six patterns whose small terms are dropped."""
    from tests.test_mfma_truncation_gpu import N, T, _inputs
    from mxfp8_grouped_gemm_group_amd.workloads import as_numpy
    inp, pats, S = _inputs(kind, transpose, device="cpu")
    h = as_numpy(inp)
    ref, mag = oracle.gmm_finalize_routing(
        h["x1"], h["x2"], h["scale"], h["pertoken_scale"], h["group_list"], 1, None,
        h["row_index"], None, 0.0, 0, h["out_init"], transpose, kind)
    exact = np.array([pats[n][3] for n in range(N)])
    model = np.array([pats[n][2] for n in range(N)])
    assert np.array_equal(ref[0], exact)
    assert np.array_equal(ref[1], (32.0 + T) * 2.0 ** -5 * 2.0 ** S[:, 0])
    slack = oracle.mx_group_slack(h["x1"], h["x2"], h["scale"], h["pertoken_scale"],
                                  h["group_list"], 1, None, h["row_index"], transpose, kind, 2)
    err = np.abs(model - ref[0])
    bar = 2e-5 * mag[0] + 1e-6
    assert np.all(err <= bar + slack[0])
    assert int(np.sum(err > bar)) == 6
