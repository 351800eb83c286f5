"""GPU parity: libgfr.so (through its C ABI) against the CPU oracle.

Bar: |gpu - oracle| <= 2e-5 * mag + 1e-6 per element, where mag is the sum of
the magnitudes of every term entering the element.  Integer-valued variants
must match bit for bit.  Small cases, every shape of the c1-c3 benchmark sizes
and the pages' test shapes are compared on every element; c4 and c5 on the
rows tests/coverage.py selects (seeded random rows plus rows that reach every
cooperative row group and the ragged tails), all columns, every token routed
to them.

Every case is held to that bar strictly, except the cases named in
SLACK_CASES.  The gfx950 block-scaled MFMA sums each run of 8 consecutive K
products aligned to the largest one and truncates 13 bits below it
(tests/test_mfma_truncation_gpu.py pins that behaviour through the library),
so data with a wide dynamic range inside such a run can exceed the bar.  For
the named synthetic stress cases (wide E8M0 exponent ranges, E5M2
subnormals) the bar gains the oracle's bound on that truncation
(oracle.mx_group_slack), and the number of elements that needed it is capped
and printed.  MXFP4 products never lose bits to it (an E2M1 product has at
most 4 significant bits and the 8 products of a run span less than 2^8), so no
MXFP4 case is named.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_grouped_gemm_group_amd.workloads import WORKLOADS, as_numpy, make_inputs
from tests.coverage import coverage_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL, ABS = 2e-5, 1e-6

# Cases measured to exceed the plain bar through the MFMA's in-group
# truncation: name -> the most elements allowed over the plain bar (twice the
# most seen in any K split or mode, since the FP32 summation order of atomics
# varies between runs).  Measured on the MI355X: small_t 3 of 36864 elements
# (E5M2, E8M0 exponents +-6, K 640) in every K split and in deterministic
# mode, small_t_k384 2 of 36864, small_many_n 5 of 307200 (E4M3FN, +-4),
# small_coop_t_k128 3 of 42240 (E5M2, +-4, K 128: a dominant run weighs more
# in a short sum), small_tail_n 6 of 1419264 (E4M3FN, +-4; the same six in
# every K split, with the last-round K halves and in deterministic mode, at
# 0.08 of the bound with the truncation term), small_max_e_n 8 of 153600
# (E4M3FN, +-4, 1024 experts; the same eight in K splits 0, 1 and 3, while its
# integer-valued twin matches bit for bit); every other case, each MXFP4
# one at under 1 % of the bar, stays within it.  No other case may exceed it.
SLACK_CASES = {"small_t": 6, "small_t_k384": 4, "small_many_n": 10, "small_coop_t_k128": 6,
               "small_tail_n": 12, "small_max_e_n": 16}


def _gfr():
    import mxfp8_grouped_gemm_group_amd as gfr
    gfr.load_library()
    return gfr
def run_gpu(inp, out=None, **kw):
    gfr = _gfr()
    out = inp["out"].clone() if out is None else out
    gfr.gmm_finalize_routing(
        inp["x1"], inp["x2"], inp["scale"], inp["pertoken_scale"], inp["group_list"],
        inp["group_list_type"], inp["logit"], inp["row_index"], inp["shared_input"],
        inp["shared_input_weight"], inp["shared_input_offset"], out, inp["transpose_x2"], **kw)
    torch.cuda.synchronize()
    return out


def run_oracle(inp, rows=None, **over):
    h = as_numpy(inp)
    h.update(over)
    return oracle.gmm_finalize_routing(
        h["x1"], h["x2"], h["scale"], h["pertoken_scale"], h["group_list"],
        h["group_list_type"], h["logit"], h["row_index"], h["shared_input"],
        h["shared_input_weight"], h["shared_input_offset"], h["out_init"],
        h["transpose_x2"], h["fp8_kind"], rows=rows)


def assert_parity(got, ref, mag, exact=False, what="", case=None, slack=None):
    """Element-wise acceptance.  ``case`` names the workload; only cases in
    SLACK_CASES may use ``slack`` (the truncation bound, or a callable giving
    it), and then on at most SLACK_CASES[case] elements."""
    got = got.detach().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    if exact:
        bad = np.argwhere(got != ref)
        print(f"{what}: {bad.shape[0]} of {got.size} elements differ (exact)", flush=True)
        assert bad.size == 0, f"{what}: {len(bad)} elements differ, first {bad[:3].tolist()}"
        return
    ok, worst = oracle.within_tolerance(got, ref, mag, REL, ABS)
    n_over = int(np.sum(np.abs(got - ref) > REL * mag + ABS))
    print(f"{what}: worst err/bound = {worst:.3g} ({n_over} of {got.size} over)", flush=True)
    if ok:
        return
    assert case in SLACK_CASES and slack is not None, \
        f"{what}: {n_over} elements over the bar, worst ratio {worst}"
    assert n_over <= SLACK_CASES[case], \
        f"{what}: {n_over} elements over the bar, more than the {SLACK_CASES[case]} allowed"
    if callable(slack):   # computed only when the plain tolerance is exceeded
        slack = slack()
    err = np.abs(got - ref)
    bound = REL * mag + ABS + slack
    worst2 = float(np.max(err / bound))
    print(f"{what}: with the MFMA group-truncation bound: worst err/bound = {worst2:.3g}",
          flush=True)
    assert worst2 <= 1.0, f"{what}: worst ratio {worst2} even with the truncation bound"


def slack_for(inp, rows=None):
    h = as_numpy(inp)
    return oracle.mx_group_slack(h["x1"], h["x2"], h["scale"], h["pertoken_scale"],
                                 h["group_list"], h["group_list_type"], h["logit"],
                                 h["row_index"], h["transpose_x2"], h["fp8_kind"],
                                 h["out_init"].shape[0], rows=rows)


# ---------------------------------------------------------------------------
# Full element-by-element parity on small ragged cases (several n-tiles,
# ragged M tails, empty experts, both layouts and FP8 kinds).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["small_n", "small_t", "small_n_exact", "small_t_exact",
                                  "small_big_n", "small_big_t", "small_big_n_exact",
                                  "small_big_t_exact", "small_n_pe", "small_big_t_pe",
                                  "small_n_pe_exact", "small_big_t_pe_exact", "small_t_fp4",
                                  "small_big_t_fp4", "small_t_fp4_exact",
                                  "small_big_t_fp4_exact", "small_n_fp4", "small_big_n_fp4",
                                  "small_n_fp4_exact", "small_big_n_fp4_exact",
                                  "small_t_k768", "small_big_t_k768", "small_t_k768_exact",
                                  "small_big_t_k768_exact", "small_t_fp4_k1280",
                                  "small_t_fp4_k1280_exact", "small_t_k512", "small_t_k384",
                                  "small_t_k512_exact", "small_t_k384_exact",
                                  "small_huge_n", "small_huge_t", "small_huge_n_exact",
                                  "small_huge_t_exact", "small_many_n", "small_many_t",
                                  "small_many_n_exact", "small_many_t_exact",
                                  "small_coop_t_k128", "small_coop_t_k128_exact",
                                  "small_split_n", "small_split_t", "small_split_n_exact",
                                  "small_split_t_exact", "small_tail_n", "small_tail_t",
                                  "small_tail_n_exact", "small_tail_t_exact",
                                  "small_big_t_fp4_k256", "small_big_t_fp4_k256_exact",
                                  "small_split_t_fp4", "small_split_t_fp4_exact",
                                  "small_tail_t_fp4", "small_tail_t_fp4_exact",
                                  "small_many_t_fp4", "small_many_t_fp4_exact",
                                  "small_split_n_fp4", "small_split_n_fp4_exact",
                                  "small_t_fp4_k512", "small_t_fp4_k512_exact",
                                  "small_max_e_n", "small_max_e_t", "small_max_e_n_exact",
                                  "small_max_e_t_exact"])
@pytest.mark.parametrize("split_k", [0, 1, 3])
def test_small_full(name, split_k):
    w = WORKLOADS[name]
    print(f"case {name} split_k={split_k}", flush=True)
    inp = make_inputs(w, DEV)
    got = run_gpu(inp, split_k=split_k)
    ref, mag = run_oracle(inp)
    assert_parity(got, ref, mag, exact=w.exact, what=f"{name} split_k={split_k}", case=name,
                  slack=lambda: slack_for(inp))


# K splits that are multiples of four on shapes with only wave items: the
# four K ranges of an item run in one block and are added in LDS before the
# scatter (8: two such blocks per item, each with its own atomics).
@pytest.mark.parametrize("name", ["small_split_n", "small_split_t", "small_split_n_exact",
                                  "small_split_t_exact", "small_split_t_fp4",
                                  "small_split_t_fp4_exact", "small_split_n_fp4",
                                  "small_split_n_fp4_exact"])
@pytest.mark.parametrize("split_k", [4, 8])
def test_block_split(name, split_k):
    w = WORKLOADS[name]
    print(f"case {name} split_k={split_k}", flush=True)
    inp = make_inputs(w, DEV)
    got = run_gpu(inp, split_k=split_k)
    ref, mag = run_oracle(inp)
    assert_parity(got, ref, mag, exact=w.exact, what=f"{name} split_k={split_k}", case=name,
                  slack=lambda: slack_for(inp))


# ---------------------------------------------------------------------------
# The c1-c3 benchmark shapes (and their MXFP4, per-expert-scale and integer
# variants) and the pages' test shapes: every element.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c1_exact", "c2_exact", "c3_exact",
                                  "c3_pe", "c1_fp4", "c2_fp4", "c3_fp4", "c3_fp4_exact",
                                  "c3_fp4t", "c3_fp4t_exact", "p1_tc_a", "p1_tc_b",
                                  "p2_ragged"])
def test_full_shapes_every_element(name):
    w = WORKLOADS[name]
    print(f"case {name} (every element)", flush=True)
    inp = make_inputs(w, DEV)
    got = run_gpu(inp)
    ref, mag = run_oracle(inp)
    assert_parity(got, ref, mag, exact=w.exact, what=name)


# ---------------------------------------------------------------------------
# c4 and c5 (and variants): the coverage rows, every column.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c4", "c5", "c4_exact", "c5_exact", "c5_pe", "c4_fp4",
                                  "c5_fp4"])
def test_large_shapes_coverage_rows(name):
    w = WORKLOADS[name]
    inp = make_inputs(w, DEV)
    rows = coverage_rows(w, inp["row_index"].cpu().numpy())
    print(f"case {name} ({rows.size} of {w.batch} rows)", flush=True)
    assert rows.size >= 16 + 2
    got = run_gpu(inp)
    ref, mag = run_oracle(inp, rows=rows)
    assert_parity(got[torch.as_tensor(rows, device=DEV)], ref, mag, exact=w.exact, what=name)


@pytest.mark.parametrize("name", ["c5", "c5_exact", "c4", "c4_exact", "small_n", "small_t", "small_big_n",
                                  "small_big_t_exact", "small_t_fp4", "small_big_n_fp4",
                                  "small_big_t_k768", "small_huge_t", "small_huge_n_exact"])
def test_deterministic_mode(name):
    """Deterministic mode: bitwise repeatable, within tolerance of the oracle
    (bit-exact on integer data).  c4 holds a cooperative expert whose last row
    group has 9 rows (waves without live rows in every step): a missed wait
    there showed as results that changed from launch to launch."""
    w = WORKLOADS[name]
    print(f"case {name} deterministic", flush=True)
    inp = make_inputs(w, DEV)
    a = run_gpu(inp, deterministic=True)
    b = run_gpu(inp, deterministic=True)
    assert torch.equal(a, b)
    rows = coverage_rows(w, inp["row_index"].cpu().numpy()) if w.M > 2000 else None
    ref, mag = run_oracle(inp, rows=rows)
    got = a if rows is None else a[torch.as_tensor(rows, device=DEV)]
    assert_parity(got, ref, mag, exact=w.exact, what=name + " det", case=name,
                  slack=lambda: slack_for(inp, rows))


# ---------------------------------------------------------------------------
# Edge cases and invariants.
# ---------------------------------------------------------------------------
def test_logit_zero_gives_init_plus_shared_bitwise():
    w = WORKLOADS["small_n"]
    inp = make_inputs(w, DEV)
    inp["logit"] = torch.zeros_like(inp["logit"])
    got = run_gpu(inp)
    ref, _ = run_oracle(inp)
    # out = fp32(init + w * shared): one rounding of the exact double result
    assert np.array_equal(got.cpu().numpy(), ref.astype(np.float32))


def test_logit_and_shared_absent():
    w = WORKLOADS["small_t"]
    inp = make_inputs(w, DEV)
    inp["logit"] = None
    inp["shared_input"] = None
    got = run_gpu(inp)
    ref, mag = run_oracle(inp)
    assert_parity(got, ref, mag, what="small_t no logit / no shared", case="small_t",
                  slack=lambda: slack_for(inp))


def test_empty_groups_and_no_tokens():
    w = WORKLOADS["small_n"]
    inp = make_inputs(w, DEV)
    inp["group_list"] = torch.zeros_like(inp["group_list"])
    got = run_gpu(inp)
    ref, mag = run_oracle(inp)
    assert_parity(got, ref, mag, what="all experts empty")


def test_m_zero_shared_only():
    w = WORKLOADS["small_n"]
    inp = make_inputs(w, DEV)
    K, N = w.K, w.N
    KB = (K + 63) // 64
    inp["x1"] = inp["x1"][:0].contiguous()
    inp["pertoken_scale"] = inp["pertoken_scale"][:0].contiguous()
    inp["logit"] = inp["logit"][:0].contiguous()
    inp["row_index"] = inp["row_index"][:0].contiguous()
    inp["group_list"] = torch.zeros_like(inp["group_list"])
    got = run_gpu(inp)
    want = inp["out"].clone()
    off, R = inp["shared_input_offset"], inp["shared_input"].shape[0]
    want[off:off + R] += inp["shared_input_weight"] * inp["shared_input"].float()
    assert torch.equal(got, want)
    assert KB > 0


def test_device_status_bits():
    gfr = _gfr()
    w = WORKLOADS["small_n"]
    inp = make_inputs(w, DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    ri = inp["row_index"].clone()
    ri[40] = w.batch + 5          # token 40 belongs to expert 1 (counts 0, 37, 1, ...)
    inp2 = dict(inp, row_index=ri)
    got = run_gpu(inp2, status=status)
    assert int(status.item()) & gfr.DEV_BAD_ROW_INDEX
    # everything else is as if token 40 had logit 0
    lg = inp["logit"].clone()
    lg[40] = 0
    ref, mag = run_oracle(dict(inp, logit=lg))
    assert_parity(got, ref, mag, what="small_n bad row_index skipped", case="small_n",
                  slack=lambda: slack_for(dict(inp, logit=lg)))

    status.zero_()
    g = inp["group_list"].clone()
    g[2] = -3
    run_gpu(dict(inp, group_list=g), status=status)
    assert int(status.item()) & gfr.DEV_BAD_GROUP_LIST


def test_invalid_group_list_clamped_bitwise_exact():
    """An invalid group_list is clamped into [0, M) and flagged: counts past
    the rows left (one as large as 2^40) and negative counts (a decreasing
    prefix list) give exactly the valid list with the clamped ranges
    (integer-exact data, so any summation order gives the same bits)."""
    gfr = _gfr()
    w = WORKLOADS["small_n_exact"]                  # counts (0, 37, 1, 120, 0, 95, 47), M 300
    inp = make_inputs(w, DEV)
    valid = torch.tensor([0, 37, 1, 262, 0, 0, 0], dtype=torch.int64, device=DEV)
    want = run_gpu(dict(inp, group_list=valid))
    ref, mag = run_oracle(dict(inp, group_list=valid))
    assert_parity(want, ref, mag, exact=True, what="clamped ranges")
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    counts = torch.tensor([0, 37, 1, 1 << 40, 5, 95, 47], dtype=torch.int64, device=DEV)
    got = run_gpu(dict(inp, group_list=counts), status=status)
    assert int(status.item()) & gfr.DEV_BAD_GROUP_LIST
    assert torch.equal(got, want)
    status.zero_()
    prefix = torch.tensor([0, 37, 38, 5000, 4000, 300, 300], dtype=torch.int64, device=DEV)
    got = run_gpu(dict(inp, group_list=prefix, group_list_type=0), status=status)
    assert int(status.item()) & gfr.DEV_BAD_GROUP_LIST
    assert torch.equal(got, want)


def test_group_list_type_equivalence_bitwise_exact():
    w = WORKLOADS["small_n_exact"]
    inp = make_inputs(w, DEV)
    a = run_gpu(inp)
    g = torch.cumsum(inp["group_list"], 0)
    b = run_gpu(dict(inp, group_list=g, group_list_type=0))
    assert torch.equal(a, b)


@pytest.mark.parametrize("deterministic", [False, True])
def test_row_index_int32_equals_int64_bitwise_exact(deterministic):
    """row_index may be int32 through the descriptor ABI ([P1] §5.4 passes it
    as int32): integer-exact data gives the same bits as int64 in both modes."""
    for name in ("small_n_exact", "small_big_t_exact"):
        w = WORKLOADS[name]
        inp = make_inputs(w, DEV)
        a = run_gpu(inp, deterministic=deterministic)
        b = run_gpu(dict(inp, row_index=inp["row_index"].to(torch.int32)),
                    deterministic=deterministic)
        assert torch.equal(a, b), name
