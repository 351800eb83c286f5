"""GPU parity of the W4A8 variant (gfr_w4a8_finalize_routing, through the C
ABI) against the oracle (oracle.w4a8_finalize_routing).

The integer products are exact on both sides; the GPU applies the scales in
FP32 and adds rows with FP32 atomics.  Bar: |gpu - oracle| <= 2e-5 * mag +
1e-6 per element.  The *_exact variants (x1 in [-8, 7], power-of-two scales,
offsets and per-token scales, logits in {1, 1/2, 1/4}, integer init and
shared rows) are exact in FP32 in any summation order and must match bit for
bit, at the page's full shape too.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_grouped_gemm_group_amd.workloads import WORKLOADS, make_w4a8_inputs
from tests.coverage import coverage_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL, ABS = 2e-5, 1e-6


def run_gpu(inp, **kw):
    import mxfp8_grouped_gemm_group_amd as gfr
    gfr.load_library()
    out = inp["out"].clone()
    gfr.w4a8_finalize_routing(inp["x1"], inp["x2"], inp["scale"], inp["offset"],
                              inp["pertoken_scale"], inp["group_list"], inp["group_list_type"],
                              inp["logit"], inp["row_index"], inp["shared_input"],
                              inp["shared_input_weight"], inp["shared_input_offset"], out, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def run_oracle(inp, rows=None):
    c = lambda t: None if t is None else t.cpu().numpy()
    sh = inp["shared_input"]
    sh = None if sh is None else sh.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return oracle.w4a8_finalize_routing(
        c(inp["x1"]), c(inp["x2"]), c(inp["scale"]), c(inp["offset"]), c(inp["pertoken_scale"]),
        c(inp["group_list"]), inp["group_list_type"], c(inp["logit"]), c(inp["row_index"]), sh,
        inp["shared_input_weight"], inp["shared_input_offset"], c(inp["out"]), rows=rows)


def check(got, ref, mag, exact, what):
    if exact:
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{what}: {len(bad)} elements differ, first {bad[:3].tolist()}"
        print(f"{what}: bit-exact ({got.size} elements)", flush=True)
        return
    ok, worst = oracle.within_tolerance(got, ref, mag, REL, ABS)
    print(f"{what}: worst err/bound = {worst:.3g}", flush=True)
    assert ok


SMALL = ["w4a8_small", "w4a8_small_big", "w4a8_small_exact", "w4a8_small_big_exact"]


@pytest.mark.parametrize("split_k", [0, 1, 3])
@pytest.mark.parametrize("name", SMALL)
def test_w4a8_small_full(name, split_k):
    w = WORKLOADS[name]
    print(f"case {name} split_k={split_k}", flush=True)
    inp = make_w4a8_inputs(w, DEV)
    got = run_gpu(inp, split_k=split_k)
    ref, mag = run_oracle(inp)
    check(got, ref, mag, w.exact, name)


@pytest.mark.parametrize("name", ["w4a8_p3", "w4a8_p3_exact"])
def test_w4a8_full_shape_coverage_rows(name):
    w = WORKLOADS[name]
    inp = make_w4a8_inputs(w, DEV)
    rows = coverage_rows(w, inp["row_index"].cpu().numpy())
    print(f"case {name} ({rows.size} of {w.batch} rows)", flush=True)
    got = run_gpu(inp)
    ref, mag = run_oracle(inp, rows)
    check(got[rows], ref, mag, w.exact, name)


@pytest.mark.parametrize("name", ["w4a8_small", "w4a8_small_big_exact"])
def test_w4a8_deterministic(name):
    w = WORKLOADS[name]
    print(f"case {name} deterministic", flush=True)
    inp = make_w4a8_inputs(w, DEV)
    a = run_gpu(inp, deterministic=True)
    b = run_gpu(inp, deterministic=True)
    assert np.array_equal(a, b), "deterministic mode is not bitwise repeatable"
    ref, mag = run_oracle(inp)
    check(a, ref, mag, w.exact, name + " det")


def test_w4a8_symmetric_equals_zero_offset():
    w = WORKLOADS["w4a8_small_exact"]
    inp = make_w4a8_inputs(w, DEV)
    a = run_gpu(dict(inp, offset=None))
    b = run_gpu(dict(inp, offset=torch.zeros_like(inp["offset"])))
    assert np.array_equal(a, b)
