"""GPU parity of the upstream step (gfr_gemm1_swiglu_quant, through the C ABI)
against the oracle (oracle.gemm1).

The output is quantised: every code and scale byte is a decision taken on a
floating-point value, and the GPU's FP32 gate/up sums differ from the oracle's
float64 ones by summation order (and by the block-scaled MFMA's in-group
truncation).  So each decision is checked against the set of decisions that
values within that error would produce:

  * gate and up are bounded by the operator's bar, REL * mag + ABS, plus the
    oracle's MFMA group-truncation bound (mx_group_slack);
  * SiLU is 1.1-Lipschitz, so sw = SiLU(gate) * up is bounded by
    d_sw = 1.1 (|up| + d_up) d_gate + |SiLU(gate)| d_up + 2^-20 |sw|
    (the last term covers the FP32 evaluation of exp, the division and the
    product, each a few units in the last place);
  * a block's exponent must lie between the exponents of the smallest and
    the largest block maximum those bounds allow;
  * under the GPU's exponent, each code's value must lie between the codes of
    (sw - d_sw) / 2^X and (sw + d_sw) / 2^X (the encoding is monotone).
Away from rounding midpoints and powers of two that interval holds a single
code, so the test is exact almost everywhere; the share of codes equal to the
oracle's own encoding is printed and required to be at least 99 %.  Rows of
tokens in no expert's range must keep their previous contents.
"""
import numpy as np
import pytest
import torch

from oracle import gemm1 as og
from mxfp8_grouped_gemm_group_amd.workloads import GEMM1_WORKLOADS, make_gemm1_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL, ABS = 2e-5, 1e-6
SENTINEL = 0x55
OUT_KIND = {torch.float8_e4m3fn: 0, torch.float8_e5m2: 1}


def _host(inp):
    u8 = lambda x: x.detach().contiguous().view(torch.uint8).cpu().numpy()
    return dict(xin=u8(inp["xin"]), w13=u8(inp["w13"]), scale=u8(inp["scale"]),
                xin_scale=u8(inp["xin_scale"]), group_list=inp["group_list"].cpu().numpy())


def run_gpu(inp, **kw):
    import mxfp8_grouped_gemm_group_amd as gfr
    gfr.load_library()
    M, I = inp["xin"].shape[0], (inp["w13"].shape[1] if inp["transpose_w13"]
                                 else inp["w13"].shape[2]) // 2
    q = torch.full((M, I), SENTINEL, dtype=torch.uint8, device=DEV).view(inp["out_dtype"])
    s = torch.full((M, I // 64, 2), SENTINEL, dtype=torch.uint8, device=DEV)
    gfr.gemm1_swiglu_quant(inp["xin"], inp["w13"], inp["scale"], inp["xin_scale"],
                           inp["group_list"], inp["group_list_type"], inp["transpose_w13"],
                           inp["out_dtype"], x1_out=q, x1_scale_out=s, **kw)
    torch.cuda.synchronize()
    return q.view(torch.uint8).cpu().numpy(), s.cpu().numpy().reshape(M, -1)


def run_oracle(inp, rows):
    h = _host(inp)
    return og.gemm1_swiglu_quant(h["xin"], h["w13"], h["scale"], h["xin_scale"],
                                 h["group_list"], inp["group_list_type"], inp["transpose_w13"],
                                 0 if inp["xin"].dtype == torch.float8_e4m3fn else 1,
                                 OUT_KIND[inp["out_dtype"]], rows=rows, with_slack=True)


def check(q, s, r, rows, out_kind, what):
    """q, s: GPU codes [M, I] and scale bytes [M, I/32]; r: oracle result for
    `rows` (token indices)."""
    routed = r["routed"]
    # untouched rows
    un = rows[~routed]
    assert (q[un] == SENTINEL).all() and (s[un] == SENTINEL).all(), f"{what}: unrouted row written"
    rr = rows[routed]
    qg, sg = q[rr], s[rr]
    g, u, sw = r["gate"][routed], r["up"][routed], r["sw"][routed]
    dg = REL * r["gmag"][routed] + ABS + r["gslack"][routed]
    du = REL * r["umag"][routed] + ABS + r["uslack"][routed]
    dsw = 1.1 * (np.abs(u) + du) * dg + np.abs(og.silu(g)) * du + 2.0 ** -20 * np.abs(sw)
    R, I = sw.shape
    nb = I // 32
    Xg = sg.astype(np.int64) - 127
    a = np.abs(sw).reshape(R, nb, 32)
    d = dsw.reshape(R, nb, 32)
    x_lo = og.block_exponent(np.maximum(a - d, 0).max(axis=2), out_kind)
    x_hi = og.block_exponent((a + d).max(axis=2), out_kind)
    bad_x = (Xg < x_lo) | (Xg > x_hi)
    assert not bad_x.any(), (f"{what}: block exponent outside its interval at "
                             f"{np.argwhere(bad_x)[:3].tolist()}")
    Xe = np.repeat(Xg, 32, axis=1)
    lo = og.fp8_decode(og.fp8_encode(np.ldexp(sw - dsw, -Xe), out_kind), out_kind)
    hi = og.fp8_decode(og.fp8_encode(np.ldexp(sw + dsw, -Xe), out_kind), out_kind)
    val = og.fp8_decode(qg, out_kind)
    bad = (val < lo) | (val > hi)
    assert not bad.any(), (f"{what}: {int(bad.sum())} codes outside their interval, first "
                           f"{np.argwhere(bad)[:3].tolist()}")
    same = (og.fp8_decode(r["codes"][routed], out_kind) == val).mean() if val.size else 1.0
    same_x = (r["X"][routed] == Xg).mean() if Xg.size else 1.0
    print(f"{what}: {val.size} codes, {same * 100:.3f} % equal to the oracle's, "
          f"{same_x * 100:.3f} % of block exponents", flush=True)
    assert same >= 0.99 and same_x >= 0.99


SMALL = ["g1_small", "g1_small_t", "g1_big", "g1_big_t_pe", "g1_llada_op"]


@pytest.mark.parametrize("name", SMALL)
def test_gemm1_small_full(name):
    w = GEMM1_WORKLOADS[name]
    print(f"case {name}", flush=True)
    inp = make_gemm1_inputs(w, DEV)
    q, s = run_gpu(inp)
    rows = np.arange(w.M)
    r = run_oracle(inp, rows)
    check(q, s, r, rows, OUT_KIND[inp["out_dtype"]], name)


@pytest.mark.parametrize("name", ["g1_llada", "g1_c2t", "g1_c3"])
def test_gemm1_full_shapes_sampled(name):
    w = GEMM1_WORKLOADS[name]
    print(f"case {name}", flush=True)
    inp = make_gemm1_inputs(w, DEV)
    q, s = run_gpu(inp)
    rng = np.random.default_rng(1)
    c = w.counts()
    ends = np.cumsum(c)
    starts = ends - c
    # first and last token of up to 12 non-empty experts, plus random tokens
    ex = rng.permutation(np.flatnonzero(c > 0))[:12]
    rows = np.unique(np.concatenate([starts[ex], ends[ex] - 1,
                                     rng.choice(w.M, 12, replace=False)]))
    r = run_oracle(inp, rows)
    check(q, s, r, rows, OUT_KIND[inp["out_dtype"]], name)


def test_gemm1_feeds_the_finalize_operator():
    """x1 / pertoken_scale produced by the upstream step are accepted by
    gmm_finalize_routing and give the oracle's result on those codes (the
    down projection of the FFN)."""
    import oracle
    import mxfp8_grouped_gemm_group_amd as gfr
    w = GEMM1_WORKLOADS["g1_small"]
    inp = make_gemm1_inputs(w, DEV)
    q, s = gfr.gemm1_swiglu_quant(inp["xin"], inp["w13"], inp["scale"], inp["xin_scale"],
                                  inp["group_list"], inp["group_list_type"],
                                  inp["transpose_w13"], inp["out_dtype"])
    torch.cuda.synchronize()
    M, I, N, E = w.M, w.I, 256, w.E
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    w2 = torch.randn((E, I, N), generator=g, device=DEV).to(torch.float8_e4m3fn)
    sc2 = torch.full(((I + 63) // 64, N, 2), 126, dtype=torch.uint8, device=DEV)
    batch = 64
    row_index = torch.arange(M, device=DEV, dtype=torch.int64) % batch
    logit = torch.rand(M, generator=g, device=DEV)
    out = torch.zeros((batch, N), device=DEV)
    gfr.gmm_finalize_routing(q, w2, sc2, s, inp["group_list"], inp["group_list_type"], logit,
                             row_index, None, 1.0, 0, out, False)
    torch.cuda.synchronize()
    u8 = lambda x: x.contiguous().view(torch.uint8).cpu().numpy()
    ref, mag = oracle.gmm_finalize_routing(
        u8(q), u8(w2), u8(sc2), s.cpu().numpy(), inp["group_list"].cpu().numpy(),
        inp["group_list_type"], logit.cpu().numpy(), row_index.cpu().numpy(), None, 1.0, 0,
        np.zeros((batch, N), np.float32), False, 0)
    # MX-quantised rows use the whole code range inside each 8-element run, so
    # the block-scaled MFMA's in-group truncation applies: bar + its bound
    slack = oracle.mx_group_slack(
        u8(q), u8(w2), u8(sc2), s.cpu().numpy(), inp["group_list"].cpu().numpy(),
        inp["group_list_type"], logit.cpu().numpy(), row_index.cpu().numpy(), False, 0, batch)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    worst = float(np.max(err / (REL * mag + ABS + slack)))
    print(f"gemm1 -> finalize: worst err / (bar + truncation bound) = {worst:.3g}", flush=True)
    assert worst <= 1.0


def test_gemm1_status_and_limits():
    import mxfp8_grouped_gemm_group_amd as gfr
    inp = make_gemm1_inputs(GEMM1_WORKLOADS["g1_small_t"], DEV)
    with pytest.raises(ValueError):
        gfr.gemm1_swiglu_quant(inp["xin"], inp["w13"][:, :100], inp["scale"], inp["xin_scale"],
                               inp["group_list"], 0, True)
    # I % 64 != 0 is rejected by the library (the binding passes it through)
    w13 = inp["w13"][:, :2 * 288].contiguous()
    sc = inp["scale"][:2 * 288].contiguous()
    with pytest.raises(gfr.GfrError) as e:
        gfr.gemm1_swiglu_quant(inp["xin"], w13, sc, inp["xin_scale"], inp["group_list"], 0, True)
    assert e.value.code == 4
