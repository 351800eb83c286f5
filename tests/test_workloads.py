"""Seeded input generators: shapes, determinism and the routing recipes."""
import numpy as np
import pytest
import torch

from mxfp8_grouped_gemm_group_amd.workloads import (GEMM1_WORKLOADS, WORKLOADS, as_numpy,
                                                    make_gemm1_inputs, make_inputs)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "p1_tc_a", "p1_tc_b",
                                  "p2_ragged", "small_n", "small_t", "small_big_n", "small_big_t",
                                  "small_t_fp4", "c5_fp4"])
def test_counts(name):
    w = WORKLOADS[name]
    c = w.counts()
    assert c.shape == (w.E,) and (c >= 0).all() and c.sum() <= w.M
    if w.groups == "uniform":
        assert c.max() - c.min() <= 1 and c.sum() == w.M
        assert (np.diff(c) <= 0).all()   # remainder goes to leading experts


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_zipf_routing_has_empty_and_heavy_experts(name):
    c = WORKLOADS[name].counts()
    assert c.sum() == WORKLOADS[name].M
    assert (c == 0).sum() == WORKLOADS[name].E // 16
    assert c.max() > 500


@pytest.mark.parametrize("name", ["small_n", "small_t", "small_n_exact", "small_big_n",
                                  "small_big_t_exact", "small_n_pe", "small_big_t_pe",
                                  "small_t_fp4", "small_big_t_fp4_exact",
                                  "small_big_n_fp4_exact"])
def test_make_inputs_shapes_and_determinism(name):
    w = WORKLOADS[name]
    a = make_inputs(w)
    b = make_inputs(w)
    KB = (w.K + 63) // 64
    per = 2 if w.fp8 == "e2m1" else 1       # MXFP4: two elements per byte along the last axis
    assert a["x1"].shape == (w.M, w.K // per)
    assert a["x2"].shape == ((w.E, w.N, w.K // per) if w.transpose_x2 else (w.E, w.K, w.N // per))
    s3 = (w.N, KB, 2) if w.transpose_x2 else (KB, w.N, 2)
    assert a["scale"].shape == (((w.E,) + s3) if w.scale_per_expert else s3)
    assert a["pertoken_scale"].shape == (w.M, KB, 2)
    assert a["out"].shape == (w.batch, w.N) and a["out"].dtype == torch.float32
    assert a["shared_input"].shape == (w.R, w.N)
    assert int(a["row_index"].min()) >= 0 and int(a["row_index"].max()) < w.batch
    g = a["group_list"].numpy()
    assert np.array_equal(np.diff(np.concatenate([[0], g])) if w.group_list_type == 0 else g,
                          w.counts())
    na, nb = as_numpy(a), as_numpy(b)
    for k in ("x1", "x2", "scale", "pertoken_scale", "row_index", "out_init", "logit"):
        assert np.array_equal(na[k], nb[k])
    if w.exact and w.fp8 == "e2m1":
        codes = np.concatenate([na["x1"] & 15, na["x1"] >> 4])   # E2M1 0, +-1, +-2 only
        assert set(np.unique(codes)) <= {0, 2, 4, 10, 12}
    elif w.exact:
        v = a["x1"].to(torch.float32)
        assert torch.equal(v, v.round()) and v.abs().max() <= 2


@pytest.mark.parametrize("name", ["c4", "c5", "w4a8_p3"])
def test_coverage_rows_reach_every_cooperative_group(name):
    from tests.coverage import COOP_MIN_ROWS, GROUP_STEP, coverage_rows
    w = WORKLOADS[name]
    ri = np.random.default_rng(5).permutation(np.tile(np.arange(w.batch), -(-w.M // w.batch)))[:w.M]
    rows = coverage_rows(w, ri)
    assert np.all(np.diff(rows) > 0) and rows[0] >= 0 and rows[-1] < w.batch
    assert rows.size >= 18 and {0, w.batch - 1} <= set(rows.tolist())
    if w.R > 0:
        for e in (w.shared_offset - 1, w.shared_offset, w.shared_offset + w.R - 1,
                  w.shared_offset + w.R):
            assert not 0 <= e < w.batch or e in rows
    sel = np.isin(ri, rows)
    c = w.counts()
    s = np.concatenate([[0], np.cumsum(c)[:-1]])
    n_coop = 0
    for e in range(w.E):
        if c[e] >= COOP_MIN_ROWS:
            n_coop += 1
            for g0 in range(0, c[e], GROUP_STEP):
                assert sel[s[e] + g0: s[e] + min(c[e], g0 + GROUP_STEP)].any(), (e, g0)
            assert sel[s[e] + c[e] - 1]
    assert n_coop > 0


@pytest.mark.parametrize("name", ["g1_small", "g1_small_t", "g1_big", "g1_big_t_pe",
                                  "g1_llada_op"])
def test_gemm1_inputs_shapes_and_determinism(name):
    w = GEMM1_WORKLOADS[name]
    a, b = make_gemm1_inputs(w), make_gemm1_inputs(w)
    KB = (w.H + 63) // 64
    assert a["xin"].shape == (w.M, w.H)
    assert a["w13"].shape == ((w.E, 2 * w.I, w.H) if w.transpose_w13 else (w.E, w.H, 2 * w.I))
    s3 = (2 * w.I, KB, 2) if w.transpose_w13 else (KB, 2 * w.I, 2)
    assert a["scale"].shape == (((w.E,) + s3) if w.scale_per_expert else s3)
    assert a["xin_scale"].shape == (w.M, KB, 2)
    for k in ("xin", "w13", "scale", "xin_scale", "group_list"):
        assert torch.equal(a[k].view(torch.uint8) if a[k].dtype != torch.int64 else a[k],
                           b[k].view(torch.uint8) if b[k].dtype != torch.int64 else b[k])
    c = w.counts()
    assert c.shape == (w.E,) and c.sum() <= w.M and w.I % 64 == 0 and w.H % 128 == 0
    if w.zero_rows:
        assert (a["xin"][: w.zero_rows].view(torch.uint8) == 0).all()


def test_gemm1_llada_op_counts_follow_the_page():
    assert list(GEMM1_WORKLOADS["g1_llada_op"].counts()) == [0, 1, 2, 4, 8, 16, 32, 0]
