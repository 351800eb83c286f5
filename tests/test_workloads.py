"""Seeded input generators: shapes, determinism and the routing recipes."""
import numpy as np
import pytest
import torch

from mxfp8_grouped_gemm_group_amd.workloads import (GEMM1_WORKLOADS, WORKLOADS, as_numpy,
                                                    make_gemm1_inputs, make_inputs, sample_rows)


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


def test_sample_rows_cover_shared_edges():
    w = WORKLOADS["c4"]
    r = sample_rows(w, 16)
    for e in (127, 128, 383, 384, 0, 511):
        assert e in r


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
