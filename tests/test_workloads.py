"""Seeded input generators: shapes, determinism and the routing recipes."""
import numpy as np
import pytest
import torch

from mxfp8_grouped_gemm_group_amd.workloads import WORKLOADS, make_inputs, as_numpy, sample_rows


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
