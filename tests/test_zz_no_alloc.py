"""The allocation-free deterministic entry point (gmm_finalize_routing_det_noalloc).

Its workspace is the library's static per-GPU scratch instead of a caller
buffer.  Through the C ABI it must give exactly the bits of
gmm_finalize_routing_ex in deterministic mode (same kernels, same fixed
summation order), on two calls in a row, the second with smaller inputs (the
scratch keeps the first call's contents), and set the same device status
bits.
"""
import pytest
import torch

from mxfp8_grouped_gemm_group_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _args(inp):
    return (inp["x1"], inp["x2"], inp["scale"], inp["pertoken_scale"], inp["group_list"],
            inp["group_list_type"], inp["logit"], inp["row_index"], inp["shared_input"],
            inp["shared_input_weight"], inp["shared_input_offset"])


def test_noalloc_equals_workspace_call_twice_shrinking():
    import mxfp8_grouped_gemm_group_amd as gfr
    gfr.load_library()
    for name in ("c3", "small_big_t"):     # second call: smaller M, N, batch, K
        w = WORKLOADS[name]
        print(f"case {name}", flush=True)
        inp = make_inputs(w, DEV)
        want = inp["out"].clone()
        gfr.gmm_finalize_routing(*_args(inp), want, inp["transpose_x2"], deterministic=True)
        got = inp["out"].clone()
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        gfr.gmm_finalize_routing_det_noalloc(*_args(inp), got, inp["transpose_x2"], status=st)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{name}: differs from the workspace call"
        assert int(st.item()) == 0


def test_noalloc_status_bits():
    import mxfp8_grouped_gemm_group_amd as gfr
    inp = make_inputs(WORKLOADS["small_n"], DEV)
    inp["row_index"] = inp["row_index"].clone()
    inp["row_index"][40] = WORKLOADS["small_n"].batch + 1     # a routed token's row
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = inp["out"].clone()
    gfr.gmm_finalize_routing_det_noalloc(*_args(inp), out, inp["transpose_x2"], status=st)
    want = inp["out"].clone()
    st2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    gfr.gmm_finalize_routing(*_args(inp), want, inp["transpose_x2"], deterministic=True,
                             status=st2)
    torch.cuda.synchronize()
    assert int(st.item()) & gfr.DEV_BAD_ROW_INDEX and int(st.item()) == int(st2.item())
    assert torch.equal(out, want)
