"""The library's entry points under HIP graph capture.

Each call is captured once (inputs and outputs preallocated, the output reset
inside the graph where the call accumulates into it), then replayed several
times with unrelated eager work and synchronisations in between; every replay
is checked against an eager call: bit for bit where the result is
deterministic (integer-exact inputs in both scatter modes, the upstream step,
integer-exact W4A8).  The library clears its workspace with a fill
kernel, never with a memset node.
"""
import pytest
import torch

from mxfp8_grouped_gemm_group_amd.workloads import (GEMM1_WORKLOADS, WORKLOADS, make_gemm1_inputs,
                                                    make_inputs, make_w4a8_inputs)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


def _gfr():
    import mxfp8_grouped_gemm_group_amd as gfr
    gfr.load_library()
    return gfr


def _replay_and_check(call, out, eager, check):
    """Capture call() (which writes out) and compare REPLAYS replays with eager."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                        # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    a = torch.randn(512, 512, device=DEV)
    for i in range(REPLAYS):
        out.fill_(float("nan")) if out.dtype.is_floating_point else out.fill_(0x55)
        g.replay()
        torch.cuda.synchronize()
        check(out, eager, i)
        _ = (a @ a).sum().item()      # eager work between replays
    del g


@pytest.mark.parametrize("deterministic", [False, True])
def test_finalize_under_graph(deterministic):
    gfr = _gfr()
    # integer-valued inputs: exact in FP32 in any atomic order, so every
    # replay must equal the eager call bit for bit in both modes
    w = WORKLOADS["small_big_n_exact"]
    inp = make_inputs(w, DEV)
    init = inp["out"].clone()
    ws = torch.empty(max(1, gfr.workspace_size(w.M, w.K, w.N, w.E, w.batch, True)),
                     dtype=torch.uint8, device=DEV) if deterministic else None
    out = torch.empty_like(init)

    def call():
        out.copy_(init)
        gfr.gmm_finalize_routing(inp["x1"], inp["x2"], inp["scale"], inp["pertoken_scale"],
                                 inp["group_list"], inp["group_list_type"], inp["logit"],
                                 inp["row_index"], inp["shared_input"],
                                 inp["shared_input_weight"], inp["shared_input_offset"], out,
                                 inp["transpose_x2"], deterministic=deterministic, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()

    def check(o, e, i):
        assert torch.equal(o, e), f"replay {i} differs from the eager call"

    _replay_and_check(call, out, eager, check)


def test_gemm1_under_graph():
    gfr = _gfr()
    w = GEMM1_WORKLOADS["g1_big"]
    inp = make_gemm1_inputs(w, DEV)
    q = torch.zeros((w.M, w.I), dtype=torch.uint8, device=DEV).view(inp["out_dtype"])
    qs = torch.zeros((w.M, w.I // 64, 2), dtype=torch.uint8, device=DEV)

    def call():
        gfr.gemm1_swiglu_quant(inp["xin"], inp["w13"], inp["scale"], inp["xin_scale"],
                               inp["group_list"], inp["group_list_type"], inp["transpose_w13"],
                               inp["out_dtype"], x1_out=q, x1_scale_out=qs)

    call()
    torch.cuda.synchronize()
    eager_q, eager_s = q.view(torch.uint8).clone(), qs.clone()
    qb = q.view(torch.uint8)

    def check(o, e, i):
        assert torch.equal(qb, eager_q) and torch.equal(qs, eager_s), f"replay {i} differs"

    # every routed row is rewritten, so resetting the codes shows a stale replay
    _replay_and_check(call, qb, None, check)


def test_w4a8_exact_under_graph():
    gfr = _gfr()
    w = WORKLOADS["w4a8_small_big_exact"]
    inp = make_w4a8_inputs(w, DEV)
    init = inp["out"].clone()
    out = torch.empty_like(init)

    def call():
        out.copy_(init)
        gfr.w4a8_finalize_routing(inp["x1"], inp["x2"], inp["scale"], inp["offset"],
                                  inp["pertoken_scale"], inp["group_list"],
                                  inp["group_list_type"], inp["logit"], inp["row_index"],
                                  inp["shared_input"], inp["shared_input_weight"],
                                  inp["shared_input_offset"], out)

    call()
    torch.cuda.synchronize()
    eager = out.clone()

    def check(o, e, i):
        assert torch.equal(o, e), f"replay {i} differs from the eager call"

    _replay_and_check(call, out, eager, check)
