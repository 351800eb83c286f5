"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before any device call."""
import ctypes
import os
import re

import pytest

import mxfp8_grouped_gemm_group_amd as gfr
from mxfp8_grouped_gemm_group_amd._binding import GfrOptions

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, re.M))
    return names


def test_library_exports_every_declared_function():
    lib = gfr.load_library()
    names = _declared_functions()
    assert {"gmm_finalize_routing", "gmm_finalize_routing_ex", "gfr_workspace_size",
            "gfr_status_string", "gfr_gemm1_swiglu_quant", "gfr_w4a8_finalize_routing"} <= names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(0, 9):
        assert gfr.status_string(code)
    assert gfr.status_string(0) == "ok"
    assert gfr.status_string(999) == "unknown status"


def test_workspace_size():
    assert gfr.workspace_size(768, 8192, 4096, 32, 256, False) == 0
    need = gfr.workspace_size(768, 8192, 4096, 32, 256, True)
    assert need >= 768 * 4096 * 4 + 4 * (2 * 256 + 257 + 768)


def _call(**over):
    """Call gmm_finalize_routing_ex with fake non-null pointers and overrides;
    only argument combinations that fail host validation are used, so nothing
    is ever launched and no pointer is dereferenced."""
    lib = gfr.load_library()
    fake = 0x10000
    a = dict(x1=fake, x2=fake, scale=fake, pts=fake, group_list=fake, gtype=1, logit=fake,
             row_index=fake, shared=fake, sw=1.0, soff=0, out=fake, trans=0, kind=0,
             M=768, K=8192, N=4096, E=32, batch=256, R=256, stream=None, opts=None)
    a.update(over)
    return lib.gmm_finalize_routing_ex(
        a["x1"], a["x2"], a["scale"], a["pts"], a["group_list"], a["gtype"], a["logit"],
        a["row_index"], a["shared"], a["sw"], a["soff"], a["out"], a["trans"], a["kind"],
        a["M"], a["K"], a["N"], a["E"], a["batch"], a["R"], a["stream"], a["opts"])


@pytest.mark.parametrize("over,code", [
    (dict(x1=None), 1), (dict(x2=None), 1), (dict(scale=None), 1), (dict(pts=None), 1),
    (dict(group_list=None), 1), (dict(row_index=None), 1), (dict(out=None), 1),
    (dict(M=-1), 2), (dict(K=0), 2), (dict(E=0), 2), (dict(batch=-3), 2),
    (dict(soff=-1), 3), (dict(soff=1), 3), (dict(R=257), 3),
    (dict(K=8000), 4), (dict(N=4100), 4), (dict(E=1025), 4), (dict(M=1 << 31), 4),
    (dict(x1=0x10004), 5), (dict(x2=0x10008), 5), (dict(scale=0x10001), 5),
    (dict(shared=0x10002), 5),
    (dict(kind=3), 7), (dict(gtype=2), 7), (dict(trans=3), 7),
    # MXFP4: [K,N] x2 needs N % 32 (16-byte rows), [N,K] x2 K % 256
    (dict(kind=2, N=4112), 4), (dict(kind=2, trans=1, K=8064), 4),
])
def test_host_validation(over, code):
    assert _call(**over) == code


def test_deterministic_needs_workspace():
    opts = GfrOptions(1, None, 0, None, 0)
    assert _call(opts=ctypes.byref(opts)) == 6
    opts = GfrOptions(1, 0x10000, 100, None, 0)
    assert _call(opts=ctypes.byref(opts)) == 6


def test_deterministic_alignment():
    big = 1 << 40
    # workspace not 256-byte aligned
    opts = GfrOptions(1, 0x10010, big, None, 0)
    assert _call(opts=ctypes.byref(opts)) == 5
    # out only 4-byte aligned: fine for atomics, not for the float4 row reduction
    opts = GfrOptions(1, 0x10000, big, None, 0)
    assert _call(out=0x10004, opts=ctypes.byref(opts)) == 5


def test_scale_per_expert_flag_is_validated():
    opts = GfrOptions(0, None, 0, None, 0, 2)
    assert _call(opts=ctypes.byref(opts)) == 7


def test_empty_output_is_a_noop():
    # N = 0 or batch = 0: valid per the empty-tensor rules, returns before any launch
    assert _call(N=0) == 0
    assert _call(batch=0, R=0, shared=None) == 0


def _call_gemm1(**over):
    """gfr_gemm1_swiglu_quant with fake non-null pointers; only combinations
    that fail host validation (or are no-ops) are used: nothing is launched."""
    lib = gfr.load_library()
    fake = 0x10000
    a = dict(xin=fake, w13=fake, scale=fake, xs=fake, gl=fake, gtype=1, q=fake, qs=fake,
             trans=0, kind=0, okind=0, M=768, H=4096, I=8192, E=32, stream=None, opts=None)
    a.update(over)
    return lib.gfr_gemm1_swiglu_quant(
        a["xin"], a["w13"], a["scale"], a["xs"], a["gl"], a["gtype"], a["q"], a["qs"],
        a["trans"], a["kind"], a["okind"], a["M"], a["H"], a["I"], a["E"], a["stream"], a["opts"])


@pytest.mark.parametrize("over,code", [
    (dict(xin=None), 1), (dict(w13=None), 1), (dict(scale=None), 1), (dict(xs=None), 1),
    (dict(gl=None), 1), (dict(q=None), 1), (dict(qs=None), 1),
    (dict(M=-1), 2), (dict(H=0), 2), (dict(I=-64), 2), (dict(E=0), 2),
    (dict(H=4000), 4), (dict(I=8160), 4), (dict(E=1025), 4), (dict(kind=2), 4),
    (dict(H=65536, I=32768), 4),                         # 2I * H >= 2^31
    (dict(xin=0x10008), 5), (dict(w13=0x10004), 5), (dict(scale=0x10001), 5),
    (dict(kind=3), 7), (dict(okind=2), 7), (dict(gtype=2), 7), (dict(trans=2), 7),
    (dict(M=0, xin=None, gl=None), 0), (dict(I=0), 0),  # nothing to produce
])
def test_gemm1_host_validation(over, code):
    assert _call_gemm1(**over) == code


def test_gemm1_scale_per_expert_flag_is_validated():
    opts = GfrOptions(0, None, 0, None, 0, 2)
    assert _call_gemm1(opts=ctypes.byref(opts)) == 7


def _call_w4a8(**over):
    """gfr_w4a8_finalize_routing with fake pointers; only failing or no-op
    argument combinations are used: nothing is launched."""
    lib = gfr.load_library()
    fake = 0x10000
    a = dict(x1=fake, x2=fake, scale=fake, offset=None, pts=fake, gl=fake, gtype=1, logit=fake,
             ri=fake, shared=fake, sw=1.0, soff=0, out=fake, M=4096, K=2048, N=7168, E=256,
             batch=512, R=512, stream=None, opts=None)
    a.update(over)
    return lib.gfr_w4a8_finalize_routing(
        a["x1"], a["x2"], a["scale"], a["offset"], a["pts"], a["gl"], a["gtype"], a["logit"],
        a["ri"], a["shared"], a["sw"], a["soff"], a["out"], a["M"], a["K"], a["N"], a["E"],
        a["batch"], a["R"], a["stream"], a["opts"])


@pytest.mark.parametrize("over,code", [
    (dict(x1=None), 1), (dict(x2=None), 1), (dict(scale=None), 1), (dict(pts=None), 1),
    (dict(gl=None), 1), (dict(ri=None), 1), (dict(out=None), 1),
    (dict(M=-1), 2), (dict(K=0), 2), (dict(E=0), 2),
    (dict(soff=1), 3), (dict(R=513), 3),
    (dict(K=2000), 4), (dict(K=131072), 4), (dict(N=7184), 4), (dict(E=1025), 4),
    (dict(x1=0x10008), 5), (dict(x2=0x10004), 5), (dict(scale=0x10004), 5),
    (dict(offset=0x10004), 5), (dict(pts=0x10002), 5), (dict(shared=0x10002), 5),
    (dict(gtype=2), 7),
    (dict(N=0), 0), (dict(batch=0, R=0, shared=None), 0),
])
def test_w4a8_host_validation(over, code):
    assert _call_w4a8(**over) == code


def test_w4a8_options_are_validated():
    assert _call_w4a8(opts=ctypes.byref(GfrOptions(0, None, 0, None, 0, 1))) == 7
    assert _call_w4a8(opts=ctypes.byref(GfrOptions(1, None, 0, None, 0, 0))) == 6
