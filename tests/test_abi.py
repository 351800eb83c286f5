"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before any device call --
the raw calls' size, pointer, alignment and enum checks, and the descriptor
calls' dtype, rank and shape checks (every argument combination used here
fails validation or is a no-op, so nothing is ever launched and no pointer is
dereferenced)."""
import ctypes
import os
import re

import pytest

import mxfp8_grouped_gemm_group_amd as gfr
from mxfp8_grouped_gemm_group_amd._binding import GfrOptions, GfrTensor

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
            "gfr_status_string", "gfr_gemm1_swiglu_quant", "gfr_w4a8_finalize_routing",
            "gmm_finalize_routing_raw", "gmm_finalize_routing_raw_ex", "gfr_workspace_size_raw",
            "gfr_gemm1_swiglu_quant_raw", "gfr_w4a8_finalize_routing_raw",
            "gmm_finalize_routing_det_noalloc"} <= names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(0, 12):
        assert gfr.status_string(code) != "unknown status"
    assert gfr.status_string(0) == "ok"
    assert gfr.status_string(999) == "unknown status"


def test_workspace_size():
    assert gfr.workspace_size(768, 8192, 4096, 32, 256, False) == 0
    need = gfr.workspace_size(768, 8192, 4096, 32, 256, True)
    assert need >= 768 * 4096 * 4 + 4 * (2 * 256 + 257 + 768)


def _call(**over):
    """Call gmm_finalize_routing_raw_ex with fake non-null pointers and overrides;
    only argument combinations that fail host validation are used, so nothing
    is ever launched and no pointer is dereferenced."""
    lib = gfr.load_library()
    fake = 0x10000
    a = dict(x1=fake, x2=fake, scale=fake, pts=fake, group_list=fake, gtype=1, logit=fake,
             row_index=fake, shared=fake, sw=1.0, soff=0, out=fake, trans=0, kind=0,
             M=768, K=8192, N=4096, E=32, batch=256, R=256, stream=None, opts=None)
    a.update(over)
    return lib.gmm_finalize_routing_raw_ex(
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
    """gfr_gemm1_swiglu_quant_raw with fake non-null pointers; only combinations
    that fail host validation (or are no-ops) are used: nothing is launched."""
    lib = gfr.load_library()
    fake = 0x10000
    a = dict(xin=fake, w13=fake, scale=fake, xs=fake, gl=fake, gtype=1, q=fake, qs=fake,
             trans=0, kind=0, okind=0, M=768, H=4096, I=8192, E=32, stream=None, opts=None)
    a.update(over)
    return lib.gfr_gemm1_swiglu_quant_raw(
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
    """gfr_w4a8_finalize_routing_raw with fake pointers; only failing or no-op
    argument combinations are used: nothing is launched."""
    lib = gfr.load_library()
    fake = 0x10000
    a = dict(x1=fake, x2=fake, scale=fake, offset=None, pts=fake, gl=fake, gtype=1, logit=fake,
             ri=fake, shared=fake, sw=1.0, soff=0, out=fake, M=4096, K=2048, N=7168, E=256,
             batch=512, R=512, stream=None, opts=None)
    a.update(over)
    return lib.gfr_w4a8_finalize_routing_raw(
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


# ---------------------------------------------------------------------------
# Descriptor calls.
# ---------------------------------------------------------------------------
FAKE = 0x10000
E4M3, E5M2, FP4, E8M0, U8, BF16, F32, I64, I32, I8, INT4 = range(11)


def D(dtype, *shape, data=FAKE, ndim=None):
    t = GfrTensor()
    t.data = data
    t.dtype = dtype
    t.ndim = len(shape) if ndim is None else ndim
    for i, n in enumerate(shape):
        t.shape[i] = n
    return t


def _c3_descs(**over):
    """Descriptors of c3's shapes (M 768, K 8192, N 4096, E 32, batch 256, R 256)."""
    M, K, N, E, B, R = 768, 8192, 4096, 32, 256, 256
    KB = K // 64
    d = dict(x1=D(E4M3, M, K), x2=D(E4M3, E, K, N), scale=D(E8M0, KB, N, 2),
             pts=D(U8, M, KB, 2), gl=D(I64, E), logit=D(F32, M), ri=D(I64, M),
             shared=D(BF16, R, N), out=D(F32, B, N), gtype=0, sw=1.0, soff=0, trans=0, kind=0)
    d.update(over)
    return d


def _args(d):
    r = lambda t: None if t is None else ctypes.byref(t)
    return [r(d["x1"]), r(d["x2"]), r(d["scale"]), r(d["pts"]), r(d["gl"]), d["gtype"],
            r(d["logit"]), r(d["ri"]), r(d["shared"]), d["sw"], d["soff"], r(d["out"]),
            d["trans"], d["kind"]]


def _call_desc(opts=None, **over):
    return gfr.load_library().gmm_finalize_routing_ex(*_args(_c3_descs(**over)), None, opts)


M_, K_, N_, E_, KB_ = 768, 8192, 4096, 32, 128


@pytest.mark.parametrize("over,code", [
    # required descriptors, and data of non-empty tensors
    (dict(x1=None), 1), (dict(x2=None), 1), (dict(scale=None), 1), (dict(pts=None), 1),
    (dict(gl=None), 1), (dict(ri=None), 1), (dict(out=None), 1),
    (dict(x1=D(E4M3, M_, K_, data=None)), 1), (dict(out=D(F32, 256, N_, data=None)), 1),
    # dtypes
    (dict(x1=D(E5M2, M_, K_)), 9), (dict(x2=D(E5M2, E_, K_, N_)), 9), (dict(kind=1), 9),
    (dict(x1=D(U8, M_, K_)), 9), (dict(scale=D(F32, KB_, N_, 2)), 9),
    (dict(pts=D(I8, M_, KB_, 2)), 9), (dict(gl=D(I32, E_)), 9), (dict(ri=D(F32, M_)), 9),
    (dict(logit=D(BF16, M_)), 9), (dict(shared=D(F32, 256, N_)), 9),
    (dict(out=D(BF16, 256, N_)), 9),
    # ranks
    (dict(x1=D(E4M3, M_ * K_)), 10), (dict(x2=D(E4M3, E_ * K_, N_)), 10),
    (dict(scale=D(E8M0, KB_ * N_ * 2)), 10), (dict(pts=D(U8, M_, KB_ * 2)), 10),
    (dict(gl=D(I64, E_, 1)), 10), (dict(ri=D(I64, M_, 1)), 10), (dict(logit=D(F32, 1, M_)), 10),
    (dict(shared=D(BF16, 256 * N_)), 10), (dict(out=D(F32, 256 * N_)), 10),
    (dict(x1=D(E4M3, M_, K_, ndim=5)), 10), (dict(x1=D(E4M3, M_, K_, ndim=0)), 10),
    # shapes: every extent against the sizes the others fix
    (dict(x2=D(E4M3, E_, K_ + 128, N_)), 2), (dict(scale=D(E8M0, KB_ + 1, N_, 2)), 2),
    (dict(scale=D(E8M0, N_, KB_, 2)), 2), (dict(scale=D(E8M0, KB_, N_, 1)), 2),
    (dict(scale=D(E8M0, E_ + 1, KB_, N_, 2)), 2), (dict(pts=D(U8, M_ - 1, KB_, 2)), 2),
    (dict(pts=D(U8, M_, KB_ - 1, 2)), 2), (dict(gl=D(I64, E_ + 1)), 2),
    (dict(ri=D(I64, M_ + 1)), 2), (dict(logit=D(F32, M_ - 1)), 2),
    (dict(out=D(F32, 256, N_ - 16)), 2), (dict(shared=D(BF16, 256, N_ + 16)), 2),
    (dict(x1=D(E4M3, -1, K_)), 2),
    # [N, K] layout: scale must follow it
    (dict(trans=1, x2=D(E4M3, E_, N_, K_)), 2),
    # MXFP4: packed last axis
    (dict(kind=2, x1=D(FP4, M_, K_ // 2), x2=D(FP4, E_, K_, N_)), 2),
    # values the raw layer rejects
    (dict(soff=1), 3), (dict(shared=D(BF16, 257, N_)), 3),
    (dict(x1=D(E4M3, M_, K_ - 64), x2=D(E4M3, E_, K_ - 64, N_), scale=D(E8M0, KB_ - 1, N_, 2),
          pts=D(U8, M_, KB_ - 1, 2)), 4),
    (dict(x1=D(E4M3, M_, K_, data=FAKE + 8)), 5),
    (dict(kind=5), 7), (dict(gtype=2), 7), (dict(trans=2), 7),
])
def test_descriptor_validation(over, code):
    assert _call_desc(**over) == code


def test_descriptor_options():
    # a per-expert flag needs a 4-D scale; an unknown flag value is an argument error
    assert _call_desc(ctypes.byref(GfrOptions(0, None, 0, None, 0, 1))) == 10
    assert _call_desc(ctypes.byref(GfrOptions(0, None, 0, None, 0, 2))) == 7
    # deterministic mode without workspace
    assert _call_desc(ctypes.byref(GfrOptions(1, None, 0, None, 0, 0))) == 6


def test_descriptor_noops():
    # empty outputs: valid, nothing launched
    assert _call_desc(out=D(F32, 256, 0, data=None), x2=D(E4M3, E_, K_, 0, data=None),
                      scale=D(E8M0, KB_, 0, 2, data=None), shared=None) == 0
    assert _call_desc(out=D(F32, 0, N_, data=None), shared=None) == 0


def test_descriptor_workspace_size_matches_raw():
    lib = gfr.load_library()
    n = ctypes.c_size_t(0)
    opts = GfrOptions(1, None, 0, None, 0, 0)
    rc = lib.gfr_workspace_size(*_args(_c3_descs()), ctypes.byref(opts), ctypes.byref(n))
    assert rc == 0 and n.value == gfr.workspace_size(768, 8192, 4096, 32, 256, True)
    opts = GfrOptions(0, None, 0, None, 0, 0)
    rc = lib.gfr_workspace_size(*_args(_c3_descs()), ctypes.byref(opts), ctypes.byref(n))
    assert rc == 0 and n.value == 0
    # it validates like the call: a bad shape is reported, bytes untouched
    n.value = 7
    rc = lib.gfr_workspace_size(*_args(_c3_descs(gl=D(I64, 31))), ctypes.byref(opts),
                                ctypes.byref(n))
    assert rc == 2 and n.value == 7
    assert lib.gfr_workspace_size(*_args(_c3_descs()), None, None) == 1
    # int32 row_index and a 4-D per-expert scale are accepted
    rc = lib.gfr_workspace_size(*_args(_c3_descs(ri=D(I32, 768),
                                                 scale=D(E8M0, 32, 128, 4096, 2))),
                                ctypes.byref(opts), ctypes.byref(n))
    assert rc == 0


def _w4a8_descs(**over):
    M, K, N, E, B = 4096, 2048, 7168, 256, 512
    d = dict(x1=D(I8, M, K), x2=D(INT4, E, K, N // 2), scale=D(F32, E, 1, N),
             offset=D(F32, E, 1, N), pts=D(F32, M), gl=D(I64, E), gtype=1, logit=D(F32, M),
             ri=D(I64, M), shared=D(BF16, B, N), sw=1.0, soff=0, out=D(F32, B, N))
    d.update(over)
    r = lambda t: None if t is None else ctypes.byref(t)
    return [r(d["x1"]), r(d["x2"]), r(d["scale"]), r(d["offset"]), r(d["pts"]), r(d["gl"]),
            d["gtype"], r(d["logit"]), r(d["ri"]), r(d["shared"]), d["sw"], d["soff"],
            r(d["out"])]


@pytest.mark.parametrize("over,code", [
    (dict(x1=None), 1), (dict(x2=None), 1), (dict(scale=None), 1), (dict(pts=None), 1),
    (dict(x1=D(U8, 4096, 2048)), 9), (dict(x2=D(I8, 256, 2048, 3584)), 9),
    (dict(scale=D(BF16, 256, 1, 7168)), 9), (dict(pts=D(F32, 4096, 1)), 10),
    (dict(x2=D(INT4, 256, 2048, 3584, 1)), 10),
    (dict(x2=D(INT4, 256, 2047, 3584)), 2), (dict(scale=D(F32, 256, 1, 7167)), 2),
    (dict(offset=D(F32, 255, 1, 7168)), 2), (dict(pts=D(F32, 4095)), 2),
    (dict(out=D(F32, 512, 7166)), 2), (dict(gl=D(I64, 255)), 2),
    (dict(soff=1), 3), (dict(gtype=3), 7),
])
def test_w4a8_descriptor_validation(over, code):
    assert gfr.load_library().gfr_w4a8_finalize_routing(*_w4a8_descs(**over), None, None) == code


def _gemm1_descs(**over):
    M, H, I, E = 768, 4096, 8192, 32
    d = dict(xin=D(E4M3, M, H), w13=D(E4M3, E, H, 2 * I), scale=D(E8M0, H // 64, 2 * I, 2),
             xs=D(U8, M, H // 64, 2), gl=D(I64, E), gtype=1, q=D(E4M3, M, I),
             qs=D(U8, M, I // 64, 2), trans=0)
    d.update(over)
    r = lambda t: None if t is None else ctypes.byref(t)
    return [r(d["xin"]), r(d["w13"]), r(d["scale"]), r(d["xs"]), r(d["gl"]), d["gtype"],
            r(d["q"]), r(d["qs"]), d["trans"]]


@pytest.mark.parametrize("over,code", [
    (dict(xin=None), 1), (dict(q=None), 1),
    (dict(xin=D(FP4, 768, 2048)), 9), (dict(w13=D(E5M2, 32, 4096, 16384)), 9),
    (dict(q=D(BF16, 768, 8192)), 9), (dict(scale=D(F32, 64, 16384, 2)), 9),
    (dict(xin=D(E4M3, 768 * 4096)), 10), (dict(qs=D(U8, 768, 256)), 10),
    (dict(w13=D(E4M3, 32, 4096, 16383)), 2), (dict(scale=D(E8M0, 64, 16384, 1)), 2),
    (dict(xs=D(U8, 767, 64, 2)), 2), (dict(q=D(E4M3, 768, 8191)), 2),
    (dict(qs=D(U8, 768, 127, 2)), 2), (dict(gl=D(I64, 31)), 2),
    (dict(trans=1), 2), (dict(gtype=2), 7),
])
def test_gemm1_descriptor_validation(over, code):
    assert gfr.load_library().gfr_gemm1_swiglu_quant(*_gemm1_descs(**over), None, None) == code


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """c5's weighted rows (16384 x 4096 float32 = 256 MiB) exceed the static
    scratch: rejected on the host, nothing launched."""
    lib = gfr.load_library()
    M, K, N, E, B = 16384, 7168, 4096, 256, 2048
    d = _c3_descs(x1=D(E5M2, M, K), x2=D(E5M2, E, N, K), scale=D(E8M0, N, K // 64, 2),
                  pts=D(U8, M, K // 64, 2), gl=D(I64, E), logit=D(F32, M), ri=D(I64, M),
                  shared=D(BF16, B, N), out=D(F32, B, N), trans=1, kind=1)
    assert lib.gmm_finalize_routing_det_noalloc(*_args(d), None, None) == 11
    # validation comes first, as in the other calls
    assert lib.gmm_finalize_routing_det_noalloc(*_args(_c3_descs(gl=D(I64, 3))), None, None) == 2
    assert gfr.status_string(11) != "unknown status"
