"""Tiny raw-code inputs for the oracle's pins, and an independent float64
reference built from library primitives.

The reference follows the golden description of the grouped_matmul_finalize_
routing MXFP8 page (§6.3: expand every E8M0 scale over 32 K elements, do the
matmul per expert, weight by logit, index_add into out, add the shared input)
using torch's own float8/bfloat16 decoding, ``np.repeat``, ``numpy.matmul`` and
``np.add.at`` -- none of which the C oracle uses.
"""
import numpy as np
import torch

_F8 = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


# The FP4 E2M1 value set (OCP Microscaling formats v1.0, element table): codes
# 0..7 are +0, 0.5, 1, 1.5, 2, 3, 4, 6 and codes 8..15 their negatives.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def unpack_e2m1(packed):
    """[..., L/2] bytes -> [..., L] codes, element 2j from the low nibble of byte j."""
    packed = np.ascontiguousarray(packed)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


def pack_e2m1(codes):
    """[..., L] codes (0..15) -> [..., L/2] bytes (inverse of unpack_e2m1)."""
    codes = np.ascontiguousarray(codes).astype(np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def decode_np(codes, kind):
    """Decode raw codes: kind 0/1 (FP8 E4M3FN/E5M2, with torch), 2 (packed
    E2M1, with the value table) or 'bf16' (with torch)."""
    codes = np.ascontiguousarray(codes)
    if kind == "bf16":
        return torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    if kind == 2:
        return E2M1_VALUES[unpack_e2m1(codes)]
    return torch.from_numpy(codes).view(_F8[kind]).to(torch.float64).numpy()


def _encode(values, kind):
    t = torch.as_tensor(np.asarray(values, np.float32))
    return t.to(_F8[kind]).view(torch.uint8).numpy()


def _finite_codes(kind):
    c = np.arange(256, dtype=np.uint8)
    v = decode_np(c, kind)
    return c[np.isfinite(v)]


def tiny_case(seed, E, M, K, N, transpose, kind, gtype, groups=None, batch=None,
              routing="random", unit_scales=False, logit="random", shared=True,
              exact=False, per_expert=False):
    rng = np.random.default_rng(seed)
    KB = (K + 63) // 64
    x2s = (E, N, K) if transpose else (E, K, N)
    if kind == 2:   # packed E2M1 along the last axis
        pool = np.array([0, 2, 4, 10, 12], np.uint8) if exact else np.arange(16, dtype=np.uint8)
        x1 = pack_e2m1(rng.choice(pool, size=(M, K)))       # exact: 0, +-1, +-2
        x2 = pack_e2m1(rng.choice(pool, size=x2s))
    elif exact:
        x1 = _encode(rng.integers(-2, 3, size=(M, K)), kind)
        x2 = _encode(rng.integers(-2, 3, size=x2s), kind)
    else:
        fc = _finite_codes(kind)
        x1 = rng.choice(fc, size=(M, K))
        x2 = rng.choice(fc, size=(E, N, K) if transpose else (E, K, N))
    lo, hi = (0, 1) if exact else (-4, 4)
    if unit_scales:
        pts = np.full((M, KB, 2), 127, np.uint8)
        sc = np.full((N, KB, 2) if transpose else (KB, N, 2), 127, np.uint8)
    else:
        pts = (127 + rng.integers(lo, hi + 1, size=(M, KB, 2))).astype(np.uint8)
        sc = (127 + rng.integers(lo, hi + 1,
                                 size=(N, KB, 2) if transpose else (KB, N, 2))).astype(np.uint8)
    if per_expert:   # a leading expert axis: (E, N, KB, 2) or (E, KB, N, 2)
        sc = (127 + rng.integers(lo, hi + 1, size=(E,) + sc.shape)).astype(np.uint8)
    if groups is None:
        used = int(rng.integers(M // 2, M + 1))
        cuts = np.sort(rng.integers(0, used + 1, size=E - 1))
        counts = np.diff(np.concatenate([[0], cuts, [used]])).astype(np.int64)
    else:
        counts = np.asarray(groups, np.int64)
    group_list = np.cumsum(counts) if gtype == 0 else counts.copy()
    if batch is None:
        batch = M if routing == "identity" else max(2, M // 2)
    if routing == "identity":
        row_index = np.arange(M, dtype=np.int64)
    else:
        row_index = rng.integers(0, batch, size=M).astype(np.int64)
    if logit == "ones":
        lg = np.ones(M, np.float32)
    elif exact:
        lg = rng.choice(np.array([1.0, 0.5, 0.25], np.float32), size=M)
    else:
        lg = rng.random(M, dtype=np.float32)
    if shared:
        R = int(rng.integers(1, batch + 1))
        off = int(rng.integers(0, batch - R + 1))
        vals = rng.integers(-4, 5, size=(R, N)) if exact else rng.standard_normal((R, N))
        sh = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        sw = 0.75 if exact else 1.3
    else:
        sh, off, sw = None, 0, 1.0
    init = (rng.integers(-4, 5, size=(batch, N)) if exact
            else rng.standard_normal((batch, N))).astype(np.float32)
    return dict(x1=x1, x2=x2, scale=sc, pertoken_scale=pts, group_list=group_list,
                group_list_type=gtype, logit=lg, row_index=row_index, shared_input=sh,
                shared_input_weight=sw, shared_input_offset=off, out_init=init,
                transpose_x2=transpose, fp8_kind=kind)


def numpy_reference(c):
    """Independent float64 formulation (see module docstring)."""
    kind = c["fp8_kind"]
    x1 = decode_np(c["x1"], kind)      # E2M1: unpacked to [M, K] here
    M, K = x1.shape
    s1 = np.exp2(c["pertoken_scale"].astype(np.float64) - 127).reshape(M, -1)
    x1dq = x1 * np.repeat(s1, 32, axis=1)[:, :K]
    x2 = decode_np(c["x2"], kind)
    E = x2.shape[0]
    sc = c["scale"]
    sc4 = sc if sc.ndim == 4 else np.broadcast_to(sc, (E,) + sc.shape)   # per-expert view
    x2dq = np.empty((E, K, x2.shape[1] if c["transpose_x2"] else x2.shape[2]))
    for e in range(E):
        if c["transpose_x2"]:
            N = x2.shape[1]
            s2 = np.exp2(sc4[e].astype(np.float64) - 127).reshape(N, -1)       # [N, 2KB]
            x2dq[e] = (x2[e] * np.repeat(s2, 32, axis=1)[:, :K]).T
        else:
            N = x2.shape[2]
            s3 = np.exp2(sc4[e].astype(np.float64) - 127)                        # [KB, N, 2]
            s2 = np.moveaxis(s3, 2, 1).reshape(-1, N)                             # [2KB, N]
            x2dq[e] = x2[e] * np.repeat(s2, 32, axis=0)[:K]
    counts = (np.diff(np.concatenate([[0], c["group_list"]])) if c["group_list_type"] == 0
              else c["group_list"])
    out = c["out_init"].astype(np.float64).copy()
    lg = c["logit"] if c["logit"] is not None else np.ones(M, np.float32)
    start = 0
    for e, cnt in enumerate(counts):
        rows = slice(start, start + int(cnt))
        mm = x1dq[rows] @ x2dq[e]
        np.add.at(out, c["row_index"][rows], mm * lg[rows, None].astype(np.float64))
        start += int(cnt)
    if c["shared_input"] is not None:
        sh = decode_np(c["shared_input"], "bf16")
        off = c["shared_input_offset"]
        out[off:off + sh.shape[0]] += c["shared_input_weight"] * sh
    return out
