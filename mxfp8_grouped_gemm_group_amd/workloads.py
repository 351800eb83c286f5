"""Seeded synthetic inputs for the fused MXFP8 grouped-matmul + finalize-routing op.

This module only draws inputs.  It holds none of the operator's arithmetic, so
both the GPU library's tests/benchmark and the CPU oracle can take their inputs
from it.  The construction follows the test-tensor recipe of the page
"基于 PyPTO 的 MoE 融合算子实践：grouped_matmul_finalize_routing 的 MXFP8 实现与精度验证"
(§3.3 tensor construction: FP8 data cast from N(0,1), E8M0 scales, ceil(K/64)
scale blocks of 2, ``row_index = arange(M) % batch``, bf16 shared input, FP32
out; §4.3 ``make_group_list``: uniform groups whose remainder goes to the
leading experts) and the shape table of its §4.1/§6.2.

Random streams:
  * small arrays (scale exponents, logits, routing, shared input, out init) come
    from ``numpy.random.default_rng(seed)`` in a fixed draw order, so they are
    identical on every machine;
  * the large FP8 operands x1/x2 come from ``torch.randn`` with a
    ``torch.Generator`` seeded from the same seed *on the target device* (so the
    GPU can draw a 1 GB weight tensor in milliseconds).  The values therefore
    depend on the device type; the oracle always receives host copies of the
    very tensors the GPU path consumes.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence, Tuple, Union

import numpy as np
import torch

FP8_DTYPES = {"e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2,
              "e2m1": torch.float4_e2m1fn_x2}
FP8_KIND = {"e4m3fn": 0, "e5m2": 1, "e2m1": 2, "w4a8": 8}


@dataclass(frozen=True)
class Workload:
    """One operator invocation's shapes and input distributions."""
    name: str
    batch: int
    K: int
    N: int
    E: int
    M: int
    fp8: str = "e4m3fn"                 # "e4m3fn" | "e5m2" | "e2m1" (MXFP4, packed)
    transpose_x2: bool = False
    group_list_type: int = 1             # 0 prefix sums, 1 counts
    groups: Union[str, Tuple] = "uniform"  # "uniform" | ("zipf", s) | explicit counts
    exp_range: Tuple[int, int] = (-3, 3)  # E8M0 exponents drawn uniformly in [lo, hi]
    logit: str = "uniform"               # "uniform" | "softmax" | "none"
    row_index: str = "mod"               # "mod" (arange % batch) | "perm"
    shared_rows: Optional[int] = None    # None -> batch rows; 0 -> no shared input
    shared_weight: float = 1.0
    shared_offset: int = 0
    out_init: str = "zeros"              # "zeros" | "normal"
    exact: bool = False                  # integer-valued variant, exact in FP32
    seed: int = 0
    topk: int = 0                        # informational (M = batch * topk)
    scale_per_expert: bool = False       # weight scales with a leading expert axis
    w4a8_offset: bool = True             # W4A8 ("w4a8"): asymmetric offset present

    @property
    def fp8_kind(self) -> int:
        return FP8_KIND[self.fp8]

    @property
    def R(self) -> int:
        return self.batch if self.shared_rows is None else self.shared_rows

    def counts(self) -> np.ndarray:
        """Tokens per expert (int64 [E]); deterministic in the seed."""
        return _counts(self)

    def flops(self) -> int:
        """2*M_routed*K*N: one K x N contraction per routed token."""
        return 2 * int(self.counts().sum()) * self.K * self.N

    def algorithmic_bytes(self) -> int:
        """Bytes a single pass must move at least once (HBM roofline numerator).

        x2 of non-empty experts, x1, both scale tensors, logit, row_index,
        group_list, out read + write, shared input.
        """
        c = self.counts()
        active = int((c > 0).sum())
        M_r = int(c.sum())
        K, N = self.K, self.N
        kb32 = 2 * ((K + 63) // 64)
        if self.fp8 == "w4a8":   # int8 x1, int4 x2, FP32 scale (+ offset) and per-token scale
            b = active * K * N // 2 + M_r * K
            b += 4 * N * active * (2 if self.w4a8_offset else 1) + 4 * M_r
        else:
            eb = 0.5 if self.fp8 == "e2m1" else 1   # bytes per element of x1 / x2
            b = int(eb * (active * K * N + M_r * K))
            b += M_r * kb32 + N * kb32 * (active if self.scale_per_expert else 1)
        b += (4 * M_r if self.logit != "none" else 0) + 8 * M_r + 8 * self.E
        b += 8 * self.batch * N + 2 * self.R * N
        return b


# --------------------------------------------------------------------------
# Named workloads.  c1..c5 are the five benchmark configurations (shape sets of
# the page's §4.1/§6.2 plus larger routed-MoE shapes); the rest are parity
# cases: the page's registered test configurations (batch 4 and 128, topk 8,
# K 7168, N 4096, E 8), the ragged zero/odd/power-of-two counts pattern of the
# companion LLaDA2.0 grouped-GEMM page's operator test, and small ragged cases
# that span several tiles.
# --------------------------------------------------------------------------
WORKLOADS: Dict[str, Workload] = {}


def _reg(w: Workload) -> Workload:
    WORKLOADS[w.name] = w
    return w


C1 = _reg(Workload("c1", batch=64, topk=2, M=128, K=5120, N=4096, E=8, fp8="e4m3fn",
                   groups="uniform", group_list_type=1, exp_range=(-3, 3), seed=1001))
C2 = _reg(Workload("c2", batch=128, topk=2, M=256, K=6144, N=4096, E=16, fp8="e5m2",
                   transpose_x2=True, groups="uniform", group_list_type=1, exp_range=(-4, 4),
                   shared_weight=0.5, out_init="normal", seed=1002))
C3 = _reg(Workload("c3", batch=256, topk=3, M=768, K=8192, N=4096, E=32, fp8="e4m3fn",
                   groups="uniform", group_list_type=0, exp_range=(-3, 3), seed=1003))
C4 = _reg(Workload("c4", batch=512, topk=6, M=3072, K=7168, N=4096, E=64, fp8="e4m3fn",
                   groups=("zipf", 1.1), group_list_type=1, exp_range=(-6, 6),
                   row_index="perm", shared_rows=256, shared_weight=0.75, shared_offset=128,
                   seed=1004))
C5 = _reg(Workload("c5", batch=2048, topk=8, M=16384, K=7168, N=4096, E=256, fp8="e5m2",
                   transpose_x2=True, groups=("zipf", 1.2), group_list_type=1,
                   exp_range=(-8, 8), logit="softmax", row_index="perm", seed=1005))

P1_TC_A = _reg(Workload("p1_tc_a", batch=4, topk=8, M=32, K=7168, N=4096, E=8, seed=1011))
P1_TC_B = _reg(Workload("p1_tc_b", batch=128, topk=8, M=1024, K=7168, N=4096, E=8, seed=1012))
P2_RAGGED = _reg(Workload("p2_ragged", batch=16, M=63, K=7168, N=4096, E=8,
                          groups=(0, 1, 2, 4, 8, 16, 32, 0), seed=1013))

# Small cases the oracle finishes in well under a second; several n-tiles,
# ragged tails in M, N and the number of K steps.
SMALL_N = _reg(Workload("small_n", batch=37, M=300, K=1024, N=704, E=7, fp8="e4m3fn",
                        groups=(0, 37, 1, 120, 0, 95, 47), group_list_type=1,
                        exp_range=(-5, 5), row_index="perm", shared_rows=20,
                        shared_weight=0.75, shared_offset=9, out_init="normal", seed=1021))
SMALL_T = _reg(Workload("small_t", batch=64, M=200, K=640, N=576, E=5, fp8="e5m2",
                        transpose_x2=True, groups=(33, 0, 64, 100, 3), group_list_type=0,
                        exp_range=(-6, 6), shared_weight=0.5, out_init="normal", seed=1022))

# Large experts at a size the oracle checks element by element: 300 rows (two
# row groups of 256, the second with 44 rows), 141 (one group of 256 with two
# full, one partial and one empty wave), 70 (a 128-row group), 5 (a 32-row
# tile); partial column tiles in both layouts.
SMALL_BIG_N = _reg(Workload("small_big_n", batch=100, M=516, K=768, N=320, E=5, fp8="e4m3fn",
                            groups=(0, 300, 70, 5, 141), group_list_type=1, exp_range=(-4, 4),
                            row_index="perm", shared_rows=30, shared_weight=0.5,
                            shared_offset=50, out_init="normal", seed=1023))
SMALL_BIG_T = _reg(Workload("small_big_t", batch=86, M=516, K=640, N=352, E=4, fp8="e5m2",
                            transpose_x2=True, groups=(141, 5, 300, 70), group_list_type=0,
                            exp_range=(-4, 4), row_index="perm", seed=1024))

# An expert with more than four 256-row groups (1300 rows: six groups, the last
# with 20 rows), so the cooperative units' order has a short last band of row
# groups, beside an empty expert and a 128-row group (77 rows).
SMALL_HUGE_N = _reg(Workload("small_huge_n", batch=200, M=1377, K=256, N=320, E=3,
                             fp8="e4m3fn", groups=(1300, 0, 77), group_list_type=1,
                             exp_range=(-4, 4), row_index="perm", shared_rows=40,
                             shared_weight=0.75, shared_offset=100, seed=1029))
SMALL_HUGE_T = _reg(Workload("small_huge_t", batch=200, M=1377, K=512, N=352, E=3,
                             fp8="e5m2", transpose_x2=True, groups=(77, 1300, 0),
                             group_list_type=0, exp_range=(-4, 4), row_index="perm",
                             out_init="normal", seed=1030))

# Many cooperative experts, several with the same rows per group (ties in the
# cost order), beside small and empty experts: more cooperative units than
# workgroups, so the snake deal runs over several rounds.
_MANY = (130, 256, 200, 130, 64, 90, 300, 256, 129, 0, 180, 64, 128, 257, 200, 40,
         130, 75, 5, 256, 0, 200, 99, 64, 31, 512, 130, 1, 140, 256)
SMALL_MANY_N = _reg(Workload("small_many_n", batch=600, M=sum(_MANY), K=256, N=512,
                             E=len(_MANY), fp8="e4m3fn", groups=_MANY, group_list_type=1,
                             exp_range=(-4, 4), row_index="perm", seed=1036))
SMALL_MANY_T = _reg(Workload("small_many_t", batch=600, M=sum(_MANY), K=512, N=320,
                             E=len(_MANY), fp8="e5m2", transpose_x2=True, groups=_MANY,
                             group_list_type=0, exp_range=(-4, 4), row_index="perm",
                             out_init="normal", seed=1037))

# [N, K] cooperative units with K = 128: two 64-K steps, too few for the
# four-step scale windows (per-step scale loads), in a 256-row group (300
# rows: two groups, the second short) and a 128-row group (70 rows).
SMALL_COOP_T_K128 = _reg(Workload("small_coop_t_k128", batch=120, M=370, K=128, N=352, E=3,
                                  fp8="e5m2", transpose_x2=True, groups=(300, 0, 70),
                                  group_list_type=1, exp_range=(-4, 4), row_index="perm",
                                  shared_rows=24, shared_weight=0.5, shared_offset=60,
                                  out_init="normal", seed=1038))

# Only experts below the cooperative size, few items and K long enough for a
# K split of four or more (32 K steps in either layout): the automatic split
# puts the four K ranges of an item into one block and adds them in LDS
# before the scatter.  Partial last column tile, a two-tile expert (40 rows),
# an empty expert, tokens routed twice to a row (topk 2).
SMALL_SPLIT_N = _reg(Workload("small_split_n", batch=21, topk=2, M=42, K=2048, N=320, E=4,
                              fp8="e4m3fn", groups=(10, 0, 29, 3), group_list_type=1,
                              exp_range=(-4, 4), logit="softmax", row_index="perm",
                              shared_rows=6, shared_weight=0.5, shared_offset=3,
                              out_init="normal", seed=1039))
SMALL_SPLIT_T = _reg(Workload("small_split_t", batch=31, topk=2, M=62, K=4096, N=352, E=3,
                              fp8="e5m2", transpose_x2=True, groups=(5, 17, 40),
                              group_list_type=0, exp_range=(-4, 4), row_index="perm",
                              out_init="normal", seed=1040))

# More units than workgroups with a short last round (two large experts and
# 150 small ones, eight column tiles, 16 K steps): the last round's units are
# cut into K halves so that they fill it.  A token of each batch row is
# routed twice (topk 2).
_TAIL = (150, 151) + tuple(1 + (7 * i) % 32 for i in range(150))
SMALL_TAIL_N = _reg(Workload("small_tail_n", batch=sum(_TAIL) // 2, topk=2, M=sum(_TAIL),
                             K=1024, N=1024, E=len(_TAIL), fp8="e4m3fn", groups=_TAIL,
                             group_list_type=1, exp_range=(-4, 4), logit="softmax",
                             row_index="perm", seed=1052))
SMALL_TAIL_T = _reg(Workload("small_tail_t", batch=sum(_TAIL) // 2, topk=2, M=sum(_TAIL),
                             K=2048, N=1024, E=len(_TAIL), fp8="e5m2", transpose_x2=True,
                             groups=_TAIL, group_list_type=0, exp_range=(-4, 4),
                             row_index="perm", out_init="normal", seed=1053))

# The small [N, K] cases again with K = 768 (six 128-K steps instead of five)
SMALL_T_K768 = _reg(replace(SMALL_T, name="small_t_k768", K=768, seed=1025))
SMALL_BIG_T_K768 = _reg(replace(SMALL_BIG_T, name="small_big_t_k768", K=768, seed=1026))
# ... K = 512 (exactly one four-step scale window per row) and K = 384 (rows too
# short for a window: per-step scale loads)
SMALL_T_K512 = _reg(replace(SMALL_T, name="small_t_k512", K=512, seed=1027))
SMALL_T_K384 = _reg(replace(SMALL_T, name="small_t_k384", K=384, seed=1028))

# Per-expert weight scales (a leading expert axis on scale; CANN V3 Atlas 350
# scale notes).
SMALL_N_PE = _reg(replace(SMALL_N, name="small_n_pe", scale_per_expert=True, seed=1031))
SMALL_BIG_T_PE = _reg(replace(SMALL_BIG_T, name="small_big_t_pe", scale_per_expert=True,
                              seed=1032))
C3_PE = _reg(replace(C3, name="c3_pe", scale_per_expert=True, seed=1033))
C5_PE = _reg(replace(C5, name="c5_pe", scale_per_expert=True, seed=1035))

# MXFP4 ([P3] Atlas 350 MX notes): E2M1 x1 and transposed x2, two elements per
# byte along K; K a multiple of 256 ...
SMALL_T_FP4 = _reg(replace(SMALL_T, name="small_t_fp4", fp8="e2m1", K=768, seed=1041))
SMALL_BIG_T_FP4 = _reg(replace(SMALL_BIG_T, name="small_big_t_fp4", fp8="e2m1", K=768,
                               seed=1042))
SMALL_T_FP4_K512 = _reg(replace(SMALL_T, name="small_t_fp4_k512", fp8="e2m1", K=512,
                                seed=1059))
SMALL_T_FP4_K1280 = _reg(replace(SMALL_T, name="small_t_fp4_k1280", fp8="e2m1", K=1280,
                                 seed=1051))
# ... K = 256 (one 256-K step per row: per-step scale loads) in cooperative
# units of both sizes and wave items; the K-split, short-last-round and
# many-cooperative-expert cases in MXFP4 (32, 16 and 4 steps of 256 K)
SMALL_BIG_T_FP4_K256 = _reg(replace(SMALL_BIG_T, name="small_big_t_fp4_k256", fp8="e2m1",
                                    K=256, seed=1054))
SMALL_SPLIT_T_FP4 = _reg(replace(SMALL_SPLIT_T, name="small_split_t_fp4", fp8="e2m1", K=8192,
                                 seed=1055))
SMALL_TAIL_T_FP4 = _reg(replace(SMALL_TAIL_T, name="small_tail_t_fp4", fp8="e2m1", K=4096,
                                seed=1056))
SMALL_MANY_T_FP4 = _reg(replace(SMALL_MANY_T, name="small_many_t_fp4", fp8="e2m1", K=1024,
                                seed=1057))
C2_FP4 = _reg(replace(C2, name="c2_fp4", fp8="e2m1", seed=1043))
C3_FP4T = _reg(replace(C3, name="c3_fp4t", fp8="e2m1", transpose_x2=True, seed=1044))
C5_FP4 = _reg(replace(C5, name="c5_fp4", fp8="e2m1", seed=1045))
# ... and with [K, N] x2 packed along N (N a multiple of 32); K = 640 is not a
# multiple of 256; small_split_n_fp4 has 32 K steps of 64 (block-split units).
SMALL_N_FP4 = _reg(replace(SMALL_N, name="small_n_fp4", fp8="e2m1", seed=1046))
SMALL_SPLIT_N_FP4 = _reg(replace(SMALL_SPLIT_N, name="small_split_n_fp4", fp8="e2m1",
                                 seed=1058))
SMALL_BIG_N_FP4 = _reg(replace(SMALL_BIG_N, name="small_big_n_fp4", fp8="e2m1", K=640,
                               seed=1047))
C1_FP4 = _reg(replace(C1, name="c1_fp4", fp8="e2m1", seed=1048))
C3_FP4 = _reg(replace(C3, name="c3_fp4", fp8="e2m1", seed=1049))
C4_FP4 = _reg(replace(C4, name="c4_fp4", fp8="e2m1", seed=1050))

# The A2/A3 W4A8 variant ([P3] A2/A3 notes: INT8 x1 with k 2048, INT4 x2 with
# n 7168, e up to 256): small ragged cases and the page's shape with a
# skewed routing of 4096 tokens (batch 512, topk 8).
# The largest expert count the library takes (1024), Zipf-routed: cooperative
# experts beside hundreds of one- to three-row-tile experts and empty ones,
# four group_list entries per work-list thread all in use.
SMALL_MAX_E_N = _reg(Workload("small_max_e_n", batch=600, M=3000, K=256, N=256, E=1024,
                              fp8="e4m3fn", groups=("zipf", 1.2), group_list_type=1,
                              exp_range=(-4, 4), row_index="perm", seed=1064))
SMALL_MAX_E_T = _reg(Workload("small_max_e_t", batch=600, M=3000, K=512, N=256, E=1024,
                              fp8="e5m2", transpose_x2=True, groups=("zipf", 1.1),
                              group_list_type=0, exp_range=(-4, 4), row_index="perm",
                              out_init="normal", seed=1065))
W4A8_SMALL = _reg(replace(SMALL_N, name="w4a8_small", fp8="w4a8", seed=1061))
W4A8_SMALL_BIG = _reg(replace(SMALL_BIG_N, name="w4a8_small_big", fp8="w4a8", K=640,
                              w4a8_offset=False, seed=1062))
W4A8_P3 = _reg(Workload("w4a8_p3", batch=512, topk=8, M=4096, K=2048, N=7168, E=256,
                        fp8="w4a8", groups=("zipf", 1.2), group_list_type=1, logit="softmax",
                        row_index="perm", seed=1063))

# Integer-valued variants: every partial sum is exactly representable in FP32,
# so any summation order must reproduce the oracle bit for bit.
for _base in (C1, C2, C3, C4, C5, SMALL_N, SMALL_T, SMALL_BIG_N, SMALL_BIG_T, SMALL_HUGE_N,
              SMALL_COOP_T_K128, SMALL_SPLIT_N, SMALL_SPLIT_T, SMALL_TAIL_N, SMALL_TAIL_T,
              SMALL_HUGE_T, SMALL_MANY_N, SMALL_MANY_T, SMALL_T_K768,
              SMALL_BIG_T_K768, SMALL_T_K512, SMALL_T_K384, SMALL_T_FP4_K1280, SMALL_T_FP4_K512,
              SMALL_N_PE,
              SMALL_BIG_T_PE, SMALL_T_FP4, SMALL_BIG_T_FP4, SMALL_BIG_T_FP4_K256,
              SMALL_SPLIT_T_FP4, SMALL_TAIL_T_FP4, SMALL_MANY_T_FP4, C3_FP4T, SMALL_N_FP4,
              SMALL_SPLIT_N_FP4,
              SMALL_BIG_N_FP4, C3_FP4, W4A8_SMALL, W4A8_SMALL_BIG, W4A8_P3, SMALL_MAX_E_N,
              SMALL_MAX_E_T):
    _reg(replace(_base, name=_base.name + "_exact", exact=True, seed=_base.seed + 100,
                 logit="exact" if _base.logit != "none" else "none"))


# --------------------------------------------------------------------------
# Drawing.
# --------------------------------------------------------------------------
def make_group_list(counts: np.ndarray, group_list_type: int) -> np.ndarray:
    """counts -> group_list in the requested format (0: prefix sums, 1: counts)."""
    counts = np.asarray(counts, np.int64)
    return np.cumsum(counts) if group_list_type == 0 else counts.copy()


def _counts(w: Workload) -> np.ndarray:
    if isinstance(w.groups, tuple) and w.groups and w.groups[0] == "zipf":
        return _zipf_counts(w.M, w.E, float(w.groups[1]), w.seed)
    if isinstance(w.groups, tuple):
        c = np.asarray(w.groups, np.int64)
        assert c.shape == (w.E,) and int(c.sum()) <= w.M
        return c
    # Uniform; a remainder goes one each to the leading experts.
    c = np.full(w.E, w.M // w.E, np.int64)
    c[: w.M % w.E] += 1
    return c


def _zipf_counts(M: int, E: int, s: float, seed: int) -> np.ndarray:
    """Skewed routing: a seeded permutation ranks the experts; the last E/16 of
    it are forced empty; the others get floor(M * r^-s / H) tokens by rank r,
    and the remainder goes one each to the lowest-id active experts."""
    rng = np.random.default_rng(seed + 7)
    perm = rng.permutation(E)
    n_empty = E // 16
    active = perm[: E - n_empty]
    ranks = np.arange(1, active.size + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    c = np.zeros(E, np.int64)
    c[active] = np.floor(M * p).astype(np.int64)
    rem = M - int(c.sum())
    for e in np.sort(active)[:rem]:
        c[e] += 1
    return c


def _fp8_from_normal(shape, dtype, gen, device, exact: bool) -> torch.Tensor:
    if exact:
        v = torch.randint(-2, 3, shape, generator=gen, device=device, dtype=torch.int32)
        return v.to(torch.float32).to(dtype)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


# E2M1 magnitudes by code 0..7 and the midpoints between them: a value goes to
# the nearest code (input drawing only; the operator never encodes).
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_from_normal(shape, gen, device, exact):
    """N(0,1) (or, exact: uniform over {0, +-1, +-2}) rounded to E2M1 codes and
    packed two per byte along the last axis (element 2j in the low nibble)."""
    if exact:
        v = torch.randint(-2, 3, shape, generator=gen, device=device).to(torch.float32)
    else:
        v = torch.randn(shape, generator=gen, device=device)
    mid = torch.tensor(_E2M1_MID, device=device)
    code = torch.bucketize(v.abs(), mid).to(torch.uint8)
    code = code | ((v < 0) & (code > 0)).to(torch.uint8) << 3
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous()          # uint8; the caller views it as float4_e2m1fn_x2


def make_inputs(w: Workload, device: Union[str, torch.device] = "cpu") -> dict:
    """Draw one invocation's inputs.  Returns a dict keyed by argument name.

    x1 / x2 are float8 tensors; scale / pertoken_scale are uint8 E8M0 codes;
    shared_input is bfloat16; out is the FP32 initial value.
    """
    device = torch.device(device)
    rng = np.random.default_rng(w.seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = FP8_DTYPES[w.fp8]
    M, K, N, E, B = w.M, w.K, w.N, w.E, w.batch
    KB = (K + 63) // 64

    x2_shape = (N, K) if w.transpose_x2 else (K, N)
    if w.fp8 == "e2m1":
        x1 = _e2m1_from_normal((M, K), gen, device, w.exact).view(dt)
        x2 = torch.empty((E,) + x2_shape[:-1] + (x2_shape[-1] // 2,), dtype=torch.uint8,
                         device=device)
        for e in range(E):
            x2[e] = _e2m1_from_normal(x2_shape, gen, device, w.exact)
        x2 = x2.view(dt)
    else:
        x1 = _fp8_from_normal((M, K), dt, gen, device, w.exact)
        x2 = torch.empty((E,) + x2_shape, dtype=dt, device=device)
        for e in range(E):  # per expert, so large configs never hold an FP32 copy
            x2[e] = _fp8_from_normal(x2_shape, dt, gen, device, w.exact)

    lo, hi = (0, 1) if w.exact else w.exp_range
    pts = (127 + rng.integers(lo, hi + 1, size=(M, KB, 2))).astype(np.uint8)
    sc_shape = (N, KB, 2) if w.transpose_x2 else (KB, N, 2)
    if w.scale_per_expert:
        sc_shape = (E,) + sc_shape
    sc = (127 + rng.integers(lo, hi + 1, size=sc_shape)).astype(np.uint8)

    d = dict(x1=x1, x2=x2, scale=_t(sc, device), pertoken_scale=_t(pts, device),
             fp8_kind=w.fp8_kind,
             transpose_x2=bool(w.transpose_x2))
    d.update(_routing_inputs(w, rng, device))
    return d


def _t(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _routing_inputs(w: Workload, rng, device) -> dict:
    """group_list, row_index, logit, shared input and out's initial value
    (drawn after the operands, in this order)."""
    M, N, B = w.M, w.N, w.batch
    counts = _counts(w)
    group_list = make_group_list(counts, w.group_list_type)

    if w.row_index == "mod":
        row_index = np.arange(M, dtype=np.int64) % B
    else:
        reps = -(-M // B)
        row_index = rng.permutation(np.tile(np.arange(B, dtype=np.int64), reps))[:M]

    if w.logit == "none":
        logit = None
    elif w.logit == "exact":
        logit = rng.choice(np.array([1.0, 0.5, 0.25], np.float32), size=M)
    elif w.logit == "softmax":
        # softmax over each output row's tokens (its top-k routing weights)
        s = rng.standard_normal(M)
        ex = np.exp(s - s.max())
        den = np.bincount(row_index, weights=ex, minlength=B)
        logit = (ex / den[row_index]).astype(np.float32)
    else:
        logit = rng.random(M, dtype=np.float32)

    R = w.R
    if R > 0:
        if w.exact:
            shared = torch.from_numpy(rng.integers(-4, 5, size=(R, N)).astype(np.float32))
        else:
            shared = torch.from_numpy(rng.standard_normal((R, N), dtype=np.float32))
        shared = shared.to(torch.bfloat16).to(device)
    else:
        shared = None

    if w.out_init == "normal":
        if w.exact:
            init = rng.integers(-4, 5, size=(B, N)).astype(np.float32)
        else:
            init = rng.standard_normal((B, N), dtype=np.float32)
    else:
        init = np.zeros((B, N), np.float32)

    t = lambda a: _t(a, device)
    return dict(
        group_list=t(group_list), group_list_type=w.group_list_type,
        logit=None if logit is None else t(logit), row_index=t(row_index),
        shared_input=shared, shared_input_weight=float(w.shared_weight),
        shared_input_offset=int(w.shared_offset) if R > 0 else 0,
        out=t(init),
    )


def make_w4a8_inputs(w: Workload, device="cpu") -> dict:
    """Inputs of the W4A8 variant: x1 int8 [M, K] (uniform over the int8
    range; exact variant: [-8, 7]); x2 uint8 [E, K, N/2] (uniform bytes, i.e.
    uniform signed 4-bit pairs); scale float32 [E, 1, N] uniform in
    [0.001, 0.01] (exact: 2^-4); offset [E, 1, N] uniform in [-0.01, 0.01]
    (exact: 0, +-2^-5) or None; pertoken_scale float32 [M] uniform in
    [0.5, 2] (exact: 1 or 0.5); routing, shared input and out as make_inputs."""
    assert w.fp8 == "w4a8"
    device = torch.device(device)
    rng = np.random.default_rng(w.seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    M, K, N, E = w.M, w.K, w.N, w.E
    lo, hi = (-8, 8) if w.exact else (-128, 128)
    x1 = torch.randint(lo, hi, (M, K), generator=gen, device=device, dtype=torch.int8)
    x2 = torch.empty((E, K, N // 2), dtype=torch.uint8, device=device)
    for e in range(E):
        x2[e] = torch.randint(0, 256, (K, N // 2), generator=gen, device=device,
                              dtype=torch.uint8)
    if w.exact:
        sc = np.full((E, 1, N), 2.0 ** -4, np.float32)
        of = rng.choice(np.array([0.0, 2.0 ** -5, -2.0 ** -5], np.float32), size=(E, 1, N))
        pts = rng.choice(np.array([1.0, 0.5], np.float32), size=M)
    else:
        sc = rng.uniform(0.001, 0.01, size=(E, 1, N)).astype(np.float32)
        of = rng.uniform(-0.01, 0.01, size=(E, 1, N)).astype(np.float32)
        pts = rng.uniform(0.5, 2.0, size=M).astype(np.float32)
    d = dict(x1=x1, x2=x2, scale=_t(sc, device),
             offset=_t(of, device) if w.w4a8_offset else None, pertoken_scale=_t(pts, device))
    d.update(_routing_inputs(w, rng, device))
    return d


def as_numpy(inputs: dict) -> dict:
    """Host numpy copies of an input dict in the oracle's raw-code form."""
    def u8(x):
        return x.detach().contiguous().view(torch.uint8).cpu().numpy()

    d = dict(inputs)
    d["x1"] = u8(inputs["x1"])
    d["x2"] = u8(inputs["x2"])
    d["scale"] = u8(inputs["scale"])
    d["pertoken_scale"] = u8(inputs["pertoken_scale"])
    d["group_list"] = inputs["group_list"].cpu().numpy()
    d["row_index"] = inputs["row_index"].cpu().numpy()
    d["logit"] = None if inputs["logit"] is None else inputs["logit"].cpu().numpy()
    sh = inputs["shared_input"]
    d["shared_input"] = None if sh is None else sh.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    d["out_init"] = inputs["out"].cpu().numpy()
    del d["out"]
    return d


# --------------------------------------------------------------------------
# The upstream step of the MoE FFN (gate||up grouped matmul, SwiGLU, MX
# quantisation; gfr_gemm1_swiglu_quant).  Shapes: the LLaDA2.0-mini grouped
# GEMM page's model dimensions (H 2048, I 512, E 256) and its operator test's
# token counts [0, 1, 2, 4, 8, 16, 32, 0]; the upstream steps of c2 and c3
# (H = their N, I = their K: the step that produces their x1); small ragged
# cases that span several tiles and every item class.  Drawing as for the
# finalize-routing inputs: FP8 data from N(0,1), E8M0 exponents uniform.
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Gemm1Workload:
    name: str
    M: int
    H: int
    I: int
    E: int
    fp8: str = "e4m3fn"                    # xin / w13
    out_fp8: str = "e4m3fn"                # x1 codes
    transpose_w13: bool = False
    group_list_type: int = 1
    groups: Union[str, Tuple] = "uniform"
    exp_range: Tuple[int, int] = (-3, 3)
    scale_per_expert: bool = False
    zero_rows: int = 0                     # leading xin rows set to zero (all-zero MX blocks)
    seed: int = 0

    def counts(self) -> np.ndarray:
        return _counts(self)

    def flops(self) -> int:
        """2 * routed tokens * H * 2I."""
        return 2 * int(self.counts().sum()) * self.H * 2 * self.I

    def algorithmic_bytes(self) -> int:
        """w13 of non-empty experts, xin, both scale tensors, group_list, and the
        written x1 codes and scales of the routed rows."""
        c = self.counts()
        active = int((c > 0).sum())
        M_r = int(c.sum())
        H, N2 = self.H, 2 * self.I
        kb32 = 2 * ((H + 63) // 64)
        b = active * H * N2 + M_r * H + M_r * kb32
        b += N2 * kb32 * (active if self.scale_per_expert else 1) + 8 * self.E
        b += M_r * self.I + M_r * (self.I // 32)
        return b


GEMM1_WORKLOADS: Dict[str, Gemm1Workload] = {}


def _reg1(w: Gemm1Workload) -> Gemm1Workload:
    GEMM1_WORKLOADS[w.name] = w
    return w


_reg1(Gemm1Workload("g1_small", M=300, H=1024, I=384, E=7, groups=(0, 37, 1, 120, 0, 95, 47),
                    exp_range=(-5, 5), zero_rows=2, seed=2001))
_reg1(Gemm1Workload("g1_small_t", M=200, H=640, I=320, E=5, fp8="e5m2", transpose_w13=True,
                    groups=(33, 0, 64, 100, 3), group_list_type=0, seed=2002))
# large experts: 256-row cooperative groups (300, 141), a 128-row group (70),
# a wave item (5)
_reg1(Gemm1Workload("g1_big", M=516, H=768, I=192, E=5, out_fp8="e5m2",
                    groups=(0, 300, 70, 5, 141), seed=2003))
_reg1(Gemm1Workload("g1_big_t_pe", M=516, H=640, I=256, E=4, fp8="e5m2", out_fp8="e5m2",
                    transpose_w13=True, groups=(141, 5, 300, 70), group_list_type=0,
                    scale_per_expert=True, seed=2004))
_reg1(Gemm1Workload("g1_llada_op", M=63, H=2048, I=512, E=8,
                    groups=(0, 1, 2, 4, 8, 16, 32, 0), seed=2005))
_reg1(Gemm1Workload("g1_llada", M=4096, H=2048, I=512, E=256, groups=("zipf", 1.2),
                    seed=2006))
_reg1(Gemm1Workload("g1_c2t", M=256, H=4096, I=6144, E=16, fp8="e5m2", transpose_w13=True,
                    exp_range=(-4, 4), seed=2007))
_reg1(Gemm1Workload("g1_c3", M=768, H=4096, I=8192, E=32, group_list_type=0, seed=2008))


def make_gemm1_inputs(w: Gemm1Workload, device="cpu") -> dict:
    """Draw one upstream-step invocation's inputs (keys: the binding's
    argument names, plus out_dtype)."""
    device = torch.device(device)
    rng = np.random.default_rng(w.seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = FP8_DTYPES[w.fp8]
    M, H, N2, E = w.M, w.H, 2 * w.I, w.E
    KB = (H + 63) // 64
    xin = _fp8_from_normal((M, H), dt, gen, device, False)
    if w.zero_rows:
        xin[: w.zero_rows] = torch.zeros((w.zero_rows, H), dtype=torch.float32,
                                         device=device).to(dt)
    shape = (N2, H) if w.transpose_w13 else (H, N2)
    w13 = torch.empty((E,) + shape, dtype=dt, device=device)
    for e in range(E):
        w13[e] = _fp8_from_normal(shape, dt, gen, device, False)
    lo, hi = w.exp_range
    xs = (127 + rng.integers(lo, hi + 1, size=(M, KB, 2))).astype(np.uint8)
    sc_shape = (N2, KB, 2) if w.transpose_w13 else (KB, N2, 2)
    if w.scale_per_expert:
        sc_shape = (E,) + sc_shape
    sc = (127 + rng.integers(lo, hi + 1, size=sc_shape)).astype(np.uint8)
    gl = make_group_list(_counts(w), w.group_list_type)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(xin=xin, w13=w13, scale=t(sc), xin_scale=t(xs), group_list=t(gl),
                group_list_type=w.group_list_type, transpose_w13=bool(w.transpose_w13),
                out_dtype=FP8_DTYPES[w.out_fp8])
