/*
 * gfr.h — C ABI of the MI355X (gfx950) fused MXFP8 grouped-matmul +
 * finalize-routing library (libgfr.so).
 *
 * The operation is the MoE "grouped matmul, then finalize routing" combine
 * defined on two pages:
 *   [P1] "基于 PyPTO 的 MoE 融合算子实践：grouped_matmul_finalize_routing 的
 *        MXFP8 实现与精度验证" — §2.1 formula and expanded form, §2.2 the four
 *        stages, §3.1 input/output table, §4.2 constraints, §4.3 group_list
 *        formats, §5.3 kernel stages, §5.4 host wrapper (out is in/out);
 *   [P3] CANN "aclnnGroupedMatmulFinalizeRoutingV3" — formulas 1-4, Atlas 350
 *        MX parameter notes (shapes, empty-tensor rules), two-phase
 *        workspace-size/execute call, determinism note.
 *
 * For every expert e, with token rows [start_e, end_e) taken from group_list:
 *
 *   out[row_index[t], n] += logit[t] * sum_k dq(x1[t, k]) * dq(x2[e, k, n])
 *   out[off + r, n]      += shared_input_weight * shared_input[r, n]
 *
 * where dq(v) = FP8 value * 2^(E8M0 - 127) with one E8M0 scale per 32
 * consecutive K elements: the scale tensors have a trailing (ceil(K/64), 2)
 * pair of axes, and element j of the pair for 64-block b covers
 * k in [64b + 32j, 64b + 32j + 32).
 *
 * Two layers of entry points:
 *  - the tensor-descriptor calls (gmm_finalize_routing, gmm_finalize_routing_ex,
 *    gfr_workspace_size, gfr_w4a8_finalize_routing, gfr_gemm1_swiglu_quant)
 *    take every tensor as a gfr_tensor and derive all sizes from the shapes;
 *    each descriptor's dtype, rank and shape is checked against the others on
 *    the host before anything is enqueued (GFR_ERR_BAD_DTYPE / _BAD_RANK /
 *    _BAD_SHAPE), as [P3]'s first phase validates the parameters;
 *  - the raw calls (*_raw) take device pointers plus the sizes M, K, N, E,
 *    batch, R and trust them: each buffer must hold at least the bytes its
 *    documented shape implies at those sizes, or the kernels read or write
 *    past it.  The descriptor calls check exactly that and then call them.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major storage
 *    owned by the caller; the library never allocates, frees or retains them.
 *    Descriptors themselves are read on the host during the call only.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is the
 *    null stream).  Nothing is synchronised and no device memory is read on the
 *    host: group_list is consumed on the device.
 *  - Arguments are validated on the host before anything is launched; on a
 *    nonzero return nothing was enqueued and `out` is untouched.
 *  - Data errors only visible on the device (see GFR_DEV_*) never cause an
 *    out-of-bounds access: the offending work is skipped and, if a status word
 *    is supplied through gfr_options, a bit is OR-ed into it.
 *  - In the default mode `out` is updated with FP32 atomics, so the bitwise
 *    result may vary between runs ([P3] determinism note); set
 *    gfr_options.deterministic for a fixed summation order.
 */
#ifndef GFR_H
#define GFR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum gfr_status {
    GFR_OK = 0,
    GFR_ERR_NULL_ARG = 1,        /* a required pointer is NULL */
    GFR_ERR_BAD_SHAPE = 2,       /* negative or inconsistent sizes */
    GFR_ERR_BAD_OFFSET = 3,      /* shared_input_offset < 0 or off + rows > batch */
    GFR_ERR_UNSUPPORTED = 4,     /* valid per the pages but not implemented here */
    GFR_ERR_BAD_ALIGNMENT = 5,   /* x1 / x2 / scale / shared_input not 16-byte aligned,
                                    out not 4-byte (deterministic mode: 16-byte) aligned,
                                    workspace not 256-byte aligned */
    GFR_ERR_WORKSPACE_TOO_SMALL = 6,
    GFR_ERR_BAD_ARG = 7,         /* unknown enum value (fp8_kind, group_list_type) */
    GFR_ERR_HIP = 8,             /* a HIP runtime call failed */
    GFR_ERR_BAD_DTYPE = 9,       /* a descriptor's dtype is not one its argument takes,
                                    or x1 / x2 do not match fp8_kind */
    GFR_ERR_BAD_RANK = 10,       /* a descriptor's ndim is not its argument's rank */
    GFR_ERR_SCRATCH_TOO_SMALL = 11  /* the allocation-free call needs more than
                                       GFR_STATIC_SCRATCH_BYTES of scratch */
};

/* Element types of a gfr_tensor.  Packed types hold two 4-bit elements per
 * byte along the last axis (element 2j in the low nibble of byte j); their
 * descriptor's last extent counts bytes. */
enum gfr_dtype {
    GFR_DT_FP8_E4M3FN = 0,
    GFR_DT_FP8_E5M2 = 1,
    GFR_DT_FP4_E2M1X2 = 2,   /* MXFP4 elements, packed */
    GFR_DT_E8M0 = 3,         /* E8M0 scale codes, one byte each */
    GFR_DT_U8 = 4,           /* raw bytes: accepted wherever E8M0 codes are */
    GFR_DT_BF16 = 5,
    GFR_DT_F32 = 6,
    GFR_DT_I64 = 7,
    GFR_DT_I32 = 8,
    GFR_DT_I8 = 9,
    GFR_DT_INT4X2 = 10       /* signed 4-bit (two's complement) elements, packed */
};

/* A tensor argument: device pointer to contiguous row-major storage of
 * shape[0] x ... x shape[ndim - 1] elements of dtype (1 <= ndim <= 4; the
 * unused extents are ignored).  data may be NULL only when the tensor holds
 * no element. */
typedef struct gfr_tensor {
    void *data;
    int32_t dtype;
    int32_t ndim;
    int64_t shape[4];
} gfr_tensor;

/* Element formats of x1 and x2 ([P1] §3.1: FP8 E4M3FN or E5M2; [P3] Atlas
 * 350 MX notes: the MXFP4 variant, FP4 E2M1 elements stored two per byte
 * along the contiguous axis, element 2j in the low nibble of byte j). */
enum gfr_fp8_kind { GFR_FP8_E4M3FN = 0, GFR_FP8_E5M2 = 1, GFR_FP4_E2M1 = 2 };

/* group_list formats ([P1] §4.3): 0 = prefix sums, expert i owns
 * [group_list[i-1], group_list[i]) with group_list[-1] = 0; 1 = counts, expert
 * i owns [sum(group_list[:i]), sum(group_list[:i]) + group_list[i]). */
enum gfr_group_list_type { GFR_GROUP_LIST_CUMSUM = 0, GFR_GROUP_LIST_COUNT = 1 };

/* Bits OR-ed into gfr_options.status_dev by the device. */
#define GFR_DEV_BAD_GROUP_LIST 0x1 /* negative count, decreasing prefix, or total > M:
                                      ranges are clamped to [0, M) */
#define GFR_DEV_BAD_ROW_INDEX 0x2  /* row_index outside [0, batch): token skipped */

/* Limits of this implementation. */
#define GFR_MAX_EXPERTS 1024       /* [P3] Atlas 350 notes: e <= 1024 */
/* Static device scratch per GPU of gmm_finalize_routing_det_noalloc. */
#define GFR_STATIC_SCRATCH_BYTES (64u << 20)

typedef struct gfr_options {
    /* 0: scatter-add with FP32 atomics (default).  1: deterministic — the
     * matmul writes logit-weighted rows to the workspace, then each output row
     * is reduced in a fixed order: initial value, tokens in ascending t, then
     * the shared term.  Needs gfr_workspace_size() bytes of workspace
     * (256-byte aligned) and a 16-byte aligned out (GFR_ERR_BAD_ALIGNMENT). */
    int deterministic;
    /* Device workspace (may be NULL when 0 bytes are required). */
    void *workspace;
    size_t workspace_bytes;
    /* Optional device int32 word; GFR_DEV_* bits are OR-ed into it. */
    int32_t *status_dev;
    /* K-split factor for the atomic mode; 0 = chosen on the device from the
     * routed work size.  Ignored (1) in deterministic mode. */
    int split_k;
    /* 0: scale is shared by all experts (3-D, [P1] §3.1).  1: scale carries a
     * leading expert axis ([P3] Atlas 350 scale notes: (e, n, ceil(k/64), 2)
     * when transpose_x2, by the same reading (e, ceil(k/64), n, 2)
     * otherwise); expert e's rows use slice e.  The descriptor calls take
     * this from the rank of scale (4-D: per expert); a nonzero value there
     * requires a 4-D scale (GFR_ERR_BAD_RANK). */
    int scale_per_expert;
} gfr_options;

/* ======================================================================== *
 * Tensor-descriptor calls                                                  *
 * ======================================================================== */

/*
 * gmm_finalize_routing — the fused operator ([P1] §2.1–2.2; [P3] formulas),
 * in [P1]'s parameter order.  Sizes come from the descriptors (elements):
 *
 *  x1              [M, K] of dtype FP8_E4M3FN / FP8_E5M2 / FP4_E2M1X2 (then
 *                  [M, K/2] bytes), routed tokens sorted by expert.
 *  x2              [E, K, N], or [E, N, K] when transpose_x2 != 0, of x1's
 *                  dtype (FP4_E2M1X2: the last extent halved, packed along it).
 *  scale           E8M0 (or U8) [ceil(K/64), N, 2], or [N, ceil(K/64), 2]
 *                  when transpose_x2 != 0; shared by all experts ([P1] §3.1),
 *                  or 4-D with a leading E extent (per expert, [P3]).
 *  pertoken_scale  E8M0 (or U8) [M, ceil(K/64), 2].
 *  group_list      I64 [E], format per group_list_type.
 *  logit           F32 [M], or NULL (descriptor or data) for weight 1 ([P1]
 *                  §5.1 has_logit).
 *  row_index       I64 or I32 [M]: destination row of each token, in
 *                  [0, batch) ([P1] §3.1 int64; §5.4 passes int32).
 *  shared_input    BF16 [R, N], or NULL (no shared expert).
 *  shared_input_weight, shared_input_offset: shared rows land in
 *                  out[offset, offset + R); offset >= 0 and offset + R <= batch
 *                  ([P3] Atlas 350 notes).
 *  out             F32 [batch, N]; read as the initial value and updated in
 *                  place ([P1] §3.1, §5.4).
 *  transpose_x2    0 or 1 (the weight-scale layout follows it, [P3]).
 *  fp8_kind        gfr_fp8_kind; must name x1's and x2's dtype.
 *  stream          hipStream_t.
 *
 * M = 0 leaves only the shared term; N = 0 or batch = 0 is a no-op ([P3]
 * empty-tensor notes).  Errors: GFR_ERR_NULL_ARG (a required descriptor, or
 * the data of a non-empty tensor, is NULL), GFR_ERR_BAD_DTYPE,
 * GFR_ERR_BAD_RANK, GFR_ERR_BAD_SHAPE (an extent disagrees with the sizes the
 * others fix), GFR_ERR_BAD_OFFSET, GFR_ERR_BAD_ARG, GFR_ERR_UNSUPPORTED and
 * GFR_ERR_BAD_ALIGNMENT as for gmm_finalize_routing_raw_ex, GFR_ERR_HIP.
 * Returns a gfr_status.
 */
int gmm_finalize_routing(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                         const gfr_tensor *pertoken_scale, const gfr_tensor *group_list,
                         int group_list_type, const gfr_tensor *logit,
                         const gfr_tensor *row_index, const gfr_tensor *shared_input,
                         float shared_input_weight, int64_t shared_input_offset,
                         const gfr_tensor *out, int transpose_x2, int fp8_kind, void *stream);

/* gmm_finalize_routing with options (NULL = atomic mode, no workspace, no
 * status word, K split chosen on the device).  GFR_ERR_WORKSPACE_TOO_SMALL
 * when the deterministic mode is asked for without gfr_workspace_size()
 * bytes of workspace. */
int gmm_finalize_routing_ex(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                            const gfr_tensor *pertoken_scale, const gfr_tensor *group_list,
                            int group_list_type, const gfr_tensor *logit,
                            const gfr_tensor *row_index, const gfr_tensor *shared_input,
                            float shared_input_weight, int64_t shared_input_offset,
                            const gfr_tensor *out, int transpose_x2, int fp8_kind, void *stream,
                            const gfr_options *opts);

/* The first phase of [P3]'s two-phase call ("GetWorkspaceSize", then
 * execute): validates the same arguments as gmm_finalize_routing_ex (data
 * pointers are not dereferenced; opts' workspace fields are ignored) and
 * stores the workspace bytes the call needs in *bytes (0 in atomic mode).
 * Pure host work.  Returns a gfr_status. */
int gfr_workspace_size(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                       const gfr_tensor *pertoken_scale, const gfr_tensor *group_list,
                       int group_list_type, const gfr_tensor *logit,
                       const gfr_tensor *row_index, const gfr_tensor *shared_input,
                       float shared_input_weight, int64_t shared_input_offset,
                       const gfr_tensor *out, int transpose_x2, int fp8_kind,
                       const gfr_options *opts, size_t *bytes);

/*
 * gfr_gemm1_swiglu_quant — the upstream step of the MoE FFN whose output is
 * this library's x1 / pertoken_scale: the gate||up grouped matmul and SwiGLU
 * of "LLaDA2.0-mini MoE 融合算子实战：基于 PyPTO 的 Grouped GEMM 单内核实现"
 * ([P2] §3.1 w13 layout, §3.2 two-stage expert FFN, §3.3 SwiGLU), with MXFP8
 * operands as in [P1], followed by MX block quantisation.  For every expert e
 * and token t in its group_list range:
 *
 *   gate_up[t, j] = sum_k dq(xin[t, k]) * dq(w13[e, k, j]),  j < 2I  (FP32)
 *   sw[t, i]      = SiLU(gate_up[t, i]) * gate_up[t, I + i],
 *                   SiLU(g) = g / (1 + exp(-g))   (FP32; first I columns gate)
 *
 * and each 32-element block i in [32b, 32b + 32) of row t is encoded as
 *   X = floor(log2(max |sw|)) - emax   (emax 8 for E4M3FN, 15 for E5M2;
 *       -127 for an all-zero block; clamped to >= -127),
 *   x1_out[t, i] = FP8 code nearest to sw[t, i] / 2^X (ties to even,
 *       saturating at the largest finite value),
 *   x1_scale_out[t, b / 2, b % 2] = X + 127 (E8M0).
 * The pages define only the dequantisation of MX data; this encoding is the
 * OCP Microscaling rule, and dequantising the output reproduces sw within
 * half a code step (values that scale past the largest finite code saturate).
 *
 *  xin             FP8 [M, H] (dtype FP8_E4M3FN or FP8_E5M2), tokens sorted
 *                  by expert.
 *  w13             [E, H, 2I], or [E, 2I, H] when transpose_w13 != 0, of
 *                  xin's dtype.
 *  scale           E8M0 (or U8) [ceil(H/64), 2I, 2], or [2I, ceil(H/64), 2]
 *                  when transpose_w13; 4-D with a leading E extent for
 *                  per-expert scales.
 *  xin_scale       E8M0 (or U8) [M, ceil(H/64), 2].
 *  group_list      I64 [E], format per group_list_type.
 *  x1_out          [M, I], dtype FP8_E4M3FN or FP8_E5M2: the output codes
 *                  (written; rows of tokens in no expert's range are left
 *                  untouched).
 *  x1_scale_out    E8M0 (or U8) [M, I/64, 2] (written, same rows).
 *  transpose_w13   0 or 1.
 *  stream          hipStream_t.
 *  opts            may be NULL; only status_dev is used (the output is
 *                  written once per element: no atomics, no K split, bitwise
 *                  repeatable); a nonzero scale_per_expert requires a 4-D scale.
 *
 * M = 0 or I = 0 is a no-op.  Limits (GFR_ERR_UNSUPPORTED): H % 128 != 0,
 * I % 64 != 0, E outside [1, 1024], 2I * H >= 2^31.  xin, w13 and scale must
 * be 16-byte aligned.  Returns a gfr_status.
 */
int gfr_gemm1_swiglu_quant(const gfr_tensor *xin, const gfr_tensor *w13, const gfr_tensor *scale,
                           const gfr_tensor *xin_scale, const gfr_tensor *group_list,
                           int group_list_type, const gfr_tensor *x1_out,
                           const gfr_tensor *x1_scale_out, int transpose_w13, void *stream,
                           const gfr_options *opts);

/*
 * gfr_w4a8_finalize_routing — the A2/A3 W4A8 variant of the operator ([P3]
 * A2/A3 parameter notes: INT8 x1, INT4 x2, INT64-typed fused scale (e, 1, n),
 * FP32 offset (e, 1, n), FP32 perTokenScale (m); pseudo-quant notes: scale is
 * the offline fusion of per-channel and per-group scales, offset the
 * asymmetric term antiquantOffset * scale; formula 1 for the product).  For
 * every expert e and token t in its group_list range:
 *
 *   y[t, n] = pertoken_scale[t] * ( scale[e, n] * sum_k x1[t, k] * w[e, k, n]
 *                                   + offset[e, n] * sum_k x1[t, k] )
 *   out[row_index[t], n] += logit[t] * y[t, n]
 *   out[off + r, n]      += shared_input_weight * shared_input[r, n]
 *
 *  x1              I8 [M, K].
 *  x2              INT4X2 (or U8) [E, K, N/2] bytes: signed 4-bit weights,
 *                  two per byte along n, element 2j in the low nibble (the
 *                  pages' (e, k, n/8) INT32 packing read as little-endian
 *                  nibbles).
 *  scale           F32 [E, 1, N]: the fused per-channel scale (the pages
 *                  type it INT64; its value is taken here as FP32).
 *  offset          F32 [E, 1, N], or NULL for symmetric weights.
 *  pertoken_scale  F32 [M].
 *  group_list, group_list_type, logit, row_index, shared_input (BF16 [R, N]),
 *  shared_input_weight, shared_input_offset, out (F32 [batch, N], in/out),
 *  stream: as gmm_finalize_routing.
 *  opts            as gmm_finalize_routing_ex (deterministic mode, workspace
 *                  from gfr_workspace_size_raw, status word, K split);
 *                  scale_per_expert must be 0 (the scale always has an expert
 *                  axis).
 *
 * The pages' bias input (8 * w * scale summed over k) restores a term that
 * their kernel's INT4 decomposition of the activations drops; the integer
 * products here are exact, so it has no counterpart.  Integer sums are exact;
 * the scaling is FP32.
 *
 * Limits (GFR_ERR_UNSUPPORTED): K % 128 != 0, K > 65536, N % 32 != 0, E
 * outside [1, 1024], M or batch >= 2^31.  x1 and x2 must be 16-byte aligned,
 * scale and offset 8-byte aligned.  Returns a gfr_status.
 */
int gfr_w4a8_finalize_routing(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                              const gfr_tensor *offset, const gfr_tensor *pertoken_scale,
                              const gfr_tensor *group_list, int group_list_type,
                              const gfr_tensor *logit, const gfr_tensor *row_index,
                              const gfr_tensor *shared_input, float shared_input_weight,
                              int64_t shared_input_offset, const gfr_tensor *out, void *stream,
                              const gfr_options *opts);

/*
 * gmm_finalize_routing_det_noalloc — gmm_finalize_routing_ex in deterministic
 * mode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Its
 * workspace (the weighted rows W [M, N] float32 and the CSR of row_index,
 * gfr_workspace_size bytes) is a static device array of
 * GFR_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on until
 * the process ends; the call allocates and frees nothing.
 *
 *  Arguments as gmm_finalize_routing; status_dev as gfr_options.status_dev
 *  (may be NULL).  The result is the deterministic mode's: bitwise equal to
 *  gmm_finalize_routing_ex with opts.deterministic = 1.
 *
 * GFR_ERR_SCRATCH_TOO_SMALL when the call needs more than
 * GFR_STATIC_SCRATCH_BYTES (4 * M * N bytes plus 4 * (3 * batch + 2 * M) for the
 * CSR, each rounded up to 256: about M * N <= 16.7 M), with nothing enqueued;
 * the other errors as gmm_finalize_routing_ex.  Every call on one GPU uses that
 * GPU's one array and leaves its contents behind (what must start at zero is
 * cleared by each call on its stream): calls that overlap in time on one GPU
 * race, so the caller orders them (one stream, or events between streams).
 */
int gmm_finalize_routing_det_noalloc(const gfr_tensor *x1, const gfr_tensor *x2,
                                     const gfr_tensor *scale, const gfr_tensor *pertoken_scale,
                                     const gfr_tensor *group_list, int group_list_type,
                                     const gfr_tensor *logit, const gfr_tensor *row_index,
                                     const gfr_tensor *shared_input, float shared_input_weight,
                                     int64_t shared_input_offset, const gfr_tensor *out,
                                     int transpose_x2, int fp8_kind, void *stream,
                                     int32_t *status_dev);

/* ======================================================================== *
 * Raw calls: device pointers plus sizes, semantics as the descriptor calls *
 * above.  Nothing ties the sizes to the buffers: every buffer must hold at  *
 * least the bytes of its shape at the given M, K, N, E, batch and R (x1 and *
 * x2 packed for FP4 as above, row_index int64); a smaller buffer is read or *
 * written out of bounds.                                                    *
 * ======================================================================== */

/* gmm_finalize_routing on pointers and sizes.  M, K, N count elements (FP4:
 * x1 is [M, K/2] bytes, x2 [E, N, K/2] or [E, K, N/2] bytes).
 *
 * Implementation limits (GFR_ERR_UNSUPPORTED): K % 128 != 0, N % 16 != 0,
 * E outside [1, 1024], M or batch >= 2^31; for GFR_FP4_E2M1 also K % 256 != 0
 * with transpose_x2 == 1, N % 32 != 0 with transpose_x2 == 0.  x1, x2 and
 * scale must be 16-byte aligned (GFR_ERR_BAD_ALIGNMENT).  Atomic mode needs no
 * workspace.  Returns a gfr_status. */
int gmm_finalize_routing_raw(const void *x1, const void *x2, const uint8_t *scale,
                             const uint8_t *pertoken_scale, const int64_t *group_list,
                             int group_list_type, const float *logit,
                             const int64_t *row_index, const uint16_t *shared_input,
                             float shared_input_weight, int64_t shared_input_offset,
                             float *out, int transpose_x2, int fp8_kind,
                             int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                             int64_t shared_rows, void *stream);

/* gmm_finalize_routing_raw with options (as gmm_finalize_routing_ex). */
int gmm_finalize_routing_raw_ex(const void *x1, const void *x2, const uint8_t *scale,
                                const uint8_t *pertoken_scale, const int64_t *group_list,
                                int group_list_type, const float *logit,
                                const int64_t *row_index, const uint16_t *shared_input,
                                float shared_input_weight, int64_t shared_input_offset,
                                float *out, int transpose_x2, int fp8_kind,
                                int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                                int64_t shared_rows, void *stream,
                                const gfr_options *opts);

/* Workspace bytes of a call with these sizes and options (first phase of
 * [P3]'s two-phase call, sizes only).  Pure host arithmetic.  Returns a
 * gfr_status. */
int gfr_workspace_size_raw(int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                           const gfr_options *opts, size_t *bytes);

/* gfr_gemm1_swiglu_quant on pointers and sizes: xin [M, H], w13 [E, H, 2I] or
 * [E, 2I, H], x1_out [M, I] bytes; fp8_kind names xin's and w13's format,
 * out_kind x1_out's (GFR_FP8_E4M3FN or GFR_FP8_E5M2); opts->scale_per_expert
 * selects a 4-D scale.  Limits as gfr_gemm1_swiglu_quant. */
int gfr_gemm1_swiglu_quant_raw(const void *xin, const void *w13, const uint8_t *scale,
                               const uint8_t *xin_scale, const int64_t *group_list,
                               int group_list_type, void *x1_out, uint8_t *x1_scale_out,
                               int transpose_w13, int fp8_kind, int out_kind, int64_t M,
                               int64_t H, int64_t I, int64_t E, void *stream,
                               const gfr_options *opts);

/* gfr_w4a8_finalize_routing on pointers and sizes (x2 [E, K, N/2] bytes,
 * scale / offset [E, 1, N]).  Limits as gfr_w4a8_finalize_routing. */
int gfr_w4a8_finalize_routing_raw(const int8_t *x1, const uint8_t *x2, const float *scale,
                                  const float *offset, const float *pertoken_scale,
                                  const int64_t *group_list, int group_list_type,
                                  const float *logit, const int64_t *row_index,
                                  const uint16_t *shared_input, float shared_input_weight,
                                  int64_t shared_input_offset, float *out, int64_t M, int64_t K,
                                  int64_t N, int64_t E, int64_t batch, int64_t shared_rows,
                                  void *stream, const gfr_options *opts);

/* Static, NUL-terminated description of a gfr_status. */
const char *gfr_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GFR_H */
