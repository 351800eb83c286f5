// Host side of the C ABI in include/gfr.h: argument validation, workspace
// sizing and dispatch.  No device memory is read and nothing is synchronised;
// every error is returned before anything is enqueued.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "gfr.h"
#include "gfr_internal.h"

namespace {

constexpr int64_t kMaxRows = (int64_t{1} << 31) - 1;

bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Shape / pointer / enum checks shared by the call and the size query.
int check_sizes(int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch) {
    if (M < 0 || K <= 0 || N < 0 || E <= 0 || batch < 0) return GFR_ERR_BAD_SHAPE;
    if (E > GFR_MAX_EXPERTS) return GFR_ERR_UNSUPPORTED;
    if (M > kMaxRows || batch > kMaxRows || K > kMaxRows || N > kMaxRows) return GFR_ERR_UNSUPPORTED;
    if (K % 128 != 0 || N % 16 != 0) return GFR_ERR_UNSUPPORTED;
    // One expert's weight slice and the weight-scale tensor are addressed with
    // 32-bit buffer offsets.
    if (K * N > kMaxRows || M * K > int64_t{1} << 40) return GFR_ERR_UNSUPPORTED;
    // Work-item count (one K split, the narrower of the two layouts' column
    // tiles) must fit an int32.
    const int64_t n_tiles = (N + gfr::kTileNNK - 1) / gfr::kTileNNK;
    if ((M / gfr::kTileM + E) * n_tiles > kMaxRows) return GFR_ERR_UNSUPPORTED;
    return GFR_OK;
}

int validate(const void *x1, const void *x2, const uint8_t *scale, const uint8_t *pts,
             const int64_t *group_list, int group_list_type, const int64_t *row_index,
             const uint16_t *shared, int64_t shared_off, float *out, int transpose_x2,
             int fp8_kind, int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
             int64_t shared_rows) {
    int rc = check_sizes(M, K, N, E, batch);
    if (rc != GFR_OK) return rc;
    if (fp8_kind != GFR_FP8_E4M3FN && fp8_kind != GFR_FP8_E5M2 && fp8_kind != GFR_FP4_E2M1)
        return GFR_ERR_BAD_ARG;
    if (group_list_type != GFR_GROUP_LIST_CUMSUM && group_list_type != GFR_GROUP_LIST_COUNT)
        return GFR_ERR_BAD_ARG;
    if (transpose_x2 != 0 && transpose_x2 != 1) return GFR_ERR_BAD_ARG;
    // E2M1 weight rows / columns are read in whole 16-byte chunks: [N, K] steps
    // are 256 K wide, and a [K, N] row (N / 2 bytes) must be 16-byte aligned.
    if (fp8_kind == GFR_FP4_E2M1 && (transpose_x2 ? K % 256 != 0 : N % 32 != 0))
        return GFR_ERR_UNSUPPORTED;
    const bool routed = M > 0 && N > 0 && batch > 0;
    if (routed && (!x1 || !x2 || !scale || !pts || !group_list || !row_index))
        return GFR_ERR_NULL_ARG;
    if (N > 0 && batch > 0 && !out) return GFR_ERR_NULL_ARG;
    if (shared) {
        if (shared_rows < 0) return GFR_ERR_BAD_SHAPE;
        if (shared_off < 0 || shared_off + shared_rows > batch) return GFR_ERR_BAD_OFFSET;
        if (!aligned(shared, 16)) return GFR_ERR_BAD_ALIGNMENT;
    }
    if (routed && (!aligned(x1, 16) || !aligned(x2, 16) || !aligned(scale, 16)))
        return GFR_ERR_BAD_ALIGNMENT;
    if (out && !aligned(out, 4)) return GFR_ERR_BAD_ALIGNMENT;
    return GFR_OK;
}

// Launch the finalize-routing path for a filled parameter block: one fused
// launch (atomic mode) or prep + fused + fixed-order reduce (deterministic).
int dispatch_finalize(gfr::FusedParams &p, int transpose_x2, int kind, int64_t M, int64_t N,
                      int64_t batch, hipStream_t s, const gfr_options *opts) {
    if (opts && opts->deterministic) {
        const gfr::DetLayout d = gfr::det_layout(M, N, batch);
        char *ws = static_cast<char *>(opts->workspace);
        p.wbuf = reinterpret_cast<float *>(ws + d.wbuf);
        p.det_total = reinterpret_cast<int32_t *>(ws + d.total_tokens);
        if (gfr::launch_deterministic_prep(p, opts->workspace, s) != hipSuccess) return GFR_ERR_HIP;
        if (gfr::launch_fused(p, transpose_x2, kind, s) != hipSuccess) return GFR_ERR_HIP;
        if (gfr::launch_deterministic_reduce(p, opts->workspace, s) != hipSuccess)
            return GFR_ERR_HIP;
        return GFR_OK;
    }
    if (gfr::launch_fused(p, transpose_x2, kind, s) != hipSuccess) return GFR_ERR_HIP;
    return GFR_OK;
}

// Deterministic-mode workspace and alignment checks (shared by both entries).
int check_det(const gfr_options *opts, const float *out, int64_t M, int64_t N, int64_t batch) {
    if (!(opts && opts->deterministic)) return GFR_OK;
    const gfr::DetLayout d = gfr::det_layout(M, N, batch);
    if (!opts->workspace || opts->workspace_bytes < d.total) return GFR_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(opts->workspace, 256)) return GFR_ERR_BAD_ALIGNMENT;
    if (!aligned(out, 16)) return GFR_ERR_BAD_ALIGNMENT;   // float4 row reduction
    return GFR_OK;
}

}  // namespace

extern "C" {

const char *gfr_status_string(int status) {
    switch (status) {
    case GFR_OK: return "ok";
    case GFR_ERR_NULL_ARG: return "a required pointer is NULL";
    case GFR_ERR_BAD_SHAPE: return "negative or inconsistent sizes";
    case GFR_ERR_BAD_OFFSET: return "shared_input_offset out of range (need 0 <= offset and offset + shared_rows <= batch)";
    case GFR_ERR_UNSUPPORTED: return "unsupported configuration (needs K % 128 == 0, N % 16 == 0, 1 <= E <= 1024, M, batch < 2^31; E2M1 also K % 256 == 0 with [N,K] weights, N % 32 == 0 with [K,N])";
    case GFR_ERR_BAD_ALIGNMENT: return "x1, x2, scale and shared_input must be 16-byte aligned";
    case GFR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small (query gfr_workspace_size)";
    case GFR_ERR_BAD_ARG: return "unknown fp8_kind, group_list_type or transpose flag";
    case GFR_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int gfr_workspace_size(int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                       const gfr_options *opts, size_t *bytes) {
    if (!bytes) return GFR_ERR_NULL_ARG;
    const int rc = check_sizes(M, K, N, E, batch);
    if (rc != GFR_OK) return rc;
    *bytes = (opts && opts->deterministic) ? gfr::det_layout(M, N, batch).total : 0;
    return GFR_OK;
}

int gmm_finalize_routing_ex(const void *x1, const void *x2, const uint8_t *scale,
                            const uint8_t *pertoken_scale, const int64_t *group_list,
                            int group_list_type, const float *logit,
                            const int64_t *row_index, const uint16_t *shared_input,
                            float shared_input_weight, int64_t shared_input_offset,
                            float *out, int transpose_x2, int fp8_kind,
                            int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                            int64_t shared_rows, void *stream, const gfr_options *opts) {
    int rc = validate(x1, x2, scale, pertoken_scale, group_list, group_list_type, row_index,
                      shared_input, shared_input_offset, out, transpose_x2, fp8_kind, M, K, N,
                      E, batch, shared_rows);
    if (rc != GFR_OK) return rc;
    if (N == 0 || batch == 0) return GFR_OK;  // empty output: nothing to do
    const int per_expert = opts ? opts->scale_per_expert : 0;
    if (per_expert != 0 && per_expert != 1) return GFR_ERR_BAD_ARG;
    rc = check_det(opts, out, M, N, batch);
    if (rc != GFR_OK) return rc;
    if (!shared_input) shared_rows = 0;

    gfr::FusedParams p{};
    p.x1 = static_cast<const uint8_t *>(x1);
    p.x2 = static_cast<const uint8_t *>(x2);
    p.scale = scale;
    p.pts = pertoken_scale;
    p.group_list = group_list;
    p.logit = logit;
    p.row_index = row_index;
    p.shared = shared_rows > 0 ? shared_input : nullptr;
    p.shared_w = shared_input_weight;
    p.shared_off = static_cast<int32_t>(shared_input_offset);
    p.shared_rows = static_cast<int32_t>(shared_rows);
    p.out = out;
    p.status = opts ? opts->status_dev : nullptr;
    p.M = static_cast<int32_t>(M);
    p.K = static_cast<int32_t>(K);
    p.N = static_cast<int32_t>(N);
    p.E = static_cast<int32_t>(E);
    p.batch = static_cast<int32_t>(batch);
    p.group_list_type = group_list_type;
    p.split_k = opts ? opts->split_k : 0;
    p.scale_e_stride = per_expert ? (K / 32) * N : 0;   // ceil(K/64) * N * 2 bytes
    return dispatch_finalize(p, transpose_x2, fp8_kind, M, N, batch,
                             static_cast<hipStream_t>(stream), opts);
}

int gfr_w4a8_finalize_routing(const int8_t *x1, const uint8_t *x2, const float *scale,
                              const float *offset, const float *pertoken_scale,
                              const int64_t *group_list, int group_list_type, const float *logit,
                              const int64_t *row_index, const uint16_t *shared_input,
                              float shared_input_weight, int64_t shared_input_offset, float *out,
                              int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                              int64_t shared_rows, void *stream, const gfr_options *opts) {
    int rc = check_sizes(M, K, N, E, batch);
    if (rc != GFR_OK) return rc;
    if (group_list_type != GFR_GROUP_LIST_CUMSUM && group_list_type != GFR_GROUP_LIST_COUNT)
        return GFR_ERR_BAD_ARG;
    // 16-byte weight rows (N/2 bytes); 16 * |sum of K products| < 2^31
    if (N % 32 != 0 || K > 65536) return GFR_ERR_UNSUPPORTED;
    const bool routed = M > 0 && N > 0 && batch > 0;
    if (routed && (!x1 || !x2 || !scale || !pertoken_scale || !group_list || !row_index))
        return GFR_ERR_NULL_ARG;
    if (N > 0 && batch > 0 && !out) return GFR_ERR_NULL_ARG;
    if (shared_input) {
        if (shared_rows < 0) return GFR_ERR_BAD_SHAPE;
        if (shared_input_offset < 0 || shared_input_offset + shared_rows > batch)
            return GFR_ERR_BAD_OFFSET;
        if (!aligned(shared_input, 16)) return GFR_ERR_BAD_ALIGNMENT;
    }
    if (routed && (!aligned(x1, 16) || !aligned(x2, 16) || !aligned(scale, 8) ||
                   !aligned(offset, 8) || !aligned(pertoken_scale, 4)))
        return GFR_ERR_BAD_ALIGNMENT;
    if (out && !aligned(out, 4)) return GFR_ERR_BAD_ALIGNMENT;
    if (N == 0 || batch == 0) return GFR_OK;
    if (opts && opts->scale_per_expert != 0) return GFR_ERR_BAD_ARG;   // scale is [E, 1, N]
    rc = check_det(opts, out, M, N, batch);
    if (rc != GFR_OK) return rc;
    if (!shared_input) shared_rows = 0;

    gfr::FusedParams p{};
    p.x1 = reinterpret_cast<const uint8_t *>(x1);
    p.x2 = x2;
    p.w_scale = scale;
    p.w_offset = offset;
    p.pts_f = pertoken_scale;
    p.group_list = group_list;
    p.logit = logit;
    p.row_index = row_index;
    p.shared = shared_rows > 0 ? shared_input : nullptr;
    p.shared_w = shared_input_weight;
    p.shared_off = static_cast<int32_t>(shared_input_offset);
    p.shared_rows = static_cast<int32_t>(shared_rows);
    p.out = out;
    p.status = opts ? opts->status_dev : nullptr;
    p.M = static_cast<int32_t>(M);
    p.K = static_cast<int32_t>(K);
    p.N = static_cast<int32_t>(N);
    p.E = static_cast<int32_t>(E);
    p.batch = static_cast<int32_t>(batch);
    p.group_list_type = group_list_type;
    p.split_k = opts ? opts->split_k : 0;
    return dispatch_finalize(p, 0, gfr::kKindW4A8, M, N, batch, static_cast<hipStream_t>(stream),
                             opts);
}

int gmm_finalize_routing(const void *x1, const void *x2, const uint8_t *scale,
                         const uint8_t *pertoken_scale, const int64_t *group_list,
                         int group_list_type, const float *logit,
                         const int64_t *row_index, const uint16_t *shared_input,
                         float shared_input_weight, int64_t shared_input_offset,
                         float *out, int transpose_x2, int fp8_kind,
                         int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                         int64_t shared_rows, void *stream) {
    return gmm_finalize_routing_ex(x1, x2, scale, pertoken_scale, group_list, group_list_type,
                                   logit, row_index, shared_input, shared_input_weight,
                                   shared_input_offset, out, transpose_x2, fp8_kind, M, K, N,
                                   E, batch, shared_rows, stream, nullptr);
}

int gfr_gemm1_swiglu_quant(const void *xin, const void *w13, const uint8_t *scale,
                           const uint8_t *xin_scale, const int64_t *group_list,
                           int group_list_type, void *x1_out, uint8_t *x1_scale_out,
                           int transpose_w13, int fp8_kind, int out_kind, int64_t M, int64_t H,
                           int64_t I, int64_t E, void *stream, const gfr_options *opts) {
    if (M < 0 || H <= 0 || I < 0 || E <= 0) return GFR_ERR_BAD_SHAPE;
    if (fp8_kind != GFR_FP8_E4M3FN && fp8_kind != GFR_FP8_E5M2 && fp8_kind != GFR_FP4_E2M1)
        return GFR_ERR_BAD_ARG;
    if (out_kind != GFR_FP8_E4M3FN && out_kind != GFR_FP8_E5M2) return GFR_ERR_BAD_ARG;
    if (group_list_type != GFR_GROUP_LIST_CUMSUM && group_list_type != GFR_GROUP_LIST_COUNT)
        return GFR_ERR_BAD_ARG;
    if (transpose_w13 != 0 && transpose_w13 != 1) return GFR_ERR_BAD_ARG;
    const int per_expert = opts ? opts->scale_per_expert : 0;
    if (per_expert != 0 && per_expert != 1) return GFR_ERR_BAD_ARG;
    if (fp8_kind == GFR_FP4_E2M1) return GFR_ERR_UNSUPPORTED;
    // the x2 limits of the main operator with N = 2I, and whole 64-column
    // output blocks (one item covers 64 or 32 outputs, two MX blocks or one)
    int rc = check_sizes(M, H, 2 * I, E, M);
    if (rc != GFR_OK) return rc;
    if (I % 64 != 0) return GFR_ERR_UNSUPPORTED;
    if (M == 0 || I == 0) return GFR_OK;   // nothing to produce
    if (!xin || !w13 || !scale || !xin_scale || !group_list || !x1_out || !x1_scale_out)
        return GFR_ERR_NULL_ARG;
    if (!aligned(xin, 16) || !aligned(w13, 16) || !aligned(scale, 16)) return GFR_ERR_BAD_ALIGNMENT;

    gfr::FusedParams p{};
    p.x1 = static_cast<const uint8_t *>(xin);
    p.x2 = static_cast<const uint8_t *>(w13);
    p.scale = scale;
    p.pts = xin_scale;
    p.group_list = group_list;
    p.status = opts ? opts->status_dev : nullptr;
    p.M = static_cast<int32_t>(M);
    p.K = static_cast<int32_t>(H);
    p.N = static_cast<int32_t>(2 * I);
    p.E = static_cast<int32_t>(E);
    p.batch = static_cast<int32_t>(M);
    p.group_list_type = group_list_type;
    p.split_k = 1;
    p.scale_e_stride = per_expert ? (H / 32) * (2 * I) : 0;
    p.q_out = static_cast<uint8_t *>(x1_out);
    p.qs_out = x1_scale_out;
    p.I = static_cast<int32_t>(I);
    p.out_kind = out_kind;
    if (gfr::launch_gemm1(p, transpose_w13, fp8_kind, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return GFR_ERR_HIP;
    return GFR_OK;
}

}  // extern "C"
