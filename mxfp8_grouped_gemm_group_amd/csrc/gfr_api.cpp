// Host side of the C ABI in include/gfr.h: tensor-descriptor validation,
// argument checks, workspace sizing and dispatch.  No device memory is read
// and nothing is synchronised; every error is returned before anything is
// enqueued.
//
// The descriptor calls resolve every size from the shapes and check each
// tensor's dtype, rank and extents against the others (the parameter check of
// the first phase of the CANN two-phase call, "aclnnGroupedMatmulFinalize
// RoutingV3"), then run the raw layer, which checks the sizes against the
// implementation's limits, pointers, alignment and enums.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <initializer_list>

#include "gfr.h"
#include "gfr_internal.h"

namespace {

constexpr int64_t kMaxRows = (int64_t{1} << 31) - 1;

bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// ---------------------------------------------------------------------------
// Raw layer: sizes given by the caller.
// ---------------------------------------------------------------------------

// Size limits shared by the calls and the size query.
int check_sizes(int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch) {
    if (M < 0 || K <= 0 || N < 0 || E <= 0 || batch < 0) return GFR_ERR_BAD_SHAPE;
    if (E > GFR_MAX_EXPERTS) return GFR_ERR_UNSUPPORTED;
    if (M > kMaxRows || batch > kMaxRows || K > kMaxRows || N > kMaxRows) return GFR_ERR_UNSUPPORTED;
    if (K % 128 != 0 || N % 16 != 0) return GFR_ERR_UNSUPPORTED;
    // One expert's weight slice (and, for [N, K] weights, a 128-column tile
    // past its end) and the weight-scale tensor are addressed with 32-bit
    // buffer offsets.
    if (K * (N + 128) > kMaxRows || M * K > int64_t{1} << 40) return GFR_ERR_UNSUPPORTED;
    // Work-item count (one K split, the narrower of the two layouts' column
    // tiles) must fit an int32.
    const int64_t n_tiles = (N + gfr::kTileNNK - 1) / gfr::kTileNNK;
    if ((M / gfr::kTileM + E) * n_tiles > kMaxRows) return GFR_ERR_UNSUPPORTED;
    return GFR_OK;
}

int validate(const void *x1, const void *x2, const uint8_t *scale, const uint8_t *pts,
             const int64_t *group_list, int group_list_type, const void *row_index,
             const uint16_t *shared, int64_t shared_off, const float *out, int transpose_x2,
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

// Deterministic-mode workspace and alignment checks.
int check_det(const gfr_options *opts, const float *out, int64_t M, int64_t N, int64_t batch) {
    if (!(opts && opts->deterministic)) return GFR_OK;
    const gfr::DetLayout d = gfr::det_layout(M, N, batch);
    if (!opts->workspace || opts->workspace_bytes < d.total) return GFR_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(opts->workspace, 256)) return GFR_ERR_BAD_ALIGNMENT;
    if (!aligned(out, 16)) return GFR_ERR_BAD_ALIGNMENT;   // float4 row reduction
    return GFR_OK;
}

int finalize_impl(const void *x1, const void *x2, const uint8_t *scale,
                  const uint8_t *pertoken_scale, const int64_t *group_list, int group_list_type,
                  const float *logit, const void *row_index, bool ri32,
                  const uint16_t *shared_input, float shared_input_weight,
                  int64_t shared_input_offset, float *out, int transpose_x2, int fp8_kind,
                  int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch, int64_t shared_rows,
                  void *stream, const gfr_options *opts) {
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
    p.row_index_i32 = ri32 ? 1 : 0;
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

int w4a8_impl(const int8_t *x1, const uint8_t *x2, const float *scale, const float *offset,
              const float *pertoken_scale, const int64_t *group_list, int group_list_type,
              const float *logit, const void *row_index, bool ri32, const uint16_t *shared_input,
              float shared_input_weight, int64_t shared_input_offset, float *out, int64_t M,
              int64_t K, int64_t N, int64_t E, int64_t batch, int64_t shared_rows, void *stream,
              const gfr_options *opts) {
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
    p.row_index_i32 = ri32 ? 1 : 0;
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

// ---------------------------------------------------------------------------
// Descriptor layer.
// ---------------------------------------------------------------------------

// An optional tensor is absent when its descriptor or its data is NULL
// (with no element, NULL data is a present but empty tensor).
bool present(const gfr_tensor *t) { return t && t->data; }

int64_t numel(const gfr_tensor *t) {
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
    return n;
}

// Rank in `ranks` (GFR_ERR_BAD_RANK), no negative extent (GFR_ERR_BAD_SHAPE),
// dtype in `dtypes` (GFR_ERR_BAD_DTYPE), data present when the tensor holds
// any element (GFR_ERR_NULL_ARG).
int check_desc(const gfr_tensor *t, std::initializer_list<int> ranks,
               std::initializer_list<int> dtypes) {
    if (!t) return GFR_ERR_NULL_ARG;
    bool rank_ok = false;
    for (int r : ranks) rank_ok |= t->ndim == r;
    if (!rank_ok || t->ndim < 1 || t->ndim > 4) return GFR_ERR_BAD_RANK;
    for (int i = 0; i < t->ndim; ++i)
        if (t->shape[i] < 0) return GFR_ERR_BAD_SHAPE;
    bool dtype_ok = false;
    for (int d : dtypes) dtype_ok |= t->dtype == d;
    if (!dtype_ok) return GFR_ERR_BAD_DTYPE;
    if (!t->data && numel(t) > 0) return GFR_ERR_NULL_ARG;
    return GFR_OK;
}

bool shape_is(const gfr_tensor *t, std::initializer_list<int64_t> s) {
    if (static_cast<size_t>(t->ndim) != s.size()) return false;
    int i = 0;
    for (int64_t v : s)
        if (t->shape[i++] != v) return false;
    return true;
}

#define GFR_TRY(expr)                  \
    do {                               \
        const int rc_ = (expr);        \
        if (rc_ != GFR_OK) return rc_; \
    } while (0)

const std::initializer_list<int> kScaleTypes = {GFR_DT_E8M0, GFR_DT_U8};
const std::initializer_list<int> kRowIndexTypes = {GFR_DT_I64, GFR_DT_I32};

struct Dims {
    int64_t M = 0, K = 0, N = 0, E = 0, batch = 0, R = 0;
    int per_expert = 0;
    bool ri32 = false;
};

// Checks shared by the routing arguments of both finalize variants: logit,
// row_index, shared_input, out, group_list.  Fills batch, R and ri32.
int resolve_routing(const gfr_tensor *group_list, const gfr_tensor *logit,
                    const gfr_tensor *row_index, const gfr_tensor *shared_input,
                    const gfr_tensor *out, Dims &d) {
    GFR_TRY(check_desc(group_list, {1}, {GFR_DT_I64}));
    GFR_TRY(check_desc(row_index, {1}, kRowIndexTypes));
    GFR_TRY(check_desc(out, {2}, {GFR_DT_F32}));
    if (present(logit)) GFR_TRY(check_desc(logit, {1}, {GFR_DT_F32}));
    if (present(shared_input)) GFR_TRY(check_desc(shared_input, {2}, {GFR_DT_BF16}));
    d.batch = out->shape[0];
    if (out->shape[1] != d.N) return GFR_ERR_BAD_SHAPE;
    if (!shape_is(group_list, {d.E}) || !shape_is(row_index, {d.M})) return GFR_ERR_BAD_SHAPE;
    if (present(logit) && !shape_is(logit, {d.M})) return GFR_ERR_BAD_SHAPE;
    d.R = 0;
    if (present(shared_input)) {
        if (shared_input->shape[1] != d.N) return GFR_ERR_BAD_SHAPE;
        d.R = shared_input->shape[0];
    }
    d.ri32 = row_index->dtype == GFR_DT_I32;
    return GFR_OK;
}

int resolve_finalize(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                     const gfr_tensor *pts, const gfr_tensor *group_list,
                     const gfr_tensor *logit, const gfr_tensor *row_index,
                     const gfr_tensor *shared_input, const gfr_tensor *out, int transpose_x2,
                     int fp8_kind, const gfr_options *opts, Dims &d) {
    if (!x1 || !x2 || !scale || !pts || !group_list || !row_index || !out)
        return GFR_ERR_NULL_ARG;
    if (transpose_x2 != 0 && transpose_x2 != 1) return GFR_ERR_BAD_ARG;
    int elem;
    switch (fp8_kind) {
    case GFR_FP8_E4M3FN: elem = GFR_DT_FP8_E4M3FN; break;
    case GFR_FP8_E5M2: elem = GFR_DT_FP8_E5M2; break;
    case GFR_FP4_E2M1: elem = GFR_DT_FP4_E2M1X2; break;
    default: return GFR_ERR_BAD_ARG;
    }
    GFR_TRY(check_desc(x1, {2}, {elem}));
    GFR_TRY(check_desc(x2, {3}, {elem}));
    GFR_TRY(check_desc(scale, {3, 4}, kScaleTypes));
    GFR_TRY(check_desc(pts, {3}, kScaleTypes));
    const int64_t per = fp8_kind == GFR_FP4_E2M1 ? 2 : 1;   // elements per stored byte
    d.M = x1->shape[0];
    d.K = x1->shape[1] * per;
    d.E = x2->shape[0];
    if (transpose_x2) {
        d.N = x2->shape[1];
        if (x2->shape[2] * per != d.K) return GFR_ERR_BAD_SHAPE;
    } else {
        if (x2->shape[1] != d.K) return GFR_ERR_BAD_SHAPE;
        d.N = x2->shape[2] * per;
    }
    const int64_t KB = (d.K + 63) / 64;
    d.per_expert = scale->ndim == 4;
    if (opts && opts->scale_per_expert != 0 && opts->scale_per_expert != 1) return GFR_ERR_BAD_ARG;
    if (opts && opts->scale_per_expert && !d.per_expert) return GFR_ERR_BAD_RANK;
    const int64_t s0 = transpose_x2 ? d.N : KB, s1 = transpose_x2 ? KB : d.N;
    if (d.per_expert ? !shape_is(scale, {d.E, s0, s1, 2}) : !shape_is(scale, {s0, s1, 2}))
        return GFR_ERR_BAD_SHAPE;
    if (!shape_is(pts, {d.M, KB, 2})) return GFR_ERR_BAD_SHAPE;
    return resolve_routing(group_list, logit, row_index, shared_input, out, d);
}

int resolve_w4a8(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                 const gfr_tensor *offset, const gfr_tensor *pts, const gfr_tensor *group_list,
                 const gfr_tensor *logit, const gfr_tensor *row_index,
                 const gfr_tensor *shared_input, const gfr_tensor *out, Dims &d) {
    if (!x1 || !x2 || !scale || !pts || !group_list || !row_index || !out)
        return GFR_ERR_NULL_ARG;
    GFR_TRY(check_desc(x1, {2}, {GFR_DT_I8}));
    GFR_TRY(check_desc(x2, {3}, {GFR_DT_INT4X2, GFR_DT_U8}));
    GFR_TRY(check_desc(scale, {3}, {GFR_DT_F32}));
    if (present(offset)) GFR_TRY(check_desc(offset, {3}, {GFR_DT_F32}));
    GFR_TRY(check_desc(pts, {1}, {GFR_DT_F32}));
    d.M = x1->shape[0];
    d.K = x1->shape[1];
    d.E = x2->shape[0];
    if (x2->shape[1] != d.K) return GFR_ERR_BAD_SHAPE;
    d.N = 2 * x2->shape[2];
    if (!shape_is(scale, {d.E, 1, d.N})) return GFR_ERR_BAD_SHAPE;
    if (present(offset) && !shape_is(offset, {d.E, 1, d.N})) return GFR_ERR_BAD_SHAPE;
    if (!shape_is(pts, {d.M})) return GFR_ERR_BAD_SHAPE;
    return resolve_routing(group_list, logit, row_index, shared_input, out, d);
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
    case GFR_ERR_BAD_DTYPE: return "a tensor's dtype is not one its argument takes (or x1 / x2 do not match fp8_kind)";
    case GFR_ERR_BAD_RANK: return "a tensor's rank is not its argument's";
    case GFR_ERR_SCRATCH_TOO_SMALL: return "the call needs more than the library's static scratch (GFR_STATIC_SCRATCH_BYTES per GPU); use gmm_finalize_routing_ex with a workspace";
    default: return "unknown status";
    }
}

// ---- raw calls --------------------------------------------------------------

int gfr_workspace_size_raw(int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                           const gfr_options *opts, size_t *bytes) {
    if (!bytes) return GFR_ERR_NULL_ARG;
    const int rc = check_sizes(M, K, N, E, batch);
    if (rc != GFR_OK) return rc;
    *bytes = (opts && opts->deterministic) ? gfr::det_layout(M, N, batch).total : 0;
    return GFR_OK;
}

int gmm_finalize_routing_raw_ex(const void *x1, const void *x2, const uint8_t *scale,
                                const uint8_t *pertoken_scale, const int64_t *group_list,
                                int group_list_type, const float *logit,
                                const int64_t *row_index, const uint16_t *shared_input,
                                float shared_input_weight, int64_t shared_input_offset,
                                float *out, int transpose_x2, int fp8_kind,
                                int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                                int64_t shared_rows, void *stream, const gfr_options *opts) {
    return finalize_impl(x1, x2, scale, pertoken_scale, group_list, group_list_type, logit,
                         row_index, false, shared_input, shared_input_weight,
                         shared_input_offset, out, transpose_x2, fp8_kind, M, K, N, E, batch,
                         shared_rows, stream, opts);
}

int gmm_finalize_routing_raw(const void *x1, const void *x2, const uint8_t *scale,
                             const uint8_t *pertoken_scale, const int64_t *group_list,
                             int group_list_type, const float *logit,
                             const int64_t *row_index, const uint16_t *shared_input,
                             float shared_input_weight, int64_t shared_input_offset,
                             float *out, int transpose_x2, int fp8_kind,
                             int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
                             int64_t shared_rows, void *stream) {
    return finalize_impl(x1, x2, scale, pertoken_scale, group_list, group_list_type, logit,
                         row_index, false, shared_input, shared_input_weight,
                         shared_input_offset, out, transpose_x2, fp8_kind, M, K, N, E, batch,
                         shared_rows, stream, nullptr);
}

int gfr_w4a8_finalize_routing_raw(const int8_t *x1, const uint8_t *x2, const float *scale,
                                  const float *offset, const float *pertoken_scale,
                                  const int64_t *group_list, int group_list_type,
                                  const float *logit, const int64_t *row_index,
                                  const uint16_t *shared_input, float shared_input_weight,
                                  int64_t shared_input_offset, float *out, int64_t M, int64_t K,
                                  int64_t N, int64_t E, int64_t batch, int64_t shared_rows,
                                  void *stream, const gfr_options *opts) {
    return w4a8_impl(x1, x2, scale, offset, pertoken_scale, group_list, group_list_type, logit,
                     row_index, false, shared_input, shared_input_weight, shared_input_offset,
                     out, M, K, N, E, batch, shared_rows, stream, opts);
}

int gfr_gemm1_swiglu_quant_raw(const void *xin, const void *w13, const uint8_t *scale,
                               const uint8_t *xin_scale, const int64_t *group_list,
                               int group_list_type, void *x1_out, uint8_t *x1_scale_out,
                               int transpose_w13, int fp8_kind, int out_kind, int64_t M,
                               int64_t H, int64_t I, int64_t E, void *stream,
                               const gfr_options *opts) {
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

// ---- descriptor calls ---------------------------------------------------------

int gmm_finalize_routing_ex(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                            const gfr_tensor *pertoken_scale, const gfr_tensor *group_list,
                            int group_list_type, const gfr_tensor *logit,
                            const gfr_tensor *row_index, const gfr_tensor *shared_input,
                            float shared_input_weight, int64_t shared_input_offset,
                            const gfr_tensor *out, int transpose_x2, int fp8_kind, void *stream,
                            const gfr_options *opts) {
    Dims d;
    GFR_TRY(resolve_finalize(x1, x2, scale, pertoken_scale, group_list, logit, row_index,
                             shared_input, out, transpose_x2, fp8_kind, opts, d));
    gfr_options o = opts ? *opts : gfr_options{};
    o.scale_per_expert = d.per_expert;
    return finalize_impl(
        x1->data, x2->data, static_cast<const uint8_t *>(scale->data),
        static_cast<const uint8_t *>(pertoken_scale->data),
        static_cast<const int64_t *>(group_list->data), group_list_type,
        present(logit) ? static_cast<const float *>(logit->data) : nullptr, row_index->data,
        d.ri32,
        present(shared_input) ? static_cast<const uint16_t *>(shared_input->data) : nullptr,
        shared_input_weight, shared_input_offset, static_cast<float *>(out->data), transpose_x2,
        fp8_kind, d.M, d.K, d.N, d.E, d.batch, d.R, stream, &o);
}

int gmm_finalize_routing(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                         const gfr_tensor *pertoken_scale, const gfr_tensor *group_list,
                         int group_list_type, const gfr_tensor *logit,
                         const gfr_tensor *row_index, const gfr_tensor *shared_input,
                         float shared_input_weight, int64_t shared_input_offset,
                         const gfr_tensor *out, int transpose_x2, int fp8_kind, void *stream) {
    return gmm_finalize_routing_ex(x1, x2, scale, pertoken_scale, group_list, group_list_type,
                                   logit, row_index, shared_input, shared_input_weight,
                                   shared_input_offset, out, transpose_x2, fp8_kind, stream,
                                   nullptr);
}

int gfr_workspace_size(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                       const gfr_tensor *pertoken_scale, const gfr_tensor *group_list,
                       int group_list_type, const gfr_tensor *logit,
                       const gfr_tensor *row_index, const gfr_tensor *shared_input,
                       float shared_input_weight, int64_t shared_input_offset,
                       const gfr_tensor *out, int transpose_x2, int fp8_kind,
                       const gfr_options *opts, size_t *bytes) {
    (void)shared_input_weight;
    if (!bytes) return GFR_ERR_NULL_ARG;
    Dims d;
    GFR_TRY(resolve_finalize(x1, x2, scale, pertoken_scale, group_list, logit, row_index,
                             shared_input, out, transpose_x2, fp8_kind, opts, d));
    GFR_TRY(validate(x1->data, x2->data, static_cast<const uint8_t *>(scale->data),
                     static_cast<const uint8_t *>(pertoken_scale->data),
                     static_cast<const int64_t *>(group_list->data), group_list_type,
                     row_index->data,
                     present(shared_input) ? static_cast<const uint16_t *>(shared_input->data)
                                           : nullptr,
                     shared_input_offset, static_cast<const float *>(out->data), transpose_x2,
                     fp8_kind, d.M, d.K, d.N, d.E, d.batch, d.R));
    *bytes = (opts && opts->deterministic) ? gfr::det_layout(d.M, d.N, d.batch).total : 0;
    return GFR_OK;
}

int gmm_finalize_routing_det_noalloc(const gfr_tensor *x1, const gfr_tensor *x2,
                                     const gfr_tensor *scale, const gfr_tensor *pertoken_scale,
                                     const gfr_tensor *group_list, int group_list_type,
                                     const gfr_tensor *logit, const gfr_tensor *row_index,
                                     const gfr_tensor *shared_input, float shared_input_weight,
                                     int64_t shared_input_offset, const gfr_tensor *out,
                                     int transpose_x2, int fp8_kind, void *stream,
                                     int32_t *status_dev) {
    Dims d;
    GFR_TRY(resolve_finalize(x1, x2, scale, pertoken_scale, group_list, logit, row_index,
                             shared_input, out, transpose_x2, fp8_kind, nullptr, d));
    const uint16_t *shared =
        present(shared_input) ? static_cast<const uint16_t *>(shared_input->data) : nullptr;
    GFR_TRY(validate(x1->data, x2->data, static_cast<const uint8_t *>(scale->data),
                     static_cast<const uint8_t *>(pertoken_scale->data),
                     static_cast<const int64_t *>(group_list->data), group_list_type,
                     row_index->data, shared, shared_input_offset,
                     static_cast<const float *>(out->data), transpose_x2, fp8_kind, d.M, d.K,
                     d.N, d.E, d.batch, d.R));
    if (d.N == 0 || d.batch == 0) return GFR_OK;   // empty output: nothing to do
    if (gfr::det_layout(d.M, d.N, d.batch).total > GFR_STATIC_SCRATCH_BYTES)
        return GFR_ERR_SCRATCH_TOO_SMALL;
    void *ws = nullptr;
    if (gfr::static_scratch(&ws) != hipSuccess) return GFR_ERR_HIP;
    gfr_options o{};
    o.deterministic = 1;
    o.workspace = ws;
    o.workspace_bytes = GFR_STATIC_SCRATCH_BYTES;
    o.status_dev = status_dev;
    o.scale_per_expert = d.per_expert;
    return finalize_impl(
        x1->data, x2->data, static_cast<const uint8_t *>(scale->data),
        static_cast<const uint8_t *>(pertoken_scale->data),
        static_cast<const int64_t *>(group_list->data), group_list_type,
        present(logit) ? static_cast<const float *>(logit->data) : nullptr, row_index->data,
        d.ri32, shared, shared_input_weight, shared_input_offset,
        static_cast<float *>(out->data), transpose_x2, fp8_kind, d.M, d.K, d.N, d.E, d.batch,
        d.R, stream, &o);
}

int gfr_w4a8_finalize_routing(const gfr_tensor *x1, const gfr_tensor *x2, const gfr_tensor *scale,
                              const gfr_tensor *offset, const gfr_tensor *pertoken_scale,
                              const gfr_tensor *group_list, int group_list_type,
                              const gfr_tensor *logit, const gfr_tensor *row_index,
                              const gfr_tensor *shared_input, float shared_input_weight,
                              int64_t shared_input_offset, const gfr_tensor *out, void *stream,
                              const gfr_options *opts) {
    Dims d;
    GFR_TRY(resolve_w4a8(x1, x2, scale, offset, pertoken_scale, group_list, logit, row_index,
                         shared_input, out, d));
    return w4a8_impl(
        static_cast<const int8_t *>(x1->data), static_cast<const uint8_t *>(x2->data),
        static_cast<const float *>(scale->data),
        present(offset) ? static_cast<const float *>(offset->data) : nullptr,
        static_cast<const float *>(pertoken_scale->data),
        static_cast<const int64_t *>(group_list->data), group_list_type,
        present(logit) ? static_cast<const float *>(logit->data) : nullptr, row_index->data,
        d.ri32,
        present(shared_input) ? static_cast<const uint16_t *>(shared_input->data) : nullptr,
        shared_input_weight, shared_input_offset, static_cast<float *>(out->data), d.M, d.K,
        d.N, d.E, d.batch, d.R, stream, opts);
}

int gfr_gemm1_swiglu_quant(const gfr_tensor *xin, const gfr_tensor *w13, const gfr_tensor *scale,
                           const gfr_tensor *xin_scale, const gfr_tensor *group_list,
                           int group_list_type, const gfr_tensor *x1_out,
                           const gfr_tensor *x1_scale_out, int transpose_w13, void *stream,
                           const gfr_options *opts) {
    if (!xin || !w13 || !scale || !xin_scale || !group_list || !x1_out || !x1_scale_out)
        return GFR_ERR_NULL_ARG;
    if (transpose_w13 != 0 && transpose_w13 != 1) return GFR_ERR_BAD_ARG;
    GFR_TRY(check_desc(xin, {2}, {GFR_DT_FP8_E4M3FN, GFR_DT_FP8_E5M2}));
    GFR_TRY(check_desc(w13, {3}, {xin->dtype}));
    GFR_TRY(check_desc(scale, {3, 4}, kScaleTypes));
    GFR_TRY(check_desc(xin_scale, {3}, kScaleTypes));
    GFR_TRY(check_desc(group_list, {1}, {GFR_DT_I64}));
    GFR_TRY(check_desc(x1_out, {2}, {GFR_DT_FP8_E4M3FN, GFR_DT_FP8_E5M2}));
    GFR_TRY(check_desc(x1_scale_out, {3}, kScaleTypes));
    const int64_t M = xin->shape[0], H = xin->shape[1], E = w13->shape[0];
    int64_t N2;
    if (transpose_w13) {
        if (w13->shape[2] != H) return GFR_ERR_BAD_SHAPE;
        N2 = w13->shape[1];
    } else {
        if (w13->shape[1] != H) return GFR_ERR_BAD_SHAPE;
        N2 = w13->shape[2];
    }
    if (N2 % 2 != 0) return GFR_ERR_BAD_SHAPE;
    const int64_t I = N2 / 2, KB = (H + 63) / 64;
    const int per_expert = scale->ndim == 4;
    if (opts && opts->scale_per_expert != 0 && opts->scale_per_expert != 1) return GFR_ERR_BAD_ARG;
    if (opts && opts->scale_per_expert && !per_expert) return GFR_ERR_BAD_RANK;
    const int64_t s0 = transpose_w13 ? N2 : KB, s1 = transpose_w13 ? KB : N2;
    if (per_expert ? !shape_is(scale, {E, s0, s1, 2}) : !shape_is(scale, {s0, s1, 2}))
        return GFR_ERR_BAD_SHAPE;
    if (!shape_is(xin_scale, {M, KB, 2}) || !shape_is(group_list, {E}) ||
        !shape_is(x1_out, {M, I}) || !shape_is(x1_scale_out, {M, (I + 63) / 64, 2}))
        return GFR_ERR_BAD_SHAPE;
    gfr_options o = opts ? *opts : gfr_options{};
    o.scale_per_expert = per_expert;
    const int kind = xin->dtype == GFR_DT_FP8_E4M3FN ? GFR_FP8_E4M3FN : GFR_FP8_E5M2;
    const int okind = x1_out->dtype == GFR_DT_FP8_E4M3FN ? GFR_FP8_E4M3FN : GFR_FP8_E5M2;
    return gfr_gemm1_swiglu_quant_raw(
        xin->data, w13->data, static_cast<const uint8_t *>(scale->data),
        static_cast<const uint8_t *>(xin_scale->data),
        static_cast<const int64_t *>(group_list->data), group_list_type, x1_out->data,
        static_cast<uint8_t *>(x1_scale_out->data), transpose_w13, kind, okind, M, H, I, E,
        stream, &o);
}

}  // extern "C"
