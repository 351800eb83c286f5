// Internal interface between the host API (gfr_api.cpp) and the kernels
// (gfr_kernels.hip).  Not installed; the public ABI is include/gfr.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gfr {

// Tile shape of one routed work item: 32 token rows x kTileN output columns,
// consumed in K steps of kStepK (32x32x64 block-scaled MFMAs); one step of the
// weight tile is 8 KB in either layout.  [K, N] weights: 128 columns x 64 K
// (each 128-byte row segment of x2 read whole); [N, K] weights: 64 columns x
// 128 K (each column's 128-byte K segment read whole).
constexpr int kTileM = 32;
constexpr int kTileN = 128;
constexpr int kStepK = 64;
constexpr int kTileNNK = 64;
constexpr int kStepKNK = 128;
constexpr int kWaveSize = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWaveSize * kWavesPerBlock;
constexpr int kMaxExperts = 1024;

// Everything a launch needs; device pointers, plain sizes.
struct FusedParams {
    const uint8_t *x1;
    const uint8_t *x2;
    const uint8_t *scale;
    const uint8_t *pts;
    const int64_t *group_list;
    const float *logit;        // may be null (weight 1)
    const void *row_index;     // int64 [M], or int32 [M] when row_index_i32
    int32_t row_index_i32;
    const uint16_t *shared;    // may be null
    float shared_w;
    int32_t shared_off;
    int32_t shared_rows;
    float *out;
    float *wbuf;               // deterministic mode: weighted rows [M, N]; else null
    int32_t *status;           // may be null
    int32_t *det_total;        // deterministic mode: routed-token total written here
    int32_t M, K, N, E, batch;
    int32_t group_list_type;
    int32_t split_k;           // 0: chosen on the device
    int64_t scale_e_stride;    // bytes between experts' weight scales (0: shared)
    // Upstream step (gate||up matmul + SwiGLU + MX quantisation); x2 then
    // holds 2I columns (N = 2I) and the output goes to q_out / qs_out.
    uint8_t *q_out;            // [M, I] FP8 codes
    uint8_t *qs_out;           // [M, I/64, 2] E8M0 block scales
    int32_t I;
    int32_t out_kind;          // 0 E4M3FN, 1 E5M2
    // W4A8 variant: x1 int8, x2 int4 pairs; FP32 scales
    const float *w_scale;      // [E, 1, N] fused per-channel scale
    const float *w_offset;     // [E, 1, N] asymmetric term, or null
    const float *pts_f;        // [M] per-token scale
};

// Internal element kind of the W4A8 variant (launch_fused's fp8_kind).
constexpr int kKindW4A8 = 8;

// Deterministic-mode workspace layout (all offsets 256-byte aligned):
//   wbuf          float [M, N]     weighted matmul rows
//   counts        int32 [batch]    tokens per output row (cleared each call)
//   cursor        int32 [batch]    fill positions
//   offsets       int32 [batch+1]  exclusive prefix of counts
//   tokens        int32 [M]        tokens grouped by output row (any order)
//   sorted        int32 [M]        the same, ascending within each row
//   total_tokens  int32            routed tokens (sum of group counts)
struct DetLayout {
    size_t wbuf, counts, cursor, offsets, tokens, sorted, total_tokens, total;
};
DetLayout det_layout(int64_t M, int64_t N, int64_t batch);

// Device address of the library's static scratch array on the current device
// (GFR_STATIC_SCRATCH_BYTES bytes, 256-byte aligned), looked up once per
// device with hipGetSymbolAddress; allocates nothing.
hipError_t static_scratch(void **ptr);

// Launchers; return hipSuccess or the launch error.
hipError_t launch_fused(const FusedParams &p, int transpose_x2, int fp8_kind,
                        hipStream_t stream);
hipError_t launch_gemm1(const FusedParams &p, int transpose_w13, int fp8_kind,
                        hipStream_t stream);
hipError_t launch_deterministic_prep(const FusedParams &p, void *workspace,
                                     hipStream_t stream);
hipError_t launch_deterministic_reduce(const FusedParams &p, void *workspace,
                                       hipStream_t stream);

}  // namespace gfr
