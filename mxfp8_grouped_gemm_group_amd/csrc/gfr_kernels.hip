// gfx950 kernels of the fused MXFP8 grouped-matmul + finalize-routing operator.
//
// Operation (page "grouped_matmul_finalize_routing 的 MXFP8 实现与精度验证",
// §2.1 formula, §2.2 four stages; CANN "aclnnGroupedMatmulFinalizeRoutingV3",
// formulas 1-4):
//   out[row_index[t], n] += logit[t] * sum_k dq(x1[t,k]) dq(x2[e(t),k,n])
//   out[off + r, n]      += shared_w * shared_input[r, n]
//
// One persistent launch does all of it:
//   * prologue — every workgroup turns group_list into per-expert token ranges
//     and a prefix of work items in LDS (no host round trip; ragged and empty
//     experts cost nothing);
//   * routed items — (expert, 32-token m-tile, 128-column n-tile, K split)
//     per wave, or (expert, 128-token group, n-tile, K split) per workgroup
//     for large experts.  Weight tiles stream global -> LDS ring with
//     direct-to-LDS buffer loads, x1 and the scales go to VGPRs; the [K, N]
//     layout is read out of LDS K-contiguous with transpose reads; the
//     contraction is v_mfma_scale_f32_32x32x64_f8f6f4 with the E8M0 scales fed
//     per lane (one scale per 32 K elements of one row / column);
//   * epilogue — acc * logit, then FP32 atomic add into out[row_index[t], n]
//     (or, in deterministic mode, a plain store of the weighted row);
//   * shared items — the bf16 shared-expert axpy, atomically, same launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "gfr.h"
#include "gfr_internal.h"

namespace gfr {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 ld16(const uint8_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ uint2 ld8(const uint8_t *p) {
    return *reinterpret_cast<const uint2 *>(p);
}
__device__ __forceinline__ uint32_t ld4(const uint8_t *p) {
    return *reinterpret_cast<const uint32_t *>(p);
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v2i lds_v2i_t;

// Raw buffer resource over [base, base + bytes); the wave-uniform base and
// row offsets live in SGPRs, each lane keeps one 32-bit offset.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int n = bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

__device__ __forceinline__ void flag(int32_t *status, int32_t bit) {
    if (status) atomicOr(status, bit);
}

// The lane index through an opaque copy.  Per-lane offsets and row numbers
// derived from it are then computed in the item that uses them: derived from
// threadIdx directly, the compiler hoists them out of the loop over units,
// where the constants of every kind of item stay live across all of them and
// push the main loops into spills (whose reloads wait for every load and
// atomic in flight).
__device__ __forceinline__ int lane_id() {
    int l;
    asm volatile("v_and_b32 %0, 63, %1" : "=v"(l) : "v"(static_cast<int>(threadIdx.x)));
    return l;
}

// Lane l of the wave gets v[0] op v[1] op ... op v[l]: DPP row shifts within
// each row of 16 lanes, then row broadcasts of lanes 15 and 31 (gfx9 DPP),
// seven steps that stay in the VALU (a shuffle scan sends every step through
// the LDS crossbar).  op is associative with identity 0; every lane of the
// wave takes part.
template <int CTRL, int ROWS, int BANKS, bool BOUND>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {   // lanes not written give 0
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROWS, BANKS, BOUND));
}
template <class F>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, F op) {
    uint32_t x = op(v, dpp_u32<0x111, 0xf, 0xf, true>(v));   // row_shr:1
    x = op(x, dpp_u32<0x112, 0xf, 0xf, true>(v));            // row_shr:2
    x = op(x, dpp_u32<0x113, 0xf, 0xf, true>(v));            // row_shr:3
    x = op(x, dpp_u32<0x114, 0xf, 0xe, false>(x));           // row_shr:4 into lanes 4-15
    x = op(x, dpp_u32<0x118, 0xf, 0xc, false>(x));           // row_shr:8 into lanes 8-15
    x = op(x, dpp_u32<0x142, 0xa, 0xf, false>(x));           // row_bcast:15 into rows 1, 3
    x = op(x, dpp_u32<0x143, 0xc, 0xf, false>(x));           // row_bcast:31 into rows 2, 3
    return x;
}

// Exclusive block-wide scans of NV 32-bit values per thread at once (v is
// replaced by its exclusive prefix, total gets the block's): wave scans,
// then the wave totals through LDS (s: 4 NV words; two barriers in all).
template <int NV, class F>
__device__ __forceinline__ void block_scan_u32(uint32_t (&v)[NV], uint32_t (&total)[NV],
                                               uint32_t *s, F op) {
    const int lane = threadIdx.x & (kWaveSize - 1), wv = threadIdx.x / kWaveSize;
    uint32_t ex[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const uint32_t x = wave_incl_scan(v[n], op);
        if (lane == kWaveSize - 1) s[wv * NV + n] = x;
        ex[n] = dpp_u32<0x138, 0xf, 0xf, true>(x);   // wave_shr:1: lane l - 1's, lane 0 0
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int i = 0; i < kWavesPerBlock; ++i) {
            const uint32_t t = s[i * NV + n];
            if (i < wv) before = op(before, t);
            all = op(all, t);
        }
        total[n] = all;
        v[n] = op(before, ex[n]);
    }
    __syncthreads();   // s may be reused after return
}

// As block_scan_u32, with an operator that also takes the value's index n.
template <int NV, class F>
__device__ __forceinline__ void block_scan_u32_by(uint32_t (&v)[NV], uint32_t (&total)[NV],
                                                  uint32_t *s, F op) {
    const int lane = threadIdx.x & (kWaveSize - 1), wv = threadIdx.x / kWaveSize;
    uint32_t ex[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        const uint32_t x = wave_incl_scan(v[n], [&](uint32_t a, uint32_t b) { return op(n, a, b); });
        if (lane == kWaveSize - 1) s[wv * NV + n] = x;
        ex[n] = dpp_u32<0x138, 0xf, 0xf, true>(x);   // wave_shr:1: lane l - 1's, lane 0 0
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int i = 0; i < kWavesPerBlock; ++i) {
            const uint32_t t = s[i * NV + n];
            if (i < wv) before = op(n, before, t);
            all = op(n, all, t);
        }
        total[n] = all;
        v[n] = op(n, before, ex[n]);
    }
    __syncthreads();   // s may be reused after return
}

// value 0 saturating at cap, the others plain sums
struct TokItemsOp {
    uint32_t cap;
    __device__ uint32_t operator()(int n, uint32_t a, uint32_t b) const {
        return n == 0 ? (a >= cap - b ? cap : a + b) : a + b;
    }
};

struct AddU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
// a + b saturated at cap (a, b <= cap): associative, identity 0
struct SatAddU32 {
    uint32_t cap;
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
        return a >= cap - b ? cap : a + b;
    }
};

// ---------------------------------------------------------------------------
// Work list (group_list -> expert ranges -> item prefix), built in LDS by
// every workgroup.  group_list formats per the page's §4.3: type 0 = prefix
// sums, type 1 = counts.  Invalid lists are clamped into [0, M) and flagged.
// ---------------------------------------------------------------------------
struct WorkList {
    int *start;   // [E]   first token of expert e
    int *cnt;     // [E]   tokens of expert e
    int *spref;   // [n_we+1] prefix of wave items (one K split), experts in `wperm` order
    int *wperm;   // [n_we]  experts with wave items, in the order their items are dealt
    int *lpref;   // [n_ce+1] prefix of cooperative block items, experts in `perm` order
    int *perm;    // [n_ce]  cooperative experts, most rows per cooperative group first
    int routed_tokens;  // sum of counts
    int sitems;         // spref[E]
    int litems;         // lpref[n_ce]
    int n_ce;           // experts with cooperative units
    int n_we;           // experts with wave items
};

// Experts with at least this many tokens are processed by cooperative block
// items: the four waves of a block share one weight-tile stream and each
// applies it to its own 32 rows, so one streamed tile serves 128 rows.
// Where the larger experts run two-fragment units (kinds with WIDE groups),
// experts of 64-95 tokens stream faster as wave items of two or three row
// tiles (c4 -1.8 %, c5 -0.8 %, c5_pe -1.1 %, g1_c2t -1.1 % against 64;
// thresholds of 80, 112 and 128 were each slower on one of c4, c5_fp4 or c5);
// with one-fragment units 64 stays (96: c4_fp4 +30 %, g1_llada +11 %).
constexpr int kCoopMinRows = 64;
constexpr int kCoopMinRowsWide = 96;
constexpr int kCoopRows = kTileM * kWavesPerBlock;   // 128

// Rows of one cooperative unit: experts with more than 128 rows use 256-row
// groups (each wave two 32-row fragments: twice the MFMAs per streamed and
// per LDS-read weight step), smaller ones 128-row groups.  Units whose
// fragment has 8 accumulators (FP4 [K,N]; the upstream step with [K,N]
// weights, gate and up side by side) keep one fragment: two would not fit the
// register file.  WIDE says whether two-fragment groups are used.
template <bool WIDE>
__device__ __forceinline__ int coop_group_rows(int cnt) {
    return (WIDE && cnt > kCoopRows) ? 2 * kCoopRows : kCoopRows;
}

constexpr int kPerThread = kMaxExperts / kBlockThreads;  // experts per thread

// Row groups per band in the order cooperative units are taken.  With the
// 128-column [N, K] units (ck_unit), 4 measured best: c5 1808 µs against 1819
// with 2 and 1866 with 1, c4 459 against 473 and 484, c5_pe 1859 against 1897
// and 1932.
constexpr int kCoopBand = 4;

template <bool WIDE>
__device__ __forceinline__ void build_work_list(const FusedParams &p, int n_tiles,
                                                int n_tiles_coop, WorkList &wl,
                                                int64_t *s_scan) {
    const int tid = threadIdx.x;
    constexpr int kMinRows = WIDE ? kCoopMinRowsWide : kCoopMinRows;
    static_assert(kPerThread == 4, "one thread reads 4 consecutive group_list entries");
    // All loads are issued before any is used (one memory latency, not one per
    // entry); reads past the list (or of an absent list when M = 0) return 0.
    const rsrc_t rg = make_rsrc(p.group_list, p.M > 0 ? static_cast<int64_t>(p.E) * 8 : 0);
    const int e0 = tid * kPerThread;
    const v4i g01 = __builtin_amdgcn_raw_buffer_load_b128(rg, e0 * 8, 0, 0);
    const v4i g23 = __builtin_amdgcn_raw_buffer_load_b128(rg, e0 * 8 + 16, 0, 0);
    const v2i gp = e0 > 0 ? __builtin_amdgcn_raw_buffer_load_b64(rg, e0 * 8 - 8, 0, 0) : v2i{0, 0};
    auto i64 = [](int lo, int hi) {
        return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                    static_cast<uint32_t>(lo));
    };
    const int64_t g[kPerThread + 1] = {i64(gp.x, gp.y), i64(g01.x, g01.y), i64(g01.z, g01.w),
                                       i64(g23.x, g23.y), i64(g23.z, g23.w)};
    int c[kPerThread];
    int64_t csum = 0;
    bool bad = false;
    uint32_t *const s32 = reinterpret_cast<uint32_t *>(s_scan);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = e0 + i;
        int64_t v = 0;
        if (e < p.E && p.M > 0) {
            v = p.group_list_type == GFR_GROUP_LIST_COUNT ? g[i + 1] : g[i + 1] - g[i];
            if (v < 0) { bad = true; v = 0; }
            if (v > p.M) { bad = true; v = p.M; }
        }
        c[i] = static_cast<int>(v);
        csum += c[i];
    }
    // Both item counts of an expert: wave items low, block items high (each
    // total stays below 2^31: the host bounds (M/32 + E) * ceil(N/128)).
    // Wave items in expert order here; with cooperative units of two
    // fragments they are reordered below.
    auto item_counts = [&](int cnt) -> int64_t {
        const int64_t si = cnt >= kMinRows ? 0 : ((cnt + kTileM - 1) / kTileM) * n_tiles;
        const int gr = coop_group_rows<WIDE>(cnt);
        const int64_t li = cnt >= kMinRows ? ((cnt + gr - 1) / gr) * n_tiles_coop : 0;
        return si | (li << 32);
    };
    // One scan for the tokens and both item counts of the counts as read.
    // The token scan saturates at M + 1 (with invalid lists the raw sum can
    // exceed M many times over; every prefix above M is treated alike).  For
    // a valid list (at most M tokens) no count is clamped and the item
    // prefixes stand; an invalid one is clamped against the token prefix and
    // its items scanned again.  (One scan less than tokens, then items: c1
    // -1.4 %, c1_fp4 -1.2 %.)
    const uint32_t cap = static_cast<uint32_t>(p.M) + 1u;
    int64_t items[kPerThread];
    int64_t isum = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        items[i] = item_counts(c[i]);
        isum += items[i];
    }
    uint32_t v3[3] = {static_cast<uint32_t>(csum < cap ? csum : cap),
                      static_cast<uint32_t>(isum), static_cast<uint32_t>(isum >> 32)}, t3[3];
    block_scan_u32_by<3>(v3, t3, s32, TokItemsOp{cap});
    const int64_t total_tokens = t3[0];
    int64_t run = v3[0];
    int ccnt[kPerThread];
    int64_t total_items = static_cast<int64_t>(t3[1]) | (static_cast<int64_t>(t3[2]) << 32);
    int64_t ipre = static_cast<int64_t>(v3[1]) | (static_cast<int64_t>(v3[2]) << 32);
    const bool clamp = total_tokens > p.M;   // block-uniform
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = tid * kPerThread + i;
        int cnt = c[i];
        if (run + cnt > p.M) { bad = true; cnt = run < p.M ? static_cast<int>(p.M - run) : 0; }
        ccnt[i] = cnt;
        if (e < p.E) {
            wl.start[e] = static_cast<int>(run < p.M ? run : p.M);
            wl.cnt[e] = cnt;
        }
        run += c[i];
    }
    if (clamp) {
        isum = 0;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            items[i] = item_counts(ccnt[i]);
            isum += items[i];
        }
        uint32_t iv[2] = {static_cast<uint32_t>(isum), static_cast<uint32_t>(isum >> 32)}, it[2];
        block_scan_u32<2>(iv, it, s32, AddU32{});
        total_items = static_cast<int64_t>(it[0]) | (static_cast<int64_t>(it[1]) << 32);
        ipre = static_cast<int64_t>(iv[0]) | (static_cast<int64_t>(iv[1]) << 32);
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = tid * kPerThread + i;
        if (e < p.E) {
            wl.spref[e] = static_cast<int>(ipre & 0xffffffff);
            wl.wperm[e] = e;
            wl.lpref[e] = static_cast<int>(ipre >> 32);
        }
        ipre += items[i];
    }
    if (tid == 0) {
        wl.spref[p.E] = static_cast<int>(total_items & 0xffffffff);
        wl.lpref[p.E] = static_cast<int>(total_items >> 32);
    }
    wl.routed_tokens = static_cast<int>(total_tokens < p.M ? total_tokens : p.M);
    wl.sitems = static_cast<int>(total_items & 0xffffffff);
    wl.litems = static_cast<int>(total_items >> 32);
    wl.n_ce = 0;
    wl.n_we = p.E;
    if (bad && blockIdx.x == 0) flag(p.status, GFR_DEV_BAD_GROUP_LIST);
    __syncthreads();
    if (wl.litems == 0) return;
    if (!WIDE) {
        // one-fragment units: cooperative experts in index order (their cost
        // does not follow the rows per group the same way; measured)
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int e = tid * kPerThread + i;
            if (e < p.E) wl.perm[e] = e;
        }
        wl.n_ce = p.E;
        __syncthreads();
        return;
    }

    // Beside two-fragment cooperative units (the snake deal) wave items go in
    // classes by the expert's row tiles -- one, two, three or more -- dealt
    // in that order: a unit of four wave items of a one-row-tile expert
    // streams four weight tiles, of a two-row-tile expert two (its waves pair
    // up on a tile), so the costly units come first and the cheap ones fill
    // the end of the launch, like a longest-first schedule (c5 -1.9 %, c5_pe
    // -2.1 %, c4 -1.3 %).  Within a class the experts keep their index
    // order.  (It costs about a microsecond of start-up, so shapes without
    // cooperative units keep the expert order: c1 +2.5 % with the classes.)
    {
        int wcls[kPerThread];
        // scan values: class items 0..2, class experts (0 | 1 << 16, 2)
        uint32_t cv[5] = {0, 0, 0, 0, 0}, ct[5];
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const uint32_t si = static_cast<uint32_t>(items[i] & 0xffffffff);
            const int mt = (ccnt[i] + kTileM - 1) / kTileM;
            wcls[i] = si > 0 ? (mt < 3 ? mt - 1 : 2) : -1;
            cv[0] += wcls[i] == 0 ? si : 0u;
            cv[1] += wcls[i] == 1 ? si : 0u;
            cv[2] += wcls[i] == 2 ? si : 0u;
            cv[3] += wcls[i] == 0 ? 1u : wcls[i] == 1 ? 1u << 16 : 0u;
            cv[4] += wcls[i] == 2 ? 1u : 0u;
        }
        block_scan_u32<5>(cv, ct, s32, AddU32{});   // also orders the writes above before these
        const uint32_t n0 = ct[3] & 0xffff, n1 = ct[3] >> 16;
        uint32_t ri[3] = {cv[0], ct[0] + cv[1], ct[0] + ct[1] + cv[2]};   // item offsets
        uint32_t re[3] = {cv[3] & 0xffff, n0 + (cv[3] >> 16), n0 + n1 + cv[4]};   // ranks
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int k = wcls[i];
            if (k < 0) continue;
            const uint32_t rank = k == 0 ? re[0] : k == 1 ? re[1] : re[2];
            const uint32_t off = k == 0 ? ri[0] : k == 1 ? ri[1] : ri[2];
            wl.spref[rank] = static_cast<int>(off);
            wl.wperm[rank] = tid * kPerThread + i;
            const uint32_t si = static_cast<uint32_t>(items[i] & 0xffffffff);
            if (k == 0) { ri[0] += si; re[0] += 1; }
            else if (k == 1) { ri[1] += si; re[1] += 1; }
            else { ri[2] += si; re[2] += 1; }
        }
        wl.n_we = static_cast<int>(n0 + n1 + ct[4]);
        if (tid == 0) wl.spref[wl.n_we] = static_cast<int>(ct[0] + ct[1] + ct[2]);
    }
    // Cooperative experts in the order their units are dealt: more rows per
    // cooperative group first (a unit's time grows with its live rows: their
    // x1 loads), ties by expert index.  The cooperative experts are first
    // compacted into a list of unique order values ((256 - key) << 10 | e,
    // smaller = earlier) in perm; each one's rank is the number of smaller
    // values in that list, counted four entries per LDS read.  (Only the
    // cooperative experts are visited: a pass over all E was 13 µs at E 256.)
    // lpref is then rebuilt as the prefix of cooperative units in that order.
    static_assert(kMaxExperts <= 1024, "expert index in 10 bits");
    int ord[kPerThread];
    int ncoop = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = tid * kPerThread + i;
        const bool coop = e < p.E && (items[i] >> 32) > 0;
        const int key = coop ? min(ccnt[i], coop_group_rows<WIDE>(ccnt[i])) : 0;
        ord[i] = coop ? ((2 * kCoopRows - key) << 10) | e : -1;
        ncoop += coop;
    }
    uint32_t sl[1] = {static_cast<uint32_t>(ncoop)}, sl_total[1];
    block_scan_u32<1>(sl, sl_total, s32, AddU32{});
    const int n_ce = static_cast<int>(sl_total[0]);
    int slot = static_cast<int>(sl[0]);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
        if (ord[i] >= 0) wl.perm[slot++] = ord[i];
    __syncthreads();
    int rank[kPerThread] = {};
    const int4 *lst = reinterpret_cast<const int4 *>(wl.perm);
    for (int j = 0; j < n_ce; j += 4) {
        const int4 v = lst[j >> 2];
        const int vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (j + q >= n_ce) break;
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) rank[i] += vv[q] < ord[i];
        }
    }
    __syncthreads();   // every thread has read the list
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
        if (ord[i] >= 0) wl.perm[rank[i]] = tid * kPerThread + i;
    __syncthreads();
    int lv[kPerThread];
    uint32_t lsum[1] = {0}, ltotal[1];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int r = tid * kPerThread + i;
        lv[i] = r < n_ce ? wl.lpref[wl.perm[r] + 1] - wl.lpref[wl.perm[r]] : 0;
        lsum[0] += static_cast<uint32_t>(lv[i]);
    }
    block_scan_u32<1>(lsum, ltotal, s32, AddU32{});   // ends synchronised
    int lpre = static_cast<int>(lsum[0]);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int r = tid * kPerThread + i;
        if (r <= n_ce) wl.lpref[r] = static_cast<int>(lpre);
        lpre += lv[i];
    }
    wl.n_ce = n_ce;
    __syncthreads();
}

// Largest e in [0, E) with pref[e] <= q (pref non-decreasing, pref[0] = 0).
__device__ __forceinline__ int find_expert(const int *pref, int E, int q) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] <= q) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Routed item: 32 tokens [m0, m0 + mcount) of expert e, columns
// [n0, n0 + 128), K steps [ks0, ks1) of 64.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 for one 64-wide K step
// (lane l, c = l % 32, g = l / 32), as measured on gfx950 with one-hot data
// and a distinct scale per lane:
//   A / B: row (column) c; bytes 0..15 hold K [16g, 16g + 16) and bytes
//          16..31 hold K [32 + 16g, 48 + 16g) of the step, i.e. a lane carries
//          half of each of the step's two 32-element scale blocks;
//   scales: the E8M0 of 32-block b of row (column) c comes from lane c + 32b,
//          so lane (c, g) supplies block g.
//   D: 16 floats; element r is row 8(r/4) + 4g + r%4, column c.
// Column c of MFMA j maps to output column n0 + 32j + c in both layouts: the
// [K, N] tile's operands come out of LDS K-contiguous per column through
// transpose reads, the [N, K] tile's through plain 16-byte reads.
// ---------------------------------------------------------------------------

// s_waitcnt vmcnt(N) (other counters untouched), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Every LDS read issued so far has returned, and (a memory clobber) the
// compiler moves no memory access across this point: the reads of a stage
// made with ordinary loads or builtins are done before that stage is
// refilled or a barrier hands it to the other waves.
__device__ __forceinline__ void lds_reads_done() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// LDS reads of the weight tile.  They are inline asm because the compiler's
// wait insertion cannot tell which direct-to-LDS load wrote which slot and
// would otherwise drain every outstanding load before each read; the explicit
// vmcnt wait before them orders the data.  The reads of a step are issued
// without waiting; lds_wait() waits for them and, since it takes the
// destination registers as in/out operands, nothing that uses them can be
// scheduled before it.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t *)p));
}

// The [K, N] tile's MFMA operands of one step: ds_read_b64_tr_b8 (gfx950 LDS
// transpose read).  Measured semantics: in each group of 16 lanes, output lane
// 8h + j receives byte j of the 8-byte rows addressed by lanes 2i + h,
// i = 0..7, as its bytes i.  So if lane 2i + h of the group points at K row
// k0 + i, columns c0 + 8h .. c0 + 8h + 7, lane 8h + j gets K rows k0 .. k0 + 7
// of column c0 + 8h + j: 8 bytes of its operand.  For 32-column group j the
// reads at a[j] + {0, 8, 32, 40} rows give operand bytes 0-7, 8-15, 16-23,
// 24-31 (t[4j + q]).
#define GFR_TR4(J)                                              \
    "ds_read_b64_tr_b8 %[t" #J "0], %[a" #J "]\n\t"             \
    "ds_read_b64_tr_b8 %[t" #J "1], %[a" #J "] offset:1024\n\t" \
    "ds_read_b64_tr_b8 %[t" #J "2], %[a" #J "] offset:4096\n\t" \
    "ds_read_b64_tr_b8 %[t" #J "3], %[a" #J "] offset:5120\n\t"
__device__ __forceinline__ void lds_issue_kn(const uint32_t (&a)[4], v2i (&t)[16]) {
    static_assert(8 * kTileN == 1024 && 32 * kTileN == 4096 && 40 * kTileN == 5120,
                  "row offsets of the four reads");
    asm volatile(GFR_TR4(0) GFR_TR4(1) GFR_TR4(2) GFR_TR4(3)
                 : [t00] "=&v"(t[0]), [t01] "=&v"(t[1]), [t02] "=&v"(t[2]), [t03] "=&v"(t[3]),
                   [t10] "=&v"(t[4]), [t11] "=&v"(t[5]), [t12] "=&v"(t[6]), [t13] "=&v"(t[7]),
                   [t20] "=&v"(t[8]), [t21] "=&v"(t[9]), [t22] "=&v"(t[10]), [t23] "=&v"(t[11]),
                   [t30] "=&v"(t[12]), [t31] "=&v"(t[13]), [t32] "=&v"(t[14]), [t33] "=&v"(t[15])
                 : [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3])
                 : "memory");
}
#undef GFR_TR4

__device__ __forceinline__ void lds_wait(v2i (&t)[16]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]),
                   "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]),
                   "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
                 :
                 : "memory");
}

// The FP4 [K, N] tile's operands of one step: ds_read_b64_tr_b4.  Measured
// semantics: in each group of 16 lanes, output lane j receives nibble j of the
// 8-byte rows addressed by lanes i = 0..15, as its nibble i (low nibble
// first).  So if lane i points at K row k0 + i, columns c0 .. c0 + 15 (8
// bytes), lane j gets K rows k0 .. k0 + 15 of column c0 + j: 8 bytes of its
// operand.  For 32-column group j the reads at a[j] and 16 rows further give
// operand bytes 0-7 (t[2j]) and 8-15 (t[2j + 1]).
#define GFR_TR2(J)                                              \
    "ds_read_b64_tr_b4 %[t" #J "0], %[a" #J "]\n\t"             \
    "ds_read_b64_tr_b4 %[t" #J "1], %[a" #J "] offset:2048\n\t"
__device__ __forceinline__ void lds_issue_kn4(const uint32_t (&a)[8], v2i (&t)[16]) {
    static_assert(16 * kTileN == 2048, "row offset of the second read");
    asm volatile(GFR_TR2(0) GFR_TR2(1) GFR_TR2(2) GFR_TR2(3) GFR_TR2(4) GFR_TR2(5) GFR_TR2(6)
                     GFR_TR2(7)
                 : [t00] "=&v"(t[0]), [t01] "=&v"(t[1]), [t10] "=&v"(t[2]), [t11] "=&v"(t[3]),
                   [t20] "=&v"(t[4]), [t21] "=&v"(t[5]), [t30] "=&v"(t[6]), [t31] "=&v"(t[7]),
                   [t40] "=&v"(t[8]), [t41] "=&v"(t[9]), [t50] "=&v"(t[10]), [t51] "=&v"(t[11]),
                   [t60] "=&v"(t[12]), [t61] "=&v"(t[13]), [t70] "=&v"(t[14]), [t71] "=&v"(t[15])
                 : [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]),
                   [a4] "v"(a[4]), [a5] "v"(a[5]), [a6] "v"(a[6]), [a7] "v"(a[7])
                 : "memory");
}
#undef GFR_TR2

// The [N, K] tile's operands of one step: 16-byte reads at a[sh] (column
// group 0, t[2 sh]) and a[sh] + 4096 (column group 1, t[2 sh + 1]), issued
// without waiting.
__device__ __forceinline__ void lds_issue_nk(const uint32_t (&a)[4], v4i (&t)[8]) {
    static_assert(32 * kStepKNK == 4096, "column group stride");
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:4096\n\t"
        "ds_read_b128 %2, %9\n\t"
        "ds_read_b128 %3, %9 offset:4096\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %10 offset:4096\n\t"
        "ds_read_b128 %6, %11\n\t"
        "ds_read_b128 %7, %11 offset:4096"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]),
          "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}

__device__ __forceinline__ void lds_wait(v4i (&t)[8]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]),
                   "+v"(t[6]), "+v"(t[7])
                 :
                 : "memory");
}

// D += A * B with per-lane E8M0 scales; OPSEL_B picks the byte of sb.
template <int FMT, int OPSEL_B>
__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f acc, uint32_t sa, uint32_t sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, FMT, FMT, 0, sa,
                                                            OPSEL_B, sb);
}

__device__ __forceinline__ v8i cat(v4i lo, v4i hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-wave LDS ring: kStages slots of one K step of the 64 x 128 weight tile.
constexpr int kStages = 4;
constexpr int kSlotBytes = kStepK * kTileN;            // 8 KB
static_assert(kStepKNK * kTileNNK == kSlotBytes, "both layouts move 8 KB per step");
constexpr int kRingBytes = kStages * kSlotBytes;       // 32 KB per wave
constexpr int kBLoadsPerStep = kSlotBytes / (kWaveSize * 16);   // 8 x 1 KB

// Registers that travel with one K step (the weight tile itself is in LDS).
// Scales are loaded as the aligned dword that holds them and the byte is
// selected when the step is consumed: a byte load would be zero-extended where
// the compiler chooses, which can force an early wait on the load.
template <int AL, int RF, int SB>
struct StepRegs {
    v4i a[RF][AL];       // x1 row bytes of fragment f: FP8 [K,N] bytes [16g, +16),
                         // [32 + 16g, +16) of the step's 64; [N,K] bytes 32q + 16g
                         // of the step's 128; FP4 [K,N] bytes [16g, +16) of 32
    uint32_t sa[RF][1];  // x1 scale bytes of the step
    uint32_t sb[SB][1];  // weight scale bytes of column group j
};

// Destination row and weight of the tile's 32 (or 64) rows, loaded when the
// item starts (their latency hides behind the weight stream): lane l holds row
// l's, and the epilogue fetches them with a lane shuffle.  A row past the
// expert's last token, or with row_index outside [0, batch) (flagged), gets
// dst = -1 and is skipped.
struct RowInfo {
    v2i dst;      // row_index[t] as two dwords (low, high)
    float w;
    bool live;    // lane < 32 and the row is one of the expert's tokens
};

// PTS (W4A8): the row weight also carries the FP32 per-token scale.
template <int RF, bool PTS = false>
__device__ __forceinline__ RowInfo load_row_info(const FusedParams &p, int m0, int mcount) {
    const int lane = lane_id();
    constexpr int kRows = kTileM * RF;
    RowInfo ri{v2i{0, 0}, 0.0f, lane < kRows && lane < mcount};
    const int cnt = mcount < kRows ? (mcount > 0 ? mcount : 0) : kRows;
    if (p.row_index_i32) {   // sign-extended to the two-dword form
        const rsrc_t rr = make_rsrc(static_cast<const int32_t *>(p.row_index) + m0,
                                    static_cast<int64_t>(cnt) * 4);
        const int v = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rr, 4 * lane, 0, 0));
        ri.dst = v2i{v, v >> 31};
    } else {
        const rsrc_t rr = make_rsrc(static_cast<const int64_t *>(p.row_index) + m0,
                                    static_cast<int64_t>(cnt) * 8);
        ri.dst = __builtin_amdgcn_raw_buffer_load_b64(rr, 8 * lane, 0, 0);
    }
    if (p.logit) {
        const rsrc_t rl = make_rsrc(p.logit + m0, static_cast<int64_t>(cnt) * 4);
        ri.w = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, 4 * lane, 0, 0));
    } else {
        ri.w = 1.0f;
    }
    if constexpr (PTS) {
        const rsrc_t rp = make_rsrc(p.pts_f + m0, static_cast<int64_t>(cnt) * 4);
        ri.w *= __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, 4 * lane, 0, 0));
    }
    return ri;
}

// Destination row of each lane's tile row (-1: skip), flagging bad indices.
__device__ __forceinline__ int row_dst(const FusedParams &p, const RowInfo &ri) {
    const int64_t d = static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(ri.dst.y)) << 32) |
                                           static_cast<uint32_t>(ri.dst.x));
    if (!ri.live) return -1;
    if (d < 0 || d >= p.batch) {
        flag(p.status, GFR_DEV_BAD_ROW_INDEX);
        return -1;
    }
    return static_cast<int>(d);
}

// Epilogue: weight each row by its logit and scatter-add (or store) it.
// acc element (j, r) of lane (c, g) is row 8(r/4) + 4g + r%4 and output column
// n0 + 32j + c, so each atomic instruction covers 32 adjacent columns.
template <int NJ, int RF, int NA>
__device__ __forceinline__ void epilogue(const FusedParams &p, const v16f (&accs)[RF][NA],
                                         int m0, int n0, bool store_rows, RowInfo ri) {
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    const int my_dst = row_dst(p, ri);
#pragma unroll
    for (int f = 0; f < RF; ++f) {
    const v16f (&acc)[NA] = accs[f];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 32 * f + 8 * (r >> 2) + 4 * g + (r & 3);
        const int dst = __shfl(my_dst, row);
        const float w = __shfl(ri.w, row);
        if (dst < 0) continue;
        const int t = m0 + row;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int col = n0 + 32 * j + c;
            if (col >= p.N) continue;
            const float v = acc[j][r] * w;
            if (store_rows)
                p.wbuf[static_cast<int64_t>(t) * p.N + col] = v;
            else
                unsafeAtomicAdd(p.out + static_cast<int64_t>(dst) * p.N + col, v);
        }
    }
    }
}

// Epilogue of a block-split wave unit: the block's four waves computed four
// K ranges of one item (same 32 rows, same 32 NA columns: NA = 4, or 8 for
// MXFP4 [K,N]).  Each wave leaves its NA accumulator groups in its own part
// of the LDS ring (NA x 4 KB), as [group j][register r][lane] (every store
// and load covers 64 consecutive dwords); after a block barrier wave w adds
// up the four waves' groups NA/4 w .. NA/4 (w + 1) - 1 in wave order and
// scatters their columns.  One atomic per output element instead of one per
// K range.  Every wave of the block must call it (block barrier), each after
// its last read of its own ring region.
template <int NA>
__device__ __forceinline__ void split_epilogue(const FusedParams &p, const v16f (&acc)[1][NA],
                                               int m0, int n0, bool store_rows, RowInfo ri,
                                               char *ring) {
    constexpr int G = NA / kWavesPerBlock;   // groups summed by each wave
    static_assert(NA % kWavesPerBlock == 0 && NA * 16 * kWaveSize * 4 <= kRingBytes,
                  "a wave's accumulators fit its ring region");
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float *own = reinterpret_cast<float *>(ring + w * kRingBytes);
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) own[(16 * j + r) * kWaveSize + lane] = acc[0][j][r];
    __syncthreads();
    v16f sum[1][G];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) sum[0][jj] = v16f{};
#pragma unroll
    for (int w2 = 0; w2 < kWavesPerBlock; ++w2) {
        const float *src = reinterpret_cast<const float *>(ring + w2 * kRingBytes) +
                           16 * G * w * kWaveSize + lane;
#pragma unroll
        for (int jj = 0; jj < G; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[0][jj][r] += src[(16 * jj + r) * kWaveSize];
    }
    epilogue<G, 1, G>(p, sum, m0, n0 + 32 * G * w, store_rows, ri);
}

// W4A8 epilogue.  acc[f][j] / acc[f][4 + j] hold 16 * the exact integer
// products of the odd / even weight columns n0 + 2(32j + c) + {1, 0}; rsum
// the lane's share of its row's x1 sum (K halves g = 0, 1 in lanes c, c + 32).
//   y = (logit * pts) * (scale[e, n] * P + offset[e, n] * sum_k x1)
// scattered like the MX operator's rows.
// Scale and offset of this lane's column pairs (2m, 2m + 1), loaded when the
// item starts: used first inside the per-row branches next to atomics, a load
// still in flight there would cost a full vmcnt drain per row.
struct ColScales {
    float2 sc[4], of[4];
};

__device__ __forceinline__ ColScales load_col_scales(const FusedParams &p, int e, int n0) {
    const int c = threadIdx.x & 31;
    const int N = p.N;
    ColScales cs;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + 2 * (32 * j + c);
        const int64_t at = static_cast<int64_t>(e) * N + (col < N ? col : n0);
        cs.sc[j] = *reinterpret_cast<const float2 *>(p.w_scale + at);
        cs.of[j] = p.w_offset ? *reinterpret_cast<const float2 *>(p.w_offset + at)
                              : float2{0.f, 0.f};
    }
    return cs;
}

template <int RF>
__device__ __forceinline__ void epilogue_w4a8(const FusedParams &p, const v16i (&acc)[RF][8],
                                              const int (&rsum)[RF], const ColScales &cs, int m0,
                                              int n0, bool store_rows, RowInfo ri) {
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    const int N = p.N;
    const int my_dst = row_dst(p, ri);
    const float2 (&sc)[4] = cs.sc;
    const float2 (&of)[4] = cs.of;
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        const int rs = rsum[f] + __shfl_xor(rsum[f], 32);   // row 32f + c, whole K range
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = 8 * (r >> 2) + 4 * g + (r & 3);
            const int row = 32 * f + rl;
            const int dst = __shfl(my_dst, row);
            const float w = __shfl(ri.w, row);
            const float S = static_cast<float>(__shfl(rs, rl));
            if (dst < 0) continue;
            const int t = m0 + row;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + 2 * (32 * j + c);
                if (col >= N) continue;
                const float pe = static_cast<float>(acc[f][4 + j][r] >> 4);   // exact
                const float po = static_cast<float>(acc[f][j][r] >> 4);
                const float ve = (sc[j].x * pe + of[j].x * S) * w;
                const float vo = (sc[j].y * po + of[j].y * S) * w;
                if (store_rows) {
                    *reinterpret_cast<float2 *>(p.wbuf + static_cast<int64_t>(t) * N + col) =
                        float2{ve, vo};
                } else {
                    float *o = p.out + static_cast<int64_t>(dst) * N + col;
                    unsafeAtomicAdd(o, ve);
                    unsafeAtomicAdd(o + 1, vo);
                }
            }
        }
    }
}

// FP32 -> FP8 code nearest to y, ties to even, saturating at the largest
// finite value (E4M3FN: bias 7, 3 mantissa bits, 0x7E = 448; E5M2: bias 15,
// 2 bits, 0x7B = 57344).  With e = max(floor(log2|y|), 1 - bias) the
// representable magnitudes near |y| are multiples of 2^(e - mbits);
// r = rint(|y| * 2^(mbits - e)) (exact scaling) and the code is
// ((e + bias) << mbits) + r - 2^mbits, which carries r = 2^(mbits + 1) into
// the next exponent and gives the subnormal codes for e = 1 - bias.
template <int BIAS, int MBITS, int MAXCODE>
__device__ __forceinline__ uint32_t fp8_encode(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80;
    const float a = fabsf(y);
    const int be = static_cast<int>(__float_as_uint(a) >> 23);   // a >= 0: no sign bit
    const int e = max(be - 127, 1 - BIAS);                        // be = 0: zero or subnormal
    const float sc = __uint_as_float(static_cast<uint32_t>(127 + MBITS - e) << 23);
    const int r = static_cast<int>(rintf(a * sc));
    const int code = min(((e + BIAS) << MBITS) + r - (1 << MBITS), MAXCODE);
    return static_cast<uint32_t>(code) | sign;
}

// Epilogue of the upstream step: accumulator groups j < NJ/2 hold gate
// columns n0 + 32j + c and groups j >= NJ/2 the matching up columns, so
// sw = SiLU(gate) * up = gate / (1 + exp(-gate)) * up in FP32.  Each 32-column
// group of a row is one MX block: its largest magnitude (a max over the 32
// lanes of the half-wave that hold the row) gives the block exponent
// X = floor(log2(amax)) - emax (emax 8 for E4M3FN, 15 for E5M2; -127 for an
// all-zero block, never below -127), and each element is encoded as
// fp8(sw * 2^-X).  Codes go to q_out[t, :] (32 adjacent bytes per row and
// group), the scale byte X + 127 to qs_out[t, col / 32].
template <int NJ, int RF, int NA>
__device__ __forceinline__ void epilogue_swiglu(const FusedParams &p, const v16f (&accs)[RF][NA],
                                                int m0, int mcount, int n0) {
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    const int I = p.I;
    const bool e5 = p.out_kind == GFR_FP8_E5M2;
    const int emax = e5 ? 15 : 8;
#pragma unroll
    for (int f = 0; f < RF; ++f) {
#pragma unroll
        for (int jj = 0; jj < NJ / 2; ++jj) {
            if (n0 + 32 * jj >= I) continue;   // past I (whole 32-blocks, wave-uniform)
            float sw[16], am[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float gt = accs[f][jj][r], ut = accs[f][jj + NJ / 2][r];
                sw[r] = gt / (1.0f + expf(-gt)) * ut;
                am[r] = fabsf(sw[r]);
            }
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1)
#pragma unroll
                for (int r = 0; r < 16; ++r) am[r] = fmaxf(am[r], __shfl_xor(am[r], off));
            const int col = n0 + 32 * jj + c;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * f + 8 * (r >> 2) + 4 * g + (r & 3);
                if (row >= mcount) continue;
                const int be = static_cast<int>(__float_as_uint(am[r]) >> 23);
                const int X = be == 0 ? -127 : max(be - 127 - emax, -127);
                const float y = sw[r] * __uint_as_float(static_cast<uint32_t>(127 - X) << 23);
                const uint32_t q = e5 ? fp8_encode<15, 2, 0x7B>(y) : fp8_encode<7, 3, 0x7E>(y);
                const int64_t t = m0 + row;
                p.q_out[t * I + col] = static_cast<uint8_t>(q);
                if (c == 0) p.qs_out[t * (I / 32) + (n0 / 32 + jj)] = static_cast<uint8_t>(X + 127);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Routed item mainloop.  Per K step
//   * the 64 x 128 weight tile is moved global -> LDS with 8 direct-to-LDS
//     16-byte loads into a ring slot, and each wave loads its x1 bytes and the
//     scales into registers;
//   * a wave waits (vmcnt) until the slot it is about to use has landed, with
//     the later steps' loads still in flight;
//   * it reads its MFMA operands from LDS and runs 4 MFMAs (32 rows x 128 cols).
// Two modes:
//   wave (COOP = false): one wave owns the item, its own ring (kStages slots)
//     and all 8 tile loads per step;
//   cooperative (COOP = true): the four waves of a block share one ring
//     (kCoopStagesKN / kCoopStagesNK slots); wave w issues tile loads 2w and 2w+1 of each step
//     and applies the tile to its own 32 rows (rows 32w.. of a 128-row
//     group); one s_barrier per step publishes the tile and retires the slot
//     that is refilled next.
// [K, N]: the slot is row-major [64 K rows][128 B] with the eight 16-byte
//   chunks of row r XOR-swizzled by 2 ((r >> 1) & 3); the operand comes out
//   of LDS already K-contiguous per column (ds_read_b64_tr_b8).  A half wave
//   of a transposing read (the 64 banks serve 32 lanes of 8 bytes at once)
//   is two 16-lane groups reading logical chunks 2j and 2j + 1 of the same
//   8 rows: with the even swizzle one group lands on even physical chunks and
//   the other on odd ones, 64 distinct banks (with (r >> 1) & 3 both groups
//   covered the same four chunks: two-way conflicts, 0.96 conflict cycles
//   per conflict-free cycle in c3; p1_tc_b -3 %, c3 -0.8 %).
// [N, K]: the slot is [128 cols][64 K bytes] with the four 16-byte chunks of
//   a column XOR-swizzled by (col >> 1) & 3 so that 16-byte LDS reads of 32
//   lanes do not collide on banks.
// ---------------------------------------------------------------------------
constexpr int kCoopStagesKN = 8;   // vmcnt range caps these: (D - 1) * ops < 64
constexpr int kCoopStagesNK = 8;
constexpr int kCoopStagesKN4 = 6;  // FP4 [K, N]: eight weight-scale loads per step
static_assert(kCoopStagesKN * kSlotBytes <= kWavesPerBlock * kRingBytes &&
                  kCoopStagesNK * kSlotBytes <= kWavesPerBlock * kRingBytes &&
                  kCoopStagesKN4 * kSlotBytes <= kWavesPerBlock * kRingBytes,
              "cooperative ring fits the block's LDS");

// One 32-bit element k (uniform, 0..3; larger values read element 3) of w.
// Cache policy of the weight loads of a wave item whose weights no other
// item reads (NT): non-temporal, as the page's kernel marks each expert's
// weight tile non-cacheable to spare L2 (§5.3).  A probe streaming 1 GB as 32
// experts x 8192 rows x 4 KB in 128-byte pieces of 64 rows (the [K,N] wave
// items' pattern) read 6.3 TB/s with the default policy and 6.9-7.0 TB/s
// with nt; where weights are shared through L2 (cooperative units, the row
// tiles of one expert) the default policy is kept.
constexpr int kNonTemporal = 2;
constexpr int kStreamMinBytes = 256 << 10;   // an item's weight bytes for nt loads

__device__ __forceinline__ uint32_t pick(const v4i &w, int k) {
    return static_cast<uint32_t>(k <= 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w);
}

// a compile-time int passed to generic lambdas
template <int V>
struct IntC {
    static constexpr int value = V;
};

// An empty use of a loaded register: the load stays, and the compiler waits
// for it here.  The cooperative units' explicit vmcnt waits count every load
// a step issues, so a load whose result a loop instance never reads (the
// scales of a fragment without live rows) must not be dropped: the waits
// would then let that many of the step's later tile loads pass unfinished.
template <class T>
__device__ __forceinline__ void keep_loaded(const T &v) {
    asm volatile("" ::"v"(v));
}

// Rotation of an [N, K] wave item's K order.  A step reads the same 128-byte
// piece of 128 weight rows (columns); where a row is 4 KB long (MXFP4 K 8192)
// every item in flight then hits the same in-row offset, the rows of
// different column tiles and experts lie a multiple of 512 KB apart, and the
// reads crowd onto a few memory channels: streaming 128 rows x 4 KB this way
// ran at 3.9 TB/s, against 5.6 with each item starting at its own step, the
// same as reading the bytes in order (c3_fp4t 149 -> 116 µs).  So an item
// runs its steps from ks0 + rot to ks1 - 1, then from ks0 to ks0 + rot - 1,
// rot chosen by expert: the column tiles of one expert keep the same order,
// as they share its x1 rows through L2 (keyed on the column tile as well, c5
// ran 2 % slower).  With scale windows of WIN steps, rot = n mod WIN + WIN h
// (n steps in the range): the wrap then falls on a window boundary.  The
// addition order changes with rot; the sum does not.  The cooperative units
// keep the plain order (rotated, c5 ran 1-3 % slower).
__device__ __forceinline__ int k_rotation(int e, int n, int win) {
    const int q = n / win;   // whole windows in the range
    if (q < 2) return 0;
    return n % win + win * (e % q);
}

// split: the block's LDS ring when the item is one of a block-split wave
// unit's four K ranges (split_epilogue), else null.
template <int FMT, bool KN, bool COOP, int RF, int OP, bool WS = false, bool NT = false>
__device__ __forceinline__ void routed_item(const FusedParams &p, int e, int m0, int mcount, int n0,
                            int ks0, int ks1, bool store_rows, char *ring, int w,
                            char *split = nullptr) {
    static_assert(RF == 1 || (COOP && RF == 2), "two row fragments only in cooperative units");
    // FP4 E2M1 (MFMA format 4): elements packed two per byte along the
    // contiguous axis (x1 along K, [K, N] weights along N).  An FP4 MFMA
    // operand is 16 bytes per lane: lane (c, g) holds K [32g, 32g + 32) of
    // its row / column, nibble i = K 32g + i (low nibble first) -- measured
    // with one-hot operands against an FP8 operand of known layout.  FP4
    // [K, N] steps are 64 K x 256 columns (the slot keeps 64 rows of 128
    // bytes), eight MFMAs per step.  (MXFP4 [N, K] items are ck_unit's and
    // cw_item's.)
    constexpr bool FP4 = FMT == 4;
    constexpr bool KN4 = FP4 && KN;
    static_assert(!FP4 || KN, "MXFP4 here only with [K, N] weights");
    // FMT 8, the W4A8 variant: INT8 x1 and signed INT4 [K, N] weights packed
    // two per byte along N.  Its slot is FP8's (64 K rows of 128 bytes, here
    // 256 columns) and its operands come out of LDS the same way, as
    // K-contiguous bytes of a byte column 2j|2j+1.  v_mfma_i32_32x32x32_i8
    // multiplies them twice: with byte & 0xF0 (= 16 * the odd column's
    // value) and with (byte << 4) & 0xF0 (= 16 * the even column's value),
    // both exact; acc[f][j] holds the odd columns, acc[f][4 + j] the even ones.
    // Lane (c, g) supplies K bytes [16g, 16g + 16) of each 32-K half to both
    // operands: the product pairs A and B bytes by position, so any K order
    // shared by the two is exact.
    constexpr bool I8 = FMT == 8;
    static_assert(!I8 || (KN && OP == 0), "W4A8: [K, N] weights, finalize routing");
    // OP 0: finalize routing (weight columns n0 + tile column).  OP 1: the
    // upstream step.  [N,K] weights: the tile's first half of columns comes
    // from the gate block [n0, n0 + 32) and its second half from the up block
    // [I + n0, I + n0 + 32) of the 2I weight columns.  [K,N] weights (SPLIT):
    // every K step is taken twice, as two virtual steps -- first the gate
    // tile [n0, n0 + 128), then the up tile [I + n0, I + n0 + 128) -- so each
    // weight row segment read stays a whole 128 bytes; the halves accumulate
    // into acc[f][0..3] and acc[f][4..7].
    static_assert(OP == 0 || !FP4, "the upstream step is MXFP8 only");
    constexpr bool SPLIT = OP == 1 && KN;
    constexpr int kVS = SPLIT ? 2 : 1;      // virtual steps per K step
    constexpr int kHalf = (KN ? kTileN : kTileNNK) / 2;
    const int up0 = OP == 1 ? __builtin_amdgcn_readfirstlane(p.I) : 0;
    constexpr int D = !COOP ? kStages
                      : RF == 2 ? 4
                      : KN4 ? kCoopStagesKN4
                      : (KN ? kCoopStagesKN : kCoopStagesNK);
    constexpr int kTileLoads = COOP ? kBLoadsPerStep / kWavesPerBlock : kBLoadsPerStep;
    // The item is wave-uniform; say so, so that descriptors and offsets stay
    // in SGPRs (a descriptor in VGPRs turns every buffer load into a loop).
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mcount = __builtin_amdgcn_readfirstlane(mcount);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    ks0 = __builtin_amdgcn_readfirstlane(ks0);
    ks1 = __builtin_amdgcn_readfirstlane(ks1);
    w = __builtin_amdgcn_readfirstlane(w);
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    const int K = p.K, N = p.N, KS = p.K / 32;
    const int Kb = FP4 ? K / 2 : K;    // bytes of one x1 row / one [N, K] weight column
    const int Nb = FP4 || I8 ? N / 2 : N;    // bytes of one [K, N] weight row
    // x1 rows of this tile; padding rows read row 0 and are zeroed before use
    // (a cooperative wave past the expert's last row has mcount <= 0: its
    // loads have an empty range and return zeros, its epilogue writes nothing)
    if (mcount < 0) mcount = 0;
    auto wcol = [&](int tc) {
        return OP == 0 || SPLIT || tc < kHalf ? n0 + tc : up0 + n0 + tc - kHalf;
    };
    bool arow_ok[RF];
    int va[RF], vsa[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        arow_ok[f] = kTileM * f + c < mcount;
        const int arow = arow_ok[f] ? kTileM * f + c : 0;
        va[f] = arow * Kb + 16 * g;
        vsa[f] = arow * KS;       // + (2 ks) & ~3 or 4 ks: KS is a multiple of 4
    }
    const rsrc_t ra = make_rsrc(p.x1 + static_cast<int64_t>(m0) * Kb, static_cast<int64_t>(mcount) * Kb);
    const rsrc_t rsa = make_rsrc(p.pts + static_cast<int64_t>(m0) * KS, static_cast<int64_t>(mcount) * KS);
    const int64_t wbytes = KN ? static_cast<int64_t>(K) * Nb : static_cast<int64_t>(N) * Kb;
    const rsrc_t rb = make_rsrc(p.x2 + e * wbytes, wbytes);
    const rsrc_t rsb = make_rsrc(p.scale + e * p.scale_e_stride, static_cast<int64_t>(KS) * N);
    const int u0 = COOP ? w * kTileLoads : 0;   // first tile load this wave issues
    // Weight-tile load offsets (lane part) and weight-scale offsets.  Columns
    // past N (last partial n-tile) re-read column n0; their results are never
    // written.
    int vb[KN ? (KN4 || SPLIT ? 2 : 1) : kTileLoads];
    int vsb[KN4 || SPLIT ? 8 : 4];
    uint32_t tr_addr[KN4 ? 8 : 4] = {};   // [K,N]: per 32-column group, slot-relative
    int sb_shift = 0;
    if constexpr (KN4) {
        // load u, lane l: K row r = 8u + l/8 (row offset in soffset); it fills
        // physical chunk l%8 of the slot row, which holds logical chunk
        // (l%8) ^ ((r >> 1) & 7) = (l%8) ^ (4 (u & 1) + l/16): one offset for
        // even and one for odd loads.  Chunk = 16 bytes = 32 columns.
        const int n0b = n0 / 2;
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int cb = n0b + 16 * ((lane & 7) ^ (4 * par + (lane >> 4)));
            vb[par] = (lane >> 3) * Nb + (cb < Nb ? cb : n0b);
        }
        // transpose reads: lane s of 16-lane group G reads K row 32g + s (16
        // rows further in the second read), the 8 bytes of columns
        // 32j + 16(G & 1) .. + 15 (half G & 1 of logical chunk j); the slot
        // row pitch is 128 bytes, and (row >> 1) & 7 = s >> 1
        const int G = lane >> 4, sl = lane & 15;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            tr_addr[j] = (32 * g + sl) * kTileN + 16 * (j ^ (sl >> 1)) + 8 * (G & 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = n0 + 32 * j + c;
            vsb[j] = ((col < N ? col : n0) & ~1) * 2;
        }
        sb_shift = 8 * (2 * (c & 1) + g);
    } else if (KN && I8) {
        // as for FP8 [K, N] below, in bytes: the tile's 128 byte columns are
        // weight columns [n0, n0 + 256)
        const int n0b = n0 / 2;
        const int cb = n0b + 16 * ((lane & 7) ^ (2 * ((lane >> 4) & 3)));
        vb[0] = (lane >> 3) * Nb + (cb < Nb ? cb : n0b);
        const int G = lane >> 4, sl = lane & 15, i = sl >> 1, h = sl & 1;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            tr_addr[j] = (16 * g + i) * kTileN + 16 * ((2 * j + (G & 1)) ^ (2 * ((i >> 1) & 3))) + 8 * h;
    } else if (KN) {
        // load u, lane l: K row r = 8u + l/8 (row offset in soffset); it fills
        // physical chunk l%8 of the slot row, which holds logical chunk
        // (l%8) ^ 2 ((r >> 1) & 3) = (l%8) ^ 2 ((l >> 4) & 3)
        const int chunk_col = wcol(16 * ((lane & 7) ^ (2 * ((lane >> 4) & 3))));
        vb[0] = (lane >> 3) * N + (chunk_col < N ? chunk_col : n0);
        if constexpr (SPLIT) {   // the up tile: same chunk, I columns further
            const int up_col = up0 + chunk_col;
            vb[1] = (lane >> 3) * N + (up_col < N ? up_col : up0 + n0);
        }
        // transpose reads: lane s of 16-lane group G reads K row
        // 16g + (s >> 1) + (read's K offset), columns 32j + 16(G & 1) + 8(s & 1)
        const int G = lane >> 4, sl = lane & 15, i = sl >> 1, h = sl & 1;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            tr_addr[j] = (16 * g + i) * kTileN + 16 * ((2 * j + (G & 1)) ^ (2 * ((i >> 1) & 3))) + 8 * h;
        // scale byte (ks, col, g) is byte 2 col + g of row ks of [K/64, N, 2];
        // the aligned dword holds columns col & ~1 and col | 1
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = wcol(32 * j + c);
            vsb[j] = ((col < N ? col : n0) & ~1) * 2;
            if constexpr (SPLIT) {
                const int up_col = up0 + col;
                vsb[4 + j] = ((up_col < N ? up_col : up0 + n0) & ~1) * 2;
            }
        }
        sb_shift = 8 * (2 * (c & 1) + g);
    } else {
        // load u, lane l: tile column 8u + l/8 (its 128-byte K segment of the
        // step); it fills physical chunk l%8 of that column's 128-byte slot
        // row, which holds logical chunk (l%8) ^ ((col >> 1) & 7), col = 8u + l/8
#pragma unroll
        for (int uu = 0; uu < kTileLoads; ++uu) {
            const int u = u0 + uu;
            const int tcol = 8 * u + (lane >> 3);
            const int col = wcol(tcol);
            vb[uu] = (col < N ? col : n0) * Kb + 16 * ((lane & 7) ^ ((tcol >> 1) & 7));
        }
        // scale bytes (col, 32-block 4ks + b) of [N, K/64, 2]: the aligned
        // dword at col * KS + 4 ks holds the step's four
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int cj = wcol(32 * j + c);
            vsb[j] = (cj < N ? cj : n0) * KS;
        }
        vsb[2] = vsb[3] = 0;
    }

    // (the upstream step has no row_index / logit)
    const RowInfo rinfo = OP == 0 ? load_row_info<RF, I8>(p, m0, mcount) : RowInfo{};
    constexpr int NA = KN4 || SPLIT || I8 ? 8 : 4;   // accumulators per row fragment
    using Acc = std::conditional_t<I8, v16i, v16f>;
    Acc acc[RF][NA];
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int j = 0; j < NA; ++j) acc[f][j] = Acc{};
    int rsum[RF] = {};   // W4A8: sum of this lane's x1 bytes (its row, its K halves)
    ColScales cscale;
    if constexpr (I8) cscale = load_col_scales(p, e, n0);
    // bytes of an x1 row per step: FP8 [K,N] 64, FP4 [K,N] 32, [N,K] 128 (the
    // [N,K] weight column moves the same 128 bytes)
    constexpr int kStepA = KN ? (FP4 ? kStepK / 2 : kStepK) : kStepKNK;
    constexpr int kAL = KN ? (FP4 ? 1 : 2) : 4;      // x1 loads per step
    // WS ([N, K], 4-slot ring; K >= 512): the x1 and weight scales are loaded
    // once per window of four steps, 16 bytes per x1 row and per weight
    // column (the four steps' dwords) instead of a gather per step: each load
    // instruction touches 32 rows, so this is 4x fewer scattered cache-line
    // accesses.  The window load goes first in the load
    // group of the window's first step (item-relative steps 4m, a multiple of
    // the ring depth), into the "next" register set, which becomes "current"
    // after the window's last step; a window that would run past the row's
    // end starts earlier (still 16 bytes inside the row) and the steps' dword
    // index is shifted by the difference.
    static_assert(!WS || (!I8 && !KN && D == 4), "windowed scales: [N, K], 4 slots");
    constexpr int kSA = I8 || WS ? 0 : 1;            // x1-scale loads per step and fragment
    constexpr int kSB = I8 || (WS && !KN) ? 0 : KN4 ? 8 : KN ? 4 : 2;   // weight-scale loads per step
    constexpr int kXW = WS ? RF + 2 : 0;   // loads per window
    // 32-element scale blocks per step and row: [K,N] 2, [N,K] 4
    constexpr int kBlk = KN ? 2 : 4;
    StepRegs<kAL, RF, (kSB > 0 ? kSB : 1)> regs[D];

    // hf: SPLIT's tile of virtual step vs (0 gate, 1 up) = vs & 1, passed as
    // the unrolled ring index's parity so that it is a compile-time constant
    // (ks0 * 2 and D are even; for the clamped re-reads past the last step it
    // may differ, and those are never consumed)
    // WS: scale windows, [0] current, [1] next
    v4i wsa[2][RF], wsb[2][2];
    int wdl[2] = {0, 0};   // WS: step shift of a window moved back from the row end
    // steps of a whole row; each takes kBlk scale bytes of it
    const int k_row = K / (KN ? kStepK : kStepKNK);
    auto wload = [&](int vs, int set) {   // the window starting at step vs
        const int start = vs < k_row - 4 ? vs : k_row - 4;
        wdl[set] = vs - start;
#pragma unroll
        for (int f = 0; f < RF; ++f)
            wsa[set][f] = __builtin_amdgcn_raw_buffer_load_b128(rsa, vsa[f] + kBlk * start, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            wsb[set][j] = __builtin_amdgcn_raw_buffer_load_b128(rsb, vsb[j] + kBlk * start, 0, 0);
    };

    // The weight-tile loads of a step (into LDS slot `slot`).
    auto issue_tile = [&](int vs, int slot, int hf) {
        const int ks = SPLIT ? vs >> 1 : vs;       // K step of virtual step vs
        const int k0 = ks * kStepA;
        __builtin_amdgcn_sched_barrier(0);
        // (the instruction's immediate offset would move both addresses, so
        // each 1 KB destination gets its own LDS pointer)
#pragma unroll
        for (int uu = 0; uu < kTileLoads; ++uu) {
            const int u = u0 + uu;
            lds_void_t *dst = (lds_void_t *)(ring + slot * kSlotBytes + u * 1024);
            if (KN)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, dst, 16, vb[KN4 ? (u & 1) : SPLIT ? hf : 0], (ks * kStepK + 8 * u) * Nb,
                    0, NT ? kNonTemporal : 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, vb[uu], k0, 0, NT ? kNonTemporal : 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // The register loads of a step: the window's scales (WS, first step of a
    // window), x1 bytes and scales (into register set `slot`).
    auto issue_regs = [&](int vs, int slot, int hf, bool wstart) {
        const int ks = SPLIT ? vs >> 1 : vs;       // K step of virtual step vs
        const int k0 = ks * kStepA;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (WS) {
            if (wstart) wload(vs, 1);
        }
        StepRegs<kAL, RF, (kSB > 0 ? kSB : 1)> &r = regs[slot];
#pragma unroll
        for (int f = 0; f < RF; ++f)
#pragma unroll
            for (int q = 0; q < kAL; ++q)
                r.a[f][q] = __builtin_amdgcn_raw_buffer_load_b128(ra, va[f], k0 + 32 * q, 0);
        // x1 scale bytes of the step: [K,N] (2 ks + g) & 3 of the dword at
        // (2 ks) & ~3; [N,K] the step's kBlk bytes at kBlk ks
#pragma unroll
        for (int f = 0; f < RF * kSA; ++f)
            r.sa[f][0] = __builtin_amdgcn_raw_buffer_load_b32(rsa, vsa[f],
                                                              KN ? (2 * ks) & ~3 : kBlk * ks, 0);
#pragma unroll
        for (int j = 0; j < kSB; ++j)
            r.sb[j][0] = __builtin_amdgcn_raw_buffer_load_b32(
                rsb, SPLIT ? vsb[4 * hf + j] : vsb[j], KN ? ks * 2 * N : kBlk * ks, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // B operands of one step in registers, double-buffered across steps.
    using BTile = std::conditional_t<KN, v2i[16], v4i[8]>;
    BTile bt[2];
    // [N,K] reads: 64-K half s, 16-byte half h of the lane's 32 operand bytes
    // = logical chunk 4s + 2h + g of column 32j + c (column c's slot row at
    // 128 c, group j 4 KB further)
    uint32_t nk_off[4] = {0, 0, 0, 0};
    if (!KN) {
        const int f = (c >> 1) & 7;
#pragma unroll
        for (int sh = 0; sh < 4; ++sh)
            nk_off[sh] = c * 128 + 16 * ((2 * sh + g) ^ f);   // sh = 2s + h
    }
    auto read_b = [&](int slot, BTile &b) {
        const uint32_t base = lds_addr(ring + slot * kSlotBytes);
        if constexpr (KN4) {
            uint32_t a[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = base + tr_addr[j];
            lds_issue_kn4(a, b);
        } else if constexpr (KN) {
            const uint32_t a[4] = {base + tr_addr[0], base + tr_addr[1], base + tr_addr[2],
                                   base + tr_addr[3]};
            lds_issue_kn(a, b);
        } else {
            const uint32_t a[4] = {base + nk_off[0], base + nk_off[1], base + nk_off[2],
                                   base + nk_off[3]};
            lds_issue_nk(a, b);
        }
    };

    auto mma = [&](int slot, const BTile &b, bool live, int vs, int hf, int wpos) {
        const int ks = SPLIT ? vs >> 1 : vs;
        StepRegs<kAL, RF, (kSB > 0 ? kSB : 1)> &r = regs[slot];
        // padding rows and padding steps (re-reads past the last K step)
        // multiply a zero operand
#pragma unroll
        for (int f = 0; f < RF; ++f) {
            const bool on = arow_ok[f] && live;
            if constexpr (I8) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {   // the two 32-K halves of the step
                    const v4i a = on ? r.a[f][h2] : v4i{};
                    rsum[f] = __builtin_amdgcn_sdot4(a.x, 0x01010101, rsum[f], false);
                    rsum[f] = __builtin_amdgcn_sdot4(a.y, 0x01010101, rsum[f], false);
                    rsum[f] = __builtin_amdgcn_sdot4(a.z, 0x01010101, rsum[f], false);
                    rsum[f] = __builtin_amdgcn_sdot4(a.w, 0x01010101, rsum[f], false);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const v4i bw = {b[4 * j + 2 * h2].x, b[4 * j + 2 * h2].y,
                                        b[4 * j + 2 * h2 + 1].x, b[4 * j + 2 * h2 + 1].y};
                        const v4i m = {static_cast<int>(0xF0F0F0F0u), static_cast<int>(0xF0F0F0F0u),
                                       static_cast<int>(0xF0F0F0F0u), static_cast<int>(0xF0F0F0F0u)};
                        acc[f][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bw & m, acc[f][j], 0, 0, 0);
                        acc[f][4 + j] =
                            __builtin_amdgcn_mfma_i32_32x32x32_i8(a, (bw << 4) & m, acc[f][4 + j], 0, 0, 0);
                    }
                }
            } else if constexpr (KN4) {
                // one 64-K step, eight 32-column groups; 16-byte operands
                const v4i z = {0, 0, 0, 0};
                const v8i a = on ? cat(r.a[f][0], z) : v8i{};
                const uint32_t sa = r.sa[f][0] >> (8 * (2 * (ks & 1) + g));
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const v8i bj = {b[2 * j].x, b[2 * j].y, b[2 * j + 1].x, b[2 * j + 1].y,
                                    0, 0, 0, 0};
                    acc[f][j] = mfma<FMT, 0>(a, bj, acc[f][j], sa, r.sb[j][0] >> sb_shift);
                }
            } else if constexpr (KN) {
                const v8i a = on ? cat(r.a[f][0], r.a[f][1]) : v8i{};
                // byte (2 ks + g) & 3 of the x1 scale dword
                const uint32_t sa = r.sa[f][0] >> (8 * (2 * (ks & 1) + g));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v8i bj = {b[4 * j].x,     b[4 * j].y,     b[4 * j + 1].x, b[4 * j + 1].y,
                                    b[4 * j + 2].x, b[4 * j + 2].y, b[4 * j + 3].x, b[4 * j + 3].y};
                    if constexpr (SPLIT) {
                        if (hf)
                            acc[f][4 + j] = mfma<FMT, 0>(a, bj, acc[f][4 + j], sa,
                                                         r.sb[j][0] >> sb_shift);
                        else
                            acc[f][j] = mfma<FMT, 0>(a, bj, acc[f][j], sa, r.sb[j][0] >> sb_shift);
                    } else {
                        acc[f][j] = mfma<FMT, 0>(a, bj, acc[f][j], sa, r.sb[j][0] >> sb_shift);
                    }
                }
            } else {
                // two 64-K halves s, two 32-column groups j; the scale of
                // 32-block 4 ks + 2 s + g is byte 2 s + g of each scale dword
                uint32_t sa = r.sa[f][0], sb[2] = {r.sb[0][0], r.sb[1][0]};
                if constexpr (WS) {
                    sa = pick(wsa[0][f], wpos + wdl[0]);
                    sb[0] = pick(wsb[0][0], wpos + wdl[0]);
                    sb[1] = pick(wsb[0][1], wpos + wdl[0]);
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    v8i a = on ? cat(r.a[f][2 * s2], r.a[f][2 * s2 + 1]) : v8i{};
                    const int shf = 8 * (2 * s2 + g);
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[f][j] = mfma<FMT, 0>(a, cat(b[2 * (2 * s2) + j], b[2 * (2 * s2 + 1) + j]),
                                                 acc[f][j], sa >> shf, sb[j] >> shf);
                }
            }
        }
    };

    // Vector-memory instructions per step (one group), in issue order:
    // x1 (2 or 4), x1 scale (1), weight scales (4 or 2), weight tile (all 8,
    // or this wave's 2); [N, K] (kTileFirst) issues the weight tile first,
    // and only MFMAs come between it and the rest, so the groups stay
    // contiguous.  Every iteration issues the same
    // groups (past the last step the last step is re-read; those are L2 hits
    // and are never consumed), so each wait is a constant count of later
    // groups allowed to be pending.  The ring has D slots and the prologue
    // fills all of them; iteration i
    //   waits until step i + 1 has landed (D - 2 later groups pending);
    //   [cooperative: s_barrier, so every wave's share of step i + 1 is in
    //   and every wave has finished reading step i's slot];
    //   issues the LDS reads of step i + 1;
    //   [N, K]: refills step i's slot with step i + D's weight tile;
    //   runs step i's MFMAs (operands read in the previous iteration);
    //   refills step i's registers with step i + D's x1 bytes and scales
    //   ([K, N]: then step i's slot with step i + D's weight tile);
    //   waits for the LDS reads of step i + 1.
    // WS adds the kXW window loads to the group of every item-relative step
    // 4m >= 4 (issued in iterations with d = 0): the wait in iteration d = 1
    // or 2 has one such group among the two later ones.
    constexpr int kOpsPerStep = RF * (kAL + kSA) + kSB + kTileLoads;
    constexpr bool kTileFirst = !KN;
    static_assert((D - 1) * kOpsPerStep < 64 && (D - 2) * kOpsPerStep + kXW < 64, "vmcnt range");
    static_assert(D % 2 == 0, "operand double buffer alternates with the slot index");
    const int n_steps = (ks1 - ks0) * kVS;        // virtual steps
    // [N, K] wave items: rotated K order (windows of four steps)
    const int rot = !KN && !COOP ? k_rotation(e, n_steps, WS ? 4 : 1) : 0;
    auto step_of = [&](int i) {
        const int j = (i < n_steps ? i : n_steps - 1) + rot;
        return ks0 * kVS + (j < n_steps ? j : j - n_steps);
    };

    if constexpr (WS) wload(step_of(0), 0);   // older than every step's loads
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if constexpr (kTileFirst) issue_tile(step_of(d), d, d & 1);
        issue_regs(step_of(d), d, d & 1, false);
        if constexpr (!kTileFirst) issue_tile(step_of(d), d, d & 1);
    }
    wait_vmcnt<(D - 1) * kOpsPerStep>();
    if (COOP) __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_b(0, bt[0]);
    lds_wait(bt[0]);
    for (int i0 = 0; i0 < n_steps; i0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = i0 + d;
            if (WS && (d == 1 || d == 2))
                wait_vmcnt<(D - 2) * kOpsPerStep + kXW>();
            else
                wait_vmcnt<(D - 2) * kOpsPerStep>();
            if (COOP) __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_b((d + 1) % D, bt[(d + 1) & 1]);
            // [N, K]: slot d was read into registers last iteration (and, in
            // a cooperative unit, by every wave: the barrier above), so its
            // refill goes out before this step's MFMAs, which would otherwise
            // hold it back (a wave issues in order); the register loads of
            // step i + D follow the MFMAs that consume register set d.
            // [K, N] measured faster with the whole group after the MFMAs.
            if constexpr (kTileFirst) issue_tile(step_of(i + D), d, d & 1);
            mma(d, bt[d & 1], i < n_steps, step_of(i), d & 1, d);
            __builtin_amdgcn_sched_barrier(0);
            issue_regs(step_of(i + D), d, d & 1, d == 0);
            if constexpr (!kTileFirst) issue_tile(step_of(i + D), d, d & 1);
            lds_wait(bt[(d + 1) & 1]);
            if constexpr (WS) {
                if (d == 3) {   // the next window becomes current
#pragma unroll
                    for (int f = 0; f < RF; ++f) wsa[0][f] = wsa[1][f];
                    wsb[0][0] = wsb[1][0];
                    wsb[0][1] = wsb[1][1];
                    wdl[0] = wdl[1];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // Drain the trailing re-reads before the ring is reused.
    wait_vmcnt<0>();
    if constexpr (OP == 1)
        epilogue_swiglu<SPLIT ? 8 : 2, RF, NA>(p, acc, m0, mcount, n0);
    else if constexpr (I8)
        epilogue_w4a8<RF>(p, acc, rsum, cscale, m0, n0, store_rows, rinfo);
    else if constexpr (KN && !COOP && RF == 1 && OP == 0) {
        if (split)
            split_epilogue<NA>(p, acc, m0, n0, store_rows, rinfo, split);
        else
            epilogue<NA, 1, NA>(p, acc, m0, n0, store_rows, rinfo);
    } else
        epilogue<KN4 ? 8 : KN ? 4 : 2, RF, NA>(p, acc, m0, n0, store_rows, rinfo);
}

// ---------------------------------------------------------------------------
// Cooperative unit for FP8 and MXFP4 [N, K] weights (finalize operator): RF x
// 128 rows of one expert (wave w: rows [32 RF w, 32 RF (w + 1)) of the group)
// x 128 columns, in K steps of 128 bytes of a row (128 K, MXFP4 256 K: two
// elements per byte).  Every operand is staged through LDS with
// direct-to-LDS loads of whole 128-byte lines -- one load covers 8 rows (or
// columns) x 128 B, so each line is requested once per step -- where a
// register gather of the MFMA layout touches 32 rows x 32 B per load, and a
// 64-K step leaves every line to be requested twice.  A stage holds the
// step's 128 weight columns (16 KB) and the four waves' x1 rows (RF x 32 x
// 128 B each); both use the [N, K] wave items' slot layout (128-byte rows,
// 16-byte chunks XOR-swizzled by (row >> 1) & 7) and operand reads.  Two
// stages: a step's loads are issued right after the barrier that frees its
// stage, before the previous step's 16 (RF 2) MFMAs, which cover their
// latency.  Scales: one 16-byte load per x1 row and weight column per four
// steps (MXFP4: two, eight scale bytes a step) (WS), or per-step dwords
// (MXFP4: qwords) for shorter K ranges.
// ---------------------------------------------------------------------------
constexpr int kCkStages = 2;
constexpr int kCkWSlot = kTileN * kStepKNK;   // 16 KB: 128 columns x 128 K

// Operand reads of one 64-K half s of a step, reads h = 0, 1 (logical chunk
// 4s + 2h + g of row c: bytes 32 h + 16 g of the half), issued without
// waiting: t[2j + h] = weight column group j (columns 32j..), t[8 + 2f + h]
// = x1 fragment f (rows 32f..); wa* / xa* = slot base + the lane's row
// offset for h = 0, 1.
template <int NT>
__device__ __forceinline__ void lds_issue_w8(uint32_t wa0, uint32_t wa1, v4i (&t)[NT]) {
    static_assert(32 * kStepKNK == 4096 && NT >= 8, "group stride; eight reads");
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %8 offset:4096\n\t"
        "ds_read_b128 %3, %9 offset:4096\n\t"
        "ds_read_b128 %4, %8 offset:8192\n\t"
        "ds_read_b128 %5, %9 offset:8192\n\t"
        "ds_read_b128 %6, %8 offset:12288\n\t"
        "ds_read_b128 %7, %9 offset:12288"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]),
          "=&v"(t[6]), "=&v"(t[7])
        : "v"(wa0), "v"(wa1)
        : "memory");
}

template <int RF, int NT>
__device__ __forceinline__ void lds_issue_ck(uint32_t wa0, uint32_t wa1, uint32_t xa0,
                                             uint32_t xa1, v4i (&t)[NT]) {
    static_assert(NT >= 8 + 2 * RF, "operand buffer holds the reads");
    lds_issue_w8(wa0, wa1, t);
    if constexpr (RF == 2)
        asm volatile(
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %5\n\t"
            "ds_read_b128 %2, %4 offset:4096\n\t"
            "ds_read_b128 %3, %5 offset:4096"
            : "=&v"(t[8]), "=&v"(t[9]), "=&v"(t[10]), "=&v"(t[11])
            : "v"(xa0), "v"(xa1)
            : "memory");
    else
        asm volatile(
            "ds_read_b128 %0, %2\n\t"
            "ds_read_b128 %1, %3"
            : "=&v"(t[8]), "=&v"(t[9])
            : "v"(xa0), "v"(xa1)
            : "memory");
}

template <int N>
__device__ __forceinline__ void lds_wait_all(v4i (&t)[N]) {
    static_assert(N == 8 || N == 10 || N == 12, "operand buffer of one half step");
    if constexpr (N == 8)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]),
                       "+v"(t[6]), "+v"(t[7])
                     :
                     : "memory");
    else if constexpr (N == 12)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]),
                       "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11])
                     :
                     : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]),
                       "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9])
                     :
                     : "memory");
}

template <int FMT, int RF, bool WS>
__device__ __forceinline__ void ck_unit(const FusedParams &p, int e, int m0, int mcount, int n0,
                                        int ks0, int ks1, bool store_rows, char *ring, int w) {
    // Stages: the weight tile two (16 KB each), the x1 rows three with scale
    // windows (K >= 512) -- x1 is two thirds of a step's bytes, so its loads
    // go out two steps ahead -- or two without.
    constexpr int DW = kCkStages;
    constexpr int DX = WS ? 3 : 2;
    constexpr int kXSlot = RF * kTileM * kStepKNK;                // one wave's x1 per step
    constexpr int kXStage = kWavesPerBlock * kXSlot;              // 32 KB (RF 2), 16 KB (RF 1)
    static_assert(DW * kCkWSlot + DX * kXStage <= kWavesPerBlock * kRingBytes,
                  "stages fit the block's LDS ring");
    constexpr int kWLd = kCkWSlot / 1024 / kWavesPerBlock;        // weight loads per wave: 4
    constexpr int kXLd = kXSlot / 1024;                           // x1 loads per wave: 4 RF
    constexpr int kNH = 8 + 2 * RF;                               // operand reads per half step
    // MXFP4: a step is 128 bytes of a row = 256 K (8 scale bytes), so a
    // 16-byte scale window covers two steps instead of four
    constexpr bool FP4 = FMT == 4;
    constexpr int kWin = FP4 ? 2 : 4;                             // steps per scale window
    constexpr int kScW = FP4 ? 2 : 1;                             // scale dwords per step
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mcount = __builtin_amdgcn_readfirstlane(mcount);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    ks0 = __builtin_amdgcn_readfirstlane(ks0);
    ks1 = __builtin_amdgcn_readfirstlane(ks1);
    w = __builtin_amdgcn_readfirstlane(w);
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    const int K = p.K, N = p.N, KS = p.K / 32;
    const int Kb = FP4 ? K / 2 : K;    // bytes of an x1 row / a weight column
    if (mcount < 0) mcount = 0;
    // x1 rows of this wave (rows past the expert's last token read as zero
    // through the range-checked descriptor), the expert's weights, the scales
    const rsrc_t ra = make_rsrc(p.x1 + static_cast<int64_t>(m0) * Kb, static_cast<int64_t>(mcount) * Kb);
    const rsrc_t rsa = make_rsrc(p.pts + static_cast<int64_t>(m0) * KS, static_cast<int64_t>(mcount) * KS);
    const int64_t wbytes = static_cast<int64_t>(N) * Kb;
    const rsrc_t rb = make_rsrc(p.x2 + e * wbytes, wbytes);
    const rsrc_t rsb = make_rsrc(p.scale + e * p.scale_e_stride, static_cast<int64_t>(KS) * N);
    // load v of 8 rows (columns): row 8v + l/8 fills physical chunk l%8 of its
    // slot row, which holds logical chunk (l%8) ^ ((row >> 1) & 7) =
    // (l%8) ^ ((4v + l/16) & 7).  Columns past N re-read column n0.
    int vw[kWLd], vx[kXLd];
#pragma unroll
    for (int uu = 0; uu < kWLd; ++uu) {
        const int u = w * kWLd + uu;
        const int col = n0 + 8 * u + (lane >> 3);
        vw[uu] = (col < N ? col : n0) * Kb + 16 * ((lane & 7) ^ ((4 * u + (lane >> 4)) & 7));
    }
#pragma unroll
    for (int v = 0; v < kXLd; ++v)
        vx[v] = (8 * v + (lane >> 3)) * Kb + 16 * ((lane & 7) ^ ((4 * v + (lane >> 4)) & 7));
    uint32_t o[4];
#pragma unroll
    for (int sh = 0; sh < 4; ++sh) o[sh] = c * kStepKNK + 16 * ((2 * sh + g) ^ ((c >> 1) & 7));
    // scale rows: x1 row 32f + c (row 0 past the last token: its operand is
    // zero), weight column 32j + c; each holds the step's four (FP4: eight)
    // bytes
    int vsa[RF], vsb[4];
#pragma unroll
    for (int f = 0; f < RF; ++f)
        vsa[f] = (kTileM * f + c < mcount ? kTileM * f + c : 0) * KS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + 32 * j + c;
        vsb[j] = (col < N ? col : n0) * KS;
    }
    const RowInfo rinfo = load_row_info<RF>(p, m0, mcount);
    v16f acc[RF][4];
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[f][j] = v16f{};

    const int k_row = Kb / kStepKNK;
    const int n_steps = ks1 - ks0;
    auto step_of = [&](int i) { return ks0 + (i < n_steps ? i : n_steps - 1); };
    // WS: scale windows of kWin steps, [0] current / [1] next; wdl = shift
    // of a window moved back from the row end
    v4i wa[2][RF], wb[2][4];
    int wdl[2] = {0, 0};
    auto wload = [&](int ks, int set) {
        const int start = ks < k_row - kWin ? ks : k_row - kWin;
        wdl[set] = ks - start;
#pragma unroll
        for (int f = 0; f < RF; ++f)
            wa[set][f] =
                __builtin_amdgcn_raw_buffer_load_b128(rsa, vsa[f] + 4 * kScW * start, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            wb[set][j] =
                __builtin_amdgcn_raw_buffer_load_b128(rsb, vsb[j] + 4 * kScW * start, 0, 0);
    };
    // per-step scale dwords (no WS), register set = weight stage
    uint32_t sa_r[DW][RF][kScW], sb_r[DW][4][kScW];
    char *const wring = ring;                                  // DW weight stages
    char *const xring = ring + DW * kCkWSlot + w * kXSlot;     // this wave's DX x1 slots
    auto issue_w = [&](int ks, int ws) {
        char *st = wring + ws * kCkWSlot;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int uu = 0; uu < kWLd; ++uu)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void_t *)(st + (w * kWLd + uu) * 1024), 16, vw[uu], ks * kStepKNK, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto issue_x = [&](int ks, int xs) {
        char *st = xring + xs * kXStage;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < kXLd; ++v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t *)(st + v * 1024), 16, vx[v],
                                                     ks * kStepKNK, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto issue_scales = [&](int ks, int set) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < RF; ++f) {
            if constexpr (FP4) {
                const v2i v = __builtin_amdgcn_raw_buffer_load_b64(rsa, vsa[f], 8 * ks, 0);
                sa_r[set][f][0] = static_cast<uint32_t>(v.x);
                sa_r[set][f][1] = static_cast<uint32_t>(v.y);
            } else {
                sa_r[set][f][0] = __builtin_amdgcn_raw_buffer_load_b32(rsa, vsa[f], 4 * ks, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (FP4) {
                const v2i v = __builtin_amdgcn_raw_buffer_load_b64(rsb, vsb[j], 8 * ks, 0);
                sb_r[set][j][0] = static_cast<uint32_t>(v.x);
                sb_r[set][j][1] = static_cast<uint32_t>(v.y);
            } else {
                sb_r[set][j][0] = __builtin_amdgcn_raw_buffer_load_b32(rsb, vsb[j], 4 * ks, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // operands of half s of the step in weight stage ws / x1 stage xs
    // LF: fragments of this wave with live rows (a constant of the loop
    // instance); the others' reads and MFMAs are skipped
    auto read_half = [&](int ws, int xs, int s2, v4i (&t)[kNH], auto lf_c) {
        constexpr int LF = decltype(lf_c)::value;
        if constexpr (LF > 0) {
            const uint32_t wbase = lds_addr(wring + ws * kCkWSlot);
            const uint32_t xbase = lds_addr(xring + xs * kXStage);
            lds_issue_ck<LF>(wbase + o[2 * s2], wbase + o[2 * s2 + 1], xbase + o[2 * s2],
                             xbase + o[2 * s2 + 1], t);
        }
    };
    v4i hb[2][kNH];   // [0]: half 0 of a step, [1]: half 1
    // (x1 rows past the expert's last token are zero in LDS: the DMA reads
    // them through the range-checked descriptor)
    // FP8: the half is one 64-K MFMA per (f, j), lane (c, g) holding bytes
    // 16g and 32 + 16g of it; the scale of 32-block 2 s + g is byte 2 s + g
    // of the step's dword.  FP4: the half is 128 K, two MFMAs h, lane (c, g)
    // holding 16 bytes = K [64h + 32g, +32) of it (the chunk the FP8 read
    // gives as its 2h-th); the scale of 32-block 4 s + 2 h + g is byte 2 h + g
    // of the step's dword s.
    auto mma_half = [&](const v4i (&t)[kNH], int s2, int set, int wpos, auto lf_c) {
        constexpr int LF = decltype(lf_c)::value;
        const int sw = kScW * (wpos + wdl[0]) + (FP4 ? s2 : 0);   // window dword
        uint32_t sa[RF], sb[4];
#pragma unroll
        for (int f = 0; f < RF; ++f) {
            sa[f] = sa_r[set][f][FP4 ? s2 : 0];
            if constexpr (WS) sa[f] = pick(wa[0][f], sw);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sb[j] = sb_r[set][j][FP4 ? s2 : 0];
            if constexpr (WS) sb[j] = pick(wb[0][j], sw);
        }
        // the scales of fragments without live rows, consumed where their
        // MFMAs would be (keep_loaded)
#pragma unroll
        for (int f = LF; f < RF; ++f) {
            if constexpr (WS)
                keep_loaded(wa[0][f]);
            else
                keep_loaded(sa_r[set][f][FP4 ? s2 : 0]);
        }
        if constexpr (LF == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (WS)
                    keep_loaded(wb[0][j]);
                else
                    keep_loaded(sb_r[set][j][FP4 ? s2 : 0]);
            }
        }
        if constexpr (FP4) {
            const v4i z = {0, 0, 0, 0};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int shf = 8 * (2 * h + g);
#pragma unroll
                for (int f = 0; f < LF; ++f) {
                    const v8i a = cat(t[8 + 2 * f + h], z);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[f][j] = mfma<FMT, 0>(a, cat(t[2 * j + h], z), acc[f][j],
                                                 sa[f] >> shf, sb[j] >> shf);
                }
            }
        } else {
            const int shf = 8 * (2 * s2 + g);
#pragma unroll
            for (int f = 0; f < LF; ++f) {
                const v8i a = cat(t[8 + 2 * f], t[8 + 2 * f + 1]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[f][j] = mfma<FMT, 0>(a, cat(t[2 * j], t[2 * j + 1]), acc[f][j],
                                             sa[f] >> shf, sb[j] >> shf);
            }
        }
    };

    // Prologue.  WS: window 0, then weights and x1 of step 0, weights and x1
    // of step 1, x1 of step 2, so that in every iteration the youngest group
    // in flight is the x1 two steps ahead.  Without WS: two steps, each with
    // its per-step scales.
    if constexpr (WS) {
        wload(step_of(0), 0);
        issue_w(step_of(0), 0);
        issue_x(step_of(0), 0);
        issue_w(step_of(1), 1);
        issue_x(step_of(1), 1);
        issue_x(step_of(2), 2);
        wait_vmcnt<kWLd + 2 * kXLd>();
    } else {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            issue_w(step_of(d), d);
            issue_x(step_of(d), d);
            issue_scales(step_of(d), d);
        }
        wait_vmcnt<kWLd + kXLd + RF + 4>();
    }
    static_assert(kWLd + 2 * kXLd < 64 && kWLd + kXLd + RF + 4 < 64, "vmcnt range");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // A wave without live rows in a fragment still moves its share of every
    // step (the loads, waits and barriers are the block's) but reads and
    // multiplies only its live fragments.
    auto main_loop = [&](auto lf_c) {
        read_half(0, 0, 0, hb[0], lf_c);
        lds_wait_all(hb[0]);
        // Iteration i (half 0 of step i already in hb[0]; xs = x1 stage of step i):
        //   read half 1; half 0's MFMAs; wait for the reads;
        //   wait for step i + 1 (WS: everything but the x1 of step i + 2) and
        //   barrier: every wave's share of step i + 1 is in and every wave has
        //   read all of step i; read half 0 of step i + 1; refill: weights of step
        //   i + 2 into step i's weight stage (WS: with the next window when step
        //   i + 2 starts one), x1 of step i + DX into step i's x1 stage; half 1's
        //   MFMAs; per-step scales of step i + 2 into the set just consumed; wait
        //   for the reads.
        int xs = 0;
        for (int i0 = 0; i0 < n_steps; i0 += DW) {
#pragma unroll
            for (int d = 0; d < DW; ++d) {
                const int i = i0 + d;
                const bool live = i < n_steps;
                const int xn = xs + 1 == DX ? 0 : xs + 1;   // x1 stage of step i + 1
                read_half(d, xs, 1, hb[1], lf_c);
                if (live) mma_half(hb[0], 0, d, i & (kWin - 1), lf_c);   // padding steps: none
                lds_wait_all(hb[1]);
                if constexpr (WS)
                    wait_vmcnt<kXLd>();
                else
                    wait_vmcnt<0>();
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                read_half((d + 1) % DW, xn, 0, hb[0], lf_c);
                if constexpr (WS) {
                    if (((i + 2) & (kWin - 1)) == 0) wload(step_of(i + 2), 1);
                }
                issue_w(step_of(i + 2), d);
                issue_x(step_of(i + DX), xs);
                if (live) mma_half(hb[1], 1, d, i & (kWin - 1), lf_c);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!WS) issue_scales(step_of(i + 2), d);
                lds_wait_all(hb[0]);
                if constexpr (WS) {
                    if ((i & (kWin - 1)) == kWin - 1) {   // the next window becomes current
#pragma unroll
                        for (int f = 0; f < RF; ++f) wa[0][f] = wa[1][f];
#pragma unroll
                        for (int j = 0; j < 4; ++j) wb[0][j] = wb[1][j];
                        wdl[0] = wdl[1];
                    }
                }
                xs = xn;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    if (mcount > (RF - 1) * kTileM)
        main_loop(IntC<RF>{});
    else if (RF == 2 && mcount > 0)
        main_loop(IntC<1>{});
    else
        main_loop(IntC<0>{});
    wait_vmcnt<0>();   // the trailing re-reads, before the stages are reused
    epilogue<4, RF, 4>(p, acc, m0, n0, store_rows, rinfo);
}

// ---------------------------------------------------------------------------
// Cooperative unit for FP8 [K, N] weights (finalize operator): ck_unit's
// structure -- RF x 128 rows of one expert x 128 columns in K steps of 128,
// two weight stages, two or three x1 stages, the x1 rows staged through LDS
// as whole 128-byte lines -- with the [K, N] weight tile: a stage holds the
// step's 128 K rows x 128 bytes as two 64-K halves of the [K, N] slot layout
// (16-byte chunks of row r XOR-swizzled by 2 ((r >> 1) & 3)), moved by 16
// direct-to-LDS loads of 8 K rows (four per wave; every K row segment of the
// tile is one 128-byte line), and read K-contiguous per column with
// transposing reads.  Against the 64-K cooperative units each x1 line is
// requested once per step instead of twice.  Weight scales ([K/64, N, 2]):
// the step's two 64-K rows, per-step dwords loaded with the weights; x1
// scales: ck_unit's windows of four steps (WS) or per-step dwords.
// ---------------------------------------------------------------------------
template <int FMT, int RF, bool WS>
__device__ __forceinline__ void kc_unit(const FusedParams &p, int e, int m0, int mcount, int n0,
                                        int ks0, int ks1, bool store_rows, char *ring, int w) {
    constexpr int DW = kCkStages;
    constexpr int DX = WS ? 3 : 2;
    constexpr int kXSlot = RF * kTileM * kStepKNK;                // one wave's x1 per step
    constexpr int kXStage = kWavesPerBlock * kXSlot;
    static_assert(DW * kCkWSlot + DX * kXStage <= kWavesPerBlock * kRingBytes,
                  "stages fit the block's LDS ring");
    constexpr int kWLd = kCkWSlot / 1024 / kWavesPerBlock;        // weight loads per wave: 4
    constexpr int kXLd = kXSlot / 1024;                           // x1 loads per wave: 4 RF
    constexpr int kSbLd = 8;                                      // weight-scale dwords per step
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mcount = __builtin_amdgcn_readfirstlane(mcount);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    ks0 = __builtin_amdgcn_readfirstlane(ks0);
    ks1 = __builtin_amdgcn_readfirstlane(ks1);
    w = __builtin_amdgcn_readfirstlane(w);
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    const int K = p.K, N = p.N, KS = p.K / 32;
    if (mcount < 0) mcount = 0;
    const rsrc_t ra = make_rsrc(p.x1 + static_cast<int64_t>(m0) * K, static_cast<int64_t>(mcount) * K);
    const rsrc_t rsa = make_rsrc(p.pts + static_cast<int64_t>(m0) * KS, static_cast<int64_t>(mcount) * KS);
    const int64_t wbytes = static_cast<int64_t>(K) * N;
    const rsrc_t rb = make_rsrc(p.x2 + e * wbytes, wbytes);
    const rsrc_t rsb = make_rsrc(p.scale + e * p.scale_e_stride, static_cast<int64_t>(KS) * N);
    // weight load u (u = 4w + uu): K row 8u + l/8 of the step (row offset in
    // the scalar offset); it fills physical chunk l%8 of its slot row, which
    // holds logical chunk (l%8) ^ 2 ((l >> 4) & 3); columns past N re-read n0
    const int chunk_col = n0 + 16 * ((lane & 7) ^ (2 * ((lane >> 4) & 3)));
    const int vw = (lane >> 3) * N + (chunk_col < N ? chunk_col : n0);
    // x1 load v of 8 rows: ck_unit's
    int vx[kXLd];
#pragma unroll
    for (int v = 0; v < kXLd; ++v)
        vx[v] = (8 * v + (lane >> 3)) * K + 16 * ((lane & 7) ^ ((4 * v + (lane >> 4)) & 7));
    uint32_t o[4];   // x1 operand reads (ck_unit's)
#pragma unroll
    for (int sh = 0; sh < 4; ++sh) o[sh] = c * kStepKNK + 16 * ((2 * sh + g) ^ ((c >> 1) & 7));
    // transposing reads of a 64-K half: lane s of 16-lane group G reads K row
    // 16g + (s >> 1) (+ the read's offset), columns 32j + 16(G & 1) + 8(s & 1)
    uint32_t tr[4];
    {
        const int G = lane >> 4, sl = lane & 15, ii = sl >> 1, h = sl & 1;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            tr[j] = (16 * g + ii) * kTileN + 16 * ((2 * j + (G & 1)) ^ (2 * ((ii >> 1) & 3))) + 8 * h;
    }
    // scale rows: x1 row 32f + c (row 0 past the last token: its operand is
    // zero); weight scale dword of (64-K row, column pair of 32j + c)
    int vsa[RF], vsb[4];
#pragma unroll
    for (int f = 0; f < RF; ++f)
        vsa[f] = (kTileM * f + c < mcount ? kTileM * f + c : 0) * KS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + 32 * j + c;
        vsb[j] = ((col < N ? col : n0) & ~1) * 2;
    }
    const int sb_shift = 8 * (2 * (c & 1) + g);
    const RowInfo rinfo = load_row_info<RF>(p, m0, mcount);
    v16f acc[RF][4];
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[f][j] = v16f{};

    const int k_row = K / kStepKNK;
    const int n_steps = ks1 - ks0;
    auto step_of = [&](int i) { return ks0 + (i < n_steps ? i : n_steps - 1); };
    v4i wa[2][RF];   // WS: x1 scale windows, [0] current / [1] next
    int wdl[2] = {0, 0};
    auto wload = [&](int ks, int set) {
        const int start = ks < k_row - 4 ? ks : k_row - 4;
        wdl[set] = ks - start;
#pragma unroll
        for (int f = 0; f < RF; ++f)
            wa[set][f] = __builtin_amdgcn_raw_buffer_load_b128(rsa, vsa[f] + 4 * start, 0, 0);
    };
    uint32_t sa_r[DW][RF], sb_r[DW][2][4];   // per-step scale dwords, set = weight stage
    char *const wring = ring;
    char *const xring = ring + DW * kCkWSlot + w * kXSlot;
    // the weight tile of step ks into stage ws
    auto issue_w = [&](int ks, int ws) {
        char *st = wring + ws * kCkWSlot;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int uu = 0; uu < kWLd; ++uu) {
            const int u = w * kWLd + uu;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void_t *)(st + u * 1024), 16, vw, (ks * kStepKNK + 8 * u) * N, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // its scales into register set ws (issued after the MFMAs that still
    // read that set)
    auto issue_sc = [&](int ks, int ws) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sb_r[ws][h][j] = __builtin_amdgcn_raw_buffer_load_b32(rsb, vsb[j],
                                                                      (2 * ks + h) * 2 * N, 0);
        if constexpr (!WS) {
#pragma unroll
            for (int f = 0; f < RF; ++f)
                sa_r[ws][f] = __builtin_amdgcn_raw_buffer_load_b32(rsa, vsa[f], 4 * ks, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto issue_x = [&](int ks, int xs) {
        char *st = xring + xs * kXStage;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < kXLd; ++v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t *)(st + v * 1024), 16, vx[v],
                                                     ks * kStepKNK, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // operands of half s2 of the step in weight stage ws / x1 stage xs
    struct Half {
        v8i b[4];
        v8i a[RF];
    };
    // LF: fragments of this wave with live rows (a constant of the loop
    // instance); the others' reads and MFMAs are skipped
    auto read_half = [&](int ws, int xs, int s2, Half &t, auto lf_c) {
        constexpr int LF = decltype(lf_c)::value;
        if constexpr (LF == 0) return;
        char *wb = wring + ws * kCkWSlot + s2 * (kStepK * kTileN);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lds_v2i_t *q = (lds_v2i_t *)(wb + tr[j]);
            const v2i r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(q);
            const v2i r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(q + 1024 / 8);
            const v2i r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(q + 4096 / 8);
            const v2i r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(q + 5120 / 8);
            t.b[j] = v8i{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
        }
        char *xb = xring + xs * kXStage;
#pragma unroll
        for (int f = 0; f < LF; ++f) {
            const v4i lo = *reinterpret_cast<const __attribute__((address_space(3))) v4i *>(
                (lds_void_t *)(xb + f * 4096 + o[2 * s2]));
            const v4i hi = *reinterpret_cast<const __attribute__((address_space(3))) v4i *>(
                (lds_void_t *)(xb + f * 4096 + o[2 * s2 + 1]));
            t.a[f] = cat(lo, hi);
        }
    };
    Half hb[2];   // [0]: half 0 of a step, [1]: half 1
    auto mma_half = [&](const Half &t, int s2, int set, int wpos, auto lf_c) {
        constexpr int LF = decltype(lf_c)::value;
        const int shf = 8 * (2 * s2 + g);
        // the scales of fragments without live rows, consumed where their
        // MFMAs would be (keep_loaded)
#pragma unroll
        for (int f = LF; f < RF; ++f) {
            if constexpr (WS)
                keep_loaded(wa[0][f]);
            else
                keep_loaded(sa_r[set][f]);
        }
        if constexpr (LF == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) keep_loaded(sb_r[set][s2][j]);
        }
#pragma unroll
        for (int f = 0; f < LF; ++f) {
            uint32_t sa = 0;
            if constexpr (WS)
                sa = pick(wa[0][f], wpos + wdl[0]);
            else
                sa = sa_r[set][f];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[f][j] = mfma<FMT, 0>(t.a[f], t.b[j], acc[f][j], sa >> shf,
                                         sb_r[set][s2][j] >> sb_shift);
        }
    };

    // Prologue (ck_unit's): WS: window 0, then weights and x1 of step 0,
    // weights and x1 of step 1, x1 of step 2; without: two steps.
    // (scale loads are register loads: the compiler waits for them before
    // their use; the explicit waits count them only as later loads)
    constexpr int kSc = kSbLd + (WS ? 0 : RF);   // scale loads per step
    if constexpr (WS) {
        wload(step_of(0), 0);
        issue_w(step_of(0), 0);
        issue_sc(step_of(0), 0);
        issue_x(step_of(0), 0);
        issue_w(step_of(1), 1);
        issue_sc(step_of(1), 1);
        issue_x(step_of(1), 1);
        issue_x(step_of(2), 2);
        wait_vmcnt<kWLd + kSc + 2 * kXLd>();
    } else {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            issue_w(step_of(d), d);
            issue_sc(step_of(d), d);
            issue_x(step_of(d), d);
        }
        wait_vmcnt<kWLd + kSc + kXLd>();
    }
    static_assert(kWLd + kSc + 2 * kXLd < 64 && kXLd + kSc < 64, "vmcnt range");
    lds_reads_done();
    __builtin_amdgcn_s_barrier();
    lds_reads_done();
    __builtin_amdgcn_sched_barrier(0);
    // Iteration i (ck_unit's order): read half 1; half 0's MFMAs; wait for
    // step i + 1 and barrier; read half 0 of step i + 1; refill: weights of
    // step i + 2 into step i's weight stage (WS: with the next window when
    // step i + 2 starts one), x1 of step i + DX into step i's x1 stage; half
    // 1's MFMAs; step i + 2's scales into the register set just consumed.
    // A wave without live rows in a fragment still moves its share of every
    // step (the loads, waits and barriers are the block's) but reads and
    // multiplies only its live fragments.
    auto main_loop = [&](auto lf_c) {
        read_half(0, 0, 0, hb[0], lf_c);
        int xs = 0;
        for (int i0 = 0; i0 < n_steps; i0 += DW) {
#pragma unroll
            for (int d = 0; d < DW; ++d) {
                const int i = i0 + d;
                const bool live = i < n_steps;
                const int xn = xs + 1 == DX ? 0 : xs + 1;
                read_half(d, xs, 1, hb[1], lf_c);
                if (live) mma_half(hb[0], 0, d, i & 3, lf_c);
                // step i + 1's tile and x1 are in: pending may be the scales of
                // step i + 1 (issued last) and, WS, the x1 of step i + 2
                if constexpr (WS)
                    wait_vmcnt<kXLd + kSc>();
                else
                    wait_vmcnt<kSc>();
                lds_reads_done();   // this wave's reads of step i are done ...
                __builtin_amdgcn_s_barrier();   // ... and every wave's: its stages may be refilled
                lds_reads_done();
                __builtin_amdgcn_sched_barrier(0);
                read_half((d + 1) % DW, xn, 0, hb[0], lf_c);
                if constexpr (WS) {
                    if (((i + 2) & 3) == 0) wload(step_of(i + 2), 1);
                }
                issue_w(step_of(i + 2), d);
                issue_x(step_of(i + DX), xs);
                if (live) mma_half(hb[1], 1, d, i & 3, lf_c);
                __builtin_amdgcn_sched_barrier(0);
                issue_sc(step_of(i + 2), d);
                if constexpr (WS) {
                    if ((i & 3) == 3) {   // the next window becomes current
#pragma unroll
                        for (int f = 0; f < RF; ++f) wa[0][f] = wa[1][f];
                        wdl[0] = wdl[1];
                    }
                }
                xs = xn;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    if (mcount > (RF - 1) * kTileM)
        main_loop(IntC<RF>{});
    else if (RF == 2 && mcount > 0)
        main_loop(IntC<1>{});
    else
        main_loop(IntC<0>{});
    wait_vmcnt<0>();   // the trailing re-reads, before the stages are reused
    epilogue<4, RF, 4>(p, acc, m0, n0, store_rows, rinfo);
}

// ---------------------------------------------------------------------------
// Wave item for FP8 and MXFP4 [N, K] weights (finalize operator, experts
// below the cooperative size): 32 tokens x 128 columns, K steps of 128 bytes
// of a row (MXFP4: 256 K), one wave.
// The weight tile moves global -> LDS in the cooperative units' slot layout
// (16 loads of 8 columns x 128 B per step, two 16 KB stages per wave);
// the x1 rows go to registers in the MFMA layout (four 32-row gathers per
// step, each line's four 32-byte pieces in one step).  Against 64-column
// items, each x1 row is gathered once per 128 columns instead of 64.  A
// step's loads are issued before the second half of the previous step's
// MFMAs; the wave's other loads in flight and the block's other three waves
// keep the memory system busy meanwhile.
// ---------------------------------------------------------------------------
// split: as for routed_item.
template <int FMT, bool WS, bool NT = false>
__device__ __forceinline__ void cw_item(const FusedParams &p, int e, int m0, int mcount, int n0,
                                        int ks0, int ks1, bool store_rows, char *ring,
                                        char *split) {
    constexpr int D = kCkStages;
    static_assert(D * kCkWSlot <= kRingBytes, "a wave's stages fit its ring");
    constexpr int kWLd = kCkWSlot / 1024;   // 16 weight loads per step
    constexpr bool FP4 = FMT == 4;          // 128 bytes a step = 256 K, 8 scale bytes
    constexpr int kWin = FP4 ? 2 : 4;       // steps per 16-byte scale window
    constexpr int kScW = FP4 ? 2 : 1;       // scale dwords per step
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mcount = __builtin_amdgcn_readfirstlane(mcount);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    ks0 = __builtin_amdgcn_readfirstlane(ks0);
    ks1 = __builtin_amdgcn_readfirstlane(ks1);
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    const int K = p.K, N = p.N, KS = p.K / 32;
    const int Kb = FP4 ? K / 2 : K;         // bytes of an x1 row / a weight column
    if (mcount < 0) mcount = 0;
    const rsrc_t ra = make_rsrc(p.x1 + static_cast<int64_t>(m0) * Kb, static_cast<int64_t>(mcount) * Kb);
    const rsrc_t rsa = make_rsrc(p.pts + static_cast<int64_t>(m0) * KS, static_cast<int64_t>(mcount) * KS);
    const int64_t wbytes = static_cast<int64_t>(N) * Kb;
    const rsrc_t rb = make_rsrc(p.x2 + e * wbytes, wbytes);
    const rsrc_t rsb = make_rsrc(p.scale + e * p.scale_e_stride, static_cast<int64_t>(KS) * N);
    // load u of 8 columns: column n0 + 8u + l/8 (lane offset below, 8u rows in
    // the scalar offset; columns past N lie past the expert's slice and read as
    // zero), physical chunk l%8 holding logical chunk (l%8) ^ ((4u + l/16) & 7)
    int vw[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        vw[par] = (n0 + (lane >> 3)) * Kb + 16 * ((lane & 7) ^ ((4 * par + (lane >> 4)) & 7));
    uint32_t o[4];
#pragma unroll
    for (int sh = 0; sh < 4; ++sh) o[sh] = c * kStepKNK + 16 * ((2 * sh + g) ^ ((c >> 1) & 7));
    // x1: lane (c, g) gathers row c's bytes 32q + 16g of the step (rows past
    // the last token read as zero); its scales sit in row c (row 0 past it)
    const int arow = c < mcount ? c : 0;
    const int va = arow * Kb + 16 * g;
    const int vsa = arow * KS;
    int vsb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + 32 * j + c;
        vsb[j] = (col < N ? col : n0) * KS;
    }
    const RowInfo rinfo = load_row_info<1>(p, m0, mcount);
    v16f acc[1][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[0][j] = v16f{};

    const int k_row = Kb / kStepKNK;
    const int n_steps = ks1 - ks0;
    const int rot = k_rotation(e, n_steps, WS ? kWin : 1);
    auto step_of = [&](int i) {   // rotated; past the range: the last step again
        const int j = (i < n_steps ? i : n_steps - 1) + rot;
        return ks0 + (j < n_steps ? j : j - n_steps);
    };
    v4i wa[2], wb[2][4];   // WS windows of kWin steps: [0] current, [1] next
    int wdl[2] = {0, 0};
    auto wload = [&](int ks, int set) {
        const int start = ks < k_row - kWin ? ks : k_row - kWin;
        const int off = 4 * kScW * start;
        wdl[set] = ks - start;
        if (set) {
            wa[1] = __builtin_amdgcn_raw_buffer_load_b128(rsa, vsa + off, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wb[1][j] = __builtin_amdgcn_raw_buffer_load_b128(rsb, vsb[j] + off, 0, 0);
        } else {
            wa[0] = __builtin_amdgcn_raw_buffer_load_b128(rsa, vsa + off, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wb[0][j] = __builtin_amdgcn_raw_buffer_load_b128(rsb, vsb[j] + off, 0, 0);
        }
    };
    v4i xr[D][4];                             // x1 operands of a step, register set = stage
    uint32_t sa_r[D][kScW], sb_r[D][4][kScW];  // per-step scale dwords (no WS)
    auto issue_dma = [&](int ks, int stage) {
        char *st = ring + stage * kCkWSlot;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kWLd; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t *)(st + u * 1024), 16,
                                                     vw[u & 1], 8 * u * Kb + ks * kStepKNK, 0,
                                                     NT ? kNonTemporal : 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto issue_regs = [&](int ks, int set) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xr[set][q] = __builtin_amdgcn_raw_buffer_load_b128(ra, va, ks * kStepKNK + 32 * q, 0);
        if constexpr (!WS && FP4) {
            const v2i v = __builtin_amdgcn_raw_buffer_load_b64(rsa, vsa, 8 * ks, 0);
            sa_r[set][0] = static_cast<uint32_t>(v.x);
            sa_r[set][1] = static_cast<uint32_t>(v.y);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v2i u = __builtin_amdgcn_raw_buffer_load_b64(rsb, vsb[j], 8 * ks, 0);
                sb_r[set][j][0] = static_cast<uint32_t>(u.x);
                sb_r[set][j][1] = static_cast<uint32_t>(u.y);
            }
        } else if constexpr (!WS) {
            sa_r[set][0] = __builtin_amdgcn_raw_buffer_load_b32(rsa, vsa, 4 * ks, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sb_r[set][j][0] = __builtin_amdgcn_raw_buffer_load_b32(rsb, vsb[j], 4 * ks, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto read_half = [&](int stage, int s2, v4i (&t)[8]) {
        const uint32_t base = lds_addr(ring + stage * kCkWSlot);
        lds_issue_w8(base + o[2 * s2], base + o[2 * s2 + 1], t);
    };
    v4i hb[2][8];
    // operands and scale bytes as in ck_unit's halves (FP4: two MFMAs h per
    // half, x1 bytes 32 h + 16 g of the half = xr[2 s + h])
    auto mma_half = [&](const v4i (&t)[8], int s2, int set, int wpos) {
        const int sw = kScW * (wpos + wdl[0]) + (FP4 ? s2 : 0);   // window dword
        uint32_t sa = sa_r[set][FP4 ? s2 : 0], sb[4];
        if constexpr (WS) sa = pick(wa[0], sw);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sb[j] = sb_r[set][j][FP4 ? s2 : 0];
            if constexpr (WS) sb[j] = pick(wb[0][j], sw);
        }
        if constexpr (FP4) {
            const v4i z = {0, 0, 0, 0};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int shf = 8 * (2 * h + g);
                const v8i a = cat(xr[set][2 * s2 + h], z);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[0][j] = mfma<FMT, 0>(a, cat(t[2 * j + h], z), acc[0][j], sa >> shf,
                                             sb[j] >> shf);
            }
        } else {
            const int shf = 8 * (2 * s2 + g);
            const v8i a = cat(xr[set][2 * s2], xr[set][2 * s2 + 1]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[0][j] = mfma<FMT, 0>(a, cat(t[2 * j], t[2 * j + 1]), acc[0][j], sa >> shf,
                                         sb[j] >> shf);
        }
    };

    if constexpr (WS) wload(step_of(0), 0);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        issue_dma(step_of(d), d);
        issue_regs(step_of(d), d);
    }
    constexpr int kOps = kWLd + 4 + (WS ? 0 : 5);
    static_assert((D - 1) * kOps < 64, "vmcnt range");
    wait_vmcnt<(D - 1) * kOps>();
    __builtin_amdgcn_sched_barrier(0);
    read_half(0, 0, hb[0]);
    lds_wait_all(hb[0]);
    // Iteration i (half 0 of step i already in hb[0]): read half 1; half 0's
    // MFMAs; wait for the reads and for step i + 1 (all loads issued so far);
    // read half 0 of step i + 1; refill step i's stage with step i + 2 (WS:
    // with the next window when step i + 2 starts one); half 1's MFMAs; x1 and
    // scales of step i + 2 into the register set just consumed.
    for (int i0 = 0; i0 < n_steps; i0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = i0 + d;
            const bool live = i < n_steps;
            read_half(d, 1, hb[1]);
            if (live) mma_half(hb[0], 0, d, i & (kWin - 1));
            lds_wait_all(hb[1]);
            wait_vmcnt<0>();
            __builtin_amdgcn_sched_barrier(0);
            read_half((d + 1) % D, 0, hb[0]);
            if constexpr (WS) {
                if (((i + D) & (kWin - 1)) == 0) wload(step_of(i + D), 1);
            }
            issue_dma(step_of(i + D), d);
            if (live) mma_half(hb[1], 1, d, i & (kWin - 1));
            __builtin_amdgcn_sched_barrier(0);
            issue_regs(step_of(i + D), d);
            lds_wait_all(hb[0]);
            if constexpr (WS) {
                if ((i & (kWin - 1)) == kWin - 1) {   // the next window becomes current
                    wa[0] = wa[1];
#pragma unroll
                    for (int j = 0; j < 4; ++j) wb[0][j] = wb[1][j];
                    wdl[0] = wdl[1];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vmcnt<0>();
    if (split)
        split_epilogue(p, acc, m0, n0, store_rows, rinfo, split);
    else
        epilogue<4, 1, 4>(p, acc, m0, n0, store_rows, rinfo);
}

// ---------------------------------------------------------------------------
// Wave item for FP8 [K, N] weights (finalize operator, experts below the
// cooperative size): 32 tokens x 128 columns, K steps of 128, one wave.
// A step's weight tile is 128 K rows x 128 B (16 KB: two 64-K halves of the
// [K, N] slot layout, rows' 16-byte chunks XOR-swizzled by 2 ((r >> 1) & 3)),
// moved by 16 direct-to-LDS loads of 8 rows x 128 B and read K-contiguous
// with ds_read_b64_tr_b8 one 64-K half at a time; the x1 rows are gathered
// into registers, each row's 128-byte line once per step (with 64-K steps
// the line is requested twice: the 32 KB L1 does not keep it between steps).
// Two 16 KB stages per wave, loads of step i + 2 issued before the second
// half of step i's MFMAs.  Weight scales: the step's two [K/64, N, 2] rows
// per column group (one line each); x1 scales: windows of four steps.
// ---------------------------------------------------------------------------
template <int FMT, bool WS, bool NT = false>
__device__ __forceinline__ void kw_item(const FusedParams &p, int e, int m0, int mcount, int n0,
                                        int ks0, int ks1, bool store_rows, char *ring,
                                        char *split) {
    constexpr int D = kCkStages;
    constexpr int kSlot = kStepKNK * kTileN;   // 16 KB
    static_assert(D * kSlot <= kRingBytes, "a wave's stages fit its ring");
    constexpr int kWLd = kSlot / 1024;         // 16 weight loads per step
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mcount = __builtin_amdgcn_readfirstlane(mcount);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    ks0 = __builtin_amdgcn_readfirstlane(ks0);
    ks1 = __builtin_amdgcn_readfirstlane(ks1);
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    const int K = p.K, N = p.N, KS = p.K / 32;
    if (mcount < 0) mcount = 0;
    const rsrc_t ra = make_rsrc(p.x1 + static_cast<int64_t>(m0) * K, static_cast<int64_t>(mcount) * K);
    const rsrc_t rsa = make_rsrc(p.pts + static_cast<int64_t>(m0) * KS, static_cast<int64_t>(mcount) * KS);
    const int64_t wbytes = static_cast<int64_t>(K) * N;
    const rsrc_t rb = make_rsrc(p.x2 + e * wbytes, wbytes);
    const rsrc_t rsb = make_rsrc(p.scale + e * p.scale_e_stride, static_cast<int64_t>(KS) * N);
    // load u, lane l: K row 8u + l/8 of the step (row offset in the scalar
    // offset), physical chunk l%8 of the slot row holding logical chunk
    // (l%8) ^ 2 ((r >> 1) & 3) = (l%8) ^ 2 ((l >> 4) & 3); columns past N re-read
    // column n0
    const int chunk_col = n0 + 16 * ((lane & 7) ^ (2 * ((lane >> 4) & 3)));
    const int vw = (lane >> 3) * N + (chunk_col < N ? chunk_col : n0);
    // transpose reads of a 64-K half (see lds_issue_kn): lane s of 16-lane
    // group G reads K row 16g + (s >> 1) (+ the read's offset), columns
    // 32j + 16(G & 1) + 8(s & 1)
    uint32_t tr[4];
    {
        const int G = lane >> 4, sl = lane & 15, ii = sl >> 1, h = sl & 1;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            tr[j] = (16 * g + ii) * kTileN + 16 * ((2 * j + (G & 1)) ^ (2 * ((ii >> 1) & 3))) + 8 * h;
    }
    // x1: lane (c, g) gathers row c's bytes 32q + 16g of the step (rows past
    // the last token read as zero); scales of row c (row 0 past it)
    const int arow = c < mcount ? c : 0;
    const int va = arow * K + 16 * g;
    const int vsa = arow * KS;
    // weight scale byte (64-block b, col, g) is byte 2 col + g of row b of
    // [K/64, N, 2]; the aligned dword holds columns col & ~1 and col | 1
    int vsb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = n0 + 32 * j + c;
        vsb[j] = ((col < N ? col : n0) & ~1) * 2;
    }
    const int sb_shift = 8 * (2 * (c & 1) + g);
    const RowInfo rinfo = load_row_info<1>(p, m0, mcount);
    v16f acc[1][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[0][j] = v16f{};

    const int k_row = K / kStepKNK;
    const int n_steps = ks1 - ks0;
    auto step_of = [&](int i) { return ks0 + (i < n_steps ? i : n_steps - 1); };
    v4i wa[2];          // WS: x1 scale windows of four steps, [0] current, [1] next
    int wdl[2] = {0, 0};
    auto wload = [&](int ks, int set) {
        const int start = ks < k_row - 4 ? ks : k_row - 4;
        wdl[set] = ks - start;
        if (set)
            wa[1] = __builtin_amdgcn_raw_buffer_load_b128(rsa, vsa + 4 * start, 0, 0);
        else
            wa[0] = __builtin_amdgcn_raw_buffer_load_b128(rsa, vsa + 4 * start, 0, 0);
    };
    v4i xr[D][4];                     // x1 operands of a step, register set = stage
    uint32_t sa_r[D], sb_r[D][2][4];   // x1 scale dword (no WS); weight scales, 64-K half h
    auto issue_dma = [&](int ks, int stage) {
        char *st = ring + stage * kSlot;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kWLd; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t *)(st + u * 1024), 16, vw,
                                                     (ks * kStepKNK + 8 * u) * N, 0,
                                                     NT ? kNonTemporal : 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto issue_regs = [&](int ks, int set) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xr[set][q] = __builtin_amdgcn_raw_buffer_load_b128(ra, va, ks * kStepKNK + 32 * q, 0);
        if constexpr (!WS) sa_r[set] = __builtin_amdgcn_raw_buffer_load_b32(rsa, vsa, 4 * ks, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sb_r[set][h][j] = __builtin_amdgcn_raw_buffer_load_b32(rsb, vsb[j],
                                                                       (2 * ks + h) * 2 * N, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // B operands of a 64-K half: column group j from four transposing reads
    // (K rows +0, +8, +32, +40 of the lane's start row: byte offsets 0,
    // 1024, 4096, 5120), built in place as the MFMA's eight registers (the
    // compiler's own read, so it places the waits and the registers)
    auto read_half = [&](int stage, int s2, v8i (&t)[4]) {
        char *base = ring + stage * kSlot + s2 * (kStepK * kTileN);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lds_v2i_t *q = (lds_v2i_t *)(base + tr[j]);
            const v2i r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(q);
            const v2i r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(q + 1024 / 8);
            const v2i r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(q + 4096 / 8);
            const v2i r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(q + 5120 / 8);
            t[j] = v8i{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
        }
    };
    v8i hb[2][4];
    auto mma_half = [&](const v8i (&b)[4], int s2, int set, int wpos) {
        // x1 scale: byte 2 s + g of the step's dword (windowed: of the
        // window's dword for this step)
        uint32_t sa = sa_r[set];
        if constexpr (WS) sa = pick(wa[0], wpos + wdl[0]);
        sa >>= 8 * (2 * s2 + g);
        const v8i a = cat(xr[set][2 * s2], xr[set][2 * s2 + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[0][j] = mfma<FMT, 0>(a, b[j], acc[0][j], sa, sb_r[set][s2][j] >> sb_shift);
    };

    if constexpr (WS) wload(step_of(0), 0);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        issue_dma(step_of(d), d);
        issue_regs(step_of(d), d);
    }
    constexpr int kOps = kWLd + 4 + 8 + (WS ? 0 : 1);
    static_assert((D - 1) * kOps < 64, "vmcnt range");
    wait_vmcnt<(D - 1) * kOps>();
    __builtin_amdgcn_sched_barrier(0);
    read_half(0, 0, hb[0]);
    // Iteration i (half 0 of step i already in hb[0]): read half 1; half 0's
    // MFMAs; wait for the reads and for step i + 1 (all loads issued so far);
    // read half 0 of step i + 1; refill step i's stage with step i + 2 (WS:
    // with the next window when step i + 2 starts one); half 1's MFMAs; x1
    // and scales of step i + 2 into the register set just consumed.
    for (int i0 = 0; i0 < n_steps; i0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = i0 + d;
            const bool live = i < n_steps;
            read_half(d, 1, hb[1]);
            if (live) mma_half(hb[0], 0, d, i & 3);
            wait_vmcnt<0>();
            lds_reads_done();   // stage d's reads are done before its refill below
            __builtin_amdgcn_sched_barrier(0);
            read_half((d + 1) % D, 0, hb[0]);
            if constexpr (WS) {
                if (((i + D) & 3) == 0) wload(step_of(i + D), 1);
            }
            issue_dma(step_of(i + D), d);
            if (live) mma_half(hb[1], 1, d, i & 3);
            __builtin_amdgcn_sched_barrier(0);
            issue_regs(step_of(i + D), d);
            if constexpr (WS) {
                if ((i & 3) == 3) {   // the next window becomes current
                    wa[0] = wa[1];
                    wdl[0] = wdl[1];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vmcnt<0>();
    if (split)
        split_epilogue(p, acc, m0, n0, store_rows, rinfo, split);
    else
        epilogue<4, 1, 4>(p, acc, m0, n0, store_rows, rinfo);
}

// Shared-expert term out[off + r, n] += w * shared_input[r, n], as one
// contiguous slice of the R*N elements per wave, so every wave carries the
// same small share (done after its routed work).  Lane l handles elements
// 64i + l of the slice: every load and atomic covers 64 adjacent elements.
__device__ __forceinline__ void shared_slice(const FusedParams &p, int64_t wave, int64_t waves) {
    const int lane = lane_id();
    const int64_t total = static_cast<int64_t>(p.shared_rows) * p.N;
    int64_t per = (total + waves - 1) / waves;
    per = (per + kWaveSize - 1) / kWaveSize * kWaveSize;
    const int64_t begin = wave * per;
    const int64_t end = begin + per < total ? begin + per : total;
    float *o = p.out + static_cast<int64_t>(p.shared_off) * p.N;
    constexpr int kBatch = 16;   // loads in flight per lane before their atomics
    for (int64_t b = begin; b < end; b += kBatch * kWaveSize) {
        // a descriptor over the rest of the slice: loads past it return 0
        const int64_t left = end - b;
        const rsrc_t rs = make_rsrc(p.shared + b, 2 * (left < kBatch * kWaveSize ? left : kBatch * kWaveSize));
        uint16_t h[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            h[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * (i * kWaveSize + lane), 0, 0);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int64_t e = b + i * kWaveSize + lane;
            if (e < end)
                unsafeAtomicAdd(o + e, p.shared_w * __uint_as_float(static_cast<uint32_t>(h[i]) << 16));
        }
    }
}

// One block per CU (the weight rings fill most of the 160 KB of LDS).
//
// Work is dealt in block units: the cooperative units of the large experts
// (expert, 128- or 256-row group, column tile, K split) and the wave items of
// the small experts (expert, 32-row tile, column tile, K split), four
// consecutive ones per unit, one per wave.  Each kind is dealt to the blocks
// round-robin, and every block alternates between its units of the two kinds.
//
// OP 0 is the finalize-routing operator; OP 1 the upstream step, whose items
// cover a 128- ([K,N]) or 32-column ([N,K]) block of the I outputs (twice that
// many weight columns: gate and up) and always the whole K range (its
// epilogue is not linear, so there is no K split).
template <int FMT, bool TRANS, int OP>
__device__ __forceinline__ void run_units(const FusedParams &p) {
    __shared__ int s_start[kMaxExperts];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_spref[kMaxExperts + 1];
    __shared__ int s_wperm[kMaxExperts];
    __shared__ int s_lpref[kMaxExperts + 1];
    __shared__ __attribute__((aligned(16))) int s_perm[kMaxExperts];
    __shared__ int64_t s_scan[kBlockThreads];
    __shared__ __attribute__((aligned(16))) char s_ring[kWavesPerBlock * kRingBytes];

    // columns per item: [N, K] 64, [K, N] 128 (FP8) or 256 (FP4)
    constexpr int kTN = TRANS ? kTileNNK : (FMT == 4 || FMT == 8 ? 2 * kTileN : kTileN);
    // output columns per item: the weight columns, or for the upstream step
    // half of them ([N,K]: gate and up columns in one tile) or all of them
    // ([K,N]: gate and up tiles streamed in turn)
    // FP8 and MXFP4 [N, K] finalize: ck_unit / cw_item, 128-column tiles for
    // both kinds
    constexpr bool kTB = TRANS && (FMT == 0 || FMT == 1 || FMT == 4) && OP == 0;
    constexpr int kOutN = kTB ? kTileN : OP == 0 || !TRANS ? kTN : kTN / 2;
    const int n_tiles = ((OP == 0 ? p.N : p.I) + kOutN - 1) / kOutN;
    constexpr int kOutNC = kOutN;                   // output columns per cooperative unit
    const int n_tiles_c = n_tiles;
    WorkList wl{s_start, s_cnt, s_spref, s_wperm, s_lpref, s_perm, 0, 0, 0, 0, 0};
    // two-fragment cooperative groups except where a fragment has 8
    // accumulators (MXFP4 and W4A8 [K, N], the upstream step with [K, N])
    constexpr bool kWide = FMT != 8 && !(OP == 1 && !TRANS) && (FMT != 4 || TRANS);
    build_work_list<kWide>(p, n_tiles, n_tiles_c, wl, s_scan);
    if (OP == 0 && p.det_total && blockIdx.x == 0 && threadIdx.x == 0)
        *p.det_total = wl.routed_tokens;

    const bool store_rows = OP == 0 && p.wbuf != nullptr;
    // [N, K]: windowed scale loads in the 4-slot-ring items (the upstream
    // step's; a window is four 128-K steps of a row's scale bytes: K >= 512)
    constexpr bool kWS = TRANS && FMT != 8;
    const bool ws_ok = kWS && p.K >= 4 * kStepKNK;
    // K elements per step: 64 ([K,N]), 128 ([N,K] FP8), 256 ([N,K] FP4): one
    // step always moves 8 KB of the weight tile
    const int k_steps = p.K / (!TRANS ? kStepK : FMT == 4 ? 2 * kStepKNK : kStepKNK);
    const int k_steps_c = k_steps;                          // steps of a cooperative unit
    // FP8 [K, N] finalize beside cooperative units: wave items are kw_item's,
    // in K steps of 128 (half the x1 requests per weight byte; the x1 rows
    // compete with the cooperative units' for the L2; c4 444 -> 426 µs).
    // Without cooperative units they are routed_item's, whose four 8 KB
    // slots keep more weight bytes in flight (c3 189 against 192 µs).
    constexpr bool kKW = !TRANS && (FMT == 0 || FMT == 1) && OP == 0;
    const bool kw_on = kKW && wl.litems > 0;
    const int k_steps_w = p.K / kStepKNK;
    const bool wsc_tb = p.K >= 4 * kStepKNK;                // ck_unit: a window of four steps
    const int blocks = gridDim.x;
    int S = p.split_k;
    const int base_units = wl.litems + (wl.sitems + kWavesPerBlock - 1) / kWavesPerBlock;
    if (OP == 1 || store_rows) {
        S = 1;
    } else if (S <= 0) {
        // Enough K splits to give every block a unit (long K runs stream
        // best, and every split adds a set of atomics), keeping >= 8 K steps
        // each.
        S = base_units > 0 ? blocks / base_units : 1;
        S = S < k_steps / 8 ? S : k_steps / 8;
        S = S > 1 ? S : 1;
    }
    S = S < k_steps ? S : k_steps;
    // Unit and item numbers below are 32-bit: keep (items) x S under 2^30
    // (the host bounds the items; only an explicit split could reach it).
    while (S > 1 && static_cast<int64_t>(wl.litems + wl.sitems) * S >= (int64_t{1} << 30)) S >>= 1;
    // Block-split wave units (FP8 finalize, only wave items, K split into a
    // multiple of four ranges): the four waves of a unit take four K ranges
    // of one item and add their partial sums in LDS before the scatter
    // (split_epilogue), so each output element gets one atomic per four
    // ranges.  c1 (16 tokens per expert, four ranges) spends a fifth of its
    // time in atomics otherwise.  An explicit split that is not a multiple of
    // four keeps one item per wave.
    constexpr bool kSplitOK = OP == 0 && (FMT == 0 || FMT == 1 || FMT == 4);
    const bool bsplit = kSplitOK && !store_rows && wl.litems == 0 && S >= kWavesPerBlock &&
                        (p.split_k <= 0 || p.split_k % kWavesPerBlock == 0);
    if (bsplit) S -= S % kWavesPerBlock;
    const int coop_units = static_cast<int>(wl.litems) * S;
    const int wave_items = static_cast<int>(wl.sitems) * S;
    const int units = coop_units + (wave_items + kWavesPerBlock - 1) / kWavesPerBlock;

    // Everything that selects a work item is wave-uniform; readfirstlane makes
    // that visible to the compiler so buffer descriptors and row offsets live
    // in SGPRs (otherwise each buffer load becomes a waterfall loop).
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Workgroups are dealt to the 8 XCDs round-robin.  Cooperative units are
    // taken in an XCD-grouped order (consecutive units on one XCD): the row
    // groups of one column tile then share its weights, and the column tiles
    // of one row group its x1 rows, through that XCD's L2 (without it the
    // large experts' weights are read from HBM once per row group).  Wave
    // units are taken in plain order (measured faster for streaming: each XCD
    // then reads many experts' weights at once).
    const int xcd_block =
        (blocks % 8 == 0) ? static_cast<int>(blockIdx.x % 8) * (blocks / 8) + blockIdx.x / 8
                          : blockIdx.x;
    const int waves = static_cast<int>(blocks) * kWavesPerBlock;
    // One-fragment cooperative units (no snake deal) take ranks in chunks of
    // 16 per XCD: ranks 16c .. 16c + 15 are blocks of XCD c mod 8.  Sixteen
    // consecutive units (the row groups of a band over four column tiles)
    // still share one XCD's L2, and when there are more units than blocks
    // the blocks that also take a wave unit spread over the XCDs instead of
    // filling the first ones (g1_llada 146 -> 134 µs, c4_fp4 -1 %).
    const int coop_rank =
        (blocks % 128 == 0)
            ? ((static_cast<int>(blockIdx.x / 8) / 16) * 8 + static_cast<int>(blockIdx.x % 8)) * 16 +
                  static_cast<int>(blockIdx.x / 8) % 16
            : xcd_block;

    // The deal.  With two-fragment cooperative units present, units g = 0,
    // 1, ... (the cooperative units in the order of the work list, experts
    // with the most rows per group first, then the wave units) go to ranks in
    // snake order -- round k = g / blocks runs over the ranks forward when k
    // is even and backward when it is odd -- so that every rank gets costly
    // and cheap units alike (a cooperative unit's time grows with its live
    // rows: c4 523 -> 501 µs, c5 2355 -> 2278).  Ranks are XCD-grouped
    // (consecutive ranks on one XCD, so consecutive cooperative units share
    // an L2).  Otherwise (one-fragment cooperative units, where the snake
    // measured slower, or none) the cooperative units go round-robin over
    // ranks in XCD chunks of 16 (coop_rank) and the wave units round-robin in
    // plain block order (measured fastest for pure streaming).
    // A block alternates between its cooperative and its wave units (even
    // blocks start with a cooperative unit, odd ones with a wave unit):
    // cooperative units hardly use HBM (their weights are shared through L2)
    // and wave units stream it, so mixing them keeps HBM busy while the
    // cooperative work proceeds (c5 2412 -> 2369 µs, c5_fp4 1732 -> 1619,
    // c4 516 -> 506 against all cooperative units first).  Block parity is
    // XCD parity, so at a given time an XCD runs mostly one kind; starting
    // half of each XCD's blocks with each kind (parity of blockIdx / 8 or
    // / 16) measured slower: c5 +1.4-3.5 %, c4 +1.5-2.5 %.
    //
    // A last round with at most half as many units as blocks would leave the
    // other blocks idle for a whole unit (c4: 896 units, 3.5 per block, so
    // half the blocks ran a fourth one).  In atomic finalize mode each of its
    // units is cut into K ranges instead (tT = blocks / units left, or tT + 1
    // for the last ones so that every rank gets a piece; at least eight K
    // steps each) and the pieces fill the round; a piece adds its partial
    // sums like any K split.  The deal is over positions: positions below
    // R * blocks (R full rounds) are units, the next ones the pieces of the
    // last round's units in order (unit_of).
    const bool snake = kWide && coop_units > 0;
    const bool tail_ok = OP == 0 && !store_rows && !bsplit;
    auto tail_factor = [&](int n) -> int {   // pieces per unit of n's last round
        const int left = n % blocks;
        if (!tail_ok || left == 0 || 2 * left > blocks) return 1;
        const int t = blocks / left;
        const int kmax = (k_steps / S) / 8;
        return static_cast<int>(t < kmax ? t : kmax) > 1 ? static_cast<int>(t < kmax ? t : kmax) : 1;
    };
    // the split sequence: the single snake sequence, or the wave units when
    // there are no cooperative ones
    const int seq_n = snake ? units : coop_units == 0 ? units : 0;
    const int tT = seq_n > 0 ? tail_factor(seq_n) : 1;
    const int seq_full = seq_n / blocks * blocks;
    // The cut round's pieces fill every rank: its last t_x units get one
    // piece more (tT + 1) where a piece still has eight K steps (c4: 104
    // units, 56 in halves and 48 in thirds, none of 256 ranks idle; -2.8 %
    // against halves only, which left 48 ranks without a fourth unit)
    const int t_left = seq_n - seq_full;
    const int t_x = (tT > 1 && tT + 1 <= (k_steps / S) / 8) ? blocks - t_left * tT : 0;
    const int t_n1 = (t_left - t_x) * tT;   // positions of the units cut in tT
    const int seq_pos = tT > 1 ? seq_full + t_n1 + t_x * (tT + 1) : seq_n;
    // position of the split sequence -> unit, piece and pieces of that unit
    auto unit_of = [&](int g, int &piece, int &T) -> int {
        T = tT;
        if (g < seq_full || tT == 1) {
            piece = 0;
            return g;
        }
        const int q = g - seq_full;
        if (q < t_n1) {
            piece = q % tT;
            return seq_full + q / tT;
        }
        T = tT + 1;
        piece = (q - t_n1) % T;
        return seq_full + (t_left - t_x) + (q - t_n1) / T;
    };
    auto g_of = [&](int k) {
        return k * blocks + ((k & 1) ? blocks - 1 - xcd_block : xcd_block);
    };
    int n_coop = 0, n_wave = 0;
    if (snake) {
        // this rank's rounds: the cooperative ones (positions below g_coop,
        // where the wave units start), then the wave ones.  g_of(k) lies in
        // [k blocks, (k + 1) blocks), so the rounds below position X are
        // X / blocks and possibly one more.  (In closed form: a loop over the
        // rounds took 3 µs of c5's start with its integer divisions.)
        auto rounds_below = [&](int X) {
            const int kq = X / blocks;
            return kq + (g_of(kq) < X ? 1 : 0);
        };
        const int g_coop =
            coop_units <= seq_full || tT == 1 ? coop_units
            : coop_units - seq_full < t_left - t_x
                ? seq_full + (coop_units - seq_full) * tT
                : seq_full + t_n1 + (coop_units - seq_full - (t_left - t_x)) * (tT + 1);
        n_coop = rounds_below(g_coop < seq_pos ? g_coop : seq_pos);
        n_wave = rounds_below(seq_pos) - n_coop;
    } else {
        const int wave_pos = coop_units == 0 ? seq_pos : units - coop_units;
        n_coop = coop_units > coop_rank ? (coop_units - coop_rank + blocks - 1) / blocks : 0;
        n_wave = wave_pos > blockIdx.x ? (wave_pos - blockIdx.x + blocks - 1) / blocks : 0;
    }
    auto coop_pos = [&](int i) { return snake ? g_of(i) : coop_rank + i * blocks; };
    auto wave_pos_of = [&](int j) {
        return snake ? g_of(n_coop + j) : coop_units + blockIdx.x + j * blocks;
    };
    int i_coop = 0, i_wave = 0;
    for (int uu = 0; uu < n_coop + n_wave; ++uu) {
        const bool take_coop = i_wave >= n_wave ||
                               (i_coop < n_coop && ((uu + blockIdx.x) & 1) == 0);
        const int g = take_coop ? coop_pos(i_coop++) : wave_pos_of(i_wave++);
        int piece = 0, pT = 1;
        const int u = unit_of(g, piece, pT);
        // K range of a last-round piece inside its unit's range
        auto narrow = [&](int &a, int &b) {
            if (tT > 1 && g >= seq_full) {
                const int span = b - a;
                const int a0 = a;
                a = a0 + span * piece / pT;
                b = a0 + span * (piece + 1) / pT;
            }
        };
        __syncthreads();   // the previous unit's waves are done with the LDS
        if (u < coop_units) {
            const int q = static_cast<int>(u / S);
            const int rk = __builtin_amdgcn_readfirstlane(find_expert(s_lpref, wl.n_ce, q));
            const int e = __builtin_amdgcn_readfirstlane(s_perm[rk]);
            const int e_cnt = __builtin_amdgcn_readfirstlane(s_cnt[e]);
            const int e_start = __builtin_amdgcn_readfirstlane(s_start[e]);
            const int e_pref = __builtin_amdgcn_readfirstlane(s_lpref[rk]);
            const int gr = coop_group_rows<kWide>(e_cnt);
            const int mg_count = (e_cnt + gr - 1) / gr;
            // Units of one expert, K split s outermost, then bands of
            // kCoopBand row groups; within a band the row groups of one
            // column tile are consecutive, then the next column tile.  The
            // blocks of one XCD (consecutive units) then share both the
            // band's x1 rows and its column tiles' weights through L2.
            const int local = u - static_cast<int>(e_pref) * S;
            const int per_s = static_cast<int>(mg_count) * n_tiles_c;
            const int s = static_cast<int>(local / per_s);
            const int r = static_cast<int>(local - s * per_s);
            const int band = r / (kCoopBand * n_tiles_c);
            const int j = r - band * kCoopBand * n_tiles_c;
            const int hb = min(kCoopBand, mg_count - band * kCoopBand);
            const int mg = band * kCoopBand + j % hb;
            const int nt = j / hb;
            const int wr = gr / kWavesPerBlock;               // rows per wave: 32 or 64
            const int row0 = mg * gr + w * wr;                // this wave's rows
            const int mcount = min(wr, e_cnt - row0);
            const int m0 = e_start + (mcount > 0 ? row0 : 0);
            int ks0 = static_cast<int>(static_cast<int>(k_steps_c) * s / S);
            int ks1 = static_cast<int>(static_cast<int>(k_steps_c) * (s + 1) / S);
            narrow(ks0, ks1);
            if constexpr (kTB) {
                if (gr > kCoopRows) {
                    if (wsc_tb)
                        ck_unit<FMT, 2, true>(p, e, m0, mcount, nt * kOutNC, ks0, ks1,
                                              store_rows, s_ring, w);
                    else
                        ck_unit<FMT, 2, false>(p, e, m0, mcount, nt * kOutNC, ks0, ks1,
                                               store_rows, s_ring, w);
                } else if (wsc_tb) {
                    ck_unit<FMT, 1, true>(p, e, m0, mcount, nt * kOutNC, ks0, ks1, store_rows,
                                          s_ring, w);
                } else {
                    ck_unit<FMT, 1, false>(p, e, m0, mcount, nt * kOutNC, ks0, ks1, store_rows,
                                           s_ring, w);
                }
            } else if constexpr (kKW) {
                int k0c = static_cast<int>(static_cast<int>(k_steps_w) * s / S);
                int k1c = static_cast<int>(static_cast<int>(k_steps_w) * (s + 1) / S);
                narrow(k0c, k1c);
                if (gr > kCoopRows) {
                    if (wsc_tb)
                        kc_unit<FMT, 2, true>(p, e, m0, mcount, nt * kOutNC, k0c, k1c,
                                              store_rows, s_ring, w);
                    else
                        kc_unit<FMT, 2, false>(p, e, m0, mcount, nt * kOutNC, k0c, k1c,
                                               store_rows, s_ring, w);
                } else if (wsc_tb) {
                    kc_unit<FMT, 1, true>(p, e, m0, mcount, nt * kOutNC, k0c, k1c, store_rows,
                                          s_ring, w);
                } else {
                    kc_unit<FMT, 1, false>(p, e, m0, mcount, nt * kOutNC, k0c, k1c, store_rows,
                                           s_ring, w);
                }
            } else {
                if (kWide && gr > kCoopRows) {
                    if constexpr (kWS) {
                        if (ws_ok) {
                            routed_item<FMT, !TRANS, true, 2, OP, true>(
                                p, e, m0, mcount, nt * kOutN, ks0, ks1, store_rows, s_ring, w);
                            continue;
                        }
                    }
                    routed_item<FMT, !TRANS, true, (kWide ? 2 : 1), OP>(
                        p, e, m0, mcount, nt * kOutN, ks0, ks1, store_rows, s_ring, w);
                } else {
                    routed_item<FMT, !TRANS, true, 1, OP>(p, e, m0, mcount, nt * kOutN, ks0,
                                                          ks1, store_rows, s_ring, w);
                }
            }
        } else {
            const int it = (u - coop_units) * kWavesPerBlock + w;
            if (it >= wave_items) continue;
            const int q = static_cast<int>(it / S);
            const int rk = __builtin_amdgcn_readfirstlane(find_expert(s_spref, wl.n_we, q));
            const int e = __builtin_amdgcn_readfirstlane(s_wperm[rk]);
            const int e_cnt = __builtin_amdgcn_readfirstlane(s_cnt[e]);
            const int e_start = __builtin_amdgcn_readfirstlane(s_start[e]);
            const int e_pref = __builtin_amdgcn_readfirstlane(s_spref[rk]);
            const int mt_count = (e_cnt + kTileM - 1) / kTileM;
            const int local = it - static_cast<int>(e_pref) * S;
            // items of an expert: row tiles fastest, then K ranges, then
            // column tiles; block-split: K ranges fastest (a unit's four
            // waves share the row and column tile)
            int mt, s, nt;
            if (bsplit) {
                s = static_cast<int>(local % S);
                const int rest = local / S;
                mt = static_cast<int>(rest % mt_count);
                nt = static_cast<int>(rest / mt_count);
            } else {
                mt = static_cast<int>(local % mt_count);
                const int rest = local / mt_count;
                s = static_cast<int>(rest % S);
                nt = static_cast<int>(rest / S);
            }
            const int m0 = e_start + mt * kTileM;
            const int mcount = min(kTileM, e_cnt - mt * kTileM);
            int ks0 = static_cast<int>(static_cast<int>(k_steps) * s / S);
            int ks1 = static_cast<int>(static_cast<int>(k_steps) * (s + 1) / S);
            narrow(ks0, ks1);
            char *own = s_ring + w * kRingBytes;
            char *split = bsplit ? s_ring : nullptr;
            // Non-temporal weight loads where no other item reads this K range
            // of these weights (one row tile) and the range is long: on short
            // ranges (80-192 KB per item: c1_fp4, c2_fp4) they ran 5-13 %
            // slower, on long ones up to 9 % faster (c3, c3_fp4, g1_llada).
            const bool stream =
                e_cnt <= kTileM &&
                (ks1 - ks0) * (kTB ? kCkWSlot : kSlotBytes) >= kStreamMinBytes;
            if constexpr (kTB) {
                if (wsc_tb) {
                    if (stream)
                        cw_item<FMT, true, true>(p, e, m0, mcount, nt * kOutN, ks0, ks1,
                                                 store_rows, own, split);
                    else
                        cw_item<FMT, true>(p, e, m0, mcount, nt * kOutN, ks0, ks1, store_rows,
                                           own, split);
                } else if (stream) {
                    cw_item<FMT, false, true>(p, e, m0, mcount, nt * kOutN, ks0, ks1, store_rows,
                                              own, split);
                } else {
                    cw_item<FMT, false>(p, e, m0, mcount, nt * kOutN, ks0, ks1, store_rows, own,
                                        split);
                }
            } else {
                if constexpr (kKW) {
                    if (kw_on) {
                        int k0w = static_cast<int>(static_cast<int>(k_steps_w) * s / S);
                        int k1w = static_cast<int>(static_cast<int>(k_steps_w) * (s + 1) / S);
                        narrow(k0w, k1w);
                        if (wsc_tb) {
                            if (stream)
                                kw_item<FMT, true, true>(p, e, m0, mcount, nt * kOutN, k0w, k1w,
                                                         store_rows, own, split);
                            else
                                kw_item<FMT, true>(p, e, m0, mcount, nt * kOutN, k0w, k1w,
                                                   store_rows, own, split);
                        } else if (stream) {
                            kw_item<FMT, false, true>(p, e, m0, mcount, nt * kOutN, k0w, k1w,
                                                      store_rows, own, split);
                        } else {
                            kw_item<FMT, false>(p, e, m0, mcount, nt * kOutN, k0w, k1w,
                                                store_rows, own, split);
                        }
                        continue;
                    }
                }
                if constexpr (kWS) {
                    if (ws_ok) {
                        if (stream)
                            routed_item<FMT, !TRANS, false, 1, OP, true, true>(
                                p, e, m0, mcount, nt * kOutN, ks0, ks1, store_rows, own, w);
                        else
                            routed_item<FMT, !TRANS, false, 1, OP, true>(
                                p, e, m0, mcount, nt * kOutN, ks0, ks1, store_rows, own, w);
                        continue;
                    }
                }
                if (stream)
                    routed_item<FMT, !TRANS, false, 1, OP, false, true>(
                        p, e, m0, mcount, nt * kOutN, ks0, ks1, store_rows, own, w, split);
                else
                    routed_item<FMT, !TRANS, false, 1, OP>(p, e, m0, mcount, nt * kOutN, ks0,
                                                           ks1, store_rows, own, w, split);
            }
        }
    }
    // The shared-expert term last: at the start its loads would delay the
    // first weight loads by a memory latency.
    if (OP == 0 && p.shared && !store_rows)
        shared_slice(p, blockIdx.x * kWavesPerBlock + w, waves);
}

template <int FMT, bool TRANS>
__global__ __launch_bounds__(kBlockThreads, 1) void fused_kernel(FusedParams p) {
    run_units<FMT, TRANS, 0>(p);
}

// The upstream step of the MoE FFN: x2 = w13 ([E, H, 2I] or [E, 2I, H]),
// x1 = the expert-sorted input tokens, output MX-quantised SwiGLU rows.
template <int FMT, bool TRANS>
__global__ __launch_bounds__(kBlockThreads, 1) void gemm1_swiglu_kernel(FusedParams p) {
    run_units<FMT, TRANS, 1>(p);
}

// ---------------------------------------------------------------------------
// Deterministic mode: CSR of row_index, then a fixed-order reduction
//   out[b] = ((init + W[t_1]) + W[t_2]) + ... + shared,  t_1 < t_2 < ...
// ---------------------------------------------------------------------------
// Destination row of token t (int64 or int32 row_index).
__device__ __forceinline__ int64_t row_of(const FusedParams &p, int t) {
    return p.row_index_i32 ? static_cast<int64_t>(static_cast<const int32_t *>(p.row_index)[t])
                           : static_cast<const int64_t *>(p.row_index)[t];
}

__global__ void det_count_kernel(FusedParams p, int *counts) {
    const int T = *p.det_total;
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
        const int64_t b = row_of(p, t);
        if (b >= 0 && b < p.batch) atomicAdd(counts + b, 1);
    }
}

// One workgroup: the counts (at most M < 2^31 in all) in chunks of four per
// thread, each chunk a 32-bit DPP block scan plus the carry of the chunks
// before it.
__global__ void det_scan_kernel(FusedParams p, const int *counts, int *offsets, int *cursor) {
    __shared__ uint32_t s_scan[4];
    constexpr int kPer = 4;                       // counts per thread and chunk
    constexpr int kChunk = kBlockThreads * kPer;
    uint32_t carry = 0;
    for (int base = 0; base < p.batch; base += kChunk) {
        const int b0 = base + threadIdx.x * kPer;
        uint32_t c[kPer], sum = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            c[i] = b0 + i < p.batch ? static_cast<uint32_t>(counts[b0 + i]) : 0u;
            sum += c[i];
        }
        uint32_t v[1] = {sum}, tot[1];
        block_scan_u32<1>(v, tot, s_scan, AddU32{});   // ends synchronised
        uint32_t run = carry + v[0];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (b0 + i < p.batch) {
                offsets[b0 + i] = static_cast<int>(run);
                cursor[b0 + i] = static_cast<int>(run);
            }
            run += c[i];
        }
        carry += tot[0];
    }
    if (threadIdx.x == 0) offsets[p.batch] = static_cast<int>(carry);
}

__global__ void det_fill_kernel(FusedParams p, int *cursor, int *tokens) {
    const int T = *p.det_total;
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
        const int64_t b = row_of(p, t);
        if (b >= 0 && b < p.batch) tokens[atomicAdd(cursor + b, 1)] = t;
    }
}

constexpr int kDetSortTile = 512;   // tokens compared per LDS pass

// One wave per output row: the row's tokens (filled in arbitrary order) are
// written to `sorted` in ascending t.  Tokens are distinct, so the position of
// t is the number of smaller tokens in the row (counted against LDS tiles of
// the row's list).
__global__ __launch_bounds__(kBlockThreads) void det_sort_kernel(FusedParams p, const int *offsets,
                                                               const int *tokens, int *sorted) {
    __shared__ int s_tile[kWavesPerBlock][kDetSortTile];
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wv = threadIdx.x >> 6;
    int *tile = s_tile[wv];
    const int wave = blockIdx.x * kWavesPerBlock + wv;
    const int waves = gridDim.x * kWavesPerBlock;
    for (int b = wave; b < p.batch; b += waves) {
        const int o0 = offsets[b], L = offsets[b + 1] - o0;
        for (int i0 = 0; i0 < L; i0 += kWaveSize) {
            const int i = i0 + lane;
            const int ti = i < L ? tokens[o0 + i] : 0;
            int rank = 0;
            for (int j0 = 0; j0 < L; j0 += kDetSortTile) {
                const int jn = L - j0 < kDetSortTile ? L - j0 : kDetSortTile;
                __builtin_amdgcn_wave_barrier();
                for (int j = lane; j < jn; j += kWaveSize) tile[j] = tokens[o0 + j0 + j];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                for (int j = 0; j < jn; ++j) rank += tile[j] < ti;
            }
            if (i < L) sorted[o0 + rank] = ti;
        }
    }
}

// out[b, c] = ((init + W[t_1, c]) + W[t_2, c]) + ... + shared term, with
// t_1 < t_2 < ... the tokens routed to row b: the same order for every
// element and every run.  Work item = (row, 256 columns); lane l handles
// columns 4l .. 4l + 3 of the item (N is a multiple of 4), loading a few
// tokens' rows ahead of the additions.
__global__ __launch_bounds__(kBlockThreads) void det_reduce_kernel(FusedParams p,
                                                                   const int *offsets,
                                                                   const int *sorted) {
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int waves = gridDim.x * kWavesPerBlock;
    constexpr int kCols = 4 * kWaveSize;
    const int chunks = (p.N + kCols - 1) / kCols;
    const int64_t items = static_cast<int64_t>(p.batch) * chunks;
    constexpr int kAhead = 4;
    for (int64_t it = wave; it < items; it += waves) {
        const int b = static_cast<int>(it / chunks);
        const int col = static_cast<int>(it % chunks) * kCols + 4 * lane;
        const bool ok = col < p.N;
        const int o0 = offsets[b], L = offsets[b + 1] - o0;
        float4 acc = ok ? *reinterpret_cast<const float4 *>(p.out + static_cast<int64_t>(b) * p.N + col)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i0 = 0; i0 < L; i0 += kAhead) {
            float4 v[kAhead];
#pragma unroll
            for (int k = 0; k < kAhead; ++k) {
                const int i = i0 + k;
                v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (ok && i < L) {
                    const int t = sorted[o0 + i];
                    v[k] = *reinterpret_cast<const float4 *>(p.wbuf + static_cast<int64_t>(t) * p.N + col);
                }
            }
#pragma unroll
            for (int k = 0; k < kAhead; ++k) {
                if (i0 + k < L) {
                    acc.x += v[k].x;
                    acc.y += v[k].y;
                    acc.z += v[k].z;
                    acc.w += v[k].w;
                }
            }
        }
        if (!ok) continue;
        if (p.shared && b >= p.shared_off && b < p.shared_off + p.shared_rows) {
            const uint2 h = *reinterpret_cast<const uint2 *>(
                p.shared + static_cast<int64_t>(b - p.shared_off) * p.N + col);
            acc.x += p.shared_w * __uint_as_float(h.x << 16);
            acc.y += p.shared_w * __uint_as_float(h.x & 0xffff0000u);
            acc.z += p.shared_w * __uint_as_float(h.y << 16);
            acc.w += p.shared_w * __uint_as_float(h.y & 0xffff0000u);
        }
        *reinterpret_cast<float4 *>(p.out + static_cast<int64_t>(b) * p.N + col) = acc;
    }
}

__global__ void fill_zero_kernel(int *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0;
}

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int FMT, bool TRANS>
hipError_t launch_fused_t(const FusedParams &p, hipStream_t stream) {
    const int grid = device_cu_count();
    hipLaunchKernelGGL((fused_kernel<FMT, TRANS>), dim3(grid), dim3(kBlockThreads), 0, stream, p);
    return hipGetLastError();
}

template <int FMT, bool TRANS>
hipError_t launch_gemm1_t(const FusedParams &p, hipStream_t stream) {
    const int grid = device_cu_count();
    hipLaunchKernelGGL((gemm1_swiglu_kernel<FMT, TRANS>), dim3(grid), dim3(kBlockThreads), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

// Scratch of the allocation-free deterministic entry point: the deterministic
// mode's workspace (weighted rows and the row_index CSR) for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy until the
// process ends; every call on that GPU shares it.  In host code the name is
// only a handle for hipGetSymbolAddress: kernels get the address it returns.
static __device__ __align__(256) unsigned char scratch[GFR_STATIC_SCRATCH_BYTES];

hipError_t static_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

DetLayout det_layout(int64_t M, int64_t N, int64_t batch) {
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    DetLayout d{};
    d.wbuf = 0;
    d.counts = up(static_cast<size_t>(M) * N * sizeof(float));
    d.cursor = d.counts + up(static_cast<size_t>(batch) * sizeof(int));
    d.offsets = d.cursor + up(static_cast<size_t>(batch) * sizeof(int));
    d.tokens = d.offsets + up((static_cast<size_t>(batch) + 1) * sizeof(int));
    d.sorted = d.tokens + up(static_cast<size_t>(M) * sizeof(int));
    d.total_tokens = d.sorted + up(static_cast<size_t>(M) * sizeof(int));
    d.total = d.total_tokens + 256;
    return d;
}

hipError_t launch_gemm1(const FusedParams &p, int transpose_w13, int fp8_kind,
                        hipStream_t stream) {
    if (fp8_kind == GFR_FP8_E4M3FN)
        return transpose_w13 ? launch_gemm1_t<0, true>(p, stream) : launch_gemm1_t<0, false>(p, stream);
    return transpose_w13 ? launch_gemm1_t<1, true>(p, stream) : launch_gemm1_t<1, false>(p, stream);
}

hipError_t launch_fused(const FusedParams &p, int transpose_x2, int fp8_kind,
                        hipStream_t stream) {
    if (fp8_kind == kKindW4A8)
        return launch_fused_t<8, false>(p, stream);
    if (fp8_kind == GFR_FP4_E2M1)
        return transpose_x2 ? launch_fused_t<4, true>(p, stream) : launch_fused_t<4, false>(p, stream);
    if (fp8_kind == GFR_FP8_E4M3FN)
        return transpose_x2 ? launch_fused_t<0, true>(p, stream) : launch_fused_t<0, false>(p, stream);
    return transpose_x2 ? launch_fused_t<1, true>(p, stream) : launch_fused_t<1, false>(p, stream);
}

// Workspace regions: see DetLayout.  The counts are cleared by a fill kernel
// (not a memset node) so the sequence stays safe under graph capture.
hipError_t launch_deterministic_prep(const FusedParams &p, void *workspace,
                                     hipStream_t stream) {
    const DetLayout d = det_layout(p.M, p.N, p.batch);
    int *counts = reinterpret_cast<int *>(static_cast<char *>(workspace) + d.counts);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(device_cu_count()), dim3(kBlockThreads), 0,
                       stream, counts, p.batch);
    return hipGetLastError();
}

hipError_t launch_deterministic_reduce(const FusedParams &p, void *workspace,
                                       hipStream_t stream) {
    const DetLayout d = det_layout(p.M, p.N, p.batch);
    char *ws = static_cast<char *>(workspace);
    int *counts = reinterpret_cast<int *>(ws + d.counts);
    int *cursor = reinterpret_cast<int *>(ws + d.cursor);
    int *offsets = reinterpret_cast<int *>(ws + d.offsets);
    int *tokens = reinterpret_cast<int *>(ws + d.tokens);
    int *sorted = reinterpret_cast<int *>(ws + d.sorted);
    const int cu = device_cu_count();
    hipLaunchKernelGGL(det_count_kernel, dim3(cu), dim3(kBlockThreads), 0, stream, p, counts);
    hipLaunchKernelGGL(det_scan_kernel, dim3(1), dim3(kBlockThreads), 0, stream, p, counts,
                       offsets, cursor);
    hipLaunchKernelGGL(det_fill_kernel, dim3(cu), dim3(kBlockThreads), 0, stream, p, cursor,
                       tokens);
    hipLaunchKernelGGL(det_sort_kernel, dim3(cu), dim3(kBlockThreads), 0, stream, p, offsets,
                       tokens, sorted);
    // eight blocks per CU: each wave's rows are chains of dependent loads
    // (offsets, token list, rows), so more waves in flight pay (c5: 78 -> 63
    // µs against four per CU; sixteen or 32 per CU no faster)
    hipLaunchKernelGGL(det_reduce_kernel, dim3(cu * 8), dim3(kBlockThreads), 0, stream, p,
                       offsets, sorted);
    return hipGetLastError();
}

}  // namespace gfr
