// C ABI of libw4a16.so: argument validation, the dispatch / split-K policy and the entry
// points declared in include/w4a16.h.  Every compute call only enqueues kernels on the
// caller's stream; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdint.h>

#include "internal.h"
#include "w4a16.h"

namespace {

using namespace w4a16;

// Policy constants.
constexpr int64_t kQmvMaxRows = 8;        // decode rows served by qmv ("Week 2 Day 6", Task 1)
constexpr int64_t kSkinnyMaxRows = 32;    // rows served by the skinny path
constexpr int64_t kQmvKernelRows = 16;    // rows one matvec MFMA operand covers
// LDS a wide-kernel workgroup may use on the skinny path (two workgroups per compute unit)
constexpr size_t kQmvWideSkinnyLds = 80 * 1024;
constexpr int64_t kQmvPerRowMaxRows = 2;   // rows the per-row width-generic kernel serves
constexpr int kQmvBitsWaves = 4;           // waves splitting K in the width-generic kernels
constexpr int kSplitMinGroups = 4;        // fewest groups one split-K slice may own
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
// Largest K: keeps every per-lane buffer offset of the kernels (at most 256 K bytes past a
// wave's base) inside 32 bits.
constexpr int64_t kMaxK = int64_t{1} << 20;

std::atomic<int> g_cu_cache[64];

int query_num_cus(int32_t* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_DEVICE;
    if (dev >= 0 && dev < 64) {
        const int cached = g_cu_cache[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *out = cached;
            return W4A16_OK;
        }
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return W4A16_ERR_DEVICE;
    if (dev >= 0 && dev < 64) g_cu_cache[dev].store(cus, std::memory_order_relaxed);
    *out = cus;
    return W4A16_OK;
}

int check_shape(int64_t M, int64_t N, int64_t K, int32_t group) {
    if (M < 1 || N < 1 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxK) return W4A16_ERR_SHAPE;
    if (group != W4A16_GROUP) return W4A16_ERR_GROUP;
    if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Byte ranges [p, p + n) of two buffers share at least one byte.
bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

// Pointer checks of a projection y [M, N] = x [M, K] . dequant(wq [N, K * bits / 32])^T (shape
// already validated): non-null, aligned, and the output sharing no byte with an input.
int check_buffers(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b, const uint16_t* y,
                  int64_t M, int64_t N, int64_t K, int32_t bits = 4) {
    if (!x || !wq || !s || !b || !y) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(s, 2) || !aligned(b, 2) || !aligned(y, 2))
        return W4A16_ERR_ALIGN;
    const uint64_t ny = static_cast<uint64_t>(M) * N * 2, sb = static_cast<uint64_t>(N) * (K / W4A16_GROUP) * 2;
    if (overlaps(y, ny, x, static_cast<uint64_t>(M) * K * 2) ||
        overlaps(y, ny, wq, static_cast<uint64_t>(N) * K * bits / 8) || overlaps(y, ny, s, sb) ||
        overlaps(y, ny, b, sb))
        return W4A16_ERR_OVERLAP;
    return W4A16_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

void plan_qmv(int64_t M, int64_t N, int64_t K, int32_t cus, w4a16_plan_t* p) {
    // Measured on MI355X (K = 1024 .. 9728, N = 1024 .. 151936, M = 1 .. 16, random data): below
    // 16k columns the row-amortized kernel (exact codes on the matrix core, s * P + b * X per
    // group) leads by 5-22%, except for long K (64 groups or more) at up to 8 rows, where the
    // 16-column dequantizing kernel whose four waves split K leads by 5-20%; around 16k columns
    // the 64-column kernel leads; from 24k columns (16k at 32 groups or more) the persistent wide
    // kernel, which streams whole blocks per wave, wins by 1.4x on the 151936-column head.
    // Up to 4 rows below 32k columns and 5 to 8 rows below 16k columns (qmv_burst_shape gives
    // the row, group and width limits), the burst kernel (every load of a wave issued at once,
    // in its packed or 16-column form) leads all of them: at up to 4 rows by 15-25% below 16k
    // columns and by 7-39% against the wide kernel at 16k-32k columns; at 5 to 8 rows by 7-10%.
    const int64_t blocks16 = ceil_div(N, 16);
    const int64_t G = K / W4A16_GROUP;
    int variant;
    QmvBurstShape burst{};
    if (qmv_burst_shape(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), &burst))
        variant = kQmvBurstVariant;
    else if (qmv_wide_fits(static_cast<int>(M), static_cast<int>(K)) && (blocks16 >= 1536 || (blocks16 >= 1024 && G >= 32)))
        variant = kQmvWideVariant;
    else if (blocks16 >= 1024)
        variant = 1;
    else if (G >= 64 && M <= kQmvMaxRows)
        variant = 0;
    else
        variant = kQmvAmortizedVariant;
    const QmvShape& v = kQmvVariants[variant];
    p->path = W4A16_PATH_QMV;
    p->tile_m = 16;
    p->tile_n = v.cb * v.wn * 16;
    p->tile_k = W4A16_GROUP;
    int waves = v.wn * v.kw;
    if (variant == kQmvWideVariant) {
        // persistent: at most as many workgroups as are resident at once (the launch asks the
        // runtime how many fit per compute unit; 32 waves per compute unit is the register limit)
        waves = qmv_wide_waves(static_cast<int>(M));
        p->tile_n = 16;
        p->grid_x = static_cast<int32_t>(std::min<int64_t>(ceil_div(blocks16, waves), int64_t{32 / waves} * cus));
    } else if (variant == kQmvBurstVariant) {
        waves = burst.kw;
        p->tile_n = burst.cols;
        p->grid_x = static_cast<int32_t>(ceil_div(N, burst.cols));
    } else {
        p->grid_x = static_cast<int32_t>(ceil_div(N, p->tile_n));
    }
    p->grid_y = 1;
    p->grid_z = 1;
    p->block_threads = 64 * waves;
    p->split_k = 1;
    p->k_waves = variant == kQmvBurstVariant ? burst.kw : v.kw;
    p->variant = variant;
    p->workspace_bytes = 0;
}

uint64_t round256(uint64_t v) { return (v + 255) / 256 * 256; }

// Bytes of the activations' group sums (exact-code mode), at the start of the workspace.
uint64_t group_sum_bytes(int64_t M, int64_t K) {
    return round256(static_cast<uint64_t>(M) * group_sum_cols(static_cast<int>(K)) * 2);
}

// Split-K slices for a grid of `tiles` output tiles (of an M x N output) over G groups: the
// caller's split_k if nonzero (at most G), else the policy's (skinny: the rule of the 32-row
// tiles).
int64_t tile_split(int64_t tiles, int64_t M, int64_t N, int64_t G, int32_t split_k, int32_t cus, bool skinny) {
    int64_t S = 1;
    if (split_k == 0) {
        if (skinny) {
            // skinny tiles: about one work unit per compute unit (measured best: gate S = 3 for
            // 76 tiles, q S = 4..8 for 32, down / o / k,v S = 8), at most 8 slices of >= 2 groups
            if (tiles < cus) {
                S = std::min<int64_t>({cus / tiles, 8, G / 2});
                if (S < 2) S = 1;
            }
        } else if (tiles < cus && G >= 2 * kSplitMinGroups) {
            // Split only an under-filled grid, by a cost model fitted to sweeps of S = 1..8 on
            // MI355X (64 x 128 tiles; M = 128 and 512; the q, k/v, o, gate and down shapes of
            // the 2560-wide layer): rounds of one work unit per compute unit x groups per
            // slice x 0.75 us, plus 2 us and 0.3 us per MB of fp32 partials for a split.  It
            // picks the measured best S (or one within 0.7 us) on every swept shape, e.g.
            // S = 3 for 160 tiles of K = 4096 or 9728, S = 1 for 152 tiles of K = 2560; every
            // slice keeps at least kSplitMinGroups groups.
            double best = 0.0;
            const int64_t s_max = std::min<int64_t>(8, G / kSplitMinGroups);
            for (int64_t s = 1; s <= s_max; ++s) {
                double t = static_cast<double>(ceil_div(tiles * s, cus)) * static_cast<double>(ceil_div(G, s)) * 0.75;
                if (s > 1) t += 2.0 + 0.3 * static_cast<double>(s * M * N) * 4.0 / 1e6;
                if (s == 1 || t < best) {
                    best = t;
                    S = s;
                }
            }
        }
    } else {
        S = split_k < 1 ? 1 : split_k;
        if (S > G) S = G;
    }
    return S;
}

// skinny: 32-row tiles and the skinny split rule (rows 17..32, or a wide head at 9..16 rows).
// codes: the exact-code mode (codes on the matrix core, per-group scaling, bias from the group
// sums of the activations), which needs the group sums in the workspace.
void plan_qmm(int64_t M, int64_t N, int64_t K, int32_t split_k, int32_t cus, w4a16_plan_t* p,
              bool skinny = false, bool codes = true) {
    const int64_t G = K / W4A16_GROUP;
    // Measured on MI355X: 64 x 128 tiles (three waves per SIMD) lead up to about a thousand
    // rows, where the grid is small; 128 x 128 tiles (two waves per SIMD) lead beyond.  For at
    // most 32 rows, 32 x 128 tiles (three waves per SIMD, three stages) lead on every layer shape
    // and on the vocabulary head.
    int variant = skinny ? kQmmSkinnyVariant : (M <= 1024 ? 1 : 0);
    const int64_t tile_n = kQmmVariants[variant].tile_n();
    const int64_t tiles = ceil_div(M, kQmmVariants[variant].bm) * ceil_div(N, tile_n);
    const int64_t S = tile_split(tiles, M, N, G, split_k, cus, skinny);
    // At most one work unit per compute unit: the same tiles with two waves per column strip
    // (measured on MI355X: 512-row q 23.6 -> 21.4 us, k/v 16.4 -> 15.0 us, 128-row gate 22.6 ->
    // 21.7 us; with more units per compute unit it measured 0-6% slower).
    if (variant == 1 && tiles * S <= cus) variant = kQmmKSplitVariant;
    // Unsplit grids of more than one tile per compute unit: 96-row tiles with two waves per
    // column strip (two resident per compute unit) when they need fewer rounds of tiles per
    // compute unit, and at most two (measured on MI355X at 512 rows, K = 2560, N = 9728: 456
    // tiles in 38.0 us against 608 64-row tiles in 43.0 us; with as many rounds, as for the
    // 4096-wide q or the split o and down, they measured 4-13% slower).
    if (variant == 1 && S == 1) {
        const int64_t tiles96 = ceil_div(M, kQmmVariants[kQmmRows96Variant].bm) * ceil_div(N, tile_n);
        const int64_t rounds64 = ceil_div(tiles, cus), rounds96 = ceil_div(tiles96, cus);
        if (rounds96 < rounds64 && rounds96 <= 2) variant = kQmmRows96Variant;
    }
    const QmmShape& v = kQmmVariants[variant];
    p->path = skinny ? W4A16_PATH_SKINNY : W4A16_PATH_QMM;
    p->tile_m = v.bm;
    p->tile_n = static_cast<int32_t>(tile_n);
    p->tile_k = W4A16_GROUP;
    p->grid_x = static_cast<int32_t>(ceil_div(N, tile_n));
    p->grid_y = static_cast<int32_t>(ceil_div(M, v.bm));
    p->grid_z = static_cast<int32_t>(S);
    p->block_threads = 64 * v.nwaves;
    p->split_k = static_cast<int32_t>(S);
    p->k_waves = v.ksplit;
    codes = codes && variant == kQmmCodesTileVariant;
    p->variant = variant + (codes ? kQmmCodesVariantOffset : 0);
    p->workspace_bytes = (codes ? group_sum_bytes(M, K) : 0) +
                         (S > 1 ? static_cast<uint64_t>(S) * M * N * sizeof(float) : 0);
}

bool plan_codes(const w4a16_plan_t& p) { return p.variant >= kQmmCodesVariantOffset; }
int plan_tile_variant(const w4a16_plan_t& p) { return p.variant % kQmmCodesVariantOffset; }

// Skinny rows (at most 32): up to 16 rows the matvec kernels (their 16-row MFMA operand covers
// them; measured 1.1-1.7x faster than tiles at 9..16 rows), except where the wide kernel's
// activation tile would leave fewer than two workgroups per compute unit; above 16 rows the
// 32-row MFMA tiles with split-K.
void plan_skinny(int64_t M, int64_t N, int64_t K, int32_t split_k, int32_t cus, w4a16_plan_t* p) {
    if (M <= kQmvKernelRows) {
        plan_qmv(M, N, K, cus, p);
        const bool wide_too_big = p->variant == kQmvWideVariant &&
                                  qmv_wide_static_lds(static_cast<int>(M)) + qmv_wide_lds_bytes(static_cast<int>(M), static_cast<int>(K)) >
                                      kQmvWideSkinnyLds;
        if (!wide_too_big) {
            p->path = W4A16_PATH_SKINNY;
            return;
        }
    }
    plan_qmm(M, N, K, split_k, cus, p, true);
}

int make_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t path, int32_t split_k, int32_t num_cus,
              w4a16_plan_t* out) {
    if (!out) return W4A16_ERR_NULL;
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    if (path != W4A16_PATH_AUTO && path != W4A16_PATH_QMV && path != W4A16_PATH_QMM && path != W4A16_PATH_SKINNY)
        return W4A16_ERR_UNSUPPORTED;
    if (split_k < 0) return W4A16_ERR_SHAPE;
    int32_t cus = num_cus;
    if (cus <= 0) {
        st = query_num_cus(&cus);
        if (st != W4A16_OK) return st;
    }
    if (path == W4A16_PATH_AUTO)
        path = M <= kQmvMaxRows ? W4A16_PATH_QMV : (M <= kSkinnyMaxRows ? W4A16_PATH_SKINNY : W4A16_PATH_QMM);
    if (path == W4A16_PATH_QMV) {
        if (M > kQmvMaxRows) return W4A16_ERR_UNSUPPORTED;
        plan_qmv(M, N, K, cus, out);
    } else if (path == W4A16_PATH_SKINNY) {
        if (M > kSkinnyMaxRows) return W4A16_ERR_UNSUPPORTED;
        plan_skinny(M, N, K, split_k, cus, out);
    } else {
        plan_qmm(M, N, K, split_k, cus, out);
    }
    out->num_cus = cus;
    return W4A16_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH; }

// a skinny plan of at most 16 rows runs the matvec kernels (tile_m = 16); otherwise tiles
bool uses_qmv_kernels(const w4a16_plan_t& p) {
    return p.path == W4A16_PATH_QMV || (p.path == W4A16_PATH_SKINNY && p.tile_m == kQmvKernelRows);
}

int run_plan(const w4a16_plan_t& p, const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
             uint16_t* y, int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t stream) {
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (uses_qmv_kernels(p)) return to_status(launch_qmv(p.variant, x, wq, s, b, y, m, n, k, stream));
    // workspace: [group sums (exact-code mode)][fp32 split-K partials]
    uint16_t* xsum = nullptr;
    uint8_t* rest = static_cast<uint8_t*>(workspace);
    if (plan_codes(p)) {
        xsum = static_cast<uint16_t*>(workspace);
        rest += group_sum_bytes(M, K);
        const hipError_t e0 = launch_act_group_sums(x, xsum, m, k, group_sum_cols(k), stream);
        if (e0 != hipSuccess) return to_status(e0);
    }
    float* ws = reinterpret_cast<float*>(rest);
    hipError_t e = launch_qmm(plan_tile_variant(p), x, xsum, wq, s, b, y, ws, m, n, k, p.split_k, stream);
    if (e != hipSuccess || p.split_k == 1) return to_status(e);
    return to_status(launch_splitk_reduce(ws, y, M * N, p.split_k, stream));
}

// Fit a tile plan to the caller's workspace: the exact-code mode needs the group sums, a split
// needs the partials.  Without room the plan drops the exact-code mode (same result within the
// tolerance), then, under the policy, the split (the unsplit plan computes the same result); a
// forced split with too little room for its partials is an error.
template <typename Replan>
int fit_workspace(w4a16_plan_t& p, int32_t split_k, void* workspace, size_t ws_bytes, Replan replan) {
    auto fits = [&](const w4a16_plan_t& q) {
        return q.workspace_bytes == 0 || (workspace != nullptr && aligned(workspace, 16) && ws_bytes >= q.workspace_bytes);
    };
    if (fits(p)) return W4A16_OK;
    if (plan_codes(p)) {
        replan(p.split_k, false);
        if (fits(p)) return W4A16_OK;
    }
    if (split_k > 1)
        return workspace != nullptr && !aligned(workspace, 16) ? W4A16_ERR_ALIGN : W4A16_ERR_WORKSPACE;
    replan(1, false);
    return W4A16_OK;
}

int run_qmm(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b, uint16_t* y, int64_t M,
            int64_t N, int64_t K, int32_t group, int32_t path, int32_t split_k, void* workspace, size_t ws_bytes,
            void* stream) {
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    st = check_buffers(x, wq, s, b, y, M, N, K);
    if (st != W4A16_OK) return st;
    if (split_k < 0) return W4A16_ERR_SHAPE;
    w4a16_plan_t p;
    st = make_plan(M, N, K, group, path, split_k, 0, &p);
    if (st != W4A16_OK) return st;
    if (!uses_qmv_kernels(p)) {
        const bool skinny = p.path == W4A16_PATH_SKINNY;
        const int32_t cus = p.num_cus;
        st = fit_workspace(p, split_k, workspace, ws_bytes, [&](int32_t S, bool codes) {
            plan_qmm(M, N, K, S, cus, &p, skinny, codes);
            p.num_cus = cus;
        });
        if (st != W4A16_OK) return st;
    }
    return run_plan(p, x, wq, s, b, y, M, N, K, workspace, static_cast<hipStream_t>(stream));
}

// Grouped projections of one input.  With more than 32 rows the projections' 128-column tiles
// form one grid: the tile form and the split that the qmm policy takes for M rows and the summed
// tile columns (a split's partials of every projection in one array, summed by one grouped
// slice-sum launch); with at most 32 rows, or one projection, each projection runs its own
// w4a16_linear dispatch and the workspace is the largest of theirs.
static_assert(W4A16_MAX_GROUPED == kMaxGroupedProjections, "one limit for the ABI and the kernel");
int make_grouped_plan(int32_t count, const int64_t* N, int64_t M, int64_t K, int32_t group, int32_t num_cus,
                      w4a16_plan_t* out, bool codes = true, int32_t split_k = 0) {
    if (!out || !N) return W4A16_ERR_NULL;
    if (count < 1 || count > W4A16_MAX_GROUPED) return W4A16_ERR_SHAPE;
    int64_t tiles_n = 0;
    for (int32_t p = 0; p < count; ++p) {
        const int st = check_shape(M, N[p], K, group);
        if (st != W4A16_OK) return st;
        tiles_n += ceil_div(N[p], kGroupedTileN);
    }
    if (tiles_n * kGroupedTileN > kMaxDim) return W4A16_ERR_SHAPE;
    int32_t cus = num_cus;
    if (cus <= 0) {
        const int st = query_num_cus(&cus);
        if (st != W4A16_OK) return st;
    }
    if (count == 1 || M <= kSkinnyMaxRows) {
        uint64_t ws = 0;
        for (int32_t p = count - 1; p >= 0; --p) {      // leaves the first projection's plan in *out
            const int st = make_plan(M, N[p], K, group, W4A16_PATH_AUTO, 0, cus, out);
            if (st != W4A16_OK) return st;
            ws = std::max<uint64_t>(ws, out->workspace_bytes);
        }
        if (count > 1) out->path = W4A16_PATH_PER_PROJECTION;
        out->workspace_bytes = ws;
        return W4A16_OK;
    }
    plan_qmm(M, tiles_n * kGroupedTileN, K, split_k, cus, out, false, codes);
    out->path = W4A16_PATH_GROUPED;
    out->num_cus = cus;
    return W4A16_OK;
}

int run_grouped(const uint16_t* x, int32_t count, const uint32_t* const* wq, const uint16_t* const* s,
                const uint16_t* const* b, uint16_t* const* y, const int64_t* N, int64_t M, int64_t K, int32_t group,
                void* workspace, size_t ws_bytes, void* stream) {
    if (!wq || !s || !b || !y || !N) return W4A16_ERR_NULL;
    if (count < 1 || count > W4A16_MAX_GROUPED) return W4A16_ERR_SHAPE;
    for (int32_t p = 0; p < count; ++p) {
        int st = check_shape(M, N[p], K, group);
        if (st != W4A16_OK) return st;
        st = check_buffers(x, wq[p], s[p], b[p], y[p], M, N[p], K);
        if (st != W4A16_OK) return st;
    }
    // an output may share no byte with another projection's output or inputs either
    for (int32_t p = 0; p < count; ++p) {
        const uint64_t ny = static_cast<uint64_t>(M) * N[p] * 2;
        for (int32_t q = 0; q < count; ++q) {
            if (q == p) continue;
            const uint64_t sb = static_cast<uint64_t>(N[q]) * (K / W4A16_GROUP) * 2;
            if (overlaps(y[p], ny, y[q], static_cast<uint64_t>(M) * N[q] * 2) ||
                overlaps(y[p], ny, wq[q], static_cast<uint64_t>(N[q]) * K / 2) || overlaps(y[p], ny, s[q], sb) ||
                overlaps(y[p], ny, b[q], sb))
                return W4A16_ERR_OVERLAP;
        }
    }
    w4a16_plan_t pl;
    int st = make_grouped_plan(count, N, M, K, group, 0, &pl);
    if (st != W4A16_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (pl.path != W4A16_PATH_GROUPED) {
        // stream order keeps the shared workspace of consecutive calls apart
        for (int32_t p = 0; p < count; ++p) {
            st = run_qmm(x, wq[p], s[p], b[p], y[p], M, N[p], K, group, W4A16_PATH_AUTO, 0, workspace, ws_bytes,
                         stream);
            if (st != W4A16_OK) return st;
        }
        return W4A16_OK;
    }
    const int32_t cus = pl.num_cus;
    st = fit_workspace(pl, 0, workspace, ws_bytes, [&](int32_t S, bool codes) {
        make_grouped_plan(count, N, M, K, group, cus, &pl, codes, S);
    });
    if (st != W4A16_OK) return st;
    QmmGroups g{};
    g.count = count;
    int tn = 0;
    for (int32_t p = 0; p < count; ++p) {
        g.wq[p] = wq[p];
        g.s[p] = s[p];
        g.b[p] = b[p];
        g.y[p] = y[p];
        g.n[p] = static_cast<int>(N[p]);
        g.tn_first[p] = tn;
        tn += static_cast<int>(ceil_div(N[p], kGroupedTileN));
    }
    const int m = static_cast<int>(M), k = static_cast<int>(K);
    // workspace: [group sums (exact-code mode)][fp32 split-K partials of the concatenated columns]
    uint16_t* xsum = nullptr;
    uint8_t* rest = static_cast<uint8_t*>(workspace);
    if (plan_codes(pl)) {
        xsum = static_cast<uint16_t*>(workspace);
        rest += group_sum_bytes(M, K);
        const hipError_t e0 = launch_act_group_sums(x, xsum, m, k, group_sum_cols(k), hs);
        if (e0 != hipSuccess) return to_status(e0);
    }
    float* ws = pl.split_k > 1 ? reinterpret_cast<float*>(rest) : nullptr;
    hipError_t e = launch_qmm_grouped(plan_tile_variant(pl), x, xsum, g, ws, m, k, pl.split_k, hs);
    if (e != hipSuccess || pl.split_k == 1) return to_status(e);
    return to_status(launch_splitk_reduce_grouped(ws, g, m, pl.split_k, hs));
}

// Gate / up pair with SwiGLU: one tile kernel computes both projections of the same columns.
// Tiles: 32 rows up to 32 rows; above, 64-row tiles in the exact-code mode (measured on MI355X
// against the dequantizing 64- and 128-row tiles: 87 vs 98 us at 512 rows and 497 vs 560 us at
// 4096 rows, K = 2560, N = 9728); without the exact-code mode 64 rows up to ~1k and 128 beyond;
// unsplit grids that 96-row tiles cover in fewer rounds per compute unit take those (below).
// The split follows the qmm rule on the same tile grid.  Workspace: [group sums (exact-code
// mode)][gate partials][up partials], the partials 2 * S * M * N fp32.
void plan_gate_up(int64_t M, int64_t N, int64_t K, int32_t split_k, int32_t cus, w4a16_plan_t* p,
                  bool codes = true) {
    const bool skinny = M <= kSkinnyMaxRows;
    codes = codes && !skinny;
    int variant = skinny ? 0 : (codes ? kGateUpCodesTileVariant : (M <= 1024 ? 1 : 2));
    int64_t tile_n = kGateUpVariants[variant].tile_n();
    int64_t tiles = ceil_div(M, kGateUpVariants[variant].bm) * ceil_div(N, tile_n);
    const int64_t S = tile_split(tiles, M, N, K / W4A16_GROUP, split_k, cus, skinny);
    // A grid of at most one work unit per compute unit does not repay the exact-code form's
    // pre-pass: the dequantizing 64-row tiles (measured on MI355X at 128 rows, K = 2560, N = 9728,
    // 152 tiles: 35.3 us against 38.3 us with the group sums).
    if (codes && tiles * S <= cus) {
        variant = 1;
        codes = false;
    }
    // Unsplit 64-row grids of more than one tile per compute unit: dequantizing 96-row tiles when
    // they need fewer rounds of tiles per compute unit, and at most two (measured on MI355X, K =
    // 2560, N = 9728: 512 rows 73.5-76.4 us against 86-87 us for the 64-row exact-code tiles,
    // 256 rows 46 against 55 us; at 1024 rows, four rounds against five, 145 against 141 us).
    if (!skinny && S == 1) {
        const int64_t tiles96 = ceil_div(M, kGateUpVariants[kGateUpRows96Variant].bm) * ceil_div(N, tile_n);
        if (ceil_div(tiles96, cus) < ceil_div(tiles, cus) && ceil_div(tiles96, cus) <= 2) {
            variant = kGateUpRows96Variant;
            codes = false;
            tiles = tiles96;
        }
    }
    const QmmShape& v = kGateUpVariants[variant];
    tile_n = v.tile_n();
    p->path = W4A16_PATH_GATE_UP;
    p->tile_m = v.bm;
    p->tile_n = static_cast<int32_t>(tile_n);
    p->tile_k = W4A16_GROUP;
    p->grid_x = static_cast<int32_t>(ceil_div(N, tile_n));
    p->grid_y = static_cast<int32_t>(ceil_div(M, v.bm));
    p->grid_z = static_cast<int32_t>(S);
    p->block_threads = 64 * v.nwaves;
    p->split_k = static_cast<int32_t>(S);
    p->k_waves = 1;
    p->variant = variant + (codes ? kQmmCodesVariantOffset : 0);
    p->workspace_bytes = (codes ? group_sum_bytes(M, K) : 0) +
                         (S > 1 ? 2ull * static_cast<uint64_t>(S) * M * N * sizeof(float) : 0);
}

int make_gate_up_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, int32_t num_cus,
                      w4a16_plan_t* out) {
    if (!out) return W4A16_ERR_NULL;
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    if (split_k < 0) return W4A16_ERR_SHAPE;
    int32_t cus = num_cus;
    if (cus <= 0) {
        st = query_num_cus(&cus);
        if (st != W4A16_OK) return st;
    }
    plan_gate_up(M, N, K, split_k, cus, out);
    out->num_cus = cus;
    return W4A16_OK;
}

int run_gate_up(const uint16_t* x, const uint32_t* wq_g, const uint16_t* s_g, const uint16_t* b_g,
                const uint32_t* wq_u, const uint16_t* s_u, const uint16_t* b_u, uint16_t* h, int64_t M, int64_t N,
                int64_t K, int32_t group, int32_t split_k, void* workspace, size_t ws_bytes, void* stream) {
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    st = check_buffers(x, wq_g, s_g, b_g, h, M, N, K);
    if (st != W4A16_OK) return st;
    st = check_buffers(x, wq_u, s_u, b_u, h, M, N, K);
    if (st != W4A16_OK) return st;
    if (split_k < 0) return W4A16_ERR_SHAPE;
    w4a16_plan_t p;
    st = make_gate_up_plan(M, N, K, group, split_k, 0, &p);
    if (st != W4A16_OK) return st;
    const int32_t cus = p.num_cus;
    st = fit_workspace(p, split_k, workspace, ws_bytes, [&](int32_t S, bool codes) {
        plan_gate_up(M, N, K, S, cus, &p, codes);
        p.num_cus = cus;
    });
    if (st != W4A16_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    uint16_t* xsum = nullptr;
    uint8_t* rest = static_cast<uint8_t*>(workspace);
    if (plan_codes(p)) {
        xsum = static_cast<uint16_t*>(workspace);
        rest += group_sum_bytes(M, K);
        const hipError_t e0 = launch_act_group_sums(x, xsum, m, k, group_sum_cols(k), s);
        if (e0 != hipSuccess) return to_status(e0);
    }
    float* ws = reinterpret_cast<float*>(rest);
    hipError_t e = launch_gate_up(plan_tile_variant(p), x, xsum, wq_g, s_g, b_g, wq_u, s_u, b_u, h, ws, m, n, k,
                                  p.split_k, s);
    if (e != hipSuccess || p.split_k == 1) return to_status(e);
    return to_status(launch_splitk_reduce_glu(ws, h, M * N, p.split_k, s));
}

// Width-generic matvec: bits in {1, 2, 3, 4, 8}, M <= 8.  Routing by (bits, M), measured on
// MI355X (K = 2560 .. 9728, N = 1024 .. 151936, M = 1 .. 8, random data): the row-amortized
// kernel is never more than 7% behind the per-row one and up to 35% ahead of it (the 151936-
// column head), at every width and row count, so the policy takes it; at 4 bits the policy is
// that of qmv_w4a16, whose kernel families include the same row-amortized kernel.
bool bits_ok(int32_t bits) { return bits == 1 || bits == 2 || bits == 3 || bits == 4 || bits == 8; }

int plan_qmv_affine(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, int32_t mode, int32_t num_cus,
                    w4a16_plan_t* p) {
    if (!p) return W4A16_ERR_NULL;
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    if (!bits_ok(bits) || M > kQmvMaxRows || mode < W4A16_QMV_POLICY || mode > W4A16_QMV_BURST)
        return W4A16_ERR_UNSUPPORTED;
    if (mode == W4A16_QMV_PER_ROW && M > kQmvPerRowMaxRows) return W4A16_ERR_UNSUPPORTED;
    if (mode == W4A16_QMV_FAMILIES && bits != 4) return W4A16_ERR_UNSUPPORTED;
    QmvBurstShape burst{};
    const bool burst_fits = qmv_bits_burst_shape(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), &burst);
    if (mode == W4A16_QMV_BURST && !burst_fits) return W4A16_ERR_UNSUPPORTED;
    int32_t cus = num_cus;
    if (cus <= 0) {
        st = query_num_cus(&cus);
        if (st != W4A16_OK) return st;
    }
    // Measured on MI355X (graph replay over rotating weights): the burst form leads the
    // row-amortized kernel at every width where it applies -- at M = 1 by 10-25% on 2560 -> 9728
    // (1, 2, 3, 8 bits: 6.5 / 6.6 / 7.3 / 7.7 us against 7.3 / 7.6 / 8.1 / 10.3), by 35-42% on
    // 9728 -> 2560 and by 25-40% on 2560 -> 1024; at M = 4 on 2560 -> 1024 by 21-37%; the
    // 16-column form at M = 4 on 2560 -> 9728 and 4096 by 2-15% (8 bits: 9.9 against 11.6 us),
    // at M = 8 by 0-11% (within 1% at 1 and 2 bits on 4096 columns).
    if (mode == W4A16_QMV_POLICY)
        mode = bits == 4 ? W4A16_QMV_FAMILIES : (burst_fits ? W4A16_QMV_BURST : W4A16_QMV_AMORTIZED);
    if (mode == W4A16_QMV_FAMILIES) {
        plan_qmv(M, N, K, cus, p);
        p->num_cus = cus;
        p->variant = mode;
        return W4A16_OK;
    }
    if (mode == W4A16_QMV_BURST) {
        p->path = W4A16_PATH_QMV;
        p->tile_m = burst.rows;
        p->tile_n = burst.cols;
        p->tile_k = W4A16_GROUP;
        p->grid_x = static_cast<int32_t>(ceil_div(N, burst.cols));
        p->grid_y = 1;
        p->grid_z = 1;
        p->block_threads = 64 * burst.kw;
        p->split_k = 1;
        p->k_waves = burst.kw;
        p->num_cus = cus;
        p->variant = mode;
        p->workspace_bytes = 0;
        return W4A16_OK;
    }
    p->path = W4A16_PATH_QMV;
    p->tile_m = mode == W4A16_QMV_PER_ROW ? static_cast<int32_t>(kQmvPerRowMaxRows) : static_cast<int32_t>(kQmvKernelRows);
    p->tile_n = 16;
    p->tile_k = W4A16_GROUP;
    p->grid_x = static_cast<int32_t>(ceil_div(N, 16));
    p->grid_y = 1;
    p->grid_z = 1;
    p->block_threads = 64 * kQmvBitsWaves;
    p->split_k = 1;
    p->k_waves = kQmvBitsWaves;
    p->num_cus = cus;
    p->variant = mode;
    p->workspace_bytes = 0;
    return W4A16_OK;
}

int run_qmv_affine(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b, uint16_t* y,
                   int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, int32_t mode, void* stream) {
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    if (!bits_ok(bits)) return W4A16_ERR_UNSUPPORTED;
    st = check_buffers(x, wq, s, b, y, M, N, K, bits);
    if (st != W4A16_OK) return st;
    w4a16_plan_t p;
    st = plan_qmv_affine(M, N, K, group, bits, mode, 0, &p);
    if (st != W4A16_OK) return st;
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (p.variant == W4A16_QMV_FAMILIES) {
        plan_qmv(M, N, K, p.num_cus, &p);
        return to_status(launch_qmv(p.variant, x, wq, s, b, y, m, n, k, hs));
    }
    if (p.variant == W4A16_QMV_BURST) return to_status(launch_qmv_bits_burst(bits, x, wq, s, b, y, m, n, k, hs));
    return to_status(launch_qmv_bits(bits, p.variant == W4A16_QMV_PER_ROW ? kQmvBitsRows : kQmvBitsMatrix, x, wq, s,
                                     b, y, m, n, k, hs));
}

// W4A8 (int8 activations, "Feature Request: Metal prefill speedup (~68%) on M5 Max", feature
// list and Related work): tiles of 32 rows up to 32 rows, 64 up to ~1k, 128 beyond; the split
// rule of the W4A16 tiles.  workspace_bytes covers the fp32 partials only.
void plan_w4a8(int64_t M, int64_t N, int64_t K, int32_t split_k, int32_t cus, w4a16_plan_t* p) {
    plan_qmm(M, N, K, split_k, cus, p, M <= kSkinnyMaxRows, false);
    int variant = M <= kSkinnyMaxRows ? 0 : (M <= 1024 ? 1 : 2);
    // at most one work unit per compute unit: two waves per column block, as for the W4A16 tiles
    if (variant == 1 && ceil_div(M, 64) * ceil_div(N, 128) * p->split_k <= cus) variant = kW4A8KSplitVariant;
    const QmmShape& v = kW4A8Variants[variant];
    const int64_t tile_n = v.tile_n();
    if (v.bm != p->tile_m || tile_n != p->tile_n) {
        p->tile_m = v.bm;
        p->tile_n = static_cast<int32_t>(tile_n);
        p->grid_x = static_cast<int32_t>(ceil_div(N, tile_n));
        p->grid_y = static_cast<int32_t>(ceil_div(M, v.bm));
    }
    p->path = W4A16_PATH_W4A8;
    p->block_threads = 64 * v.nwaves;
    p->k_waves = v.ksplit;
    p->variant = variant;
    p->workspace_bytes = p->split_k > 1 ? static_cast<uint64_t>(p->split_k) * M * N * sizeof(float) : 0;
}

int make_w4a8_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, int32_t num_cus,
                   w4a16_plan_t* out) {
    if (!out) return W4A16_ERR_NULL;
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    if (split_k < 0) return W4A16_ERR_SHAPE;
    int32_t cus = num_cus;
    if (cus <= 0) {
        st = query_num_cus(&cus);
        if (st != W4A16_OK) return st;
    }
    plan_w4a8(M, N, K, split_k, cus, out);
    out->num_cus = cus;
    return W4A16_OK;
}

// Byte sizes of the activation buffers that w4a8_linear carves from its workspace.
struct W4A8Act {
    uint64_t xq, sx, xsum, total;
};
W4A8Act w4a8_act_bytes(int64_t M, int64_t K) {
    W4A8Act a;
    a.xq = round256(static_cast<uint64_t>(M) * K);
    a.sx = round256(static_cast<uint64_t>(M) * sizeof(float));
    a.xsum = round256(static_cast<uint64_t>(M) * w4a8_xsum_cols(static_cast<int>(K)) * 2);
    a.total = a.xq + a.sx + a.xsum;
    return a;
}

int run_quantize_rows(const uint16_t* x, int8_t* xq, float* sx, uint16_t* xsum, int64_t M, int64_t K,
                      int32_t group, void* stream) {
    int st = check_shape(M, 1, K, group);
    if (st != W4A16_OK) return st;
    if (!x || !xq || !sx || !xsum) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(sx, 4) || !aligned(xsum, 16)) return W4A16_ERR_ALIGN;
    const uint64_t nx = static_cast<uint64_t>(M) * K * 2, nq = static_cast<uint64_t>(M) * K,
                   ns = static_cast<uint64_t>(M) * 4,
                   nk = static_cast<uint64_t>(M) * w4a8_xsum_cols(static_cast<int>(K)) * 2;
    if (overlaps(x, nx, xq, nq) || overlaps(x, nx, sx, ns) || overlaps(x, nx, xsum, nk) || overlaps(xq, nq, sx, ns) ||
        overlaps(xq, nq, xsum, nk) || overlaps(sx, ns, xsum, nk))
        return W4A16_ERR_OVERLAP;
    return to_status(launch_quantize_rows_int8(x, xq, sx, xsum, static_cast<int>(M), static_cast<int>(K),
                                               w4a8_xsum_cols(static_cast<int>(K)), static_cast<hipStream_t>(stream)));
}

int run_w4a8(const int8_t* xq, const float* sx, const uint16_t* xsum, const uint32_t* wq, const uint16_t* s,
             const uint16_t* b, uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k,
             void* workspace, size_t ws_bytes, void* stream) {
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    if (!xq || !sx || !xsum || !wq || !s || !b || !y) return W4A16_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(sx, 4) || !aligned(xsum, 16) || !aligned(wq, 16) || !aligned(s, 2) ||
        !aligned(b, 2) || !aligned(y, 2))
        return W4A16_ERR_ALIGN;
    {
        const uint64_t ny = static_cast<uint64_t>(M) * N * 2, sb = static_cast<uint64_t>(N) * (K / W4A16_GROUP) * 2;
        if (overlaps(y, ny, xq, static_cast<uint64_t>(M) * K) || overlaps(y, ny, sx, static_cast<uint64_t>(M) * 4) ||
            overlaps(y, ny, xsum, static_cast<uint64_t>(M) * w4a8_xsum_cols(static_cast<int>(K)) * 2) ||
            overlaps(y, ny, wq, static_cast<uint64_t>(N) * K / 2) || overlaps(y, ny, s, sb) || overlaps(y, ny, b, sb))
            return W4A16_ERR_OVERLAP;
    }
    if (split_k < 0) return W4A16_ERR_SHAPE;
    w4a16_plan_t p;
    st = make_w4a8_plan(M, N, K, group, split_k, 0, &p);
    if (st != W4A16_OK) return st;
    if (p.split_k > 1) {
        const bool ws_ok = workspace != nullptr && aligned(workspace, 16) && ws_bytes >= p.workspace_bytes;
        if (!ws_ok) {
            if (split_k > 1) return workspace != nullptr && !aligned(workspace, 16) ? W4A16_ERR_ALIGN
                                                                                     : W4A16_ERR_WORKSPACE;
            plan_w4a8(M, N, K, 1, p.num_cus, &p);   // the unsplit plan computes the same result
        }
    }
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    float* ws = static_cast<float*>(workspace);
    const int k = static_cast<int>(K);
    hipError_t e = launch_qmm_w4a8(p.variant, xq, sx, xsum, wq, s, b, y, ws, static_cast<int>(M), static_cast<int>(N),
                                   k, w4a8_xsum_cols(k), p.split_k, hs);
    if (e != hipSuccess || p.split_k == 1) return to_status(e);
    return to_status(launch_splitk_reduce(ws, y, M * N, p.split_k, hs));
}

int run_w4a8_linear(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b, uint16_t* y,
                    int64_t M, int64_t N, int64_t K, int32_t group, void* workspace, size_t ws_bytes, void* stream) {
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    st = check_buffers(x, wq, s, b, y, M, N, K);
    if (st != W4A16_OK) return st;
    if (!workspace) return W4A16_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return W4A16_ERR_ALIGN;
    const W4A8Act a = w4a8_act_bytes(M, K);
    if (ws_bytes < a.total) return W4A16_ERR_WORKSPACE;
    uint8_t* base = static_cast<uint8_t*>(workspace);
    int8_t* xq = reinterpret_cast<int8_t*>(base);
    float* sx = reinterpret_cast<float*>(base + a.xq);
    uint16_t* xsum = reinterpret_cast<uint16_t*>(base + a.xq + a.sx);
    st = run_quantize_rows(x, xq, sx, xsum, M, K, group, stream);
    if (st != W4A16_OK) return st;
    return run_w4a8(xq, sx, xsum, wq, s, b, y, M, N, K, group, 0, base + a.total, ws_bytes - a.total, stream);
}

// Device scratch of w4a16_linear_noalloc (for callers that cannot allocate): the exact-code
// form's activation group sums and the split-K partials of its plans.  Every GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` only names the symbol;
// its device address, per device, comes from hipGetSymbolAddress (g_scratch below).
constexpr size_t kScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[64];   // device address of `scratch` per device, set on the first call there

// The current device's address of `scratch`, resolved once per device with that device current.
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return W4A16_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return W4A16_ERR_DEVICE;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return W4A16_OK;
}

// w4a16_linear with its workspace in `scratch`: the policy plan is fitted to the scratch (no
// exact-code form, then no split, when it needs more; same result), a forced split whose
// partials do not fit is rejected.  Nothing here allocates; every partial and group sum a launch
// reads is written by an earlier launch of the same call, so the scratch needs no clearing.
int run_linear_noalloc(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b, uint16_t* y,
                       int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, void* stream) {
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    st = check_buffers(x, wq, s, b, y, M, N, K);
    if (st != W4A16_OK) return st;
    if (split_k < 0) return W4A16_ERR_SHAPE;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != W4A16_OK) return st;
    return run_qmm(x, wq, s, b, y, M, N, K, group, W4A16_PATH_AUTO, split_k, ws, kScratchBytes, stream);
}

}  // namespace

namespace w4a16 {

LaunchTiming& launch_timing() {
    thread_local LaunchTiming t;
    return t;
}

}  // namespace w4a16

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

int w4a16_time_next_launch(void* start_event, void* stop_event) {
    w4a16::launch_timing() = w4a16::LaunchTiming{static_cast<hipEvent_t>(start_event),
                                                  static_cast<hipEvent_t>(stop_event)};
    return W4A16_OK;
}

const char* w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "W4A16_OK";
        case W4A16_ERR_NULL: return "W4A16_ERR_NULL";
        case W4A16_ERR_SHAPE: return "W4A16_ERR_SHAPE";
        case W4A16_ERR_GROUP: return "W4A16_ERR_GROUP";
        case W4A16_ERR_ALIGN: return "W4A16_ERR_ALIGN";
        case W4A16_ERR_WORKSPACE: return "W4A16_ERR_WORKSPACE";
        case W4A16_ERR_UNSUPPORTED: return "W4A16_ERR_UNSUPPORTED";
        case W4A16_ERR_LAUNCH: return "W4A16_ERR_LAUNCH";
        case W4A16_ERR_DEVICE: return "W4A16_ERR_DEVICE";
        case W4A16_ERR_OVERLAP: return "W4A16_ERR_OVERLAP";
        default: return "unknown";
    }
}

int w4a16_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t path, int32_t split_k, int32_t num_cus,
               w4a16_plan_t* out) {
    return make_plan(M, N, K, group, path, split_k, num_cus, out);
}

uint64_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, int32_t num_cus) {
    w4a16_plan_t p;
    if (make_plan(M, N, K, group, W4A16_PATH_AUTO, 0, num_cus, &p) != W4A16_OK) return 0;
    return p.workspace_bytes;
}

int qmv_w4a16(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, uint16_t* y,
              int64_t M, int64_t N, int64_t K, int32_t group, void* stream) {
    int st = check_shape(M, N, K, group);
    if (st != W4A16_OK) return st;
    st = check_buffers(x, wq, scales, biases, y, M, N, K);
    if (st != W4A16_OK) return st;
    if (M > kQmvMaxRows) return W4A16_ERR_UNSUPPORTED;
    w4a16_plan_t p;
    st = make_plan(M, N, K, group, W4A16_PATH_QMV, 1, 0, &p);
    if (st != W4A16_OK) return st;
    return run_plan(p, x, wq, scales, biases, y, M, N, K, nullptr, static_cast<hipStream_t>(stream));
}

int qmm_w4a16(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, uint16_t* y,
              int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, void* workspace,
              size_t workspace_bytes, void* stream) {
    return run_qmm(x, wq, scales, biases, y, M, N, K, group, W4A16_PATH_QMM, split_k, workspace, workspace_bytes,
                   stream);
}

int w4a16_linear(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, uint16_t* y,
                 int64_t M, int64_t N, int64_t K, int32_t group, void* workspace, size_t workspace_bytes,
                 void* stream) {
    return run_qmm(x, wq, scales, biases, y, M, N, K, group, W4A16_PATH_AUTO, 0, workspace, workspace_bytes, stream);
}

int w4a16_linear_noalloc(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                         uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, void* stream) {
    return run_linear_noalloc(x, wq, scales, biases, y, M, N, K, group, split_k, stream);
}

int w4a16_grouped_plan(int32_t count, const int64_t* N, int64_t M, int64_t K, int32_t group, int32_t num_cus,
                       w4a16_plan_t* out) {
    return make_grouped_plan(count, N, M, K, group, num_cus, out);
}

int w4a16_linear_grouped(const uint16_t* x, int32_t count, const uint32_t* const* wq, const uint16_t* const* scales,
                         const uint16_t* const* biases, uint16_t* const* y, const int64_t* N, int64_t M, int64_t K,
                         int32_t group, void* workspace, size_t workspace_bytes, void* stream) {
    return run_grouped(x, count, wq, scales, biases, y, N, M, K, group, workspace, workspace_bytes, stream);
}

int qmv_affine_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, int32_t mode, int32_t num_cus,
                    w4a16_plan_t* out) {
    return plan_qmv_affine(M, N, K, group, bits, mode, num_cus, out);
}

int qmv_affine(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, uint16_t* y,
               int64_t M, int64_t N, int64_t K, int32_t group, int32_t bits, int32_t mode, void* stream) {
    return run_qmv_affine(x, wq, scales, biases, y, M, N, K, group, bits, mode, stream);
}

int w4a16_gate_up_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, int32_t num_cus,
                       w4a16_plan_t* out) {
    return make_gate_up_plan(M, N, K, group, split_k, num_cus, out);
}

int w4a16_gate_up_swiglu(const uint16_t* x, const uint32_t* wq_gate, const uint16_t* scales_gate,
                         const uint16_t* biases_gate, const uint32_t* wq_up, const uint16_t* scales_up,
                         const uint16_t* biases_up, uint16_t* h, int64_t M, int64_t N, int64_t K, int32_t group,
                         int32_t split_k, void* workspace, size_t workspace_bytes, void* stream) {
    return run_gate_up(x, wq_gate, scales_gate, biases_gate, wq_up, scales_up, biases_up, h, M, N, K, group, split_k,
                       workspace, workspace_bytes, stream);
}

int64_t w4a8_xsum_cols(int64_t K) {
    if (K < 1 || K > kMaxK || K % W4A16_GROUP != 0) return 0;
    return w4a8_xsum_cols(static_cast<int>(K));
}

int w4a8_quantize_rows(const uint16_t* x, int8_t* xq, float* sx, uint16_t* xsum, int64_t M, int64_t K, int32_t group,
                       void* stream) {
    return run_quantize_rows(x, xq, sx, xsum, M, K, group, stream);
}

int w4a8_plan(int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k, int32_t num_cus, w4a16_plan_t* out) {
    return make_w4a8_plan(M, N, K, group, split_k, num_cus, out);
}

int qmm_w4a8(const int8_t* xq, const float* sx, const uint16_t* xsum, const uint32_t* wq, const uint16_t* scales,
             const uint16_t* biases, uint16_t* y, int64_t M, int64_t N, int64_t K, int32_t group, int32_t split_k,
             void* workspace, size_t workspace_bytes, void* stream) {
    return run_w4a8(xq, sx, xsum, wq, scales, biases, y, M, N, K, group, split_k, workspace, workspace_bytes, stream);
}

uint64_t w4a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, int32_t num_cus) {
    w4a16_plan_t p;
    if (make_w4a8_plan(M, N, K, group, 0, num_cus, &p) != W4A16_OK) return 0;
    return w4a8_act_bytes(M, K).total + p.workspace_bytes;
}

int w4a8_linear(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, uint16_t* y,
                int64_t M, int64_t N, int64_t K, int32_t group, void* workspace, size_t workspace_bytes, void* stream) {
    return run_w4a8_linear(x, wq, scales, biases, y, M, N, K, group, workspace, workspace_bytes, stream);
}

}  // extern "C"
