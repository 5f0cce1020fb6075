// qmm: W4A16 projection for prefill rows, tiled on the gfx950 matrix cores, with split-K.
//
// The pages' matrix path ("Week 2 Day 6: SIMD-Matrix Prefill", "From a Matvec to a Cooperative
// Tile" and Tasks 2-3) shares activations and dequantized weights across a result tile, loads
// device memory in contiguous chunks, pads the staged activation rows against bank conflicts,
// fetches one group's scale and bias once for all of its reduction sub-steps, keeps bf16
// operands with fp32 accumulators, and casts once at the final store.  Task 5 and "Benchmark
// Analysis: Identify Under-Filled Prefill Shapes" add split-K for grids with too few tiles.
//
// MI355X design (not the pages' 32x32x32 / 128-thread Apple tile):
//  * The contraction runs on v_mfma_f32_32x32x16_bf16, the bf16 shape with the higher
//    sustained rate on gfx950.
//  * Workgroup tile BM x BN with NW waves; each wave owns NB 32-column blocks for all BM rows
//    (with KS = 2 two waves share a strip, each taking half of every group's MFMA sub-steps).
//    A group's codes for the tile's columns are staged in LDS by direct loads, like the
//    activations; each wave unpacks and dequantizes only its own columns' codes, in registers,
//    once per workgroup, and every dequantized operand feeds BM / 32 MFMAs.
//  * Exact-code form (template CODES > 0, used for the 128-row projection tiles and the 64-row
//    gate / up tiles): instead of dequantizing,
//    the wave feeds the raw codes as exact bf16 integers, the matrix core returns each group's
//    P = sum_k x q in fp32, and the accumulators take acc += s * P once per group; the bias term
//    sum_g b * X (X = the activations' group sums, from act_group_sums_kernel) is one small MFMA
//    contraction per tile in the epilogue.  Fewer VALU instructions per MFMA, and no weight is
//    rounded to bf16.
//  * One pipeline step is one 128-value quantization group: the scale and bias of a column are
//    loaded once per step and serve all eight 16-value MFMA sub-steps of the group (the
//    analogue of the page's four reduction tiles per group).
//  * K mapping inside a group: lane half h = l / 32 of a wave holds words 8h .. 8h + 7 of its
//    column's group (64 contiguous codes); MFMA sub-step t takes word 8h + t from half h, so
//    its 16 reduction values are {64h + 8t + e}.  The activation fragment is read from LDS at
//    the same offsets.
//  * Activations (shared by every wave) are staged in LDS, double buffered, by the gfx950
//    direct global-to-LDS loads (global_load_lds_dwordx4): no registers and almost no VALU
//    work per staged byte.  One wave instruction writes 1 KB = four 256-byte rows.  Rows are
//    unpadded; instead the 16-byte chunk position p of row r holds activation chunk
//    p ^ (r & 7), so eight lanes reading one chunk of eight consecutive rows hit eight
//    different bank groups (conflict-free 16-byte reads).  Rows past M are loaded from row M-1
//    (in bounds); they only feed output rows that are never stored.
//  * One barrier per group: the wave's own direct loads for the next group are waited for
//    (vmcnt) before the barrier that ends the current group, and the next buffer is refilled
//    only after that barrier.  The weight registers ping-pong between even and odd groups.
//  * The dequantization of MFMA sub-step t + 1 is issued next to the MFMAs of sub-step t so the
//    VALU work hides under the matrix core.
//  * Code and activation loads are 16 bytes per lane: a column's group is 64 contiguous bytes
//    read by four lanes, the activation tile row-contiguously.  Scales and biases come as one
//    bf16 per column and group, or (SBQ = 4) four consecutive groups in one 8-byte load.
//  * Tile order: workgroup i runs on XCD i % 8; the remap below hands each XCD a contiguous run
//    of work indices, and work indices walk the tile grid in bands of up to 8 M-tiles (4 for
//    128-row tiles), N-tile by N-tile, so the workgroups resident on one XCD share activation
//    rows and weight columns in its L2.  With 128-row tiles the 64 workgroups resident on an XCD
//    cover 4 x 16 tiles instead of 8 x 8, which reads fewer activation rows per round of tiles
//    (measured at 4096 rows: L2 fetches of the gate tile 448 -> 274 MB, of down 520 -> 337 MB,
//    1.5% and 0.5% faster, outputs bit-identical; 2-tile bands measured the same).
//  * Split-K: the work index also selects one of S contiguous runs of groups (sizes differ by at
//    most one).  Each slice writes fp32 partials; splitk_reduce sums them in slice order, so the
//    result is deterministic.
#include "device_common.h"
#include "internal.h"

#include <type_traits>

namespace w4a16 {

// SiLU in fp32: z * sigmoid(z) = z / (1 + e^-z); e^-z overflows to inf for z < -88 and the
// quotient is then -0, the limit.
__device__ __forceinline__ float silu_f32(float z) { return z / (1.f + expf(-z)); }

// NP weight sets share every activation fragment: NP = 1 is the projection; NP = 2 is the
// gate / up pair with h = silu(gate) * up formed from the fp32 accumulators in the epilogue
// (the SwiGLU fused into the mat-mat of "Feature Request: Metal prefill speedup (~68%) on M5
// Max").  Weight set p of column block cb is block j = p * NB + cb.
template <int BM, int NB, int NW, int WAVES_PER_SIMD, int STAGES, int NP = 1, int CODES = 0, int SBQ = 1, int KS = 1,
          bool GRP = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD, WAVES_PER_SIMD))) void qmm_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, const uint32_t* __restrict__ wq2, const uint16_t* __restrict__ scales2,
    const uint16_t* __restrict__ biases2, uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N, int K,
    int split, int tiles_m, int tiles_n, const uint16_t* __restrict__ xsum, int KB, const QmmGroups grp) {
    // KS = 2: two waves share each column strip, one taking sub-steps 0..3 of every group and
    // the other 4..7; their partial accumulators are added through LDS at the end
    static_assert(KS == 1 || (KS == 2 && NP == 1), "K-split waves: single projections");
    constexpr int WN = NW / KS;                   // waves across the tile's columns
    constexpr int TSUB = 8 / KS;                  // MFMA sub-steps per group and wave
    constexpr int BN = WN * NB * 32;              // output columns of the tile (per weight set)
    constexpr int J = NP * NB;                    // weight blocks per wave
    static_assert(NP == 1 || NP == 2, "one projection or the gate / up pair");
    constexpr int RB = BM / 32;                   // 32-row blocks per wave
    constexpr int TILE = BM * kGroup;             // bf16 elements of one staged activation tile
    constexpr int DMA_PER_WAVE = BM / (4 * NW);   // 1 KB direct loads per wave per group
    static_assert(BM % (4 * NW) == 0 && BM % 32 == 0, "tile shape");
    static_assert(WN == 4 && NW % 4 == 0, "row & 15 of a direct load must not depend on the instruction index");
    static_assert(STAGES >= 2 && STAGES <= 3, "stage count");
    // one LDS object per stage: the compiler's wait insertion can then tell that a direct load
    // into one stage does not feed fragment reads of another
    __shared__ __attribute__((aligned(16))) uint16_t xs0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t xs2[STAGES > 2 ? TILE : 8];
    // codes of one group, per stage: each wave's J blocks of 32 columns x 64 bytes
    constexpr int CODES_BYTES = WN * J * 2048;
    __shared__ __attribute__((aligned(16))) uint8_t cs0[CODES_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t cs1[CODES_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t cs2[STAGES > 2 ? CODES_BYTES : 16];

    const int tiles = tiles_m * tiles_n;
    const int work = xcd_remap(blockIdx.x, tiles * split);
    const int z = work / tiles;
    int tm, tn;
    band_order<(BM >= 128 ? kBandM128 : kBandM)>(work - z * tiles, tiles_m, tiles_n, tm, tn);

    const int G = K >> 7;
    const int row_bytes = K >> 1;
    // SBQ = 4: scales and biases come four groups per 8-byte load, so slices start on multiples
    // of four groups (the launcher picks it only for G % 4 == 0 and 8-byte aligned arrays)
    static_assert(SBQ == 1 || (SBQ == 4 && STAGES == 2), "quad scale loads need the two-stage waits");
    const int g_units = G / SBQ;
    const int g_begin = SBQ * static_cast<int>(static_cast<int64_t>(z) * g_units / split);
    const int g_end = SBQ * static_cast<int>(static_cast<int64_t>(z + 1) * g_units / split);
    const int groups = g_end - g_begin;
    const int m0 = tm * BM;
    int n0 = tn * BN;
    // grouped launches: the split-K partials of every projection share one [split][M][NG] array
    // of the concatenated tile columns (NG = the launch's N, before a projection takes over)
    const int NG = N, n0g = n0;
    // Grouped launch: the projection that owns column tile tn takes over the weight, scale,
    // bias and output pointers and the column count (scalar selects with constant indices, so
    // the argument block is never copied to be indexed).
    if constexpr (GRP) {
        // (readfirstlane: the tile index is uniform, and saying so keeps the selects scalar)
        const int p = __builtin_amdgcn_readfirstlane(
            (grp.count > 1 && tn >= grp.tn_first[1] ? 1 : 0) + (grp.count > 2 && tn >= grp.tn_first[2] ? 1 : 0) +
            (grp.count > 3 && tn >= grp.tn_first[3] ? 1 : 0));
        auto pick = [p](auto a0, auto a1, auto a2, auto a3) { return p == 0 ? a0 : p == 1 ? a1 : p == 2 ? a2 : a3; };
        wq = pick(grp.wq[0], grp.wq[1], grp.wq[2], grp.wq[3]);
        scales = pick(grp.s[0], grp.s[1], grp.s[2], grp.s[3]);
        biases = pick(grp.b[0], grp.b[1], grp.b[2], grp.b[3]);
        y = pick(grp.y[0], grp.y[1], grp.y[2], grp.y[3]);
        N = pick(grp.n[0], grp.n[1], grp.n[2], grp.n[3]);
        n0 = (tn - pick(grp.tn_first[0], grp.tn_first[1], grp.tn_first[2], grp.tn_first[3])) * BN;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kh = wave / WN, wn = wave % WN;     // K half (KS = 2) and column strip of this wave
    const int half = lane >> 5;
    auto clamp_records = [](int64_t bytes) { return static_cast<int>(bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes); };
    auto stage = [&](auto ic) -> uint16_t* {
        constexpr int i = decltype(ic)::value;
        if constexpr (i == 0) return xs0;
        else if constexpr (i == 1) return xs1;
        else return xs2;
    };
    auto cstage = [&](auto ic) -> uint8_t* {
        constexpr int i = decltype(ic)::value;
        if constexpr (i == 0) return cs0;
        else if constexpr (i == 1) return cs1;
        else return cs2;
    };

    // Every load goes through a buffer resource.  Loads for groups past this slice use
    // resources with zero records: they fetch nothing, write zeros, and keep the per-group load
    // count that the waits rely on.  Reads past the last row or column are out of range and
    // return zeros; only byte offsets inside a valid row go into scalar offsets.
    //
    // Activations: resource based at the tile's first row.  Instruction i of this wave fills
    // rows 4 * (i * NW + wave) + 0..3; lane l writes chunk position l % 16 of row l / 16 with
    // activation chunk (l % 16) ^ (row & 15).  Row & 15 does not depend on i (rows advance by
    // 4 * NW = 16 per instruction), so one lane offset plus a row step serves every instruction.
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x + static_cast<size_t>(m0) * K), 0,
        clamp_records(static_cast<int64_t>(M - m0) * K * 2), 0x00020000);
    const int xrow0 = 4 * wave + (lane >> 4);
    const uint32_t xvoff = static_cast<uint32_t>(xrow0 * K + (((lane & 15) ^ (xrow0 & 15)) << 3)) * 2u;
    // Weights, scales, biases: resources based at the workgroup's first column.  Lane half h of
    // column block cb takes words 8h .. 8h + 7 of its column's group (two 16-byte loads).
    const int64_t cols_left = static_cast<int64_t>(N - n0);
    __amdgpu_buffer_rsrc_t wrsrc[NP], srsrc[NP], brsrc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const uint32_t* wp = p == 0 ? wq : wq2;
        const uint16_t* sp = p == 0 ? scales : scales2;
        const uint16_t* bp = p == 0 ? biases : biases2;
        wrsrc[p] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(wp) + static_cast<size_t>(n0) * row_bytes), 0,
            clamp_records(cols_left * row_bytes), 0x00020000);
        srsrc[p] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sp + static_cast<size_t>(n0) * G), 0,
                                                     clamp_records(cols_left * G * 2), 0x00020000);
        brsrc[p] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(bp + static_cast<size_t>(n0) * G), 0,
                                                     clamp_records(cols_left * G * 2), 0x00020000);
    }
    auto dead = [&](__amdgpu_buffer_rsrc_t r) {
        (void)r;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, 0, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t none = dead(xrsrc);
    // Codes go through LDS by direct loads that read whole 64-byte column groups: instruction i
    // of block cb fills 16 columns, lane l taking column 16 i + l / 4 and writing its 16 bytes to
    // slot l % 4 of that column's 64 bytes.  Slot p holds chunk p ^ ((column / 4) & 3), so the 16
    // lanes that later read one chunk of 16 consecutive columns hit 16 different bank groups.
    // (column / 4) & 3 = (l / 16) & 3 for both instructions.
    uint32_t cvoff[NB], sbvoff[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        const int c = (wn * NB + cb) * 32 + (lane & 31);       // column within the tile
        cvoff[cb] = static_cast<uint32_t>(((wn * NB + cb) * 32 + (lane >> 2)) * row_bytes +
                                          16 * ((lane & 3) ^ ((lane >> 4) & 3)));
        sbvoff[cb] = static_cast<uint32_t>(c * G * 2);
    }
    // this lane's two chunks (2 half, 2 half + 1) of its column's group in a stage's code block
    const int ccol = lane & 31;
    const int cread0 = ccol * 64 + 16 * ((2 * half) ^ ((ccol >> 2) & 3));
    const int cread1 = ccol * 64 + 16 * ((2 * half + 1) ^ ((ccol >> 2) & 3));

    // packed bf16 scale (bias) bits of one block: one value (SBQ = 1) or four consecutive
    // groups starting at a multiple of four, group r % 4 in bits 16 (r % 4) .. (SBQ = 4)
    struct Slot {
        uint64_t s[J], b[J];
    };
    // this slot's value for relative group r (bf16 bits)
    auto sb_bits = [](uint64_t v, int r) -> uint32_t {
        if constexpr (SBQ == 1) {
            (void)r;
            return static_cast<uint32_t>(v);
        } else {
            return static_cast<uint32_t>(v >> (16 * (r & 3))) & 0xFFFFu;
        }
    };
    // exact-code mode reads the biases once, in the epilogue.  With SBQ = 4 only the first group
    // of each four loads scales and biases (the wait before each group is vmcnt(0) with two
    // stages, so the count may vary); the others copy them from the previous group's slot.
    constexpr int kLoadsPerGroup = DMA_PER_WAVE + (2 / KS) * J + (CODES > 0 ? 1 : 2) * J;
    // all loads of group g (relative index j = g - g_begin) into stage / slot ic; prev is the
    // slot of group j - 1
    auto issue = [&](int j, auto ic, Slot& o, const Slot& prev, auto quad) {
        const bool live = j >= 0 && j < groups;
        const int g = g_begin + (live ? j : 0);
        const __amdgpu_buffer_rsrc_t xr = live ? xrsrc : none;
        uint16_t* xt = stage(ic);
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; ++i) {
            uint16_t* dst = xt + __builtin_amdgcn_readfirstlane(4 * (i * NW + wave) * kGroup);
            const uint32_t voff = xvoff + static_cast<uint32_t>(i) * (4 * NW * 2) * static_cast<uint32_t>(K);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, voff, static_cast<uint32_t>(g) * (kGroup * 2), 0, 0);
        }
        // the empty asm statements keep every load a separate instruction, so the per-group
        // count used by the waits is exact
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int p = j / NB, cb = j % NB;
            const __amdgpu_buffer_rsrc_t wr = live ? wrsrc[p] : none;
            const __amdgpu_buffer_rsrc_t sr = live ? srsrc[p] : none;
            const __amdgpu_buffer_rsrc_t br = live ? brsrc[p] : none;
            uint8_t* cdst = cstage(ic) + (wn * J + j) * 2048;
            // (offsets go through locals: an array element as a builtin operand made the host pass
            // drop the kernel's launch stub)
            const uint32_t co = cvoff[cb], cg = static_cast<uint32_t>(g) * 64u;
            if constexpr (KS == 1) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, cdst, 16, co, cg, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, cdst + 1024, 16, co + 16u * static_cast<uint32_t>(row_bytes),
                                                         cg, 0, 0);
            } else {   // the two waves of a strip load one half of its columns each
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr, cdst + __builtin_amdgcn_readfirstlane(kh * 1024), 16,
                    co + 16u * static_cast<uint32_t>(kh) * static_cast<uint32_t>(row_bytes), cg, 0, 0);
            }
            asm volatile("" ::: "memory");
            if constexpr (SBQ == 1) {
                (void)prev;
                (void)quad;
                o.s[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, sbvoff[cb], g * 2, 0);
                asm volatile("" ::: "memory");
                if constexpr (CODES == 0) {
                    o.b[j] = __builtin_amdgcn_raw_buffer_load_b16(br, sbvoff[cb], g * 2, 0);
                    asm volatile("" ::: "memory");
                } else {
                    (void)br;
                    o.b[j] = 0;
                }
            } else if constexpr (decltype(quad)::value) {   // group j = 0 mod 4
                o.s[j] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(sr, sbvoff[cb], g * 2, 0));
                asm volatile("" ::: "memory");
                if constexpr (CODES == 0) {
                    o.b[j] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(br, sbvoff[cb], g * 2, 0));
                    asm volatile("" ::: "memory");
                } else {
                    (void)br;
                    o.b[j] = 0;
                }
            } else {
                o.s[j] = prev.s[j];
                o.b[j] = prev.b[j];
            }
        }
    };

    // LDS element offset of the A fragment of sub-step t for this lane (row block 0):
    // row r = lane % 32, chunk 8 * half + t stored at position (8 * half + t) ^ (r & 15)
    // = 8 * (half ^ (r >> 3 & 1)) + (t ^ (r & 7)); with the row part a multiple of 128 this is
    // one lane constant XOR (t << 3).
    const int arow = lane & 31;
    // (with KS = 2 this wave's sub-steps start at 4 kh: chunk 8 half + 4 kh + tt)
    const int abase = (arow * kGroup + (((half ^ ((arow >> 3) & 1)) << 6) | ((arow & 7) << 3))) ^ (kh << 5);

    f32x16_t acc[RB][J];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rb][j][r] = 0.f;

    // One group: eight MFMA sub-steps.  Operands are double buffered by sub-step parity: while
    // the MFMAs of sub-step t run, the fragment reads and the dequantization of sub-step t + 1
    // are already issued.  The scheduling barrier at the end of each sub-step bounds the live
    // registers to two sub-steps' operands.
    // Exact-code mode (CODES > 0): the matrix core multiplies the raw codes (exact bf16
    // integers), giving the group's P = sum_k x q in fp32, which is scaled into the accumulators,
    // acc += s * P.  CODES == 1 scales group t at the start of group t + 1, before its first
    // MFMA overwrites the one P set, while that group's LDS reads complete; CODES == 2 spreads
    // the scaling of group t over the MFMAs of group t + 1 (a ring of STAGES P sets, one per
    // pipeline position).  The bias term sum_g b X is added
    // once per tile from the group sums of the activations.
    constexpr int PSETS = CODES == 2 ? STAGES : 1;
    f32x16_t Pr[PSETS][RB][J];
    float s_last[J];
#pragma unroll
    for (int j = 0; j < J; ++j) s_last[j] = 0.f;
#pragma unroll
    for (int i = 0; i < PSETS; ++i)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) Pr[i][rb][j][r] = 0.f;
    // this lane's code words of block j: words 8 half .. 8 half + 7 of its column's group
    // (KS = 2: the four of this wave's sub-steps, 8 half + 4 kh ..)
    constexpr int WCH = 2 / KS;   // 16-byte chunks per lane and block
    const int cread_k = kh ? cread1 : cread0;
    auto read_codes = [&](auto ic, u32x4_t (&w)[J][WCH]) {
        const uint8_t* cb = cstage(ic) + wn * J * 2048;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if constexpr (KS == 1) {
                w[j][0] = *reinterpret_cast<const u32x4_t*>(cb + j * 2048 + cread0);
                w[j][1] = *reinterpret_cast<const u32x4_t*>(cb + j * 2048 + cread1);
            } else {
                w[j][0] = *reinterpret_cast<const u32x4_t*>(cb + j * 2048 + cread_k);
            }
        }
    };

    auto compute_codes = [&](auto ic, const Slot& o, auto pc, int r) {
        constexpr int PC = PSETS == 1 ? 0 : decltype(pc)::value;
        constexpr int PP = PSETS == 1 ? 0 : (PC + STAGES - 1) % STAGES;
        const uint16_t* xt = stage(ic);
        u32x4_t ow[J][WCH];
        read_codes(ic, ow);
        bf16x8_t a[2][RB], bw[2][J];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) a[0][rb] = *reinterpret_cast<const bf16x8_t*>(xt + abase + rb * 32 * kGroup);
        if constexpr (PSETS == 1) {
            // the previous group's scaling (s_last = 0 before the first group), issued while this
            // group's LDS reads complete and after the previous group's MFMAs have drained
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int j = 0; j < J; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[rb][j][r] = __builtin_fmaf(s_last[j], Pr[0][rb][j][r], acc[rb][j][r]);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) bw[0][j] = codes_bf16_natural(ow[j][0][0]);
#pragma unroll
        for (int t = 0; t < TSUB; ++t) {
            const int cur = t & 1, nxt = cur ^ 1;
            if (t < TSUB - 1) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    a[nxt][rb] = *reinterpret_cast<const bf16x8_t*>(xt + (abase ^ ((t + 1) << 3)) + rb * 32 * kGroup);
#pragma unroll
                for (int j = 0; j < J; ++j) bw[nxt][j] = codes_bf16_natural(ow[j][(t + 1) >> 2][(t + 1) & 3]);
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const f32x16_t zero = {};
                    Pr[PC][rb][j] = mfma32x32x16(a[cur][rb], bw[cur][j], t == 0 ? zero : Pr[PC][rb][j]);
                }
            if constexpr (PSETS > 1) {
                // a TSUB-th of the previous group's scaling per sub-step
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int j = 0; j < J; ++j)
#pragma unroll
                        for (int r = 2 * KS * t; r < 2 * KS * (t + 1); ++r)
                            acc[rb][j][r] = __builtin_fmaf(s_last[j], Pr[PP][rb][j][r], acc[rb][j][r]);
            }
            // the next sub-step's fragment reads first, then each MFMA followed by a share of the
            // conversion and scaling VALU (measured 0.7-2.9% faster on the 1024- and 4096-row
            // exact-code tiles than reads spread between the MFMAs)
            __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);                                 // LDS reads
#pragma unroll
            for (int i = 0; i < RB * J; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, (11 * J + 2 * RB * J + RB * J - 1) / (RB * J), 0);  // VALU
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) s_last[j] = bf16_bits_to_f32(sb_bits(o.s[j], r));
    };

    // Dequantizing mode: the MFMAs of a group's last sub-step are issued at the start of the
    // next group, right after that group's LDS reads (code words and first activation
    // fragments), so the matrix core works while those reads and the first dequantization
    // complete instead of idling after the barrier.  Their operands wait in registers; they
    // are zero before the first group (adding exact zeros) and issued after the last group.
    // Each accumulator still takes its MFMAs in the same order, so results are unchanged.
    bf16x8_t pend_a[RB], pend_b[J];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) pend_a[rb] = bf16x8_t{};
#pragma unroll
    for (int j = 0; j < J; ++j) pend_b[j] = bf16x8_t{};
    auto compute = [&](auto ic, const Slot& o, int r) {
        u32x4_t ow[J][WCH];
        read_codes(ic, ow);
        float s[J], b[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            s[j] = bf16_bits_to_f32(sb_bits(o.s[j], r));
            b[j] = bf16_bits_to_f32(sb_bits(o.b[j], r));
        }
        const uint16_t* xt = stage(ic);
        bf16x8_t a[2][RB], bw[2][J];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) a[0][rb] = *reinterpret_cast<const bf16x8_t*>(xt + abase + rb * 32 * kGroup);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < J; ++j) acc[rb][j] = mfma32x32x16(pend_a[rb], pend_b[j], acc[rb][j]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < J; ++j) bw[0][j] = dequant_word(ow[j][0][0], s[j], b[j]);
#pragma unroll
        for (int t = 0; t < TSUB; ++t) {
            const int cur = t & 1, nxt = cur ^ 1;
            if (t < TSUB - 1) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    a[nxt][rb] = *reinterpret_cast<const bf16x8_t*>(xt + (abase ^ ((t + 1) << 3)) + rb * 32 * kGroup);
#pragma unroll
                for (int j = 0; j < J; ++j)
                    bw[nxt][j] = dequant_word(ow[j][(t + 1) >> 2][(t + 1) & 3], s[j], b[j]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int j = 0; j < J; ++j) acc[rb][j] = mfma32x32x16(a[cur][rb], bw[cur][j], acc[rb][j]);
                if constexpr (RB * J == 1) {
                    // one MFMA per sub-step (32-row tiles): the next fragment read goes ahead of
                    // it, then the next sub-step's dequantization (measured 5% faster on the
                    // 24- and 32-row gate projection than the interleave below)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 21, 0);  // VALU
                } else if constexpr (KS == 1) {
                    // one wave per column strip: the next sub-step's fragment reads first, then
                    // each MFMA followed by a share of its dequantization (measured 1.2-2% faster
                    // on the 512-row q|k|v, o and down tiles than reads spread between the MFMAs)
                    __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);  // LDS reads
#pragma unroll
                    for (int i = 0; i < RB * J; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, (20 * J + RB * J - 1) / (RB * J), 0);  // VALU
                    }
                } else {
                    // interleave: each MFMA is followed by a share of the next sub-step's
                    // dequantization (VALU) and fragment reads, so the wave keeps issuing while
                    // the matrix core works
#pragma unroll
                    for (int i = 0; i < RB * J; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, (20 * J + RB * J - 1) / (RB * J), 0);  // VALU
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                          // LDS read
                    }
                }
            } else {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) pend_a[rb] = a[cur][rb];
#pragma unroll
                for (int j = 0; j < J; ++j) pend_b[j] = bw[cur][j];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // STAGES-deep pipeline over positions P = 0, 1, ...: position P loads group
    // t + STAGES - 1 into stage P % STAGES and computes group t = P - pad - (STAGES - 1) from
    // stage (P + 1) % STAGES, where pad < STAGES makes the position count a multiple of
    // STAGES, so the loop has one exit, at the end of its unrolled body (a mid-body exit made
    // the compiler copy the accumulators at every back-edge).  Before computing, a position
    // waits until only the newest STAGES - 2 groups of loads are outstanding (group t has landed
    // for this wave) and meets the other waves at the barrier (group t has landed for all of
    // them, and all have finished reading the stage about to be refilled).  Positions with
    // t < 0 only load (group indices below 0 are dead loads).  Keeping the fill inside the loop
    // (no peeled prologue) lets the compiler see that each stage's reads depend on that stage's
    // loads alone.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using C0 = std::integral_constant<int, 1 % STAGES>;
    using C1 = std::integral_constant<int, 2 % STAGES>;
    using C2 = std::integral_constant<int, 3 % STAGES>;
    // SBQ = 4 (two stages, a multiple of four groups per slice): the body has four positions
    // and three leading fill positions, so every group j = 0 mod 4 is issued at the body's last
    // position, the only one that loads scales and biases (the others copy them forward).
    using QN = std::false_type;
    using QY = std::true_type;
    Slot slot0, slot1, slot2;
    const int pad = SBQ == 4 ? 3 : (STAGES - (groups + STAGES - 1) % STAGES) % STAGES;
    int t = -(STAGES - 1) - pad;
    asm volatile("" : "+s"(t));   // opaque start: the fill iterations are not peeled off the loop
    if (groups > 0) {
#define W4A16_QMM_STEP(d, I, C, SLOT_IN, SLOT_C, Q)                                                \
        if constexpr (STAGES > d || SBQ == 4) {                                                  \
            if (t >= 0) {                                                                        \
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"((STAGES - 2) * kLoadsPerGroup) : "memory"); \
                __builtin_amdgcn_s_barrier();                                                    \
                asm volatile("" ::: "memory");                                                   \
            }                                                                                    \
            issue(t + STAGES - 1, I{}, SLOT_IN, SLOT_C, Q{});                                    \
            if (t >= 0) {                                                                        \
                if constexpr (CODES > 0) compute_codes(C{}, SLOT_C, I{}, t);                     \
                else compute(C{}, SLOT_C, t);                                                    \
            }                                                                                    \
            ++t;                                                                                 \
        }
        if constexpr (SBQ == 4) {
            for (;;) {
                W4A16_QMM_STEP(0, I0, C0, slot0, slot1, QN)
                W4A16_QMM_STEP(1, I1, C1, slot1, slot0, QN)
                W4A16_QMM_STEP(2, I0, C0, slot0, slot1, QN)
                W4A16_QMM_STEP(3, I1, C1, slot1, slot0, QY)
                if (t >= groups) break;
            }
        } else {
            for (;;) {
                W4A16_QMM_STEP(0, I0, C0, slot0, (STAGES == 3 ? slot1 : slot1), QN)
                W4A16_QMM_STEP(1, I1, C1, slot1, (STAGES == 3 ? slot2 : slot0), QN)
                W4A16_QMM_STEP(2, I2, C2, slot2, slot0, QN)
                if (t >= groups) break;
            }
        }
#undef W4A16_QMM_STEP
    }
    if constexpr (CODES == 0) {
        // the last group's deferred sub-step
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < J; ++j) acc[rb][j] = mfma32x32x16(pend_a[rb], pend_b[j], acc[rb][j]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no direct load may outlive the wave

    if constexpr (CODES > 0) {
        // the last group's scaling: its P sits in the P set of the body's last position
        constexpr int PL = PSETS == 1 ? 0 : STAGES - 1;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[rb][j][r] = __builtin_fmaf(s_last[j], Pr[PL][rb][j][r], acc[rb][j][r]);
        // bias term, once per output (slice 0, K half 0): acc += xsum . baug^T over KB / 16
        // sub-steps, with baug[n, k'] = b[n, k' / 2] (zero for k' / 2 >= G) against the hi / lo
        // halves of X
        if (z == 0 && kh == 0) {
            const __amdgpu_buffer_rsrc_t xsr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(xsum + static_cast<size_t>(m0) * KB), 0,
                clamp_records(static_cast<int64_t>(M - m0) * KB * 2), 0x00020000);
            for (int u = 0; u < KB / 16; ++u) {
                const int g0 = 8 * u + 4 * half;
                bf16x8_t bfrag[J];
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const int p = j / NB, cb = j % NB;
                    uint32_t bb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t off = sbvoff[cb] + static_cast<uint32_t>(g0 + i < G ? g0 + i : 0) * 2u;
                        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(brsrc[p], off, 0, 0);
                        bb[i] = g0 + i < G ? v : 0u;
                    }
                    bfrag[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{bb[0] | (bb[0] << 16), bb[1] | (bb[1] << 16),
                                                                    bb[2] | (bb[2] << 16), bb[3] | (bb[3] << 16)});
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const uint32_t off = static_cast<uint32_t>(((rb * 32 + arow) * KB + 16 * u + 8 * half) * 2);
                    const bf16x8_t afrag =
                        __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(xsr, off, 0, 0));
#pragma unroll
                    for (int j = 0; j < J; ++j) acc[rb][j] = mfma32x32x16(afrag, bfrag[j], acc[rb][j]);
                }
            }
        }
    }

    // KS = 2: the two waves of a strip add their partial sums.  Of the RB * 16 accumulator
    // elements e = 16 rb + r, K half 0 finishes e < 8 RB and K half 1 the rest; each writes the
    // other's elements to the activation stage of its own K half, and reads its partner's.
    if constexpr (KS == 2) {
        __syncthreads();   // every wave is done with the stages
        constexpr int HALF = RB * 8;
        static_assert(WN * HALF * J * 64 * 4 <= TILE * 2, "partial sums fit one activation stage");
        float* mine = reinterpret_cast<float*>(kh == 0 ? xs0 : xs1) + wn * HALF * J * 64;
        const float* theirs = reinterpret_cast<const float*>(kh == 0 ? xs1 : xs0) + wn * HALF * J * 64;
        // element indices stay compile-time constants (a runtime index would move acc to scratch);
        // the barrier between handing over and adding sits outside the K-half branches, so every
        // wave of the workgroup reaches the same one
        auto hand_over = [&](auto khc) {
            constexpr int off = decltype(khc)::value == 0 ? HALF : 0;   // the partner's elements
#pragma unroll
            for (int e = 0; e < HALF; ++e)
#pragma unroll
                for (int j = 0; j < J; ++j) mine[(e * J + j) * 64 + lane] = acc[(e + off) >> 4][j][(e + off) & 15];
        };
        auto add_partner = [&](auto khc) {
            constexpr int off = decltype(khc)::value == 0 ? 0 : HALF;   // this wave's elements
#pragma unroll
            for (int e = 0; e < HALF; ++e)
#pragma unroll
                for (int j = 0; j < J; ++j) acc[(e + off) >> 4][j][(e + off) & 15] += theirs[(e * J + j) * 64 + lane];
        };
        if (kh == 0)
            hand_over(std::integral_constant<int, 0>{});
        else
            hand_over(std::integral_constant<int, 1>{});
        __syncthreads();
        if (kh == 0)
            add_partner(std::integral_constant<int, 0>{});
        else
            add_partner(std::integral_constant<int, 1>{});
    }

    // epilogue: D layout puts rows 8 * (r / 4) + 4 * half + r % 4 of column lane % 32 in this lane
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (KS == 2) {
                if ((16 * rb + r < RB * 8) != (kh == 0)) continue;
            }
            const int m = m0 + rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (m >= M) continue;
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                const int col = n0 + (wn * NB + cb) * 32 + (lane & 31);
                if (col >= N) continue;
                const size_t idx = static_cast<size_t>(m) * N + col;
                if constexpr (NP == 1) {
                    if (split == 1) {
                        y[idx] = f32_to_bf16_bits(acc[rb][cb][r]);
                    } else if constexpr (GRP) {
                        ws[(static_cast<size_t>(z) * M + m) * NG + (n0g - n0) + col] = acc[rb][cb][r];
                    } else {
                        ws[static_cast<size_t>(z) * M * N + idx] = acc[rb][cb][r];
                    }
                } else {
                    // gate partials in plane 0, up partials in plane 1 (each [split][M][N])
                    const float gv = acc[rb][cb][r], uv = acc[rb][NB + cb][r];
                    if (split == 1) {
                        y[idx] = f32_to_bf16_bits(silu_f32(gv) * uv);
                    } else {
                        ws[static_cast<size_t>(z) * M * N + idx] = gv;
                        ws[(static_cast<size_t>(split) + z) * M * N + idx] = uv;
                    }
                }
            }
        }
    }
}

// Group sums of the activations for the exact-code mode: one workgroup per row; X[m, g] is the
// fp32 sum of the group's 128 values (each lane adds 8, then a fixed xor tree over the 16 lanes
// of the group), stored as hi = bf16(X) and lo = bf16(X - hi) at columns 2g and 2g + 1 of xsum
// [M, KB]; columns 2G .. KB - 1 are zero.
__global__ __launch_bounds__(256) void act_group_sums_kernel(const uint16_t* __restrict__ x,
                                                             uint16_t* __restrict__ xsum, int K, int KB) {
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const int chunks = K >> 3;
    const uint16_t* xr = x + static_cast<size_t>(m) * K;
    uint16_t* out = xsum + static_cast<size_t>(m) * KB;
    const int iters = (chunks + 255) >> 8;
    for (int it = 0; it < iters; ++it) {
        const int c = tid + 256 * it;
        const bool valid = c < chunks;     // uniform over each 16-lane group (chunks % 16 == 0)
        float v = 0.f;
        if (valid) {
            const u32x4_t q = load16(xr + 8 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) v += __uint_as_float(q[i] << 16) + __uint_as_float(q[i] & 0xFFFF0000u);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (valid && (tid & 15) == 0) {
            const int g = c >> 4;
            const uint16_t hi = f32_to_bf16_bits(v);
            out[2 * g] = hi;
            out[2 * g + 1] = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
        }
    }
    for (int k = 2 * (K >> 7) + tid; k < KB; k += 256) out[k] = 0;
}

hipError_t launch_act_group_sums(const uint16_t* x, uint16_t* xsum, int M, int K, int KB, hipStream_t stream) {
    hipLaunchKernelGGL(act_group_sums_kernel, dim3(M), dim3(256), 0, stream, x, xsum, K, KB);
    return hipGetLastError();
}

// gate / up pair: h = bf16(silu(sum_z gate partial) * sum_z up partial), slices in order
__global__ __launch_bounds__(256) void splitk_reduce_glu_kernel(const float* __restrict__ ws, uint16_t* __restrict__ h,
                                                                int64_t MN, int split) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= MN) return;
    float g = ws[i], u = ws[split * MN + i];
    for (int z = 1; z < split; ++z) {
        g += ws[z * MN + i];
        u += ws[(split + z) * MN + i];
    }
    h[i] = f32_to_bf16_bits(silu_f32(g) * u);
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ y,
                                                            int64_t MN, int split) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= MN) return;
    float v = ws[i];
    for (int z = 1; z < split; ++z) v += ws[z * MN + i];
    y[i] = f32_to_bf16_bits(v);
}

const QmmShape kQmmVariants[kNumQmmVariants] = {
    {128, 1, 4, 2},  // 0: 128 x 128 tile, 4 waves of 128 x 32, two waves per SIMD, 2 stages
    {64, 1, 4, 2},   // 1:  64 x 128 tile, 4 waves of  64 x 32, three waves per SIMD (48 KB of LDS
                     //     per workgroup: three resident per compute unit), 2 stages
    {64, 1, 4, 3},   // 2:  64 x 128 tile, two waves per SIMD, 3 stages
    {32, 1, 4, 2},   // 3:  32 x 128 tile, 4 waves of 32 x 32, four waves per SIMD, 2 stages
    {32, 1, 4, 3},   // 4:  32 x 128 tile, three waves per SIMD (48 KB of LDS), 3 stages (skinny M)
    {64, 1, 8, 2, 2},  // 5:  64 x 128 tile, 8 waves: two per 32-column strip, each taking half of
                       //     every group's sub-steps; six waves per SIMD
    {96, 1, 8, 2, 2},  // 6:  96 x 128 tile, 8 waves as variant 5; four waves per SIMD (two tiles)
};

// Scales and biases four groups per load (two-stage instances) when the group count is a
// multiple of four, both arrays are 8-byte aligned and the slices stay long (their boundaries
// then fall on multiples of four groups).  Measured on MI355X at 512 rows: +3-4% on the q, gate
// and down (3 slices of 25 groups) projections, -1% on 3-4 slices of 5-11 groups.
static bool quad_scales(int K, int split, const uint16_t* s, const uint16_t* b) {
    const int G = K / kGroup;
    return G % 4 == 0 && (split == 1 || G / split >= 16) && reinterpret_cast<uintptr_t>(s) % 8 == 0 &&
           reinterpret_cast<uintptr_t>(b) % 8 == 0;
}

// grp: a grouped launch (N is then the concatenated column tiles' width, and wq, s, b, y are
// placeholders that the kernel replaces per tile), or null for one projection.
template <int BM, int NB, int NW, int WAVES_PER_SIMD, int STAGES, int CM = 0, int CODES_WPS = WAVES_PER_SIMD,
          int KS = 1, bool GROUPED_FORM = false>
static hipError_t launch_qmm_t(const uint16_t* x, const uint16_t* xsum, int KB, const uint32_t* wq, const uint16_t* s,
                               const uint16_t* b, uint16_t* y, float* ws, int M, int N, int K, int split,
                               hipStream_t stream, const QmmGroups* grp = nullptr) {
    constexpr int BN = NW / KS * NB * 32;
    static_assert(BN == kGroupedTileN, "grouped launches assume 128-column tiles");
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const dim3 grid(tiles_m * tiles_n * split);
    bool quad = STAGES == 2;
    if (grp) {
        for (int p = 0; p < grp->count; ++p) quad = quad && quad_scales(K, split, grp->s[p], grp->b[p]);
    } else {
        quad = quad && quad_scales(K, split, s, b);
    }
    // only the tile forms a grouped plan can pick are compiled in the grouped form
    if (grp && !GROUPED_FORM) return hipErrorInvalidValue;
    const QmmGroups none{};
    const QmmGroups& g = grp ? *grp : none;
#define W4A16_LAUNCH_QMM(WPS, CODES, SBQ, XS)                                                                        \
    do {                                                                                                          \
        if constexpr (GROUPED_FORM) {                                                                             \
            if (grp) {                                                                                            \
                W4A16_LAUNCH((qmm_kernel<BM, NB, NW, WPS, STAGES, 1, CODES, SBQ, KS, true>), grid,               \
                                   dim3(64 * NW), 0, stream, x, wq, s, b, nullptr, nullptr, nullptr, y, ws, M, N, K, \
                                   split, tiles_m, tiles_n, XS, KB, g);                                           \
                break;                                                                                            \
            }                                                                                                     \
        }                                                                                                         \
        W4A16_LAUNCH((qmm_kernel<BM, NB, NW, WPS, STAGES, 1, CODES, SBQ, KS>), grid, dim3(64 * NW), 0,             \
                           stream, x, wq, s, b, nullptr, nullptr, nullptr, y, ws, M, N, K, split, tiles_m, tiles_n,  \
                           XS, KB, g);                                                                            \
    } while (0)
    if constexpr (CM > 0) {
        if (xsum) {
            if constexpr (STAGES == 2) {
                if (quad) {
                    W4A16_LAUNCH_QMM(CODES_WPS, CM, 4, xsum);
                    return hipGetLastError();
                }
            }
            W4A16_LAUNCH_QMM(CODES_WPS, CM, 1, xsum);
            return hipGetLastError();
        }
    }
    if constexpr (STAGES == 2) {
        if (quad) {
            W4A16_LAUNCH_QMM(WAVES_PER_SIMD, 0, 4, nullptr);
            return hipGetLastError();
        }
    }
    W4A16_LAUNCH_QMM(WAVES_PER_SIMD, 0, 1, nullptr);
#undef W4A16_LAUNCH_QMM
    return hipGetLastError();
}

template <int BM, int WAVES_PER_SIMD, int STAGES, int CM = 0, int CODES_WPS = WAVES_PER_SIMD>
static hipError_t launch_gate_up_t(const uint16_t* x, const uint16_t* xsum, int KB, const uint32_t* wg,
                                   const uint16_t* sg, const uint16_t* bg, const uint32_t* wu, const uint16_t* su,
                                   const uint16_t* bu, uint16_t* h, float* ws, int M, int N, int K, int split,
                                   hipStream_t stream) {
    constexpr int BN = 4 * 32;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const dim3 grid(tiles_m * tiles_n * split);
    const bool quad = STAGES == 2 && quad_scales(K, split, sg, bg) && quad_scales(K, split, su, bu);
#define W4A16_LAUNCH_GU(WPS, CODES, SBQ, XS)                                                                       \
    W4A16_LAUNCH((qmm_kernel<BM, 1, 4, WPS, STAGES, 2, CODES, SBQ>), grid, dim3(256), 0, stream, x, wg, sg, bg,       \
                       wu, su, bu, h, ws, M, N, K, split, tiles_m, tiles_n, XS, KB, QmmGroups{})
    if constexpr (CM > 0) {
        if (xsum) {
            if constexpr (STAGES == 2) {
                if (quad) {
                    W4A16_LAUNCH_GU(CODES_WPS, CM, 4, xsum);
                    return hipGetLastError();
                }
            }
            W4A16_LAUNCH_GU(CODES_WPS, CM, 1, xsum);
            return hipGetLastError();
        }
    }
    if (xsum) return hipErrorInvalidValue;   // this instance runs the dequantizing form only
    if constexpr (STAGES == 2) {
        if (quad) {
            W4A16_LAUNCH_GU(WAVES_PER_SIMD, 0, 4, nullptr);
            return hipGetLastError();
        }
    }
    W4A16_LAUNCH_GU(WAVES_PER_SIMD, 0, 1, nullptr);
#undef W4A16_LAUNCH_GU
    return hipGetLastError();
}

// One tile form; grp != null makes it a grouped launch (unsplit, N = the concatenated tiles' width).
static hipError_t dispatch_qmm(int variant, const uint16_t* x, const uint16_t* xsum, const uint32_t* wq,
                               const uint16_t* scales, const uint16_t* biases, uint16_t* y, float* ws, int M, int N,
                               int K, int split, hipStream_t stream, const QmmGroups* grp) {
    const int KB = group_sum_cols(K);
    // the exact-code mode is compiled for the 128-row tiles, where it measured faster
    if (xsum && variant != kQmmCodesTileVariant) return hipErrorInvalidValue;
    switch (variant) {
        case 0: return launch_qmm_t<128, 1, 4, 2, 2, 1, 2, 1, true>(x, xsum, KB, wq, scales, biases, y, ws, M, N, K,
                                                                    split, stream, grp);
        case 1: return launch_qmm_t<64, 1, 4, 3, 2, 0, 3, 1, true>(x, nullptr, KB, wq, scales, biases, y, ws, M, N, K,
                                                                   split, stream, grp);
        case 2: return launch_qmm_t<64, 1, 4, 2, 3>(x, nullptr, KB, wq, scales, biases, y, ws, M, N, K, split, stream,
                                                     grp);
        case 3: return launch_qmm_t<32, 1, 4, 4, 2>(x, nullptr, KB, wq, scales, biases, y, ws, M, N, K, split, stream,
                                                     grp);
        case 4: return launch_qmm_t<32, 1, 4, 3, 3>(x, nullptr, KB, wq, scales, biases, y, ws, M, N, K, split, stream,
                                                     grp);
        case 5: return launch_qmm_t<64, 1, 8, 6, 2, 0, 6, 2, true>(x, nullptr, KB, wq, scales, biases, y, ws, M, N, K,
                                                                   split, stream, grp);
        case 6: return launch_qmm_t<96, 1, 8, 4, 2, 0, 4, 2, true>(x, nullptr, KB, wq, scales, biases, y, ws, M, N, K,
                                                                   split, stream, grp);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_qmm(int variant, const uint16_t* x, const uint16_t* xsum, const uint32_t* wq, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* y, float* ws, int M, int N, int K, int split,
                      hipStream_t stream) {
    return dispatch_qmm(variant, x, xsum, wq, scales, biases, y, ws, M, N, K, split, stream, nullptr);
}

int grouped_columns(const QmmGroups& groups) {
    const int last = groups.count - 1;
    return (groups.tn_first[last] + (groups.n[last] + kGroupedTileN - 1) / kGroupedTileN) * kGroupedTileN;
}

hipError_t launch_qmm_grouped(int variant, const uint16_t* x, const uint16_t* xsum, const QmmGroups& groups,
                              float* ws, int M, int K, int split, hipStream_t stream) {
    if (groups.count < 1 || groups.count > kMaxGroupedProjections || split < 1 || (split > 1 && !ws))
        return hipErrorInvalidValue;
    return dispatch_qmm(variant, x, xsum, groups.wq[0], groups.s[0], groups.b[0], groups.y[0], ws, M,
                        grouped_columns(groups), K, split, stream, &groups);
}

// Slice sums of a grouped split launch: element (m, c) of the [M][NG] partial planes belongs to
// the projection that owns column tile c / 128; y_p[m][c - 128 tn_first[p]] = bf16(sum_z), slices
// in order.  Columns past a projection's last column (its ragged tile) are skipped.
__global__ __launch_bounds__(256) void splitk_reduce_grouped_kernel(const float* __restrict__ ws, const QmmGroups g,
                                                                    int M, int NG, int split) {
    const int64_t MN = static_cast<int64_t>(M) * NG;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= MN) return;
    const int m = static_cast<int>(i / NG), c = static_cast<int>(i - static_cast<int64_t>(m) * NG);
    const int tn = c / kGroupedTileN;
    const int p = (g.count > 1 && tn >= g.tn_first[1] ? 1 : 0) + (g.count > 2 && tn >= g.tn_first[2] ? 1 : 0) +
                  (g.count > 3 && tn >= g.tn_first[3] ? 1 : 0);
    auto pick = [p](auto a0, auto a1, auto a2, auto a3) { return p == 0 ? a0 : p == 1 ? a1 : p == 2 ? a2 : a3; };
    const int n = pick(g.n[0], g.n[1], g.n[2], g.n[3]);
    const int local = c - pick(g.tn_first[0], g.tn_first[1], g.tn_first[2], g.tn_first[3]) * kGroupedTileN;
    if (local >= n) return;
    float v = ws[i];
    for (int z = 1; z < split; ++z) v += ws[z * MN + i];
    uint16_t* y = pick(g.y[0], g.y[1], g.y[2], g.y[3]);
    y[static_cast<size_t>(m) * n + local] = f32_to_bf16_bits(v);
}

hipError_t launch_splitk_reduce_grouped(const float* ws, const QmmGroups& groups, int M, int split,
                                        hipStream_t stream) {
    const int NG = grouped_columns(groups);
    const int64_t MN = static_cast<int64_t>(M) * NG;
    hipLaunchKernelGGL(splitk_reduce_grouped_kernel, dim3(static_cast<unsigned>((MN + 255) / 256)), dim3(256), 0,
                       stream, ws, groups, M, NG, split);
    return hipGetLastError();
}

const QmmShape kGateUpVariants[kNumGateUpVariants] = {
    {32, 1, 4, 2},   // 0:  32 x 128 tile of h (gate and up: 2 x 32 columns per wave), three waves per
                     //     SIMD (48 KB of LDS per workgroup)
    {64, 1, 4, 2},   // 1:  64 x 128 tile of h, two waves per SIMD (64 KB of LDS per workgroup)
    {128, 1, 4, 2},  // 2: 128 x 128 tile of h, one wave per SIMD
    {96, 1, 4, 2},   // 3:  96 x 128 tile of h, two waves per SIMD
};

hipError_t launch_gate_up(int variant, const uint16_t* x, const uint16_t* xsum, const uint32_t* wq_gate,
                          const uint16_t* s_gate, const uint16_t* b_gate, const uint32_t* wq_up, const uint16_t* s_up,
                          const uint16_t* b_up, uint16_t* h, float* ws, int M, int N, int K, int split,
                          hipStream_t stream) {
    const int KB = group_sum_cols(K);
    if (xsum && variant != kGateUpCodesTileVariant) return hipErrorInvalidValue;
    switch (variant) {
        case 0: return launch_gate_up_t<32, 3, 2>(x, xsum, KB, wq_gate, s_gate, b_gate, wq_up, s_up, b_up, h, ws, M, N, K,
                                                  split, stream);
        case 1: return launch_gate_up_t<64, 2, 2, 1, 2>(x, xsum, KB, wq_gate, s_gate, b_gate, wq_up, s_up, b_up, h, ws, M, N, K,
                                                  split, stream);
        case 2: return launch_gate_up_t<128, 1, 2>(x, xsum, KB, wq_gate, s_gate, b_gate, wq_up, s_up, b_up, h, ws, M, N,
                                                   K, split, stream);
        case 3: return launch_gate_up_t<96, 2, 2>(x, xsum, KB, wq_gate, s_gate, b_gate, wq_up, s_up, b_up, h, ws, M, N,
                                                  K, split, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_splitk_reduce_glu(const float* ws, uint16_t* h, int64_t MN, int split, hipStream_t stream) {
    const int64_t blocks = (MN + 255) / 256;
    hipLaunchKernelGGL(splitk_reduce_glu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ws, h, MN,
                       split);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* ws, uint16_t* y, int64_t MN, int split, hipStream_t stream) {
    const int64_t blocks = (MN + 255) / 256;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ws, y, MN,
                       split);
    return hipGetLastError();
}

}  // namespace w4a16
