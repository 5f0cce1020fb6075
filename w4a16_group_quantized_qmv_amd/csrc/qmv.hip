// qmv: W4A16 projection for decode rows (M <= 16 in the kernel; the C ABI serves M <= 8).
//
// The pages keep a dedicated matvec for M <= 8 ("Week 2 Day 6: SIMD-Matrix Prefill", Task 1)
// and reuse one dequantized group across all M input rows ("Route affine qmv_wide by
// bit-width and batch size #5").  On gfx950 the reuse across rows is done by the matrix core:
// the M rows (zero-padded to 16) form the A operand of v_mfma_f32_16x16x32_bf16 and 16 weight
// columns form B, so one unpacked group of codes serves every row at no VALU cost per row.
//
// Arithmetic per (column n, group g), with P = sum_{k in g} x[m,k] * q[n,k] and
// X = sum_{k in g} x[m,k] (both fp32, from the matrix core):
//     y[m, n] += s[n, g] * P + b[n, g] * X
// which is sum_{k in g} x[m,k] * (s q + b) regrouped.  The codes enter the MFMA as exact bf16
// integers (see codes_bf16_permuted), so no weight is rounded before the contraction.
//
// Memory (the kernel is bound by HBM bandwidth):
//  * Weights stream once, through the gfx950 direct global-to-LDS buffer loads: no registers
//    and no VALU work per loaded byte.  One load instruction moves 8 columns x 128 contiguous
//    bytes (the two groups of a group pair), so every request is a whole 128-byte line; loads
//    of 16 columns x 64 bytes measured about 20% slower on MI355X.
//  * The destination slot of each 16-byte chunk is permuted so that the MFMA operand read --
//    16 lanes, one per column, same group and same 32-value quarter -- touches 16 different
//    bank groups (conflict free).  Reads past the last column hit the buffer bound and return
//    zeros; those columns are never stored.
//  * Each wave owns a private double-buffered LDS region: the next group pair streams in while
//    the current one is computed, with no workgroup barrier.
//  * Activations, scales and biases are small and L2-resident; they are prefetched one group
//    pair ahead in registers.
// A workgroup is wn x kw waves: wn waves side by side along N, kw waves splitting the group
// pairs of the same columns; the kw partial sums are added in wave order through LDS, so the
// result does not depend on timing.
#include "device_common.h"
#include "internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace w4a16 {

namespace {

constexpr int kPairBytes = 2048;   // one 16-column block x one group pair of packed codes

// bytes of permuted activations in the wide kernel's dynamic LDS (whole 1 KB units)
__device__ __forceinline__ int qmv_wide_x_bytes(int M, int K) { return (M * (K >> 3) + 63) / 64 * 1024; }

// LDS byte offset (within a block's 2 KB) of the 16-byte chunk h of column c, group g (0/1):
// columns 0..7 fill the first kilobyte, columns 8..15 the second, and within each kilobyte the
// slot is 16 * h + (c % 8) + 8 * (g or 1 - g) so that c = 0..15 at fixed (g, h) cover all
// sixteen 16-byte bank groups.
__device__ __forceinline__ int pair_slot(int c, int g, int h) {
    return c < 8 ? 16 * (16 * h + c + 8 * g) : 1024 + 16 * (16 * h + (c - 8) + 8 * (1 - g));
}

}  // namespace

template <int CB, int WN, int KW>
__global__ __launch_bounds__(64 * WN * KW) void qmv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int N, int K) {
    // two separate LDS objects (not one array indexed by buffer): the compiler's wait
    // insertion can then tell that a direct load into one buffer does not feed reads of the other
    __shared__ __attribute__((aligned(16))) uint8_t wbuf0[WN * KW][CB * kPairBytes];
    __shared__ __attribute__((aligned(16))) uint8_t wbuf1[WN * KW][CB * kPairBytes];

    const int G = K >> 7;
    const int pairs = (G + 1) >> 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps resources in SGPRs
    const int wn = wave % WN;
    const int wk = wave / WN;
    const int col0 = (blockIdx.x * WN + wn) * (CB * 16);
    const int p0 = static_cast<int>(static_cast<int64_t>(wk) * pairs / KW);
    const int p1 = static_cast<int>(static_cast<int64_t>(wk + 1) * pairs / KW);
    const int c = lane & 15;      // column within a 16-column block (B operand / D layout)
    const int kq = lane >> 4;     // 32-value quarter of each group held by this lane
    const int arow = lane & 15;   // activation row fed by this lane (A operand)
    const bool arow_ok = arow < M;
    const int row_bytes = K >> 1;

    // weight stream: buffer resource based at this wave's first column; reads past the last
    // column fall outside the resource and return zeros
    const uint8_t* wbase = reinterpret_cast<const uint8_t*>(wq) + static_cast<size_t>(col0) * row_bytes;
    const int64_t wbytes = col0 < N ? static_cast<int64_t>(N - col0) * row_bytes : 0;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(wbase), 0, static_cast<int>(wbytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : wbytes), 0x00020000);
    // load lane l fills slot l of each kilobyte: invert pair_slot for its column / group / chunk
    const int lh = lane >> 4, lr = lane & 15;
    const uint32_t voff_lo = static_cast<uint32_t>((lr & 7) * row_bytes + (lr >> 3) * 64 + lh * 16);
    const uint32_t voff_hi = static_cast<uint32_t>((8 + (lr & 7)) * row_bytes + (1 - (lr >> 3)) * 64 + lh * 16);
    // every byte offset that can cross the last column goes into the per-lane offset, which the
    // range check always covers; the scalar offset stays zero
    auto stage_w = [&](int pair, int buf) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            uint8_t* dst = (buf ? &wbuf1[wave][0] : &wbuf0[wave][0]) + cb * kPairBytes;
            const uint32_t step = static_cast<uint32_t>(pair) * 128u + static_cast<uint32_t>(cb * 16 * row_bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, dst, 16, voff_lo + step, 0, 0, kStreamedOnce);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, dst + 1024, 16, voff_hi + step, 0, 0, kStreamedOnce);
        }
    };
    const int rd0 = pair_slot(c, 0, kq), rd1 = pair_slot(c, 1, kq);

    int col[CB];
    bool col_ok[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        col[cb] = col0 + cb * 16 + c;
        col_ok[cb] = col[cb] < N;
    }

    // small operands of one group pair -- activations (2 groups x 4 x 16 B), scales, biases --
    // through buffer loads: rows >= M and columns >= N read as zeros, and every pair issues the
    // same number of loads (the LDS waits below count them)
    auto clamp_records = [](int64_t bytes) { return static_cast<int>(bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes); };
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), 0, clamp_records(static_cast<int64_t>(M) * K * 2), 0x00020000);
    // scales / biases: resources based at this wave's first column (offsets stay small)
    const int sb_records = clamp_records(col0 < N ? static_cast<int64_t>(N - col0) * G * 2 : 0);
    const size_t sb_base = static_cast<size_t>(col0) * G;
    const __amdgpu_buffer_rsrc_t srsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales + sb_base), 0, sb_records, 0x00020000);
    const __amdgpu_buffer_rsrc_t brsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(biases + sb_base), 0, sb_records, 0x00020000);
    const uint32_t xvoff = arow_ok ? static_cast<uint32_t>(arow * K + kq * 32) * 2u : 0x80000000u;
    uint32_t sboff[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) sboff[cb] = col_ok[cb] ? static_cast<uint32_t>((cb * 16 + c) * G * 2) : 0x80000000u;
    constexpr int kLoadsPerPair = 2 * CB + 8 + 4 * CB;   // direct + activation + scale/bias loads

    struct Small {
        u32x4_t xv[2][4];
        uint16_t s[2][CB], b[2][CB];
    };
    auto load_small = [&](int pair, Small& o) {
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
            const int g = min(2 * pair + g2, G - 1);   // an odd count repeats the last group (unused)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                o.xv[g2][t] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, xvoff, (g * kGroup + t * 8) * 2, 0));
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                // the empty asm statements keep each load a separate instruction (no merging),
                // so the per-pair load count used by the LDS waits is exact
                o.s[g2][cb] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, sboff[cb], g * 2, 0);
                asm volatile("" ::: "memory");
                o.b[g2][cb] = __builtin_amdgcn_raw_buffer_load_b16(brsrc, sboff[cb], g * 2, 0);
                asm volatile("" ::: "memory");
            }
        }
    };

    const bf16x8_t ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                           __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4_t yacc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) yacc[cb] = zero4;

    auto compute = [&](int pair, int buf, const Small& o) {
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
            if (2 * pair + g2 >= G) break;  // odd group count: the last pair has one group
            bf16x8_t a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) a[t] = permute_like_codes(o.xv[g2][t]);
            // X[m] = sum of the group's activations of row m, by the matrix core (B = ones)
            f32x4_t xs = mfma16x16x32(a[0], ones, zero4);
#pragma unroll
            for (int t = 1; t < 4; ++t) xs = mfma16x16x32(a[t], ones, xs);
            const int rd = g2 == 0 ? rd0 : rd1;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const uint8_t* src = (buf ? &wbuf1[wave][0] : &wbuf0[wave][0]) + cb * kPairBytes + rd;
                const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(src);
                f32x4_t p = mfma16x16x32(a[0], codes_bf16_permuted(wv[0]), zero4);
#pragma unroll
                for (int t = 1; t < 4; ++t) p = mfma16x16x32(a[t], codes_bf16_permuted(wv[t]), p);
                const float s = bf16_bits_to_f32(o.s[g2][cb]);
                const float b = bf16_bits_to_f32(o.b[g2][cb]);
#pragma unroll
                for (int r = 0; r < 4; ++r) yacc[cb][r] = __builtin_fmaf(s, p[r], __builtin_fmaf(b, xs[r], yacc[cb][r]));
            }
        }
    };

    // One group pair per step, two steps per iteration with ping-pong buffers (registers and
    // LDS), so no operand is ever copied.  The next pair's loads are always issued (the last
    // step re-reads its own pair into the idle buffer): every step has the same load count and
    // the wait before each compute is exact -- it retires the loads of the pair computed now
    // while the next pair stays in flight.
    if (p0 < p1) {
        Small sa, sb;
        stage_w(p0, 0);
        load_small(p0, sa);
        for (int p = p0;; p += 2) {
            stage_w(p + 1 < p1 ? p + 1 : p, 1);
            load_small(p + 1 < p1 ? p + 1 : p, sb);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerPair) : "memory");
            compute(p, 0, sa);
            if (p + 1 >= p1) break;
            stage_w(p + 2 < p1 ? p + 2 : p + 1, 0);
            load_small(p + 2 < p1 ? p + 2 : p + 1, sa);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerPair) : "memory");
            compute(p + 1, 1, sb);
            if (p + 2 >= p1) break;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no direct load may outlive the wave
    }

    if constexpr (KW > 1) {
        // waves 1..KW-1 of each column set publish their partial sums; wave 0 adds them in order
        __shared__ float red[KW - 1][WN][CB][4][64];
        if (wk > 0) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wk - 1][wn][cb][r][lane] = yacc[cb][r];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int j = 0; j < KW - 1; ++j)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) yacc[cb][r] += red[j][wn][cb][r][lane];
        }
    }

    if (wk == 0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * (lane >> 4) + r;
                if (m < M && col_ok[cb]) y[static_cast<size_t>(m) * N + col[cb]] = f32_to_bf16_bits(yacc[cb][r]);
            }
        }
    }
}

// Wide form (many output columns, e.g. the vocabulary head): a persistent grid of
// workgroups of W waves, as many as fit on the chip at once.
//  * Prologue, once per workgroup: the activations (all M rows, the whole K) go into LDS already
//    permuted into the MFMA A-operand order, and the per-group activation sums X[m, g] are
//    formed once (matrix core, B = ones) and kept in LDS.  The steady state then issues no
//    activation loads and no MFMA for X.
//  * Each wave then works alone: it takes the 16*CB-column blocks w, w + total waves, ... and
//    walks the (block, group pair) steps of all of them in one flat sequence with D LDS stages,
//    keeping D - 1 steps of loads in flight across block boundaries.
//  * One step is 2*CB direct loads of weights (whole 128-byte lines) plus one direct 4-byte load
//    of scales and one of biases (the two groups of a pair are adjacent in memory).
// A block's sums are stored when its last pair is done.  Needs an even group count.
template <int CB, int D, int W>
__global__ __launch_bounds__(64 * W) void qmv_wide_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int N, int K) {
    static_assert(D >= 2 && D <= 6, "stage count");
    static_assert(CB >= 1 && CB <= 4, "one scale load serves at most 64 columns");
    constexpr int kSbOff = CB * kPairBytes;         // scales of the stage, then biases at +256
    constexpr int kStage = kSbOff + 512;
    // one LDS object per stage: the compiler's wait insertion can then tell that a direct load
    // into one stage does not feed reads of another
    __shared__ __attribute__((aligned(16))) uint8_t st0[W][kStage];
    __shared__ __attribute__((aligned(16))) uint8_t st1[W][kStage];
    __shared__ __attribute__((aligned(16))) uint8_t st2[W][D > 2 ? kStage : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st3[W][D > 3 ? kStage : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st4[W][D > 4 ? kStage : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st5[W][D > 5 ? kStage : 16];
    // dynamic LDS: permuted activations (qmv_wide_x_bytes), then X[g][16 rows] as fp32, then
    // 192 M + 16 bytes of zeros
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];

    const int G = K >> 7;
    const int pairs = G >> 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row_bytes = K >> 1;
    const int kq = lane >> 4;
    const int arow = lane & 15;
    const bool arow_ok = arow < M;
    float* const xsum = reinterpret_cast<float*>(xl + qmv_wide_x_bytes(M, K));
    const int zero_off = qmv_wide_x_bytes(M, K) + G * 64;
    auto clamp_records = [](int64_t bytes) { return static_cast<int>(bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes); };
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const u32x4_t zero_u4 = {0u, 0u, 0u, 0u};
    // the A operand of MFMA step t of group g for this lane (row arow, quarter kq); rows >= M
    // are zero and never stored.  Chunk ((4 g + t) * 4 + kq) * M + m holds row m.
    auto read_a = [&](int g, int t) -> u32x4_t {
        const int chunk = ((4 * g + t) * 4 + kq) * M + arow;
        return arow_ok ? *reinterpret_cast<const u32x4_t*>(xl + chunk * 16) : zero_u4;
    };

    const int waves = gridDim.x * W;
    const int gw = blockIdx.x * W + wave;
    const int blocks = (N + CB * 16 - 1) / (CB * 16);
    const int my_blocks = gw < blocks ? (blocks - gw + waves - 1) / waves : 0;
    const int T = my_blocks * pairs;

    const int c = lane & 15;
    const int lh = lane >> 4, lr = lane & 15;
    const uint32_t voff_lo = static_cast<uint32_t>((lr & 7) * row_bytes + (lr >> 3) * 64 + lh * 16);
    const uint32_t voff_hi = static_cast<uint32_t>((8 + (lr & 7)) * row_bytes + (1 - (lr >> 3)) * 64 + lh * 16);
    const uint32_t sb_voff = lane < 16 * CB ? static_cast<uint32_t>(lane * G * 2) : 0x80000000u;
    const int rd0 = pair_slot(c, 0, kq), rd1 = pair_slot(c, 1, kq);
    // steady-state operand reads without branches: lanes of padding rows read the zero area at
    // the same sub-step strides (their group stride is 0)
    const int a_base = arow_ok ? (kq * M + arow) * 16 : zero_off;
    const int a_gstride = arow_ok ? 256 * M : 0;
    const int a_tstride = 64 * M;

    auto stage = [&](auto ic) -> uint8_t* {
        constexpr int i = decltype(ic)::value;
        if constexpr (i == 0) return &st0[wave][0];
        else if constexpr (i == 1) return &st1[wave][0];
        else if constexpr (i == 2) return &st2[wave][0];
        else if constexpr (i == 3) return &st3[wave][0];
        else if constexpr (i == 4) return &st4[wave][0];
        else return &st5[wave][0];
    };

    // issue side: the next step to load is pair ip of block ib.  The block's buffer resources
    // are rebuilt when ib changes; past this wave's last block they have zero records, so the
    // remaining loads fetch nothing but keep the per-step load count the waits rely on.
    int ib = gw, ip = 0;
    __amdgpu_buffer_rsrc_t wrsrc, srsrc, brsrc;
    auto set_block = [&]() {
        const bool live = ib < blocks;
        const int col0 = live ? ib * (CB * 16) : 0;
        const int64_t cols = live ? static_cast<int64_t>(N - col0) : 0;
        wrsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(wq) + static_cast<size_t>(col0) * row_bytes), 0,
            clamp_records(cols * row_bytes), 0x00020000);
        const size_t sb_base = static_cast<size_t>(col0) * G;
        const int sb_records = clamp_records(cols * G * 2);
        srsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales + sb_base), 0, sb_records, 0x00020000);
        brsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(biases + sb_base), 0, sb_records, 0x00020000);
    };
    set_block();
    constexpr int kLoadsPerStep = 2 * CB + 2;
    auto issue = [&](auto ic) {
        uint8_t* dst = stage(ic);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const uint32_t step = static_cast<uint32_t>(ip) * 128u + static_cast<uint32_t>(cb * 16 * row_bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, dst + cb * kPairBytes, 16, voff_lo + step, 0, 0,
                                                     kStreamedOnce);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, dst + cb * kPairBytes + 1024, 16, voff_hi + step, 0, 0,
                                                     kStreamedOnce);
        }
        const uint32_t sbo = sb_voff + static_cast<uint32_t>(ip) * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, dst + kSbOff, 4, sbo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, dst + kSbOff + 256, 4, sbo, 0, 0, 0);
        if (++ip == pairs) {
            ip = 0;
            ib += waves;
            set_block();
        }
    };

    // The first D - 1 steps of weights go out before the activations are staged, so the weight
    // stream's first memory latency overlaps the prologue (whose waits on its own loads also
    // cover these; the loop below skips its fill loads).
    if (T > 0) {
        issue(std::integral_constant<int, 0>{});
        if constexpr (D > 2) issue(std::integral_constant<int, 1>{});
        if constexpr (D > 3) issue(std::integral_constant<int, 2>{});
        if constexpr (D > 4) issue(std::integral_constant<int, 3>{});
        if constexpr (D > 5) issue(std::integral_constant<int, 4>{});
    }

    // ---- prologue 1: activations into LDS in A-operand order, permuted like the codes
    {
        const int chunks = M * (K >> 3);
        const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(x), 0, clamp_records(static_cast<int64_t>(M) * K * 2), 0x00020000);
        for (int i = wave; i * 64 < chunks; i += W) {
            const int d = i * 64 + lane;
            uint32_t voff = 0x80000000u;            // past the end: out of range, reads zeros
            if (d < chunks) {
                const int m = d % M;
                int r = d / M;
                const int q = r & 3;
                r >>= 2;
                const int t = r & 3;
                const int g = r >> 2;
                voff = static_cast<uint32_t>(m * K + g * kGroup + q * 32 + t * 8) * 2u;
            }
            const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, voff, 0, 0));
            *reinterpret_cast<bf16x8_t*>(xl + i * 1024 + lane * 16) = permute_like_codes(v);
        }
        for (int i = threadIdx.x; i * 16 < 192 * M + 16; i += 64 * W)
            *reinterpret_cast<u32x4_t*>(xl + zero_off + i * 16) = zero_u4;
        __syncthreads();
    }
    // ---- prologue 2: X[m, g] = sum of the group's activations of row m, by the matrix core
    {
        const bf16x8_t ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                               __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
        for (int g = wave; g < G; g += W) {
            f32x4_t xs = zero4;
#pragma unroll
            for (int t = 0; t < 4; ++t) xs = mfma16x16x32(__builtin_bit_cast(bf16x8_t, read_a(g, t)), ones, xs);
            // D layout: lane (c, q) holds rows 4q .. 4q + 3, the same for every column c
            if ((lane & 15) == 0) *reinterpret_cast<f32x4_t*>(xsum + g * 16 + 4 * kq) = xs;
        }
        __syncthreads();
    }

    if (T == 0) return;

    f32x4_t yacc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) yacc[cb] = zero4;

    // compute side: step (block cbk, pair cp)
    int done = 0, cbk = gw, cp = 0;
    auto compute = [&](auto ic) {
        const uint8_t* src = stage(ic);
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
            const int g = 2 * cp + g2;
            bf16x8_t a[4];
            const uint8_t* ab = xl + a_base + g * a_gstride;
#pragma unroll
            for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const bf16x8_t*>(ab + t * a_tstride);
            const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(xsum + g * 16 + 4 * kq);
            const int rd = g2 == 0 ? rd0 : rd1;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(src + cb * kPairBytes + rd);
                f32x4_t p = mfma16x16x32(a[0], codes_bf16_permuted(wv[0]), zero4);
#pragma unroll
                for (int t = 1; t < 4; ++t) p = mfma16x16x32(a[t], codes_bf16_permuted(wv[t]), p);
                const int so = kSbOff + 4 * (cb * 16 + c) + 2 * g2;
                const float s = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(src + so));
                const float b = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(src + so + 256));
#pragma unroll
                for (int r = 0; r < 4; ++r) yacc[cb][r] = __builtin_fmaf(s, p[r], __builtin_fmaf(b, xs[r], yacc[cb][r]));
            }
        }
        if (++cp == pairs) {   // block finished: store it, start the next one
            const int col0 = cbk * (CB * 16);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int col = col0 + cb * 16 + c;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * kq + r;
                    if (m < M && col < N) y[static_cast<size_t>(m) * N + col] = f32_to_bf16_bits(yacc[cb][r]);
                }
                yacc[cb] = zero4;
            }
            cp = 0;
            cbk += waves;
        }
        ++done;
    };

    // D-stage pipeline over steps t = -(D - 1), ..., T - 1: position d of the D-fold unrolled
    // body loads step t + D - 1 into stage d, waits until only the newest D - 1 steps of loads
    // are outstanding (so step t has landed) and computes step t from stage (d + 1) % D.  The
    // stage being loaded was computed one position earlier; its LDS reads have all returned
    // (their values fed the MFMAs).  The first D - 1 positions (the fill, loaded before the
    // prologue) do nothing.  Keeping the fill
    // inside the loop (no peeled prologue) lets the compiler see that each stage's reads
    // depend on that stage's loads alone.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    using C0 = std::integral_constant<int, 1 % D>;
    using C1 = std::integral_constant<int, 2 % D>;
    using C2 = std::integral_constant<int, 3 % D>;
    using C3 = std::integral_constant<int, 4 % D>;
    using C4 = std::integral_constant<int, 5 % D>;
    using C5 = std::integral_constant<int, 6 % D>;
    int t = -(D - 1);
    asm volatile("" : "+s"(t));   // opaque start: the fill iterations are not peeled off the loop
#define W4A16_WIDE_STEP(d, I, C)                                                          \
    if constexpr (D > d) {                                                                \
        if (t >= 0) issue(I{});                                                           \
        if (t >= 0) {                                                                     \
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((D - 1) * kLoadsPerStep) : "memory"); \
            compute(C{});                                                                 \
            if (done >= T) break;                                                         \
        }                                                                                 \
        ++t;                                                                              \
    }
    for (;;) {
        W4A16_WIDE_STEP(0, I0, C0)
        W4A16_WIDE_STEP(1, I1, C1)
        W4A16_WIDE_STEP(2, I2, C2)
        W4A16_WIDE_STEP(3, I3, C3)
        W4A16_WIDE_STEP(4, I4, C4)
        W4A16_WIDE_STEP(5, I5, C5)
    }
#undef W4A16_WIDE_STEP
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no direct load may outlive the wave
}

const QmvShape kQmvVariants[kNumQmvVariants] = {
    {1, 1, 4},   // 0: 16 columns per workgroup, 4 waves split K
    {2, 2, 2},   // 1: 64 columns per workgroup, 2 waves split K
    {1, 4, 1},   // 2: wide: persistent, 16-column blocks, 8-wave (M <= 4) or 4-wave workgroups, 2 LDS stages
    {1, 1, 4},   // 3: row-amortized (width-generic kernel at 4 bits), 16 columns, 4 waves split K
    {1, 1, 0},   // 4: burst, 16 columns, 1..16 waves split K (the count depends on the shape)
};

template <int CB, int WN, int KW>
static hipError_t launch_qmv_t(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                               uint16_t* y, int M, int N, int K, hipStream_t stream) {
    const int cols_per_block = CB * WN * 16;
    const dim3 grid((N + cols_per_block - 1) / cols_per_block);
    W4A16_LAUNCH((qmv_kernel<CB, WN, KW>), grid, dim3(64 * WN * KW), 0, stream, x, wq, s, b, y, M, N, K);
    return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
struct WideLaunchCache {
    std::atomic<bool> ready{false};
    std::atomic<int> cus{0};
    std::atomic<uint64_t> occupancy{0};
};
}  // namespace

template <int CB, int D, int W>
static hipError_t launch_qmv_wide_t(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                                    uint16_t* y, int M, int N, int K, hipStream_t stream) {
    static_assert(CB == 1 && D == kQmvWideStages, "qmv_wide_fits describes this instance");
    if (!qmv_wide_fits(M, K) || W != qmv_wide_waves(M)) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    const int blocks = (N + CB * 16 - 1) / (CB * 16);
    const size_t xbytes = qmv_wide_lds_bytes(M, K);
    auto kern = qmv_wide_kernel<CB, D, W>;
    // Per device, once: the compute-unit count, and permission for the largest dynamic LDS the
    // fit check admits.  Per activation size: resident workgroups per compute unit (cached for
    // the last size asked; a race only repeats the query).
    static WideLaunchCache caches[kMaxDevices];   // per instance
    WideLaunchCache& cache = caches[dev];
    if (!cache.ready.load(std::memory_order_acquire)) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(160 * 1024 - qmv_wide_static_lds(M)));
        if (e != hipSuccess) return e;
        cache.cus.store(cus, std::memory_order_relaxed);
        cache.ready.store(true, std::memory_order_release);
    }
    const int cus = cache.cus.load(std::memory_order_relaxed);
    const uint64_t packed = cache.occupancy.load(std::memory_order_relaxed);   // xbytes << 8 | per_cu
    int per_cu = (packed >> 8) == xbytes ? static_cast<int>(packed & 0xFF) : 0;
    if (per_cu == 0) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * W, xbytes);
        if (e != hipSuccess) return e;
        per_cu = std::max(1, std::min(per_cu, 255));
        cache.occupancy.store((static_cast<uint64_t>(xbytes) << 8) | static_cast<uint64_t>(per_cu),
                              std::memory_order_relaxed);
    }
    const int wgs = std::min(per_cu * cus, (blocks + W - 1) / W);
    W4A16_LAUNCH(kern, dim3(wgs), dim3(64 * W), xbytes, stream, x, wq, s, b, y, M, N, K);
    return hipGetLastError();
}

hipError_t launch_qmv(int variant, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* y, int M, int N, int K, hipStream_t stream) {
    switch (variant) {
        case 0: return launch_qmv_t<1, 1, 4>(x, wq, scales, biases, y, M, N, K, stream);
        case 1: return launch_qmv_t<2, 2, 2>(x, wq, scales, biases, y, M, N, K, stream);
        case kQmvWideVariant:
            // the wide kernel loads the scales (biases) of a group pair as one 4-byte word
            if (reinterpret_cast<uintptr_t>(scales) % 4 != 0 || reinterpret_cast<uintptr_t>(biases) % 4 != 0)
                return launch_qmv_t<2, 2, 2>(x, wq, scales, biases, y, M, N, K, stream);
            return qmv_wide_waves(M) == 8
                       ? launch_qmv_wide_t<1, kQmvWideStages, 8>(x, wq, scales, biases, y, M, N, K, stream)
                       : launch_qmv_wide_t<1, kQmvWideStages, 4>(x, wq, scales, biases, y, M, N, K, stream);
        case kQmvAmortizedVariant: return launch_qmv_bits(4, kQmvBitsMatrix, x, wq, scales, biases, y, M, N, K, stream);
        case kQmvBurstVariant: return launch_qmv_burst(x, wq, scales, biases, y, M, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
