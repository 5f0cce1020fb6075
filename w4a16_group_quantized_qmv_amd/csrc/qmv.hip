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
// Memory: the weights stream once from HBM with 16-byte loads; lane group h = l / 16 of a wave
// reads 64 contiguous bytes (one 128-value group) of 16 consecutive columns.  Activations are
// re-read from L2 (they are at most 16 x K bf16).  A workgroup is wn x kw waves: wn waves side
// by side along N, kw waves splitting the groups of the same columns; the kw partial sums are
// added in wave order through LDS, so the result does not depend on timing.
#include "device_common.h"
#include "internal.h"

namespace w4a16 {

template <int CB, int WN, int KW>
__global__ __launch_bounds__(64 * WN * KW) void qmv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int N, int K) {
    const int G = K >> 7;
    const int words_per_row = K >> 3;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave % WN;
    const int wk = wave / WN;
    const int col0 = (blockIdx.x * WN + wn) * (CB * 16);
    const int g0 = static_cast<int>(static_cast<int64_t>(wk) * G / KW);
    const int g1 = static_cast<int>(static_cast<int64_t>(wk + 1) * G / KW);
    const int arow = lane & 15;   // activation row fed by this lane (A operand)
    const int kq = lane >> 4;     // 32-value quarter of each group held by this lane
    const bool arow_ok = arow < M;

    int col[CB];
    bool col_ok[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        col[cb] = col0 + cb * 16 + (lane & 15);
        col_ok[cb] = col[cb] < N;
    }
    const uint16_t* xrow = x + static_cast<size_t>(arow_ok ? arow : 0) * K + kq * 32;

    f32x4_t yacc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) yacc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wcur[CB], wnxt[CB], xcur[4], xnxt[4];
    uint16_t scur[CB], bcur[CB], snxt[CB], bnxt[CB];

    auto load_group = [&](int g, u32x4_t* wv, u32x4_t* xv, uint16_t* sv, uint16_t* bv) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (col_ok[cb]) {
                const size_t row = static_cast<size_t>(col[cb]);
                wv[cb] = load16(wq + row * words_per_row + g * kWordsPerGroup + kq * 4);
                sv[cb] = scales[row * G + g];
                bv[cb] = biases[row * G + g];
            } else {
                wv[cb] = u32x4_t{0u, 0u, 0u, 0u};
                sv[cb] = 0;
                bv[cb] = 0;
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
            xv[t] = arow_ok ? load16(xrow + g * kGroup + t * 8) : u32x4_t{0u, 0u, 0u, 0u};
    };

    const bf16x8_t ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                           __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

    if (g0 < g1) load_group(g0, wcur, xcur, scur, bcur);
    for (int g = g0; g < g1; ++g) {
        if (g + 1 < g1) load_group(g + 1, wnxt, xnxt, snxt, bnxt);

        bf16x8_t a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = permute_like_codes(xcur[t]);
        // X[m] = sum of the group's activations of row m, by the matrix core (B = ones)
        f32x4_t xs = mfma16x16x32(a[0], ones, zero4);
#pragma unroll
        for (int t = 1; t < 4; ++t) xs = mfma16x16x32(a[t], ones, xs);

#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            f32x4_t p = mfma16x16x32(a[0], codes_bf16_permuted(wcur[cb][0]), zero4);
#pragma unroll
            for (int t = 1; t < 4; ++t) p = mfma16x16x32(a[t], codes_bf16_permuted(wcur[cb][t]), p);
            const float s = bf16_bits_to_f32(scur[cb]);
            const float b = bf16_bits_to_f32(bcur[cb]);
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[cb][r] = __builtin_fmaf(s, p[r], __builtin_fmaf(b, xs[r], yacc[cb][r]));
        }

        if (g + 1 < g1) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                wcur[cb] = wnxt[cb];
                scur[cb] = snxt[cb];
                bcur[cb] = bnxt[cb];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) xcur[t] = xnxt[t];
        }
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

const QmvShape kQmvVariants[kNumQmvVariants] = {
    {4, 4, 1},   // 0: wide N, one wave per 64 columns, no K split
    {1, 1, 4},   // 1: 16 columns per workgroup, 4 waves split K
    {1, 1, 8},   // 2: 16 columns per workgroup, 8 waves split K
    {1, 1, 16},  // 3: 16 columns per workgroup, 16 waves split K
    {2, 2, 2},   // 4: 64 columns per workgroup, 2 waves split K
};

template <int CB, int WN, int KW>
static hipError_t launch_qmv_t(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                               uint16_t* y, int M, int N, int K, hipStream_t stream) {
    const int cols_per_block = CB * WN * 16;
    const dim3 grid((N + cols_per_block - 1) / cols_per_block);
    hipLaunchKernelGGL((qmv_kernel<CB, WN, KW>), grid, dim3(64 * WN * KW), 0, stream, x, wq, s, b, y, M, N, K);
    return hipGetLastError();
}

hipError_t launch_qmv(int variant, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* y, int M, int N, int K, hipStream_t stream) {
    switch (variant) {
        case 0: return launch_qmv_t<4, 4, 1>(x, wq, scales, biases, y, M, N, K, stream);
        case 1: return launch_qmv_t<1, 1, 4>(x, wq, scales, biases, y, M, N, K, stream);
        case 2: return launch_qmv_t<1, 1, 8>(x, wq, scales, biases, y, M, N, K, stream);
        case 3: return launch_qmv_t<1, 1, 16>(x, wq, scales, biases, y, M, N, K, stream);
        case 4: return launch_qmv_t<2, 2, 2>(x, wq, scales, biases, y, M, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
