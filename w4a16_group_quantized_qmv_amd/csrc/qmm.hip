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
//  * Workgroup tile BM x BN with NW waves; each wave owns NB 16-column blocks for all BM rows, so
//    each weight is unpacked and dequantized exactly once per workgroup, in registers, by the
//    wave that uses it.  Weights never pass through LDS.
//  * One pipeline step is one 128-value quantization group: the scale and bias of a column are
//    loaded once per step and serve all four 32-value MFMA sub-steps of the group (the analogue
//    of the page's four reduction tiles per group).
//  * Activations (shared by every wave) are staged in LDS, double buffered, with a row stride of
//    136 bf16 (272 bytes): sixteen lanes reading 16 bytes from sixteen consecutive rows then
//    touch all 64 banks once.
//  * Global loads are 16 bytes per lane: a lane group reads 64 contiguous bytes (one group) of
//    16 consecutive weight columns; the activation tile is read row-contiguously.
//  * Tile order is XCD-aware: workgroup i runs on XCD i % 8, and the remap below hands each XCD
//    a contiguous run of tiles in M-fastest order, so the M-tiles that re-read the same weight
//    columns share one L2.
//  * Split-K: blockIdx selects one of S contiguous runs of groups (sizes differ by at most one).
//    Each slice writes fp32 partials; splitk_reduce sums them in slice order (deterministic).
#include "device_common.h"
#include "internal.h"

namespace w4a16 {

constexpr int kLdsStride = kGroup + 8;  // bf16 elements per staged activation row

// Linear workgroup index -> work index such that XCD c (= i % 8) receives the contiguous range
// of work indices [start_c, start_c + count_c).
__device__ __forceinline__ int xcd_remap(int i, int total) {
    const int per = total >> 3, rem = total & 7;
    const int c = i & 7, k = i >> 3;
    return c * per + (c < rem ? c : rem) + k;
}

template <int BM, int NB, int NW>
__global__ __launch_bounds__(64 * NW) void qmm_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N, int K,
    int split, int tiles_m, int tiles_n) {
    constexpr int BN = NW * NB * 16;
    constexpr int THREADS = 64 * NW;
    constexpr int RB = BM / 16;                   // 16-row blocks per wave
    constexpr int XCHUNKS = BM * 16 / THREADS;    // 16-byte activation chunks per thread per group
    static_assert(BM * 16 % THREADS == 0, "activation tile must divide evenly among threads");
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kLdsStride];

    const int tiles = tiles_m * tiles_n;
    const int work = xcd_remap(blockIdx.x, tiles * split);
    const int z = work / tiles;
    const int tile = work - z * tiles;
    const int tm = tile % tiles_m;
    const int tn = tile / tiles_m;

    const int G = K >> 7;
    const int words_per_row = K >> 3;
    const int g_begin = static_cast<int>(static_cast<int64_t>(z) * G / split);
    const int g_end = static_cast<int>(static_cast<int64_t>(z + 1) * G / split);
    const int m0 = tm * BM;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kq = lane >> 4;

    int col[NB];
    bool col_ok[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        col[cb] = tn * BN + (wave * NB + cb) * 16 + (lane & 15);
        col_ok[cb] = col[cb] < N;
    }

    // activation staging: chunk c = tid + i * THREADS covers row c / 16, 16-byte chunk c % 16
    auto load_x = [&](int g, u32x4_t* xr) {
#pragma unroll
        for (int i = 0; i < XCHUNKS; ++i) {
            const int c = threadIdx.x + i * THREADS;
            const int r = c >> 4, kc = c & 15;
            xr[i] = (m0 + r < M) ? load16(x + static_cast<size_t>(m0 + r) * K + g * kGroup + kc * 8)
                                 : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    auto store_x = [&](int buf, const u32x4_t* xr) {
#pragma unroll
        for (int i = 0; i < XCHUNKS; ++i) {
            const int c = threadIdx.x + i * THREADS;
            const int r = c >> 4, kc = c & 15;
            *reinterpret_cast<u32x4_t*>(&xs[buf][r * kLdsStride + kc * 8]) = xr[i];
        }
    };
    auto load_w = [&](int g, u32x4_t* wv, uint16_t* sv, uint16_t* bv) {
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
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
    };

    f32x4_t acc[RB][NB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t xr[XCHUNKS];
    u32x4_t wcur[NB], wnxt[NB];
    uint16_t scur[NB], bcur[NB], snxt[NB], bnxt[NB];

    if (g_begin < g_end) {
        load_x(g_begin, xr);
        load_w(g_begin, wcur, scur, bcur);
        store_x(0, xr);
    }
    __syncthreads();

    for (int g = g_begin; g < g_end; ++g) {
        const int buf = (g - g_begin) & 1;
        const bool more = g + 1 < g_end;
        if (more) {
            load_x(g + 1, xr);
            load_w(g + 1, wnxt, snxt, bnxt);
        }
        float s[NB], b[NB];
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            s[cb] = bf16_bits_to_f32(scur[cb]);
            b[cb] = bf16_bits_to_f32(bcur[cb]);
        }
        const uint16_t* xt = &xs[buf][(lane & 15) * kLdsStride + kq * 32];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8_t bw[NB];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) bw[cb] = dequant_word(wcur[cb][t], s[cb], b[cb]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xt + rb * 16 * kLdsStride + t * 8);
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) acc[rb][cb] = mfma16x16x32(a, bw[cb], acc[rb][cb]);
            }
        }
        if (more) {
            store_x(buf ^ 1, xr);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                wcur[cb] = wnxt[cb];
                scur[cb] = snxt[cb];
                bcur[cb] = bnxt[cb];
            }
        }
        __syncthreads();
    }

    // epilogue: D layout puts rows 4 * (lane / 16) + r of column lane % 16 in this lane
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + rb * 16 + 4 * (lane >> 4) + r;
            if (m >= M) continue;
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                if (!col_ok[cb]) continue;
                const size_t idx = static_cast<size_t>(m) * N + col[cb];
                if (split == 1)
                    y[idx] = f32_to_bf16_bits(acc[rb][cb][r]);
                else
                    ws[static_cast<size_t>(z) * M * N + idx] = acc[rb][cb][r];
            }
        }
    }
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
    {128, 4, 4},  // 0: 128 x 256 tile, 4 waves of 128 x 64
    {128, 2, 4},  // 1: 128 x 128 tile, 4 waves of 128 x 32
    {64, 2, 4},   // 2:  64 x 128 tile, 4 waves of  64 x 32
};

template <int BM, int NB, int NW>
static hipError_t launch_qmm_t(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                               uint16_t* y, float* ws, int M, int N, int K, int split, hipStream_t stream) {
    constexpr int BN = NW * NB * 16;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const dim3 grid(tiles_m * tiles_n * split);
    hipLaunchKernelGGL((qmm_kernel<BM, NB, NW>), grid, dim3(64 * NW), 0, stream, x, wq, s, b, y, ws, M, N, K, split,
                       tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_qmm(int variant, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* y, float* ws, int M, int N, int K, int split,
                      hipStream_t stream) {
    switch (variant) {
        case 0: return launch_qmm_t<128, 4, 4>(x, wq, scales, biases, y, ws, M, N, K, split, stream);
        case 1: return launch_qmm_t<128, 2, 4>(x, wq, scales, biases, y, ws, M, N, K, split, stream);
        case 2: return launch_qmm_t<64, 2, 4>(x, wq, scales, biases, y, ws, M, N, K, split, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_splitk_reduce(const float* ws, uint16_t* y, int64_t MN, int split, hipStream_t stream) {
    const int64_t blocks = (MN + 255) / 256;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ws, y, MN,
                       split);
    return hipGetLastError();
}

}  // namespace w4a16
