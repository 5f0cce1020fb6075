// Host-side launchers shared between the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// qmv: one workgroup covers wn * cb * 16 output columns; kw of its waves split the K groups
// of those columns and are summed in wave order through LDS.
struct QmvShape {
    int cb;   // 16-column blocks per wave
    int wn;   // waves side by side along N
    int kw;   // waves along K
};

// Kernel instances compiled for qmv (index = plan variant).
constexpr int kNumQmvVariants = 5;
extern const QmvShape kQmvVariants[kNumQmvVariants];

hipError_t launch_qmv(int variant, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* y, int M, int N, int K, hipStream_t stream);

// qmm: workgroup tile of bm rows x (nwaves * nb * 32) columns; every wave owns nb 32-column
// blocks for all bm rows.
struct QmmShape {
    int bm;
    int nb;
    int nwaves;
};

constexpr int kNumQmmVariants = 5;
extern const QmmShape kQmmVariants[kNumQmmVariants];

// split == 1 writes bf16 y; split > 1 writes fp32 partials ws[z][M][N] for z < split.
hipError_t launch_qmm(int variant, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* y, float* ws, int M, int N, int K, int split,
                      hipStream_t stream);

// y[i] = bf16(sum_{z < split} ws[z][i]) summed in slice order.
hipError_t launch_splitk_reduce(const float* ws, uint16_t* y, int64_t MN, int split, hipStream_t stream);

}  // namespace w4a16
