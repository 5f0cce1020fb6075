// Host-side launchers shared between the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// Kernel-timestamp request (w4a16_time_next_launch), one per host thread: while armed, the next
// contraction kernel this thread launches (a tile or matvec kernel; not a group-sum pre-pass or
// a split-K slice sum) is launched through hipExtLaunchKernel with these events, which then hold
// the kernel's execution start and end, and the request is cleared.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming& launch_timing();

// hipExtLaunchKernel packs the arguments by the types it is given, so each one is first
// converted to the kernel's own parameter type.
// A request met by a launch into a stream under graph capture is consumed without timing: the
// kernel is captured as a plain launch.
template <typename... P, typename... A>
inline void launch_timed(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t lds, hipStream_t stream,
                         A... args) {
    const LaunchTiming t = launch_timing();
    launch_timing() = LaunchTiming{};
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone) {
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, static_cast<P>(args)...);
        return;
    }
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, t.start, t.stop, 0u, static_cast<P>(args)...);
}

// Every contraction kernel launch goes through this: a plain launch unless a timing request is
// armed on the calling thread.
#define W4A16_LAUNCH(kernel, grid, block, lds, stream, ...)                                            \
    do {                                                                                               \
        const ::w4a16::LaunchTiming& w4a16_lt_ = ::w4a16::launch_timing();                             \
        if (w4a16_lt_.start != nullptr || w4a16_lt_.stop != nullptr)                                   \
            ::w4a16::launch_timed(kernel, dim3(grid), dim3(block), static_cast<uint32_t>(lds), stream, \
                                  __VA_ARGS__);                                                        \
        else                                                                                           \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                          \
    } while (0)

// Cache policy of the weight loads of the persistent wide matvec, the 16-column K-split matvec
// and the packed burst forms: non-temporal (the codes of a decode matvec are read once per
// call; measured on MI355X: the 151936-column head 41.5 against 44.3 us alone and 40.6 against
// 49.3 us inside the 512-row step, the 13 MB packed-burst shapes 3% faster; the K-split
// matvec within 1%).  The 16-column burst forms measured 1-5% slower with it and the tile
// kernels, whose M-tiles re-read the same codes from L2, keep the default policy.
constexpr int kStreamedOnce = 2;

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

// The wide (persistent) qmv instances: 16-column blocks, 2 LDS stages, workgroups of
// qmv_wide_waves(M) waves.
constexpr int kQmvWideVariant = 2;
// The row-amortized kernel of the width-generic matvec at 4 bits (16 columns, 4 waves split K):
// exact integer codes on the matrix core and y += s * P + b * X per group.
constexpr int kQmvAmortizedVariant = 3;
// The burst kernel (4-bit, at most 8 rows): a workgroup of up to kQmvBurstMaxWaves waves on one
// 16-column block (or 4 in the packed form), each wave owning at most kQmvBurstMaxGroups groups
// (or steps of 4) and issuing all their loads before it computes; the wave count depends on the
// shape (qmv_burst_shape).
constexpr int kQmvBurstVariant = 4;
constexpr int kQmvBurstMaxWaves = 16;
constexpr int kQmvBurstMaxGroups = 5;
// The burst kernel's form for an M x N x K matvec: packed (4 K slices in the MFMA's spare rows,
// 4 columns per workgroup, gpw steps of 4 groups per wave, rows = activation row slots) or not
// (16 columns per workgroup, gpw groups per wave, 4 or 8 row slots); kw waves per workgroup.
// False where it does not apply: more than 8 rows, 2048 column blocks or more, or 1664 blocks
// or more under 32 groups where the wide kernel applies; at 1 and 2 rows more than 128 groups;
// at 3 and 4 rows more than 80 groups, or 1024 blocks or more at 32 groups or more; at 5 to 8
// rows 1024 blocks or more, or more than 64 groups.
struct QmvBurstShape {
    int packed, kw, gpw, rows, cols;
};
bool qmv_burst_shape(int M, int N, int K, QmvBurstShape* out);
hipError_t launch_qmv_burst(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            uint16_t* y, int M, int N, int K, hipStream_t stream);
constexpr int kQmvWideStages = 2;
// Its LDS: per wave and stage one 2 KB block of codes plus 512 bytes of scales and biases
// (with 1 KB allowed for the kernel's small placeholder objects); dynamically the permuted
// activations (whole 1 KB units of 64 chunks of 16 bytes), the per-group activation sums
// (16 fp32 per group) and a zero area that the operand reads of padding rows (M..15) address
// (four sub-step strides of 64 M bytes).
// Eight waves per workgroup up to 4 rows (half the activation copies per compute unit: on the
// 151936-column vocabulary head at M = 1 measured 41-42 us against 44-47 us with four), four
// beyond, where the activation tile grows.
inline int qmv_wide_waves(int M) { return M <= 4 ? 8 : 4; }
inline size_t qmv_wide_static_lds(int M) {
    return static_cast<size_t>(qmv_wide_waves(M)) * (2048 + 512) * kQmvWideStages + 1024;
}
inline size_t qmv_wide_x_bytes_host(int M, int K) {
    const size_t chunks = static_cast<size_t>(M) * (K / 8);
    return (chunks + 63) / 64 * 1024;
}
inline size_t qmv_wide_zero_bytes(int M) { return static_cast<size_t>(192 * M + 16); }
inline size_t qmv_wide_lds_bytes(int M, int K) {
    return qmv_wide_x_bytes_host(M, K) + static_cast<size_t>(K / 128) * 64 + qmv_wide_zero_bytes(M);
}
// The wide kernel needs an even group count, at most 16 rows and its LDS within a workgroup's
// 160 KB.
inline bool qmv_wide_fits(int M, int K) {
    return (K / 128) % 2 == 0 && M >= 1 && M <= 16 && qmv_wide_static_lds(M) + qmv_wide_lds_bytes(M, K) <= 160 * 1024;
}

hipError_t launch_qmv(int variant, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* y, int M, int N, int K, hipStream_t stream);

// qmm: workgroup tile of bm rows x (nwaves * nb * 32) columns; every wave owns nb 32-column
// blocks for all bm rows.
struct QmmShape {
    int bm;
    int nb;
    int nwaves;
    int stages;       // groups in flight: LDS activation tiles and weight register sets
    int ksplit = 1;   // waves per 32-column strip, splitting each group's MFMA sub-steps
    int tile_n() const { return nwaves / ksplit * nb * 32; }
};

constexpr int kNumQmmVariants = 7;
// 64 x 128 tiles with two waves per column strip: for grids of at most one work unit per
// compute unit (twice the waves per tile)
constexpr int kQmmKSplitVariant = 5;
// 96 x 128 tiles with two waves per column strip: when they need fewer rounds of tiles per
// compute unit than the 64-row tiles, at most two
constexpr int kQmmRows96Variant = 6;
constexpr int kQmmSkinnyVariant = 4;   // 32 x 128 tiles, three stages: at most 32 rows
extern const QmmShape kQmmVariants[kNumQmmVariants];

// Columns of a per-row group-sum buffer: two bf16 halves per 128-value group, rounded up to the
// 16-value MFMA step.
inline int group_sum_cols(int K) { return ((2 * (K / 128) + 15) / 16) * 16; }
// Exact-code mode of the tile kernels needs the activations' group sums: xsum [M, KB] bf16,
// columns 2g / 2g + 1 = hi / lo of the fp32 sum of group g, zeros beyond 2G.
hipError_t launch_act_group_sums(const uint16_t* x, uint16_t* xsum, int M, int K, int KB, hipStream_t stream);
// Plans report the exact-code mode as the tile variant plus this offset.  It is compiled for the
// 128-row tiles (variant kQmmCodesTileVariant), where it measured faster than dequantizing.
constexpr int kQmmCodesVariantOffset = 10;
constexpr int kQmmCodesTileVariant = 0;

// split == 1 writes bf16 y; split > 1 writes fp32 partials ws[z][M][N] for z < split.  xsum != nullptr
// selects the exact-code mode (codes on the matrix core, y = sum_g s P + sum_g b X), else weights are
// dequantized to bf16 in registers.
hipError_t launch_qmm(int variant, const uint16_t* x, const uint16_t* xsum, const uint32_t* wq, const uint16_t* scales,
                      const uint16_t* biases, uint16_t* y, float* ws, int M, int N, int K, int split,
                      hipStream_t stream);

// Grouped projections of one input (at most kMaxGroupedProjections): y_p = x . dequant(wq_p)^T,
// one launch over the concatenation of the projections' column tiles.  Projection p owns the
// column tiles [tn_first[p], tn_first[p + 1]) of 128 columns each (its last tile may be ragged).
constexpr int kMaxGroupedProjections = 4;
constexpr int kGroupedTileN = 128;   // columns per tile of every qmm tile form
struct QmmGroups {
    const uint32_t* wq[kMaxGroupedProjections];
    const uint16_t* s[kMaxGroupedProjections];
    const uint16_t* b[kMaxGroupedProjections];
    uint16_t* y[kMaxGroupedProjections];
    int n[kMaxGroupedProjections];
    int tn_first[kMaxGroupedProjections];
    int count;
};
// Columns of the concatenated tile grid (a multiple of 128).
int grouped_columns(const QmmGroups& groups);
// split > 1 writes fp32 partials ws[z][M][grouped_columns] (every projection's columns at its
// tiles' place), summed into the outputs by launch_splitk_reduce_grouped.
hipError_t launch_qmm_grouped(int variant, const uint16_t* x, const uint16_t* xsum, const QmmGroups& groups,
                              float* ws, int M, int K, int split, hipStream_t stream);
hipError_t launch_splitk_reduce_grouped(const float* ws, const QmmGroups& groups, int M, int split,
                                        hipStream_t stream);

// Gate / up pair with SwiGLU: h = bf16(silu(x . gate^T) * (x . up^T)), one tile kernel for both
// projections.  split > 1 writes fp32 partials ws[0][z][M][N] (gate) and ws[1][z][M][N] (up).
// xsum != nullptr selects the exact-code mode, compiled for the 64-row tiles
// (kGateUpCodesTileVariant), where it measured faster than dequantizing at 512 and 4096 rows.
constexpr int kNumGateUpVariants = 4;
constexpr int kGateUpCodesTileVariant = 1;
// 96 x 128 tiles (dequantizing, two resident per compute unit): when they need fewer rounds of
// tiles per compute unit than the 64-row tiles, at most two
constexpr int kGateUpRows96Variant = 3;
extern const QmmShape kGateUpVariants[kNumGateUpVariants];
hipError_t launch_gate_up(int variant, const uint16_t* x, const uint16_t* xsum, const uint32_t* wq_gate,
                          const uint16_t* s_gate, const uint16_t* b_gate, const uint32_t* wq_up, const uint16_t* s_up,
                          const uint16_t* b_up, uint16_t* h, float* ws, int M, int N, int K, int split,
                          hipStream_t stream);
// h[i] = bf16(silu(sum_z ws[0][z][i]) * sum_z ws[1][z][i]), slices summed in order.
hipError_t launch_splitk_reduce_glu(const float* ws, uint16_t* h, int64_t MN, int split, hipStream_t stream);

// Width-generic affine matvec (1, 2, 3, 4 or 8 bits per code, M <= 8): row-amortized on the
// matrix core (mode kQmvBitsMatrix) or per row with dot products (kQmvBitsRows, M <= 2).
constexpr int kQmvBitsMatrix = 0, kQmvBitsRows = 1;
// The burst forms of the width-generic matvec (at most 8 rows; the packed layout up to 4 rows,
// the 16-column one from 3 rows): its shape, false where neither applies (the 4-bit burst
// domains: 2048 column blocks or more, more than 128 groups; beyond the packed domain 1024
// blocks or more, more than 80 groups at 3 and 4 rows or 64 at 5 to 8); and its launch.
bool qmv_bits_burst_shape(int M, int N, int K, QmvBurstShape* out);
hipError_t launch_qmv_bits_burst(int bits, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                                 const uint16_t* biases, uint16_t* y, int M, int N, int K, hipStream_t stream);
hipError_t launch_qmv_bits(int bits, int mode, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                           const uint16_t* biases, uint16_t* y, int M, int N, int K, hipStream_t stream);

// W4A8: per-row int8 activations (codes stored in the int8 kernel's operand order, one fp32
// scale per row, exact per-group code sums as bf16 hi / lo pairs in xsum [M, KB]) and the int8
// tile kernel.  split > 1 writes fp32 partials ws[z][M][N], summed by launch_splitk_reduce.
inline int w4a8_xsum_cols(int K) { return group_sum_cols(K); }
hipError_t launch_quantize_rows_int8(const uint16_t* x, int8_t* xq, float* sx, uint16_t* xsum, int M, int K, int KB,
                                     hipStream_t stream);
constexpr int kNumW4A8Variants = 4;
constexpr int kW4A8KSplitVariant = 3;   // 64 x 128 tiles, two waves per column block
extern const QmmShape kW4A8Variants[kNumW4A8Variants];
hipError_t launch_qmm_w4a8(int variant, const int8_t* xq, const float* sx, const uint16_t* xsum, const uint32_t* wq,
                           const uint16_t* scales, const uint16_t* biases, uint16_t* y, float* ws, int M, int N,
                           int K, int KB, int split, hipStream_t stream);

// y[i] = bf16(sum_{z < split} ws[z][i]) summed in slice order.
hipError_t launch_splitk_reduce(const float* ws, uint16_t* y, int64_t MN, int split, hipStream_t stream);

}  // namespace w4a16
