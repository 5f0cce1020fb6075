// qmv_burst: the 4-bit affine matvec for up to eight decode rows, one HBM round trip per wave.
//
// The operation is the one of the W4 layout ("Week 2 Day 6" and the qmv_wide pages): a
// column's 4-bit codes packed eight per uint32, low nibble first; one bf16 scale and bias per
// 128 reduction values, w = s * q + b; y[m, n] = sum_k x[m, k] * w[n, k] in fp32.
//
// Why a separate kernel: at decode widths a matvec over a few MB of codes is latency bound,
// not bandwidth bound.  The loop kernels keep one group in flight per wave, so a wave waits
// for HBM once per group pair.  Here a workgroup is KW waves on one 16-column block, wave w
// owns at most GPW consecutive groups, and it issues every load of its share -- codes,
// scales, biases and its slice of the activations -- before the first matrix-core
// instruction, then waits once.  Many short waves (KW up to 16 per block, GPW 2..5 groups
// each) put the whole matrix in flight within about one memory latency.  KW is a kernel
// argument: read from the workgroup size, it costs a dependent load from the dispatch packet
// before the first address (measured 0.2-0.3 us per launch).
//
// Per group (lane l: column c = l % 16, reduction values kq*32 .. kq*32 + 31, kq = l / 16 --
// the B operand of v_mfma_f32_16x16x32_bf16), the codes become exact bf16 integers in the
// permuted order of codes_bf16_permuted(); the activations (rows 0..M-1 of the A operand,
// zero beyond; 4 row slots per chunk up to 4 rows, 8 up to 8) are put in the same order once,
// into the wave's own LDS slice, and read back as A operands.  P = sum x*q and X = sum x come from the matrix core and y += s*P + b*X, the
// row-amortized form of the affine dequantization.  The waves' partial sums are added in wave
// order through LDS, so a result does not depend on timing.  Every load goes through a buffer
// resource: columns past N and rows past M read zeros.
//
// Packed form (qmv_burst_packed_kernel): with at most 4 rows, 12 of the A operand's 16 rows are
// padding.  The packed form fills them with 4 K slices: A rows 4s + m hold row m of the
// activations of slice s, and B columns 4s + j hold column j's codes of slice s, so one MFMA
// works on 4 columns x 4 groups instead of 16 columns x 1 group (the same 1 KB of codes).  Of
// its 16 x 16 result only the 4 diagonal 4 x 4 blocks (slice s of A against slice s of B) are
// wanted; the others are computed and dropped, which costs nothing on a path that waits on
// memory.  A workgroup then covers 4 columns, so a narrow matrix (1024 or 2560 columns) spreads
// over 4x as many workgroups and fills the compute units the 16-column form leaves idle.
#include "device_common.h"
#include "internal.h"

#include <atomic>

namespace w4a16 {

namespace {

constexpr int kBurstRows = 4;        // rows the packed form serves (4 K slices of 4 rows fill the A operand)
constexpr int kBurstMaxRows = 8;     // rows the 16-column form serves (8 row slots from 5 rows)

// LDS of a KW-wave workgroup of the 16-column form: each wave's activation slice (GPW groups x
// 16 chunks of 16 bytes x MR row slots), then the partial sums of waves 1..KW-1 (4 fp32 per
// lane, one 16-byte slot).
constexpr size_t burst_lds_bytes(int kw, int gpw, int mr) {
    return static_cast<size_t>(kw) * gpw * 16 * mr * 16 + static_cast<size_t>(kw - 1) * 4 * 64 * 4;
}

}  // namespace

template <int GPW, int MR>
__global__ __launch_bounds__(64 * kQmvBurstMaxWaves) void qmv_burst_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int N, int K, int KW) {
    extern __shared__ __attribute__((aligned(16))) u32x4_t lds[];
    const int G = K >> 7;
    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col0 = blockIdx.x * 16;
    // wave w owns groups w*GPW .. w*GPW + GPW - 1 (the last wave fewer: KW = ceil(G / GPW))
    const int g0 = wk * GPW;
    const int ng = min(GPW, G - g0);
    const int c = lane & 15, kq = lane >> 4;
    const int row_bytes = K / 2;
    auto clamp_records = [](int64_t bytes) { return static_cast<int>(bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes); };
    const int64_t cols = static_cast<int64_t>(N - col0);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(wq) + static_cast<size_t>(col0) * row_bytes), 0,
        clamp_records(cols * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(scales + static_cast<size_t>(col0) * G), 0, clamp_records(cols * G * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(biases + static_cast<size_t>(col0) * G), 0, clamp_records(cols * G * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), 0, clamp_records(static_cast<int64_t>(M) * K * 2), 0x00020000);
    // a zero-sized resource: loads of groups the wave does not own return zeros
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, 0, 0x00020000);
    const uint32_t wvoff = static_cast<uint32_t>(c * row_bytes + kq * 16);
    const uint32_t sbvoff = static_cast<uint32_t>(c * G * 2);
    static_assert(MR == 4 || MR == 8, "row slots: a power of two that divides the 64 lanes");
    u32x4_t* const xs = lds + static_cast<size_t>(wk) * GPW * 16 * MR;
    f32x4_t* const red = reinterpret_cast<f32x4_t*>(lds + static_cast<size_t>(KW) * GPW * 16 * MR);

    // 1. every load of the wave: codes (16 bytes per lane and group), scales, biases, then the
    //    activation slice: chunk j = ((gl * 4 + t) * 4 + q) * MR + m holds row m's 8 values
    //    gl*128 + q*32 + t*8 .. +7 of the wave's group gl (q: the lanes' kq, t: the operand), MR
    //    row slots per chunk (4 or 8).
    //    Groups past the wave's share read through the zero-sized resource; every offset is
    //    wave-uniform arithmetic, so no load needs a per-lane resource or offset loop.
    uint32_t w[GPW][4];
    uint16_t sv[GPW], bv[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const u32x4_t v = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(i < ng ? wr : none, wvoff, (g0 + i) * 64, 0));
        w[i][0] = v[0];
        w[i][1] = v[1];
        w[i][2] = v[2];
        w[i][3] = v[3];
    }
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        sv[i] = __builtin_amdgcn_raw_buffer_load_b16(i < ng ? sr : none, sbvoff, (g0 + i) * 2, 0);
        bv[i] = __builtin_amdgcn_raw_buffer_load_b16(i < ng ? br : none, sbvoff, (g0 + i) * 2, 0);
    }
    constexpr int XL = GPW * 16 * MR / 64;
    u32x4_t xv[XL];
#pragma unroll
    for (int j0 = 0; j0 < XL; ++j0) {
        const int j = j0 * 64 + lane;
        const int m = j % MR, r = j / MR;
        const int q = r & 3, t = (r >> 2) & 3, gl = r >> 4;
        const uint32_t voff = m < M && gl < ng
                                  ? static_cast<uint32_t>(m * K + (g0 + gl) * kGroup + q * 32 + t * 8) * 2u
                                  : 0x80000000u;   // past the end: reads zero
        xv[j0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, voff, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);   // all loads issued before anything waits on one
#pragma unroll
    for (int j0 = 0; j0 < XL; ++j0) xs[j0 * 64 + lane] = __builtin_bit_cast(u32x4_t, permute_like_codes(xv[j0]));
    // the slice is the wave's own: LDS accesses of one wave complete in order, so only the
    // compiler must keep the reads below after these writes
    asm volatile("" ::: "memory");

    // 2. every group: rows 4*kq + r of column c.  A group past the wave's share has zero codes,
    //    scale, bias and activations and adds exactly +0; computing it anyway keeps its loads
    //    unconditional, so the compiler cannot sink them below the wait
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const u32x4_t zu = {0u, 0u, 0u, 0u};
    const bf16x8_t ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                           __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
    const int arow = lane & 15;
    f32x4_t yacc = zero4;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        f32x4_t xsum = zero4, p = zero4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const u32x4_t av = arow < M ? xs[((i * 4 + t) * 4 + kq) * MR + arow] : zu;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
            xsum = mfma16x16x32(a, ones, xsum);
            p = mfma16x16x32(a, codes_bf16_permuted(w[i][t]), p);
        }
        const float s = bf16_bits_to_f32(sv[i]), b = bf16_bits_to_f32(bv[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[r] = __builtin_fmaf(s, p[r], __builtin_fmaf(b, xsum[r], yacc[r]));
    }

    // 3. waves 1..KW-1 hand their sums to wave 0 (one 16-byte slot per lane), which adds them
    //    in wave order, reading four waves' slots before it adds them: a read per wave and add
    //    would wait out the LDS latency up to 15 times
    if (KW > 1) {
        if (wk > 0) red[(wk - 1) * 64 + lane] = yacc;
        __syncthreads();
        if (wk == 0) {
            int j = 0;
            for (; j + 4 <= KW - 1; j += 4) {
                f32x4_t v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = red[(j + u) * 64 + lane];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int r = 0; r < 4; ++r) yacc[r] += v[u][r];
            }
            for (; j < KW - 1; ++j) {
                const f32x4_t v = red[j * 64 + lane];
#pragma unroll
                for (int r = 0; r < 4; ++r) yacc[r] += v[r];
            }
        }
    }
    if (wk == 0) {
        const int col = col0 + c;
        if (col < N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * kq + r;
                if (m < M) y[static_cast<size_t>(m) * N + col] = f32_to_bf16_bits(yacc[r]);
            }
        }
    }
}

template <int GPW, int MR>
__global__ __launch_bounds__(64 * kQmvBurstMaxWaves) void qmv_burst_packed_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int N, int K, int KW) {
    extern __shared__ __attribute__((aligned(16))) u32x4_t lds[];
    constexpr int GW = 4 * GPW;   // groups per wave: GPW steps of 4 slices
    const int G = K >> 7;
    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col0 = blockIdx.x * 4;
    const int g0 = wk * GW;       // step i, slice s: group g0 + 4 i + s
    const int c = lane & 15, kq = lane >> 4;
    const int sl = c >> 2, j = c & 3;   // this lane's slice and column (B operand), or slice and row (A)
    const int row_bytes = K / 2;
    auto clamp_records = [](int64_t bytes) { return static_cast<int>(bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes); };
    const int64_t cols = static_cast<int64_t>(N - col0);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(wq) + static_cast<size_t>(col0) * row_bytes), 0,
        clamp_records(cols * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(scales + static_cast<size_t>(col0) * G), 0, clamp_records(cols * G * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(biases + static_cast<size_t>(col0) * G), 0, clamp_records(cols * G * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), 0, clamp_records(static_cast<int64_t>(M) * K * 2), 0x00020000);
    u32x4_t* const xs = lds + static_cast<size_t>(wk) * GW * 16 * MR;
    float* const red = reinterpret_cast<float*>(lds + static_cast<size_t>(KW) * GW * 16 * MR);

    // 1. every load of the wave.  Codes and scales: lane (s, j, kq) takes column j's 16 bytes at
    //    kq*16 of group g0 + 4 i + s (the four slices of a step are 256 contiguous bytes of the
    //    column).  Activations: chunk jj = ((gl * 4 + t) * 4 + q) * MR + m holds row m's values
    //    gl*128 + q*32 + t*8 .. +7 of the wave's group gl, MR row slots per chunk (1, 2 or 4).
    //    Past the last group, column or row the per-lane offset passes the resource's end and
    //    the load returns zeros.
    uint32_t w[GPW][4];
    uint16_t sv[GPW], bv[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int g = g0 + 4 * i + sl;
        const uint32_t voff = g < G ? static_cast<uint32_t>(j * row_bytes + g * 64 + kq * 16) : 0x80000000u;
        const u32x4_t v =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, 0, kStreamedOnce));
        w[i][0] = v[0];
        w[i][1] = v[1];
        w[i][2] = v[2];
        w[i][3] = v[3];
    }
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int g = g0 + 4 * i + sl;
        const uint32_t voff = g < G ? static_cast<uint32_t>((j * G + g) * 2) : 0x80000000u;
        sv[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, voff, 0, 0);
        bv[i] = __builtin_amdgcn_raw_buffer_load_b16(br, voff, 0, 0);
    }
    constexpr int XL = GW * 16 * MR / 64;
    u32x4_t xv[XL];
#pragma unroll
    for (int j0 = 0; j0 < XL; ++j0) {
        const int jj = j0 * 64 + lane;
        const int m = jj % MR, rr = jj / MR;
        const int q = rr & 3, t = (rr >> 2) & 3, gl = rr >> 4;
        const uint32_t voff = m < M && g0 + gl < G
                                  ? static_cast<uint32_t>(m * K + (g0 + gl) * kGroup + q * 32 + t * 8) * 2u
                                  : 0x80000000u;
        xv[j0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, voff, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);   // all loads issued before anything waits on one
#pragma unroll
    for (int j0 = 0; j0 < XL; ++j0) xs[j0 * 64 + lane] = __builtin_bit_cast(u32x4_t, permute_like_codes(xv[j0]));
    asm volatile("" ::: "memory");   // the wave's own slice: only the compiler must keep the order

    // 2. every step: A lane (row 4 s + m, kq) reads slice s's row m; the result lane (c, kq) holds
    //    rows 4 kq .. 4 kq + 3 of column c, wanted where kq is column c's slice
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const u32x4_t zu = {0u, 0u, 0u, 0u};
    const bf16x8_t ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                           __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
    const int am = j < MR ? j : 0;
    f32x4_t yacc = zero4;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        f32x4_t xsum = zero4, p = zero4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const u32x4_t av = j < M && j < MR ? xs[(((4 * i + sl) * 4 + t) * 4 + kq) * MR + am] : zu;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
            xsum = mfma16x16x32(a, ones, xsum);
            p = mfma16x16x32(a, codes_bf16_permuted(w[i][t]), p);
        }
        const float s = bf16_bits_to_f32(sv[i]), b = bf16_bits_to_f32(bv[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[r] = __builtin_fmaf(s, p[r], __builtin_fmaf(b, xsum[r], yacc[r]));
    }

    // 3. the wanted lanes (kq == slice) hand rows 0..3 of their column to LDS; wave 0, lane
    //    16 s + 4 j + m, adds its (slice, column, row) over the waves in wave order, then the
    //    four slices of each output in a fixed pattern
    if (kq == sl) {
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wk * 64 + sl * 16 + j * 4 + r] = yacc[r];
    }
    __syncthreads();
    if (wk == 0) {
        float acc = 0.f;
        int w2 = 0;
        for (; w2 + 4 <= KW; w2 += 4) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = red[(w2 + u) * 64 + lane];
#pragma unroll
            for (int u = 0; u < 4; ++u) acc += v[u];
        }
        for (; w2 < KW; ++w2) acc += red[w2 * 64 + lane];
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        const int jo = (lane >> 2) & 3, m = lane & 3;
        if (lane < 16 && m < M && col0 + jo < N) y[static_cast<size_t>(m) * N + col0 + jo] = f32_to_bf16_bits(acc);
    }
}

bool qmv_burst_shape(int M, int N, int K, QmvBurstShape* out) {
    const int G = K / kGroup;
    if (M < 1 || M > kBurstMaxRows || K % kGroup != 0 || G < 1 || N < 1) return false;
    const int blocks = (N + 15) / 16;
    if (M > kBurstRows) {
        // 5..8 rows: the 16-column form with 8 row slots, below 1024 column blocks and up to 64
        // groups (16 waves of at most 4; more would pass the LDS).  Measured on MI355X (graph
        // replay, rotating weights): M = 8 on 9728 x 2560 9.5 us against 10.3 for the
        // row-amortized loop kernel, 4096 x 2560 5.4 against 5.8, 1024 x 2560 5.1 against 5.5;
        // M = 5 8.3 / 5.0 / 4.7 against 9.2 / 5.4 / 5.1; two groups per wave measured best.
        if (blocks >= 1024 || G > 4 * kQmvBurstMaxWaves) return false;
        int g = 2;
        const int need = (G + kQmvBurstMaxWaves - 1) / kQmvBurstMaxWaves;
        if (need > g) g = need;
        out->packed = 0;
        out->gpw = g;
        out->kw = (G + g - 1) / g;
        out->rows = 2 * kBurstRows;
        out->cols = 16;
        return true;
    }
    // From 2048 column blocks of 16 the persistent wide kernel leads both forms (151936 x 2560:
    // 43 us against 50-55; 32768 and 65536 x 2560: 13.0 and 21.2 against 14.5 and 24.9), and
    // from 1664 blocks under 32 groups where it applies (30000 x 2560: 12.9 against 13.6 us at
    // M = 1, 13.1 against 15.4 at M = 2; 24600 x 2560: 12.9 against 12.0 and 13.2 against 13.3).
    if (blocks >= 2048 || (blocks >= 1664 && G < 32 && qmv_wide_fits(M, K))) return false;
    // The packed form.  At 1 and 2 rows below 2048 blocks and up to 128 groups (graph-replayed,
    // rotating weights, M = 1, N x K: 9728 x 2560 6.7 us against 7.1-7.6 for the 16-column
    // form, 2560 x 9728 7.5-7.8 against 9.0, 1024 x 2560 3.3 against 4.1; from 1024 blocks, two steps
    // per wave, against the wide kernel: 16400 x 9728 27.3 against 42.3 us, 20000 x 8192 23.4
    // against 38.1, 16400 x 4096 11.6 against 16.1, 24600 x 4096 15.4 against 18.6; beyond 80
    // groups against the K-split kernel: 1000 x 16384 5.5 against 17.4).  At 3 and
    // 4 rows, whose 4-row activation slots take 4x the LDS and loads, only up to 160 blocks and
    // 64 groups (M = 4: 1024 x 2560 3.8 against 4.5, 2560 x 4096 6.7 against 6.9; 2560 x 9728
    // 15.7 against 10.6).  One step of 4 groups per wave below 1024 blocks up to 64 groups, two
    // steps otherwise.
    if ((M <= 2 && G <= 8 * kQmvBurstMaxWaves) || (blocks <= 160 && G <= 4 * kQmvBurstMaxWaves)) {
        out->packed = 1;
        out->gpw = blocks >= 1024 || G > 4 * kQmvBurstMaxWaves ? 2 : 1;
        out->kw = (G + 4 * out->gpw - 1) / (4 * out->gpw);
        out->rows = M == 1 ? 1 : (M == 2 ? 2 : 4);
        out->cols = 4;
        return true;
    }
    // The 16-column form at 3 and 4 rows: the fewer groups a wave owns the better while the
    // launch has fewer than 1024 blocks (two per wave), from 1024 blocks three (16400 x 2560:
    // 8.5 us, the wide kernel 10.9), but not from 32 groups (16400 x 4096: 18.2 us, the wide
    // kernel 16.2); above 32 groups, as few groups per wave as 16 waves allow, up to 80 groups.
    if ((blocks >= 1024 && G >= 32) || G > kQmvBurstMaxWaves * kQmvBurstMaxGroups) return false;
    int g = blocks >= 1024 ? 3 : 2;
    const int need = (G + kQmvBurstMaxWaves - 1) / kQmvBurstMaxWaves;
    if (need > g) g = need;
    out->packed = 0;
    out->gpw = g;
    out->kw = (G + g - 1) / g;
    out->rows = kBurstRows;
    out->cols = 16;
    return true;
}

namespace {

constexpr int kMaxDevices = 64;

// Once per kernel instance and device: permission for the largest dynamic LDS its launches
// use (16 waves), which may pass the 64 KB a launch gets by default.
template <typename Kern>
hipError_t allow_lds(Kern kern, size_t bytes, std::atomic<bool> (&ready)[kMaxDevices]) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!ready[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(bytes));
        if (e != hipSuccess) return e;
        ready[dev].store(true, std::memory_order_release);
    }
    return hipSuccess;
}

// LDS of a KW-wave packed workgroup: each wave's activation slots (4 GPW groups x 16 chunks x
// MR rows of 16 bytes), then 64 fp32 partial sums per wave.
constexpr size_t packed_lds_bytes(int kw, int gpw, int mr) {
    return static_cast<size_t>(kw) * 4 * gpw * 16 * mr * 16 + static_cast<size_t>(kw) * 64 * 4;
}

}  // namespace

template <int GPW, int MR>
static hipError_t launch_burst_t(int kw, const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                                 uint16_t* y, int M, int N, int K, hipStream_t stream) {
    static std::atomic<bool> ready[kMaxDevices];
    auto kern = qmv_burst_kernel<GPW, MR>;
    const hipError_t e = allow_lds(kern, burst_lds_bytes(kQmvBurstMaxWaves, GPW, MR), ready);
    if (e != hipSuccess) return e;
    W4A16_LAUNCH(kern, dim3((N + 15) / 16), dim3(64 * kw), burst_lds_bytes(kw, GPW, MR), stream, x, wq, s, b, y,
                       M, N, K, kw);
    return hipGetLastError();
}

template <int GPW, int MR>
static hipError_t launch_packed_t(int kw, const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                                  uint16_t* y, int M, int N, int K, hipStream_t stream) {
    static std::atomic<bool> ready[kMaxDevices];
    auto kern = qmv_burst_packed_kernel<GPW, MR>;
    const hipError_t e = allow_lds(kern, packed_lds_bytes(kQmvBurstMaxWaves, GPW, MR), ready);
    if (e != hipSuccess) return e;
    W4A16_LAUNCH(kern, dim3((N + 3) / 4), dim3(64 * kw), packed_lds_bytes(kw, GPW, MR), stream, x, wq, s, b, y,
                       M, N, K, kw);
    return hipGetLastError();
}

hipError_t launch_qmv_burst(const uint16_t* x, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                            uint16_t* y, int M, int N, int K, hipStream_t stream) {
    QmvBurstShape sh;
    if (!qmv_burst_shape(M, N, K, &sh)) return hipErrorInvalidValue;
    const int kw = sh.kw, G = K / kGroup;
    if (sh.packed) {
        // the waves' shares of 4 gpw groups cover every group; the row slots cover M
        if (kw < 1 || kw > kQmvBurstMaxWaves || static_cast<int64_t>(kw) * 4 * sh.gpw < G || sh.rows < M)
            return hipErrorInvalidValue;
        const int key = sh.gpw * 10 + sh.rows;
        switch (key) {
            case 11: return launch_packed_t<1, 1>(kw, x, wq, scales, biases, y, M, N, K, stream);
            case 12: return launch_packed_t<1, 2>(kw, x, wq, scales, biases, y, M, N, K, stream);
            case 14: return launch_packed_t<1, 4>(kw, x, wq, scales, biases, y, M, N, K, stream);
            case 21: return launch_packed_t<2, 1>(kw, x, wq, scales, biases, y, M, N, K, stream);
            case 22: return launch_packed_t<2, 2>(kw, x, wq, scales, biases, y, M, N, K, stream);
            default: return hipErrorInvalidValue;
        }
    }
    // the waves' shares of gpw groups cover every group, within the workgroup bound
    if (kw < 1 || kw > kQmvBurstMaxWaves || static_cast<int64_t>(kw) * sh.gpw < G) return hipErrorInvalidValue;
    if (sh.rows < M) return hipErrorInvalidValue;
    switch (sh.gpw * 100 + sh.rows) {
        case 204: return launch_burst_t<2, 4>(kw, x, wq, scales, biases, y, M, N, K, stream);
        case 304: return launch_burst_t<3, 4>(kw, x, wq, scales, biases, y, M, N, K, stream);
        case 404: return launch_burst_t<4, 4>(kw, x, wq, scales, biases, y, M, N, K, stream);
        case 504: return launch_burst_t<5, 4>(kw, x, wq, scales, biases, y, M, N, K, stream);
        case 208: return launch_burst_t<2, 8>(kw, x, wq, scales, biases, y, M, N, K, stream);
        case 308: return launch_burst_t<3, 8>(kw, x, wq, scales, biases, y, M, N, K, stream);
        case 408: return launch_burst_t<4, 8>(kw, x, wq, scales, biases, y, M, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
