// qmv_bits: affine matvec for decode rows (M <= 8) at 1, 2, 3, 4 or 8 bits per code.
//
// "Route affine qmv_wide by bit-width and batch size #5" routes affine quantized matvecs by
// code width and row count between a per-row kernel and a row-amortized kernel that
// dequantizes a group once and reuses it across the M rows.  Both exist here for every width,
// sharing the load and unpack code; the dispatch policy picks one from measurements.
//
// Format (the width-generic reading of the W4 layout): a column's row of words is one bit
// stream, lowest bits first, element k in stream bits BITS*k .. BITS*k + BITS - 1; at 1, 2, 4
// and 8 bits that is element (32/BITS)*j + i in bits BITS*i .. of word j, at 3 bits every 32
// codes fill three words and two of them straddle a word.  One bf16 scale and bias per 128
// reduction values; w = s * q + b.
//
// Lane layout, per 128-value group of one 16-column block: lane l holds column c = l % 16 and
// the 32 consecutive reduction values kq*32 .. kq*32 + 31 of the group, kq = l / 16 -- the B
// operand of v_mfma_f32_16x16x32_bf16.  Its codes are 4*BITS contiguous bytes of the column's
// row, loaded with one buffer load (two at 8 bits).  They become exact bf16 integers:
//   * 1, 2 and 4 bits: masked words hold one code per byte; a byte 0..15 read as an OCP e4m3
//     value is q * 2^-9, so the scaled converter with scale 2^9 gives q exactly, two per
//     instruction (the same identity the 4-bit kernels use);
//   * 3 bits: each 24 stream bits (8 codes) are spread in two bit-field inserts to one pair
//     of codes per byte (codes 2i, 2i + 1 in bits 0..2, 3..5 of byte i), then masked into
//     one code per byte and converted as above;
//   * 8 bits: v_cvt_f32_ubyte* then a bf16 pack (integers up to 255 are exact in bf16).
// The unpack order is not the natural one (except at 8 bits), so the activations are put in the
// same order with v_perm_b32 (CodeOrder below); any bijection of the reduction index works as
// long as codes and activations agree.
//
// Modes:
//   * kMatrix (row-amortized): the M rows (zero-padded to 16) are the A operand; per group
//     P = sum x*q and X = sum x come from the matrix core and y += s*P + b*X.
//   * kRows (per-row): for each row, P and X from v_dot2_f32_bf16 on (activation, code) pairs;
//     rows are not amortized.  Serves M <= 2.
// A workgroup is KW waves on one 16-column block, splitting its groups; the partial sums are
// added in wave order through LDS, so results do not depend on timing.  Every load goes through
// a buffer resource: columns past N and rows past M read zeros, and byte offsets that can pass
// the end of a buffer are in the per-lane (range-checked) offset.
#include "device_common.h"
#include "internal.h"

#include <atomic>

namespace w4a16 {

namespace {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));

// Reduction offset (0..31 within the lane's 32 values) of B-operand element 8t + e.
template <int BITS>
struct CodeOrder;
template <>
struct CodeOrder<8> {
    static constexpr int at(int i) { return i; }
};
template <>
struct CodeOrder<4> {   // per word t: [q0, q2, q1, q3, q4, q6, q5, q7]
    static constexpr int at(int i) {
        constexpr int w[8] = {0, 2, 1, 3, 4, 6, 5, 7};
        return 8 * (i / 8) + w[i % 8];
    }
};
template <>
struct CodeOrder<3> {   // operand t: codes 8t + [0, 2, 4, 6, 1, 3, 5, 7]
    static constexpr int at(int i) {
        const int e = i % 8;
        return 8 * (i / 8) + 2 * (e % 4) + e / 4;
    }
};
template <>
struct CodeOrder<2> {   // operand t: word t/2, shifts 2*i0 and 2*(i0+1), i0 = 2*(t%2)
    static constexpr int at(int i) {
        const int t = i / 8, e = i % 8, i0 = 2 * (t % 2) + e / 4, pos = e % 4;
        return 16 * (t / 2) + i0 + 4 * pos;
    }
};
template <>
struct CodeOrder<1> {   // operand t: shifts 2t and 2t + 1
    static constexpr int at(int i) {
        const int t = i / 8, e = i % 8, sh = 2 * t + e / 4, pos = e % 4;
        return sh + 8 * pos;
    }
};

// The lane's 32 codes (BITS words: 4*BITS bytes) as four B operands of exact bf16 integers,
// element 8t + e holding reduction offset CodeOrder<BITS>::at(8t + e).
template <int BITS>
__device__ __forceinline__ void codes_to_bf16(const uint32_t (&w)[BITS], u32x4_t (&bop)[4]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t v = w[2 * t + h];
                const bf16x2_t lo = {static_cast<__bf16>(static_cast<float>(v & 0xFFu)),
                                     static_cast<__bf16>(static_cast<float>((v >> 8) & 0xFFu))};
                const bf16x2_t hi = {static_cast<__bf16>(static_cast<float>((v >> 16) & 0xFFu)),
                                     static_cast<__bf16>(static_cast<float>(v >> 24))};
                bop[t][2 * h] = __builtin_bit_cast(uint32_t, lo);
                bop[t][2 * h + 1] = __builtin_bit_cast(uint32_t, hi);
            }
        }
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int t = 0; t < 4; ++t) bop[t] = __builtin_bit_cast(u32x4_t, codes_bf16_permuted(w[t]));
    } else if constexpr (BITS == 3) {
        // operand t: stream bits 24t .. 24t + 23 (low 24 bits of the chunk; the rest is ignored)
        const uint32_t chunk[4] = {w[0], __builtin_amdgcn_alignbit(w[1], w[0], 24),
                                   __builtin_amdgcn_alignbit(w[2], w[1], 16), w[2] >> 8};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t u = chunk[t];
            // codes 4..7 to bits 16..27 (bits 12..15 and 28..31 are left over, never read)
            u = (u & 0x00000FFFu) | ((u << 4) & ~0x00000FFFu);
            // codes 2, 3 and 6, 7 to bytes 1 and 3: byte i holds codes 2i, 2i + 1 in bits 0..5
            u = (u & 0x003F003Fu) | ((u << 2) & ~0x003F003Fu);
            const uint32_t m0 = u & 0x07070707u, m1 = (u >> 3) & 0x07070707u;
            bop[t][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m0, 512.0f, false));
            bop[t][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m0, 512.0f, true));
            bop[t][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m1, 512.0f, false));
            bop[t][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m1, 512.0f, true));
        }
    } else {
        constexpr uint32_t mask = BITS == 2 ? 0x03030303u : 0x01010101u;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t v = BITS == 2 ? w[t / 2] : w[0];
            const int s0 = BITS == 2 ? 2 * (2 * (t % 2)) : 2 * t;     // shift of the first masked word
            const uint32_t m0 = (v >> s0) & mask, m1 = (v >> (s0 + BITS)) & mask;
            bop[t][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m0, 512.0f, false));
            bop[t][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m0, 512.0f, true));
            bop[t][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m1, 512.0f, false));
            bop[t][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m1, 512.0f, true));
        }
    }
}

// Activation pair (a, b) of the lane's 32 values (xv: natural order, dword d = values 2d, 2d+1)
// as one dword: a in the low half, b in the high half.
template <int A, int B>
__device__ __forceinline__ uint32_t act_pair(const u32x4_t (&xv)[4]) {
    constexpr uint32_t sel = (2u * (A % 2)) | ((2u * (A % 2) + 1u) << 8) | ((4u + 2u * (B % 2)) << 16) |
                             ((5u + 2u * (B % 2)) << 24);
    return __builtin_amdgcn_perm(xv[(B / 2) / 4][(B / 2) % 4], xv[(A / 2) / 4][(A / 2) % 4], sel);
}

template <int BITS, int T, int E2>
__device__ __forceinline__ uint32_t act_dword(const u32x4_t (&xv)[4]) {
    return act_pair<CodeOrder<BITS>::at(8 * T + 2 * E2), CodeOrder<BITS>::at(8 * T + 2 * E2 + 1)>(xv);
}

// The activations in the codes' order, as four operands.
template <int BITS>
__device__ __forceinline__ void acts_in_code_order(const u32x4_t (&xv)[4], u32x4_t (&aop)[4]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int t = 0; t < 4; ++t) aop[t] = xv[t];
    } else {
        aop[0] = u32x4_t{act_dword<BITS, 0, 0>(xv), act_dword<BITS, 0, 1>(xv), act_dword<BITS, 0, 2>(xv),
                         act_dword<BITS, 0, 3>(xv)};
        aop[1] = u32x4_t{act_dword<BITS, 1, 0>(xv), act_dword<BITS, 1, 1>(xv), act_dword<BITS, 1, 2>(xv),
                         act_dword<BITS, 1, 3>(xv)};
        aop[2] = u32x4_t{act_dword<BITS, 2, 0>(xv), act_dword<BITS, 2, 1>(xv), act_dword<BITS, 2, 2>(xv),
                         act_dword<BITS, 2, 3>(xv)};
        aop[3] = u32x4_t{act_dword<BITS, 3, 0>(xv), act_dword<BITS, 3, 1>(xv), act_dword<BITS, 3, 2>(xv),
                         act_dword<BITS, 3, 3>(xv)};
    }
}

// AUX: the loads' cache policy (kStreamedOnce where the kernel measured faster with it).
template <int BITS, int AUX = 0>
__device__ __forceinline__ void load_codes(const __amdgpu_buffer_rsrc_t& r, uint32_t voff, uint32_t soff,
                                           uint32_t (&w)[BITS]) {
    if constexpr (BITS == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
    } else if constexpr (BITS == 2) {
        const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX));
        w[0] = v[0];
        w[1] = v[1];
    } else if constexpr (BITS == 3) {
        const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, AUX);
        w[0] = v[0];
        w[1] = v[1];
        w[2] = v[2];
    } else {
#pragma unroll
        for (int h = 0; h < BITS / 4; ++h) {
            const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16 * h, AUX));
#pragma unroll
            for (int i = 0; i < 4; ++i) w[4 * h + i] = v[i];
        }
    }
}

}  // namespace

constexpr int kMatrix = kQmvBitsMatrix, kRows = kQmvBitsRows;

template <int BITS, int KW, int MODE>
__global__ __launch_bounds__(64 * KW) void qmv_bits_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int N, int K) {
    constexpr int MR = MODE == kRows ? 2 : 1;   // rows held per lane in the per-row mode
    const int G = K >> 7;
    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col0 = blockIdx.x * 16;
    const int g0 = static_cast<int>(static_cast<int64_t>(wk) * G / KW);
    const int g1 = static_cast<int>(static_cast<int64_t>(wk + 1) * G / KW);
    const int c = lane & 15, kq = lane >> 4;
    const int row_bytes = K / 8 * BITS;
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
    const uint32_t wvoff = static_cast<uint32_t>(c * row_bytes + kq * 4 * BITS);
    const uint32_t sbvoff = static_cast<uint32_t>(c * G * 2);

    // one group's operands: codes, scale, bias, activations of the lane's rows
    struct Step {
        uint32_t w[BITS];
        uint16_t s, b;
        u32x4_t xv[MR][4];
    };
    auto load_step = [&](int g, Step& o) {
        load_codes<BITS>(wr, wvoff, static_cast<uint32_t>(g * 16 * BITS), o.w);
        o.s = __builtin_amdgcn_raw_buffer_load_b16(sr, sbvoff, g * 2, 0);
        o.b = __builtin_amdgcn_raw_buffer_load_b16(br, sbvoff, g * 2, 0);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            // matrix mode: lane row l % 16; per-row mode: rows 0 and 1 (broadcast over columns)
            const int row = MODE == kMatrix ? (lane & 15) : r;
            const uint32_t xvoff = row < M ? static_cast<uint32_t>(row * K + kq * 32) * 2u : 0x80000000u;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                o.xv[r][t] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, xvoff, (g * kGroup + t * 8) * 2, 0));
        }
    };

    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const bf16x8_t ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                           __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
    const bf16x2_t ones2 = {__bf16(1.f), __bf16(1.f)};
    f32x4_t yacc = zero4;          // matrix mode: rows 4*kq + r of column c
    float racc[MR] = {};           // per-row mode: partial sums of rows 0..MR-1 over this lane's values

    auto compute = [&](const Step& o) {
        u32x4_t bop[4];
        codes_to_bf16<BITS>(o.w, bop);
        const float s = bf16_bits_to_f32(o.s), b = bf16_bits_to_f32(o.b);
        if constexpr (MODE == kMatrix) {
            u32x4_t aop[4];
            acts_in_code_order<BITS>(o.xv[0], aop);
            f32x4_t xs = zero4, p = zero4;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, aop[t]);
                xs = mfma16x16x32(a, ones, xs);
                p = mfma16x16x32(a, __builtin_bit_cast(bf16x8_t, bop[t]), p);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[r] = __builtin_fmaf(s, p[r], __builtin_fmaf(b, xs[r], yacc[r]));
        } else {
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                if (r >= M) break;
                u32x4_t aop[4];
                acts_in_code_order<BITS>(o.xv[r], aop);
                float p = 0.f, xs = 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        // elements are copied out before the bit cast: a cast applied to the
                        // vector element itself reads element 0
                        const uint32_t a = aop[t][d], q = bop[t][d], xn = o.xv[r][t][d];
                        p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                                           __builtin_bit_cast(bf16x2_t, q), p, false);
                        xs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xn), ones2, xs, false);
                    }
                racc[r] = __builtin_fmaf(s, p, __builtin_fmaf(b, xs, racc[r]));
            }
        }
    };

    // one group in flight ahead of the one computed, in ping-pong register sets
    if (g0 < g1) {
        Step sa, sb;
        load_step(g0, sa);
        for (int g = g0;; g += 2) {
            if (g + 1 < g1) load_step(g + 1, sb);
            compute(sa);
            if (g + 1 >= g1) break;
            if (g + 2 < g1) load_step(g + 2, sa);
            compute(sb);
            if (g + 2 >= g1) break;
        }
    }

    // per-row mode: the four lanes of a column (kq = 0..3) hold quarters of the sums
    if constexpr (MODE == kRows) {
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            racc[r] += __shfl_xor(racc[r], 16);
            racc[r] += __shfl_xor(racc[r], 32);
        }
    }

    if constexpr (KW > 1) {
        __shared__ float red[KW - 1][4][64];
        if (wk > 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wk - 1][r][lane] = MODE == kMatrix ? yacc[r] : (r < MR ? racc[r < MR ? r : 0] : 0.f);
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int j = 0; j < KW - 1; ++j) {
                if constexpr (MODE == kMatrix) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) yacc[r] += red[j][r][lane];
                } else {
#pragma unroll
                    for (int r = 0; r < MR; ++r) racc[r] += red[j][r][lane];
                }
            }
        }
    }

    if (wk == 0) {
        const int col = col0 + c;
        if (col < N) {
            if constexpr (MODE == kMatrix) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * kq + r;
                    if (m < M) y[static_cast<size_t>(m) * N + col] = f32_to_bf16_bits(yacc[r]);
                }
            } else if (kq == 0) {
#pragma unroll
                for (int r = 0; r < MR; ++r)
                    if (r < M) y[static_cast<size_t>(r) * N + col] = f32_to_bf16_bits(racc[r]);
            }
        }
    }
}

template <int BITS, int KW, int MODE>
static hipError_t launch_qmv_bits_t(const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                                    uint16_t* y, int M, int N, int K, hipStream_t stream) {
    if (M < 1 || M > (MODE == kRows ? 2 : 16)) return hipErrorInvalidValue;   // rows one operand holds
    W4A16_LAUNCH((qmv_bits_kernel<BITS, KW, MODE>), dim3((N + 15) / 16), dim3(64 * KW), 0, stream, x, wq, s, b,
                       y, M, N, K);
    return hipGetLastError();
}

// Burst form of the width-generic matvec, at most 4 rows: the packed layout of the 4-bit burst
// kernel (qmv_burst.hip) -- 4 K slices in the MFMA's spare rows, A rows 4s + m holding row m of
// slice s, B columns 4s + j holding column j's codes of slice s, the 4 diagonal 4 x 4 blocks of
// the result kept -- with the codes of any width.  A workgroup covers 4 columns with KW waves;
// wave w takes GPW steps of 4 consecutive groups and issues every load of them (codes: 4*BITS
// bytes per lane and group; scales, biases; its activation slots) before its first MFMA.  The
// activations are staged in their natural order and put in the codes' order (CodeOrder) as they
// are read back.  Wave 0 adds the waves' sums in wave order and the 4 slices in a fixed lane
// pattern, so results do not depend on timing.
template <int BITS, int GPW, int MR>
__global__ __launch_bounds__(64 * kQmvBurstMaxWaves) void qmv_bits_burst_kernel(
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
    const int sl = c >> 2, j = c & 3;   // slice and column (B operand) or slice and row (A operand)
    const int row_bytes = K / 8 * BITS;
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

    // 1. every load of the wave (past the last group, column or row the per-lane offset passes
    //    the resource's end and the load returns zeros)
    uint32_t w[GPW][BITS];
    uint16_t sv[GPW], bv[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int g = g0 + 4 * i + sl;
        const uint32_t voff =
            g < G ? static_cast<uint32_t>(j * row_bytes + g * 16 * BITS + kq * 4 * BITS) : 0x80000000u;
        load_codes<BITS, kStreamedOnce>(wr, voff, 0, w[i]);
    }
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int g = g0 + 4 * i + sl;
        const uint32_t voff = g < G ? static_cast<uint32_t>((j * G + g) * 2) : 0x80000000u;
        sv[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, voff, 0, 0);
        bv[i] = __builtin_amdgcn_raw_buffer_load_b16(br, voff, 0, 0);
    }
    // activation chunk jj = ((gl * 4 + t) * 4 + q) * MR + m: row m's values gl*128 + q*32 + t*8 .. +7
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
    for (int j0 = 0; j0 < XL; ++j0) xs[j0 * 64 + lane] = xv[j0];
    asm volatile("" ::: "memory");   // the wave's own slots: only the compiler must keep the order

    // 2. every step: the result lane (c, kq) holds rows 4 kq .. 4 kq + 3 of column c, wanted where
    //    kq is column c's slice
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const u32x4_t zu = {0u, 0u, 0u, 0u};
    const bf16x8_t ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                           __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
    const bool arow = j < M && j < MR;
    const int am = j < MR ? j : 0;
    f32x4_t yacc = zero4;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        u32x4_t xn[4], aop[4], bop[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) xn[t] = arow ? xs[(((4 * i + sl) * 4 + t) * 4 + kq) * MR + am] : zu;
        acts_in_code_order<BITS>(xn, aop);
        codes_to_bf16<BITS>(w[i], bop);
        f32x4_t xsum = zero4, p = zero4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, aop[t]);
            xsum = mfma16x16x32(a, ones, xsum);
            p = mfma16x16x32(a, __builtin_bit_cast(bf16x8_t, bop[t]), p);
        }
        const float s = bf16_bits_to_f32(sv[i]), b = bf16_bits_to_f32(bv[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[r] = __builtin_fmaf(s, p[r], __builtin_fmaf(b, xsum[r], yacc[r]));
    }

    // 3. the wanted lanes hand rows 0..3 of their column to LDS; wave 0, lane 16 s + 4 j + m, adds
    //    its (slice, column, row) over the waves in wave order, then the 4 slices of each output
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

// The 16-column burst form at any width (3 to 8 rows, where the packed form's 4-row slots would
// take too much LDS): the layout of the 4-bit 16-column burst kernel (qmv_burst.hip) -- KW
// waves on one 16-column block, wave w owning groups w*GPW .. w*GPW + GPW - 1 and issuing every
// load of them before its first MFMA -- with the codes of any width and the activations staged
// in natural order, put in the width's code order as they are read back.  MR row slots (4 or 8)
// per activation chunk; wave 0 adds the waves' sums in wave order.
template <int BITS, int GPW, int MR>
__global__ __launch_bounds__(64 * kQmvBurstMaxWaves) void qmv_bits_burst16_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, int M, int N, int K, int KW) {
    static_assert(MR == 4 || MR == 8, "row slots: a power of two that divides the 64 lanes");
    extern __shared__ __attribute__((aligned(16))) u32x4_t lds[];
    const int G = K >> 7;
    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col0 = blockIdx.x * 16;
    const int g0 = wk * GPW;
    const int ng = min(GPW, G - g0);
    const int c = lane & 15, kq = lane >> 4;
    const int row_bytes = K / 8 * BITS;
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
    const uint32_t wvoff = static_cast<uint32_t>(c * row_bytes + kq * 4 * BITS);
    const uint32_t sbvoff = static_cast<uint32_t>(c * G * 2);
    u32x4_t* const xs = lds + static_cast<size_t>(wk) * GPW * 16 * MR;
    f32x4_t* const red = reinterpret_cast<f32x4_t*>(lds + static_cast<size_t>(KW) * GPW * 16 * MR);

    // 1. every load of the wave; slots past its share read through the zero-sized resource and
    //    add exactly +0 below, which keeps every load unconditional
    uint32_t w[GPW][BITS];
    uint16_t sv[GPW], bv[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) load_codes<BITS>(i < ng ? wr : none, wvoff, static_cast<uint32_t>((g0 + i) * 16 * BITS), w[i]);
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        sv[i] = __builtin_amdgcn_raw_buffer_load_b16(i < ng ? sr : none, sbvoff, (g0 + i) * 2, 0);
        bv[i] = __builtin_amdgcn_raw_buffer_load_b16(i < ng ? br : none, sbvoff, (g0 + i) * 2, 0);
    }
    // activation chunk j = ((gl * 4 + t) * 4 + q) * MR + m: row m's values gl*128 + q*32 + t*8 .. +7
    constexpr int XL = GPW * 16 * MR / 64;
    u32x4_t xv[XL];
#pragma unroll
    for (int j0 = 0; j0 < XL; ++j0) {
        const int j = j0 * 64 + lane;
        const int m = j % MR, r = j / MR;
        const int q = r & 3, t = (r >> 2) & 3, gl = r >> 4;
        const uint32_t voff = m < M && gl < ng
                                  ? static_cast<uint32_t>(m * K + (g0 + gl) * kGroup + q * 32 + t * 8) * 2u
                                  : 0x80000000u;
        xv[j0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, voff, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);   // all loads issued before anything waits on one
#pragma unroll
    for (int j0 = 0; j0 < XL; ++j0) xs[j0 * 64 + lane] = xv[j0];
    asm volatile("" ::: "memory");   // the wave's own slice: only the compiler must keep the order

    // 2. every group: rows 4*kq + r of column c
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const u32x4_t zu = {0u, 0u, 0u, 0u};
    const bf16x8_t ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                           __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};
    const int arow = lane & 15;
    f32x4_t yacc = zero4;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        u32x4_t xn[4], aop[4], bop[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) xn[t] = arow < M ? xs[((i * 4 + t) * 4 + kq) * MR + arow] : zu;
        acts_in_code_order<BITS>(xn, aop);
        codes_to_bf16<BITS>(w[i], bop);
        f32x4_t xsum = zero4, p = zero4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, aop[t]);
            xsum = mfma16x16x32(a, ones, xsum);
            p = mfma16x16x32(a, __builtin_bit_cast(bf16x8_t, bop[t]), p);
        }
        const float s = bf16_bits_to_f32(sv[i]), b = bf16_bits_to_f32(bv[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[r] = __builtin_fmaf(s, p[r], __builtin_fmaf(b, xsum[r], yacc[r]));
    }

    // 3. waves 1..KW-1 hand their sums to wave 0 (one 16-byte slot per lane), which adds them in
    //    wave order, four waves' slots read before they are added
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

bool qmv_bits_burst_shape(int M, int N, int K, QmvBurstShape* out) {
    const int G = K / kGroup;
    if (M < 1 || M > 8 || K % kGroup != 0 || G < 1 || N < 1) return false;
    // The 4-bit burst forms' domains.  Packed: below 2048 column blocks of 16 and up to 128
    // groups, at 3 and 4 rows up to 160 blocks and 64 groups; one step per wave below 1024
    // blocks up to 64 groups, two otherwise.  16 columns: the rest below 1024 blocks, up to 80
    // groups at 3 and 4 rows (4 row slots) and 64 at 5 to 8 rows (8 slots), two groups per wave
    // or as few as 16 waves allow.
    const int blocks = (N + 15) / 16;
    if (M <= 4 && blocks < 2048 && G <= 8 * kQmvBurstMaxWaves && (M <= 2 || (blocks <= 160 && G <= 64))) {
        out->packed = 1;
        out->gpw = blocks >= 1024 || G > 4 * kQmvBurstMaxWaves ? 2 : 1;
        out->kw = (G + 4 * out->gpw - 1) / (4 * out->gpw);
        out->rows = M == 1 ? 1 : (M == 2 ? 2 : 4);
        out->cols = 4;
        return true;
    }
    if (M <= 2 || blocks >= 1024 || G > (M <= 4 ? kQmvBurstMaxGroups : 4) * kQmvBurstMaxWaves) return false;
    int g = 2;
    const int need = (G + kQmvBurstMaxWaves - 1) / kQmvBurstMaxWaves;
    if (need > g) g = need;
    out->packed = 0;
    out->gpw = g;
    out->kw = (G + g - 1) / g;
    out->rows = M <= 4 ? 4 : 8;
    out->cols = 16;
    return true;
}

namespace {

constexpr int kMaxDevices = 64;

constexpr size_t bits_burst_lds_bytes(int kw, int gpw, int mr) {
    return static_cast<size_t>(kw) * 4 * gpw * 16 * mr * 16 + static_cast<size_t>(kw) * 64 * 4;
}

template <int BITS, int GPW, int MR>
hipError_t launch_bits_burst_t(int kw, const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                               uint16_t* y, int M, int N, int K, hipStream_t stream) {
    static std::atomic<bool> ready[kMaxDevices];   // per instance and device: the LDS permission is set
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    auto kern = qmv_bits_burst_kernel<BITS, GPW, MR>;
    if (!ready[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(bits_burst_lds_bytes(kQmvBurstMaxWaves, GPW, MR)));
        if (e != hipSuccess) return e;
        ready[dev].store(true, std::memory_order_release);
    }
    W4A16_LAUNCH(kern, dim3((N + 3) / 4), dim3(64 * kw), bits_burst_lds_bytes(kw, GPW, MR), stream, x, wq, s, b,
                       y, M, N, K, kw);
    return hipGetLastError();
}

constexpr size_t bits_burst16_lds_bytes(int kw, int gpw, int mr) {
    return static_cast<size_t>(kw) * gpw * 16 * mr * 16 + static_cast<size_t>(kw - 1) * 64 * 16;
}

template <int BITS, int GPW, int MR>
hipError_t launch_bits_burst16_t(int kw, const uint16_t* x, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                                 uint16_t* y, int M, int N, int K, hipStream_t stream) {
    static std::atomic<bool> ready[kMaxDevices];   // per instance and device: the LDS permission is set
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    auto kern = qmv_bits_burst16_kernel<BITS, GPW, MR>;
    if (!ready[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(bits_burst16_lds_bytes(kQmvBurstMaxWaves, GPW, MR)));
        if (e != hipSuccess) return e;
        ready[dev].store(true, std::memory_order_release);
    }
    W4A16_LAUNCH(kern, dim3((N + 15) / 16), dim3(64 * kw), bits_burst16_lds_bytes(kw, GPW, MR), stream, x, wq,
                       s, b, y, M, N, K, kw);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits_burst_w(const QmvBurstShape& sh, const uint16_t* x, const uint32_t* wq, const uint16_t* s,
                               const uint16_t* b, uint16_t* y, int M, int N, int K, hipStream_t stream) {
    if (!sh.packed) {
        switch (sh.gpw * 100 + sh.rows) {
            case 204: return launch_bits_burst16_t<BITS, 2, 4>(sh.kw, x, wq, s, b, y, M, N, K, stream);
            case 304: return launch_bits_burst16_t<BITS, 3, 4>(sh.kw, x, wq, s, b, y, M, N, K, stream);
            case 404: return launch_bits_burst16_t<BITS, 4, 4>(sh.kw, x, wq, s, b, y, M, N, K, stream);
            case 504: return launch_bits_burst16_t<BITS, 5, 4>(sh.kw, x, wq, s, b, y, M, N, K, stream);
            case 208: return launch_bits_burst16_t<BITS, 2, 8>(sh.kw, x, wq, s, b, y, M, N, K, stream);
            case 308: return launch_bits_burst16_t<BITS, 3, 8>(sh.kw, x, wq, s, b, y, M, N, K, stream);
            case 408: return launch_bits_burst16_t<BITS, 4, 8>(sh.kw, x, wq, s, b, y, M, N, K, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (sh.gpw * 10 + sh.rows) {
        case 11: return launch_bits_burst_t<BITS, 1, 1>(sh.kw, x, wq, s, b, y, M, N, K, stream);
        case 12: return launch_bits_burst_t<BITS, 1, 2>(sh.kw, x, wq, s, b, y, M, N, K, stream);
        case 14: return launch_bits_burst_t<BITS, 1, 4>(sh.kw, x, wq, s, b, y, M, N, K, stream);
        case 21: return launch_bits_burst_t<BITS, 2, 1>(sh.kw, x, wq, s, b, y, M, N, K, stream);
        case 22: return launch_bits_burst_t<BITS, 2, 2>(sh.kw, x, wq, s, b, y, M, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_qmv_bits_burst(int bits, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                                 const uint16_t* biases, uint16_t* y, int M, int N, int K, hipStream_t stream) {
    QmvBurstShape sh;
    if (!qmv_bits_burst_shape(M, N, K, &sh)) return hipErrorInvalidValue;
    // the waves' shares (4 gpw groups packed, gpw groups otherwise) cover every group; the row
    // slots cover M
    const int64_t per_wave = sh.packed ? 4 * sh.gpw : sh.gpw;
    if (sh.kw < 1 || sh.kw > kQmvBurstMaxWaves || static_cast<int64_t>(sh.kw) * per_wave < K / kGroup || sh.rows < M)
        return hipErrorInvalidValue;
    switch (bits) {
        case 1: return launch_bits_burst_w<1>(sh, x, wq, scales, biases, y, M, N, K, stream);
        case 2: return launch_bits_burst_w<2>(sh, x, wq, scales, biases, y, M, N, K, stream);
        case 3: return launch_bits_burst_w<3>(sh, x, wq, scales, biases, y, M, N, K, stream);
        case 4: return launch_bits_burst_w<4>(sh, x, wq, scales, biases, y, M, N, K, stream);
        case 8: return launch_bits_burst_w<8>(sh, x, wq, scales, biases, y, M, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

// four waves split K
hipError_t launch_qmv_bits(int bits, int mode, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                           const uint16_t* biases, uint16_t* y, int M, int N, int K, hipStream_t stream) {
    const bool rows = mode == kQmvBitsRows;
    switch (bits) {
        case 1: return rows ? launch_qmv_bits_t<1, 4, kRows>(x, wq, scales, biases, y, M, N, K, stream)
                            : launch_qmv_bits_t<1, 4, kMatrix>(x, wq, scales, biases, y, M, N, K, stream);
        case 2: return rows ? launch_qmv_bits_t<2, 4, kRows>(x, wq, scales, biases, y, M, N, K, stream)
                            : launch_qmv_bits_t<2, 4, kMatrix>(x, wq, scales, biases, y, M, N, K, stream);
        case 3: return rows ? launch_qmv_bits_t<3, 4, kRows>(x, wq, scales, biases, y, M, N, K, stream)
                            : launch_qmv_bits_t<3, 4, kMatrix>(x, wq, scales, biases, y, M, N, K, stream);
        case 4: return rows ? launch_qmv_bits_t<4, 4, kRows>(x, wq, scales, biases, y, M, N, K, stream)
                            : launch_qmv_bits_t<4, 4, kMatrix>(x, wq, scales, biases, y, M, N, K, stream);
        case 8: return rows ? launch_qmv_bits_t<8, 4, kRows>(x, wq, scales, biases, y, M, N, K, stream)
                            : launch_qmv_bits_t<8, 4, kMatrix>(x, wq, scales, biases, y, M, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
