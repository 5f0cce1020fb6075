// W4A8: the same 4-bit affine group-quantized weights, with int8 activations on the int8
// matrix cores.
//
// "Feature Request: Metal prefill speedup (~68%) on M5 Max (NAX / tensor API kernels)" lists,
// in its feature list and Related work, an int8 mat-mat for large batches (after oMLX's int8
// prefill) and gives no recipe.  The reading taken here: each activation row is quantized
// symmetrically to int8 with one fp32 scale (a = max |x|, inv = 127 / a, sx = a / 127,
// xq = clamp(rint(x * inv), -127, 127), all in fp32), and the projection uses sx * xq in place
// of x, with the weights exactly as in the W4A16 path (w = s * q + b per 128-value group).
//
// Because the codes q are integers, the affine group factorizes:
//     y[m, n] = sx[m] * ( sum_g s[n, g] * P[m, n, g]  +  sum_g b[n, g] * X[m, g] ),
//     P[m, n, g] = sum_{k in g} xq[m, k] * q[n, k]      (exact int32 on v_mfma_i32_32x32x32_i8)
//     X[m, g]    = sum_{k in g} xq[m, k]                  (exact integer, made by the quantizer)
// so no weight is ever dequantized: the matrix core multiplies raw codes, each group's int32
// result is scaled once in fp32 (one convert and one fma per accumulator element per group),
// and the bias term is one small bf16 MFMA contraction over the groups at the end of the tile
// (X split into two bf16-exact halves, so it is exact).
//
// Layouts made by w4a8_quantize_rows (the operand order of the int8 kernel):
//   xq   int8 [M, K]: each aligned run of 8 values is stored as [x0 x2 x4 x6 x1 x3 x5 x7], the
//        byte order in which a packed code word's nibbles come out of the even / odd masks
//   sx   fp32 [M]
//   xsum bf16 [M, KB], KB = 2G rounded up to a multiple of 16: xsum[m, 2g] + xsum[m, 2g + 1]
//        = X[m, g] exactly (hi = X - (X & 127), lo = X & 127), zero beyond 2G.
#include "device_common.h"
#include "internal.h"

#include <type_traits>

namespace w4a16 {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------------------ quantizer

// One workgroup per row: absmax reduction, then codes, group sums and the scale.  Every lane
// takes 8-value chunks c = tid, tid + 256, ...; the 16 chunks of one group sit in 16
// consecutive lanes of one wave, which sum their codes with xor shuffles.
__global__ __launch_bounds__(256) void quantize_rows_int8_kernel(const uint16_t* __restrict__ x,
                                                                 int8_t* __restrict__ xq, float* __restrict__ sx,
                                                                 uint16_t* __restrict__ xsum, int K, int KB) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const int chunks = K >> 3;
    const uint16_t* xr = x + static_cast<size_t>(m) * K;

    float a = 0.f;
    for (int c = tid; c < chunks; c += 256) {
        const u32x4_t v = load16(xr + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a = fmaxf(a, fabsf(__uint_as_float(v[i] << 16)));
            a = fmaxf(a, fabsf(__uint_as_float(v[i] & 0xFFFF0000u)));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    // correctly rounded fp32 divisions (the compiler's default for hipcc)
    const float inv = a > 0.f ? 127.f / a : 0.f;
    if (tid == 0) sx[m] = a / 127.f;

    const int iters = (chunks + 255) >> 8;
    for (int it = 0; it < iters; ++it) {
        const int c = tid + 256 * it;
        const bool valid = c < chunks;     // uniform over each 16-lane group (chunks % 16 == 0)
        int codes[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (valid) {
            const u32x4_t v = load16(xr + 8 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
                // the product is rounded to fp32 first, then to the nearest integer (ties to even)
                const float plo = lo * inv, phi = hi * inv;
                codes[2 * i] = static_cast<int>(fminf(fmaxf(__builtin_rintf(plo), -127.f), 127.f));
                codes[2 * i + 1] = static_cast<int>(fminf(fmaxf(__builtin_rintf(phi), -127.f), 127.f));
            }
            // [x0 x2 x4 x6 | x1 x3 x5 x7]
            const uint32_t even = (codes[0] & 0xFF) | ((codes[2] & 0xFF) << 8) | ((codes[4] & 0xFF) << 16) |
                                  (static_cast<uint32_t>(codes[6] & 0xFF) << 24);
            const uint32_t odd = (codes[1] & 0xFF) | ((codes[3] & 0xFF) << 8) | ((codes[5] & 0xFF) << 16) |
                                 (static_cast<uint32_t>(codes[7] & 0xFF) << 24);
            uint32_t* dst = reinterpret_cast<uint32_t*>(xq + static_cast<size_t>(m) * K + 8 * c);
            dst[0] = even;
            dst[1] = odd;
        }
        int s = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += codes[i];
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
        if (valid && (tid & 15) == 0) {
            const int g = c >> 4;
            const int lo = s & 127, hi = s - lo;   // both exact in bf16 (|hi| <= 2^14, 8 bits)
            xsum[static_cast<size_t>(m) * KB + 2 * g] = f32_to_bf16_bits(static_cast<float>(hi));
            xsum[static_cast<size_t>(m) * KB + 2 * g + 1] = f32_to_bf16_bits(static_cast<float>(lo));
        }
    }
    for (int k = 2 * (K >> 7) + tid; k < KB; k += 256) xsum[static_cast<size_t>(m) * KB + k] = 0;
}

// ------------------------------------------------------------------------------ int8 tile kernel

// Workgroup tile BM x 128 with four waves; each wave owns one 32-column block for all BM rows.
// One pipeline step is one 128-value group: four v_mfma_i32_32x32x32_i8 sub-steps per 32-row
// block produce the group's exact int32 P, which is scaled into the fp32 accumulators while the
// next group's MFMAs run.
//
// K mapping inside a group: lane half h of a wave holds words 8h .. 8h + 7 of its column's
// group; sub-step t takes words 8h + 2t and 8h + 2t + 1, whose even / odd nibble masks give the
// 16 codes [q0 q2 q4 q6 q1 q3 q5 q7 | ...] of values 64h + 16t .. 64h + 16t + 15, the order in
// which xq stores them.  So the activation operand of (h, t) is the 16-byte chunk 4h + t of the
// row's group.
//
// Activations are staged by direct global-to-LDS loads into unpadded 128-byte rows (one wave
// instruction writes 8 rows); chunk c of tile row r sits at slot c ^ ((r >> 1) & 7), so 16
// lanes reading one chunk of 16 consecutive rows hit 16 different 16-byte bank groups.
// KS = 2: two waves per column block, one taking sub-steps 0-1 and the other 2-3 of every group;
// their partial sums are added through the activation stages at the end.
template <int BM, int WAVES_PER_SIMD, int KS = 1>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD, WAVES_PER_SIMD))) void
qmm_w4a8_kernel(const int8_t* __restrict__ xq, const float* __restrict__ sx, const uint16_t* __restrict__ xsum,
                const uint32_t* __restrict__ wq, const uint16_t* __restrict__ scales,
                const uint16_t* __restrict__ biases, uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N,
                int K, int KB, int split, int tiles_m, int tiles_n) {
    constexpr int WN = 4;                           // waves across the tile's columns
    constexpr int NW = WN * KS;
    constexpr int TSUB = 4 / KS;                    // int8 MFMA sub-steps per group and wave
    constexpr int BN = WN * 32;
    constexpr int RB = BM / 32;
    constexpr int TILE = BM * kGroup;               // bytes of one staged activation tile
    constexpr int DMA_PER_WAVE = BM / (8 * NW);     // 1 KB direct loads per wave per group
    static_assert(BM % 32 == 0 && DMA_PER_WAVE >= 1, "tile shape");
    __shared__ __attribute__((aligned(16))) int8_t xs0[TILE];
    __shared__ __attribute__((aligned(16))) int8_t xs1[TILE];
    // codes of one group, per stage: each wave's 32 columns x 64 bytes
    __shared__ __attribute__((aligned(16))) uint8_t cs0[WN * 2048];
    __shared__ __attribute__((aligned(16))) uint8_t cs1[WN * 2048];

    const int tiles = tiles_m * tiles_n;
    const int work = xcd_remap(blockIdx.x, tiles * split);
    const int z = work / tiles;
    int tm, tn;
    // 128-row tiles walk bands of 4 M-tiles, like the W4A16 tiles (measured at 4096 rows: down
    // 0.8% faster, gate unchanged, outputs bit-identical)
    band_order<(BM >= 128 ? kBandM128 : kBandM)>(work - z * tiles, tiles_m, tiles_n, tm, tn);

    const int G = K >> 7;
    const int row_bytes = K >> 1;
    const int g_begin = static_cast<int>(static_cast<int64_t>(z) * G / split);
    const int g_end = static_cast<int>(static_cast<int64_t>(z + 1) * G / split);
    const int groups = g_end - g_begin;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kh = wave / WN, wn = wave % WN;      // K half (KS = 2) and column block
    const int half = lane >> 5;
    auto clamp_records = [](int64_t bytes) { return static_cast<int>(bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes); };

    // Activations: instruction i of wave w fills tile rows 8 (i NW + w) + 0..7; lane l writes slot
    // l % 8 of row l / 8 with chunk (l % 8) ^ ((row >> 1) & 7).  With NW = 4 that row term is
    // (4 (w & 1) + l / 16) & 7 for every i.
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(xq + static_cast<size_t>(m0) * K), 0, clamp_records(static_cast<int64_t>(M - m0) * K),
        0x00020000);
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(xq), 0, 0, 0x00020000);
    const int xrow0 = 8 * wave + (lane >> 3);
    const uint32_t xvoff = static_cast<uint32_t>(xrow0 * K + (((lane & 7) ^ ((xrow0 >> 1) & 7)) << 4));
    const int64_t cols_left = static_cast<int64_t>(N - n0);
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(wq) + static_cast<size_t>(n0) * row_bytes), 0,
        clamp_records(cols_left * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(scales + static_cast<size_t>(n0) * G), 0, clamp_records(cols_left * G * 2), 0x00020000);
    const int col = wn * 32 + (lane & 31);             // column within the tile
    const uint32_t svoff = static_cast<uint32_t>(col * G * 2);
    // Codes go through LDS by direct loads that read whole 64-byte column groups (the layout of
    // the W4A16 tile kernel): instruction i fills columns 16 i + l / 4, lane l writing its 16
    // bytes to slot l % 4 of the column's 64, slot p holding chunk p ^ ((column / 4) & 3).
    const uint32_t cvoff = static_cast<uint32_t>((wn * 32 + (lane >> 2)) * row_bytes +
                                                 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
    const int ccol = lane & 31;
    const int cread0 = ccol * 64 + 16 * ((2 * half) ^ ((ccol >> 2) & 3));
    const int cread1 = ccol * 64 + 16 * ((2 * half + 1) ^ ((ccol >> 2) & 3));

    struct Slot {
        uint16_t s;
    };
    auto stage = [&](auto ic) -> int8_t* {
        if constexpr (decltype(ic)::value == 0) return xs0;
        else return xs1;
    };
    auto cstage = [&](auto ic) -> uint8_t* {
        if constexpr (decltype(ic)::value == 0) return cs0 + wn * 2048;
        else return cs1 + wn * 2048;
    };
    auto issue = [&](int j, auto ic, Slot& o) {
        const bool live = j >= 0 && j < groups;
        const int g = g_begin + (live ? j : 0);
        const __amdgpu_buffer_rsrc_t xr = live ? xrsrc : none;
        int8_t* xt = stage(ic);
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; ++i) {
            int8_t* dst = xt + __builtin_amdgcn_readfirstlane(8 * (i * NW + wave) * kGroup);
            const uint32_t voff = xvoff + static_cast<uint32_t>(i) * (8 * NW) * static_cast<uint32_t>(K);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, voff, static_cast<uint32_t>(g) * kGroup, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t wr = live ? wrsrc : none;
        const __amdgpu_buffer_rsrc_t sr = live ? srsrc : none;
        uint8_t* cdst = cstage(ic);
        const uint32_t cg = static_cast<uint32_t>(g) * 64u;
        if constexpr (KS == 1) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, cdst, 16, cvoff, cg, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, cdst + 1024, 16, cvoff + 16u * static_cast<uint32_t>(row_bytes),
                                                     cg, 0, 0);
        } else {   // the two waves of a column block load one half of its columns each
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, cdst + __builtin_amdgcn_readfirstlane(kh * 1024), 16,
                                                     cvoff + 16u * static_cast<uint32_t>(kh) * static_cast<uint32_t>(row_bytes),
                                                     cg, 0, 0);
        }
        asm volatile("" ::: "memory");
        o.s = __builtin_amdgcn_raw_buffer_load_b16(sr, svoff, g * 2, 0);
        asm volatile("" ::: "memory");
    };

    // LDS byte offset of the A operand of sub-step t for this lane (row block 0): row
    // r = lane % 32, chunk 4 * half + t at slot (4 * half + t) ^ ((r >> 1) & 7).
    const int arow = lane & 31;
    const int asw = (arow >> 1) & 7;
    // (KS = 2: this wave's sub-step tt is t = 2 kh + tt)
    auto a_off = [&](int tt) { return arow * kGroup + ((((half << 2) | (TSUB * kh + tt)) ^ asw) << 4); };

    f32x16_t acc[RB];
    i32x16_t P0[RB], P1[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[rb][r] = 0.f;
            P0[rb][r] = 0;
            P1[rb][r] = 0;
        }
    float s_last = 0.f;

    // One group: four int8 MFMA sub-steps into Pc, with the fp32 scaling of the previous group's
    // Pp (scale s_last) spread between them.
    auto compute = [&](auto ic, const Slot& o, i32x16_t (&Pc)[RB], const i32x16_t (&Pp)[RB]) {
        const int8_t* xt = stage(ic);
        // this lane's eight code words (words 8 half .. 8 half + 7 of its column's group)
        const uint8_t* cb = cstage(ic);
        u32x4_t ow[2];
        if constexpr (KS == 1) {
            ow[0] = *reinterpret_cast<const u32x4_t*>(cb + cread0);
            ow[1] = *reinterpret_cast<const u32x4_t*>(cb + cread1);
        } else {   // sub-steps 2 kh, 2 kh + 1 use chunk kh
            ow[0] = *reinterpret_cast<const u32x4_t*>(cb + (kh ? cread1 : cread0));
            ow[1] = ow[0];
        }
        i32x4_t a[2][RB];
        i32x4_t bq[2];
        auto codes = [&](int t) {
            const uint32_t w0 = ow[t >> 1][(t & 1) * 2], w1 = ow[t >> 1][(t & 1) * 2 + 1];
            return i32x4_t{static_cast<int>(even_codes(w0)), static_cast<int>(odd_codes(w0)),
                           static_cast<int>(even_codes(w1)), static_cast<int>(odd_codes(w1))};
        };
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            a[0][rb] = *reinterpret_cast<const i32x4_t*>(xt + a_off(0) + rb * 32 * kGroup);
        bq[0] = codes(0);
        const float sp = s_last;
#pragma unroll
        for (int t = 0; t < TSUB; ++t) {
            const int cur = t & 1, nxt = cur ^ 1;
            if (t < TSUB - 1) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    a[nxt][rb] = *reinterpret_cast<const i32x4_t*>(xt + a_off(t + 1) + rb * 32 * kGroup);
                bq[nxt] = codes(t + 1);
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const i32x16_t zero = {};
                Pc[rb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[cur][rb], bq[cur], t == 0 ? zero : Pc[rb], 0, 0, 0);
            }
            // a quarter of the previous group's scaling per sub-step
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 4 * KS * t; r < 4 * KS * (t + 1); ++r)
                    acc[rb][r] = __builtin_fmaf(sp, static_cast<float>(Pp[rb][r]), acc[rb][r]);
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 14, 0);  // VALU
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        s_last = bf16_bits_to_f32(o.s);
    };

    // Two-stage pipeline (the structure of the W4A16 tile kernel): position P loads group t + 1
    // into stage P % 2 and computes group t from the other stage; the fill positions (t < 0)
    // only load, and the position count is even so the loop exits only at the end of its body.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    Slot slot0, slot1;
    const int pad = (2 - (groups + 1) % 2) % 2;
    int t = -1 - pad;
    asm volatile("" : "+s"(t));
    if (groups > 0) {
        for (;;) {
            if (t >= 0) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            issue(t + 1, I0{}, slot0);
            if (t >= 0) compute(I1{}, slot1, P1, P0);
            ++t;
            if (t >= 0) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            issue(t + 1, I1{}, slot1);
            if (t >= 0) compute(I0{}, slot0, P0, P1);
            ++t;
            if (t >= groups) break;
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no direct load may outlive the wave
    // the last group computed sits in P0 (the position count is even)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][r] = __builtin_fmaf(s_last, static_cast<float>(P0[rb][r]), acc[rb][r]);

    // Bias term, once per output (slice 0, K half 0): acc += xsum . baug^T over KB / 16 bf16
    // sub-steps, with baug[n, k'] = b[n, k' / 2] (zero for k' / 2 >= G) against xsum's hi / lo
    // halves.
    if (z == 0 && kh == 0) {
        const __amdgpu_buffer_rsrc_t xsr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(xsum + static_cast<size_t>(m0) * KB), 0,
            clamp_records(static_cast<int64_t>(M - m0) * KB * 2), 0x00020000);
        const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(biases + static_cast<size_t>(n0) * G), 0, clamp_records(cols_left * G * 2),
            0x00020000);
        for (int u = 0; u < KB / 16; ++u) {
            const int g0 = 8 * u + 4 * half;
            uint16_t bb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t off = svoff + static_cast<uint32_t>(g0 + i < G ? g0 + i : 0) * 2u;
                const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(brsrc, off, 0, 0);
                bb[i] = g0 + i < G ? v : static_cast<uint16_t>(0);
            }
            const bf16x8_t bfrag = __builtin_bit_cast(
                bf16x8_t, u32x4_t{bb[0] | (static_cast<uint32_t>(bb[0]) << 16), bb[1] | (static_cast<uint32_t>(bb[1]) << 16),
                                  bb[2] | (static_cast<uint32_t>(bb[2]) << 16), bb[3] | (static_cast<uint32_t>(bb[3]) << 16)});
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const uint32_t off = static_cast<uint32_t>(((rb * 32 + arow) * KB + 16 * u + 8 * half) * 2);
                const bf16x8_t afrag =
                    __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(xsr, off, 0, 0));
                acc[rb] = mfma32x32x16(afrag, bfrag, acc[rb]);
            }
        }
    }

    // KS = 2: the two waves of a column block add their partial sums; K half 0 finishes the
    // elements e = 16 rb + r < 8 RB, K half 1 the rest.  Each writes the elements it hands over to
    // the activation and code stages of its own K half (first and second half of them) and reads
    // its partner's.
    if constexpr (KS == 2) {
        __syncthreads();   // every wave is done with the stages
        constexpr int HALF = RB * 8;
        constexpr int CH = HALF / 2;
        static_assert(WN * CH * 64 * 4 <= TILE && WN * CH * 64 * 4 <= WN * 2048, "partial sums fit the stages");
        float* mine0 = reinterpret_cast<float*>(kh == 0 ? xs0 : xs1) + wn * CH * 64;
        float* mine1 = reinterpret_cast<float*>(kh == 0 ? cs0 : cs1) + wn * CH * 64;
        const float* theirs0 = reinterpret_cast<const float*>(kh == 0 ? xs1 : xs0) + wn * CH * 64;
        const float* theirs1 = reinterpret_cast<const float*>(kh == 0 ? cs1 : cs0) + wn * CH * 64;
        // element indices stay compile-time constants (a runtime index would move acc to scratch);
        // the barrier between handing over and adding sits outside the K-half branches, so every
        // wave of the workgroup reaches the same one
        auto hand_over = [&](auto khc) {
            constexpr int give = decltype(khc)::value == 0 ? HALF : 0;
#pragma unroll
            for (int e = 0; e < HALF; ++e) {
                float* dst = e < CH ? mine0 : mine1;
                dst[(e % CH) * 64 + lane] = acc[(e + give) >> 4][(e + give) & 15];
            }
        };
        auto add_partner = [&](auto khc) {
            constexpr int keep = decltype(khc)::value == 0 ? 0 : HALF;
#pragma unroll
            for (int e = 0; e < HALF; ++e) {
                const float* src = e < CH ? theirs0 : theirs1;
                acc[(e + keep) >> 4][(e + keep) & 15] += src[(e % CH) * 64 + lane];
            }
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

    // epilogue: y = sx[m] * acc; D layout puts rows 8 (r / 4) + 4 half + r % 4 of column
    // lane % 32 in this lane
    const int n = n0 + col;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (KS == 2) {
                if ((16 * rb + r < RB * 8) != (kh == 0)) continue;
            }
            const int m = m0 + rb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (m >= M || n >= N) continue;
            const float v = sx[m] * acc[rb][r];
            const size_t idx = static_cast<size_t>(m) * N + n;
            if (split == 1)
                y[idx] = f32_to_bf16_bits(v);
            else
                ws[static_cast<size_t>(z) * M * N + idx] = v;
        }
    }
}

const QmmShape kW4A8Variants[kNumW4A8Variants] = {
    {32, 1, 4, 2},    // 0:  32 x 128 tile, four waves per SIMD
    {64, 1, 4, 2},    // 1:  64 x 128 tile, three waves per SIMD
    {128, 1, 4, 2},   // 2: 128 x 128 tile, two waves per SIMD
    {64, 1, 8, 2, 2},  // 3:  64 x 128 tile, 8 waves: two per column block splitting each group
};

hipError_t launch_quantize_rows_int8(const uint16_t* x, int8_t* xq, float* sx, uint16_t* xsum, int M, int K, int KB,
                                     hipStream_t stream) {
    hipLaunchKernelGGL(quantize_rows_int8_kernel, dim3(M), dim3(256), 0, stream, x, xq, sx, xsum, K, KB);
    return hipGetLastError();
}

template <int BM, int WPS, int KS = 1>
static hipError_t launch_w4a8_t(const int8_t* xq, const float* sx, const uint16_t* xsum, const uint32_t* wq,
                                const uint16_t* s, const uint16_t* b, uint16_t* y, float* ws, int M, int N, int K,
                                int KB, int split, hipStream_t stream) {
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + 127) / 128;
    W4A16_LAUNCH((qmm_w4a8_kernel<BM, WPS, KS>), dim3(tiles_m * tiles_n * split), dim3(256 * KS), 0, stream,
                       xq, sx, xsum, wq, s, b, y, ws, M, N, K, KB, split, tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_qmm_w4a8(int variant, const int8_t* xq, const float* sx, const uint16_t* xsum, const uint32_t* wq,
                           const uint16_t* scales, const uint16_t* biases, uint16_t* y, float* ws, int M, int N,
                           int K, int KB, int split, hipStream_t stream) {
    switch (variant) {
        case 0: return launch_w4a8_t<32, 4>(xq, sx, xsum, wq, scales, biases, y, ws, M, N, K, KB, split, stream);
        case 1: return launch_w4a8_t<64, 3>(xq, sx, xsum, wq, scales, biases, y, ws, M, N, K, KB, split, stream);
        case 2: return launch_w4a8_t<128, 2>(xq, sx, xsum, wq, scales, biases, y, ws, M, N, K, KB, split, stream);
        case 3: return launch_w4a8_t<64, 4, 2>(xq, sx, xsum, wq, scales, biases, y, ws, M, N, K, KB, split, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
