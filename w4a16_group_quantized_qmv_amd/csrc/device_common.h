// Device helpers shared by the qmv and qmm kernels (gfx950 / CDNA4 only).
//
// Operand layouts of the two bf16 MFMA shapes used here (checked on the MI355X with an
// in-bounds probe):
//   v_mfma_f32_16x16x32_bf16 (qmv)
//     A (16 x 32):  lane l holds A[l % 16][8 * (l / 16) + e],  e = 0..7
//     B (32 x 16):  lane l holds B[8 * (l / 16) + e][l % 16]
//     D (16 x 16):  lane l, register r holds D[4 * (l / 16) + r][l % 16]
//   v_mfma_f32_32x32x16_bf16 (qmm; about twice the sustained rate of the 16x16x32 shape)
//     A (32 x 16):  lane l holds A[l % 32][8 * (l / 32) + e]
//     B (16 x 32):  lane l holds B[8 * (l / 32) + e][l % 32]
//     D (32 x 32):  lane l, register r holds D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// Any bijection between the MFMA's K index and real reduction indices is allowed as long as A
// and B use the same one; the kernels document theirs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;          // reduction values per scale/bias pair
constexpr int kWordsPerGroup = 16;   // 128 four-bit codes in sixteen 32-bit words

// Tile order of the tiled kernels (qmm and the int8 path).
constexpr int kBandM = 8;               // M-tiles per band of the tile order
constexpr int kBandM128 = 4;            // M-tiles per band for the 128-row W4A16 tiles

// Linear workgroup index -> work index such that XCD c (= i % 8) receives the contiguous range
// of work indices [start_c, start_c + count_c).
__device__ __forceinline__ int xcd_remap(int i, int total) {
    const int per = total >> 3, rem = total & 7;
    const int c = i & 7, k = i >> 3;
    return c * per + (c < rem ? c : rem) + k;
}

// Tile index -> (tm, tn): bands of up to BAND M-tiles, each band walked N-tile by N-tile.
template <int BAND = kBandM>
__device__ __forceinline__ void band_order(int tile, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int band = tile / (BAND * tiles_n);
    const int first = band * BAND;
    const int rows = min(BAND, tiles_m - first);
    const int in_band = tile - band * BAND * tiles_n;
    tm = first + in_band % rows;
    tn = in_band / rows;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (the hardware conversion, checked on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Four-bit codes as fp8 bytes.  Masking a packed word with 0x0F0F0F0F leaves the even codes
// q0, q2, q4, q6 one per byte; shifting right by 4 first gives q1, q3, q5, q7.  A byte 0..15
// read as OCP fp8 e4m3 is exactly q * 2^-9 (codes 0..7 are the subnormals m/8 * 2^-6, codes
// 8..15 are 1.mmm * 2^-6), so the scaled converters with scale 2^9 yield q itself, exactly.
__device__ __forceinline__ uint32_t even_codes(uint32_t w) { return w & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t odd_codes(uint32_t w) { return (w >> 4) & 0x0F0F0F0Fu; }

// Eight exact bf16 codes of one word in the order [q0, q2, q1, q3, q4, q6, q5, q7]
// (four instructions for eight values).  The matching activations come from
// permute_like_codes().
__device__ __forceinline__ bf16x8_t codes_bf16_permuted(uint32_t w) {
    const uint32_t ev = even_codes(w), od = odd_codes(w);
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, 512.0f, false);  // q0 q2
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, 512.0f, false);  // q1 q3
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ev, 512.0f, true);   // q4 q6
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(od, 512.0f, true);   // q5 q7
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight exact bf16 codes of one word in natural order [q0 .. q7]: the even / odd masks are
// interleaved back to bytes q0 q1 q2 q3 and q4 q5 q6 q7 (v_perm_b32), then converted two at a
// time (nine instructions for eight values).
__device__ __forceinline__ bf16x8_t codes_bf16_natural(uint32_t w) {
    const uint32_t ev = even_codes(w), od = odd_codes(w);
    const uint32_t lo = __builtin_amdgcn_perm(od, ev, 0x05010400u);   // q0 q1 q2 q3
    const uint32_t hi = __builtin_amdgcn_perm(od, ev, 0x07030602u);   // q4 q5 q6 q7
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false);  // q0 q1
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true);   // q2 q3
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false);  // q4 q5
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true);   // q6 q7
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight consecutive bf16 activations x0..x7 (as four dwords) reordered to
// [x0, x2, x1, x3, x4, x6, x5, x7], the order of codes_bf16_permuted().
__device__ __forceinline__ bf16x8_t permute_like_codes(const u32x4_t& v) {
    u32x4_t r;
    r[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);  // x0 x2
    r[1] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);  // x1 x3
    r[2] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);  // x4 x6
    r[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);  // x5 x7
    return __builtin_bit_cast(bf16x8_t, r);
}

// Dequantize one word to eight bf16 weights in natural order: w_i = bf16(fma(q_i, s, b)).
// s * q is exact in fp32, so the single fma rounding equals an fp32 multiply followed by an
// fp32 add; the result is then rounded once more to bf16 for the MFMA operand.
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w, float s, float b) {
    const uint32_t ev = even_codes(w), od = odd_codes(w);
    const f32x2_t e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, false);  // q0 q2
    const f32x2_t o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, false);  // q1 q3
    const f32x2_t e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, true);   // q4 q6
    const f32x2_t o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, true);   // q5 q7
    bf16x8_t r;
    r[0] = static_cast<__bf16>(__builtin_fmaf(e0[0], s, b));
    r[1] = static_cast<__bf16>(__builtin_fmaf(o0[0], s, b));
    r[2] = static_cast<__bf16>(__builtin_fmaf(e0[1], s, b));
    r[3] = static_cast<__bf16>(__builtin_fmaf(o0[1], s, b));
    r[4] = static_cast<__bf16>(__builtin_fmaf(e1[0], s, b));
    r[5] = static_cast<__bf16>(__builtin_fmaf(o1[0], s, b));
    r[6] = static_cast<__bf16>(__builtin_fmaf(e1[1], s, b));
    r[7] = static_cast<__bf16>(__builtin_fmaf(o1[1], s, b));
    return r;
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

}  // namespace w4a16
