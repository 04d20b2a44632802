// Device helpers shared by the libkda kernels (gfx950 / CDNA4).
//
// BF16 values live in memory as __bf16.  Conversions FP32 -> BF16 round to
// nearest even (gfx950 has a hardware instruction for the packed form).
//
// MFMA fragment convention used throughout.  A "frag" is a 16x16 FP32 tile
// in the accumulator layout of the 16x16 MFMA instructions: lane l = 16*gq + n
// holds rows 4*gq + i (i = 0..3) of column n.  A 16x16xK MFMA multiplies the
// A-register element i of lane (gq, m) with the B-register element i of lane
// (gq, n) and sums over gq and i; so the product X*Y is formed from
//   * the frag of X^T (lane (gq, m) holds X[m][4gq+i])   as the A operand, and
//   * the frag of Y   (lane (gq, n) holds Y[4gq+i][n])   as the B operand,
// and the contraction index may be renumbered freely as long as both operands
// agree.  The 16x16x32 form takes two such frags per operand (contraction
// blocks 2j and 2j+1) concatenated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;          // head dimension (K = V = 128)
constexpr int CH = 16;          // chunk length in tokens
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }

// 1/sqrt(x) (hardware approximation, ~1 ulp).
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// sigmoid(x) = 1 / (1 + exp(-x)), saturating cleanly at both ends.
__device__ __forceinline__ float sigmoidf_(float x) {
    return __builtin_amdgcn_rcpf(1.0f + fast_exp(-x));
}

// --- MFMA wrappers -------------------------------------------------------
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// FP32 -> BF16, round to nearest even.  Converted pair by pair through a
// 32-bit word: the compiler lowers a 4-wide vector truncation element by
// element in some contexts (one conversion per element plus a repack),
// while each pair here becomes one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned cvt_pk_bf16(float a, float b) {  // a in the low half
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ bf16x4 to_bf4(f32x4 x) {
    return __builtin_bit_cast(bf16x4, u32x2{cvt_pk_bf16(x[0], x[1]), cvt_pk_bf16(x[2], x[3])});
}
// BF16 of -x: the sign flipped on the packed result (one integer op per pair).
__device__ __forceinline__ bf16x4 to_bf4_neg(f32x4 x) {
    return __builtin_bit_cast(bf16x4, u32x2{cvt_pk_bf16(x[0], x[1]) ^ 0x80008000u,
                                            cvt_pk_bf16(x[2], x[3]) ^ 0x80008000u});
}
__device__ __forceinline__ f32x4 from_bf4(bf16x4 x) {
    return __builtin_convertvector(x, f32x4);
}
// FP32 x ~= hi + lo as a BF16 pair: hi keeps the top 16 bits of x (sign,
// exponent, 7 mantissa bits; truncated), lo = bf16(x - hi) where x - hi is
// exact.  The pair carries about 16 significant bits, so hi*hi' + hi*lo' +
// lo*hi' reproduces an FP32 product to ~2^-16 relative.
__device__ __forceinline__ void split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 u = __builtin_bit_cast(u32x4, x) & 0xffff0000u;
    const f32x4 h = __builtin_bit_cast(f32x4, u);
    // upper halves of (u0, u1) and (u2, u3) packed as bf16 pairs
    const u32x2 hp = {__builtin_amdgcn_perm(u[1], u[0], 0x07060302u),
                      __builtin_amdgcn_perm(u[3], u[2], 0x07060302u)};
    hi = __builtin_bit_cast(bf16x4, hp);
    lo = to_bf4(x - h);
}

// FP16 pairs.  FP16 keeps 11 significant bits (BF16 8) in a narrower range
// (|x| < 65504; below 6.1e-5 it loses bits, below 6e-8 it is zero), so it
// serves operands whose magnitude is bounded and whose small values do not
// matter.  hi = f16(x), lo = f16(x - hi) carry about 22 bits.
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x4 to_f16x4(f32x4 x) {  // round to nearest even, pair by pair
    const f16x2 a = __builtin_convertvector(f32x2{x[0], x[1]}, f16x2);
    const f16x2 b = __builtin_convertvector(f32x2{x[2], x[3]}, f16x2);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3);
}
__device__ __forceinline__ void split4_f16(f32x4 x, f16x4& hi, f16x4& lo) {
    hi = to_f16x4(x);
    lo = to_f16x4(x - __builtin_convertvector(hi, f32x4));
}
__device__ __forceinline__ f16x8 cat8h(f16x4 a, f16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 mma32h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The same pair with hi rounded to nearest (unbiased, so that hi may also
// serve alone as the operand's BF16 value): hi = bf16(x), lo = bf16(x - hi),
// where x - hi is exact.
__device__ __forceinline__ void split4_rne(f32x4 x, bf16x4& hi, bf16x4& lo) {
    hi = to_bf4(x);
    lo = to_bf4(x - from_bf4(hi));
}

// base + off elements with the byte offset formed in 32 bits, so that the
// access can use a scalar base and a 32-bit vector offset instead of 64-bit
// per-lane address arithmetic (off * sizeof(T) must stay below 2^32).
template <class T>
__device__ __forceinline__ T* at(T* base, unsigned off) {
    typedef typename std::conditional<std::is_const<T>::value, const char, char>::type C;
    return reinterpret_cast<T*>(reinterpret_cast<C*>(base) + off * (unsigned)sizeof(T));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// The 16x16 identity as an MFMA operand: lane (gq, n) holds I[4gq+i][n].
__device__ __forceinline__ bf16x4 identity_frag(int lane) {
    const int gq = lane >> 4, cl = lane & 15;
    f32x4 id;
#pragma unroll
    for (int i = 0; i < 4; ++i) id[i] = (4 * gq + i == cl) ? 1.0f : 0.0f;
    return to_bf4(id);
}
// Exact transpose of a BF16 frag through the matrix unit: if lane (gq, m)
// holds X[m][4gq+i], the result's lane (gq, n) holds X[4gq+i][n].
__device__ __forceinline__ f32x4 transpose_frag(bf16x4 x, bf16x4 ident) {
    return mma16(x, ident, zero4());
}

// Sum over each row of 16 lanes, broadcast to the row, with DPP lane swaps
// (xor 1, xor 2 inside quads, then mirrors of 8 and 16 lanes).  Every lane has
// a source in these patterns, so bound_ctrl changes nothing here; set, it lets
// the compiler fold each swap into its add (v_add_f32_dpp).
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
    return x;
}

// Sum over groups of `W` consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < W; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

}  // namespace kda
