// kda_mfma_common.h -- gfx950 matrix-core helpers shared by the bf16 kernels
// (vector types, MFMA wrappers, bf16 hi/lo splits, in-row lane operations,
// state load/store). Device code only; not part of the public ABI.
//
// Matrix-core instruction layouts relied on (64 lanes, lane l, g = l/16):
//   16x16x32 bf16: A lane l = row l%16, 8 k values; B lane l = column l%16,
//                  the same 8 k labels; D lane l = rows 4g..4g+3, column l%16.
//   16x16x16 bf16: as above with 4 k values (k = 4g..4g+3 matches D's rows).
//   16x16x4  f32 : A lane l = row l%16, k = g; B lane l = column l%16, k = g.
#pragma once

#include "kda_internal.h"

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A product that accumulates onto the result of the product just before it must have
// that product's shape (16x16x32 after 16x16x32, 16x16x16 after 16x16x16). Measured on
// gfx950: when a 16x16x16 bf16 product takes as its accumulator the result of a 16x16x32
// one (or the reverse) fewer than about five wait states later, half of its accumulator
// elements are read before that result is written, so the earlier product is lost there.
// ROCm 7.2.0's compiler (AMD clang 22, roc-7.2.0) inserts no wait states between the two.
// Split-bf16 products therefore add their lo terms with a second 16x16x32 product,
// [x_hi | x_lo] x [y_lo ; y_lo], never with a 16x16x16 one on the same accumulator.
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                      0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// x = hi + lo with hi, lo bf16: about 16 significant bits between them.
__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        __bf16 h = (__bf16)x[r];
        hi[r] = h;
        lo[r] = (__bf16)(x[r] - (float)h);
    }
}

// x = hi + lo with hi = x truncated to bf16 (its top 16 bits) and lo = x - hi (exact
// in fp32) rounded to bf16: about 16 significant bits, one op per element cheaper
__device__ __forceinline__ void split4t(f32x4 x, bf16x4 &hi, bf16x4 &lo)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t u = __float_as_uint(x[r]);
        hi[r] = __builtin_bit_cast(__bf16, (uint16_t)(u >> 16));
        lo[r] = (__bf16)(x[r] - __uint_as_float(u & 0xffff0000u));
    }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two values rounded to bf16 (ties to even) as one packed word, x[0] in the low half
__device__ __forceinline__ uint32_t pk_bf16(f32x2 x)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// truncating split of four values into packed bf16 pairs: hi = {x0|x1, x2|x3} (top 16
// bits, one byte permute per pair), lo = the exact fp32 remainders, rounded pairwise
__device__ __forceinline__ void split4t_packed(f32x4 x, bf16x4 &hi, bf16x4 &lo)
{
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    const u32x2 h = {__builtin_amdgcn_perm(u[1], u[0], 0x07060302u), __builtin_amdgcn_perm(u[3], u[2], 0x07060302u)};
    const f32x2 r01 = {x[0] - __uint_as_float(u[0] & 0xffff0000u), x[1] - __uint_as_float(u[1] & 0xffff0000u)};
    const f32x2 r23 = {x[2] - __uint_as_float(u[2] & 0xffff0000u), x[3] - __uint_as_float(u[3] & 0xffff0000u)};
    // each remainder pair is converted and kept as one packed word (one conversion per pair)
    const u32x2 l = {pk_bf16(r01), pk_bf16(r23)};
    hi = __builtin_bit_cast(bf16x4, h);
    lo = __builtin_bit_cast(bf16x4, l);
}

// {hi[0..3], lo[0..3]} with x = hi + lo: one 16x16x32 A operand that carries
// both halves of a split 16x16 tile (its first half alone is the hi tile)
__device__ __forceinline__ bf16x8 split8(f32x4 x)
{
    bf16x4 h, l;
    split4(x, h, l);
    return bf16x8{h[0], h[1], h[2], h[3], l[0], l[1], l[2], l[3]};
}

// each element rounded to the nearest bf16 (ties to even), kept as fp32
__device__ __forceinline__ f32x4 round_bf16x4(f32x4 x)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (float)(__bf16)x[r];
    return x;
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b)
{
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// logistic sigmoid from 2^x and a reciprocal
__device__ __forceinline__ float sigmoid_fast(float x)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// value of lane n of the caller's 16-lane row (DPP row_newbcast: no LDS round trip)
template <int N> __device__ __forceinline__ float row_bcast(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xf, 0xf, false));
}

// value of lane (l - n) of the same 16-lane row, 0 for lanes below n
template <int N> __device__ __forceinline__ float row_shr(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}

// C = X Y for 16x16 fp32 tiles; xt holds X^T and y holds Y, both in D layout.
__device__ __forceinline__ f32x4 mm16_f32(f32x4 xt, f32x4 y)
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mma4(xt[s], y[s], acc);
    return acc;
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
// C = X Y for 16x16 tiles with fp16 operands and fp32 accumulation; xt holds X^T and
// y holds Y in D layout (the 16x16x16 operand layout of both)
__device__ __forceinline__ f32x4 mm16_h(f32x4 xt, f32x4 y)
{
    const f16x4 a = {(_Float16)xt[0], (_Float16)xt[1], (_Float16)xt[2], (_Float16)xt[3]};
    const f16x4 b = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, z, 0, 0, 0);
}

// I + a*X in D layout (row 4g+r, column tok)
__device__ __forceinline__ f32x4 eye_plus(f32x4 x, float a, int g, int tok)
{
    f32x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = a * x[r] + ((4 * g + r == tok) ? 1.f : 0.f);
    return y;
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void bar_sync() { asm volatile("s_barrier" ::: "memory"); }

template <typename TSt>
__device__ __forceinline__ f32x4 ld_state4(const TSt *p);
template <> __device__ __forceinline__ f32x4 ld_state4<float>(const float *p)
{
    return *reinterpret_cast<const f32x4 *>(p);
}
template <> __device__ __forceinline__ f32x4 ld_state4<uint16_t>(const uint16_t *p)
{
    const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
    f32x4 y = {bf_lo(x[0]), bf_hi(x[0]), bf_lo(x[1]), bf_hi(x[1])};
    return y;
}
template <typename TSt>
__device__ __forceinline__ void st_state4(TSt *p, f32x4 x);
template <> __device__ __forceinline__ void st_state4<float>(float *p, f32x4 x)
{
    *reinterpret_cast<f32x4 *>(p) = x;
}
template <> __device__ __forceinline__ void st_state4<uint16_t>(uint16_t *p, f32x4 x)
{
    u32x2 y;
    y[0] = (uint32_t)f32_to_bf16_bits(x[0]) | ((uint32_t)f32_to_bf16_bits(x[1]) << 16);
    y[1] = (uint32_t)f32_to_bf16_bits(x[2]) | ((uint32_t)f32_to_bf16_bits(x[3]) << 16);
    *reinterpret_cast<u32x2 *>(p) = y;
}

}  // namespace kda
