// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, DPP row reductions and the internal launcher interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// bf16 values are stored as their 16-bit patterns.
typedef uint16_t bf16_bits;

// Widening a bfloat16 to float is a 16-bit shift: the bf16 is the upper half
// of the binary32 encoding.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats -> two packed bfloat16 (lo in bits 0..15), round to nearest even;
// a single v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
// Two floats -> two packed IEEE half floats (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2_t));
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Eight OCP E4M3 codes -> the eight fp16 values they encode, exactly (every
// E4M3 value, subnormals included, is an fp16 value; the NaN codes give NaN),
// with gfx950's conversion instruction, two codes per instruction.  The
// result words are taken whole: reading single halves of the builtin's
// vector result has been compiled into a copy of the low half.
__device__ __forceinline__ u32x4_t e4m3x8_to_f16(u32x2_t w) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false));
    r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true));
  }
  return r;
}

// ---------------------------------------------------------------------------
// DPP lane permutations inside a 16-lane row (gfx9 dpp_ctrl encodings).
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
  kDppRowRor8 = 0x128,       // row_ror:8  (lane i <- lane (i+8) mod 16)
  kDppRowMirror = 0x140,     // lane i <- lane 15-i
  kDppRowHalfMirror = 0x141  // lane i <- lane 7-i within each half row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Max / sum over the 16 lanes of a DPP row; every lane of the row gets the
// result (pairs see each other's values, so the result is identical in all).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Max over the four 16-lane rows for each lane position (lanes l, l^16, l^32,
// l^48), with gfx950's row-swap permutes: permlane32_swap(x, x) yields rows
// (0,1,0,1) and (2,3,2,3); permlane16_swap(y, y) yields (0,0,2,2) and
// (1,1,3,3).  Every lane of a column gets the same result.
__device__ __forceinline__ float max_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// gfx950's byte-transposing LDS read (ds_read_b64_tr_b8): within each 16-lane
// group, byte j of lane l's result is byte l % 8 of the 8 bytes addressed by
// lane 2 j + l / 8 of the group.  p must point into LDS, 8-byte aligned.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
__device__ __forceinline__ u32x2_t lds_read_tr8(const char* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)p));
}

// Wave-uniform copy of a value (held in a scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// exp2 on the hardware transcendental unit (v_exp_f32); exp(x) is evaluated
// as exp2(x * log2(e)) with the constant folded into the score scale.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// fp32 -> OCP FP8 E4M3 code (1 sign bit, 4 exponent bits with bias 7, 3
// mantissa bits, subnormals m/8 * 2^-6, no infinities, S.1111.111 = NaN):
// nearest, ties to even; magnitudes above 448 saturate to +-448; NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_from_f32(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a == a)) return 0x7Fu;
  if (a > 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);  // subnormal grid of 2^-9 (8 = smallest normal)
  const uint32_t ua = __float_as_uint(a);
  int e = (int)(ua >> 23) - 127;
  const uint32_t mant = ua & 0x7FFFFFu;
  uint32_t r = mant >> 20;
  const uint32_t rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  if (r == 8u) {
    r = 0u;
    ++e;
  }
  const uint32_t code = ((uint32_t)(e + 7) << 3) | r;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

}  // namespace pa
