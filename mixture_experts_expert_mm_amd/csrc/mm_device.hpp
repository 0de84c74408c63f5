// Device helpers for gfx950 (CDNA4): vector types, MFMA wrappers, number
// format conversions and wavefront primitives.  Wave size is 64.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// UC_MX8: MX-FP8, e4m3 activations and weights with E8M0 scales per 32
// K-values; UC_MX4: MX-FP8 activations x MX-FP4 (e2m1) weights.
enum Usecase : int { UC_BF16 = 0, UC_FP8 = 1, UC_I8 = 2, UC_MX8 = 3, UC_MX4 = 4 };
constexpr bool is_mx(int uc) { return uc == UC_MX8 || uc == UC_MX4; }
constexpr int kMxGroup = 32;   // K-values per E8M0 scale

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// two round-to-nearest-even conversions in one v_cvt_pk_bf16_f32: lo in
// bits 0-15, hi in bits 16-31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// OCP e4m3fn, saturating to +-448, round-to-nearest-even.  The hardware
// conversion rounds to nearest even; the clamp makes the saturation explicit.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// symmetric int8: round half to even, clamp to [-127, 127]
__device__ __forceinline__ int32_t f32_to_i8sym(float v) {
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int32_t)r;
}

__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// ---------------------------------------------------------------------------
// wavefront primitives
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// MFMA: one 32x32 output block, one K-step.  Each lane supplies 16 bytes
// (bf16 x8, int8 x16) or 32 bytes (e4m3 x32) of its A row and B column.
// A row  = lane % 32, B column = lane % 32; the two lane halves supply two
// disjoint K ranges, the same ones for A and B.
// Accumulator element i of lane l is C[8*(i/4) + 4*(l/32) + i%4][l%32].
// ---------------------------------------------------------------------------

template <int UC> struct Acc;
template <> struct Acc<UC_BF16> { typedef f32x16 type; };
template <> struct Acc<UC_FP8> { typedef f32x16 type; };
template <> struct Acc<UC_I8> { typedef i32x16 type; };
template <> struct Acc<UC_MX8> { typedef f32x16 type; };
template <> struct Acc<UC_MX4> { typedef f32x16 type; };

__device__ __forceinline__ void mfma_bf16(f32x16& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ void mfma_i8(i32x16& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// e4m3 x e4m3 with unit block scales (E8M0 127 = 2^0)
__device__ __forceinline__ void mfma_fp8(f32x16& c, const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1) {
  const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// MX: e4m3 A x (e4m3 or, B_FP4, e2m1) B with one E8M0 scale per K-block of
// 32: lane half k supplies, in byte OPSEL of its scale word, the scale of
// K-block k of its A row (sa) and B column (sb).  In an e4m3 operand bytes
// 0-15 of both lane halves form K-block 0 and bytes 16-31 K-block 1; an
// e2m1 operand is 16 bytes (32 values, the even K in the low nibble) in b0,
// lane half k holding K-block k, and the instruction reads only four of its
// registers.
template <int OPSEL, bool B_FP4>
__device__ __forceinline__ void mfma_mx(f32x16& c, const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1,
                                        uint32_t sa, uint32_t sb) {
  const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  if constexpr (B_FP4) {
    const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b0, 0, 1, 2, 3, -1, -1, -1, -1));
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, OPSEL, (int)sa, OPSEL, (int)sb);
  } else {
    const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, (int)sa, OPSEL, (int)sb);
  }
}

// MX shared exponent of a group of 32 values whose largest magnitude is
// amax (OCP Microscaling rule): X = floor(log2 amax) - emax of the element
// format (e4m3: 8), clamped to [-127, 127]; -127 when amax is 0 or below
// the smallest normal float.  Returns X; the E8M0 code is X + 127 and the
// element multiplier 2^-X is mx_inv_scale(X), both exact.
__device__ __forceinline__ int mx_shared_exp_e4m3(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);   // biased exponent; 0 for 0 and denormals
  const int x = e - 127 - 8;
  return x < -127 ? -127 : x;
}
__device__ __forceinline__ float mx_inv_scale(int x) { return __uint_as_float((uint32_t)(127 - x) << 23); }

__device__ __forceinline__ float acc_to_f32(float v) { return v; }
__device__ __forceinline__ float acc_to_f32(int v) { return (float)v; }

}  // namespace mm
