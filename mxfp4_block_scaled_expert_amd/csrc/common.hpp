// Shared device helpers for the gfx950 kernels of libmxq.
//
// Everything here is CDNA4-specific: wave64, the FP8/FP4 MFMA and convert
// instructions of gfx950 (OCP e4m3 / e2m1 formats), and the 16x16 MFMA
// register layouts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN): gfx950's V_CVT_PK_BF16_F32,
// one instruction per pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ uint16_t f2bf(float f) { return uint16_t(pack_bf16x2(f, 0.f)); }

// ---------------------------------------------------------------- fp8 / fp4

// Two fp32 -> two e4m3 bytes in the low half of the result (hardware RNE).
// Inputs must already be clamped to [-448, 448].
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

// e4m3 pair (low or high 16 bits of v) -> two fp32, exact.
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t v, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(v, true) : __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
}

// Four e4m3 in one dword -> four bf16 in two dwords (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t v, uint32_t& lo, uint32_t& hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

// e8m0 exponent -> fp32 2^(e - 127), the OCP MX scale value: code 0 is 2^-127 (the fp32
// subnormal 0x00400000, never flushed here), code 0xFF is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  const uint32_t bits = e == 0 ? 0x00400000u : (e == 0xffu ? 0x7fc00000u : e << 23);
  return __uint_as_float(bits);
}

// Eight e2m1 nibbles (one dword, low nibble first) times a power-of-two scale
// -> eight bf16 (four dwords).  Exact while the scaled values stay in range.
__device__ __forceinline__ void e2m1x8_to_bf16(uint32_t v, float scale, uint32_t out[4]) {
  bf16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
  bf16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
  bf16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
  bf16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
  out[0] = __builtin_bit_cast(uint32_t, r0);
  out[1] = __builtin_bit_cast(uint32_t, r1);
  out[2] = __builtin_bit_cast(uint32_t, r2);
  out[3] = __builtin_bit_cast(uint32_t, r3);
}

// ---------------------------------------------------------------- MFMA

// D(16x16 fp32) += A(16x128 e4m3) * B(128x16 e4m3).  Lane l supplies row / column
// (l % 16) and one 32-element K slice selected by l / 16, the same slice for A and B.
__device__ __forceinline__ f32x4 mfma_16x16x128_e4m3(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l: row / column l % 16,
// K slice 8 * (l / 16) .. +8.
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(const i32x4& a, const i32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 16));
  return v;
}

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace mxq
