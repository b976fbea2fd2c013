// 1x128 group quantisation step shared by the standalone quantiser and the
// fused SiLU-and-mul re-quantisation of the W8A8 MoE: 16 lanes hold one
// 128-value group, 8 bf16 values per lane.
#pragma once

#include "common.hpp"

namespace mxq {

__device__ __forceinline__ float amax8_bf16(const uint4 raw) {
  float m = 0.f;
  m = fmaxf(m, fabsf(bf16lo(raw.x))); m = fmaxf(m, fabsf(bf16hi(raw.x)));
  m = fmaxf(m, fabsf(bf16lo(raw.y))); m = fmaxf(m, fabsf(bf16hi(raw.y)));
  m = fmaxf(m, fabsf(bf16lo(raw.z))); m = fmaxf(m, fabsf(bf16hi(raw.z)));
  m = fmaxf(m, fabsf(bf16lo(raw.w))); m = fmaxf(m, fabsf(bf16hi(raw.w)));
  return m;
}

// s = max(amax, 1e-10) / 448 and q = e4m3(clamp(x / s, +-448)) for this lane's
// 8 values.  Both divisions are IEEE fp32 divisions.  Returns s.
__device__ __forceinline__ float quant8_e4m3(const uint4 raw, float group_amax, uint2& q) {
  const float s = fmaxf(group_amax, 1e-10f) / 448.0f;
  float v[8];
  v[0] = bf16lo(raw.x); v[1] = bf16hi(raw.x);
  v[2] = bf16lo(raw.y); v[3] = bf16hi(raw.y);
  v[4] = bf16lo(raw.z); v[5] = bf16hi(raw.z);
  v[6] = bf16lo(raw.w); v[7] = bf16hi(raw.w);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(v[i] / s, -448.0f), 448.0f);
  q.x = cvt_pk_e4m3(v[0], v[1]) | (cvt_pk_e4m3(v[2], v[3]) << 16);
  q.y = cvt_pk_e4m3(v[4], v[5]) | (cvt_pk_e4m3(v[6], v[7]) << 16);
  return s;
}

// SiLU-and-mul ("vLLM PR 50949 review", implementation item 2: the activation between the two
// stages): silu(g) * u with silu(g) = g / (1 + e^-g), in fp32, of a gate / up pair that has
// already been rounded to bf16; the caller rounds the result to bf16.  The standalone
// SiLU-and-mul kernel, the stage-2 activation staging of the tiny-block kernel and the stage-1
// epilogue of the expert-streaming kernel all evaluate this one expression, so they produce
// the same bits.
__device__ __forceinline__ float silu_mul_f32(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Eight gate / up bf16 pairs -> eight bf16.
__device__ __forceinline__ uint4 silu_mul8(const uint4 g, const uint4 u) {
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t hw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    hw[i] = pack_bf16x2(silu_mul_f32(bf16lo(gw[i]), bf16lo(uw[i])), silu_mul_f32(bf16hi(gw[i]), bf16hi(uw[i])));
  return make_uint4(hw[0], hw[1], hw[2], hw[3]);
}

}  // namespace mxq
