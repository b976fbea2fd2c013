// Per-token 1x128 group quantisation to e4m3 ("SGLang PR 35605 review",
// implementation item 1 and the fp8_utils.py listing: bf16 activations are
// quantised on the fly, one fp32 scale per token per 128 columns, scale tensor
// [M, K/128]).
//
//   amax = max |x|;  s = max(amax, 1e-10) / 448;  q = e4m3_rne(clamp(x / s, +-448))
//
// Both divisions are IEEE fp32 divisions (hipcc's default correctly rounded
// division), the clamp runs before the hardware convert so its overflow
// behaviour is never reached, and the sign of zero is kept: codes and scales
// are bit-exact.
//
// Layout: 16 lanes share one 128-column group, each lane owns 8 consecutive
// bf16 (one 16-byte load); the group amax is a 16-lane butterfly; each lane
// stores 8 code bytes and lane 0 of the group stores the scale.
#include "kernels.hpp"
#include "quant_common.hpp"

namespace mxq {

// x: bf16 [M, K] with row stride ldx (elements); q: [M, K] bytes, row stride ldq;
// s: fp32 [M, K/128] row-major.
__global__ __launch_bounds__(256) void quant_1x128_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                          int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                          float* __restrict__ s) {
  const int64_t groups_per_row = K >> 7;
  const int64_t total = M * groups_per_row;
  const int64_t g = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  const bool valid = g < total;
  const int64_t gg = valid ? g : 0;
  const int64_t row = gg / groups_per_row;
  const int64_t col = (gg - row * groups_per_row) * 128 + sub * 8;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (valid) raw = *reinterpret_cast<const uint4*>(x + row * ldx + col);
  const float amax = group16_max(amax8_bf16(raw));
  if (valid) {
    uint2 qv;
    const float sc = quant8_e4m3(raw, amax, qv);
    *reinterpret_cast<uint2*>(q + row * ldq + col) = qv;
    if (sub == 0) s[gg] = sc;
  }
}

void launch_quant_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq, float* s,
                        hipStream_t stream) {
  const int64_t groups = M * (K >> 7);
  if (groups == 0) return;
  const unsigned grid = unsigned(cdiv(groups * 16, 256));
  hipLaunchKernelGGL(quant_1x128_kernel, dim3(grid), dim3(256), 0, stream, x, M, K, ldx, q, ldq, s);
}

}  // namespace mxq
