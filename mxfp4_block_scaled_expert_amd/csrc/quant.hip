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

#include <algorithm>

namespace mxq {

// x: bf16 [M, K] with row stride ldx (elements); q: [M, K] bytes, row stride ldq;
// s: fp32 [M, K/128] row-major.
__global__ __launch_bounds__(256) void quant_1x128_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                          int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                          float* __restrict__ s) {
  // 32-bit group indexing (the launcher keeps M * K / 128 below 2^31)
  const uint32_t groups_per_row = uint32_t(K >> 7);
  const int64_t total = M * int64_t(groups_per_row);
  const uint32_t g = (blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  const bool valid = int64_t(g) < total;
  const uint32_t gg = valid ? g : 0u;
  const int64_t row = gg / groups_per_row;
  const int64_t col = int64_t(gg - uint32_t(row) * groups_per_row) * 128 + sub * 8;
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
  if (groups * 16 >= (int64_t(1) << 31)) {
    // split into row chunks that keep the per-launch thread index in 32 bits
    const int64_t rows = ((int64_t(1) << 30) / 16) / (K >> 7);
    for (int64_t r0 = 0; r0 < M; r0 += rows)
      launch_quant_1x128(x + r0 * ldx, std::min<int64_t>(rows, M - r0), K, ldx, q + r0 * ldq, ldq, s + r0 * (K >> 7),
                         stream);
    return;
  }
  const unsigned grid = unsigned(cdiv(groups * 16, 256));
  hipLaunchKernelGGL(quant_1x128_kernel, dim3(grid), dim3(256), 0, stream, x, M, K, ldx, q, ldq, s);
}

}  // namespace mxq
