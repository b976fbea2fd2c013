// Load-time relayout of routed-expert weights into the tiled layout the MoE
// kernels stream ("SGLang PR 32618 review": the GEMM takes packed or unpacked
// weights and its tests run both; "SGLang PR 35605 review": layout work moves
// from the forward pass to weight loading).
//
// Tiled layout of a weight tensor w[E][N][RB] (RB bytes per row, N % 16 == 0):
// rows are cut into 16-row groups and each row into 128-byte steps (the last
// one zero-padded); tile (e, g, s) is 2048 contiguous bytes at
// ((e * N/16 + g) * S + s) * 2048 with S = ceil(RB / 128).  Inside a tile,
// byte 1024 h + 16 L (h = 0, 1; L = 0..63) holds bytes [32 (L / 16) + 16 h, +16)
// of row 16 g + (L % 16): exactly the 16 bytes wave lane L loads as the
// h-th half of its MFMA operand, so one 64-lane load reads 1 KB contiguously.
//
// MX scales s[E][N][G] (G = K / 32 e8m0 bytes per row) are tiled the same way:
// tile (e, g, s) is 128 bytes at ((e * N/16 + g) * S + s) * 128, S = ceil(G / 8),
// and bytes 2 L, 2 L + 1 hold groups 8 s + 2 (L / 16) and + 1 of row 16 g + L % 16
// (0 past the row end).
#include "kernels.hpp"

namespace mxq {

__global__ __launch_bounds__(256) void prepack_w_kernel(const uint8_t* __restrict__ w, int64_t RB, int S,
                                                        int64_t total, uint8_t* __restrict__ out) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;  // 16-byte chunk of the output
  if (c >= total) return;
  const int pos = int(c & 127);
  const int64_t tile = c >> 7;
  const int64_t g = tile / S;  // global 16-row group (experts are contiguous)
  const int s = int(tile - g * S);
  const int h = pos >> 6, L = pos & 63;
  const int64_t row = g * 16 + (L & 15);
  const int64_t b = int64_t(s) * 128 + (L >> 4) * 32 + h * 16;
  i32x4 v = {0, 0, 0, 0};
  if (b + 16 <= RB) v = *reinterpret_cast<const i32x4*>(w + row * RB + b);
  *reinterpret_cast<i32x4*>(out + c * 16) = v;
}

__global__ __launch_bounds__(256) void prepack_s_kernel(const uint8_t* __restrict__ s_in, int64_t G, int S,
                                                        int64_t total, uint16_t* __restrict__ out) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;  // 2-byte pair of the output
  if (c >= total) return;
  const int L = int(c & 63);
  const int64_t tile = c >> 6;
  const int64_t g = tile / S;
  const int s = int(tile - g * S);
  const int64_t row = g * 16 + (L & 15);
  const int64_t g0 = int64_t(s) * 8 + 2 * (L >> 4);
  const uint32_t b0 = g0 < G ? s_in[row * G + g0] : 0u;
  const uint32_t b1 = g0 + 1 < G ? s_in[row * G + g0 + 1] : 0u;
  out[c] = uint16_t(b0 | (b1 << 8));
}

int64_t tiled_steps(int64_t row_bytes) { return (row_bytes + 127) / 128; }
int64_t tiled_scale_steps(int64_t groups) { return (groups + 7) / 8; }

void launch_prepack_w(const uint8_t* w, int64_t E, int64_t N, int64_t RB, uint8_t* out, hipStream_t st) {
  const int S = int(tiled_steps(RB));
  const int64_t total = E * (N / 16) * S * 128;
  if (total <= 0) return;
  hipLaunchKernelGGL(prepack_w_kernel, dim3(static_cast<unsigned>(cdiv(total, int64_t(256)))), dim3(256), 0, st,
                     w, RB, S, total, out);
}

void launch_prepack_s(const uint8_t* s, int64_t E, int64_t N, int64_t G, uint8_t* out, hipStream_t st) {
  const int S = int(tiled_scale_steps(G));
  const int64_t total = E * (N / 16) * S * 64;
  if (total <= 0) return;
  hipLaunchKernelGGL(prepack_s_kernel, dim3(static_cast<unsigned>(cdiv(total, int64_t(256)))), dim3(256), 0, st,
                     s, G, S, total, reinterpret_cast<uint16_t*>(out));
}

}  // namespace mxq
