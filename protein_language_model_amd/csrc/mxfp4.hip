// MXFP4 quantisation for gfx950: the FP4 recipe's operand format.
//
// The pages give the encoder an FP4 recipe beside the FP8 one ([TE-ESM2]
// FP8与FP4混合精度支持) without defining it; the format used is the one CDNA4's
// scaled MFMAs take natively, OCP MXFP4: E2M1 values (magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6) in blocks of 32 consecutive values along K, each block
// with one power-of-two scale X = 2^e stored as the E8M0 byte e + 127, where
// e = floor(log2 max|v|) - 2 (clamped to [-127, 127], -127 for a zero block)
// and every value is v / X rounded to the nearest E2M1 value, ties to even,
// saturating at 6.
//
// One thread per block: its 32 bf16 values are one 64-byte run, so a wave
// reads 4 KB of consecutive memory; v / X is exact (a power-of-two scaling of
// a bf16 value), and the rounding is gfx950's scaled FP4 conversion, two
// values per instruction (see e2m1_pair).
#include "common.h"

namespace esm {

namespace {

__global__ __launch_bounds__(256) void k_mx_quantize(const bf16_t* __restrict__ x, int64_t M, int32_t K,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int nb = K / 32;                     // blocks per row
  const int64_t M2 = M + (M & 1);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M2 * nb) return;
  const int64_t m = t / nb;
  const int b = (int)(t % nb);
  // scale byte of (row m, block b): K-step b / 8, position (b % 2) * 4 + (b % 8) / 2
  uint8_t* sdst = scales + mx_scale_offset(m, b, M2);
  if (m >= M) {          // the pad row of an odd M: scale 2^0, no codes
    *sdst = 127;
    return;
  }
  const bf16_t* src = x + m * K + b * 32;
  u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = *(const u32x4*)(src + 8 * i);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bflo(w[i][e])), fabsf(bfhi(w[i][e]))));
  const int ex = mx_block_exponent(amax);
  *sdst = (uint8_t)(ex + 127);
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // 8 values -> 8 nibbles, value 2j in the low nibble of byte j
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) word |= e2m1_pair(bflo(w[i][e]), bfhi(w[i][e]), ex) << (8 * e);
    out[i] = word;
  }
  *(u32x4*)(codes + m * (K / 2) + b * 16) = out;
}

}  // namespace

hipError_t launch_mx_quantize(const bf16_t* x, int64_t M, int32_t K, uint8_t* codes, uint8_t* scales,
                              hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int64_t n = (M + (M & 1)) * (K / 32);
  hipLaunchKernelGGL(k_mx_quantize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, M, K, codes, scales);
  return hipGetLastError();
}

}  // namespace esm
