// Delayed-scaling FP8 bookkeeping for gfx950: weight casts, the cast test
// hook and the end-of-step scale update.
//
// Per-tensor delayed scaling ([BIO-ACC] 2.1 and 4.1; [TE-RU] FP8 recipe
// section: amax history of 16 steps, "max" algorithm): every FP8 tensor has a
// scale s; a step casts x * s to E4M3 with the scale fixed before the step,
// records amax = max |x| on the side, and at the end of the step the amax
// enters a ring buffer of the last history_len steps and s becomes
// 448 / max(history).  A maximum that is zero or not finite keeps the previous
// scale (initially 1).  Weights are cast once with s_w = 448 / amax(W).
#include "common.h"

namespace esm {

namespace {

__device__ __forceinline__ bool finite_pos(float v) { return v > 0.f && v < __builtin_inff(); }

__global__ __launch_bounds__(256) void k_amax_bf16(const bf16_t* __restrict__ x, int64_t n8, uint32_t* amax) {
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 w = *(const u32x4*)(x + i * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bflo(w[e])), fabsf(bfhi(w[e]))));
  }
  __shared__ float red[4];
  record_amax_block<4>(amax, m, red);
}

__global__ __launch_bounds__(256) void k_quantize_weight(const bf16_t* __restrict__ x, int64_t n8,
                                                         const uint32_t* __restrict__ amax, uint8_t* __restrict__ y,
                                                         float* scale_out) {
  const float am = __uint_as_float(*amax);
  const float s = finite_pos(am) ? kE4M3Max / am : 1.0f;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *scale_out = s;
  if (i >= n8) return;
  const u32x4 w = *(const u32x4*)(x + i * 8);
  const float lo[4] = {bflo(w[0]), bfhi(w[0]), bflo(w[1]), bfhi(w[1])};
  const float hi[4] = {bflo(w[2]), bfhi(w[2]), bflo(w[3]), bfhi(w[3])};
  *(u32x2*)(y + i * 8) = u32x2{pack_e4m3x4(lo, s), pack_e4m3x4(hi, s)};
}

__global__ __launch_bounds__(256) void k_quantize_f32(const float* __restrict__ x, int64_t n,
                                                      const float* __restrict__ scale, uint8_t* __restrict__ y,
                                                      uint32_t* amax) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float m = 0.f;
  if (i < n) {
    const float v[4] = {x[i], 0.f, 0.f, 0.f};
    y[i] = (uint8_t)(pack_e4m3x4(v, scale[0]) & 0xFFu);
    m = fabsf(x[i]);
  }
  __shared__ float red[4];
  record_amax_block<4>(amax, m, red);
}

// E5M2 cast of a bf16 gradient tensor (the HYBRID recipe): y = cast(x * s),
// round to nearest even (gfx950's v_cvt_pk_bf8_f32) after clamping to
// +-57344, so it saturates (infinities included); a NaN input is written as
// the NaN code 0x7F (the clamp alone would turn it into a finite value), so
// it reaches the GEMM that reads the codes; amax of |x| recorded (NaN left
// out, as for the E4M3 casts).  8 values per thread.
__global__ __launch_bounds__(256) void k_quantize_e5m2(const bf16_t* __restrict__ x, int64_t n8,
                                                       const float* __restrict__ scale, uint8_t* __restrict__ y,
                                                       uint32_t* amax, float* __restrict__ scale_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (scale_out && i == 0) scale_out[0] = scale[0];
  float m = 0.f;
  if (i < n8) {
    const u32x4 w = *(const u32x4*)(x + 8 * i);
    const float s = scale[0];
    constexpr float kMax = 57344.0f;
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bflo(w[e]);
      v[2 * e + 1] = bfhi(w[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    float c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = __builtin_amdgcn_fmed3f(v[e] * s, -kMax, kMax);
    int lo = __builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_bf8_f32(c[4], c[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_bf8_f32(c[6], c[7], hi, true);
    uint32_t r[2] = {(uint32_t)lo, (uint32_t)hi};
    // the sum is NaN iff a value is NaN or both infinities are present
    const float chk = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    if (chk != chk) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (v[e] != v[e]) r[e / 4] = (r[e / 4] & ~(0xFFu << (8 * (e % 4)))) | (0x7Fu << (8 * (e % 4)));
    }
    *(u32x2*)(y + 8 * i) = u32x2{r[0], r[1]};
  }
  __shared__ float red[4];
  record_amax_block<4>(amax, m, red);
}

// One thread per layer: its four activation tensors share the step counter.
// One layer's end of step for its four tensors: each step's amax enters
// slot steps % HL of the tensor's history; the next scale is fmax over the
// history's max when that is positive and finite (else the scale is kept);
// the amax is cleared.  Returns whether a non-finite amax was recorded.
__device__ bool roll_histories(float* scale, uint32_t* amax, float* history, int64_t* steps, int l, int HL,
                               float fmax) {
  const int slot = (int)(steps[l] % HL);
  bool nonfinite = false;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int k = 4 * l + t;
    const float am = __uint_as_float(amax[k]);
    if (!(am < __builtin_inff())) nonfinite = true;  // Inf or NaN bits
    float* h = history + (int64_t)k * HL;
    h[slot] = am;
    float mx = 0.f;
    bool ok = true;
    for (int j = 0; j < HL; ++j) {
      const float v = h[j];
      ok = ok && v < __builtin_inff() && v == v;
      mx = fmaxf(mx, v);
    }
    if (ok && mx > 0.f) scale[k] = fmax / mx;
    amax[k] = 0u;
  }
  steps[l] += 1;
  return nonfinite;
}

__global__ void k_scale_update(Fp8State s, int32_t l0, int32_t nl) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nl) return;
  const int l = l0 + idx;
  if (!s.layer_on[l]) return;  // a bf16 layer: recorded nothing, its state stays as it is
  if (roll_histories(s.act_scale, s.act_amax, s.history, s.steps, l, s.history_len, kE4M3Max)) atomicOr(s.flags, 1u);
}

// The gradients' end of a backward step (one layer; E5M2's largest value).
__global__ void k_grad_scale_update(Fp8State s, int32_t l) {
  if (threadIdx.x != 0) return;
  if (roll_histories(s.g_scale, s.g_amax, s.g_history, s.g_steps, l, s.history_len, 57344.0f)) atomicOr(s.flags, 1u);
}

}  // namespace

hipError_t launch_amax_bf16(const bf16_t* x, int64_t n, uint32_t* amax, hipStream_t st) {
  const int64_t n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  int64_t blocks = (n8 + 255) / 256;
  blocks = blocks < 2048 ? blocks : 2048;
  hipLaunchKernelGGL(k_amax_bf16, dim3((unsigned)blocks), dim3(256), 0, st, x, n8, amax);
  return hipGetLastError();
}

hipError_t launch_quantize_weight(const bf16_t* x, int64_t n, const uint32_t* amax, uint8_t* y, float* scale_out,
                                  hipStream_t st) {
  const int64_t n8 = n / 8;
  const int64_t blocks = n8 > 0 ? (n8 + 255) / 256 : 1;
  hipLaunchKernelGGL(k_quantize_weight, dim3((unsigned)blocks), dim3(256), 0, st, x, n8, amax, y, scale_out);
  return hipGetLastError();
}

hipError_t launch_quantize_f32(const float* x, int64_t n, const float* scale, uint8_t* y, uint32_t* amax,
                               hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, n, scale, y, amax);
  return hipGetLastError();
}

hipError_t launch_quantize_e5m2(const bf16_t* x, int64_t n, const float* scale, uint8_t* y, uint32_t* amax,
                                hipStream_t st, float* scale_out) {
  if (n <= 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_quantize_e5m2, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, x, n8, scale, y, amax,
                     scale_out);
  return hipGetLastError();
}

hipError_t launch_grad_scale_update(const Fp8State& s, int32_t l, hipStream_t st) {
  hipLaunchKernelGGL(k_grad_scale_update, dim3(1), dim3(64), 0, st, s, l);
  return hipGetLastError();
}

hipError_t launch_scale_update(const Fp8State& s, int32_t l0, int32_t nl, hipStream_t st) {
  if (nl <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_scale_update, dim3((unsigned)((nl + 63) / 64)), dim3(64), 0, st, s, l0, nl);
  return hipGetLastError();
}

}  // namespace esm
