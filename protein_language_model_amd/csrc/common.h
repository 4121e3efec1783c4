// Internal definitions shared by the gfx950 kernels and the host library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace esm {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 64;
constexpr int kAttnTileRows = 128;  // query rows per attention workgroup

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Launch context handed from the host library to each launcher.
struct Launch {
  hipStream_t stream;
};

}  // namespace esm

// Host-side launchers (defined in the .hip files, called by encoder.cpp).
// Each returns hipGetLastError() after enqueueing.
namespace esm {

struct SegOut {
  int32_t* pos;      // [rows]
  int32_t* segs;     // [B, 2] (first row, length)
  int32_t* tiles;    // [cap, 2] (sequence, first query row)
  int32_t* ntiles;   // [1]
  int64_t tile_cap;
};

hipError_t launch_segment_table(int layout, const int32_t* lens, int32_t B, int64_t rows, int32_t S,
                                int32_t max_positions, const SegOut& out, hipStream_t st);

hipError_t launch_embed(const int32_t* ids, const bf16_t* table, int32_t vocab, bf16_t* x,
                        int64_t T, int32_t H, hipStream_t st);

hipError_t launch_layernorm(const bf16_t* x, const bf16_t* gamma, const bf16_t* beta, bf16_t* y,
                            int64_t M, int32_t H, float eps, hipStream_t st);

enum GemmEpi { EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_BIAS_RESIDUAL = 2, EPI_QKV_ROPE = 3 };

struct GemmArgs {
  const bf16_t* x;     // [M, K]
  const bf16_t* w;     // [N, K]
  const bf16_t* bias;  // [N] or null
  const bf16_t* res;   // [M, N] residual or null
  bf16_t* y;           // [M, N] (EPI_QKV_ROPE: planar [3, heads, M, 64])
  int64_t M;
  int32_t N, K;
  // rotary epilogue
  const int32_t* pos;      // [M] position of each row, -1 = padding row (skipped)
  const float2* rope;      // [max_positions, 32] (cos, sin)
  int32_t max_positions;
  // residual epilogue: rows whose pos < 0 are written as zero when zero_pad_rows
  int32_t zero_pad_rows;
};

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t st);

struct AttnArgs {
  const bf16_t* qkv;      // [3, heads, T, 64]
  bf16_t* ctx;            // [T, heads*64]
  const int32_t* segs;    // [B, 2]
  const int32_t* tiles;   // [cap, 2]
  const int32_t* ntiles;  // [1]
  int64_t tile_cap;
  int64_t T;
  int32_t heads;
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

}  // namespace esm
