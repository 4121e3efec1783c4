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
constexpr int kAttnTileRows = 256;  // query rows per attention workgroup (8 waves x 32)

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}
// Two floats -> two bfloat16 (RNE) in one word, lo in bits 0..15: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Operand element types of the GEMM.
constexpr int kBF16 = 0;
constexpr int kE4M3 = 1;
constexpr int kFP4 = 2;   // MXFP4: E2M1 codes, one E8M0 scale per 32 values along K
constexpr int kE5M2X = 3; // x operand E5M2 (a gradient), w operand E4M3: the HYBRID recipe's backward GEMM
constexpr float kE4M3Max = 448.0f;

// Four values v * s cast to OCP E4M3 (1.4.3, bias 7, no infinity, 0x7F = NaN,
// largest finite 448), packed little-endian into one word.  The gfx950
// converter rounds to nearest even; inputs are clamped to +-448 first
// (saturating cast, as the delayed-scaling recipe requires; s is positive and
// finite) and NaN is written as 0x7F.  NaN is detected once per four values:
// their sum is NaN iff one of them is NaN or they hold both infinities.
__device__ __forceinline__ uint32_t pack_e4m3x4(const float (&v)[4], float s) {
  float c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = __builtin_amdgcn_fmed3f(v[e] * s, -kE4M3Max, kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  uint32_t r = (uint32_t)w;
  const float chk = (v[0] + v[1]) + (v[2] + v[3]);
  if (chk != chk) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (v[e] != v[e]) r = (r & ~(0xFFu << (8 * e))) | (0x7Fu << (8 * e));
  }
  return r;
}

// MXFP4 (OCP microscaling, E2M1 values with one E8M0 scale per 32 values):
// the shared exponent of a block with maximum magnitude amax,
// e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for a zero or
// subnormal amax), read off the float's exponent field.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xff);
  const int ex = E == 0 ? -127 : E - 127 - 2;
  return ex < -127 ? -127 : (ex > 127 ? 127 : ex);
}
// E2M1 code of v (already divided by the block scale 2^e): bit 3 the sign,
// bits 2..0 the magnitude index in (0, 0.5, 1, 1.5, 2, 3, 4, 6); nearest
// value, ties to the even mantissa, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = a <= 0.25f ? 0u
                   : a < 0.75f ? 1u
                   : a <= 1.25f ? 2u
                   : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u
                   : a < 3.5f ? 5u
                   : a <= 5.0f ? 6u
                   : 7u;
  return c | ((__float_as_uint(v) >> 28) & 8u);
}
// Two values of a block with exponent ex to two E2M1 codes (v0 in bits 0..3,
// v1 in bits 4..7).  gfx950's v_cvt_scalef32_pk_fp4_f32 divides by the scale
// and rounds to nearest even with saturation at 6 -- the rule above, checked
// code by code against the definition (every midpoint and its neighbours,
// saturation, signed zero) before it was used here; its scale must be a
// normal float, so a block with ex = -127 (zero or tiny amax) takes the
// comparison chain.
__device__ __forceinline__ uint32_t e2m1_pair(float v0, float v1, int ex) {
  if (ex > -127) {
    const float X = __uint_as_float((uint32_t)(ex + 127) << 23);   // 2^ex
    return (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v0, v1, X, 0) & 0xFFu;
  }
  const float inv = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-ex = 2^127
  return e2m1_code(v0 * inv) | (e2m1_code(v1 * inv) << 4);
}

// Byte offset of the scale of (row m, block b) in the MXFP4 scale layout
// [K / 256][M2][8], blocks of a K step in the order 0, 2, 4, 6, 1, 3, 5, 7.
__device__ __forceinline__ int64_t mx_scale_offset(int64_t m, int b, int64_t M2) {
  return ((int64_t)(b / 8) * M2 + m) * 8 + ((b & 1) * 4 + ((b & 7) >> 1));
}

// Direct-to-LDS 16-byte load: lane i's 16 bytes from g land at LDS byte
// lds_base + 16 i (lds_base must be wave-uniform; it goes through M0).  Issued
// as inline assembly so the compiler keeps exact LDS wait counts for the
// fragment reads; the caller waits with vm_wait_all() before the barrier that
// publishes the tile.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Maximum of a non-negative per-lane value over the wave (fmaxf drops NaN).
__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  return m;
}

// Fold a non-negative maximum into *amax (float bits as uint32).  Non-negative
// floats order like their bit patterns, so atomicMax is exact and independent
// of the order of the updates.  A relaxed read first skips the atomic when the
// recorded value is already as large (it only grows, so a stale read can only
// cause an unneeded atomic): after the first workgroups almost all skip it.
__device__ __forceinline__ void fold_amax(uint32_t* amax, float m) {
  if (!(m > 0.f)) return;
  const uint32_t v = __float_as_uint(m);
  if (v > __hip_atomic_load(amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(amax, v);
}

// Block-wide amax: every thread of the workgroup calls this with its value
// (0 when it has none), NW = waves per workgroup; one lane folds the result.
template <int NW>
__device__ __forceinline__ void record_amax_block(uint32_t* amax, float m, float* red) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) b = fmaxf(b, red[w]);
    fold_amax(amax, b);
  }
}

// ---------------------------------------------------------------------------
// LayerNorm row statistics in pieces ([TE-RU] LayerNormLinear / LayerNormMLP:
// the LayerNorm belongs to the linear that consumes it).  A row of H values is
// cut into 256-column chunks (the GEMM's column tile); a chunk's partial
// (count, mean, sum of squared deviations M2) is built by one fixed tree:
//   * 8 leaves of 32 values, leaf (w, h) holding the columns
//     64 w + 32 j + 8 g + 4 h + e (j < 2, g < 4, e < 4) in that order -- the
//     values one MFMA lane holds for one row in the GEMM epilogue;
//   * leaves (w, 0) and (w, 1) combined, then waves ((0, 1), (2, 3)).
// The GEMM epilogue that writes a residual stream and the standalone
// statistics kernel both evaluate this tree with these functions, so they give
// identical bits for identical rows.  Partials are combined by Chan et al.'s
// pairwise update (mean and M2, no cancellation of large sums of squares).
// Contraction is off so that every product and sum is the same IEEE
// operation wherever the functions are inlined.
struct LnPart {
  float n, m, M2;
};

__device__ __forceinline__ LnPart ln_leaf(const float (&v)[32]) {
#pragma clang fp contract(off)
  float s = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) s = s + v[i];
  const float m = s * 0.03125f;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float d = v[i] - m;
    q = fmaf(d, d, q);
  }
  return LnPart{32.f, m, q};
}

// Combine partial a (columns first) with partial b; an empty side (n = 0) is
// the identity.  Equal counts (every combine inside a chunk) take the weight
// 1/2 without a division; it is the value the division gives.
__device__ __forceinline__ LnPart ln_combine(LnPart a, LnPart b) {
#pragma clang fp contract(off)
  if (b.n == 0.f) return a;
  if (a.n == 0.f) return b;
  const float n = a.n + b.n;
  const float d = b.m - a.m;
  const float wb = a.n == b.n ? 0.5f : b.n / n;
  const float m = a.m + d * wb;
  const float M2 = (a.M2 + b.M2) + (d * d) * (a.n * wb);
  return LnPart{n, m, M2};
}

// Mean and 1 / sqrt(var + eps) of a row of H <= 4096 values from its chunk
// partials part[c * ld] = (mean, M2), c < ceil(H / 256), chunk c holding
// n_c = min(256, H - 256 c) columns:
//   mean = sum_c n_c mean_c / H,   M2 = sum_c (M2_c + n_c (mean_c - mean)^2).
// All loads are issued before the first use.
__device__ __forceinline__ float2 ln_row_stats(const float2* part, int64_t ld, int H, float eps) {
  constexpr int kMaxChunks = 16;
  const int chunks = (H + 255) / 256;
  float2 p[kMaxChunks];
  // chunks past the last re-read the last one (no branch around the loads)
  // and are then zeroed: count 0 and M2 0, so they add nothing below
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) p[c] = part[(int64_t)(c < chunks ? c : chunks - 1) * ld];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
    if (c >= chunks) p[c] = make_float2(0.f, 0.f);
  const float invH = 1.0f / (float)H;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int w = H - 256 * c;
    s = fmaf((float)(w < 0 ? 0 : (w < 256 ? w : 256)), p[c].x, s);
  }
  const float mean = s * invH;
  float M2 = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int w = H - 256 * c;
    const float d = p[c].x - mean;
    M2 = M2 + fmaf((float)(w < 0 ? 0 : (w < 256 ? w : 256)) * d, d, p[c].y);
  }
  return make_float2(mean, 1.0f / sqrtf(M2 * invH + eps));
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

// out[i] = cu[b0 + i] - cu[b0] for i = 0 .. n (the cu_seqlens of sequences b0 ..
// b0 + n - 1 as a batch of their own)
hipError_t launch_rebase_cu(const int32_t* cu, int32_t b0, int32_t n, int32_t* out, hipStream_t st);
hipError_t launch_segment_table(int layout, const int32_t* lens, int32_t B, int64_t rows, int32_t S,
                                int32_t max_positions, const SegOut& out, hipStream_t st);

hipError_t launch_embed(const int32_t* ids, const bf16_t* table, int32_t vocab, bf16_t* x,
                        int64_t T, int32_t H, hipStream_t st);
// LayerNorm chunk partials [ceil(H / 256)][T] of the rows of x [T, H]; with
// ids != nullptr the rows are first gathered from table (x = E[ids], written).
hipError_t launch_row_stats(const int32_t* ids, const bf16_t* table, int32_t vocab, bf16_t* x, int64_t T, int32_t H,
                            float2* stats, hipStream_t st);
// Folded LayerNorm weight of a linear: wf [N, K] = bf16(gamma_k w_nk),
// cd[n] = (sum_k wf_nk, b_n + sum_k beta_k w_nk); bias may be null.
hipError_t launch_fold_weight(const bf16_t* w, const bf16_t* gamma, const bf16_t* beta, const bf16_t* bias,
                              int32_t N, int32_t K, bf16_t* wf, float2* cd, hipStream_t st);

// E4M3 output of a producer kernel: y = cast(v * scale[0]), amax of v
// recorded into *amax.  y == nullptr selects the bf16 output instead.
struct E4m3Out {
  uint8_t* y;
  const float* scale;  // device
  uint32_t* amax;      // device, float bits
  const int32_t* pos;  // optional [rows]: rows with pos < 0 (padding) stay out of the amax
};

hipError_t launch_pad_rows(const bf16_t* src, int32_t rows, int32_t cols, bf16_t* dst, int32_t rows_pad,
                           hipStream_t st);
hipError_t launch_take_cols(const bf16_t* src, int32_t ld_src, bf16_t* dst, int64_t T, int32_t cols, hipStream_t st);
hipError_t launch_segment_mean(const bf16_t* x, const int32_t* segs, int32_t B, int32_t H, float* out,
                               hipStream_t st);
hipError_t launch_layernorm(const bf16_t* x, const bf16_t* gamma, const bf16_t* beta, bf16_t* y,
                            int64_t M, int32_t H, float eps, const E4m3Out& q, hipStream_t st);
// LayerNorm whose output goes straight to MXFP4 (the esm_mxfp4_quantize
// layout, H % 256 == 0): the fp32 normalised values are quantised, no bf16 row.
hipError_t launch_layernorm_mx(const bf16_t* x, const bf16_t* gamma, const bf16_t* beta, uint8_t* codes,
                               uint8_t* scales, int64_t M, int32_t H, float eps, hipStream_t st);

// EPI_QKV_ROPE_LN / EPI_BIAS_GELU_LN: the rotary / GELU epilogues of a linear
// whose input is LayerNorm(x) with the LayerNorm folded away: x (the raw
// residual stream) is the GEMM operand, the weight is the prepared
// W' = gamma (.) W, and output column n is
//   r (x . W'_n) - r mu c_n + d_n,   c_n = sum_k W'_nk,  d_n = b_n + sum_k beta_k W_nk,
// with (mu, r = 1 / sqrt(var + eps)) of each row from ln_stats.
// EPI_RES_STATS: the residual epilogue that also writes the chunk partials of
// the LayerNorm statistics of its output rows (stats_out).
enum GemmEpi { EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_BIAS_RESIDUAL = 2, EPI_QKV_ROPE = 3, EPI_BIAS_GELU_E4M3 = 4,
               EPI_BIAS_GELU_MX = 5, EPI_F32_SPLIT = 6, EPI_QKV_ROPE_LN = 7, EPI_BIAS_GELU_LN = 8,
               EPI_RES_STATS = 9, EPI_F32_SPLIT_KM = 10 };

struct GemmArgs {
  int32_t dtype;       // kBF16 or kE4M3 operands
  const void* x;       // [M, K]
  const void* w;       // [N, K]
  const float* x_scale;  // E4M3: device scales; the product is divided by x_scale[0] * w_scale[0]
  const float* w_scale;
  const bf16_t* bias;  // [N] or null
  const bf16_t* res;   // [M, N] residual or null
  bf16_t* y;           // [M, N] (EPI_QKV_ROPE: planar [3, heads, M, 64])
  int64_t M;
  int32_t N, K;
  // rotary epilogue
  const int32_t* pos;      // [M] position of each row, -1 = padding row (skipped)
  const float2* rope;      // [max_positions, 32] (cos, sin)
  int32_t max_positions;
  // set when the rows hold padding (pos < 0, a bshd batch): the residual
  // epilogue writes such rows as zero and the rotary epilogue skips them
  int32_t zero_pad_rows;
  // EPI_BIAS_GELU_E4M3: y8 = cast(gelu(.) * y8_scale[0]), amax into *y8_amax
  uint8_t* y8;
  const float* y8_scale;
  uint32_t* y8_amax;
  // EPI_F32_SPLIT (bf16 operands): K cut into ksplit equal slices; slice s's
  // product, in fp32, goes to y32 + s * M * N (no bias); K % (64 ksplit) == 0.
  // EPI_F32_SPLIT_KM: the same with both operands stored contraction-major,
  // x as [K, M] and w as [K, N] row-major (a weight gradient dy^T x read from
  // dy and x as they are); any K, the slices are Kl = K rounded up to
  // 64 ksplit, divided by ksplit, long, and rows past K count as zero; M and
  // N multiples of 64.
  float* y32;
  int32_t ksplit;
  // kFP4 operands: E8M0 block scales in the esm_mxfp4_quantize layout
  // [K / 256][rows rounded up to even][8]
  const uint8_t* x_sc;
  const uint8_t* w_sc;
  // EPI_BIAS_GELU_MX: y8 = MXFP4 codes [M, N / 2] of gelu(.), y_sc their
  // block scales (the same layout, K = N)
  uint8_t* y_sc;
  // folded LayerNorm (EPI_*_LN): chunk partials [ceil(K / 256)][M] of the x
  // rows, eps, and (c_n, d_n) per output column [N]
  const float2* ln_stats;
  float ln_eps;
  const float2* ln_cd;
  // EPI_RES_STATS: chunk partials [ceil(N / 256)][M] of the output rows
  float2* stats_out;
};

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t st);
// Rounds of workgroups over the current device's compute units that
// launch_gemm runs for an M x N output (forward epilogues).
int64_t gemm_rounds(int64_t M, int32_t N);
// Matrix-core rate probe (k_mfma_peak): `blocks` workgroups of four waves,
// each wave 16 * iters v_mfma_f32_32x32x16_bf16; sink [4 * blocks] floats.
hipError_t launch_mfma_peak(int32_t iters, int32_t blocks, float* sink, hipStream_t st);
int32_t mfma_peak_blocks();  // two workgroups per compute unit of the current device

struct AttnArgs {
  const bf16_t* qkv;      // [3, heads, T, 64]
  bf16_t* ctx;            // [T, heads*64]
  E4m3Out ctx8;           // when ctx8.y is set: E4M3 context instead of ctx
  uint8_t* ctx_mx;        // when set: MXFP4 context codes [T, H / 2] instead of ctx ...
  uint8_t* ctx_mx_sc;     // ... and their block scales (esm_mxfp4_quantize layout, K = H)
  float* lse;             // when set: [heads, T] softmax normaliser log sum_j exp(q.k_j / 8)
  const int32_t* segs;    // [B, 2]
  const int32_t* tiles;   // [cap, 2]
  const int32_t* ntiles;  // [1]
  int64_t tile_cap;
  int64_t T;
  int32_t heads;
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

// Attention backward on the encoder layout: dqkv [3, heads, T, 64] from qkv,
// the forward's context out [T, H], its gradient dout [T, H] and lse
// [heads, T]; delta [heads, T] is scratch (rowsum(dout * out)).
struct AttnBwdArgs {
  const bf16_t* qkv;
  const bf16_t* out;
  const bf16_t* dout;
  const float* lse;
  float* delta;
  bf16_t* dqkv;
  const int32_t* segs;    // [B, 2]
  const int32_t* tiles;   // [cap, 2]
  const int32_t* ntiles;  // [1]
  int64_t tile_cap;
  int64_t T;
  int32_t heads;
};

hipError_t launch_attention_bwd(const AttnBwdArgs& a, hipStream_t st);

// Linear backward helpers: out [C, Rp] = in[R, C]^T with rows R .. Rp - 1 of
// the result zero (C, Rp multiples of 64); db[n] = sum_m dy[m, n] in fp32
// through part [colsum_chunks(M), N] (N a multiple of 64).
hipError_t launch_transpose_pad(const bf16_t* in, int64_t R, int32_t C, bf16_t* out, int64_t Rp, hipStream_t st);
hipError_t launch_colsum(const bf16_t* dy, int64_t M, int32_t N, float* part, float* db, hipStream_t st);
int64_t colsum_chunks(int64_t M);
// Embedding table gradient: dtable [vocab, H] fp32 = per-token sums of dx
// [M, H] bf16 over the rows holding each token (ids clamped to [0, vocab) as
// the gather clamps them), through part [colsum_chunks(M), vocab, H] fp32; H a
// multiple of 64, vocab <= kEmbedBwdMaxVocab (its LDS accumulators).
constexpr int32_t kEmbedBwdMaxVocab = 64;
hipError_t launch_embed_bwd(const int32_t* ids, const bf16_t* dx, int64_t M, int32_t H, int32_t vocab, float* part,
                            float* dtable, hipStream_t st);
// dW GEMM of the linear backward: K slices (split-K) for M rows, and the
// fixed-order sum of the slices' fp32 partials into bf16.
int32_t wgrad_splits(int64_t M, int32_t N, int32_t K);
hipError_t launch_split_reduce(const float* part, int32_t S, int64_t n, bf16_t* out, hipStream_t st,
                               const float* sa = nullptr, const float* sb = nullptr);
// out [C, Rp] bytes = transpose of in [R, C] bytes, rows R .. Rp - 1 zero; C, Rp multiples of 64
hipError_t launch_transpose8_pad(const uint8_t* in, int64_t R, int32_t C, uint8_t* out, int64_t Rp, hipStream_t st);
// LayerNorm backward: dx [M, H] bf16, dgamma and dbeta [H] fp32; stats [2M]
// and part [colsum_chunks(M), 2, H] fp32 are scratch.  H a multiple of 64, <= 4096.
// GELU backward: dz = dy GELU'(z), n % 8 == 0.  QKV/RoPE backward: planar
// dqkv [3, heads, T, 64] -> dy [T, 3H] in the fused QKV linear's interleaved
// column order, q and k rotated back by the row positions pos [T].
hipError_t launch_gelu_bwd(const bf16_t* z, const bf16_t* dy, bf16_t* dz, int64_t n, hipStream_t st);
// a = GELU(z) elementwise (the fc1 epilogue's GELU), bf16 in and out; n a multiple of 8
hipError_t launch_gelu_fwd(const bf16_t* z, bf16_t* a, int64_t n, hipStream_t st);
hipError_t launch_qkv_rope_bwd(const bf16_t* dqkv, const int32_t* pos, const float2* rope, int32_t max_positions,
                               int64_t T, int32_t heads, bf16_t* dy, hipStream_t st);
hipError_t launch_layernorm_bwd(const bf16_t* x, const bf16_t* gamma, const bf16_t* dy, const bf16_t* dres, bf16_t* dx,
                                float* dgamma, float* dbeta, int64_t M, int32_t H, float eps, float* stats, float* part,
                                hipStream_t st);

// Biased attention on [B, N, L, heads, 64] tensors: per (b, n, h),
// out = softmax(q k^T / 8 + mask[b, n, :] + pair[b, h, :, :]) v.
struct BiasedAttnArgs {
  const bf16_t* q;     // [B, N, L, heads, 64]
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* mask;  // [B, N, L] or null
  const bf16_t* pair;  // [B, heads, L, L] or null
  bf16_t* out;         // [B, N, L, heads, 64]
  int32_t B, N, L, heads;
  int32_t qtiles;      // ceil(L / kAttnTileRows)
};

hipError_t launch_biased_attention(const BiasedAttnArgs& a, hipStream_t st);

// MXFP4 quantisation of x [M, K] (K % 256 == 0): codes [M, K / 2] (value 2j
// in the low nibble of byte j), E8M0 scales [K / 256][M2][8] with M2 = M
// rounded up to even, the 8 bytes of (K step s, row m) holding the scales of
// blocks 8s + {0, 2, 4, 6, 1, 3, 5, 7}.
hipError_t launch_mx_quantize(const bf16_t* x, int64_t M, int32_t K, uint8_t* codes, uint8_t* scales,
                              hipStream_t st);

// Delayed-scaling bookkeeping (fp8.hip).
struct Fp8State {
  float* act_scale;    // [layers, 4] scale used by the current step (ln1, ctx, ln2, act)
  uint32_t* act_amax;  // [layers, 4] amax of the current step, float bits
  float* history;      // [layers, 4, history_len] ring buffer
  int64_t* steps;      // [layers] recorded steps (ring position = steps % history_len)
  uint32_t* flags;     // [1] bit 0: a non-finite amax was recorded
  float* w_scale;      // [layers, 4] weight scales (qkv, out, fc1, fc2)
  uint32_t* w_amax;    // [layers, 4]
  int32_t* layer_on;   // [layers] 1 = the layer runs FP8 (its state is updated), 0 = bf16 (state frozen)
  int32_t history_len;
  // gradients of the HYBRID backward (E5M2): per layer the output gradients
  // of the qkv, out-projection, fc1 and fc2 linears
  float* g_scale;      // [layers, 4]
  uint32_t* g_amax;    // [layers, 4] amax of the current backward step, float bits
  float* g_history;    // [layers, 4, history_len]
  int64_t* g_steps;    // [layers]
};

// amax of n bf16 values into *amax (which must start at 0).
hipError_t launch_amax_bf16(const bf16_t* x, int64_t n, uint32_t* amax, hipStream_t st);
// y = cast(x * s), s = 448 / amax (1 when amax is 0 or not finite); writes s to *scale_out.
hipError_t launch_quantize_weight(const bf16_t* x, int64_t n, const uint32_t* amax, uint8_t* y, float* scale_out,
                                  hipStream_t st);
// y = cast(x * scale[0]) with x fp32 (test hook of the cast); amax of x into *amax.
hipError_t launch_quantize_f32(const float* x, int64_t n, const float* scale, uint8_t* y, uint32_t* amax,
                               hipStream_t st);
// End of a step for layers [l0, l0 + nl): push amax into the history, new scale
// = 448 / max(history) when that is positive and finite, clear amax.
// End of a backward step of layer l: the same roll for its four gradient
// tensors with E5M2's largest value (57344).
hipError_t launch_grad_scale_update(const Fp8State& s, int32_t l, hipStream_t st);
// y = cast_e5m2(x * scale[0]), amax of x into *amax; scale[0] also copied to
// *scale_out when that is not NULL.
hipError_t launch_quantize_e5m2(const bf16_t* x, int64_t n, const float* scale, uint8_t* y, uint32_t* amax,
                                hipStream_t st, float* scale_out = nullptr);
hipError_t launch_scale_update(const Fp8State& s, int32_t l0, int32_t nl, hipStream_t st);

}  // namespace esm
