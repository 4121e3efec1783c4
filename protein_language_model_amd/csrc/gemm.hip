// MFMA GEMM for gfx950 with fused epilogues:  y = epi(x[M,K] . w[N,K]^T + b)
//
// The four linears of a pre-LN encoder layer ([BIO-ACC] 3.1: QKV projection,
// attention output projection, fc1, fc2; [TE-RU] LayerNormLinear / LayerNormMLP)
// are all "both operands K-contiguous" products, so both MFMA operands are read
// from LDS as 16-byte runs along K.  Operands are bf16, or OCP E4M3 with one
// scale per tensor for the delayed-scaling FP8 recipe ([BIO-ACC] 2.1 and 4.1;
// [TE-RU] FP8 recipe section): y = (qx . qw^T) / (s_x s_w) + b.
//
// Design (CDNA4):
//  * WAVES_M x WAVES_N waves (8 = two per SIMD: one wave's LDS reads and
//    waits overlap the other's MFMAs); each wave owns a (BM/WAVES_M) x
//    (BN/WAVES_N) tile built from 32x32 blocks, v_mfma_f32_32x32x16_bf16 for
//    bf16 and v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit block
//    scales) for FP8, with fp32 accumulators.
//  * The weight is MFMA operand A and the activations operand B, so lane l of
//    a 32x32 block holds output row m = l%32 and columns
//    n = 8*(r/4) + 4*(l/32) + r%4 (r = 0..15): four consecutive columns per
//    register group.  Columns j and j+32 of a 64-wide group sit in the same
//    lane and register of two adjacent blocks, which is what the rotary
//    epilogue needs ([TE-ESM2] 旋转位置编码集成: rotate-half pairs (i, i+32)).
//  * A K step is 128 bytes of each row (64 bf16 or 128 E4M3 values); tiles
//    live in LDS twice (double buffer) with a 16-byte-chunk XOR swizzle (chunk c of row r stored at c ^ ((r >> 1) & 7)): the 16 lanes that
//    one LDS cycle serves read 16 rows of one column and hit 16 distinct
//    16-byte bank groups of the 64-bank LDS.  The next K step is
//    fetched straight into the other LDS buffer (global_load_lds, no staging
//    registers) while the current one is multiplied.  MFMA fragments are
//    double-buffered in registers across the k sub-steps, and the
//    single barrier per K step sits before the last sub-step, so the next
//    tile's first fragments load under MFMAs.
//  * Rows beyond M and weight rows beyond N are clamped on load (never read out
//    of bounds) and skipped on store.
//  * Workgroup ids are remapped so consecutive tiles land on one XCD (ids are
//    dealt round-robin over the 8 XCDs), then grouped a few row-tiles at a
//    time so a row panel of x and the weight panels stay in that XCD's L2
//    (8 row tiles; 4 when the output is at least 4x wider than the
//    contraction, as in the first feed-forward linear, and 2 when the
//    contraction is at least 4x the output width, as in the second; chosen
//    by measurement on those shapes).
#include "common.h"

#include <type_traits>

namespace esm {

namespace {

constexpr int kXcds = 8;
constexpr int kRowBytes = 128;  // bytes of each tile row per K step

typedef int i32x8 __attribute__((ext_vector_type(8)));

// lds_dma16 with a wave-uniform base in scalar registers and a per-lane 32-bit
// byte offset (the instruction's saddr form).
__device__ __forceinline__ void lds_dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 512 zero bytes: the source of the contraction-major loads for rows past the
// contraction's end (never written).
__device__ __attribute__((aligned(16))) unsigned char g_zero_row[512];

// GELU(z) = z Phi(z), Phi the standard normal CDF (the exact, erf form; the
// pages name a fused activation only).  With q = Phi(-|z|), GELU(z) is
// z (1 - q) for z >= 0 and z q for z < 0, i.e. max(z, 0) - |z| q in both
// cases: one FMA, no select, and the negative tail is a product (no
// cancellation, sign kept).  q = 2^P(t), t = min(|z|, 9), P a degree-6
// polynomial fitted to log2 Phi(-a) on [0, 9] (gelu_tail_fit.py): beyond 9
// the tail term is held at its value there, 9 * 2^P(9) = 2.3e-18, so
// GELU(z) = z for z >= 9 and -2.3e-18 for z <= -9 (exactly: 0 > GELU(z) >
// -1.1e-18).  In fp32 |q - Phi(-|z|)| <= 6.3e-7, and relative to Phi(-|z|)
// <= 3e-5 for |z| < 4 and <= 6e-4 for |z| < 5: below half a bf16 ulp of the
// result everywhere.  The epilogue's VALU work is not hidden behind MFMAs
// (all waves of a tile reach it together), so the degree is the smallest that
// keeps that margin and the form the one with fewest instructions (the
// minimum and maximum propagate NaN: GELU(NaN) = NaN, GELU(+inf) = +inf,
// GELU(-inf) = -2.3e-18).
constexpr float kGeluP0 = -0.9999982118606567f;
constexpr float kGeluP1 = -1.1511716842651367f;
constexpr float kGeluP2 = -0.4588053524494171f;
constexpr float kGeluP3 = -0.05342535302042961f;
constexpr float kGeluP4 = 0.008116660639643669f;
constexpr float kGeluP5 = -0.0007859239703975618f;
constexpr float kGeluP6 = 3.5450411814963445e-05f;
__device__ __forceinline__ float gelu(float z) {
  const float t = __builtin_elementwise_minimum(fabsf(z), 9.0f);  // P is only fitted up to 9
  float p = fmaf(kGeluP6, t, kGeluP5);
  p = fmaf(p, t, kGeluP4);
  p = fmaf(p, t, kGeluP3);
  p = fmaf(p, t, kGeluP2);
  p = fmaf(p, t, kGeluP1);
  p = fmaf(p, t, kGeluP0);
  return fmaf(-t, __builtin_amdgcn_exp2f(p), __builtin_elementwise_maximum(z, 0.0f));
}

template <int DT>
struct Frag;
template <>
struct Frag<kBF16> {
  typedef bf16x8 T;  // 8 bf16 along K: one 16-wide sub-step
  static constexpr int kSub = 16;
};
template <>
struct Frag<kE4M3> {
  typedef i32x8 T;  // 32 E4M3 along K: one 64-wide sub-step
  static constexpr int kSub = 64;
};
template <>
struct Frag<kE5M2X> : Frag<kE4M3> {};
template <>
struct Frag<kFP4> {
  typedef i32x8 T;  // 32 E2M1 along K (one MX block) in the low 4 registers: one 64-wide sub-step
  static constexpr int kSub = 64;
};

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI, int DT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void k_gemm(GemmArgs a) {
  typedef typename Frag<DT>::T frag_t;
  // operand bytes per element = EBN / EBD: bf16 2, E4M3 1, FP4 1/2
  constexpr int EBN = DT == kBF16 ? 2 : 1;
  constexpr int EBD = DT == kFP4 ? 2 : 1;
  constexpr int kBK = kRowBytes * EBD / EBN;    // K per step, in elements
  constexpr int KK = kBK / Frag<DT>::kSub;      // k sub-steps per K step
  constexpr int FB = Frag<DT>::kSub * EBN / (32 * EBD);  // 16-byte chunks per lane per fragment
  constexpr bool MX = DT == kFP4;               // block scales: 8 bytes per tile row per K step
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M;
  constexpr int WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int RPI = 1024 / kRowBytes;         // tile rows filled by one 1 KB direct load
  constexpr int XRB = BM / (RPI * NW);          // such row blocks of the x tile per wave
  constexpr int WRB = BN / (RPI * NW);
  constexpr int kStage = (BM + BN) * kRowBytes;  // bytes per K-step stage
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(XRB * RPI * NW == BM && WRB * RPI * NW == BN, "tile rows must split evenly over the waves");
  static_assert(DT != kBF16 || KK % 2 == 0, "fragment double buffering alternates over an even number of sub-steps");
  constexpr bool ROPE = EPI == EPI_QKV_ROPE || EPI == EPI_QKV_ROPE_LN;
  constexpr bool RES = EPI == EPI_BIAS_RESIDUAL || EPI == EPI_RES_STATS;
  constexpr bool FOLD = EPI == EPI_QKV_ROPE_LN || EPI == EPI_BIAS_GELU_LN;  // LayerNorm folded into the linear
  constexpr bool STATS = EPI == EPI_RES_STATS;                              // LayerNorm partials of the output
  // EPI_F32_SPLIT_KM: operands stored contraction-major (x [K, M], w [K, N]).
  // A K step's tile of an operand is then 64 contraction rows of its 256
  // tile columns (512 bytes each) instead of 256 rows of 64 contraction
  // values: the same 32 KB, filled by the same 1 KB direct loads (two rows
  // each), with 16-byte chunk c of contraction row r stored at chunk
  // c ^ 4 (r % 4).  Fragments are read with gfx950's transposing LDS read
  // (ds_read_b64_tr_b16: in a group of 16 lanes, lane j addresses four
  // values of row r0 + j / 4 at columns c0 + 4 (j % 4), and lane i receives
  // column c0 + i of rows r0 .. r0 + 3): two reads give a lane the eight
  // contraction values of its fragment row, in the order the row-major
  // fragments hold them, so the MFMAs see the same operands as for
  // transposed copies of x and w.  Per half-wave read the four rows'
  // 64-byte column bands fall on distinct banks (checked by simulating the
  // bank map).
  constexpr bool KMAJ = EPI == EPI_F32_SPLIT_KM;
  constexpr bool SPLIT = EPI == EPI_F32_SPLIT || KMAJ;
  static_assert(!KMAJ || (DT == kBF16 && BM == 256 && BN == 256 && NW == 8 && XRB == 4 && WRB == 4),
                "contraction-major operands: bf16, 256 x 256 tiles of eight waves");
  static_assert(!ROPE || (FN % 2 == 0 && WTN % 64 == 0), "rotary pairs need 64-wide wave columns");
  static_assert(EPI != EPI_BIAS_GELU_E4M3 || DT == kE4M3, "E4M3 output is built for E4M3 operands");
  static_assert(!(FOLD || STATS) || (DT == kBF16 && BN == 256), "folded LayerNorm: bf16, 256-column tiles");

  // Two K-step stages; after the K loop the same memory stages the output,
  // the whole tile at once when it fits, else 32-row chunks of every wave's
  // tile (see the epilogue).
  constexpr bool OUT8 = EPI == EPI_BIAS_GELU_E4M3;
  constexpr bool OUTMX = EPI == EPI_BIAS_GELU_MX;
  // The feed-forward intermediate (the GELU epilogues' output) is written once
  // and read once by the next GEMM: its stores stream past the caches
  // (non-temporal), leaving them to the tiles' operand panels and to the next
  // kernels' inputs.
  constexpr bool NT_OUT = EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_LN || OUT8 || OUTMX;
  static_assert(!OUTMX || DT == kFP4, "MXFP4 output is built for MXFP4 operands");
  constexpr int OES = OUT8 ? 1 : 2;               // output bytes per element (bf16, E4M3)
  constexpr int ORB = OUTMX ? WTN / 2 : WTN * OES;  // output bytes of one row of a wave's tile
  constexpr int ECH = BM * WAVES_N * ORB <= 2 * kStage ? WTM : 32;  // staged rows per wave per chunk
  static_assert(WTM % ECH == 0, "whole chunks");
  // Residual epilogues stage the residual by direct loads one chunk ahead:
  // two staging buffers when the tile is staged in chunks.
  constexpr int kStageBufs = (RES && ECH < WTM) ? 2 : 1;
  constexpr int kEpiBytes = kStageBufs * NW * ECH * ORB;
  static_assert(kEpiBytes <= 2 * kStage, "epilogue staging fits in the K-step stages");

  // MXFP4: both stages' block scales (8 bytes per tile row) after the stages.
  // The x rows' region is rounded up to whole 128-row pieces (rows past the
  // tile are loaded clamped and never read).
  constexpr int kScRowsX = (BM + 127) / 128 * 128;
  constexpr int kScStage = MX ? (kScRowsX + BN) * 8 : 0;
  static_assert(!MX || BN % 128 == 0, "weight scale rows load in 1 KB pieces of 128 rows");
  // After the stages: folded LayerNorm -- (mu, r) of every tile row and
  // (c_n, d_n) of every tile column, written before the K loop and published
  // by its first barrier; EPI_RES_STATS -- each wave's (mean, M2) partial of
  // every tile row.
  constexpr int kFoldOff = 2 * kStage + 2 * kScStage;
  constexpr int kStatsOff = kFoldOff;
  constexpr int kExtraBytes = FOLD ? (BM + BN) * 8 : (STATS ? WAVES_N * BM * 8 : 0);
  constexpr int kSmem = kFoldOff + kExtraBytes;
  static_assert(kSmem <= 160 * 1024, "LDS of one workgroup");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem];

  const int64_t M = a.M;
  const int N = a.N, K = a.K;
  const int tilesM = (int)((M + BM - 1) / BM);
  const int tilesN = (N + BN - 1) / BN;
  const int nb = tilesM * tilesN;
  int bid = blockIdx.x;
  // Split-K: workgroup = (K slice, tile), the slice slowest.
  [[maybe_unused]] int split = 0;
  int Kl = K;
  if constexpr (SPLIT) {
    split = bid / nb;
    bid = bid % nb;
    Kl = KMAJ ? (int)(((int64_t)K + 64 * a.ksplit - 1) / (64 * a.ksplit) * 64) : K / a.ksplit;
  }
  if (bid >= nb) return;
  // XCD-aware remap: hardware deals ids round-robin over the XCDs.
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int q = nb / kXcds, rem = nb % kXcds;
  const int L = xcd * q + min(xcd, rem) + local;
  const int group_m = K >= 4 * N ? 2 : (N >= 4 * K ? 4 : 8);
  const int group = group_m * tilesN;
  const int g = L / group;
  const int first_m = g * group_m;
  const int gm = min(tilesM - first_m, group_m);
  const int within = L % group;
  const int tm = first_m + within % gm;
  const int tn = within / gm;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = lane & 31, lhalf = lane >> 5;

  // Direct-to-LDS tile loads.  One global_load_lds_dwordx4 fills 1 KB of LDS
  // (8 rows of 128 bytes), lane i writing bytes [16 i, 16 i + 16).  Lane i of
  // a wave therefore fetches row r = 8*rb + i/8 at the logical chunk that the
  // swizzle stores in physical chunk i%8: c = (i%8) ^ ((r >> 1) & 7), and
  // (r >> 1) & 7 = 4*(rb & 1) + i/16 with rb & 1 = wave & 1 (rb = wave + NW*j,
  // NW even).
  const int lr8 = lane >> 3;
  const int lchunk = ((lane & 7) ^ (((wave & 1) << 2) | (lane >> 4))) * 16;  // bytes
  // Each operand's loads address its tile's first row (a wave-uniform base
  // in scalar registers, advanced by a scalar add per K step) plus a 32-bit
  // per-lane offset of at most (BM - 1) rows: no vector instructions on
  // global addresses in the K loop.
  const int64_t rowb = (int64_t)K * EBN / EBD;  // bytes per operand row
  // contraction-major: bytes per contraction row of x ([K, M]) and of w ([K, N])
  [[maybe_unused]] const int64_t ldxb = (int64_t)M * 2, ldwb = (int64_t)N * 2;
  const unsigned char* const xbase =
      KMAJ ? (const unsigned char*)a.x + (int64_t)split * Kl * ldxb + m0 * 2
           : (const unsigned char*)a.x + m0 * rowb + (int64_t)split * Kl * EBN / EBD;
  const unsigned char* const wbase =
      KMAJ ? (const unsigned char*)a.w + (int64_t)split * Kl * ldwb + (int64_t)n0 * 2
           : (const unsigned char*)a.w + (int64_t)n0 * rowb + (int64_t)split * Kl * EBN / EBD;
  uint32_t xoff[XRB], woff[WRB];
  if constexpr (KMAJ) {
    // Block i of a wave: contraction rows 2 (wave + NW i) and + 1 of the K
    // step (lanes 0-31 and 32-63).  Lane i writes physical chunk i % 32 of
    // its row, so it fetches logical chunk (i % 32) ^ 4 (row % 4): tile
    // columns 8 c .. 8 c + 7, clamped into the operand (columns past M or N
    // are never stored).
#pragma unroll
    for (int i = 0; i < XRB; ++i) {
      const int rr = 2 * (wave + NW * i) + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (rr & 3));
      int64_t cx = m0 + 8 * c;
      cx = cx < M ? cx : M - 8;
      xoff[i] = (uint32_t)(rr * ldxb + (cx - m0) * 2);
      int64_t cw = (int64_t)n0 + 8 * c;
      cw = cw < N ? cw : N - 8;
      woff[i] = (uint32_t)(rr * ldwb + (cw - n0) * 2);
    }
  } else {
#pragma unroll
    for (int i = 0; i < XRB; ++i) {
      int64_t r = m0 + (int64_t)(wave + NW * i) * RPI + lr8;
      r = r < M ? r : M - 1;
      xoff[i] = (uint32_t)((r - m0) * rowb + lchunk);
    }
#pragma unroll
    for (int i = 0; i < WRB; ++i) {
      int r = n0 + (wave + NW * i) * RPI + lr8;
      r = r < N ? r : N - 1;
      woff[i] = (uint32_t)((int64_t)(r - n0) * rowb + lchunk);
    }
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_addr(smem);
  // MXFP4 scales of K step s: the tile's x rows then w rows, 8 bytes each, in
  // 1 KB direct loads of 128 rows (lane i: rows 2i, 2i + 1), one per wave.
  // Rows past the scale arrays' (even) row counts are clamped to the last
  // pair; those rows' outputs are never stored.
  [[maybe_unused]] const int64_t M2 = M + (M & 1);
  auto issue_scales = [&](int s, int buf) {
    if constexpr (MX) {
      constexpr int PX = kScRowsX / 128, PW = BN / 128;
      static_assert(PX + PW <= NW, "one scale piece per wave");
      if (wave_u < PX + PW) {
        const bool isx = wave_u < PX;
        const int piece = isx ? wave_u : wave_u - PX;
        int64_t r = (isx ? m0 : (int64_t)n0) + piece * 128 + 2 * lane;
        const int64_t rows2 = isx ? M2 : (int64_t)N;
        r = r < rows2 ? r : rows2 - 2;
        const uint8_t* src = (isx ? a.x_sc + (int64_t)s * M2 * 8 : a.w_sc + (int64_t)s * N * 8) + r * 8;
        const uint32_t dst = lds0 + (uint32_t)(2 * kStage + buf * kScStage + (isx ? 0 : kScRowsX * 8) + piece * 1024);
        lds_dma16(src, dst);
      }
    }
  };
  // Part p of np of K step kt's direct loads: the wave's XRB x row blocks
  // then its WRB w row blocks, numbered 0 .. XRB + WRB - 1, split into np
  // equal runs (the block scales go with part 0).
  auto issue_part = [&](int kt, int buf, int p, int np) {
    const uint32_t base = lds0 + (uint32_t)(buf * kStage);
    constexpr int NL = XRB + WRB;
    const int64_t xk = KMAJ ? (int64_t)kt * 64 * ldxb : (int64_t)kt * kRowBytes;
    const int64_t wk = KMAJ ? (int64_t)kt * 64 * ldwb : (int64_t)kt * kRowBytes;
    if constexpr (KMAJ) {
      const int64_t g0 = (int64_t)split * Kl + (int64_t)kt * 64;  // the step's first contraction row
      if (g0 + 64 > K) {
        // The step reaches past the contraction's end: rows at or past K
        // load zeros (whole-address form, one select per lane).
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          if (i < p * NL / np || i >= (p + 1) * NL / np) continue;
          const int ib = i < XRB ? i : i - XRB;
          const int rr = 2 * (wave_u + NW * ib) + (lane >> 5);
          const unsigned char* src = i < XRB ? xbase + xk + xoff[ib] : wbase + wk + woff[ib];
          if (g0 + rr >= K) src = g_zero_row + 16 * (lane & 31);
          lds_dma16(src, base + (uint32_t)(((i < XRB ? 0 : BM) + (wave_u + NW * ib) * RPI) * kRowBytes));
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (i < p * NL / np || i >= (p + 1) * NL / np) continue;
      if (i < XRB)
        lds_dma16s(xbase + xk, xoff[i], base + (uint32_t)((wave_u + NW * i) * RPI * kRowBytes));
      else
        lds_dma16s(wbase + wk, woff[i - XRB], base + (uint32_t)((BM + (wave_u + NW * (i - XRB)) * RPI) * kRowBytes));
    }
    if (p == 0) issue_scales(kt, buf);
  };
  auto issue_tile = [&](int kt, int buf) { issue_part(kt, buf, 0, 1); };
  // bf16: a K step's loads go out in three runs, ahead of the first three of
  // its four k sub-steps, not at once: a wave that issues all of them
  // back to back stalls at issue behind the address unit and starts its
  // MFMAs late (a loads + LDS + MFMA copy of the loop measured 8-12% faster
  // with the loads spread so; the 650M stack's GEMMs 6-8%).  The last run
  // still has a sub-step and a half to land before the barrier that ends the
  // K step.  The E4M3 and MXFP4 K steps hold 2-4x the flops per byte in fewer
  // MFMA cycles, and their loads need the whole step to land: spread over
  // their sub-steps they measured 10-50% slower, so they go out at once.
  constexpr int kParts = DT == kBF16 ? 3 : 1;

  // Fragment reads: row r of the tile, logical 16-byte chunk ch, stored at
  // physical chunk ch ^ ((r >> 1) & 7); every row this lane reads has
  // (r >> 1) & 7 = ((lane % 32) >> 1) & 7.  Sub-step kk covers the chunks
  // [2 FB kk, 2 FB (kk + 1)); lane half h takes FB consecutive ones.  A and B
  // fragments use the same chunk-to-k assignment, so the MFMA contracts
  // matching k.
  const int swz = (lrow >> 1) & 7;
  auto read_frag = [&](const unsigned char* rowp, int kk) -> frag_t {
    if constexpr (DT == kFP4) {
      // one MX block (32 E2M1 values, 16 bytes); the MFMA reads 4 registers
      const u32x4 v = *(const u32x4*)(rowp + (((kk * 2 + lhalf) ^ swz) * 16));
      return __builtin_bit_cast(frag_t, __builtin_shufflevector(v, u32x4{0u, 0u, 0u, 0u}, 0, 1, 2, 3, 4, 5, 6, 7));
    } else if constexpr (FB == 1) {
      return *(const frag_t*)(rowp + (((kk * 2 + lhalf) ^ swz) * 16));
    } else {
      const u32x4 lo = *(const u32x4*)(rowp + (((kk * 4 + lhalf * 2) ^ swz) * 16));
      const u32x4 hi = *(const u32x4*)(rowp + (((kk * 4 + lhalf * 2 + 1) ^ swz) * 16));
      return __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // Contraction-major fragment of tile columns R .. R + 31 at sub-step kk:
  // lanes 16 g + i (g = 0 .. 3) take column R + 16 (g % 2) + i, contraction
  // rows 16 kk + 8 (g / 2) + 0 .. 7 (two transposing reads of four rows);
  // the lane's address is row 16 kk + 8 (g / 2) + i / 4 (+ 4), columns
  // R + 16 (g % 2) + 4 (i % 4) .. + 3, whose row % 4 is i / 4.
  [[maybe_unused]] auto read_frag_km = [&](const unsigned char* op, int R, int kk) -> frag_t {
    if constexpr (KMAJ) {
      const int g = lane >> 4, i16 = lane & 15;
      const int col = R + 16 * (g & 1) + 4 * (i16 & 3);
      const int r = 16 * kk + 8 * (g >> 1) + (i16 >> 2);
      const unsigned char* p = op + r * (BM * 2) + (((col >> 3) ^ (4 * (i16 >> 2))) * 16) + (col & 7) * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * (BM * 2)));
      return __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return frag_t{};
    }
  };
  auto load_frags = [&](frag_t (&xf)[FM], frag_t (&wf)[FN], int buf, int kk) {
    const unsigned char* sx = smem + buf * kStage;
    const unsigned char* sw = sx + BM * kRowBytes;
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < FM; ++i) xf[i] = read_frag_km(sx, wm * WTM + i * 32, kk);
#pragma unroll
      for (int j = 0; j < FN; ++j) wf[j] = read_frag_km(sw, wn * WTN + j * 32, kk);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) xf[i] = read_frag(sx + (wm * WTM + i * 32 + lrow) * kRowBytes, kk);
#pragma unroll
      for (int j = 0; j < FN; ++j) wf[j] = read_frag(sw + (wn * WTN + j * 32 + lrow) * kRowBytes, kk);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // MXFP4 block scales of this lane's fragment rows for one K step: word
  // lhalf of a row's 8 bytes holds the scales of blocks lhalf, 2 + lhalf,
  // 4 + lhalf, 6 + lhalf, i.e. byte kk is the scale of sub-step kk's block.
  [[maybe_unused]] uint32_t xsc[MX ? FM : 1], wsc[MX ? FN : 1];
  auto load_scales = [&](int buf) {
    if constexpr (MX) {
      const unsigned char* sb = smem + 2 * kStage + buf * kScStage;
#pragma unroll
      for (int i = 0; i < FM; ++i) xsc[i] = *(const uint32_t*)(sb + (wm * WTM + i * 32 + lrow) * 8 + 4 * lhalf);
#pragma unroll
      for (int j = 0; j < FN; ++j) wsc[j] = *(const uint32_t*)(sb + (kScRowsX + wn * WTN + j * 32 + lrow) * 8 + 4 * lhalf);
    }
  };
  auto mfma_step_mx = [&](const frag_t (&xf)[FM], const frag_t (&wf)[FN], int kk) {
    if constexpr (MX) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          // cbsz = blgp = 4: both operands E2M1; scale bytes shifted to byte 0
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], acc[i][j], 4, 4, 0,
                                                                       (int)(wsc[j] >> (8 * kk)), 0,
                                                                       (int)(xsc[i] >> (8 * kk)));
    }
  };
  auto mfma_step = [&](const frag_t (&xf)[FM], const frag_t (&wf)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (DT == kE4M3)
          // cbsz = blgp = 0: both operands E4M3; block scales 127 = 2^0.
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], acc[i][j], 0, 0, 0, 127, 0, 127);
        else if constexpr (DT == kE5M2X)
          // blgp = 1: operand B (the x rows) E5M2; cbsz = 0: operand A (w) E4M3.
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], acc[i][j], 0, 1, 0, 127, 0, 127);
        else if constexpr (DT == kBF16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
      }
  };

  const int nk = Kl / kBK;
  issue_tile(0, 0);
  if constexpr (FOLD) {
    // Row statistics from the chunk partials of the x rows (K = the
    // LayerNorm's width), column constants from the prepared (c, d).
    // Thread t takes tile row t and tile column t (both loads in flight
    // together with the first K step's tile).
    static_assert(BM <= 64 * NW && BN <= 64 * NW, "one thread per tile row and per tile column");
    float2* rs = (float2*)(smem + kFoldOff);
    float2* cdl = rs + BM;
    // Every load is unconditional (indices clamped), so none sits behind a
    // branch that would wait for it, and all are in flight together.
    const int64_t mr = m0 + tid;
    const int nc = n0 + tid;
    const float2 cdv = a.ln_cd[nc < N ? nc : N - 1];
    const float2 st = ln_row_stats(a.ln_stats + (mr < M ? mr : M - 1), M, K, a.ln_eps);
    if (tid < BM) rs[tid] = mr < M ? st : make_float2(0.f, 1.f);
    if (tid < BN) cdl[tid] = nc < N ? cdv : make_float2(0.f, 0.f);
  }
  vm_wait_all();
  __syncthreads();
  if constexpr (FOLD) {
    // The accumulators start at -mu_m c_n + d_n / r_m, so that after the K
    // loop acc = x_m . W'_n - mu_m c_n + d_n / r_m and the epilogue only
    // scales row m by r_m.  One bf16 MFMA per 32x32 block forms it: every fp32
    // factor is split into three bf16 parts (f = f1 + f2 + f3 to 2^-24), and
    // the 16-long contraction holds the six leading cross products of each
    // term (lanes 0-31: k 0-7, the mu c term; lanes 32-63: k 8-15, d / r):
    //   k:      0      1      2      3      4      5      6, 7
    //   A[n]:  c1     c1     c2     c1     c3     c2     0   (d1 d1 d2 d1 d3 d2)
    //   B[m]: -mu1   -mu2   -mu1   -mu3   -mu1   -mu2    0   (s1 s2 s1 s3 s1 s2, s = 1/r)
    // bf16 x bf16 products are exact in fp32.
    const float2* rs = (const float2*)(smem + kFoldOff);
    const float2* cdl = rs + BM;
    auto split3 = [](float f, __bf16 (&p)[3]) {
      p[0] = (__bf16)f;
      const float r1 = f - (float)p[0];
      p[1] = (__bf16)r1;
      p[2] = (__bf16)(r1 - (float)p[1]);
    };
    auto frag6 = [](const __bf16 (&u)[3], const __bf16 (&v)[3], bool second) {
      // second = false: (u1 u1 u2 u1 u3 u2 0 0); true: (v1 v2 v1 v3 v1 v2 0 0)
      const __bf16 z = (__bf16)0.0f;
      return second ? bf16x8{v[0], v[1], v[0], v[2], v[0], v[1], z, z} : bf16x8{u[0], u[0], u[1], u[0], u[2], u[1], z, z};
    };
    bf16x8 af[FN], bfv[FM];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const float2 v = cdl[wn * WTN + 32 * j + lrow];
      __bf16 p[3];
      split3(lhalf ? v.y : v.x, p);
      af[j] = frag6(p, p, false);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const float2 v = rs[wm * WTM + 32 * i + lrow];
      __bf16 p[3];
      split3(lhalf ? 1.0f / v.y : -v.x, p);
      bfv[i] = frag6(p, p, true);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j], bfv[i], acc[i][j], 0, 0, 0);
  }
  if constexpr (DT == kFP4) {
    // One fragment set, as for E4M3, plus the K step's block scales.  This
    // lane's fragment-row LDS addresses per sub-step and its two scale-row
    // addresses are kept in registers and moved to the other stage by one add
    // each per K step (32-row blocks as immediate offsets), and each MFMA
    // takes sub-step kk's scale byte through its scale operand select, so the
    // loop spends no vector instructions on addresses or scale bytes.
    frag_t xf[FM], wf[FN];
    typedef const __attribute__((address_space(3))) u32x4* lds_u4_ptr;
    typedef const __attribute__((address_space(3))) uint32_t* lds_u1_ptr;
    uint32_t ax[KK], aw[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint32_t ch = (uint32_t)(((kk * 2 + lhalf) ^ swz) * 16);
      ax[kk] = lds0 + (uint32_t)((wm * WTM + lrow) * kRowBytes) + ch;
      aw[kk] = lds0 + (uint32_t)(BM * kRowBytes + (wn * WTN + lrow) * kRowBytes) + ch;
    }
    uint32_t asx = lds0 + (uint32_t)(2 * kStage + (wm * WTM + lrow) * 8 + 4 * lhalf);
    uint32_t asw = lds0 + (uint32_t)(2 * kStage + (kScRowsX + wn * WTN + lrow) * 8 + 4 * lhalf);
    int32_t to_other = kStage, sc_to_other = kScStage;
    auto mfma_sel = [&](int i, int j, auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      // cbsz = blgp = 4: both operands E2M1; scale byte kk of each register
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], acc[i][j], 4, 4, kk, (int)wsc[j], kk,
                                                                   (int)xsc[i]);
    };
    auto sub_step = [&](int kt, int cur, bool more, auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      __builtin_amdgcn_sched_barrier(0);
      if (more && kk < kParts) issue_part(kt + 1, cur ^ 1, kk, kParts);
      const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wf[j] = __builtin_bit_cast(frag_t, __builtin_shufflevector(*(lds_u4_ptr)(uintptr_t)(aw[kk] + j * 32 * kRowBytes),
                                                                   z4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int i = 0; i < FM; ++i)
        xf[i] = __builtin_bit_cast(frag_t, __builtin_shufflevector(*(lds_u4_ptr)(uintptr_t)(ax[kk] + i * 32 * kRowBytes),
                                                                   z4, 0, 1, 2, 3, 4, 5, 6, 7));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma_sel(i, j, kkc);
    };
    static_assert(KK == 4, "four 64-value sub-steps per MXFP4 K step");
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
#pragma unroll
      for (int i = 0; i < FM; ++i) xsc[i] = *(lds_u1_ptr)(uintptr_t)(asx + i * 32 * 8);
#pragma unroll
      for (int j = 0; j < FN; ++j) wsc[j] = *(lds_u1_ptr)(uintptr_t)(asw + j * 32 * 8);
      sub_step(kt, cur, more, std::integral_constant<int, 0>{});
      sub_step(kt, cur, more, std::integral_constant<int, 1>{});
      sub_step(kt, cur, more, std::integral_constant<int, 2>{});
      sub_step(kt, cur, more, std::integral_constant<int, 3>{});
      __builtin_amdgcn_sched_barrier(0);
      vm_wait_all();
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        ax[kk] += (uint32_t)to_other;
        aw[kk] += (uint32_t)to_other;
      }
      asx += (uint32_t)sc_to_other;
      asw += (uint32_t)sc_to_other;
      to_other = -to_other;
      sc_to_other = -sc_to_other;
    }
  } else if constexpr (DT == kE4M3 || DT == kE5M2X) {
    // One fragment set (8 registers per 32-byte fragment; a second set would
    // not fit beside the accumulators at two waves per SIMD): the other wave
    // on the SIMD multiplies while this one waits for its LDS reads.  The
    // LDS addresses of this lane's first x and w fragment rows, per sub-step
    // and 16-byte half, are kept in registers and moved to the other stage by
    // one add each per K step; the 32-row blocks are immediate offsets.
    frag_t xf[FM], wf[FN];
    typedef const __attribute__((address_space(3))) u32x4* lds_u4_ptr;
    uint32_t ax[KK][2], aw[KK][2];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ch = (uint32_t)(((kk * 4 + lhalf * 2 + h) ^ swz) * 16);
        ax[kk][h] = lds0 + (uint32_t)((wm * WTM + lrow) * kRowBytes) + ch;
        aw[kk][h] = lds0 + (uint32_t)(BM * kRowBytes + (wn * WTN + lrow) * kRowBytes) + ch;
      }
    int32_t to_other = kStage;  // byte distance to the other stage
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        if (more && kk < kParts) issue_part(kt + 1, cur ^ 1, kk, kParts);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x4 lo = *(lds_u4_ptr)(uintptr_t)(aw[kk][0] + j * 32 * kRowBytes);
          const u32x4 hi = *(lds_u4_ptr)(uintptr_t)(aw[kk][1] + j * 32 * kRowBytes);
          wf[j] = __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const u32x4 lo = *(lds_u4_ptr)(uintptr_t)(ax[kk][0] + i * 32 * kRowBytes);
          const u32x4 hi = *(lds_u4_ptr)(uintptr_t)(ax[kk][1] + i * 32 * kRowBytes);
          xf[i] = __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(xf, wf);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Next tile landed for every wave; every wave is done reading this one.
      vm_wait_all();
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ax[kk][h] += (uint32_t)to_other;
          aw[kk][h] += (uint32_t)to_other;
        }
      to_other = -to_other;
    }
  } else if constexpr (FM * FN > 8) {
    // Large wave tiles (160 x 64: 160 accumulator registers): one fragment
    // set, as for E4M3.  The fragment addresses of each (stage, sub-step)
    // are computed once (the 32-row blocks then differ by immediate offsets)
    // and the loop is unrolled over the two stages, so a K step spends no
    // vector instructions on LDS addresses.
    frag_t xf[FM], wf[FN];
    typedef const __attribute__((address_space(3))) frag_t* lds_frag_ptr;
    uint32_t ax[2][KK], aw[2][KK];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint32_t ch = (uint32_t)(((kk * 2 + lhalf) ^ swz) * 16);
        ax[b][kk] = lds0 + (uint32_t)(b * kStage + (wm * WTM + lrow) * kRowBytes) + ch;
        aw[b][kk] = lds0 + (uint32_t)(b * kStage + BM * kRowBytes + (wn * WTN + lrow) * kRowBytes) + ch;
        // kept whole in registers (not re-derived from a shared part per step)
        asm volatile("" : "+v"(ax[b][kk]), "+v"(aw[b][kk]));
      }
    auto kstep = [&](int kt, auto stage) {
      constexpr int cur = decltype(stage)::value;
      const bool more = kt + 1 < nk;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        if (more && kk < kParts) issue_part(kt + 1, cur ^ 1, kk, kParts);
        // the weight fragments first: the sub-step's first MFMAs wait for three
        // of the seven reads instead of six
#pragma unroll
        for (int j = 0; j < FN; ++j) wf[j] = *(lds_frag_ptr)(uintptr_t)(aw[cur][kk] + j * 32 * kRowBytes);
#pragma unroll
        for (int i = 0; i < FM; ++i) xf[i] = *(lds_frag_ptr)(uintptr_t)(ax[cur][kk] + i * 32 * kRowBytes);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(xf, wf);
      }
      __builtin_amdgcn_sched_barrier(0);
      vm_wait_all();
      __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
      kstep(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < nk) kstep(kt + 1, std::integral_constant<int, 1>{});
    }
  } else {
  frag_t xf[2][FM], wf[2][FN];
  load_frags(xf[0], wf[0], 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (more && kk < kParts) issue_part(kt + 1, cur ^ 1, kk, kParts);
      if (kk + 1 < KK) {
        load_frags(xf[(kk + 1) & 1], wf[(kk + 1) & 1], cur, kk + 1);
      } else if (more) {
        // Next tile landed for every wave, and every wave is done reading this
        // one; its first fragments load under the last sub-step's MFMAs.
        vm_wait_all();
        __syncthreads();
        load_frags(xf[0], wf[0], cur ^ 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(xf[kk & 1], wf[kk & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  }

  if constexpr (SPLIT) {
    // Split-K partial sums straight from the accumulators: register 4 gq + e
    // of block (i, j) is row mw + 32 i + lrow, column nw + 32 j + 8 gq +
    // 4 lhalf + e; 16-byte fp32 stores, no staging.
    const int64_t mwf = m0 + wm * WTM;
    const int nwf = n0 + wn * WTN;
    float* out = a.y32 + (int64_t)split * M * N;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = mwf + i * 32 + lrow;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = nwf + j * 32 + 8 * gq + 4 * lhalf;
          if (n < N)
            *(f32x4*)(out + m * N + n) =
                f32x4{acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]};
        }
    }
    return;
  }

  // ------------------------------------------------------------ epilogue
  // Each wave stages its (WTM x WTN) result tile in its own LDS region (free
  // once every wave is past the K loop) -- all of it, or ECH-row chunks when
  // the whole tile does not fit -- so that global memory is written (and, for
  // the residual, read) in full rows with 16-byte lanes.  The regions are
  // wave-private, so after the barrier that ends the K loop the epilogue
  // needs no further barrier.  The residual of a chunk arrives by direct
  // loads into the staging buffer, issued one chunk ahead.  Staged rows hold CPR 16-byte
  // chunks, chunk c of row r stored at c ^ ((r / RPW) % CPR), which spreads
  // the row-per-lane accesses of the MFMA layout over the banks.  E4M3
  // operands: the accumulators are first divided by s_x s_w.  E4M3 output:
  // the GELU values are cast with the output's scale, and their amax (before
  // the cast) is recorded.
  constexpr int CPR = ORB / 16;                   // 16-byte chunks per staged row
  constexpr int RPW = CPR >= 16 ? 1 : 16 / CPR;   // staged rows per 256-byte bank window
  constexpr int PASSES = ECH * CPR / 64;          // 16-byte transfers per lane per chunk
  constexpr int EPC = 16 * WTN / ORB;             // output elements per chunk
  __syncthreads();
  auto stage_at = [&](int c0) {
    return smem + ((c0 / ECH) % kStageBufs) * (NW * ECH * ORB) + wave * (ECH * ORB);
  };
  auto soff = [&](int row, int chunk) { return row * ORB + ((chunk ^ ((row / RPW) & (CPR - 1))) * 16); };
  const int64_t mw = m0 + wm * WTM;
  const int nw = n0 + wn * WTN;
  [[maybe_unused]] const float2* rs = (const float2*)(smem + kFoldOff);
  // Residual rows c0 .. c0 + ECH - 1 of the wave tile into their staging
  // buffer: one 1 KB direct load fills 1024 / (WTN * 2) rows, lane i writing
  // physical chunk i % CPR of its row, i.e. the residual's logical chunk
  // (i % CPR) ^ ((row / RPW) % CPR).  Rows past M are clamped (never stored).
  auto res_load = [&](int c0) {
    if constexpr (RES) {
      static_assert(OES == 2 && (ECH * WTN * 2) % 1024 == 0, "whole 1 KB loads of bf16 rows");
      constexpr int RPL = 1024 / (WTN * 2);  // staged rows per direct load
      if (nw >= N) return;
      const uint32_t base = lds0 + (uint32_t)(((c0 / ECH) % kStageBufs) * (NW * ECH * ORB) + wave_u * (ECH * ORB));
#pragma unroll
      for (int k = 0; k < ECH / RPL; ++k) {
        const int row = k * RPL + lane / CPR;
        int64_t m = mw + c0 + row;
        m = m < M ? m : M - 1;
        const int ch = (lane % CPR) ^ ((row / RPW) & (CPR - 1));
        lds_dma16(a.res + m * N + nw + ch * 8, base + (uint32_t)(k * 1024));
      }
    }
  };
  res_load(0);
  const bf16_t* __restrict__ bias = a.bias;
  float dq = 1.0f;
  if constexpr (DT == kE4M3 || DT == kE5M2X) dq = 1.0f / (a.x_scale[0] * a.w_scale[0]);
  float oscale = 1.0f, amax = 0.0f;
  if constexpr (OUT8) oscale = a.y8_scale[0];
  // Bias of this lane's output columns nw + 32 j + 8 gq + 4 lhalf + 0..3,
  // loaded once per tile (zeros without a bias or past N; N is a multiple of
  // 64, so a wave's 64 columns are all in range or all out).
  static_assert(FN == 2, "the epilogue assumes 64-column wave tiles");
  u32x2 bcache[FN][4];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int n = nw + j * 32 + 8 * gq + 4 * lhalf;
      bcache[j][gq] = (!FOLD && bias && nw < N) ? *(const u32x2*)(bias + n) : u32x2{0u, 0u};
    }

  // Rotary epilogue: the positions of this lane's rows (one per 32-row
  // block), loaded together before the first block needs one.
  [[maybe_unused]] int rpos[FM];
  if constexpr (ROPE) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = mw + i * 32 + lrow;
      rpos[i] = a.pos[m < M ? m : M - 1];
    }
  }

#pragma unroll
  for (int c0 = 0; c0 < WTM; c0 += ECH) {
  unsigned char* stage = stage_at(c0);
  if constexpr (RES) {
    // This chunk's residual has landed (and the previous chunk's stores,
    // which read the other buffer, have been issued); fetch the next one.
    vm_wait_all();
    if (c0 + ECH < WTM) res_load(c0 + ECH);
  }

#pragma unroll
  for (int i = c0 / 32; i < (c0 + ECH) / 32; ++i) {
    const int row = i * 32 - c0 + lrow;  // row within the staged chunk
    const int64_t m = mw + i * 32 + lrow;
    const int64_t mc = m < M ? m : M - 1;
    // folded LayerNorm: the accumulators hold (h_m . W_n^T + b_n) / r_m
    float osc = dq;
    if constexpr (FOLD) osc = rs[wm * WTM + i * 32 + lrow].y;
    if constexpr (ROPE) {
      int p = rpos[i];
      p = p < 0 ? 0 : (p < a.max_positions ? p : a.max_positions - 1);
      // The wave's 64 columns are one head's q, k or v (c = 0, 1, 2): dims
      // d = 8 gq + 4 lhalf + e of this lane pair with d + 32.  Rotation
      // factors (cos, sin) of row position p for those 16 dims, loaded at once.
      const int c = (nw % 192) / 64;
      float4 rc[4][2];
      if (c < 2) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const float4* cs = (const float4*)(a.rope + (int64_t)p * 32 + 8 * gq + 4 * lhalf);
          rc[gq][0] = cs[0];
          rc[gq][1] = cs[1];
        }
      }
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int cl = 8 * gq + 4 * lhalf;  // local column of the low half
        float lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = acc[i][0][4 * gq + e] * osc;
          hi[e] = acc[i][1][4 * gq + e] * osc;
        }
        if constexpr (!FOLD) {
          const u32x2 bl = bcache[0][gq], bh = bcache[1][gq];
          lo[0] += bflo(bl[0]); lo[1] += bfhi(bl[0]); lo[2] += bflo(bl[1]); lo[3] += bfhi(bl[1]);
          hi[0] += bflo(bh[0]); hi[1] += bfhi(bh[0]); hi[2] += bflo(bh[1]); hi[3] += bfhi(bh[1]);
        }
        if (c < 2) {
          const float cs_[4] = {rc[gq][0].x, rc[gq][0].z, rc[gq][1].x, rc[gq][1].z};
          const float sn_[4] = {rc[gq][0].y, rc[gq][0].w, rc[gq][1].y, rc[gq][1].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = lo[e], x1 = hi[e];
            lo[e] = x0 * cs_[e] - x1 * sn_[e];
            hi[e] = x1 * cs_[e] + x0 * sn_[e];
          }
        }
        *(u32x2*)(stage + soff(row, cl / 8) + 8 * lhalf) = u32x2{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3])};
        *(u32x2*)(stage + soff(row, cl / 8 + 4) + 8 * lhalf) = u32x2{pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3])};
      }
    } else if constexpr (OUTMX) {
      // GELU straight to MXFP4: the 32 columns of block j of this row are the
      // 16 of this lane (8 gq + 4 lhalf + e) and the 16 of lane l ^ 32; one
      // exchange gives the block amax, each lane stages its codes (two bytes
      // per gq, at byte 16 j + 4 gq + 2 lhalf of the staged row) and the
      // lhalf = 0 lane writes the block's scale.
      const int64_t M2 = M + (M & 1);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float v[4][4];
        float am = 0.f;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const u32x2 bb = bcache[j][gq];
          v[gq][0] = acc[i][j][4 * gq + 0] + bflo(bb[0]);
          v[gq][1] = acc[i][j][4 * gq + 1] + bfhi(bb[0]);
          v[gq][2] = acc[i][j][4 * gq + 2] + bflo(bb[1]);
          v[gq][3] = acc[i][j][4 * gq + 3] + bfhi(bb[1]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[gq][e] = gelu(v[gq][e]);
            am = fmaxf(am, fabsf(v[gq][e]));
          }
        }
        am = fmaxf(am, __shfl_xor(am, 32));
        const int ex = mx_block_exponent(am);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint32_t c2 = e2m1_pair(v[gq][0], v[gq][1], ex) | (e2m1_pair(v[gq][2], v[gq][3], ex) << 8);
          *(uint16_t*)(stage + soff(row, j) + 4 * gq + 2 * lhalf) = (uint16_t)c2;
        }
        const int nb = nw + j * 32;
        if (lhalf == 0 && m < M && nb < N) a.y_sc[mx_scale_offset(m, nb / 32, M2)] = (uint8_t)(ex + 127);
      }
    } else {
      bool zero_row = false;
      if constexpr (RES) zero_row = a.zero_pad_rows && a.pos[mc] < 0;
      [[maybe_unused]] float sv[STATS ? 32 : 1];  // EPI_RES_STATS: this lane's 32 stored values of the row
      bool count_row = false;  // E4M3 output: row enters the amax (in range, not padding)
      if constexpr (OUT8) count_row = m < M && (!a.zero_pad_rows || a.pos == nullptr || a.pos[mc] >= 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int cl = j * 32 + 8 * gq + 4 * lhalf;
          const int n = nw + cl;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * gq + e] * osc;
          if constexpr (!FOLD) {
            const u32x2 bb = bcache[j][gq];
            v[0] += bflo(bb[0]); v[1] += bfhi(bb[0]); v[2] += bflo(bb[1]); v[3] += bfhi(bb[1]);
          }
          if constexpr (EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_LN || OUT8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu(v[e]);
          }
          if constexpr (OUT8) {
            const float vm = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
            if (count_row && n < N) amax = fmaxf(amax, vm);
            // four consecutive E4M3 bytes at byte cl of the staged row
            *(uint32_t*)(stage + soff(row, cl / 16) + (cl % 16)) = pack_e4m3x4(v, oscale);
          } else {
            unsigned char* sp = stage + soff(row, cl / 8) + 8 * lhalf;
            if constexpr (RES) {
              const u32x2 rr = *(const u32x2*)sp;
              v[0] += bflo(rr[0]); v[1] += bfhi(rr[0]); v[2] += bflo(rr[1]); v[3] += bfhi(rr[1]);
              if (zero_row) v[0] = v[1] = v[2] = v[3] = 0.f;
            }
            const u32x2 packed = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
            *(u32x2*)sp = packed;
            if constexpr (STATS) {
              sv[16 * j + 4 * gq + 0] = bflo(packed[0]);
              sv[16 * j + 4 * gq + 1] = bfhi(packed[0]);
              sv[16 * j + 4 * gq + 2] = bflo(packed[1]);
              sv[16 * j + 4 * gq + 3] = bfhi(packed[1]);
            }
          }
        }
      }
      if constexpr (STATS) {
        // LayerNorm partial of the 64 stored values of this row in this
        // wave's columns: the lane's leaf, then the lane pair (lhalf 0, 1).
        LnPart p = nw < N ? ln_leaf(sv) : LnPart{0.f, 0.f, 0.f};
        const LnPart o{__shfl_xor(p.n, 32), __shfl_xor(p.m, 32), __shfl_xor(p.M2, 32)};
        p = lhalf ? ln_combine(o, p) : ln_combine(p, o);
        if (lhalf == 0) {
          float* ex = (float*)(smem + kStatsOff);
          const int r = wm * WTM + i * 32 + lrow;
          ex[2 * (wn * BM + r)] = p.m;
          ex[2 * (wn * BM + r) + 1] = p.M2;
        }
      }
    }
  }

#pragma unroll 4
  for (int p = 0; p < PASSES; ++p) {
    const int idx = p * 64 + lane, row = idx / CPR, ch = idx % CPR;
    const int64_t m = mw + c0 + row;
    const int n = nw + ch * EPC;
    if (m >= M || n >= N) continue;
    const u32x4 v = *(const u32x4*)(stage + soff(row, ch));
    if constexpr (ROPE) {
      if (a.zero_pad_rows && a.pos[m] < 0) continue;  // padding row of a bshd batch: never attended
      const int heads = N / 192;
      const int head = n / 192, c = (n % 192) / 64, d = n % 64;
      *(u32x4*)(a.y + (((int64_t)c * heads + head) * M + m) * kHeadDim + d) = v;
    } else if constexpr (OUT8) {
      __builtin_nontemporal_store(v, (u32x4*)(a.y8 + m * N + n));
    } else if constexpr (OUTMX) {
      __builtin_nontemporal_store(v, (u32x4*)(a.y8 + m * (N / 2) + n / 2));
    } else if constexpr (NT_OUT) {
      __builtin_nontemporal_store(v, (u32x4*)(a.y + m * N + n));
    } else {
      *(u32x4*)(a.y + m * N + n) = v;
    }
  }
  }
  if constexpr (OUT8) {
    __shared__ float red[NW];
    record_amax_block<NW>(a.y8_amax, amax, red);
  }
  if constexpr (STATS) {
    // The tile's chunk partial of every row: waves ((0, 1), (2, 3)) of the
    // row's wave-row, written as (mean, M2) to chunk n0 / 256.  The barrier
    // waits for the LDS writes only, not for the output stores in flight.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    const float* ex = (const float*)(smem + kStatsOff);
    for (int r = tid; r < BM; r += 64 * NW) {
      const int64_t m = m0 + r;
      if (m >= M) continue;
      LnPart w4[WAVES_N];
#pragma unroll
      for (int q = 0; q < WAVES_N; ++q)
        w4[q] = n0 + q * WTN < N ? LnPart{64.f, ex[2 * (q * BM + r)], ex[2 * (q * BM + r) + 1]} : LnPart{0.f, 0.f, 0.f};
      static_assert(!STATS || (WAVES_N == 4 && WTN == 64), "four 64-column leaves pairs per chunk");
      const LnPart c = ln_combine(ln_combine(w4[0], w4[1]), ln_combine(w4[2], w4[3]));
      a.stats_out[(int64_t)(n0 / 256) * M + m] = make_float2(c.m, c.M2);
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, int DT>
hipError_t run(const GemmArgs& a, hipStream_t st) {
  const int64_t tilesM = (a.M + BM - 1) / BM;
  const int64_t tilesN = (a.N + BN - 1) / BN;
  const int64_t nb = tilesM * tilesN * (EPI == EPI_F32_SPLIT || EPI == EPI_F32_SPLIT_KM ? a.ksplit : 1);
  hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI, DT>), dim3((unsigned)nb), dim3(64 * WM * WN), 0, st, a);
  return hipGetLastError();
}

// Compute units of the current device.
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// The tile shape the dispatch picks for an M x N output, 320-row tiles when
// they need no more rows of rounds than 256-row ones (time ~ rounds x tile
// rows; on a tie the taller tiles, fewer of them), and the rounds of
// workgroups over the compute units it then runs.
struct TileChoice {
  bool tall;
  int64_t rounds;
};
TileChoice tile_choice(int64_t M, int32_t N) {
  const int64_t tilesN = (N + 255) / 256;
  const int64_t cus = device_cus();
  const int64_t r256 = ((M + 255) / 256 * tilesN + cus - 1) / cus;
  const int64_t r320 = ((M + 319) / 320 * tilesN + cus - 1) / cus;
  const bool tall = r320 * 320 <= r256 * 256;
  return TileChoice{tall, tall ? r320 : r256};
}

template <int EPI>
hipError_t dispatch(const GemmArgs& a, hipStream_t st) {
  if constexpr (EPI == EPI_F32_SPLIT) {
    // split-K partial products (the backward's weight gradients): bf16, or
    // E5M2 x E4M3 (raw products; the reduction dequantises)
    if (a.ksplit < 1 || !a.y32) return hipErrorInvalidValue;
    if (a.dtype == kE5M2X) {
      if (a.K % (128 * a.ksplit)) return hipErrorInvalidValue;
      return run<256, 256, 2, 4, EPI, kE5M2X>(a, st);
    }
    if (a.dtype != kBF16 || a.K % (64 * a.ksplit)) return hipErrorInvalidValue;
    return run<256, 256, 2, 4, EPI, kBF16>(a, st);
  } else if constexpr (EPI == EPI_F32_SPLIT_KM) {
    // contraction-major split-K products (the linears' weight gradients)
    if (a.ksplit < 1 || !a.y32 || a.dtype != kBF16 || a.M % 64 || a.N % 64 || a.K < 0) return hipErrorInvalidValue;
    return run<256, 256, 2, 4, EPI, kBF16>(a, st);
  } else if constexpr (EPI == EPI_QKV_ROPE_LN || EPI == EPI_BIAS_GELU_LN || EPI == EPI_RES_STATS) {
    if (a.dtype != kBF16) return hipErrorInvalidValue;
    if (EPI == EPI_RES_STATS ? !a.stats_out : (!a.ln_stats || !a.ln_cd)) return hipErrorInvalidValue;
    return tile_choice(a.M, a.N).tall ? run<320, 256, 2, 4, EPI, kBF16>(a, st) : run<256, 256, 2, 4, EPI, kBF16>(a, st);
  } else {
  // 8 waves (two per SIMD, so one wave's LDS reads overlap the other's MFMAs)
  // over 256x256 tiles (128x64 per wave), or 320x256 tiles (160x64 per wave)
  // when those need fewer rounds of workgroups over the compute units: time
  // ~ rounds x tile rows (N = 1280 at T = 32293: 3 x 256 vs 2 x 320); on a
  // tie the 320-row tiles win (fewer tiles, so fewer prologues and
  // epilogues: N = 5120, 8 x 320 vs 10 x 256).  Each output element
  // accumulates the same K order in either shape, so results do not depend
  // on the choice.
  const bool tall = tile_choice(a.M, a.N).tall;
  if (a.dtype == kE5M2X) {
    // the backward's data-gradient GEMM: plain product, bias epilogue only
    if constexpr (EPI == EPI_BIAS)
      return tall ? run<320, 256, 2, 4, EPI, kE5M2X>(a, st) : run<256, 256, 2, 4, EPI, kE5M2X>(a, st);
    else return hipErrorInvalidValue;
  }
  if constexpr (EPI == EPI_BIAS_GELU_MX) {
    if (a.dtype != kFP4) return hipErrorInvalidValue;
  } else if (a.dtype == kE4M3) {
    return tall ? run<320, 256, 2, 4, EPI, kE4M3>(a, st) : run<256, 256, 2, 4, EPI, kE4M3>(a, st);
  }
  if constexpr (EPI == EPI_BIAS_GELU_E4M3) {
    if (a.dtype == kFP4) return hipErrorInvalidValue;
  } else {
    if (a.dtype == kFP4) return tall ? run<320, 256, 2, 4, EPI, kFP4>(a, st) : run<256, 256, 2, 4, EPI, kFP4>(a, st);
  }
  if constexpr (EPI == EPI_BIAS_GELU_E4M3 || EPI == EPI_BIAS_GELU_MX) return hipErrorInvalidValue;
  else return tall ? run<320, 256, 2, 4, EPI, kBF16>(a, st) : run<256, 256, 2, 4, EPI, kBF16>(a, st);
  }
}

// Matrix-core rate probe: each wave runs `iters` rounds of four independent
// chains of v_mfma_f32_32x32x16_bf16 on register operands that cycle through
// four pseudo-random sets (every MFMA sees new bits, as in a real GEMM, so the
// clock settles where real operands put it).  Nothing but the MFMAs is in the
// loop; one lane writes a value so the work is kept.
__global__ __launch_bounds__(256) void k_mfma_peak(int32_t iters, float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63, wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  bf16x8 av[4], bv[4];
  uint32_t h = lane * 2654435761u + wid * 40503u + 12345u;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h = h * 1664525u + 1013904223u;
      // values in [-2, 2): sign, exponent and mantissa bits all vary
      av[q][e] = (__bf16)((float)(int32_t)(h >> 8) * (1.0f / 4194304.0f));
      h = h * 1664525u + 1013904223u;
      bv[q][e] = (__bf16)((float)(int32_t)(h >> 8) * (1.0f / 4194304.0f));
    }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[(q + c) & 3], bv[q], acc[c], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) t += acc[c][r];
  if (lane == 0) sink[wid] = t;
}

// a = GELU(z), 8 values per thread: the fc1 epilogue's GELU on values a
// training forward keeps as bf16 (its backward takes z).
__global__ __launch_bounds__(256) void k_gelu_fwd(const bf16_t* __restrict__ z, bf16_t* __restrict__ a, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const u32x4 v = *(const u32x4*)(z + 8 * i);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf2(gelu(bflo(v[e])), gelu(bfhi(v[e])));
  *(u32x4*)(a + 8 * i) = o;
}

}  // namespace

hipError_t launch_gelu_fwd(const bf16_t* z, bf16_t* a, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_gelu_fwd, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, z, a, n8);
  return hipGetLastError();
}

hipError_t launch_mfma_peak(int32_t iters, int32_t blocks, float* sink, hipStream_t st) {
  if (iters <= 0 || blocks <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_peak, dim3((unsigned)blocks), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

int32_t mfma_peak_blocks() { return 2 * device_cus(); }

int64_t gemm_rounds(int64_t M, int32_t N) { return M > 0 && N > 0 ? tile_choice(M, N).rounds : 0; }

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  const int kb = a.dtype == kFP4 ? 2 * kRowBytes : (a.dtype == kE4M3 || a.dtype == kE5M2X ? kRowBytes : kRowBytes / 2);
  // the contraction-major product takes any contraction length (rows past
  // it load as zeros)
  if ((epi != EPI_F32_SPLIT_KM && a.K % kb != 0) || a.N % 64 != 0) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_BIAS: return dispatch<EPI_BIAS>(a, st);
    case EPI_BIAS_GELU: return dispatch<EPI_BIAS_GELU>(a, st);
    case EPI_BIAS_RESIDUAL: return dispatch<EPI_BIAS_RESIDUAL>(a, st);
    case EPI_QKV_ROPE: return dispatch<EPI_QKV_ROPE>(a, st);
    case EPI_BIAS_GELU_E4M3: return dispatch<EPI_BIAS_GELU_E4M3>(a, st);
    case EPI_BIAS_GELU_MX: return dispatch<EPI_BIAS_GELU_MX>(a, st);
    case EPI_F32_SPLIT: return dispatch<EPI_F32_SPLIT>(a, st);
    case EPI_F32_SPLIT_KM: return dispatch<EPI_F32_SPLIT_KM>(a, st);
    case EPI_QKV_ROPE_LN: return dispatch<EPI_QKV_ROPE_LN>(a, st);
    case EPI_BIAS_GELU_LN: return dispatch<EPI_BIAS_GELU_LN>(a, st);
    case EPI_RES_STATS: return dispatch<EPI_RES_STATS>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace esm
