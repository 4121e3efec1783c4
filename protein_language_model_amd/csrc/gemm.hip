// bf16 MFMA GEMM for gfx950 with fused epilogues:  y = epi(x[M,K] . w[N,K]^T + b)
//
// The four linears of a pre-LN encoder layer ([BIO-ACC] 3.1: QKV projection,
// attention output projection, fc1, fc2; [TE-RU] LayerNormLinear / LayerNormMLP)
// are all "both operands K-contiguous" products, so both MFMA operands are read
// from LDS as 16-byte runs along K.
//
// Design (CDNA4):
//  * 256 threads = 4 waves in a WAVES_M x WAVES_N grid; each wave owns a
//    (BM/WAVES_M) x (BN/WAVES_N) tile built from 32x32 blocks of
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
//  * The weight is MFMA operand A and the activations operand B, so lane l of
//    a 32x32 block holds output row m = l%32 and columns
//    n = 8*(r/4) + 4*(l/32) + r%4 (r = 0..15): four consecutive columns per
//    register group.  Columns j and j+32 of a 64-wide group sit in the same
//    lane and register of two adjacent blocks, which is what the rotary
//    epilogue needs ([TE-ESM2] 旋转位置编码集成: rotate-half pairs (i, i+32)).
//  * K step 64; tiles live in LDS twice (double buffer) with a 16-byte-chunk XOR
//    swizzle (chunk c of row r stored at c ^ (r & 7)); the next K step is
//    fetched from global memory into registers while the current one is
//    multiplied, so one barrier per K step suffices.
//  * Rows beyond M and weight rows beyond N are clamped on load (never read out
//    of bounds) and skipped on store.
//  * Workgroup ids are remapped so consecutive tiles land on one XCD (ids are
//    dealt round-robin over the 8 XCDs), then grouped GROUP_M row-tiles at a
//    time so a row panel of x and the weight panels stay in that XCD's L2.
#include "common.h"

namespace esm {

namespace {

constexpr int kBK = 64;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

__device__ __forceinline__ float gelu_erf(float z) {
  // Exact GELU z * Phi(z) ([BIO-ACC] 2.1 names the fused activation; the erf
  // form is the definition of GELU).
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs a) {
  constexpr int WTM = BM / WAVES_M;
  constexpr int WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int XCH = BM * 8 / 256;  // 16-byte chunks of x per thread per K step
  constexpr int WCH = BN * 8 / 256;
  static_assert(WAVES_M * WAVES_N == 4, "4 waves");
  static_assert(EPI != EPI_QKV_ROPE || (FN % 2 == 0 && WTN % 64 == 0), "rotary pairs need 64-wide wave columns");

  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(BM + BN) * kBK];

  const int64_t M = a.M;
  const int N = a.N, K = a.K;
  const int tilesM = (int)((M + BM - 1) / BM);
  const int tilesN = (N + BN - 1) / BN;
  const int nb = tilesM * tilesN;
  const int bid = blockIdx.x;
  if (bid >= nb) return;
  // XCD-aware remap: hardware deals ids round-robin over the XCDs.
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int q = nb / kXcds, rem = nb % kXcds;
  const int L = xcd * q + min(xcd, rem) + local;
  const int group = kGroupM * tilesN;
  const int g = L / group;
  const int first_m = g * kGroupM;
  const int gm = min(tilesM - first_m, kGroupM);
  const int within = L % group;
  const int tm = first_m + within % gm;
  const int tn = within / gm;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const bf16_t* __restrict__ X = a.x;
  const bf16_t* __restrict__ W = a.w;

  u32x4 xr[XCH], wr[WCH];
  const int crow = tid >> 3, cchk = tid & 7;
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      int64_t r = m0 + crow + 32 * i;
      r = r < M ? r : M - 1;
      xr[i] = *(const u32x4*)(X + r * K + k0 + cchk * 8);
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      int r = n0 + crow + 32 * i;
      r = r < N ? r : N - 1;
      wr[i] = *(const u32x4*)(W + (int64_t)r * K + k0 + cchk * 8);
    }
  };
  auto sstore = [&](int buf) {
    bf16_t* sx = smem[buf];
    bf16_t* sw = smem[buf] + BM * kBK;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      int r = crow + 32 * i;
      *(u32x4*)(sx + r * kBK + ((cchk ^ (r & 7)) * 8)) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      int r = crow + 32 * i;
      *(u32x4*)(sw + r * kBK + ((cchk ^ (r & 7)) * 8)) = wr[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const bf16_t* sx = smem[cur];
    const bf16_t* sw = smem[cur] + BM * kBK;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = kk * 2 + lhalf;
      bf16x8 xf[FM], wf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        int r = wm * WTM + i * 32 + lrow;
        xf[i] = *(const bf16x8*)(sx + r * kBK + ((ch ^ (r & 7)) * 8));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int r = wn * WTN + j * 32 + lrow;
        wf[j] = *(const bf16x8*)(sw + r * kBK + ((ch ^ (r & 7)) * 8));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  const bf16_t* __restrict__ bias = a.bias;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm * WTM + i * 32 + lrow;
    if (m >= M) continue;
    if constexpr (EPI == EPI_QKV_ROPE) {
      int p = a.pos[m];
      if (p < 0) continue;  // padding row of a bshd batch: never attended
      p = p < a.max_positions ? p : a.max_positions - 1;
      const int heads = N / 192;
#pragma unroll
      for (int j = 0; j < FN; j += 2) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int nlo = n0 + wn * WTN + j * 32 + 8 * gq + 4 * lhalf;
          if (nlo >= N) continue;
          const int head = nlo / 192, c = (nlo % 192) / 64, d = nlo % 64;  // d < 32
          float lo[4], hi[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = acc[i][j][4 * gq + e];
            hi[e] = acc[i][j + 1][4 * gq + e];
          }
          if (bias) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lo[e] += bf2f(bias[nlo + e]);
              hi[e] += bf2f(bias[nlo + 32 + e]);
            }
          }
          if (c < 2) {
            const float2* cs = a.rope + (int64_t)p * 32 + d;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float2 t = cs[e];
              const float x0 = lo[e], x1 = hi[e];
              lo[e] = x0 * t.x - x1 * t.y;
              hi[e] = x1 * t.x + x0 * t.y;
            }
          }
          bf16_t* dst = a.y + (((int64_t)c * heads + head) * M + m) * kHeadDim + d;
          *(u32x2*)dst = u32x2{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3])};
          *(u32x2*)(dst + 32) = u32x2{pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3])};
        }
      }
    } else {
      bool zero_row = false;
      if constexpr (EPI == EPI_BIAS_RESIDUAL) zero_row = a.zero_pad_rows && a.pos[m] < 0;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = n0 + wn * WTN + j * 32 + 8 * gq + 4 * lhalf;
          if (n >= N) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * gq + e];
          if (bias) {
            const u32x2 bb = *(const u32x2*)(bias + n);
            v[0] += bflo(bb[0]); v[1] += bfhi(bb[0]); v[2] += bflo(bb[1]); v[3] += bfhi(bb[1]);
          }
          if constexpr (EPI == EPI_BIAS_GELU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu_erf(v[e]);
          }
          if constexpr (EPI == EPI_BIAS_RESIDUAL) {
            const u32x2 rr = *(const u32x2*)(a.res + m * N + n);
            v[0] += bflo(rr[0]); v[1] += bfhi(rr[0]); v[2] += bflo(rr[1]); v[3] += bfhi(rr[1]);
            if (zero_row) v[0] = v[1] = v[2] = v[3] = 0.f;
          }
          *(u32x2*)(a.y + m * N + n) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t run(const GemmArgs& a, hipStream_t st) {
  const int64_t tilesM = (a.M + BM - 1) / BM;
  const int64_t tilesN = (a.N + BN - 1) / BN;
  const int64_t nb = tilesM * tilesN;
  hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, EPI>), dim3((unsigned)nb), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int EPI>
hipError_t dispatch(const GemmArgs& a, hipStream_t st) {
  // 256x256 tiles when they give at least ~4 waves of workgroups over the 256
  // CUs; otherwise 256x128 tiles halve the wave-quantisation loss.
  const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if constexpr (EPI == EPI_QKV_ROPE) {
    return run<256, 256, 2, 2, EPI>(a, st);
  } else {
    if (t256 >= 4 * 256) return run<256, 256, 2, 2, EPI>(a, st);
    return run<256, 128, 2, 2, EPI>(a, st);
  }
}

}  // namespace

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  switch (epi) {
    case EPI_BIAS: return dispatch<EPI_BIAS>(a, st);
    case EPI_BIAS_GELU: return dispatch<EPI_BIAS_GELU>(a, st);
    case EPI_BIAS_RESIDUAL: return dispatch<EPI_BIAS_RESIDUAL>(a, st);
    case EPI_QKV_ROPE: return dispatch<EPI_QKV_ROPE>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace esm
