// Varlen non-causal attention for gfx950, head_dim 64.
//
// For each (sequence s, head n): ctx = softmax(q k^T / 8) v over the rows of s
// only ([CARD] 描述: bidirectional BERT-style encoder; [BIO-ACC] 3.2: packed
// sequences delimited by cu_seqlens; [TE-ESM2] 注意力掩码优化).  No work is
// done across sequences: a workgroup covers one 128-row query tile of one
// sequence and one head, and streams that sequence's keys in 64-row tiles.
//
// Design (CDNA4):
//  * 4 waves x 32 query rows.  Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (operand A = keys from LDS, operand B = the
//    wave's queries held in registers), so each lane owns one query row
//    (lane % 32) and 32 of the 64 keys of a tile; the other 32 live in lane
//    l ^ 32.  Row max needs one cross-lane exchange per tile; row sums stay
//    lane-local until the end.
//  * Online softmax in fp32 with exp2 and the scale log2(e)/8 folded into one
//    multiply-add ([TE-ESM2] roadmap names FlashAttention-style attention).
//  * O^T += V^T P^T: the probabilities are already in the operand-B layout of
//    the next MFMA (keys permuted within 16-key groups, bits 2 and 3 of the key
//    index swapped), and V^T comes straight from a row-major V tile in LDS via
//    ds_read_b64_tr_b16 with the same key permutation.
//  * K/V tiles are double-buffered in LDS (rows padded to 72 elements); the
//    next tile is fetched into registers during the current tile's math.
//  * Key rows past the end of the sequence are clamped to its last row (never a
//    neighbour's row) and their scores set to -inf; query rows past the end are
//    computed from a clamped row and not stored.
#include "common.h"

namespace esm {

namespace {

constexpr int kKT = 64;     // keys per tile
constexpr int kLdsRow = 72; // padded LDS row (elements)
constexpr float kScaleLog2 = 0.18033688011112042f;  // log2(e) / sqrt(64)

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__global__ __launch_bounds__(256, 2) void k_attention(AttnArgs a) {
  const int heads = a.heads;
  const int tile = blockIdx.x / heads, head = blockIdx.x % heads;
  if (tile >= *a.ntiles) return;
  const int s = a.tiles[2 * tile], q0 = a.tiles[2 * tile + 1];
  const int64_t start = a.segs[2 * s];
  const int L = a.segs[2 * s + 1];
  if (L <= 0) return;

  __shared__ __attribute__((aligned(16))) bf16_t sk[2][kKT * kLdsRow];
  __shared__ __attribute__((aligned(16))) bf16_t sv[2][kKT * kLdsRow];

  const int64_t T = a.T;
  const bf16_t* __restrict__ Qg = a.qkv + ((int64_t)(0 * heads + head) * T) * kHeadDim;
  const bf16_t* __restrict__ Kg = a.qkv + ((int64_t)(1 * heads + head) * T) * kHeadDim;
  const bf16_t* __restrict__ Vg = a.qkv + ((int64_t)(2 * heads + head) * T) * kHeadDim;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;

  // This lane's query row (clamped into the sequence).
  const int qrow = q0 + 32 * wave + lrow;
  const int qc = qrow < L ? qrow : L - 1;
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = *(const bf16x8*)(Qg + (start + qc) * kHeadDim + kk * 16 + 8 * lhalf);

  // K/V tiles travel global -> registers -> LDS.  Two register sets (A, B)
  // keep the loads of the next two tiles in flight while a tile is used.
  u32x4 krA[2], vrA[2], krB[2], vrB[2];
  auto gload = [&](int j, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      int key = j * kKT + row;
      key = key < L ? key : L - 1;
      kr[i] = *(const u32x4*)(Kg + (start + key) * kHeadDim + ch * 8);
      vr[i] = *(const u32x4*)(Vg + (start + key) * kHeadDim + ch * 8);
    }
  };
  auto sstore = [&](int buf, const u32x4 (&kr)[2], const u32x4 (&vr)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      *(u32x4*)(&sk[buf][row * kLdsRow + ch * 8]) = kr[i];
      *(u32x4*)(&sv[buf][row * kLdsRow + ch * 8]) = vr[i];
    }
  };

  float m_i = -INFINITY, l_i = 0.f;
  f32x16 o[2];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;

  // ds_read_b64_tr_b16 addressing inside each 16-lane group: source lane j
  // points at row k0 + j/4, columns n0 + 4*(j%4); lane i then receives
  // V[k0 + 0..3][n0 + i].
  const int g16 = lane & 15;
  const int tr_row = g16 >> 2, tr_col = 4 * (g16 & 3);
  const int n0_lane = 16 * ((lane >> 4) & 1);

  const int ntk = (L + kKT - 1) / kKT;
  // A wave whose 32 query rows all lie past the end of the sequence only helps
  // to stage K/V (and meets the barriers); it skips the math.
  const bool wave_active = q0 + 32 * wave < L;
  // Tile j is in LDS buffer j & 1; its successor is in registers `nx` and the
  // one after that is loaded into `nn` during tile j.
  auto run_tile = [&](int j, const u32x4 (&nxk)[2], const u32x4 (&nxv)[2], u32x4 (&nnk)[2], u32x4 (&nnv)[2]) {
    const int cur = j & 1;
    if (j + 2 < ntk) gload(j + 2, nnk, nnv);
    if (wave_active) {
      // S^T for this tile: two 32-key blocks.
      f32x16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 kf = *(const bf16x8*)(&sk[cur][(kb * 32 + lrow) * kLdsRow + kk * 16 + 8 * lhalf]);
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], st[kb], 0, 0, 0);
        }
      }
      if ((j + 1) * kKT > L) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j * kKT + kb * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
            if (key >= L) st[kb][r] = -INFINITY;
          }
      }
      float mx = st[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_i, mx);
      const float alpha = exp2_fast((m_i - m_new) * kScaleLog2);
      const float mc = m_new * kScaleLog2;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(fmaf(st[kb][r], kScaleLog2, -mc));
          st[kb][r] = p;
          rs += p;
        }
      l_i = l_i * alpha + rs;
      m_i = m_new;
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;

      // P^T as bf16 operand B: block kb, step u covers registers 8u .. 8u+7.
      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack_bf2(st[kb][8 * u + 2 * e], st[kb][8 * u + 2 * e + 1]);
          pb[kb][u] = __builtin_bit_cast(bf16x8, w);
        }

      const bf16_t* vb = sv[cur];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int n0 = d * 32 + n0_lane;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int k0 = kb * 32 + 16 * u + 4 * lhalf;
            const bf16_t* p0 = vb + (k0 + tr_row) * kLdsRow + n0 + tr_col;
            const bf16_t* p1 = p0 + 8 * kLdsRow;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const i16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pb[kb][u], o[d], 0, 0, 0);
          }
      }
    }
    if (j + 1 < ntk) sstore(cur ^ 1, nxk, nxv);
    __syncthreads();
  };
  gload(0, krA, vrA);
  sstore(0, krA, vrA);
  if (ntk > 1) gload(1, krA, vrA);
  __syncthreads();
  for (int j = 0; j < ntk; j += 2) {
    run_tile(j, krA, vrA, krB, vrB);
    if (j + 1 < ntk) run_tile(j + 1, krB, vrB, krA, vrA);
  }

  const float lt = l_i + __shfl_xor(l_i, 32);
  const float inv = 1.0f / lt;
  const int H = heads * kHeadDim;
  if (a.ctx8.y) {
    // E4M3 context for the FP8 out-projection: cast with the tensor's delayed
    // scale, amax over the valid rows recorded by every lane of the wave.
    const float s8 = a.ctx8.scale[0];
    float amax = 0.f;
    if (qrow < L) {
      uint8_t* dst = a.ctx8.y + (start + qrow) * H + head * kHeadDim;
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int dim = d * 32 + 8 * gq + 4 * lhalf;
          const float v[4] = {o[d][4 * gq] * inv, o[d][4 * gq + 1] * inv, o[d][4 * gq + 2] * inv,
                              o[d][4 * gq + 3] * inv};
#pragma unroll
          for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(v[e]));
          *(uint32_t*)(dst + dim) = pack_e4m3x4(v, s8);
        }
    }
    __shared__ float red[4];
    record_amax_block<4>(a.ctx8.amax, amax, red);
    return;
  }
  if (qrow >= L) return;
  bf16_t* dst = a.ctx + (start + qrow) * H + head * kHeadDim;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int dim = d * 32 + 8 * gq + 4 * lhalf;
      *(u32x2*)(dst + dim) = u32x2{pack_bf2(o[d][4 * gq] * inv, o[d][4 * gq + 1] * inv),
                                   pack_bf2(o[d][4 * gq + 2] * inv, o[d][4 * gq + 3] * inv)};
    }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.tile_cap <= 0 || a.T <= 0) return hipSuccess;
  const int64_t nblk = a.tile_cap * a.heads;
  hipLaunchKernelGGL(k_attention, dim3((unsigned)nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace esm
