// Varlen non-causal attention for gfx950, head_dim 64.
//
// For each (sequence s, head n): ctx = softmax(q k^T / 8) v over the rows of s
// only ([CARD] 描述: bidirectional BERT-style encoder; [BIO-ACC] 3.2: packed
// sequences delimited by cu_seqlens; [TE-ESM2] 注意力掩码优化).  No work is
// done across sequences: a workgroup covers one 256-row query tile of one
// sequence and one head, and streams that sequence's keys in 64-row tiles.
//
// Design (CDNA4):
//  * 8 waves x 32 query rows.  Scores are formed transposed, S^T = K Q^T, with
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
//  * K/V tiles are double-buffered in LDS as 128-byte rows whose 16-byte
//    chunks are XOR-swizzled by row (kSwz), so that the key fragment reads
//    and the transposing V reads hit distinct banks.  The next tile is loaded
//    straight into LDS (global_load_lds) during the current tile's math, which
//    keeps no staging registers: 4 waves per SIMD fit (two workgroups per
//    CU).  Eight waves share each K/V tile: half the tile fills and barriers
//    per query of four.  An LDS tile holds 128 keys, computed as two 64-key
//    tiles between barriers (64 KB of LDS per workgroup).
//  * Key rows past the end of the sequence are clamped to its last row (never a
//    neighbour's row) and their scores set to -inf; query rows past the end are
//    computed from a clamped row and not stored.
//  * The context leaves as bf16, as E4M3 with the FP8 recipe's delayed scale
//    and amax, or as MXFP4 codes and block scales for an MXFP4 out-projection.
//
// The same body (attend<mode>) serves the biased attention of the
// DeepSpeed4Science page ([DS4SCI] 3.2, 5.3): q, k, v [B, N, L, heads, 64]
// with a per-key mask bias and a pair bias added to the scores
// (k_biased_attention below).
#include "common.h"

namespace esm {

namespace {

constexpr int kKT = 64;     // keys per compute tile
constexpr int kSub = 2;     // compute tiles per LDS tile (one fill and barrier)
constexpr int kLT = kKT * kSub;  // keys per LDS tile
constexpr int kNW = kAttnTileRows / 32;  // waves per workgroup, 32 query rows each
constexpr int kLdsRow = 64; // LDS row (elements): one 128-byte row per key
constexpr float kScaleLog2 = 0.18033688011112042f;  // log2(e) / sqrt(64)
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// x of lanes l and l ^ 32, in some order (one VALU swap of the wave's halves:
// whichever half moves, the two results of lane l are these two values).
__device__ __forceinline__ void pair_halves(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Chunk swizzle of LDS row r (16-byte chunk c is stored at c ^ kSwz(r)).  Over
// any 8 consecutive rows it is a permutation (key reads: eight rows, one chunk
// each, per 128-byte bank sweep); rows 4i..4i+3 get distinct values of bit 1..2
// and rows r, r+2 differ in bit 2 (transposing V reads: four rows, 32 or 64
// bytes each); rows r and r+8 differ in bit 1, so the even (odd) rows of 16
// are distinct too (key reads with a 256-byte bank sweep).
__device__ __forceinline__ int kSwz(int r) { return (((r & 3) << 1) | ((r >> 2) & 1)) ^ (((r >> 3) & 1) << 1); }

// What a workgroup adds to the scores (bit flags; 0 = the encoder's plain
// attention).  kBias: scores become s / 8 + biases, with rows whose keys are
// all -inf allowed; kMask / kPair: the per-key mask bias / the pair bias is
// present; kVec: L % 4 == 0, so four consecutive keys' biases are one aligned
// 8-byte load; kLds: L % 8 == 0, and the biases of each 64-key tile are
// staged through a wave-private LDS region by 16-byte direct loads (one
// instruction covers 8 rows x 128 bytes instead of 32 rows x 16 bytes), with
// 64-key K/V LDS tiles so that two workgroups still fit per CU.
enum AttnMode { kPlain = 0, kBias = 1, kMask = 2, kPair = 4, kVec = 8, kLds = 16 };

// Chunk swizzle of row r of a wave's staged pair bias (16-byte chunk c of the
// 128-byte row is stored at c ^ kSwzB(r)): the 16 even (odd) rows read by one
// ds_read_b64 spread over all 8 chunk positions.
__device__ __forceinline__ int kSwzB(int r) { return (r >> 1) & 7; }


// One workgroup: 256 query rows from q0 of one head of one sequence of L rows.
// Qg, Kg, Vg point at row 0 of the sequence for this head; row r of each is
// 64 contiguous values at + r * rs.  Biased modes add maskg[c] and
// pairg[r * L + c] to the score of (query row r, key c).  On return o holds
// this lane's unnormalised context (dims d * 32 + 8 g + 4 lhalf + e in
// o[d][4 g + e]), inv the reciprocal of its softmax sum and mrow the maximum
// that sum and o were taken against: a raw score of the row (q.k, before the
// scale; the biased modes: the score) at most 8 / kS below its largest.
template <int kMode>
__device__ __forceinline__ void attend(const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg,
                                       const bf16_t* __restrict__ Vg, const int64_t rs, const int L, const int q0,
                                       const bf16_t* __restrict__ maskg, const bf16_t* __restrict__ pairg,
                                       f32x16 (&o)[2], float& inv, float& mrow) {
  constexpr bool kStaged = (kMode & kLds) != 0;
  constexpr int kSubM = kStaged ? 1 : kSub;        // compute tiles per LDS tile
  constexpr int kLTM = kKT * kSubM;                // keys per LDS tile
  constexpr int kDmaPW = kLTM / 8 / kNW;           // 1 KB direct loads per tensor per wave per LDS tile
  // Wave-private bias staging (kLds): 32 pair-bias rows x 64 keys (4 KB),
  // then the tile's 64 mask values repeated 8 times (1 KB).
  constexpr int kStageElems = 32 * 64 + 512;
  __shared__ __attribute__((aligned(1024))) bf16_t sk[2][kLTM * kLdsRow];
  __shared__ __attribute__((aligned(1024))) bf16_t sv[2][kLTM * kLdsRow];
  __shared__ __attribute__((aligned(1024))) bf16_t sb[kStaged ? kNW : 1][kStaged ? kStageElems : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;

  // This lane's query row (clamped into the sequence).
  const int qrow = q0 + 32 * wave + lrow;
  const int qc = qrow < L ? qrow : L - 1;
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = *(const bf16x8*)(Qg + qc * rs + kk * 16 + 8 * lhalf);
  // Biased modes take q / 8 (exact: a power of two) so that the score MFMAs
  // accumulate s / 8 onto the biases as they are; the softmax then scales by
  // log2(e) alone.
  constexpr float kS = (kMode & kBias) != 0 ? kLog2e : kScaleLog2;
  if constexpr ((kMode & kBias) != 0) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)((float)qf[kk][e] * 0.125f);
  }
  const bf16_t* __restrict__ prow = nullptr;
  if constexpr ((kMode & kPair) != 0) prow = pairg + (int64_t)qc * L;

  // K/V tiles go straight from global memory into LDS (global_load_lds): the
  // workgroup's 8 instructions per tensor fill 1 KB (8 rows) each; in
  // instruction i of wave w, lane l writes physical chunk l % 8 of tile row
  // 8 (w + kNW i) + l / 8 and so fetches that row's logical chunk
  // (l % 8) ^ kSwz(row).  Key rows past the end of the sequence are clamped.
  const uint32_t lds_k = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&sk[0][0];
  const uint32_t lds_v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&sv[0][0];
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int src_row[kDmaPW], src_col[kDmaPW];
#pragma unroll
  for (int i = 0; i < kDmaPW; ++i) {
    src_row[i] = 8 * (wave + kNW * i) + (lane >> 3);
    src_col[i] = ((lane & 7) ^ kSwz(src_row[i])) * 8;
  }
  auto gload = [&](int j, int buf) {
#pragma unroll
    for (int i = 0; i < kDmaPW; ++i) {
      int key = j * kLTM + src_row[i];
      key = key < L ? key : L - 1;
      const int64_t at = key * rs + src_col[i];
      const uint32_t dst = (uint32_t)(buf * kLTM * kLdsRow * 2 + (wave_u + kNW * i) * 1024);
      lds_dma16(Kg + at, lds_k + dst);
      lds_dma16(Vg + at, lds_v + dst);
    }
  };
  // kLds: biases of compute tile j into this wave's region.  Pair bias:
  // instruction i, lane l fetches row 8i + l/8 of the wave's 32 query rows
  // (clamped), logical chunk (l % 8) ^ kSwzB(row) of its 64 keys; mask: every
  // lane fetches chunk l % 8.  With L % 8 == 0 a chunk of 8 keys lies wholly
  // inside or wholly past the end, where it is clamped to the last chunk.
  const uint32_t lds_b = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&sb[0][0] +
                         (kStaged ? (uint32_t)wave_u * kStageElems * 2 : 0u);
  auto bload = [&](int j) {
    if constexpr (kStaged) {
      if constexpr ((kMode & kPair) != 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 8 * i + (lane >> 3);
          int q = q0 + 32 * wave + rr;
          q = q < L ? q : L - 1;
          int key = j * kKT + 8 * ((lane & 7) ^ kSwzB(rr));
          key = key < L ? key : L - 8;
          lds_dma16(pairg + (int64_t)q * L + key, lds_b + i * 1024);
        }
      }
      if constexpr ((kMode & kMask) != 0) {
        int key = j * kKT + 8 * (lane & 7);
        key = key < L ? key : L - 8;
        lds_dma16(maskg + key, lds_b + 4096);
      }
    }
  };

  float m_i = -INFINITY, l_i = 0.f;
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
  // Swizzled in-row offsets (elements).  Key reads: row kb*32 + lrow, chunk
  // 2*kk + lhalf.  V reads: rows k0 + tr_row (+8), chunk of column n0 + tr_col;
  // 16u and 32kb leave the swizzle unchanged.
  int koff[4], voff[2][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = ((2 * kk + lhalf) ^ kSwz(lrow)) * 8;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 4 * lhalf + tr_row + 8 * h, col = d * 32 + n0_lane + tr_col;
      voff[d][h] = (((col >> 3) ^ kSwz(r)) * 8) + (col & 7);
    }

  const int ntk = (L + kKT - 1) / kKT;   // compute tiles
  const int ntl = (L + kLTM - 1) / kLTM; // LDS tiles
  // A wave whose 32 query rows all lie past the end of the sequence only helps
  // to stage K/V (and meets the barriers); it skips the math.
  const bool wave_active = q0 + 32 * wave < L;
  // LDS tile t is in buffer t & 1; tile t + 1 is fetched into the other
  // buffer during tile t's math and published by the barrier that ends it.
  gload(0, 0);
  if (wave_active) bload(0);
  vm_wait_all();
  __syncthreads();
  for (int t = 0; t < ntl; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntl) gload(t + 1, cur ^ 1);
#pragma unroll
    for (int sub = 0; sub < kSubM; ++sub) {
    const int j = t * kSubM + sub;  // compute tile: keys j*64 .. j*64+63, LDS rows sub*64 ..
    const bool active = wave_active && j < ntk;
    // S^T for this tile: two 32-key blocks; register r of block kb is key
    // j*64 + kb*32 + 8*(r/4) + 4*lhalf + r%4.  The MFMAs accumulate q.k onto
    // 0, or in the biased modes (q / 8).k onto mask + pair, which is the
    // biased score itself.  Keys past the end read a clamped bias; their
    // scores become -inf.
    f32x16 st[2];
    if (active) {
      if constexpr ((kMode & kBias) != 0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int key0 = j * kKT + kb * 32 + 8 * g + 4 * lhalf;
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (kStaged) {
              const int c = 4 * kb + g;
              const bf16_t* sbw = &sb[wave_u][0];
              if constexpr ((kMode & kPair) != 0) {
                const u32x2 w = *(const u32x2*)(sbw + lrow * 64 + ((c ^ kSwzB(lrow)) * 8) + 4 * lhalf);
                b[0] = bflo(w[0]); b[1] = bfhi(w[0]); b[2] = bflo(w[1]); b[3] = bfhi(w[1]);
              }
              if constexpr ((kMode & kMask) != 0) {
                const u32x2 w = *(const u32x2*)(sbw + 2048 + c * 8 + 4 * lhalf);
                b[0] += bflo(w[0]); b[1] += bfhi(w[0]); b[2] += bflo(w[1]); b[3] += bfhi(w[1]);
              }
            } else if constexpr ((kMode & kVec) != 0) {
              const int key = key0 < L ? key0 : L - 4;
              if constexpr ((kMode & kPair) != 0) {
                const u32x2 w = *(const u32x2*)(prow + key);
                b[0] = bflo(w[0]); b[1] = bfhi(w[0]); b[2] = bflo(w[1]); b[3] = bfhi(w[1]);
              }
              if constexpr ((kMode & kMask) != 0) {
                const u32x2 w = *(const u32x2*)(maskg + key);
                b[0] += bflo(w[0]); b[1] += bfhi(w[0]); b[2] += bflo(w[1]); b[3] += bfhi(w[1]);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int key = key0 + e < L ? key0 + e : L - 1;
                if constexpr ((kMode & kPair) != 0) b[e] = bf2f(prow[key]);
                if constexpr ((kMode & kMask) != 0) b[e] += bf2f(maskg[key]);
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) st[kb][4 * g + e] = b[e];
          }
        if constexpr (kStaged) {
          // The region is refilled with the next tile's biases once these
          // reads have returned.
          if (j + 1 < ntk) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            bload(j + 1);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
      }
    }
    if (active) {
      // The matrix core and the fp32 VALU do not run at once on a SIMD (a
      // wave's MFMAs and another wave's adds and multiplies serialise; only
      // the exponentials overlap them), so a wave entering a run of MFMAs is
      // given priority over the waves in their softmax.
      __builtin_amdgcn_s_setprio(1);
      const bf16_t* kt = sk[cur] + sub * kKT * kLdsRow;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf = *(const bf16x8*)(&kt[(kb * 32 + lrow) * kLdsRow + koff[kk]]);
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], st[kb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if ((j + 1) * kKT > L) {
        // Keys at or past L: key offset c of the tile (a constant per
        // register) against this lane's limit.
        const int lim = L - j * kKT - 4 * lhalf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) st[kb][r] = -INFINITY;
      }
      // Row max and row sum in four independent chains (short dependency
      // chains for the VALU); the chains combine in a fixed order.  The
      // maximum is IEEE 754-2019's (NaN propagating, no input
      // canonicalisation), which gfx950 issues three operands at a time.
      float m4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        m4[c] = st[c >> 1][8 * (c & 1)];
#pragma unroll
        for (int r = 1; r < 8; ++r) m4[c] = __builtin_elementwise_maximum(m4[c], st[c >> 1][8 * (c & 1) + r]);
      }
      float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m4[0], m4[1]),
                                               __builtin_elementwise_maximum(m4[2], m4[3]));
      {
        float a, b;
        pair_halves(mx, a, b);
        mx = __builtin_elementwise_maximum(a, b);
      }
      const float m_new = __builtin_elementwise_maximum(m_i, mx);
      // Lazy rescaling: the running maximum (and with it o and l) moves only
      // when some row of the wave grew by more than 8 in exp2 units; until
      // then the probabilities are taken against the older maximum and stay
      // below 2^8.  The first tile always rescales (m_i = -inf gives +inf);
      // rows all -inf so far (biased modes) give NaN and do not.
      const bool grow = (m_new - m_i) * kS > 8.f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        // Biased modes: while every key so far is -inf (masked), subtract 0,
        // so the probabilities stay 0 instead of exp(-inf - -inf) = NaN.
        const float m_sub = ((kMode & kBias) != 0 && m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast((m_i - m_sub) * kS);
        l_i *= alpha;
        m_i = m_new;
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
      const float mc = (((kMode & kBias) != 0 && m_i == -INFINITY) ? 0.f : m_i) * kS;
      // each chain starts at its first probability (the same sum as from 0:
      // probabilities are never -0)
      float s4[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(fmaf(st[kb][r], kS, -mc));
          st[kb][r] = p;
          if ((r & 7) == 0) s4[2 * kb + (r >> 3)] = p;
          else s4[2 * kb + (r >> 3)] += p;
        }
      l_i += (s4[0] + s4[1]) + (s4[2] + s4[3]);

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

      __builtin_amdgcn_s_setprio(1);
      const bf16_t* vb = sv[cur] + sub * kKT * kLdsRow;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const int k0 = kb * 32 + 16 * u + 4 * lhalf;
            const bf16_t* p0 = vb + (k0 + tr_row) * kLdsRow + voff[d][0];
            const bf16_t* p1 = vb + (k0 + tr_row + 8) * kLdsRow + voff[d][1];
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const i16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pb[kb][u], o[d], 0, 0, 0);
          }
        }
      __builtin_amdgcn_s_setprio(0);
    }
    }
    vm_wait_all();
    __syncthreads();
  }

  float la, lb;
  pair_halves(l_i, la, lb);
  const float lt = la + lb;
  inv = 1.0f / lt;
  mrow = m_i;
}

// Encoder attention: one workgroup per (256-row query tile, head) from the
// segment table; qkv planar [3][heads][T][64], context [T, heads * 64].
__global__ __launch_bounds__(64 * kNW) void k_attention(AttnArgs a) {
  const int heads = a.heads;
  const int tile = blockIdx.x / heads, head = blockIdx.x % heads;
  if (tile >= *a.ntiles) return;
  const int s = a.tiles[2 * tile], q0 = a.tiles[2 * tile + 1];
  const int64_t start = a.segs[2 * s];
  const int L = a.segs[2 * s + 1];
  if (L <= 0) return;

  const int64_t T = a.T;
  const bf16_t* Qg = a.qkv + ((int64_t)(0 * heads + head) * T + start) * kHeadDim;
  const bf16_t* Kg = a.qkv + ((int64_t)(1 * heads + head) * T + start) * kHeadDim;
  const bf16_t* Vg = a.qkv + ((int64_t)(2 * heads + head) * T + start) * kHeadDim;
  f32x16 o[2];
  float inv, mrow;
  attend<kPlain>(Qg, Kg, Vg, kHeadDim, L, q0, nullptr, nullptr, o, inv, mrow);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lhalf = lane >> 5;
  const int qrow = q0 + 32 * wave + (lane & 31);
  const int H = heads * kHeadDim;
  // The softmax normaliser a backward pass takes: log sum_j exp(q.k_j / 8)
  // = max / 8 + log(sum_j exp((q.k_j - max) / 8)).
  if (a.lse && lhalf == 0 && qrow < L) a.lse[(int64_t)head * T + start + qrow] = mrow * 0.125f - logf(inv);
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
    __shared__ float red[kNW];
    record_amax_block<kNW>(a.ctx8.amax, amax, red);
    return;
  }
  if (a.ctx_mx) {
    // MXFP4 context for the MXFP4 out-projection: block d of this head's 64
    // dims is this lane's 16 (d * 32 + 8 gq + 4 lhalf + e) and the 16 of lane
    // l ^ 32; codes of dims 8 gq + 4 lhalf + (0..3) are bytes 16 d + 4 gq +
    // 2 lhalf (+1) of the head's 32 code bytes.
    const int64_t M2 = T + (T & 1);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      float am = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) am = fmaxf(am, fabsf(o[d][r] * inv));
      am = fmaxf(am, __shfl_xor(am, 32));
      const int ex = mx_block_exponent(am);
      if (qrow < L) {
        uint8_t* dst = a.ctx_mx + (start + qrow) * (H / 2) + head * (kHeadDim / 2) + 16 * d + 2 * lhalf;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint32_t c2 = e2m1_pair(o[d][4 * gq] * inv, o[d][4 * gq + 1] * inv, ex) |
                              (e2m1_pair(o[d][4 * gq + 2] * inv, o[d][4 * gq + 3] * inv, ex) << 8);
          *(uint16_t*)(dst + 4 * gq) = (uint16_t)c2;
        }
        if (lhalf == 0) a.ctx_mx_sc[mx_scale_offset(start + qrow, 2 * head + d, M2)] = (uint8_t)(ex + 127);
      }
    }
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

// Biased attention on [B, N, L, heads, 64] tensors ([DS4SCI] 3.2, 5.3): one
// workgroup per (b, n, 256-row query tile, head), the head fastest, so with
// 8 heads every workgroup of head h lands on the same XCD and its L2 keeps
// that head's pair bias (shared by all n) resident.
template <int kMode>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu((kMode & (kVec | kLds)) ? 4 : 1, 4)))
void k_biased_attention(BiasedAttnArgs a) {
  const int heads = a.heads;
  const int h = blockIdx.x % heads;
  const int rest = blockIdx.x / heads;
  const int tile = rest % a.qtiles;
  const int64_t bn = rest / a.qtiles;
  const int64_t b = bn / a.N;
  const int L = a.L, q0 = tile * kAttnTileRows;
  const int64_t rs = (int64_t)heads * kHeadDim;
  const int64_t base = (bn * L * heads + h) * kHeadDim;
  const bf16_t* maskg = (kMode & kMask) ? a.mask + bn * L : nullptr;
  const bf16_t* pairg = (kMode & kPair) ? a.pair + (b * heads + h) * (int64_t)L * L : nullptr;
  f32x16 o[2];
  float inv, mrow;
  attend<kMode>(a.q + base, a.k + base, a.v + base, rs, L, q0, maskg, pairg, o, inv, mrow);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lhalf = lane >> 5;
  const int qrow = q0 + 32 * wave + (lane & 31);
  if (qrow >= L) return;
  bf16_t* dst = a.out + base + qrow * rs;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int dim = d * 32 + 8 * gq + 4 * lhalf;
      *(u32x2*)(dst + dim) = u32x2{pack_bf2(o[d][4 * gq] * inv, o[d][4 * gq + 1] * inv),
                                   pack_bf2(o[d][4 * gq + 2] * inv, o[d][4 * gq + 3] * inv)};
    }
}

// ------------------------------------------------------------------ backward
//
// Gradients of the encoder attention with respect to q, k and v, from the
// forward's context O and softmax normaliser lse, for an incoming gradient dO
// of the context.  Per (sequence, head), with S = q k^T / 8 and
// P = exp(S - lse):  dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with
// D = rowsum(dO * O) (= rowsum(P * dP)),  dQ = dS K / 8,  dK = dS^T Q / 8.
// P is recomputed from lse, never stored.  Two kernels, dQ first:
//  * k_attn_bwd_dq (below) also forms D for its queries from the dO row it
//    holds and the O row, and writes it for the dK/dV kernel;
//  * k_attn_bwd_dkv: one workgroup per 128 keys of one sequence and head (4
//    waves x 32 keys, K and V rows in registers as the MFMAs' B operand),
//    streaming the sequence's queries through LDS in 128-row tiles of Q and dO
//    (two 64-row compute steps per fill; direct loads, double-buffered, the
//    forward's swizzle) with their lse and D; S and dP come out query x key,
//    so each lane owns one key and the products accumulate dV^T and dK^T in
//    registers: no atomics;
//  * k_attn_bwd_dq: one workgroup per 128 queries, the forward's structure
//    with dP added: K and V tiles in LDS, S^T and dP^T key x query, and
//    dQ^T += K^T dS^T with K^T read by the transposing LDS reads.
// P and dS enter the second products as bf16 (fp32 accumulation), as P does
// in the forward.  Both big kernels hold 180-220 VGPRs (two waves per SIMD),
// so a workgroup has 4 waves and two workgroups share a CU: one's barrier
// waits are covered by the other's math.

struct AttnBwdPtrs {
  const bf16_t* Q;    // row 0 of the sequence, head; row stride 64
  const bf16_t* K;
  const bf16_t* V;
  const bf16_t* dO;   // row stride H
  const bf16_t* O;    // row stride H
  const float* lse;   // [L] of this head
  float* del;         // [L] of this head
};

__device__ __forceinline__ AttnBwdPtrs bwd_ptrs(const AttnBwdArgs& a, int head, int64_t start) {
  const int64_t T = a.T;
  AttnBwdPtrs p;
  p.Q = a.qkv + ((int64_t)(0 * a.heads + head) * T + start) * kHeadDim;
  p.K = a.qkv + ((int64_t)(1 * a.heads + head) * T + start) * kHeadDim;
  p.V = a.qkv + ((int64_t)(2 * a.heads + head) * T + start) * kHeadDim;
  p.dO = a.dout + start * ((int64_t)a.heads * kHeadDim) + head * kHeadDim;
  p.O = a.out + start * ((int64_t)a.heads * kHeadDim) + head * kHeadDim;
  p.lse = a.lse + (int64_t)head * T + start;
  p.del = a.delta + (int64_t)head * T + start;
  return p;
}

constexpr int kBT = 64;   // rows per streamed LDS tile in the backward kernels
constexpr int kBW = 4;    // waves per backward workgroup (32 rows each): two workgroups share a CU
constexpr int kBParts = kAttnTileRows / (32 * kBW);  // backward workgroups per segment-table tile

// 64 rows x 128 bytes of a row-major tensor (row stride rs elements) into a
// swizzled LDS tile: in instruction i, wave w fetches rows 8 (w + kBW i) ..
// + 7, lane l physical chunk l % 8 of row 8 (w + kBW i) + l / 8, i.e. logical
// chunk (l % 8) ^ kSwz(row).  Rows past the end of the sequence are clamped
// to its last row.
__device__ __forceinline__ void tile_dma(const bf16_t* __restrict__ g, int64_t rs, int row0, int L, uint32_t lds,
                                         int lane, int wave, int wave_u) {
#pragma unroll
  for (int i = 0; i < 8 / kBW; ++i) {
    const int r = 8 * (wave + kBW * i) + (lane >> 3);
    int row = row0 + r;
    row = row < L ? row : L - 1;
    lds_dma16(g + row * rs + ((lane & 7) ^ kSwz(r)) * 8, lds + (uint32_t)(wave_u + kBW * i) * 1024u);
  }
}

// Workgroup -> (segment-table tile, 32 kBW-row part of it, head), the head
// fastest.  Returns false (for the whole workgroup) when the part starts past
// the end of its sequence.
__device__ __forceinline__ bool bwd_block(const AttnBwdArgs& a, int& head, int& s, int& r0) {
  head = blockIdx.x % a.heads;
  const int rest = blockIdx.x / a.heads;
  const int tile = rest / kBParts, part = rest % kBParts;
  if (tile >= *a.ntiles) return false;
  s = a.tiles[2 * tile];
  r0 = a.tiles[2 * tile + 1] + part * 32 * kBW;
  return r0 < a.segs[2 * s + 1];
}

__global__ __launch_bounds__(64 * kBW) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bwd_dkv(AttnBwdArgs a) {
  const int heads = a.heads;
  int head, s, k0;
  if (!bwd_block(a, head, s, k0)) return;
  const int64_t start = a.segs[2 * s];
  const int L = a.segs[2 * s + 1];
  const AttnBwdPtrs p = bwd_ptrs(a, head, start);
  const int64_t H = (int64_t)heads * kHeadDim;

  // LDS tiles of 2 x 64 query rows (one fill and barrier per 128 queries,
  // so the next tile's loads have two compute steps to land).
  constexpr int kTR = 2 * kBT;
  __shared__ __attribute__((aligned(1024))) bf16_t sq[2][kTR * kLdsRow];
  __shared__ __attribute__((aligned(1024))) bf16_t sd[2][kTR * kLdsRow];
  __shared__ __attribute__((aligned(16))) float sl[2][kTR];   // lse * log2(e); +inf past the end
  __shared__ __attribute__((aligned(16))) float sD[2][kTR];   // D; 0 past the end

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // This lane's key (clamped): its K and V rows as the B operand, dims
  // 16 kk + 8 lhalf .. + 7 in register kk.
  const int key = k0 + 32 * wave + lrow;
  const int kc = key < L ? key : L - 1;
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    kf[kk] = *(const bf16x8*)(p.K + kc * kHeadDim + kk * 16 + 8 * lhalf);
    vf[kk] = *(const bf16x8*)(p.V + kc * kHeadDim + kk * 16 + 8 * lhalf);
  }

  const uint32_t lds_q = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&sq[0][0];
  const uint32_t lds_d = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&sd[0][0];
  auto gload = [&](int t, int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t off = (uint32_t)(buf * kTR + h * kBT) * kLdsRow * 2;
      tile_dma(p.Q, kHeadDim, t * kTR + h * kBT, L, lds_q + off, lane, wave, wave_u);
      tile_dma(p.dO, H, t * kTR + h * kBT, L, lds_d + off, lane, wave, wave_u);
    }
  };
  auto sload = [&](int t, float& l2, float& dd) {
    const int q = t * kTR + tid;
    l2 = q < L ? p.lse[q] * kLog2e : INFINITY;
    dd = q < L ? p.del[q] : 0.f;
  };

  const int g16 = lane & 15;
  const int tr_row = g16 >> 2, tr_col = 4 * (g16 & 3);
  const int n0_lane = 16 * ((lane >> 4) & 1);
  int koff[4], voff[2][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = ((2 * kk + lhalf) ^ kSwz(lrow)) * 8;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 4 * lhalf + tr_row + 8 * h, col = d * 32 + n0_lane + tr_col;
      voff[d][h] = (((col >> 3) ^ kSwz(r)) * 8) + (col & 7);
    }

  f32x16 dv[2], dk[2];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dv[d][r] = 0.f; dk[d][r] = 0.f; }

  const int ntq = (L + kBT - 1) / kBT;   // 64-query compute steps
  const int ntl = (L + kTR - 1) / kTR;   // LDS tiles
  const bool wave_active = k0 + 32 * wave < L;
  gload(0, 0);
  if (tid < kTR) {
    float l2, dd;
    sload(0, l2, dd);
    sl[0][tid] = l2;
    sD[0][tid] = dd;
  }
  vm_wait_all();
  __syncthreads();
  for (int t = 0; t < ntl; ++t) {
    const int cur = t & 1;
    float nl2 = 0.f, ndd = 0.f;
    if (t + 1 < ntl) {
      gload(t + 1, cur ^ 1);
      if (tid < kTR) sload(t + 1, nl2, ndd);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
    if (wave_active && 2 * t + sub < ntq) {
      const bf16_t* qt = sq[cur] + sub * kBT * kLdsRow;
      const bf16_t* dt = sd[cur] + sub * kBT * kLdsRow;
      const float* slt = &sl[cur][sub * kBT];
      const float* sDt = &sD[cur][sub * kBT];
      // S and dP, query x key: block qb holds queries qb*32 + 8*(r/4) +
      // 4*lhalf + r%4 of this lane's key.
      f32x16 st[2], dp[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { st[qb][r] = 0.f; dp[qb][r] = 0.f; }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 qa = *(const bf16x8*)(&qt[(qb * 32 + lrow) * kLdsRow + koff[kk]]);
          st[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], st[qb], 0, 0, 0);
          const bf16x8 da = *(const bf16x8*)(&dt[(qb * 32 + lrow) * kLdsRow + koff[kk]]);
          dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[kk], dp[qb], 0, 0, 0);
        }
      }
      // P = exp2(S log2(e) / 8 - lse log2(e)); dS = P (dP - D).  Queries past
      // the end have lse = +inf: P = 0, dS = 0.
      bf16x8 pb[2][2], sb[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q = qb * 32 + 8 * g + 4 * lhalf;
          const f32x4 l2 = *(const f32x4*)&slt[q];
          const f32x4 dd = *(const f32x4*)&sDt[q];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pr = exp2_fast(fmaf(st[qb][4 * g + e], kScaleLog2, -l2[e]));
            st[qb][4 * g + e] = pr;
            dp[qb][4 * g + e] = pr * (dp[qb][4 * g + e] - dd[e]);
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 w, x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w[e] = pack_bf2(st[qb][8 * u + 2 * e], st[qb][8 * u + 2 * e + 1]);
            x[e] = pack_bf2(dp[qb][8 * u + 2 * e], dp[qb][8 * u + 2 * e + 1]);
          }
          pb[qb][u] = __builtin_bit_cast(bf16x8, w);
          sb[qb][u] = __builtin_bit_cast(bf16x8, x);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS: the transposing reads give lane
      // (dim d*32 + lane%32) the 8 queries qb*32 + 16u + 4*lhalf + {0..3, 8..11},
      // the order in which pb / sb hold them.
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const int r0 = qb * 32 + 16 * u + 4 * lhalf + tr_row;
            const i16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(dt + r0 * kLdsRow + voff[d][0]));
            const i16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(dt + (r0 + 8) * kLdsRow + voff[d][1]));
            const i16x8 dv8 = __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7);
            dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, dv8), pb[qb][u], dv[d], 0, 0, 0);
            const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(qt + r0 * kLdsRow + voff[d][0]));
            const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(qt + (r0 + 8) * kLdsRow + voff[d][1]));
            const i16x8 q8 = __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7);
            dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q8), sb[qb][u], dk[d], 0, 0, 0);
          }
    }
    }
    if (t + 1 < ntl && tid < kTR) {
      sl[cur ^ 1][tid] = nl2;
      sD[cur ^ 1][tid] = ndd;
    }
    vm_wait_all();
    __syncthreads();
  }

  if (key >= L) return;
  bf16_t* dkg = a.dqkv + ((int64_t)(1 * heads + head) * a.T + start + key) * kHeadDim;
  bf16_t* dvg = a.dqkv + ((int64_t)(2 * heads + head) * a.T + start + key) * kHeadDim;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = d * 32 + 8 * g + 4 * lhalf;
      *(u32x2*)(dkg + dim) = u32x2{pack_bf2(dk[d][4 * g] * 0.125f, dk[d][4 * g + 1] * 0.125f),
                                   pack_bf2(dk[d][4 * g + 2] * 0.125f, dk[d][4 * g + 3] * 0.125f)};
      *(u32x2*)(dvg + dim) = u32x2{pack_bf2(dv[d][4 * g], dv[d][4 * g + 1]),
                                   pack_bf2(dv[d][4 * g + 2], dv[d][4 * g + 3])};
    }
}

__global__ __launch_bounds__(64 * kBW) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_attn_bwd_dq(AttnBwdArgs a) {
  const int heads = a.heads;
  int head, s, q0;
  if (!bwd_block(a, head, s, q0)) return;
  const int64_t start = a.segs[2 * s];
  const int L = a.segs[2 * s + 1];
  const AttnBwdPtrs p = bwd_ptrs(a, head, start);
  const int64_t H = (int64_t)heads * kHeadDim;

  __shared__ __attribute__((aligned(1024))) bf16_t sk[2][kBT * kLdsRow];
  __shared__ __attribute__((aligned(1024))) bf16_t sv[2][kBT * kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // This lane's query (clamped): q and dO rows as the B operand, its lse and D.
  const int qrow = q0 + 32 * wave + lrow;
  const int qc = qrow < L ? qrow : L - 1;
  bf16x8 qf[4], df[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qf[kk] = *(const bf16x8*)(p.Q + qc * kHeadDim + kk * 16 + 8 * lhalf);
    df[kk] = *(const bf16x8*)(p.dO + qc * H + kk * 16 + 8 * lhalf);
  }
  const float l2 = p.lse[qc] * kLog2e;
  // D = rowsum(dO * O) of this query: this lane's 32 dims, then its partner's.
  // Written for the dK/dV kernel, which runs after this one.
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const bf16x8 of = *(const bf16x8*)(p.O + qc * H + kk * 16 + 8 * lhalf);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart += (float)df[kk][e] * (float)of[e];
  }
  const float dd = dpart + __shfl_xor(dpart, 32);
  if (lhalf == 0 && qrow < L) p.del[qrow] = dd;

  const uint32_t lds_k = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&sk[0][0];
  const uint32_t lds_v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&sv[0][0];
  auto gload = [&](int j, int buf) {
    tile_dma(p.K, kHeadDim, j * kBT, L, lds_k + (uint32_t)buf * kBT * kLdsRow * 2, lane, wave, wave_u);
    tile_dma(p.V, kHeadDim, j * kBT, L, lds_v + (uint32_t)buf * kBT * kLdsRow * 2, lane, wave, wave_u);
  };

  const int g16 = lane & 15;
  const int tr_row = g16 >> 2, tr_col = 4 * (g16 & 3);
  const int n0_lane = 16 * ((lane >> 4) & 1);
  int koff[4], voff[2][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = ((2 * kk + lhalf) ^ kSwz(lrow)) * 8;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 4 * lhalf + tr_row + 8 * h, col = d * 32 + n0_lane + tr_col;
      voff[d][h] = (((col >> 3) ^ kSwz(r)) * 8) + (col & 7);
    }

  f32x16 dq[2];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[d][r] = 0.f;

  const int ntk = (L + kBT - 1) / kBT;
  const bool wave_active = q0 + 32 * wave < L;
  gload(0, 0);
  vm_wait_all();
  __syncthreads();
  for (int t = 0; t < ntk; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntk) gload(t + 1, cur ^ 1);
    if (wave_active) {
      const bf16_t* kt = sk[cur];
      const bf16_t* vt = sv[cur];
      // S^T and dP^T, key x query: block kb holds keys t*64 + kb*32 + 8*(r/4)
      // + 4*lhalf + r%4 of this lane's query.
      f32x16 st[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { st[kb][r] = 0.f; dp[kb][r] = 0.f; }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 ka = *(const bf16x8*)(&kt[(kb * 32 + lrow) * kLdsRow + koff[kk]]);
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], st[kb], 0, 0, 0);
          const bf16x8 va = *(const bf16x8*)(&vt[(kb * 32 + lrow) * kLdsRow + koff[kk]]);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[kk], dp[kb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = exp2_fast(fmaf(st[kb][r], kScaleLog2, -l2));
      if ((t + 1) * kBT > L) {
        // Keys at or past L (a sequence's last key tile only): P = 0.  The
        // empty asm keeps this a branch; as selects it ran on every tile.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t * kBT + kb * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3) >= L) st[kb][r] = 0.f;
      }
      bf16x8 sb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[kb][r] = st[kb][r] * (dp[kb][r] - dd);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = pack_bf2(dp[kb][8 * u + 2 * e], dp[kb][8 * u + 2 * e + 1]);
          sb[kb][u] = __builtin_bit_cast(bf16x8, x);
        }
      }
      // dQ^T += K^T dS^T (K^T by the transposing reads, keys in the order sb holds them).
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const int r0 = kb * 32 + 16 * u + 4 * lhalf + tr_row;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kt + r0 * kLdsRow + voff[d][0]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kt + (r0 + 8) * kLdsRow + voff[d][1]));
            const i16x8 k8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k8), sb[kb][u], dq[d], 0, 0, 0);
          }
    }
    vm_wait_all();
    __syncthreads();
  }

  if (qrow >= L) return;
  bf16_t* dqg = a.dqkv + ((int64_t)(0 * heads + head) * a.T + start + qrow) * kHeadDim;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = d * 32 + 8 * g + 4 * lhalf;
      *(u32x2*)(dqg + dim) = u32x2{pack_bf2(dq[d][4 * g] * 0.125f, dq[d][4 * g + 1] * 0.125f),
                                   pack_bf2(dq[d][4 * g + 2] * 0.125f, dq[d][4 * g + 3] * 0.125f)};
    }
}

}  // namespace

hipError_t launch_attention_bwd(const AttnBwdArgs& a, hipStream_t st) {
  if (a.tile_cap <= 0 || a.T <= 0) return hipSuccess;
  // dQ first: it also writes D, which the dK/dV kernel reads.
  const int64_t nblk = a.tile_cap * a.heads * kBParts;
  hipLaunchKernelGGL(k_attn_bwd_dq, dim3((unsigned)nblk), dim3(64 * kBW), 0, st, a);
  hipLaunchKernelGGL(k_attn_bwd_dkv, dim3((unsigned)nblk), dim3(64 * kBW), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.tile_cap <= 0 || a.T <= 0) return hipSuccess;
  const int64_t nblk = a.tile_cap * a.heads;
  hipLaunchKernelGGL(k_attention, dim3((unsigned)nblk), dim3(64 * kNW), 0, st, a);
  return hipGetLastError();
}

}  // namespace esm

namespace esm {

hipError_t launch_biased_attention(const BiasedAttnArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.N <= 0 || a.L <= 0 || a.heads <= 0) return hipSuccess;
  const int64_t nblk = (int64_t)a.B * a.N * a.qtiles * a.heads;
  const int mode = kBias | (a.mask ? kMask : 0) | (a.pair ? kPair : 0) |
                   ((a.mask || a.pair) && a.L % 8 == 0 ? kLds : (a.L % 4 == 0 ? kVec : 0));
  const dim3 grid((unsigned)nblk), block(64 * kNW);
  switch (mode) {
#define ESM_BIASED_CASE(m) \
    case m: hipLaunchKernelGGL(k_biased_attention<m>, grid, block, 0, st, a); break;
    ESM_BIASED_CASE(kBias)
    ESM_BIASED_CASE(kBias | kMask)
    ESM_BIASED_CASE(kBias | kPair)
    ESM_BIASED_CASE(kBias | kMask | kPair)
    ESM_BIASED_CASE(kBias | kVec)
    ESM_BIASED_CASE(kBias | kMask | kVec)
    ESM_BIASED_CASE(kBias | kPair | kVec)
    ESM_BIASED_CASE(kBias | kMask | kPair | kVec)
    ESM_BIASED_CASE(kBias | kMask | kLds)
    ESM_BIASED_CASE(kBias | kPair | kLds)
    ESM_BIASED_CASE(kBias | kMask | kPair | kLds)
#undef ESM_BIASED_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace esm
