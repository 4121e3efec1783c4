// Memory-bound pieces of the encoder forward on gfx950:
//   * segment table: per-sequence extents, per-row positions and the attention
//     query-tile list, built on the device from cu_seqlens (no host sync),
//   * embedding gather X0 = E[ids],
//   * row LayerNorm.
#include "common.h"

namespace esm {

namespace {

constexpr int kSegThreads = 1024;

// Sequence extents and the list of 256-row query tiles, longest sequence
// first ([BIO-ACC] 3.2: cu_seqlens = cumsum([0] + lengths); sequence s owns
// rows cu[s] .. cu[s+1]-1).  One workgroup: a counting sort of the tiles by
// sequence length (bucket = max_positions - length, so long sequences come
// first); tiles of equal-length sequences may come in any order.  Every value
// read from the device array is clamped, so inconsistent input cannot lead to
// an out-of-range row.
__global__ __launch_bounds__(kSegThreads) void k_segment_table(int layout, const int32_t* __restrict__ lens,
                                                               int32_t B, int64_t rows, int32_t S, int32_t nbins,
                                                               SegOut out) {
  extern __shared__ int32_t sh[];
  int32_t* hist = sh;           // [nbins]
  int32_t* part = sh + nbins;   // [kSegThreads]
  const int tid = threadIdx.x;
  for (int i = tid; i < nbins; i += kSegThreads) hist[i] = 0;
  __syncthreads();
  for (int s = tid; s < B; s += kSegThreads) {
    int64_t start, len;
    if (layout == 0) {
      int64_t a = lens[s], b = lens[s + 1];
      a = a < 0 ? 0 : (a > rows ? rows : a);
      b = b < a ? a : (b > rows ? rows : b);
      start = a;
      len = b - a;
    } else {
      int64_t l = lens[s];
      l = l < 0 ? 0 : (l > S ? S : l);
      start = (int64_t)s * S;
      len = l;
    }
    out.segs[2 * s] = (int32_t)start;
    out.segs[2 * s + 1] = (int32_t)len;
    const int64_t nt = (len + kAttnTileRows - 1) / kAttnTileRows;
    if (nt) atomicAdd(&hist[nbins - 1 - (int)(len < nbins - 1 ? len : nbins - 1)], (int32_t)nt);
  }
  __syncthreads();
  // Exclusive scan of the histogram: per-thread serial chunk, then a block scan.
  const int per = (nbins + kSegThreads - 1) / kSegThreads;
  const int b0 = tid * per;
  const int b1 = b0 + per < nbins ? b0 + per : nbins;
  int32_t local = 0;
  for (int i = b0; i < b1; ++i) local += hist[i];
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kSegThreads; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - local;
  for (int i = b0; i < b1; ++i) {
    const int32_t c = hist[i];
    hist[i] = run;
    run += c;
  }
  const int32_t total = part[kSegThreads - 1];
  __syncthreads();
  for (int s = tid; s < B; s += kSegThreads) {
    const int32_t len = out.segs[2 * s + 1];
    const int32_t nt = (len + kAttnTileRows - 1) / kAttnTileRows;
    if (!nt) continue;
    const int32_t base = atomicAdd(&hist[nbins - 1 - (len < nbins - 1 ? len : nbins - 1)], nt);
    for (int32_t i = 0; i < nt; ++i) {
      const int64_t idx = (int64_t)base + i;
      if (idx < out.tile_cap) {
        out.tiles[2 * idx] = s;
        out.tiles[2 * idx + 1] = i * kAttnTileRows;
      }
    }
  }
  if (tid == 0) *out.ntiles = (int32_t)(total < out.tile_cap ? total : out.tile_cap);
}

// Position of every row inside its sequence (rotary positions restart at 0 in
// each sequence); -1 marks padding rows of a bshd batch.
__global__ void k_positions(int layout, const int32_t* __restrict__ lens, int32_t B, int64_t rows, int32_t S,
                            int32_t* __restrict__ pos) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows) return;
  if (B <= 0) {
    pos[t] = -1;
    return;
  }
  if (layout == 0) {
    // last s in [0, B) with cu[s] <= t
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)lens[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int64_t a = lens[lo], b = lens[lo + 1];
    pos[t] = (a <= t && t < b) ? (int32_t)(t - a) : -1;
  } else {
    const int64_t b = t / S, p = t % S;
    int64_t l = lens[b];
    l = l < 0 ? 0 : (l > S ? S : l);
    pos[t] = p < l ? (int32_t)p : -1;
  }
}

// X0 = E[ids] ([BIO-ACC] 3.2 PackedEsm.forward: embedding of the packed ids).
__global__ void k_embed(const int32_t* __restrict__ ids, const bf16_t* __restrict__ table, int32_t vocab,
                        bf16_t* __restrict__ x, int64_t T, int32_t H) {
  const int chunks = H / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * chunks) return;
  const int64_t t = i / chunks;
  const int c = (int)(i % chunks);
  int id = ids[t];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  *(u32x4*)(x + t * H + c * 8) = *(const u32x4*)(table + (int64_t)id * H + c * 8);
}

// LayerNorm chunk partials of rows of x (optionally gathered first from the
// embedding, X0 = E[ids]): one wave per row.  The row is read, and X0 written
// when gathering, in 16-byte pieces (a wave covers 1 KB per instruction) and
// staged in the wave's own LDS region; item i = 8 * chunk + leaf of the row
// (lanes i mod 64) then takes its leaf's 32 values and the tree of ln_leaf /
// ln_combine exactly as the GEMM epilogue that writes a residual stream
// evaluates them, so a row gives the same partials whichever of the two
// produced them.  Leaf bit 0 = h, bits 1..2 = w.
__global__ __launch_bounds__(256) void k_row_stats(const int32_t* __restrict__ ids, const bf16_t* __restrict__ table,
                                                   int32_t vocab, bf16_t* __restrict__ x, int64_t T, int32_t H,
                                                   float2* __restrict__ stats) {
  extern __shared__ __attribute__((aligned(16))) unsigned char row_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  if (t >= T) return;  // the whole wave; no workgroup barrier follows
  bf16_t* row = (bf16_t*)row_lds + (int64_t)wave * H;
  const bf16_t* src = x + t * H;
  if (ids) {
    int id = ids[t];
    id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
    src = table + (int64_t)id * H;
  }
  for (int c = lane; c < H / 8; c += 64) {
    const u32x4 u = *(const u32x4*)(src + 8 * c);
    if (ids) *(u32x4*)(x + t * H + 8 * c) = u;
    *(u32x4*)(row + 8 * c) = u;
  }
  // The row's LDS writes are visible to every lane of the wave.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int chunks = (H + 255) / 256;
  const int items = (chunks * 8 + 63) & ~63;  // whole waves: every lane meets the exchanges
  for (int it = lane; it < items; it += 64) {
    const int c = it >> 3, leaf = it & 7;
    const int w = leaf >> 1, h = leaf & 1;
    const int c0 = 256 * c;
    const int cw = H - c0 < 256 ? H - c0 : 256;
    const bool valid = c < chunks && 64 * w < cw;
    LnPart p{0.f, 0.f, 0.f};
    if (valid) {
      float v[32];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 u = *(const u32x2*)(row + c0 + 64 * w + 32 * j + 8 * q + 4 * h);
          v[16 * j + 4 * q + 0] = bflo(u[0]);
          v[16 * j + 4 * q + 1] = bfhi(u[0]);
          v[16 * j + 4 * q + 2] = bflo(u[1]);
          v[16 * j + 4 * q + 3] = bfhi(u[1]);
        }
      p = ln_leaf(v);
    }
    // (w, 0) with (w, 1); then waves (0, 1) and (2, 3); then the two pairs.
    // Each pair of lanes computes combine(lower, upper) identically.
#pragma unroll
    for (int off = 1; off <= 4; off <<= 1) {
      LnPart o{__shfl_xor(p.n, off), __shfl_xor(p.m, off), __shfl_xor(p.M2, off)};
      p = (leaf & off) ? ln_combine(o, p) : ln_combine(p, o);
    }
    if (leaf == 0 && c < chunks) stats[(int64_t)c * T + t] = make_float2(p.m, p.M2);
  }
}

// Folded LayerNorm weight of one output row n per workgroup:
// wf[n, k] = bf16(gamma_k w[n, k]) (the product of two bf16 values is exact
// in fp32, then one rounding), c_n = sum_k wf[n, k] and
// d_n = b_n + sum_k beta_k w[n, k], summed in fp64 over a fixed tree.
__global__ __launch_bounds__(256) void k_fold_weight(const bf16_t* __restrict__ w, const bf16_t* __restrict__ gamma,
                                                     const bf16_t* __restrict__ beta, const bf16_t* __restrict__ bias,
                                                     int32_t K, bf16_t* __restrict__ wf, float2* __restrict__ cd) {
  const int64_t n = blockIdx.x;
  double sc = 0.0, sd = 0.0;
  for (int k = threadIdx.x; k < K; k += 256) {
    const float wv = bf2f(w[n * K + k]);
    const bf16_t f = f2bf(bf2f(gamma[k]) * wv);
    wf[n * K + k] = f;
    sc += (double)bf2f(f);
    sd += (double)bf2f(beta[k]) * (double)wv;
  }
  __shared__ double rc[256], rd[256];
  rc[threadIdx.x] = sc;
  rd[threadIdx.x] = sd;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) {
      rc[threadIdx.x] += rc[threadIdx.x + off];
      rd[threadIdx.x] += rd[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double b = bias ? (double)bf2f(bias[n]) : 0.0;
    cd[n] = make_float2((float)rc[0], (float)(rd[0] + b));
  }
}

// Rows per wave: two for rows of up to 2560 values (all of a wave's rows are
// loaded before the first is reduced, so their memory latencies overlap:
// 33 -> 30 us per 650M LayerNorm), and for the E4M3 output fewer workgroups
// fold their amax into the tensor's one amax word.
template <int CH, bool OUT8>
constexpr int ln_rows_per_wave() { return CH <= 5 ? 2 : 1; }

// Row LayerNorm, one wave per row: mean, then the biased variance from the
// centred values held in registers, y = (x - mean) * rsqrt(var + eps) * g + b
// ([BIO-ACC] 3.1 layernorm; [TE-RU] LayerNormLinear / LayerNormMLP).  With
// OUT8 the normalised row is cast to E4M3 with the tensor's delayed scale and
// its amax recorded, the quantiser that feeds an FP8 GEMM ([BIO-ACC] 2.1).
// With MX the normalised row goes straight to MXFP4: a block of 32 values is
// the 4 consecutive chunks of lanes 4k .. 4k + 3, whose amax two lane
// exchanges combine; each lane writes its 8 codes (4 bytes) and lane 4k the
// block's scale (codes [M, H / 2], scales in the esm_mxfp4_quantize layout).
template <int CH, bool OUT8, bool MX = false>
__global__ __launch_bounds__(256) void k_layernorm(const bf16_t* __restrict__ x, const bf16_t* __restrict__ gamma,
                                                   const bf16_t* __restrict__ beta, bf16_t* __restrict__ y,
                                                   int64_t M, int32_t H, float eps, E4m3Out q,
                                                   uint8_t* __restrict__ mx_codes = nullptr,
                                                   uint8_t* __restrict__ mx_scales = nullptr) {
  constexpr int RW = ln_rows_per_wave<CH, OUT8>();
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t)blockIdx.x * (4 * RW) + (threadIdx.x >> 6);
  if constexpr (!OUT8) {
    if (row0 >= M) return;
  }
  const int chunks = H / 8;
  float s8 = 1.0f, amax = 0.0f;
  if constexpr (OUT8) s8 = q.scale[0];
  // Every wave reaches the block amax reduction below; a wave past the last
  // row works on the last row and stores nothing.
  u32x4 raw[RW][CH], graw[CH], braw[CH];
  bool count[RW];  // E4M3 output: the row enters the amax (in range, not padding)
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t row_ = row0 + 4 * r;
    const int64_t row = row_ < M ? row_ : M - 1;
    const bf16_t* xr = x + row * H;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) raw[r][i] = *(const u32x4*)(xr + c * 8);
    }
    count[r] = true;
    if constexpr (OUT8) count[r] = row_ < M && (q.pos == nullptr || q.pos[row] >= 0);
  }
  // gamma and beta: loaded with the rows when a wave has several of them,
  // else at the output (fewer live registers)
  auto load_gb = [&](int i) {
    const int c = lane + 64 * i;
    if (c < chunks) {
      graw[i] = *(const u32x4*)(gamma + c * 8);
      braw[i] = *(const u32x4*)(beta + c * 8);
    }
  };
  if constexpr (RW > 1) {
#pragma unroll
    for (int i = 0; i < CH; ++i) load_gb(i);
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t row_ = row0 + 4 * r;
    const bool active = row_ < M;
    const int64_t row = active ? row_ : M - 1;
    float v[CH][8];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        const u32x4 w = raw[r][i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[i][2 * e] = bflo(w[e]);
          v[i][2 * e + 1] = bfhi(w[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += v[i][e];
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    const float mean = sum / (float)H;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[i][e] -= mean;
          sq += v[i][e] * v[i][e];
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
    const float rstd = 1.0f / sqrtf(sq / (float)H + eps);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        if constexpr (RW == 1) load_gb(i);
        const u32x4 g = graw[i];
        const u32x4 b = braw[i];
        float o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[2 * e] = v[i][2 * e] * rstd * bflo(g[e]) + bflo(b[e]);
          o[2 * e + 1] = v[i][2 * e + 1] * rstd * bfhi(g[e]) + bfhi(b[e]);
        }
        if constexpr (MX) {
          float am = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(o[e]));
          am = fmaxf(am, __shfl_xor(am, 1));
          am = fmaxf(am, __shfl_xor(am, 2));
          const int ex = mx_block_exponent(am);
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) word |= e2m1_pair(o[2 * e], o[2 * e + 1], ex) << (8 * e);
          if (active) {
            *(uint32_t*)(mx_codes + row * (H / 2) + c * 4) = word;
            if ((lane & 3) == 0) mx_scales[mx_scale_offset(row, c / 4, M + (M & 1))] = (uint8_t)(ex + 127);
          }
        } else if constexpr (OUT8) {
          const float lo[4] = {o[0], o[1], o[2], o[3]}, hi[4] = {o[4], o[5], o[6], o[7]};
          if (count[r])
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(o[e]));
          if (active) *(u32x2*)(q.y + row * H + c * 8) = u32x2{pack_e4m3x4(lo, s8), pack_e4m3x4(hi, s8)};
        } else {
          *(u32x4*)(y + row * H + c * 8) =
              u32x4{pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]), pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7])};
        }
      }
    }
  }
  if constexpr (OUT8) {
    __shared__ float red[4];
    record_amax_block<4>(q.amax, amax, red);
  }
}

// dst [rows_pad, cols] = src [rows, cols] followed by zero rows (src NULL:
// all zero).  Pads the tied decoder weight and its bias to a GEMM-sized
// number of output columns.
__global__ void k_pad_rows(const bf16_t* __restrict__ src, int32_t rows, int32_t cols, bf16_t* __restrict__ dst,
                           int32_t rows_pad) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows_pad * cols) return;
  dst[i] = (src && i < (int64_t)rows * cols) ? src[i] : (bf16_t)0;
}

// dst [T, cols] = the first cols columns of src [T, ld_src].
__global__ void k_take_cols(const bf16_t* __restrict__ src, int32_t ld_src, bf16_t* __restrict__ dst, int64_t T,
                            int32_t cols) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * cols) return;
  const int64_t t = i / cols;
  dst[i] = src[t * ld_src + (i - t * cols)];
}

// Sequence-level embedding: out[s, :] = mean of x over the rows of sequence s
// (segs[s] = first row, length), fp32; 0 for an empty sequence.  One
// workgroup per (sequence, 64-column slab), so that many workgroups share the
// sequence's rows: lane l of wave w reads row 8 w + l / 8 (+ 32 i) at the
// slab's 16-byte chunk l % 8 and sums in fp32; the 8 row lanes of a chunk are
// added by lane exchange, then the four waves in a fixed order, so the
// result does not depend on scheduling.
__global__ __launch_bounds__(256) void k_segment_mean(const bf16_t* __restrict__ x, const int32_t* __restrict__ segs,
                                                      int32_t H, float* __restrict__ out) {
  __shared__ float part[4][64];
  const int s = blockIdx.x, c0 = blockIdx.y * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t start = segs[2 * s];
  const int L = segs[2 * s + 1];
  const int ch = lane & 7;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int r = wave * 8 + (lane >> 3); r < L; r += 32) {
    const u32x4 w = *(const u32x4*)(x + (start + r) * H + c0 + ch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bflo(w[e]);
      acc[2 * e + 1] += bfhi(w[e]);
    }
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (lane < 8)
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave][lane * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int col = threadIdx.x;
    const float inv = L > 0 ? 1.0f / (float)L : 0.0f;
    out[(int64_t)s * H + c0 + col] = ((part[0][col] + part[1][col]) + (part[2][col] + part[3][col])) * inv;
  }
}

}  // namespace

hipError_t launch_segment_table(int layout, const int32_t* lens, int32_t B, int64_t rows, int32_t S,
                                int32_t max_positions, const SegOut& out, hipStream_t st) {
  // Lengths above the last bin share it (they still sort first).
  const int32_t nbins = (max_positions < 8192 ? max_positions : 8192) + 1;
  const size_t shmem = sizeof(int32_t) * ((size_t)nbins + kSegThreads);
  hipLaunchKernelGGL(k_segment_table, dim3(1), dim3(kSegThreads), shmem, st, layout, lens, B, rows, S, nbins, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows <= 0) return e;
  hipLaunchKernelGGL(k_positions, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, layout, lens, B, rows, S,
                     out.pos);
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t* ids, const bf16_t* table, int32_t vocab, bf16_t* x, int64_t T, int32_t H,
                        hipStream_t st) {
  const int64_t n = T * (H / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_embed, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ids, table, vocab, x, T, H);
  return hipGetLastError();
}

hipError_t launch_row_stats(const int32_t* ids, const bf16_t* table, int32_t vocab, bf16_t* x, int64_t T, int32_t H,
                            float2* stats, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  // One wave per row, its row staged in LDS (2 H bytes per wave): four waves
  // per workgroup up to H = 8192, one up to 32768.
  if (H % 64 || H > 32768) return hipErrorInvalidValue;
  const int wpb = H <= 8192 ? 4 : 1;
  const size_t lds = (size_t)wpb * H * 2;
  hipLaunchKernelGGL(k_row_stats, dim3((unsigned)((T + wpb - 1) / wpb)), dim3(64 * wpb), lds, st, ids, table, vocab,
                     x, T, H, stats);
  return hipGetLastError();
}

hipError_t launch_fold_weight(const bf16_t* w, const bf16_t* gamma, const bf16_t* beta, const bf16_t* bias,
                              int32_t N, int32_t K, bf16_t* wf, float2* cd, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fold_weight, dim3((unsigned)N), dim3(256), 0, st, w, gamma, beta, bias, K, wf, cd);
  return hipGetLastError();
}

template <int CH, bool OUT8>
void launch_ln(const bf16_t* x, const bf16_t* gamma, const bf16_t* beta, bf16_t* y, int64_t M, int32_t H, float eps,
               const E4m3Out& q, hipStream_t st) {
  const int rows = 4 * ln_rows_per_wave<CH, OUT8>();  // rows per workgroup
  const unsigned grid = (unsigned)((M + rows - 1) / rows);
  hipLaunchKernelGGL((k_layernorm<CH, OUT8>), dim3(grid), dim3(256), 0, st, x, gamma, beta, y, M, H, eps, q);
}

template <bool OUT8>
hipError_t layernorm_ch(const bf16_t* x, const bf16_t* gamma, const bf16_t* beta, bf16_t* y, int64_t M, int32_t H,
                        float eps, const E4m3Out& q, hipStream_t st) {
  const int ch = (H / 8 + 63) / 64;
  if (ch <= 1) launch_ln<1, OUT8>(x, gamma, beta, y, M, H, eps, q, st);
  else if (ch <= 2) launch_ln<2, OUT8>(x, gamma, beta, y, M, H, eps, q, st);
  else if (ch <= 3) launch_ln<3, OUT8>(x, gamma, beta, y, M, H, eps, q, st);
  else if (ch <= 5) launch_ln<5, OUT8>(x, gamma, beta, y, M, H, eps, q, st);
  else if (ch <= 8) launch_ln<8, OUT8>(x, gamma, beta, y, M, H, eps, q, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_layernorm_mx(const bf16_t* x, const bf16_t* gamma, const bf16_t* beta, uint8_t* codes,
                               uint8_t* scales, int64_t M, int32_t H, float eps, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (H % 256) return hipErrorInvalidValue;
  const E4m3Out none{nullptr, nullptr, nullptr, nullptr};
  const int ch = (H / 8 + 63) / 64;
  auto go = [&](auto kern, int rw) {
    const int rows = 4 * rw;
    hipLaunchKernelGGL(kern, dim3((unsigned)((M + rows - 1) / rows)), dim3(256), 0, st, x, gamma, beta,
                       (bf16_t*)nullptr, M, H, eps, none, codes, scales);
  };
  if (ch <= 1) go(k_layernorm<1, false, true>, ln_rows_per_wave<1, false>());
  else if (ch <= 2) go(k_layernorm<2, false, true>, ln_rows_per_wave<2, false>());
  else if (ch <= 3) go(k_layernorm<3, false, true>, ln_rows_per_wave<3, false>());
  else if (ch <= 5) go(k_layernorm<5, false, true>, ln_rows_per_wave<5, false>());
  else if (ch <= 8) go(k_layernorm<8, false, true>, ln_rows_per_wave<8, false>());
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_layernorm(const bf16_t* x, const bf16_t* gamma, const bf16_t* beta, bf16_t* y, int64_t M,
                            int32_t H, float eps, const E4m3Out& q, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (q.y) return layernorm_ch<true>(x, gamma, beta, y, M, H, eps, q, st);
  return layernorm_ch<false>(x, gamma, beta, y, M, H, eps, q, st);
}

}  // namespace esm

namespace esm {

hipError_t launch_pad_rows(const bf16_t* src, int32_t rows, int32_t cols, bf16_t* dst, int32_t rows_pad,
                           hipStream_t st) {
  const int64_t n = (int64_t)rows_pad * cols;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pad_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, rows, cols, dst, rows_pad);
  return hipGetLastError();
}

hipError_t launch_take_cols(const bf16_t* src, int32_t ld_src, bf16_t* dst, int64_t T, int32_t cols, hipStream_t st) {
  const int64_t n = T * cols;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_take_cols, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, ld_src, dst, T, cols);
  return hipGetLastError();
}

hipError_t launch_segment_mean(const bf16_t* x, const int32_t* segs, int32_t B, int32_t H, float* out,
                               hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (H % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_segment_mean, dim3((unsigned)B, (unsigned)(H / 64)), dim3(256), 0, st, x, segs, H, out);
  return hipGetLastError();
}

namespace {
__global__ void k_rebase_cu(const int32_t* __restrict__ cu, int32_t b0, int32_t n, int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i <= n) out[i] = cu[b0 + i] - cu[b0];
}
}  // namespace

hipError_t launch_rebase_cu(const int32_t* cu, int32_t b0, int32_t n, int32_t* out, hipStream_t st) {
  if (n < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rebase_cu, dim3((unsigned)((n + 256) / 256)), dim3(256), 0, st, cu, b0, n, out);
  return hipGetLastError();
}

}  // namespace esm
