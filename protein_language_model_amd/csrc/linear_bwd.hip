// Backward helpers for gfx950: a bf16 transpose that zero-pads the rows it
// produces and a deterministic column sum (the linear layers' backward), and
// the LayerNorm backward.
//
// For y = x W^T + b (x [M, K], W [N, K], y [M, N]) and an incoming gradient
// dy, the backward is dx = dy W, dW = dy^T x and db = the column sums of dy
// (the linears of the encoder layer; the pages time training, [BIO-ACC] 3.2
// and 6).  dx and dW run on the library's MFMA GEMM (which computes a B^T for
// row-major a [M', K'] and B [N', K']): dx = dy (W^T)^T reads W^T [K, N],
// written here; dW reads dy and x as they are, through the GEMM's
// contraction-major split-K mode.  The E4M3 / E5M2 weight gradient still takes
// byte transposes of both operands (k_transpose8_pad), rows past M zero.
#include "common.h"

namespace esm {

namespace {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Chunk swizzle of the staged tile: 16-byte chunk ch of tile row r sits at
// chunk ch ^ tp_swz(r).  It keeps each pair of chunks (2a, 2a + 1) together
// and gives the four same-parity rows that one half-wave's transposing read
// touches ({b, b + 2, b + 8, b + 10} + 4 h + 32 s) four different pairs, so
// that read, like the row-wise 16-byte writes, is free of bank conflicts
// (64 banks of 4 bytes, checked by simulating the bank map).
__device__ __forceinline__ int tp_swz(int r) { return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)); }

// out[c, r] = in[r, c] for r < R, 0 for R <= r < Rp; in [R, C] row-major,
// out [C, Rp].  One 256-thread workgroup per 64 x 64 tile: the tile's rows go
// to LDS as 16-byte chunks, and gfx950's transposing LDS read
// (ds_read_b64_tr_b16: in a group of 16 lanes, lane j addresses four
// consecutive values of row k0 + j / 4 at columns n0 + 4 (j % 4), and lane i
// receives column n0 + i of rows k0 .. k0 + 3) hands each lane four
// consecutive values of one output row; two reads make a 16-byte store, and
// the four groups of a wave store 64 contiguous bytes of each of their 16
// output rows.  C is a multiple of 64; Rp a multiple of 64 and >= R.
__global__ __launch_bounds__(256) void k_transpose_pad(const bf16_t* __restrict__ in, int64_t R, int32_t C,
                                                       bf16_t* __restrict__ out, int64_t Rp) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64 * 64];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // thread t: chunk t % 8 of rows t / 8 and t / 8 + 32 (zeros past R), both
  // loads in flight together
  {
    const int ra = t >> 3, rb = ra + 32, ch = t & 7;
    u32x4 wa = {0u, 0u, 0u, 0u}, wb = {0u, 0u, 0u, 0u};
    if (r0 + rb < R) {
      wa = *(const u32x4*)(in + (r0 + ra) * C + c0 + 8 * ch);
      wb = *(const u32x4*)(in + (r0 + rb) * C + c0 + 8 * ch);
    } else if (r0 + ra < R) {
      wa = *(const u32x4*)(in + (r0 + ra) * C + c0 + 8 * ch);
    }
    *(u32x4*)(tile + ra * 64 + 8 * (ch ^ tp_swz(ra))) = wa;
    *(u32x4*)(tile + rb * 64 + 8 * (ch ^ tp_swz(rb))) = wb;
  }
  __syncthreads();
  // wave w: output rows c0 + 16 w + i (i = lane % 16); group q = lane / 16 and
  // pass s: output columns r0 + 8 (q + 4 s) .. + 7.
  const int i = lane & 15, q = lane >> 4;
  const int col = 16 * wave + 4 * (i & 3);  // this lane's address: tile column
  const int64_t orow = c0 + 16 * wave + i;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k0 = 8 * (q + 4 * s);
    i16x4 v[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = k0 + 4 * hh + (i >> 2);  // this lane's address: tile row
      const bf16_t* p = tile + r * 64 + 8 * ((col >> 3) ^ tp_swz(r)) + (col & 7);
      v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    }
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 w = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
    *(u32x4*)(out + orow * Rp + r0 + k0) = __builtin_bit_cast(u32x4, w);
  }
}

constexpr int kSumRows = 1024;  // rows per partial column sum

// part[chunk, n] = sum of dy[m, n] over the chunk's rows m (fp32, fixed
// order): thread t adds 8 columns (one 16-byte load per row) of rows
// t / 8 + 32 i, then the 32 row groups are added in LDS in a fixed tree.
__global__ __launch_bounds__(256) void k_colsum_partial(const bf16_t* __restrict__ dy, int64_t M, int32_t N,
                                                        float* __restrict__ part) {
  __shared__ float red[32][65];
  const int64_t m0 = (int64_t)blockIdx.x * kSumRows;
  const int n0 = blockIdx.y * 64;
  const int t = threadIdx.x, cg = t & 7, rg = t >> 3;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Eight rows' loads in flight at a time; the adds keep the row order.
  for (int i0 = 0; i0 < kSumRows / 32; i0 += 8) {
    u32x4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t m = m0 + rg + 32 * (i0 + u);
      w[u] = m < M ? *(const u32x4*)(dy + m * N + n0 + cg * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (m0 + rg + 32 * (i0 + u) < M) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bflo(w[u][e]);
          acc[2 * e + 1] += bfhi(w[u][e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][cg * 8 + e] = acc[e];
  __syncthreads();
  for (int s = 16; s >= 1; s >>= 1) {
    // 64 columns x s row groups: thread t < 64 s adds row group g + s into g
    for (int i = t; i < 64 * s; i += 256) {
      const int g = i / 64, c = i % 64;
      red[g][c] += red[g + s][c];
    }
    __syncthreads();
  }
  if (t < 64) part[(int64_t)blockIdx.x * N + n0 + t] = red[0][t];
}

// dgamma[n] / dbeta[n] = sums over chunks of part[chunk, 0, n] / part[chunk, 1, n].
__global__ __launch_bounds__(256) void k_ln_cols_final(const float* __restrict__ part, int64_t chunks, int32_t H,
                                                       float* __restrict__ dgamma, float* __restrict__ dbeta) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= 2 * H) return;
  float s = 0.f;
  for (int64_t c = 0; c < chunks; ++c) s += part[c * 2 * H + n];
  if (n < H) dgamma[n] = s;
  else dbeta[n - H] = s;
}

// db[n] = sum over chunks of part[chunk * stride + n], in chunk order.
__global__ __launch_bounds__(256) void k_colsum_final(const float* __restrict__ part, int64_t chunks, int32_t N,
                                                      int32_t stride, float* __restrict__ db) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int64_t c = 0; c < chunks; ++c) s += part[c * stride + n];
  db[n] = s;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ------------------------------------------------------------ LayerNorm backward
//
// For y = gamma * (x - mu) r + beta per row (r = 1 / sqrt(var + eps), biased
// variance) and an incoming gradient dy: with xh = (x - mu) r and g = dy gamma,
// dx = r (g - mean(g) - xh mean(g xh)); dgamma and dbeta are the column sums
// of dy xh and dy.  k_ln_bwd_rows: one wave per row (lane l holds chunks
// l, l + 64, ... of 8 values), two-pass mean and variance in fp32 as the
// forward takes them, dx, and the row's mu and r for the column pass;
// k_ln_bwd_cols: per 1024-row chunk and 64 columns, the sums of dy xh and dy
// (the layout and fixed order of k_colsum_partial); k_colsum_final adds the
// chunks.

constexpr int kLnMaxCh = 8;  // chunks of 8 per lane: H <= 4096

// kLnMaxCh here is the number of 8-value chunks per lane (H <= 512 kLnMaxCh),
// a template argument so that the row lives in as few registers as H needs.
template <int kLnMaxCh>
__global__ __launch_bounds__(256) void k_ln_bwd_rows(const bf16_t* __restrict__ x, const bf16_t* __restrict__ gamma,
                                                     const bf16_t* __restrict__ dy, const bf16_t* __restrict__ dres,
                                                     bf16_t* __restrict__ dx, float* __restrict__ stats, int64_t M,
                                                     int32_t H, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;   // whole wave: no barrier below
  const int nch = H / 8;
  const bf16_t* xr = x + m * H;
  const bf16_t* gr = dy + m * H;
  float xv[kLnMaxCh][8], gv[kLnMaxCh][8];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kLnMaxCh; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      const u32x4 a = *(const u32x4*)(xr + 8 * c);
      const u32x4 d = *(const u32x4*)(gr + 8 * c);
      const u32x4 w = *(const u32x4*)(gamma + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[j][2 * e] = bflo(a[e]);
        xv[j][2 * e + 1] = bfhi(a[e]);
        gv[j][2 * e] = bflo(d[e]) * bflo(w[e]);
        gv[j][2 * e + 1] = bfhi(d[e]) * bfhi(w[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s += xv[j][e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { xv[j][e] = 0.f; gv[j][e] = 0.f; }
    }
  }
  const float inv_h = 1.0f / (float)H;
  const float mu = wave_sum(s) * inv_h;
  float v = 0.f;
#pragma unroll
  for (int j = 0; j < kLnMaxCh; ++j)
    if (lane + 64 * j < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = xv[j][e] - mu;
        v += t * t;
      }
    }
  const float r = rsqrtf(wave_sum(v) * inv_h + eps);
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int j = 0; j < kLnMaxCh; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xv[j][e] = (xv[j][e] - mu) * r;   // xh (0 past the row: not stored)
      s1 += gv[j][e];
      s2 += gv[j][e] * xv[j][e];
    }
  const float m1 = wave_sum(s1) * inv_h, m2 = wave_sum(s2) * inv_h;
  bf16_t* dr = dx + m * H;
#pragma unroll
  for (int j = 0; j < kLnMaxCh; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      float d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = r * (gv[j][e] - m1 - xv[j][e] * m2);
      if (dres) {   // a residual branch's gradient joins this one, in fp32, rounded once
        const u32x4 q = *(const u32x4*)(dres + m * H + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d[2 * e] += bflo(q[e]);
          d[2 * e + 1] += bfhi(q[e]);
        }
      }
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf2(d[2 * e], d[2 * e + 1]);
      *(u32x4*)(dr + 8 * c) = o;
    }
  }
  if (lane == 0) {
    stats[2 * m] = mu;
    stats[2 * m + 1] = r;
  }
}

// part[chunk, 0, n] = sum of dy xh, part[chunk, 1, n] = sum of dy over the
// chunk's rows (fp32, fixed order; the tree of k_colsum_partial).
__global__ __launch_bounds__(256) void k_ln_bwd_cols(const bf16_t* __restrict__ x, const bf16_t* __restrict__ dy,
                                                     const float* __restrict__ stats, int64_t M, int32_t H,
                                                     float* __restrict__ part) {
  __shared__ float red[2][32][65];
  const int64_t m0 = (int64_t)blockIdx.x * kSumRows;
  const int n0 = blockIdx.y * 64;
  const int t = threadIdx.x, cg = t & 7, rg = t >> 3;
  float ag[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, ab[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < kSumRows / 32; ++i) {
    const int64_t m = m0 + rg + 32 * i;
    if (m < M) {
      const float mu = stats[2 * m], r = stats[2 * m + 1];
      const u32x4 a = *(const u32x4*)(x + m * H + n0 + cg * 8);
      const u32x4 d = *(const u32x4*)(dy + m * H + n0 + cg * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d0 = bflo(d[e]), d1 = bfhi(d[e]);
        ag[2 * e] += d0 * ((bflo(a[e]) - mu) * r);
        ag[2 * e + 1] += d1 * ((bfhi(a[e]) - mu) * r);
        ab[2 * e] += d0;
        ab[2 * e + 1] += d1;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][rg][cg * 8 + e] = ag[e];
    red[1][rg][cg * 8 + e] = ab[e];
  }
  __syncthreads();
  for (int s = 16; s >= 1; s >>= 1) {
    for (int i = t; i < 128 * s; i += 256) {
      const int k = i / (64 * s), rem = i % (64 * s), g = rem / 64, c = rem % 64;
      red[k][g][c] += red[k][g + s][c];
    }
    __syncthreads();
  }
  if (t < 128) part[((int64_t)blockIdx.x * 2 + (t >> 6)) * H + n0 + (t & 63)] = red[t >> 6][0][t & 63];
}

// out[i] = bf16(sum over s of part[s * n + i]) in slice order (split-K
// partial sums of the dW GEMM); 4 values per thread, n % 4 == 0.
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int32_t S, int64_t n,
                                                      const float* __restrict__ sa, const float* __restrict__ sb,
                                                      bf16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *(const f32x4*)(part + i);
  for (int s = 1; s < S; ++s) {
    const f32x4 v = *(const f32x4*)(part + (int64_t)s * n + i);
    acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
  }
  if (sa) {   // FP8 operands: dequantise the sum as the GEMM epilogue does, by 1 / (s_a s_b)
    const float dq = 1.0f / (sa[0] * sb[0]);
    acc[0] *= dq; acc[1] *= dq; acc[2] *= dq; acc[3] *= dq;
  }
  *(u32x2*)(out + i) = u32x2{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3])};
}

// Byte transpose with zero rows past R: out[c, r] = in[r, c] for r < R, 0
// for R <= r < Rp; 64 x 64 tiles through LDS, 16-byte loads and stores
// (one FP8 code per byte).
__global__ __launch_bounds__(256) void k_transpose8_pad(const uint8_t* __restrict__ in, int64_t R, int32_t C,
                                                        uint8_t* __restrict__ out, int64_t Rp) {
  __shared__ uint8_t tile[64][68];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int t = threadIdx.x;
  {
    // load: thread t reads 16 consecutive columns of row t / 4
    const int r = t >> 2, c = (t & 3) * 16;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (r0 + r < R) w = *(const u32x4*)(in + (r0 + r) * C + c0 + c);
#pragma unroll
    for (int e = 0; e < 16; ++e) tile[r][c + e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
  }
  __syncthreads();
  {
    // store: thread t writes 16 consecutive rows (of in) of output row t / 4
    const int c = t >> 2, r = (t & 3) * 16;
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)tile[r + 4 * q][c] | ((uint32_t)tile[r + 4 * q + 1][c] << 8) |
             ((uint32_t)tile[r + 4 * q + 2][c] << 16) | ((uint32_t)tile[r + 4 * q + 3][c] << 24);
    *(u32x4*)(out + (int64_t)(c0 + c) * Rp + r0 + r) = w;
  }
}

// ------------------------------------------------------------ GELU, RoPE backward

// dz = dy (Phi(z) + z phi(z)), 8 values per thread (16-byte loads); n % 8 == 0.
__global__ __launch_bounds__(256) void k_gelu_bwd(const bf16_t* __restrict__ z, const bf16_t* __restrict__ dy,
                                                  bf16_t* __restrict__ dz, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const u32x4 a = *(const u32x4*)(z + 8 * i);
  const u32x4 d = *(const u32x4*)(dy + 8 * i);
  constexpr float kRsqrt2 = 0.70710678118654752f, kRsqrt2Pi = 0.39894228040143268f;
  auto dg = [&](float v) { return 0.5f * (1.0f + erff(v * kRsqrt2)) + v * kRsqrt2Pi * expf(-0.5f * v * v); };
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf2(bflo(d[e]) * dg(bflo(a[e])), bfhi(d[e]) * dg(bfhi(a[e])));
  *(u32x4*)(dz + 8 * i) = o;
}

// dy[t, 192 n + 64 c + j] from the planar gradients dqkv[c][n][t][j] of the
// rotated q, k and of v: for c < 2 each pair (j, j + 32) turns back by the
// row's angle (a = a' cos + b' sin, b = b' cos - a' sin), v is copied.  One
// thread per (t, n, c, 8 pairs); positions clamped to the table as in the
// forward epilogue.
__global__ __launch_bounds__(256) void k_qkv_rope_bwd(const bf16_t* __restrict__ dqkv, const int32_t* __restrict__ pos,
                                                      const float2* __restrict__ rope, int32_t max_positions,
                                                      int64_t T, int32_t heads, bf16_t* __restrict__ dy) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T * heads * 3 * 4) return;
  const int i0 = 8 * (int)(g & 3);
  const int64_t rest = g >> 2;
  const int c = (int)(rest % 3);
  const int n = (int)((rest / 3) % heads);
  const int64_t t = rest / (3 * heads);
  const bf16_t* src = dqkv + (((int64_t)c * heads + n) * T + t) * kHeadDim;
  bf16_t* dst = dy + t * (3 * (int64_t)heads * kHeadDim) + 192 * n + 64 * c;
  const u32x4 lo = *(const u32x4*)(src + i0);
  const u32x4 hi = *(const u32x4*)(src + 32 + i0);
  if (c == 2) {
    *(u32x4*)(dst + i0) = lo;
    *(u32x4*)(dst + 32 + i0) = hi;
    return;
  }
  int p = pos[t];
  p = p < 0 ? 0 : (p < max_positions ? p : max_positions - 1);
  const float2* cs = rope + (int64_t)p * 32 + i0;
  u32x4 oa, ob;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float2 c0 = cs[2 * e], c1 = cs[2 * e + 1];
    const float a0 = bflo(lo[e]), a1 = bfhi(lo[e]), b0 = bflo(hi[e]), b1 = bfhi(hi[e]);
    oa[e] = pack_bf2(a0 * c0.x + b0 * c0.y, a1 * c1.x + b1 * c1.y);
    ob[e] = pack_bf2(b0 * c0.x - a0 * c0.y, b1 * c1.x - a1 * c1.y);
  }
  *(u32x4*)(dst + i0) = oa;
  *(u32x4*)(dst + 32 + i0) = ob;
}

// ------------------------------------------------------------ embedding backward
//
// Under X0 = E[ids] the table gradient of token v is the sum of dX0 over the
// residues holding v.  k_embed_bwd_partial: per 1024-row chunk and 64
// columns, wave w walks rows w, w + 4, ... of the chunk in order and adds
// each into its own LDS accumulator row of that row's token (one column per
// lane, so no two lanes touch one word and the order is fixed), then the four
// waves' accumulators are added in order into part [chunk, vocab, H];
// k_embed_bwd_final adds the chunks in order.  Token ids are clamped to
// [0, vocab) as the gather clamps them.
__global__ __launch_bounds__(256) void k_embed_bwd_partial(const int32_t* __restrict__ ids,
                                                           const bf16_t* __restrict__ dx, int64_t M, int32_t H,
                                                           int32_t vocab, float* __restrict__ part) {
  extern __shared__ float acc[];   // [4][vocab][64]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * kSumRows;
  const int n0 = blockIdx.y * 64;
  float* mine = acc + (size_t)wv * vocab * 64 + lane;
  for (int v = 0; v < vocab; ++v) mine[v * 64] = 0.f;
  const int64_t mend = m0 + kSumRows < M ? m0 + kSumRows : M;
  for (int64_t m = m0 + wv; m < mend; m += 4) {
    int id = ids[m];
    id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
    mine[id * 64] += bf2f(dx[m * H + n0 + lane]);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < vocab * 64; i += 256) {
    const size_t a = (size_t)vocab * 64;
    const float s = ((acc[i] + acc[a + i]) + acc[2 * a + i]) + acc[3 * a + i];
    part[((int64_t)blockIdx.x * vocab + i / 64) * H + n0 + (i & 63)] = s;
  }
}

__global__ __launch_bounds__(256) void k_embed_bwd_final(const float* __restrict__ part, int64_t chunks, int64_t n,
                                                         float* __restrict__ dtable) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int64_t c = 0; c < chunks; ++c) s += part[c * n + i];
  dtable[i] = s;
}

}  // namespace

int64_t colsum_chunks(int64_t M) { return (M + kSumRows - 1) / kSumRows; }

int32_t wgrad_splits(int64_t M, int32_t N, int32_t K) {
  // K slices for dW [N, K] = dy^T x (contraction over M): the count that
  // minimises rounds of 256 x 256 tiles over 256 compute units per unit of
  // contraction, ceil(tiles S / 256) / S, with slices of at least 1024 rows.
  const int64_t tiles = (int64_t)((N + 255) / 256) * ((K + 255) / 256);
  const int64_t smax = M / 1024 < 1 ? 1 : (M / 1024 > 16 ? 16 : M / 1024);
  int32_t best = 1;
  double best_t = 1e30;
  for (int32_t S = 1; S <= smax; ++S) {
    const double t = (double)((tiles * S + 255) / 256) / S;
    if (t < best_t - 1e-12) { best_t = t; best = S; }
  }
  return best;
}

hipError_t launch_split_reduce(const float* part, int32_t S, int64_t n, bf16_t* out, hipStream_t st,
                               const float* sa, const float* sb) {
  if (n <= 0) return hipSuccess;
  if (n % 4 || S < 1 || (sa == nullptr) != (sb == nullptr)) return hipErrorInvalidValue;
  const int64_t nt = n / 4;
  hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, st, part, S, n, sa, sb, out);
  return hipGetLastError();
}

hipError_t launch_transpose8_pad(const uint8_t* in, int64_t R, int32_t C, uint8_t* out, int64_t Rp, hipStream_t st) {
  if (C <= 0 || Rp <= 0) return hipSuccess;
  if (C % 64 || Rp % 64 || Rp < R) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_transpose8_pad, dim3((unsigned)(Rp / 64), (unsigned)(C / 64)), dim3(256), 0, st, in, R, C, out,
                     Rp);
  return hipGetLastError();
}

hipError_t launch_gelu_bwd(const bf16_t* z, const bf16_t* dy, bf16_t* dz, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_gelu_bwd, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, z, dy, dz, n8);
  return hipGetLastError();
}

hipError_t launch_qkv_rope_bwd(const bf16_t* dqkv, const int32_t* pos, const float2* rope, int32_t max_positions,
                               int64_t T, int32_t heads, bf16_t* dy, hipStream_t st) {
  if (T <= 0 || heads <= 0) return hipSuccess;
  const int64_t nt = T * heads * 3 * 4;
  hipLaunchKernelGGL(k_qkv_rope_bwd, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, st, dqkv, pos, rope,
                     max_positions, T, heads, dy);
  return hipGetLastError();
}

hipError_t launch_layernorm_bwd(const bf16_t* x, const bf16_t* gamma, const bf16_t* dy, const bf16_t* dres, bf16_t* dx,
                                float* dgamma, float* dbeta, int64_t M, int32_t H, float eps, float* stats, float* part,
                                hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (H % 64 || H / 8 > 64 * kLnMaxCh) return hipErrorInvalidValue;
  const int ch = (H / 8 + 63) / 64;
  const dim3 rg((unsigned)((M + 3) / 4));
  if (ch <= 1) hipLaunchKernelGGL(k_ln_bwd_rows<1>, rg, dim3(256), 0, st, x, gamma, dy, dres, dx, stats, M, H, eps);
  else if (ch <= 2) hipLaunchKernelGGL(k_ln_bwd_rows<2>, rg, dim3(256), 0, st, x, gamma, dy, dres, dx, stats, M, H, eps);
  else if (ch <= 3) hipLaunchKernelGGL(k_ln_bwd_rows<3>, rg, dim3(256), 0, st, x, gamma, dy, dres, dx, stats, M, H, eps);
  else if (ch <= 5) hipLaunchKernelGGL(k_ln_bwd_rows<5>, rg, dim3(256), 0, st, x, gamma, dy, dres, dx, stats, M, H, eps);
  else hipLaunchKernelGGL(k_ln_bwd_rows<8>, rg, dim3(256), 0, st, x, gamma, dy, dres, dx, stats, M, H, eps);
  const int64_t chunks = colsum_chunks(M);
  hipLaunchKernelGGL(k_ln_bwd_cols, dim3((unsigned)chunks, (unsigned)(H / 64)), dim3(256), 0, st, x, dy, stats, M, H,
                     part);
  hipLaunchKernelGGL(k_ln_cols_final, dim3((unsigned)((2 * H + 255) / 256)), dim3(256), 0, st, part, chunks, H,
                     dgamma, dbeta);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(const bf16_t* in, int64_t R, int32_t C, bf16_t* out, int64_t Rp, hipStream_t st) {
  if (C <= 0 || Rp <= 0) return hipSuccess;
  if (C % 64 || Rp % 64 || Rp < R) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_transpose_pad, dim3((unsigned)(Rp / 64), (unsigned)(C / 64)), dim3(256), 0, st, in, R, C, out,
                     Rp);
  return hipGetLastError();
}

hipError_t launch_colsum(const bf16_t* dy, int64_t M, int32_t N, float* part, float* db, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (N % 64) return hipErrorInvalidValue;
  const int64_t chunks = colsum_chunks(M);
  if (chunks > 0)
    hipLaunchKernelGGL(k_colsum_partial, dim3((unsigned)chunks, (unsigned)(N / 64)), dim3(256), 0, st, dy, M, N,
                       part);
  hipLaunchKernelGGL(k_colsum_final, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, part, chunks, N, N, db);
  return hipGetLastError();
}

hipError_t launch_embed_bwd(const int32_t* ids, const bf16_t* dx, int64_t M, int32_t H, int32_t vocab, float* part,
                            float* dtable, hipStream_t st) {
  if (H <= 0 || vocab <= 0) return hipSuccess;
  if (H % 64 || vocab > kEmbedBwdMaxVocab) return hipErrorInvalidValue;
  const int64_t chunks = colsum_chunks(M);
  if (chunks > 0)
    hipLaunchKernelGGL(k_embed_bwd_partial, dim3((unsigned)chunks, (unsigned)(H / 64)), dim3(256),
                       (unsigned)(4 * vocab * 64 * sizeof(float)), st, ids, dx, M, H, vocab, part);
  const int64_t n = (int64_t)vocab * H;
  hipLaunchKernelGGL(k_embed_bwd_final, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, chunks, n, dtable);
  return hipGetLastError();
}

}  // namespace esm
