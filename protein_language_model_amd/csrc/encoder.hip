// Host side of the C ABI declared in include/esm_encoder.h: argument checks,
// workspace planning, the launch sequence of one encoder layer and of the
// stack, and per-kernel-class timing with HIP events.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/esm_encoder.h"
#include "common.h"

static_assert(esm::kAttnTileRows == ESM_ATTN_TILE_ROWS, "attention tile rows");

using namespace esm;

struct esm_encoder {
  esm_config cfg;
  int device = 0;
  float2* rope = nullptr;  // [max_positions, 32]
  // A second stream (default priority) for work that runs beside the
  // caller's stream inside one call (the dW path of esm_linear_bwd), forked
  // and joined with the two events; created on first use.
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool profiling = false;
  std::vector<hipEvent_t> pool;
  size_t pool_used = 0;
  std::vector<std::pair<int, size_t>> recs;  // (class, index of start event)
  double ms[ESM_K_COUNT] = {0};
  int64_t launches[ESM_K_COUNT] = {0};
  // Quantised encoders (precision FP8 or MXFP4): per-layer precision, the
  // encoder's own by default; FP8, MXFP4 and bf16 layers may be mixed.
  std::vector<int32_t> layer_prec;
  // FP8 delayed scaling: created with an FP8 encoder, or with the first FP8
  // layer of an MXFP4 encoder
  void* fp8_mem = nullptr;         // state arrays of f8
  Fp8State f8{};
  uint8_t* w8 = nullptr;           // per layer: E4M3 w_qkv | w_out | w_fc1 | w_fc2
  size_t w8_layer = 0;             // bytes per layer
  std::vector<char> prepared8;     // E4M3 weights cast since the state was created
  // MXFP4: per layer the codes and block scales of w_qkv | w_out | w_fc1 |
  // w_fc2; created with an MXFP4 encoder, or with the first MXFP4 weights
  // prepared in an FP8 encoder
  uint8_t* w4 = nullptr;
  size_t w4_layer = 0;
  std::vector<char> prepared4;     // MXFP4 weights quantised since created
  // LM head: the tied decoder weight and its bias padded to vocab_pad rows
  // (a multiple of 64 GEMM columns), refilled from the caller's on each call
  bf16_t* head_w = nullptr;        // [vocab_pad, H] then [vocab_pad]
  int32_t vocab_pad = 0;
  // this device's copy of the file-scope scratch array (esm_layer_fwd_noalloc)
  void* scratch = nullptr;
  // bf16 precision: LayerNorms folded into the QKV and fc1 linears
  // (esm_prepare_layer): per layer W'_qkv | W'_fc1 | (c, d) of qkv | of fc1
  unsigned char* fold = nullptr;
  size_t fold_layer = 0;
  std::vector<char> folded;
};

namespace {

thread_local std::string g_last_error;

// Device scratch of esm_layer_fwd_noalloc: a file-scope array, one copy on
// every device the library runs on, held until the process ends.  Host code
// never passes `scratch` itself to a kernel (in host code the name is a
// host-side stand-in, not a device address): esm_encoder_create resolves the
// array's address on each device once, with that device current, and every
// use goes through that pointer.
static __device__ __align__(256) unsigned char scratch[ESM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of `scratch` on the current device `dev` (resolved on first use).
hipError_t scratch_on_device(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

esm_status fail(esm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

esm_status ok() { return ESM_OK; }

esm_status hip_fail(hipError_t e, const char* what) {
  return fail(ESM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                      \
  do {                                           \
    hipError_t _e = (expr);                      \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int32_t kHeadMaxVocab = 4096;  // LM head decoder rows supported

// Shapes each quantised format needs (one K step of its GEMM; the MXFP4
// activation codes are staged in the QKV region).
esm_status check_fp8_shape(const esm_config* c) {
  if (c->hidden_size % 128 != 0 || c->intermediate_size % 128 != 0)
    return fail(ESM_ERR_UNSUPPORTED,
                "FP8 needs hidden_size (%d) and intermediate_size (%d) to be multiples of 128 (E4M3 K step)",
                c->hidden_size, c->intermediate_size);
  return ok();
}
esm_status check_mx_shape(const esm_config* c) {
  if (c->hidden_size % 256 != 0 || c->intermediate_size % 256 != 0 || c->intermediate_size > 8 * c->hidden_size)
    return fail(ESM_ERR_UNSUPPORTED,
                "MXFP4 needs hidden_size (%d) and intermediate_size (%d) to be multiples of 256 (one K step) and "
                "intermediate_size <= 8 * hidden_size (its codes are staged in the QKV region)",
                c->hidden_size, c->intermediate_size);
  return ok();
}

esm_status check_config(const esm_config* c) {
  if (!c) return fail(ESM_ERR_NULL, "config is NULL");
  if (c->hidden_size <= 0 || c->hidden_size % 64 != 0)
    return fail(ESM_ERR_SHAPE, "hidden_size %d must be a positive multiple of 64", c->hidden_size);
  if (c->num_attention_heads <= 0 || c->hidden_size / c->num_attention_heads * c->num_attention_heads != c->hidden_size)
    return fail(ESM_ERR_SHAPE, "num_attention_heads %d does not divide hidden_size %d", c->num_attention_heads,
                c->hidden_size);
  if (c->hidden_size / c->num_attention_heads != kHeadDim)
    return fail(ESM_ERR_UNSUPPORTED, "head_dim %d: only 64 is built", c->hidden_size / c->num_attention_heads);
  if (c->hidden_size > 4096) return fail(ESM_ERR_UNSUPPORTED, "hidden_size %d above 4096", c->hidden_size);
  if (c->intermediate_size <= 0 || c->intermediate_size % 64 != 0)
    return fail(ESM_ERR_SHAPE, "intermediate_size %d must be a positive multiple of 64", c->intermediate_size);
  if (c->num_hidden_layers < 0) return fail(ESM_ERR_SHAPE, "num_hidden_layers %d < 0", c->num_hidden_layers);
  if (c->vocab_size <= 0) return fail(ESM_ERR_SHAPE, "vocab_size %d <= 0", c->vocab_size);
  if (c->max_position_embeddings <= 0 || c->max_position_embeddings > 65536)
    return fail(ESM_ERR_SHAPE, "max_position_embeddings %d outside [1, 65536]", c->max_position_embeddings);
  if (!(c->layer_norm_eps > 0.f) || !isfinite(c->layer_norm_eps))
    return fail(ESM_ERR_SHAPE, "layer_norm_eps must be positive and finite");
  if (!(c->rope_base > 1.f) || !isfinite(c->rope_base)) return fail(ESM_ERR_SHAPE, "rope_base must be > 1");
  if (c->precision != ESM_PRECISION_BF16 && c->precision != ESM_PRECISION_FP8_DELAYED &&
      c->precision != ESM_PRECISION_MXFP4)
    return fail(ESM_ERR_UNSUPPORTED, "unknown precision %d", c->precision);
  if (c->precision == ESM_PRECISION_MXFP4) {
    esm_status s = check_mx_shape(c);
    if (s) return s;
  }
  if (c->precision == ESM_PRECISION_FP8_DELAYED) {
    esm_status s = check_fp8_shape(c);
    if (s) return s;
  }
  if (c->amax_history_len < 1 || c->amax_history_len > 1024)
    return fail(ESM_ERR_SHAPE, "amax_history_len %d outside [1, 1024]", c->amax_history_len);
  return ok();
}

// ---------------------------------------------------------------- workspace plan

constexpr int kRegions = ESM_WS_STATS + 1;

struct Plan {
  size_t off[kRegions];
  size_t size[kRegions];
  size_t total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t tile_cap(int64_t rows, int32_t seqs) { return rows / kAttnTileRows + seqs + 1; }

Plan make_plan(const esm_config& c, int64_t T, int32_t B) {
  Plan p;
  const size_t H = (size_t)c.hidden_size, F = (size_t)c.intermediate_size;
  const size_t t = (size_t)(T > 0 ? T : 0), b = (size_t)(B > 0 ? B : 0);
  size_t sizes[kRegions];
  sizes[ESM_WS_LN1] = t * H * 2;
  sizes[ESM_WS_QKV] = 3 * t * H * 2;
  sizes[ESM_WS_CTX] = t * H * 2;
  sizes[ESM_WS_X1] = t * H * 2;
  sizes[ESM_WS_LN2] = t * H * 2;
  sizes[ESM_WS_ACT] = t * F * 2;
  sizes[ESM_WS_POS] = t * 4;
  sizes[ESM_WS_TILES] = (size_t)tile_cap((int64_t)t, (int32_t)b) * 8;
  sizes[ESM_WS_NTILES] = 4;
  sizes[ESM_WS_SEGS] = b * 8;
  sizes[ESM_WS_STATS] = (H + 255) / 256 * t * 8;
  size_t o = 0;
  for (int i = 0; i < kRegions; ++i) {
    p.off[i] = o;
    p.size[i] = sizes[i];
    o += align256(sizes[i]);
  }
  p.total = o;
  return p;
}

template <class T>
T* region(void* ws, const Plan& p, int r) {
  return (T*)((char*)ws + p.off[r]);
}

// ---------------------------------------------------------------- timing

esm_status grow_pool(esm_encoder* e) {
  for (int i = 0; i < 256; ++i) {
    hipEvent_t ev;
    HIP_TRY(hipEventCreate(&ev), "hipEventCreate");
    e->pool.push_back(ev);
  }
  return ok();
}

template <class F>
esm_status timed(esm_encoder* e, int cls, hipStream_t st, const char* what, F&& launch) {
  if (!e->profiling) {
    hipError_t err = launch();
    if (err != hipSuccess) return hip_fail(err, what);
    return ok();
  }
  if (e->pool_used + 2 > e->pool.size()) {
    esm_status s = grow_pool(e);
    if (s != ESM_OK) return s;
  }
  const size_t i0 = e->pool_used;
  e->pool_used += 2;
  HIP_TRY(hipEventRecord(e->pool[i0], st), "hipEventRecord");
  hipError_t err = launch();
  if (err != hipSuccess) return hip_fail(err, what);
  HIP_TRY(hipEventRecord(e->pool[i0 + 1], st), "hipEventRecord");
  e->recs.push_back({cls, i0});
  return ok();
}

// ---------------------------------------------------------------- argument checks

esm_status check_weights(const esm_layer_weights* w, int idx) {
  if (!w) return fail(ESM_ERR_NULL, "layer %d: weights struct is NULL", idx);
  const void* req[] = {w->ln1_gamma, w->ln1_beta, w->w_qkv, w->w_out, w->ln2_gamma, w->ln2_beta, w->w_fc1, w->w_fc2};
  const char* names[] = {"ln1_gamma", "ln1_beta", "w_qkv", "w_out", "ln2_gamma", "ln2_beta", "w_fc1", "w_fc2"};
  for (int i = 0; i < 8; ++i) {
    if (!req[i]) return fail(ESM_ERR_NULL, "layer %d: %s is NULL", idx, names[i]);
    if (!aligned16(req[i])) return fail(ESM_ERR_UNSUPPORTED, "layer %d: %s not 16-byte aligned", idx, names[i]);
  }
  const void* opt[] = {w->b_qkv, w->b_out, w->b_fc1, w->b_fc2};
  for (int i = 0; i < 4; ++i)
    if (opt[i] && ((uintptr_t)opt[i] & 7u)) return fail(ESM_ERR_UNSUPPORTED, "layer %d: bias not 8-byte aligned", idx);
  return ok();
}

esm_status check_rows(const esm_encoder* e, int64_t rows, int32_t B) {
  if (rows < 0 || B < 0) return fail(ESM_ERR_SHAPE, "negative T (%lld) or B (%d)", (long long)rows, B);
  if (rows > (int64_t)INT32_MAX - 1024) return fail(ESM_ERR_SHAPE, "T = %lld rows too large", (long long)rows);
  (void)e;
  return ok();
}

esm_status check_ws(const esm_encoder* e, void* ws, size_t ws_bytes, int64_t rows, int32_t B, Plan* p) {
  *p = make_plan(e->cfg, rows, B);
  if (!ws) return fail(ESM_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws & 255u) return fail(ESM_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (ws_bytes < p->total)
    return fail(ESM_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, p->total);
  return ok();
}

// ---------------------------------------------------------------- FP8 state

bool is_fp8(const esm_encoder* e) { return e->cfg.precision == ESM_PRECISION_FP8_DELAYED; }
bool is_mx(const esm_encoder* e) { return e->cfg.precision == ESM_PRECISION_MXFP4; }
bool is_quantised(const esm_encoder* e) { return is_fp8(e) || is_mx(e); }
// Layer l of a quantised encoder runs the precision esm_set_layer_precision
// gave it (the encoder's own by default).
int32_t layer_precision(const esm_encoder* e, int32_t l) {
  return l >= 0 && (size_t)l < e->layer_prec.size() ? e->layer_prec[(size_t)l] : ESM_PRECISION_BF16;
}
bool layer_fp8(const esm_encoder* e, int32_t l) { return layer_precision(e, l) == ESM_PRECISION_FP8_DELAYED; }
bool layer_mx(const esm_encoder* e, int32_t l) { return layer_precision(e, l) == ESM_PRECISION_MXFP4; }


// MXFP4 operand: codes [rows, K / 2] then, 256-byte aligned, the block scales
// [K / 256][rows rounded up to even][8] (the esm_mxfp4_quantize layout).
struct MxOff {
  size_t codes, scales, total;
};
MxOff mx_operand(size_t rows, size_t K) {
  MxOff o;
  o.codes = 0;
  o.scales = align256(rows * K / 2);
  o.total = o.scales + (K / 256) * (rows + (rows & 1)) * 8;
  return o;
}
// The four MXFP4 weights of one layer: offsets of w_qkv, w_out, w_fc1, w_fc2.
struct W4Off {
  size_t at[4], total;
};
W4Off w4_offsets(const esm_config& c) {
  const size_t H = (size_t)c.hidden_size, F = (size_t)c.intermediate_size;
  const size_t n[4] = {3 * H, H, F, H}, k[4] = {H, H, H, F};
  W4Off o;
  size_t at = 0;
  for (int i = 0; i < 4; ++i) {
    o.at[i] = at;
    at += align256(mx_operand(n[i], k[i]).total);
  }
  o.total = at;
  return o;
}

// Byte offsets of the four E4M3 weights inside one layer's block.
struct W8Off {
  size_t qkv, out, fc1, fc2, total;
};
W8Off w8_offsets(const esm_config& c) {
  const size_t H = (size_t)c.hidden_size, F = (size_t)c.intermediate_size;
  W8Off o;
  o.qkv = 0;
  o.out = 3 * H * H;
  o.fc1 = o.out + H * H;
  o.fc2 = o.fc1 + F * H;
  o.total = o.fc2 + H * F;
  return o;
}

// Device layout of the delayed-scaling state: one allocation, 256-byte
// aligned arrays.
struct Fp8Layout {
  size_t act_scale, act_amax, history, steps, flags, w_scale, w_amax, layer_on, g_scale, g_amax, g_history, g_steps,
      total;
};
Fp8Layout fp8_layout(const esm_config& c) {
  const size_t L = (size_t)(c.num_hidden_layers > 0 ? c.num_hidden_layers : 1), HL = (size_t)c.amax_history_len;
  Fp8Layout f;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  f.act_scale = take(L * 4 * sizeof(float));
  f.act_amax = take(L * 4 * sizeof(uint32_t));
  f.history = take(L * 4 * HL * sizeof(float));
  f.steps = take(L * sizeof(int64_t));
  f.flags = take(sizeof(uint32_t));
  f.w_scale = take(L * 4 * sizeof(float));
  f.w_amax = take(L * 4 * sizeof(uint32_t));
  f.layer_on = take(L * sizeof(int32_t));
  f.g_scale = take(L * 4 * sizeof(float));
  f.g_amax = take(L * 4 * sizeof(uint32_t));
  f.g_history = take(L * 4 * HL * sizeof(float));
  f.g_steps = take(L * sizeof(int64_t));
  f.total = o;
  return f;
}

// Scales 1, empty histories, no steps, no flags, amax cleared (synchronous).
esm_status fp8_reset_state(esm_encoder* e) {
  const esm_config& c = e->cfg;
  const size_t L = (size_t)(c.num_hidden_layers > 0 ? c.num_hidden_layers : 1), HL = (size_t)c.amax_history_len;
  std::vector<float> ones(L * 4, 1.0f);
  HIP_TRY(hipMemcpy(e->f8.act_scale, ones.data(), ones.size() * sizeof(float), hipMemcpyHostToDevice), "fp8 reset");
  HIP_TRY(hipMemset(e->f8.act_amax, 0, L * 4 * sizeof(uint32_t)), "fp8 reset");
  HIP_TRY(hipMemset(e->f8.history, 0, L * 4 * HL * sizeof(float)), "fp8 reset");
  HIP_TRY(hipMemset(e->f8.steps, 0, L * sizeof(int64_t)), "fp8 reset");
  HIP_TRY(hipMemset(e->f8.flags, 0, sizeof(uint32_t)), "fp8 reset");
  HIP_TRY(hipMemcpy(e->f8.g_scale, ones.data(), ones.size() * sizeof(float), hipMemcpyHostToDevice), "fp8 reset");
  HIP_TRY(hipMemset(e->f8.g_amax, 0, L * 4 * sizeof(uint32_t)), "fp8 reset");
  HIP_TRY(hipMemset(e->f8.g_history, 0, L * 4 * HL * sizeof(float)), "fp8 reset");
  HIP_TRY(hipMemset(e->f8.g_steps, 0, L * sizeof(int64_t)), "fp8 reset");
  return ok();
}

esm_status fp8_create(esm_encoder* e) {
  const esm_config& c = e->cfg;
  const Fp8Layout f = fp8_layout(c);
  HIP_TRY(hipMalloc(&e->fp8_mem, f.total), "fp8 state");
  char* b = (char*)e->fp8_mem;
  e->f8.act_scale = (float*)(b + f.act_scale);
  e->f8.act_amax = (uint32_t*)(b + f.act_amax);
  e->f8.history = (float*)(b + f.history);
  e->f8.steps = (int64_t*)(b + f.steps);
  e->f8.flags = (uint32_t*)(b + f.flags);
  e->f8.w_scale = (float*)(b + f.w_scale);
  e->f8.w_amax = (uint32_t*)(b + f.w_amax);
  e->f8.layer_on = (int32_t*)(b + f.layer_on);
  e->f8.g_scale = (float*)(b + f.g_scale);
  e->f8.g_amax = (uint32_t*)(b + f.g_amax);
  e->f8.g_history = (float*)(b + f.g_history);
  e->f8.g_steps = (int64_t*)(b + f.g_steps);
  e->f8.history_len = c.amax_history_len;
  HIP_TRY(hipMemset(e->f8.w_scale, 0, f.total - f.w_scale), "fp8 state");
  e->w8_layer = align256(w8_offsets(c).total);
  const size_t L = (size_t)(c.num_hidden_layers > 0 ? c.num_hidden_layers : 1);
  HIP_TRY(hipMalloc((void**)&e->w8, L * e->w8_layer), "fp8 weights");
  e->prepared8.assign(L, 0);
  std::vector<int32_t> on(L);
  for (size_t l = 0; l < L; ++l) on[l] = layer_fp8(e, (int32_t)l);
  HIP_TRY(hipMemcpy(e->f8.layer_on, on.data(), L * sizeof(int32_t), hipMemcpyHostToDevice), "fp8 layer flags");
  return fp8_reset_state(e);
}

// The delayed-scaling state and E4M3 weight store, on first need.
esm_status ensure_fp8(esm_encoder* e) {
  if (e->fp8_mem) return ok();
  esm_status s = check_fp8_shape(&e->cfg);
  if (s) return s;
  s = fp8_create(e);
  if (s) {
    if (e->fp8_mem) (void)hipFree(e->fp8_mem);
    if (e->w8) (void)hipFree(e->w8);
    e->fp8_mem = nullptr;
    e->w8 = nullptr;
  }
  return s;
}

// The MXFP4 weight store, on first need.
esm_status ensure_mx(esm_encoder* e) {
  if (e->w4) return ok();
  esm_status s = check_mx_shape(&e->cfg);
  if (s) return s;
  const size_t L = (size_t)(e->cfg.num_hidden_layers > 0 ? e->cfg.num_hidden_layers : 1);
  e->w4_layer = align256(w4_offsets(e->cfg).total);
  HIP_TRY(hipMalloc((void**)&e->w4, L * e->w4_layer), "MXFP4 weights");
  e->prepared4.assign(L, 0);
  return ok();
}

// A quantised layer needs its weights in its own format.
esm_status check_quant_layer(const esm_encoder* e, int32_t l) {
  if (l < 0 || l >= e->cfg.num_hidden_layers)
    return fail(ESM_ERR_SHAPE, "layer_idx %d outside [0, num_hidden_layers = %d)", l, e->cfg.num_hidden_layers);
  if (layer_fp8(e, l) && (!e->fp8_mem || !e->prepared8[(size_t)l]))
    return fail(ESM_ERR_STATE, "FP8 weights of layer %d not prepared (esm_fp8_prepare_layer)", l);
  if (layer_mx(e, l) && (!e->w4 || !e->prepared4[(size_t)l]))
    return fail(ESM_ERR_STATE, "MXFP4 weights of layer %d not prepared (esm_mxfp4_prepare_layer)", l);
  return ok();
}

// Folded LayerNorm weights of one layer: W'_qkv [3H, H], W'_fc1 [F, H]
// (bf16), then (c, d) [3H] and [F] (float2).
struct FoldOff {
  size_t wqkv, wfc1, cdqkv, cdfc1, total;
};
FoldOff fold_offsets(const esm_config& c) {
  const size_t H = (size_t)c.hidden_size, F = (size_t)c.intermediate_size;
  FoldOff f;
  f.wqkv = 0;
  f.wfc1 = align256(3 * H * H * 2);
  f.cdqkv = f.wfc1 + align256(F * H * 2);
  f.cdfc1 = f.cdqkv + align256(3 * H * 8);
  f.total = f.cdfc1 + align256(F * 8);
  return f;
}

bool layer_folded(const esm_encoder* e, int32_t l) {
  return e->cfg.precision == ESM_PRECISION_BF16 && l >= 0 && (size_t)l < e->folded.size() && e->folded[(size_t)l];
}

// ---------------------------------------------------------------- launch sequence

esm_status run_segments(esm_encoder* e, int layout, const int32_t* lens, int32_t B, int64_t rows, int32_t S,
                        void* ws, const Plan& p, hipStream_t st) {
  SegOut so;
  so.pos = region<int32_t>(ws, p, ESM_WS_POS);
  so.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  so.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  so.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  so.tile_cap = tile_cap(rows, B);
  return timed(e, ESM_K_SEGMENT, st, "segment table", [&] {
    return launch_segment_table(layout, lens, B, rows, S, e->cfg.max_position_embeddings, so, st);
  });
}

// One pre-LN layer with MXFP4 GEMMs (the FP4 recipe): the residuals and the
// QKV and residual GEMM outputs as in the bf16 layer; each GEMM input is
// written in MXFP4 by its producer, from fp32 values, into a workspace region
// that is free at that point: LN1 -> ctx region, the attention context -> LN1
// region, LN2 -> ctx region, fc1's GELU(.) -> QKV region.  The GEMMs read
// layer li's prepared MXFP4 weights.  Quantisation is per 32-value
// block of a row, so rows stay independent (packed == each sequence alone,
// padding rows never mix in).
esm_status run_layer_mx(esm_encoder* e, const esm_layer_weights* w, int32_t li, const bf16_t* x_in, bf16_t* x_out,
                        int64_t rows, int32_t B, bool zero_pad_rows, void* ws, const Plan& p, hipStream_t st) {
  const esm_config& c = e->cfg;
  const int H = c.hidden_size, F = c.intermediate_size, heads = c.num_attention_heads;
  bf16_t* ln1 = region<bf16_t>(ws, p, ESM_WS_LN1);
  bf16_t* qkv = region<bf16_t>(ws, p, ESM_WS_QKV);
  bf16_t* ctx = region<bf16_t>(ws, p, ESM_WS_CTX);
  bf16_t* x1 = region<bf16_t>(ws, p, ESM_WS_X1);
  const int32_t* pos = region<int32_t>(ws, p, ESM_WS_POS);
  const uint8_t* w4 = e->w4 + (size_t)li * e->w4_layer;
  const W4Off wo = w4_offsets(c);
  const size_t nw[4] = {(size_t)3 * H, (size_t)H, (size_t)F, (size_t)H}, kw[4] = {(size_t)H, (size_t)H, (size_t)H,
                                                                                  (size_t)F};
  const E4m3Out none{nullptr, nullptr, nullptr, nullptr};
  esm_status s;
  GemmArgs g{};
  g.dtype = kFP4;
  g.M = rows;
  g.pos = pos;
  g.rope = e->rope;
  g.max_positions = c.max_position_embeddings;
  g.zero_pad_rows = zero_pad_rows ? 1 : 0;
  // point the GEMM at the MXFP4 operand in dst_region (quantising src [rows, K]
  // into it first unless src is null: a LayerNorm already wrote it) and at weight t
  auto operands = [&](const bf16_t* src, int K, void* dst_region, int t) -> esm_status {
    const MxOff xo = mx_operand((size_t)rows, (size_t)K);
    uint8_t* d = (uint8_t*)dst_region;
    if (src) {
      esm_status q = timed(e, ESM_K_OTHER, st, "mxfp4 quantize",
                           [&] { return launch_mx_quantize(src, rows, K, d + xo.codes, d + xo.scales, st); });
      if (q) return q;
    }
    const MxOff wq = mx_operand(nw[t], kw[t]);
    g.x = d + xo.codes;
    g.x_sc = d + xo.scales;
    g.w = w4 + wo.at[t] + wq.codes;
    g.w_sc = w4 + wo.at[t] + wq.scales;
    return ESM_OK;
  };
  // LayerNorm straight to MXFP4 in dst_region
  auto ln_mx = [&](const bf16_t* src, const void* gamma, const void* beta, void* dst_region, const char* what) {
    const MxOff xo = mx_operand((size_t)rows, (size_t)H);
    uint8_t* d = (uint8_t*)dst_region;
    return timed(e, ESM_K_LAYERNORM, st, what, [&] {
      return launch_layernorm_mx(src, (const bf16_t*)gamma, (const bf16_t*)beta, d + xo.codes, d + xo.scales, rows,
                                 H, c.layer_norm_eps, st);
    });
  };

  s = ln_mx(x_in, w->ln1_gamma, w->ln1_beta, ctx, "layernorm 1");
  if (s || (s = operands(nullptr, H, ctx, 0))) return s;
  g.bias = (const bf16_t*)w->b_qkv; g.res = nullptr; g.y = qkv;
  g.N = 3 * H; g.K = H;
  s = timed(e, ESM_K_GEMM_QKV, st, "qkv gemm", [&] { return launch_gemm(EPI_QKV_ROPE, g, st); });
  if (s) return s;

  AttnArgs aa{};
  aa.qkv = qkv; aa.ctx = ctx;
  aa.ctx8 = none;
  {
    // the attention writes its context straight to MXFP4 in the LN1 region
    const MxOff co = mx_operand((size_t)rows, (size_t)H);
    aa.ctx_mx = (uint8_t*)ln1 + co.codes;
    aa.ctx_mx_sc = (uint8_t*)ln1 + co.scales;
  }
  aa.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  aa.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  aa.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  aa.tile_cap = tile_cap(rows, B);
  aa.T = rows; aa.heads = heads;
  s = timed(e, ESM_K_ATTENTION, st, "attention", [&] { return launch_attention(aa, st); });
  if (s || (s = operands(nullptr, H, ln1, 1))) return s;
  g.bias = (const bf16_t*)w->b_out; g.res = x_in; g.y = x1;
  g.N = H; g.K = H;
  s = timed(e, ESM_K_GEMM_OUT, st, "out-proj gemm", [&] { return launch_gemm(EPI_BIAS_RESIDUAL, g, st); });
  if (s) return s;

  s = ln_mx(x1, w->ln2_gamma, w->ln2_beta, ctx, "layernorm 2");
  if (s || (s = operands(nullptr, H, ctx, 2))) return s;
  {
    // fc1's epilogue writes GELU(.) straight to MXFP4 in the QKV region
    const MxOff ao = mx_operand((size_t)rows, (size_t)F);
    g.bias = (const bf16_t*)w->b_fc1; g.res = nullptr; g.y = nullptr;
    g.y8 = (uint8_t*)qkv + ao.codes;
    g.y_sc = (uint8_t*)qkv + ao.scales;
    g.N = F; g.K = H;
    s = timed(e, ESM_K_GEMM_FC1, st, "fc1 gemm", [&] { return launch_gemm(EPI_BIAS_GELU_MX, g, st); });
    g.y8 = nullptr; g.y_sc = nullptr;
  }
  if (s || (s = operands(nullptr, F, qkv, 3))) return s;
  g.bias = (const bf16_t*)w->b_fc2; g.res = x1; g.y = x_out;
  g.N = H; g.K = F;
  return timed(e, ESM_K_GEMM_FC2, st, "fc2 gemm", [&] { return launch_gemm(EPI_BIAS_RESIDUAL, g, st); });
}

// One bf16 pre-LN layer with both LayerNorms folded into the linears that
// consume them ([TE-RU] LayerNormLinear / LayerNormMLP; [BIO-ACC] 2.1: the
// LayerNorm, the projection and the activation in one kernel): the QKV and
// fc1 GEMMs read the raw residual stream and layer li's prepared W' = gamma (.) W
// and apply each row's (mean, 1/sqrt(var + eps)) and the columns' (c, d) in
// their epilogue; the row statistics come as 256-column chunk partials,
// written by the epilogue of the GEMM that produced the residual stream (the
// out-projection for LN2, the previous layer's fc2 for LN1) or, for the first
// layer of a call, by a statistics pass.  *stats_valid says whether the
// statistics region holds the partials of x_in; on return it holds those of
// x_out.
esm_status run_layer_folded(esm_encoder* e, const esm_layer_weights* w, int32_t li, const bf16_t* x_in,
                            bf16_t* x_out, int64_t rows, int32_t B, bool zero_pad_rows, void* ws, const Plan& p,
                            bool* stats_valid, hipStream_t st) {
  const esm_config& c = e->cfg;
  const int H = c.hidden_size, F = c.intermediate_size, heads = c.num_attention_heads;
  bf16_t* qkv = region<bf16_t>(ws, p, ESM_WS_QKV);
  bf16_t* ctx = region<bf16_t>(ws, p, ESM_WS_CTX);
  bf16_t* x1 = region<bf16_t>(ws, p, ESM_WS_X1);
  bf16_t* act = region<bf16_t>(ws, p, ESM_WS_ACT);
  float2* stats = region<float2>(ws, p, ESM_WS_STATS);
  const int32_t* pos = region<int32_t>(ws, p, ESM_WS_POS);
  const FoldOff fo = fold_offsets(c);
  const unsigned char* fl = e->fold + (size_t)li * e->fold_layer;
  esm_status s;
  if (!*stats_valid) {
    s = timed(e, ESM_K_LAYERNORM, st, "layernorm statistics", [&] {
      return launch_row_stats(nullptr, nullptr, 0, (bf16_t*)x_in, rows, H, stats, st);
    });
    if (s) return s;
    *stats_valid = true;
  }
  GemmArgs g{};
  g.dtype = kBF16;
  g.M = rows;
  g.pos = pos;
  g.rope = e->rope;
  g.max_positions = c.max_position_embeddings;
  g.zero_pad_rows = zero_pad_rows ? 1 : 0;
  g.ln_eps = c.layer_norm_eps;

  g.x = x_in; g.w = fl + fo.wqkv; g.ln_stats = stats; g.ln_cd = (const float2*)(fl + fo.cdqkv);
  g.y = qkv; g.N = 3 * H; g.K = H;
  s = timed(e, ESM_K_GEMM_QKV, st, "qkv gemm", [&] { return launch_gemm(EPI_QKV_ROPE_LN, g, st); });
  if (s) return s;

  AttnArgs aa{};
  aa.qkv = qkv; aa.ctx = ctx;
  aa.ctx8 = E4m3Out{nullptr, nullptr, nullptr, nullptr};
  aa.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  aa.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  aa.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  aa.tile_cap = tile_cap(rows, B);
  aa.T = rows; aa.heads = heads;
  s = timed(e, ESM_K_ATTENTION, st, "attention", [&] { return launch_attention(aa, st); });
  if (s) return s;

  g.x = ctx; g.w = w->w_out; g.ln_stats = nullptr; g.ln_cd = nullptr;
  g.bias = (const bf16_t*)w->b_out; g.res = x_in; g.y = x1; g.stats_out = stats;
  g.N = H; g.K = H;
  s = timed(e, ESM_K_GEMM_OUT, st, "out-proj gemm", [&] { return launch_gemm(EPI_RES_STATS, g, st); });
  if (s) return s;

  g.x = x1; g.w = fl + fo.wfc1; g.ln_stats = stats; g.ln_cd = (const float2*)(fl + fo.cdfc1);
  g.bias = nullptr; g.res = nullptr; g.y = act; g.stats_out = nullptr;
  g.N = F; g.K = H;
  s = timed(e, ESM_K_GEMM_FC1, st, "fc1 gemm", [&] { return launch_gemm(EPI_BIAS_GELU_LN, g, st); });
  if (s) return s;

  g.x = act; g.w = w->w_fc2; g.ln_stats = nullptr; g.ln_cd = nullptr;
  g.bias = (const bf16_t*)w->b_fc2; g.res = x1; g.y = x_out; g.stats_out = stats;
  g.N = H; g.K = F;
  return timed(e, ESM_K_GEMM_FC2, st, "fc2 gemm", [&] { return launch_gemm(EPI_RES_STATS, g, st); });
}

// One pre-LN layer on rows already described by the segment table in ws.
// FP8: the four GEMM inputs are produced in E4M3 by their producers (LN1, the
// attention epilogue, LN2, the fc1 epilogue) with layer li's delayed scales,
// and the GEMMs read layer li's E4M3 weights.
esm_status run_layer(esm_encoder* e, const esm_layer_weights* w, int32_t li, const bf16_t* x_in, bf16_t* x_out,
                     int64_t rows, int32_t B, bool zero_pad_rows, void* ws, const Plan& p, bool* stats_valid,
                     hipStream_t st) {
  if (layer_folded(e, li)) return run_layer_folded(e, w, li, x_in, x_out, rows, B, zero_pad_rows, ws, p, stats_valid, st);
  *stats_valid = false;
  const esm_config& c = e->cfg;
  const int H = c.hidden_size, F = c.intermediate_size, heads = c.num_attention_heads;
  bf16_t* ln1 = region<bf16_t>(ws, p, ESM_WS_LN1);
  bf16_t* qkv = region<bf16_t>(ws, p, ESM_WS_QKV);
  bf16_t* ctx = region<bf16_t>(ws, p, ESM_WS_CTX);
  bf16_t* x1 = region<bf16_t>(ws, p, ESM_WS_X1);
  bf16_t* ln2 = region<bf16_t>(ws, p, ESM_WS_LN2);
  bf16_t* act = region<bf16_t>(ws, p, ESM_WS_ACT);
  const int32_t* pos = region<int32_t>(ws, p, ESM_WS_POS);
  const bool fp8 = layer_fp8(e, li);
  float* as = nullptr;                 // activation scales: ln1, ctx, ln2, act
  uint32_t* am = nullptr;              // their amax slots
  const float* wsc = nullptr;          // weight scales: qkv, out, fc1, fc2
  const uint8_t* w8 = nullptr;
  const W8Off wo = w8_offsets(c);
  if (fp8) {
    as = e->f8.act_scale + 4 * li;
    am = e->f8.act_amax + 4 * li;
    wsc = e->f8.w_scale + 4 * li;
    w8 = e->w8 + (size_t)li * e->w8_layer;
  }
  auto q8 = [&](void* y, int t, const int32_t* rows_pos) {
    return fp8 ? E4m3Out{(uint8_t*)y, as + t, am + t, rows_pos} : E4m3Out{nullptr, nullptr, nullptr, nullptr};
  };
  esm_status s;
  if (layer_mx(e, li)) return run_layer_mx(e, w, li, x_in, x_out, rows, B, zero_pad_rows, ws, p, st);

  s = timed(e, ESM_K_LAYERNORM, st, "layernorm 1", [&] {
    return launch_layernorm(x_in, (const bf16_t*)w->ln1_gamma, (const bf16_t*)w->ln1_beta, ln1, rows, H,
                            c.layer_norm_eps, q8(ln1, 0, zero_pad_rows ? pos : nullptr), st);
  });
  if (s) return s;

  GemmArgs g{};
  g.dtype = fp8 ? kE4M3 : kBF16;
  g.M = rows;
  g.pos = pos;
  g.rope = e->rope;
  g.max_positions = c.max_position_embeddings;
  g.zero_pad_rows = zero_pad_rows ? 1 : 0;
  auto operands = [&](const void* x, const void* wbf, size_t off8, int t) {
    g.x = x;
    g.w = fp8 ? (const void*)(w8 + off8) : wbf;
    g.x_scale = fp8 ? as + t : nullptr;
    g.w_scale = fp8 ? wsc + t : nullptr;
  };

  operands(ln1, w->w_qkv, wo.qkv, 0);
  g.bias = (const bf16_t*)w->b_qkv; g.res = nullptr; g.y = qkv;
  g.N = 3 * H; g.K = H;
  s = timed(e, ESM_K_GEMM_QKV, st, "qkv gemm", [&] { return launch_gemm(EPI_QKV_ROPE, g, st); });
  if (s) return s;

  AttnArgs aa{};
  aa.qkv = qkv; aa.ctx = ctx;
  aa.ctx8 = q8(ctx, 1, nullptr);
  aa.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  aa.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  aa.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  aa.tile_cap = tile_cap(rows, B);
  aa.T = rows; aa.heads = heads;
  s = timed(e, ESM_K_ATTENTION, st, "attention", [&] { return launch_attention(aa, st); });
  if (s) return s;

  operands(ctx, w->w_out, wo.out, 1);
  g.bias = (const bf16_t*)w->b_out; g.res = x_in; g.y = x1;
  g.N = H; g.K = H;
  s = timed(e, ESM_K_GEMM_OUT, st, "out-proj gemm", [&] { return launch_gemm(EPI_BIAS_RESIDUAL, g, st); });
  if (s) return s;

  s = timed(e, ESM_K_LAYERNORM, st, "layernorm 2", [&] {
    return launch_layernorm(x1, (const bf16_t*)w->ln2_gamma, (const bf16_t*)w->ln2_beta, ln2, rows, H,
                            c.layer_norm_eps, q8(ln2, 2, zero_pad_rows ? pos : nullptr), st);
  });
  if (s) return s;

  operands(ln2, w->w_fc1, wo.fc1, 2);
  g.bias = (const bf16_t*)w->b_fc1; g.res = nullptr; g.y = act;
  if (fp8) {
    g.y8 = (uint8_t*)act;
    g.y8_scale = as + 3;
    g.y8_amax = am + 3;
  }
  g.N = F; g.K = H;
  s = timed(e, ESM_K_GEMM_FC1, st, "fc1 gemm",
            [&] { return launch_gemm(fp8 ? EPI_BIAS_GELU_E4M3 : EPI_BIAS_GELU, g, st); });
  if (s) return s;

  operands(act, w->w_fc2, wo.fc2, 3);
  g.bias = (const bf16_t*)w->b_fc2; g.res = x1; g.y = x_out;
  g.N = H; g.K = F;
  return timed(e, ESM_K_GEMM_FC2, st, "fc2 gemm", [&] { return launch_gemm(EPI_BIAS_RESIDUAL, g, st); });
}

// FP8: the call was one step for the layers it ran; roll their histories.
esm_status end_of_step(esm_encoder* e, int nlayers, int32_t layer_idx, hipStream_t st) {
  if (!e->fp8_mem || nlayers == 0) return ok();
  const int32_t l0 = layer_idx >= 0 ? layer_idx : 0;
  return timed(e, ESM_K_FP8, st, "fp8 scale update", [&] { return launch_scale_update(e->f8, l0, nlayers, st); });
}

esm_status check_cu_host(const esm_encoder* e, const int32_t* cu, int32_t B, int64_t T, int32_t max_seqlen) {
  if (max_seqlen < 0 || max_seqlen > e->cfg.max_position_embeddings)
    return fail(ESM_ERR_SEQLENS, "max_seqlen %d outside [0, max_position_embeddings = %d]", max_seqlen,
                e->cfg.max_position_embeddings);
  if (cu) return esm_check_cu_seqlens(cu, B, T, max_seqlen, e->cfg.max_position_embeddings);
  return ok();
}

// Where the stack's two-group schedule splits a batch: the sequence index b
// (group 1 = sequences 0 .. b - 1, group 2 = the rest), or 0 for one group.
// The groups share no rows, so each row's arithmetic is unchanged, while the
// two streams' kernels overlap (one group's attention beside the other's
// GEMMs) and desynchronise their epilogues.  A split is taken only where
// neither group adds rounds of workgroups to the layer's GEMMs (for each
// output width, 3H, H and F, the groups' rounds sum to at most the whole
// batch's): a group whose grid spills into a nearly empty extra round leaves
// most of the chip idle, which the other stream does not fill (the
// 3B-shaped batch, T = 16208 at width 2560, ran 9% slower split).  Among the
// splits that qualify, the most balanced; none below 4096 rows or 2
// sequences, or without the host lengths.
int32_t stack_split(int32_t H, int32_t F, const int32_t* cu_host, int32_t B, int64_t T) {
  if (!cu_host || B < 2 || T < 4096 || H <= 0 || F <= 0) return 0;
  const int32_t widths[3] = {3 * H, H, F};
  int64_t whole[3];
  for (int k = 0; k < 3; ++k) whole[k] = gemm_rounds(T, widths[k]);
  int32_t bs = 0;
  int64_t best = T;
  for (int32_t b = 1; b < B; ++b) {
    const int64_t t1 = cu_host[b], t2 = T - t1;
    if (t1 <= 0 || t2 <= 0) continue;
    bool fits = true;
    for (int k = 0; k < 3 && fits; ++k) fits = gemm_rounds(t1, widths[k]) + gemm_rounds(t2, widths[k]) <= whole[k];
    const int64_t d = t1 * 2 - T;
    if (fits && (d < 0 ? -d : d) < best) {
      best = d < 0 ? -d : d;
      bs = b;
    }
  }
  return bs;
}

esm_status forward_thd(esm_encoder* e, const esm_layer_weights* w, int nlayers, int32_t layer_idx,
                       const int32_t* ids, const void* emb, const void* x_in, void* x_out, const int32_t* cu_dev,
                       const int32_t* cu_host, int32_t B, int64_t T, int32_t max_seqlen, void* ws, size_t ws_bytes,
                       esm_stream_t stream, bool two_groups = false) {
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  esm_status s = check_rows(e, T, B);
  if (s) return s;
  if (T == 0 || B == 0) return ok();
  if (!x_out) return fail(ESM_ERR_NULL, "x_out is NULL");
  if (!aligned16(x_out)) return fail(ESM_ERR_UNSUPPORTED, "x_out not 16-byte aligned");
  if (ids) {
    if (!emb) return fail(ESM_ERR_NULL, "token_ids given without an embedding table");
    if (!aligned16(emb)) return fail(ESM_ERR_UNSUPPORTED, "embedding not 16-byte aligned");
  } else {
    if (!x_in) return fail(ESM_ERR_NULL, "x_in is NULL (and no token ids)");
    if (!aligned16(x_in)) return fail(ESM_ERR_UNSUPPORTED, "x_in not 16-byte aligned");
  }
  if (!cu_dev) return fail(ESM_ERR_NULL, "cu_seqlens_dev is NULL");
  if (!w && nlayers > 0) return fail(ESM_ERR_NULL, "weights are NULL");
  for (int l = 0; l < nlayers; ++l) {
    if ((s = check_weights(&w[l], layer_idx >= 0 ? layer_idx : l))) return s;
    if ((layer_fp8(e, layer_idx >= 0 ? layer_idx : l) || layer_mx(e, layer_idx >= 0 ? layer_idx : l)) &&
        (s = check_quant_layer(e, layer_idx >= 0 ? layer_idx : l)))
      return s;
  }
  if ((s = check_cu_host(e, cu_host, B, T, max_seqlen))) return s;
  if (T == 0 || B == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  const int H = e->cfg.hidden_size;
  // One group of whole sequences (rows r0 .. r0 + Tg - 1, Bg sequences whose
  // cu_seqlens from 0 are cu_g) through the embedding and every layer, on
  // stream sg with its own workspace.
  auto run_group = [&](int64_t r0, int64_t Tg, int32_t Bg, const int32_t* cu_g, void* wsg, const Plan& pg,
                       hipStream_t sg) -> esm_status {
    esm_status q;
    if ((q = run_segments(e, 0, cu_g, Bg, Tg, 0, wsg, pg, sg))) return q;
    bf16_t* xo = (bf16_t*)x_out + r0 * H;
    const bf16_t* cur = x_in ? (const bf16_t*)x_in + r0 * H : nullptr;
    bool stats_valid = false;
    if (ids) {
      // a folded first layer takes its LayerNorm statistics from the gather
      const bool fold0 = nlayers > 0 && layer_folded(e, layer_idx >= 0 ? layer_idx : 0);
      q = timed(e, ESM_K_EMBED, sg, "embedding", [&] {
        return fold0 ? launch_row_stats(ids + r0, (const bf16_t*)emb, e->cfg.vocab_size, xo, Tg, H,
                                        region<float2>(wsg, pg, ESM_WS_STATS), sg)
                     : launch_embed(ids + r0, (const bf16_t*)emb, e->cfg.vocab_size, xo, Tg, H, sg);
      });
      if (q) return q;
      stats_valid = fold0;
      cur = xo;
    }
    for (int l = 0; l < nlayers; ++l) {
      if ((q = run_layer(e, &w[l], layer_idx >= 0 ? layer_idx : l, cur, xo, Tg, Bg, false, wsg, pg, &stats_valid,
                         sg)))
        return q;
      cur = xo;
    }
    return ok();
  };
  // Two groups of whole sequences on two streams when the host lengths are
  // known and the workspace holds both groups' plans (stack_split).
  const int32_t bs = (two_groups && !e->profiling && nlayers > 0)
                         ? stack_split(e->cfg.hidden_size, e->cfg.intermediate_size, cu_host, B, T)
                         : 0;
  if (bs > 0) {
    const int64_t T1 = cu_host[bs], T2 = T - T1;
    const int32_t B1 = bs, B2 = B - bs;
    const Plan p1 = make_plan(e->cfg, T1, B1), p2 = make_plan(e->cfg, T2, B2);
    const size_t o2 = align256(p1.total), oc = o2 + align256(p2.total), need = oc + align256((size_t)(B2 + 1) * 4);
    if (T1 > 0 && T2 > 0 && need <= ws_bytes) {
      if (!e->side) {
        HIP_TRY(hipStreamCreateWithFlags(&e->side, hipStreamNonBlocking), "hipStreamCreateWithFlags");
        HIP_TRY(hipEventCreateWithFlags(&e->fork, hipEventDisableTiming), "hipEventCreateWithFlags");
        HIP_TRY(hipEventCreateWithFlags(&e->join, hipEventDisableTiming), "hipEventCreateWithFlags");
      }
      char* wb = (char*)ws;
      int32_t* cu2 = (int32_t*)(wb + oc);
      HIP_TRY(launch_rebase_cu(cu_dev, bs, B2, cu2, st), "rebase cu_seqlens");
      HIP_TRY(hipEventRecord(e->fork, st), "hipEventRecord");
      HIP_TRY(hipStreamWaitEvent(e->side, e->fork, 0), "hipStreamWaitEvent");
      esm_status s1 = run_group(0, T1, B1, cu_dev, wb, p1, st);
      esm_status s2 = run_group(T1, T2, B2, cu2, wb + o2, p2, e->side);
      // joined on every return, so no work is left behind the caller's stream
      hipError_t j = hipEventRecord(e->join, e->side);
      if (!j) j = hipStreamWaitEvent(st, e->join, 0);
      if (s1) return s1;
      if (s2) return s2;
      if (j) return hip_fail(j, "join");
      return end_of_step(e, nlayers, layer_idx, st);
    }
  }
  if ((s = run_group(0, T, B, cu_dev, ws, p, st))) return s;
  return end_of_step(e, nlayers, layer_idx, st);
}

esm_status forward_bshd(esm_encoder* e, const esm_layer_weights* w, int nlayers, int32_t layer_idx,
                        const int32_t* ids, const void* emb, const void* x_in, void* x_out, const int32_t* sl_dev,
                        const int32_t* sl_host, int32_t B, int32_t S, void* ws, size_t ws_bytes, esm_stream_t stream) {
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (B < 0 || S < 0) return fail(ESM_ERR_SHAPE, "negative B (%d) or S (%d)", B, S);
  const int64_t rows = (int64_t)B * S;
  esm_status s = check_rows(e, rows, B);
  if (s) return s;
  if (rows == 0) return ok();
  if (S > e->cfg.max_position_embeddings)
    return fail(ESM_ERR_SEQLENS, "S = %d above max_position_embeddings %d", S, e->cfg.max_position_embeddings);
  if (!x_out) return fail(ESM_ERR_NULL, "x_out is NULL");
  if (!aligned16(x_out)) return fail(ESM_ERR_UNSUPPORTED, "x_out not 16-byte aligned");
  if (ids) {
    if (!emb) return fail(ESM_ERR_NULL, "token_ids given without an embedding table");
    if (!aligned16(emb)) return fail(ESM_ERR_UNSUPPORTED, "embedding not 16-byte aligned");
  } else {
    if (!x_in) return fail(ESM_ERR_NULL, "x_in is NULL (and no token ids)");
    if (!aligned16(x_in)) return fail(ESM_ERR_UNSUPPORTED, "x_in not 16-byte aligned");
  }
  if (!sl_dev) return fail(ESM_ERR_NULL, "seqlens_dev is NULL");
  if (!w && nlayers > 0) return fail(ESM_ERR_NULL, "weights are NULL");
  for (int l = 0; l < nlayers; ++l) {
    if ((s = check_weights(&w[l], layer_idx >= 0 ? layer_idx : l))) return s;
    if ((layer_fp8(e, layer_idx >= 0 ? layer_idx : l) || layer_mx(e, layer_idx >= 0 ? layer_idx : l)) &&
        (s = check_quant_layer(e, layer_idx >= 0 ? layer_idx : l)))
      return s;
  }
  if (sl_host && (s = esm_check_seqlens(sl_host, B, S, e->cfg.max_position_embeddings))) return s;
  if (rows == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, rows, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = run_segments(e, 1, sl_dev, B, rows, S, ws, p, st))) return s;
  const bf16_t* cur = (const bf16_t*)x_in;
  bool stats_valid = false;
  if (ids) {
    // a folded first layer takes its LayerNorm statistics from the gather
    const bool fold0 = nlayers > 0 && layer_folded(e, layer_idx >= 0 ? layer_idx : 0);
    s = timed(e, ESM_K_EMBED, st, "embedding", [&] {
      return fold0 ? launch_row_stats(ids, (const bf16_t*)emb, e->cfg.vocab_size, (bf16_t*)x_out, rows,
                                      e->cfg.hidden_size, region<float2>(ws, p, ESM_WS_STATS), st)
                   : launch_embed(ids, (const bf16_t*)emb, e->cfg.vocab_size, (bf16_t*)x_out, rows,
                                  e->cfg.hidden_size, st);
    });
    if (s) return s;
    stats_valid = fold0;
    cur = (const bf16_t*)x_out;
  }
  for (int l = 0; l < nlayers; ++l) {
    if ((s = run_layer(e, &w[l], layer_idx >= 0 ? layer_idx : l, cur, (bf16_t*)x_out, rows, B, true, ws, p,
                       &stats_valid, st)))
      return s;
    cur = (const bf16_t*)x_out;
  }
  return end_of_step(e, nlayers, layer_idx, st);
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

void esm_config_default(esm_config* c) {
  if (!c) return;
  c->hidden_size = 1280;
  c->num_attention_heads = 20;
  c->intermediate_size = 5120;
  c->num_hidden_layers = 33;
  c->vocab_size = 33;
  c->max_position_embeddings = 1026;
  c->layer_norm_eps = 1e-5f;
  c->rope_base = 10000.f;
  c->precision = ESM_PRECISION_BF16;
  c->amax_history_len = 16;
}

esm_status esm_encoder_create(const esm_config* cfg, int device, esm_encoder** out) {
  g_last_error.clear();
  if (!out) return fail(ESM_ERR_NULL, "out is NULL");
  *out = nullptr;
  esm_status s = check_config(cfg);
  if (s) return s;
  int n = 0;
  HIP_TRY(hipGetDeviceCount(&n), "hipGetDeviceCount");
  if (device < 0 || device >= n) return fail(ESM_ERR_ARCH, "device %d not present (%d devices)", device, n);
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, device), "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(ESM_ERR_ARCH, "device %d is %s; this library is built for gfx950 only", device, prop.gcnArchName);
  HIP_TRY(hipSetDevice(device), "hipSetDevice");
  void* scr = nullptr;
  HIP_TRY(scratch_on_device(device, &scr), "device scratch address (hipGetSymbolAddress)");
  esm_encoder* e = new esm_encoder();
  e->cfg = *cfg;
  e->device = device;
  e->scratch = scr;
  // Rotary table: theta = p * base^(-i/32), i < 32, in fp64 then rounded
  // ([TE-ESM2] 旋转位置编码集成).
  const int P = cfg->max_position_embeddings;
  std::vector<float2> tab((size_t)P * 32);
  for (int p = 0; p < P; ++p)
    for (int i = 0; i < 32; ++i) {
      const double th = (double)p * pow((double)cfg->rope_base, -(double)i / 32.0);
      tab[(size_t)p * 32 + i] = make_float2((float)cos(th), (float)sin(th));
    }
  hipError_t err = hipMalloc((void**)&e->rope, tab.size() * sizeof(float2));
  if (err == hipSuccess) err = hipMemcpy(e->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (err != hipSuccess) {
    if (e->rope) (void)hipFree(e->rope);
    delete e;
    return hip_fail(err, "rotary table");
  }
  if (is_quantised(e))
    e->layer_prec.assign((size_t)(cfg->num_hidden_layers > 0 ? cfg->num_hidden_layers : 1), cfg->precision);
  if ((is_fp8(e) && (s = ensure_fp8(e)) != ESM_OK) || (is_mx(e) && (s = ensure_mx(e)) != ESM_OK)) {
    esm_encoder_destroy(e);
    return s;
  }
  if (cfg->vocab_size <= kHeadMaxVocab) {
    e->vocab_pad = (cfg->vocab_size + 63) / 64 * 64;
    err = hipMalloc((void**)&e->head_w, (size_t)e->vocab_pad * ((size_t)cfg->hidden_size + 1) * sizeof(bf16_t));
    if (err != hipSuccess) {
      esm_encoder_destroy(e);
      return hip_fail(err, "LM head decoder buffer");
    }
  }
  *out = e;
  return ok();
}

esm_status esm_encoder_destroy(esm_encoder* e) {
  if (!e) return ESM_OK;
  (void)hipSetDevice(e->device);
  if (e->rope) (void)hipFree(e->rope);
  if (e->fp8_mem) (void)hipFree(e->fp8_mem);
  if (e->w8) (void)hipFree(e->w8);
  if (e->w4) (void)hipFree(e->w4);
  if (e->head_w) (void)hipFree(e->head_w);
  if (e->fold) (void)hipFree(e->fold);
  for (hipEvent_t ev : e->pool) (void)hipEventDestroy(ev);
  if (e->fork) (void)hipEventDestroy(e->fork);
  if (e->join) (void)hipEventDestroy(e->join);
  if (e->side) (void)hipStreamDestroy(e->side);
  delete e;
  return ESM_OK;
}

esm_status esm_workspace_size(const esm_encoder* e, int64_t max_tokens, int32_t max_seqs, size_t* bytes) {
  if (!e || !bytes) return fail(ESM_ERR_NULL, "encoder or bytes is NULL");
  if (max_tokens < 0 || max_seqs < 0) return fail(ESM_ERR_SHAPE, "negative sizes");
  // plus room for the stack's two-group schedule (a second plan's alignment
  // and tile slack, and the second group's rebased cu_seqlens)
  *bytes = make_plan(e->cfg, max_tokens, max_seqs).total + 8192 + align256((size_t)(max_seqs + 1) * 4);
  return ok();
}

esm_status esm_workspace_region(const esm_encoder* e, int64_t max_tokens, int32_t max_seqs, int32_t r,
                                size_t* offset, size_t* bytes) {
  if (!e || !offset || !bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (r < 0 || r > ESM_WS_STATS) return fail(ESM_ERR_UNSUPPORTED, "unknown region %d", r);
  const Plan p = make_plan(e->cfg, max_tokens, max_seqs);
  *offset = p.off[r];
  *bytes = p.size[r];
  return ok();
}

esm_status esm_layer_fwd(esm_encoder* e, const esm_layer_weights* w, int32_t layer_idx, const void* x_in, void* x_out,
                         const int32_t* cu_dev, const int32_t* cu_host, int32_t B, int64_t T, int32_t max_seqlen,
                         void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  return forward_thd(e, w, 1, layer_idx, nullptr, nullptr, x_in, x_out, cu_dev, cu_host, B, T, max_seqlen, ws,
                     ws_bytes, stream);
}

esm_status esm_layer_fwd_noalloc(esm_encoder* e, const esm_layer_weights* w, int32_t layer_idx, const void* x_in,
                                 void* x_out, const int32_t* cu_dev, const int32_t* cu_host, int32_t B, int64_t T,
                                 int32_t max_seqlen, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (!e->scratch) return fail(ESM_ERR_STATE, "device scratch not resolved");
  if (T >= 0 && B >= 0) {
    const size_t need = make_plan(e->cfg, T, B).total;
    if (need > (size_t)ESM_NOALLOC_SCRATCH_BYTES)
      return fail(ESM_ERR_WORKSPACE,
                  "T = %lld rows, B = %d sequences need %zu bytes of scratch; the allocation-free entry has %zu "
                  "(use esm_layer_fwd with a caller workspace)",
                  (long long)T, B, need, (size_t)ESM_NOALLOC_SCRATCH_BYTES);
  }
  // no timing events: recording them may create events, which allocates
  const bool prof = e->profiling;
  e->profiling = false;
  const esm_status s = forward_thd(e, w, 1, layer_idx, nullptr, nullptr, x_in, x_out, cu_dev, cu_host, B, T,
                                   max_seqlen, e->scratch, (size_t)ESM_NOALLOC_SCRATCH_BYTES, stream);
  e->profiling = prof;
  return s;
}

esm_status esm_stack_fwd(esm_encoder* e, const esm_layer_weights* w, const int32_t* ids, const void* emb,
                         const void* x_in, void* x_out, const int32_t* cu_dev, const int32_t* cu_host, int32_t B,
                         int64_t T, int32_t max_seqlen, void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  return forward_thd(e, w, e->cfg.num_hidden_layers, -1, ids, emb, x_in, x_out, cu_dev, cu_host, B, T, max_seqlen,
                     ws, ws_bytes, stream, true);
}

esm_status esm_stack_split(int32_t hidden_size, int32_t intermediate_size, const int32_t* cu_seqlens_host, int32_t B,
                           int64_t T, int32_t* split_seq) {
  g_last_error.clear();
  if (!cu_seqlens_host || !split_seq) return fail(ESM_ERR_NULL, "NULL argument");
  if (B < 0 || T < 0 || hidden_size <= 0 || intermediate_size <= 0) return fail(ESM_ERR_SHAPE, "bad sizes");
  if (cu_seqlens_host[0] != 0 || cu_seqlens_host[B] != T)
    return fail(ESM_ERR_SHAPE, "cu_seqlens must run from 0 to T");
  *split_seq = stack_split(hidden_size, intermediate_size, cu_seqlens_host, B, T);
  return ok();
}

esm_status esm_head_fwd(esm_encoder* e, const esm_head_weights* w, const void* x, void* x_final, void* logits,
                        float* seq_emb, const int32_t* cu_dev, const int32_t* cu_host, int32_t B, int64_t T,
                        int32_t max_seqlen, void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !w) return fail(ESM_ERR_NULL, "encoder or head weights NULL");
  esm_status s = check_rows(e, T, B);
  if (s) return s;
  if (T > 0 && (!x || !x_final)) return fail(ESM_ERR_NULL, "x or x_final is NULL");
  if (!aligned16(x) || !aligned16(x_final)) return fail(ESM_ERR_UNSUPPORTED, "x / x_final not 16-byte aligned");
  if (!w->final_ln_gamma || !w->final_ln_beta) return fail(ESM_ERR_NULL, "final LayerNorm weights NULL");
  if (!aligned16(w->final_ln_gamma) || !aligned16(w->final_ln_beta))
    return fail(ESM_ERR_UNSUPPORTED, "final LayerNorm weights not 16-byte aligned");
  if (logits) {
    const void* req[] = {w->lm_dense_w, w->lm_ln_gamma, w->lm_ln_beta, w->lm_decoder_w};
    for (const void* q : req) {
      if (!q) return fail(ESM_ERR_NULL, "LM head weight NULL");
      if (!aligned16(q)) return fail(ESM_ERR_UNSUPPORTED, "LM head weight not 16-byte aligned");
    }
    if (w->lm_dense_b && ((uintptr_t)w->lm_dense_b & 7u)) return fail(ESM_ERR_UNSUPPORTED, "lm_dense_b not 8-byte aligned");
    if (!e->head_w || e->vocab_pad > 3 * e->cfg.hidden_size)
      return fail(ESM_ERR_UNSUPPORTED, "vocab %d: the LM head takes up to min(%d, 3 * hidden) rows", e->cfg.vocab_size,
                  kHeadMaxVocab);
  }
  if (seq_emb && !cu_dev) return fail(ESM_ERR_NULL, "seq_emb needs cu_seqlens_dev");
  if ((s = check_cu_host(e, cu_host, B, T, max_seqlen))) return s;
  if (T == 0 && (B == 0 || !seq_emb)) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  const esm_config& c = e->cfg;
  const int H = c.hidden_size;
  if (T > 0) {
    s = timed(e, ESM_K_HEAD, st, "final layernorm", [&] {
      return launch_layernorm((const bf16_t*)x, (const bf16_t*)w->final_ln_gamma, (const bf16_t*)w->final_ln_beta,
                              (bf16_t*)x_final, T, H, c.layer_norm_eps, E4m3Out{nullptr, nullptr, nullptr, nullptr}, st);
    });
    if (s) return s;
  }
  if (seq_emb && B > 0) {
    if ((s = run_segments(e, ESM_LAYOUT_THD, cu_dev, B, T, 0, ws, p, st))) return s;
    s = timed(e, ESM_K_HEAD, st, "sequence means", [&] {
      return launch_segment_mean((const bf16_t*)x_final, region<int32_t>(ws, p, ESM_WS_SEGS), B, H, seq_emb, st);
    });
    if (s) return s;
  }
  if (!logits || T == 0) return ok();
  // LM head: dense + GELU into ACT, its LayerNorm into LN1, the decoder over
  // vocab_pad columns into the QKV region ([T, vocab_pad] bf16 fits in
  // [3, heads, T, 64]), then the first vocab columns into logits.
  const int V = c.vocab_size, VP = e->vocab_pad;
  bf16_t* dense = region<bf16_t>(ws, p, ESM_WS_ACT);
  bf16_t* hn = region<bf16_t>(ws, p, ESM_WS_LN1);
  bf16_t* padded = region<bf16_t>(ws, p, ESM_WS_QKV);
  bf16_t* wdec = e->head_w;
  bf16_t* bdec = e->head_w + (size_t)VP * H;
  s = timed(e, ESM_K_HEAD, st, "pad decoder", [&] {
    hipError_t r = launch_pad_rows((const bf16_t*)w->lm_decoder_w, V, H, wdec, VP, st);
    return r != hipSuccess ? r : launch_pad_rows((const bf16_t*)w->lm_decoder_b, w->lm_decoder_b ? V : 0, 1, bdec, VP, st);
  });
  if (s) return s;
  GemmArgs g{};
  g.dtype = kBF16;
  g.x = x_final; g.w = w->lm_dense_w; g.bias = (const bf16_t*)w->lm_dense_b; g.y = dense;
  g.M = T; g.N = H; g.K = H;
  s = timed(e, ESM_K_HEAD, st, "lm dense gemm", [&] { return launch_gemm(EPI_BIAS_GELU, g, st); });
  if (s) return s;
  s = timed(e, ESM_K_HEAD, st, "lm layernorm", [&] {
    return launch_layernorm(dense, (const bf16_t*)w->lm_ln_gamma, (const bf16_t*)w->lm_ln_beta, hn, T, H,
                            c.layer_norm_eps, E4m3Out{nullptr, nullptr, nullptr, nullptr}, st);
  });
  if (s) return s;
  g.x = hn; g.w = wdec; g.bias = bdec; g.y = padded;
  g.N = VP;
  s = timed(e, ESM_K_HEAD, st, "lm decoder gemm", [&] { return launch_gemm(EPI_BIAS, g, st); });
  if (s) return s;
  return timed(e, ESM_K_HEAD, st, "logits", [&] { return launch_take_cols(padded, VP, (bf16_t*)logits, T, V, st); });
}

esm_status esm_layer_fwd_bshd(esm_encoder* e, const esm_layer_weights* w, int32_t layer_idx, const void* x_in,
                              void* x_out, const int32_t* sl_dev, const int32_t* sl_host, int32_t B, int32_t S,
                              void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  return forward_bshd(e, w, 1, layer_idx, nullptr, nullptr, x_in, x_out, sl_dev, sl_host, B, S, ws, ws_bytes, stream);
}

esm_status esm_stack_fwd_bshd(esm_encoder* e, const esm_layer_weights* w, const int32_t* ids, const void* emb,
                              const void* x_in, void* x_out, const int32_t* sl_dev, const int32_t* sl_host, int32_t B,
                              int32_t S, void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  return forward_bshd(e, w, e->cfg.num_hidden_layers, -1, ids, emb, x_in, x_out, sl_dev, sl_host, B, S, ws, ws_bytes,
                      stream);
}

esm_status esm_segment_table(esm_encoder* e, int32_t layout, const int32_t* lens_dev, int32_t B, int64_t T, int32_t S,
                             void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !lens_dev) return fail(ESM_ERR_NULL, "encoder or lengths NULL");
  if (layout != ESM_LAYOUT_THD && layout != ESM_LAYOUT_BSHD) return fail(ESM_ERR_UNSUPPORTED, "layout %d", layout);
  if (layout == ESM_LAYOUT_BSHD) {
    if (S < 0 || B < 0) return fail(ESM_ERR_SHAPE, "negative B or S");
    T = (int64_t)B * S;
  }
  esm_status s = check_rows(e, T, B);
  if (s) return s;
  if (T == 0 && B == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  return run_segments(e, layout, lens_dev, B, T, S, ws, p, (hipStream_t)stream);
}

esm_status esm_attention_fwd(esm_encoder* e, const void* qkv, void* ctx, const int32_t* cu_dev, int32_t B, int64_t T,
                             void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !qkv || !ctx || !cu_dev) return fail(ESM_ERR_NULL, "NULL argument");
  if (!aligned16(qkv) || !aligned16(ctx)) return fail(ESM_ERR_UNSUPPORTED, "qkv/ctx not 16-byte aligned");
  esm_status s = check_rows(e, T, B);
  if (s) return s;
  if (T == 0 || B == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = run_segments(e, 0, cu_dev, B, T, 0, ws, p, st))) return s;
  AttnArgs aa{};
  aa.qkv = (const bf16_t*)qkv; aa.ctx = (bf16_t*)ctx;
  aa.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  aa.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  aa.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  aa.tile_cap = tile_cap(T, B);
  aa.T = T; aa.heads = e->cfg.num_attention_heads;
  return timed(e, ESM_K_ATTENTION, st, "attention", [&] { return launch_attention(aa, st); });
}

esm_status esm_attention_fwd_lse(esm_encoder* e, const void* qkv, void* ctx, float* lse, const int32_t* cu_dev,
                                 int32_t B, int64_t T, void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !qkv || !ctx || !lse || !cu_dev) return fail(ESM_ERR_NULL, "NULL argument");
  if (!aligned16(qkv) || !aligned16(ctx)) return fail(ESM_ERR_UNSUPPORTED, "qkv/ctx not 16-byte aligned");
  if ((uintptr_t)lse & 3u) return fail(ESM_ERR_UNSUPPORTED, "lse not 4-byte aligned");
  esm_status s = check_rows(e, T, B);
  if (s) return s;
  if (T == 0 || B == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = run_segments(e, 0, cu_dev, B, T, 0, ws, p, st))) return s;
  AttnArgs aa{};
  aa.qkv = (const bf16_t*)qkv; aa.ctx = (bf16_t*)ctx; aa.lse = lse;
  aa.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  aa.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  aa.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  aa.tile_cap = tile_cap(T, B);
  aa.T = T; aa.heads = e->cfg.num_attention_heads;
  return timed(e, ESM_K_ATTENTION, st, "attention", [&] { return launch_attention(aa, st); });
}

esm_status esm_attention_bwd(esm_encoder* e, const void* qkv, const void* ctx, const void* dctx, const float* lse,
                             float* delta, void* dqkv, const int32_t* cu_dev, int32_t B, int64_t T, void* ws,
                             size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !qkv || !ctx || !dctx || !lse || !delta || !dqkv || !cu_dev) return fail(ESM_ERR_NULL, "NULL argument");
  if (!aligned16(qkv) || !aligned16(ctx) || !aligned16(dctx) || !aligned16(dqkv))
    return fail(ESM_ERR_UNSUPPORTED, "qkv/ctx/dctx/dqkv not 16-byte aligned");
  if (((uintptr_t)lse & 3u) || ((uintptr_t)delta & 3u)) return fail(ESM_ERR_UNSUPPORTED, "lse/delta not 4-byte aligned");
  esm_status s = check_rows(e, T, B);
  if (s) return s;
  if (T == 0 || B == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = run_segments(e, 0, cu_dev, B, T, 0, ws, p, st))) return s;
  AttnBwdArgs a{};
  a.qkv = (const bf16_t*)qkv; a.out = (const bf16_t*)ctx; a.dout = (const bf16_t*)dctx;
  a.lse = lse; a.delta = delta; a.dqkv = (bf16_t*)dqkv;
  a.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  a.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  a.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  a.tile_cap = tile_cap(T, B);
  a.T = T; a.heads = e->cfg.num_attention_heads;
  return timed(e, ESM_K_ATTENTION_BWD, st, "attention_bwd", [&] { return launch_attention_bwd(a, st); });
}

esm_status esm_biased_attention_fwd(esm_encoder* e, const void* q, const void* k, const void* v,
                                    const void* mask_bias, const void* pair_bias, void* out, int32_t B, int32_t N,
                                    int32_t L, int32_t heads, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "NULL encoder");
  if (B < 0 || N < 0 || L < 0 || heads < 0 || L > 65536)
    return fail(ESM_ERR_SHAPE, "B %d N %d L %d heads %d", B, N, L, heads);
  if (B == 0 || N == 0 || L == 0 || heads == 0) return ok();
  if (!q || !k || !v || !out) return fail(ESM_ERR_NULL, "NULL argument");
  const int32_t qtiles = (L + kAttnTileRows - 1) / kAttnTileRows;
  if ((int64_t)B * N * qtiles * heads > INT32_MAX)
    return fail(ESM_ERR_SHAPE, "B %d N %d L %d heads %d: more than 2^31 - 1 workgroups", B, N, L, heads);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(ESM_ERR_UNSUPPORTED, "q/k/v/out not 16-byte aligned");
  const uintptr_t bias_align = L % 4 == 0 ? 7u : 1u;
  if (((uintptr_t)mask_bias & bias_align) || ((uintptr_t)pair_bias & bias_align))
    return fail(ESM_ERR_UNSUPPORTED, "bias not %d-byte aligned", (int)bias_align + 1);
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  BiasedAttnArgs a{};
  a.q = (const bf16_t*)q; a.k = (const bf16_t*)k; a.v = (const bf16_t*)v;
  a.mask = (const bf16_t*)mask_bias; a.pair = (const bf16_t*)pair_bias; a.out = (bf16_t*)out;
  a.B = B; a.N = N; a.L = L; a.heads = heads; a.qtiles = qtiles;
  hipStream_t st = (hipStream_t)stream;
  return timed(e, ESM_K_BIASED_ATTENTION, st, "biased attention", [&] { return launch_biased_attention(a, st); });
}

esm_status esm_mxfp4_quantize(esm_encoder* e, const void* x, int64_t M, int32_t K, void* codes, void* scales,
                              esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "NULL encoder");
  if (M < 0 || K <= 0 || K % 256) return fail(ESM_ERR_SHAPE, "M %lld K %d: K must be a positive multiple of 256",
                                              (long long)M, K);
  if (M == 0) return ok();
  if (!x || !codes || !scales) return fail(ESM_ERR_NULL, "NULL argument");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return fail(ESM_ERR_UNSUPPORTED, "x/codes/scales not 16-byte aligned");
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  return timed(e, ESM_K_OTHER, (hipStream_t)stream, "mxfp4 quantize", [&] {
    return launch_mx_quantize((const bf16_t*)x, M, K, (uint8_t*)codes, (uint8_t*)scales, (hipStream_t)stream);
  });
}

esm_status esm_linear_mxfp4_fwd(esm_encoder* e, const void* xc, const void* xs, const void* wc, const void* ws,
                                const void* b, const void* res, void* y, int64_t M, int32_t N, int32_t K, int32_t epi,
                                esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !xc || !xs || !wc || !ws || !y) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 256)
    return fail(ESM_ERR_SHAPE, "M %lld N %d K %d: N must be a positive multiple of 64 and K of 256", (long long)M, N,
                K);
  if (epi < ESM_EPI_BIAS || epi > ESM_EPI_BIAS_RESIDUAL) return fail(ESM_ERR_UNSUPPORTED, "epilogue %d", epi);
  if (epi == ESM_EPI_BIAS_RESIDUAL && !res) return fail(ESM_ERR_NULL, "residual is NULL");
  if (!aligned16(xc) || !aligned16(xs) || !aligned16(wc) || !aligned16(ws) || !aligned16(y) ||
      (res && !aligned16(res)) || (b && ((uintptr_t)b & 7u)))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  GemmArgs g{};
  g.dtype = kFP4;
  g.x = xc; g.w = wc; g.x_sc = (const uint8_t*)xs; g.w_sc = (const uint8_t*)ws;
  g.bias = (const bf16_t*)b; g.res = (const bf16_t*)res;
  g.y = (bf16_t*)y; g.M = M; g.N = N; g.K = K;
  const int kind = epi == ESM_EPI_BIAS ? EPI_BIAS : (epi == ESM_EPI_BIAS_GELU ? EPI_BIAS_GELU : EPI_BIAS_RESIDUAL);
  return timed(e, ESM_K_OTHER, (hipStream_t)stream, "mxfp4 linear",
               [&] { return launch_gemm(kind, g, (hipStream_t)stream); });
}

esm_status esm_linear_fwd(esm_encoder* e, const void* x, const void* w, const void* b, const void* res, void* y,
                          int64_t M, int32_t N, int32_t K, int32_t epi, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !x || !w || !y) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64)
    return fail(ESM_ERR_SHAPE, "M %lld N %d K %d: N and K must be positive multiples of 64", (long long)M, N, K);
  if (epi < ESM_EPI_BIAS || epi > ESM_EPI_BIAS_RESIDUAL) return fail(ESM_ERR_UNSUPPORTED, "epilogue %d", epi);
  if (epi == ESM_EPI_BIAS_RESIDUAL && !res) return fail(ESM_ERR_NULL, "residual is NULL");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (res && !aligned16(res)) || (b && ((uintptr_t)b & 7u)))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  GemmArgs g{};
  g.dtype = kBF16;
  g.x = x; g.w = w; g.bias = (const bf16_t*)b; g.res = (const bf16_t*)res;
  g.y = (bf16_t*)y; g.M = M; g.N = N; g.K = K;
  const int kind = epi == ESM_EPI_BIAS ? EPI_BIAS : (epi == ESM_EPI_BIAS_GELU ? EPI_BIAS_GELU : EPI_BIAS_RESIDUAL);
  return timed(e, ESM_K_OTHER, (hipStream_t)stream, "linear", [&] { return launch_gemm(kind, g, (hipStream_t)stream); });
}

namespace {
struct LinBwdPlan {
  int32_t splits;  // slices of the dW GEMM's contraction over M
  size_t wt, part, wpart, total;
};
LinBwdPlan lin_bwd_plan(int64_t M, int32_t N, int32_t K) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  LinBwdPlan p;
  p.splits = wgrad_splits(M, N, K);
  p.wt = 0;
  p.part = p.wt + up((size_t)K * N * 2);
  p.wpart = p.part + up((size_t)colsum_chunks(M) * N * 4);
  p.total = p.wpart + up((size_t)p.splits * N * K * 4);
  return p;
}
}  // namespace

esm_status esm_linear_bwd_workspace_size(int64_t M, int32_t N, int32_t K, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64)
    return fail(ESM_ERR_SHAPE, "M %lld N %d K %d: N and K must be positive multiples of 64", (long long)M, N, K);
  *bytes = lin_bwd_plan(M, N, K).total;
  return ok();
}

esm_status esm_linear_bwd(esm_encoder* e, const void* x, const void* w, const void* dy, void* dx, void* dw, float* db,
                          int64_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !dy || !ws) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64)
    return fail(ESM_ERR_SHAPE, "M %lld N %d K %d: N and K must be positive multiples of 64", (long long)M, N, K);
  if ((dx && !w) || (dw && !x)) return fail(ESM_ERR_NULL, "dx needs w, dw needs x");
  if (dw && M > (int64_t)INT32_MAX - 1024)
    return fail(ESM_ERR_SHAPE, "M %lld: dW takes fewer than 2^31 - 1024 rows", (long long)M);
  if (!aligned16(dy) || (x && !aligned16(x)) || (w && !aligned16(w)) || (dx && !aligned16(dx)) ||
      (dw && !aligned16(dw)) || ((uintptr_t)db & 3u) || ((uintptr_t)ws & 255u))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer (tensors 16 bytes, db 4, workspace 256)");
  const LinBwdPlan pl = lin_bwd_plan(M, N, K);
  if (ws_bytes < pl.total)
    return fail(ESM_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, pl.total);
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  bf16_t* wt = (bf16_t*)(base + pl.wt);
  float* part = (float*)(base + pl.part);
  float* wpart = (float*)(base + pl.wpart);
  if (dw && !e->side) {
    HIP_TRY(hipStreamCreateWithFlags(&e->side, hipStreamNonBlocking), "hipStreamCreateWithFlags");
    HIP_TRY(hipEventCreateWithFlags(&e->fork, hipEventDisableTiming), "hipEventCreateWithFlags");
    HIP_TRY(hipEventCreateWithFlags(&e->join, hipEventDisableTiming), "hipEventCreateWithFlags");
  }
  return timed(e, ESM_K_LINEAR_BWD, st, "linear backward", [&]() -> hipError_t {
    hipError_t r = hipSuccess;
    // The dW GEMM's output is small (N x K: tens of tiles for hundreds of
    // compute units) with a long contraction over M: it is cut into slices of
    // M (fp32 partial products summed in slice order), and it runs on the side
    // stream, forked from and joined back to st, beside the dx GEMM and the
    // column sums.  It reads dy and x as they are, contraction-major (no
    // transposed copies).  The workspace regions of the two paths are
    // disjoint.
    // Once the side stream has been forked it is joined back to st on every
    // return, errors included, so that no work on ws or dw is left running
    // behind the caller's stream.
    bool forked = false;
    if (dw) {
      if ((r = hipEventRecord(e->fork, st))) return r;
      if ((r = hipStreamWaitEvent(e->side, e->fork, 0))) return r;
      forked = true;
      // dW [N, K] = sum over m of dy[m, n] x[m, k]: each slice of M's fp32
      // product (slices of M rounded up to 64 * splits, divided by splits,
      // rows past M zero), then their sum in slice order, rounded once
      GemmArgs g{};
      g.dtype = kBF16;
      g.x = dy; g.w = x; g.M = N; g.N = K; g.K = (int32_t)M;
      g.y32 = wpart; g.ksplit = pl.splits;
      r = launch_gemm(EPI_F32_SPLIT_KM, g, e->side);
      if (!r) r = launch_split_reduce(wpart, pl.splits, (int64_t)N * K, (bf16_t*)dw, e->side);
    }
    if (!r && dx) {
      // dx [M, K] = dy [M, N] . (W^T [K, N])^T
      r = launch_transpose_pad((const bf16_t*)w, N, K, wt, N, st);
      if (!r) {
        GemmArgs g{};
        g.dtype = kBF16;
        g.x = dy; g.w = wt; g.y = (bf16_t*)dx; g.M = M; g.N = K; g.K = N;
        r = launch_gemm(EPI_BIAS, g, st);
      }
    }
    if (!r && db) r = launch_colsum((const bf16_t*)dy, M, N, part, db, st);
    if (forked) {
      hipError_t j = hipEventRecord(e->join, e->side);
      if (!j) j = hipStreamWaitEvent(st, e->join, 0);
      if (!r) r = j;
    }
    return r;
  });
}

namespace {
size_t ln_bwd_stats_bytes(int64_t M) { return ((size_t)M * 8 + 255) / 256 * 256; }
size_t ln_bwd_ws_bytes(int64_t M, int32_t H) {
  return ln_bwd_stats_bytes(M) + (size_t)colsum_chunks(M) * 2 * H * 4;
}
}  // namespace

esm_status esm_layernorm_bwd_workspace_size(int64_t M, int32_t H, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || H <= 0 || H % 64 || H > 4096)
    return fail(ESM_ERR_SHAPE, "M %lld H %d: H must be a positive multiple of 64, at most 4096", (long long)M, H);
  *bytes = ln_bwd_ws_bytes(M, H);
  return ok();
}

esm_status esm_layernorm_bwd(esm_encoder* e, const void* x, const void* gamma, const void* dy, void* dx,
                             float* dgamma, float* dbeta, int64_t M, void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !x || !gamma || !dy || !dx || !dgamma || !dbeta || !ws) return fail(ESM_ERR_NULL, "NULL argument");
  const int32_t H = e->cfg.hidden_size;
  if (M < 0) return fail(ESM_ERR_SHAPE, "M < 0");
  if (H % 64 || H > 4096) return fail(ESM_ERR_UNSUPPORTED, "hidden %d: the LayerNorm backward takes multiples of 64 up to 4096", H);
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(dy) || !aligned16(dx) || ((uintptr_t)dgamma & 3u) ||
      ((uintptr_t)dbeta & 3u) || ((uintptr_t)ws & 255u))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer (tensors 16 bytes, dgamma/dbeta 4, workspace 256)");
  const size_t need = ln_bwd_ws_bytes(M, H);
  if (ws_bytes < need) return fail(ESM_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  float* stats = (float*)ws;
  float* part = (float*)((char*)ws + ln_bwd_stats_bytes(M));
  return timed(e, ESM_K_LINEAR_BWD, st, "layernorm backward", [&] {
    return launch_layernorm_bwd((const bf16_t*)x, (const bf16_t*)gamma, (const bf16_t*)dy, nullptr, (bf16_t*)dx, dgamma,
                                dbeta, M, H, e->cfg.layer_norm_eps, stats, part, st);
  });
}

esm_status esm_e5m2_quantize(esm_encoder* e, const void* x, int64_t n, const float* scale, void* y8, uint32_t* amax,
                             esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !x || !scale || !y8 || !amax) return fail(ESM_ERR_NULL, "NULL argument");
  if (n < 0 || n % 8) return fail(ESM_ERR_SHAPE, "n %lld: a non-negative multiple of 8", (long long)n);
  if (!aligned16(x) || ((uintptr_t)y8 & 7u) || ((uintptr_t)scale & 3u) || ((uintptr_t)amax & 3u))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (n == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  return timed(e, ESM_K_LINEAR_BWD, st, "e5m2 quantize", [&] {
    return launch_quantize_e5m2((const bf16_t*)x, n, scale, (uint8_t*)y8, amax, st);
  });
}

esm_status esm_linear_e5m2_dgrad(esm_encoder* e, const void* dy8, const float* dy_scale, const void* wt8,
                                 const float* w_scale, void* dx, int64_t M, int32_t N, int32_t K,
                                 esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !dy8 || !dy_scale || !wt8 || !w_scale || !dx) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || N <= 0 || K <= 0 || N % 128 || K % 64)
    return fail(ESM_ERR_SHAPE, "M %lld N %d K %d: N a positive multiple of 128, K of 64", (long long)M, N, K);
  if (!aligned16(dy8) || !aligned16(wt8) || !aligned16(dx)) return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  GemmArgs g{};
  g.dtype = kE5M2X;
  g.x = dy8; g.w = wt8; g.x_scale = dy_scale; g.w_scale = w_scale;
  g.y = (bf16_t*)dx; g.M = M; g.N = K; g.K = N;
  return timed(e, ESM_K_LINEAR_BWD, st, "e5m2 dgrad", [&] { return launch_gemm(EPI_BIAS, g, st); });
}

namespace {
// E5M2 weight gradient: dy^T [N, Mp] and x^T [K, Mp] as bytes (rows past M
// zero), then, with S > 1 K slices, the slices' fp32 products [S, N, K].
struct E5WgradPlan {
  int32_t splits;
  int64_t Mp;
  size_t dyt, xt, wpart, total;
};
E5WgradPlan e5_wgrad_plan(int64_t M, int32_t N, int32_t K) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  E5WgradPlan p;
  p.splits = wgrad_splits(M, N, K);
  const int64_t q = 128 * (int64_t)p.splits;
  p.Mp = (M + q - 1) / q * q;
  p.dyt = 0;
  p.xt = up((size_t)N * p.Mp);
  p.wpart = p.xt + up((size_t)K * p.Mp);
  p.total = p.wpart + (p.splits > 1 ? up((size_t)p.splits * N * K * 4) : 0);
  return p;
}
}  // namespace

esm_status esm_linear_e5m2_wgrad_workspace_size(int64_t M, int32_t N, int32_t K, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64)
    return fail(ESM_ERR_SHAPE, "M %lld N %d K %d: N and K must be positive multiples of 64", (long long)M, N, K);
  *bytes = e5_wgrad_plan(M, N, K).total;
  return ok();
}

esm_status esm_linear_e5m2_wgrad(esm_encoder* e, const void* dy8, const float* dy_scale, const void* x8,
                                 const float* x_scale, void* dw, int64_t M, int32_t N, int32_t K, void* ws,
                                 size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !dy8 || !dy_scale || !x8 || !x_scale || !dw || !ws) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64)
    return fail(ESM_ERR_SHAPE, "M %lld N %d K %d: N and K must be positive multiples of 64", (long long)M, N, K);
  if (!aligned16(dy8) || !aligned16(x8) || !aligned16(dw) || ((uintptr_t)dy_scale & 3u) || ((uintptr_t)x_scale & 3u) ||
      ((uintptr_t)ws & 255u))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer (tensors 16 bytes, scales 4, workspace 256)");
  const E5WgradPlan pl = e5_wgrad_plan(M, N, K);
  if (ws_bytes < pl.total) return fail(ESM_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, pl.total);
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  uint8_t* dyt = (uint8_t*)ws + pl.dyt;
  uint8_t* xt = (uint8_t*)ws + pl.xt;
  float* wpart = (float*)((char*)ws + pl.wpart);
  return timed(e, ESM_K_LINEAR_BWD, st, "e5m2 wgrad", [&]() -> hipError_t {
    // dW [N, K] = (dy^T [N, Mp]) . (x^T [K, Mp])^T over the zero-padded rows
    hipError_t r = launch_transpose8_pad((const uint8_t*)dy8, M, N, dyt, pl.Mp, st);
    if (!r) r = launch_transpose8_pad((const uint8_t*)x8, M, K, xt, pl.Mp, st);
    if (r) return r;
    GemmArgs g{};
    g.dtype = kE5M2X;
    g.x = dyt; g.w = xt; g.x_scale = dy_scale; g.w_scale = x_scale;
    g.y = (bf16_t*)dw; g.M = N; g.N = K; g.K = pl.Mp;
    if (pl.splits > 1) {
      g.y32 = wpart; g.ksplit = pl.splits;
      r = launch_gemm(EPI_F32_SPLIT, g, st);
      if (!r) r = launch_split_reduce(wpart, pl.splits, (int64_t)N * K, (bf16_t*)dw, st, dy_scale, x_scale);
      return r;
    }
    return launch_gemm(EPI_BIAS, g, st);
  });
}

esm_status esm_gelu_bwd(esm_encoder* e, const void* z, const void* dy, void* dz, int64_t n, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !z || !dy || !dz) return fail(ESM_ERR_NULL, "NULL argument");
  if (n < 0 || n % 8) return fail(ESM_ERR_SHAPE, "n %lld: a non-negative multiple of 8", (long long)n);
  if (!aligned16(z) || !aligned16(dy) || !aligned16(dz)) return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (n == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  return timed(e, ESM_K_LINEAR_BWD, st, "gelu backward", [&] {
    return launch_gelu_bwd((const bf16_t*)z, (const bf16_t*)dy, (bf16_t*)dz, n, st);
  });
}

esm_status esm_qkv_rope_bwd(esm_encoder* e, const void* dqkv, void* dy, const int32_t* cu_dev, int32_t B, int64_t T,
                            void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !dqkv || !dy || !cu_dev) return fail(ESM_ERR_NULL, "NULL argument");
  if (!aligned16(dqkv) || !aligned16(dy)) return fail(ESM_ERR_UNSUPPORTED, "dqkv/dy not 16-byte aligned");
  esm_status s = check_rows(e, T, B);
  if (s) return s;
  if (T == 0 || B == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = run_segments(e, 0, cu_dev, B, T, 0, ws, p, st))) return s;
  const int32_t* pos = region<int32_t>(ws, p, ESM_WS_POS);
  return timed(e, ESM_K_LINEAR_BWD, st, "qkv rope backward", [&] {
    return launch_qkv_rope_bwd((const bf16_t*)dqkv, pos, e->rope, e->cfg.max_position_embeddings, T,
                               e->cfg.num_attention_heads, (bf16_t*)dy, st);
  });
}

// ---------------------------------------------------------------- training layer

namespace {

// Saved activations of one layer: the regions of esm_saved_region in order,
// each 256-byte aligned.
struct SavedPlan {
  size_t off[ESM_SAVED_COUNT], size[ESM_SAVED_COUNT], total;
};
SavedPlan saved_plan(const esm_config& c, int64_t T) {
  const size_t t = (size_t)(T > 0 ? T : 0), H = (size_t)c.hidden_size, F = (size_t)c.intermediate_size;
  const size_t nh = (size_t)c.num_attention_heads;
  const size_t sz[ESM_SAVED_COUNT] = {t * H * 2, 3 * t * H * 2, t * H * 2, nh * t * 4,
                                      t * H * 2, t * H * 2, t * F * 2, t * F * 2};
  SavedPlan p;
  size_t o = 0;
  for (int i = 0; i < ESM_SAVED_COUNT; ++i) {
    p.off[i] = o;
    p.size[i] = sz[i];
    o += align256(sz[i]);
  }
  p.total = o;
  return p;
}

// Backward workspace: the forward plan (segment table and positions; its
// activation regions hold the gradients of the same shapes), then delta
// [heads, T] fp32, dA [T, F] bf16 (later the QKV output gradient [T, 3H]; sized
// for the larger), and the linear and LayerNorm backward workspaces.
struct BwdPlan {
  Plan fwd;
  size_t delta, da, lin, lin_bytes, ln, ln_bytes, total;
};
BwdPlan bwd_plan(const esm_config& c, int64_t T, int32_t B) {
  BwdPlan b;
  b.fwd = make_plan(c, T, B);
  const int64_t t = T > 0 ? T : 0;
  const int32_t H = c.hidden_size, F = c.intermediate_size;
  size_t o = b.fwd.total;
  b.delta = o;
  o += align256((size_t)c.num_attention_heads * (size_t)t * 4);
  b.da = o;
  o += align256((size_t)t * (size_t)(F > 3 * H ? F : 3 * H) * 2);
  b.lin = o;
  b.lin_bytes = lin_bwd_plan(t, 3 * H, H).total;
  const size_t others[3] = {lin_bwd_plan(t, H, H).total, lin_bwd_plan(t, F, H).total, lin_bwd_plan(t, H, F).total};
  for (size_t v : others) b.lin_bytes = v > b.lin_bytes ? v : b.lin_bytes;
  o += align256(b.lin_bytes);
  b.ln = o;
  b.ln_bytes = ln_bwd_ws_bytes(t, H);
  o += align256(b.ln_bytes);
  b.total = o;
  return b;
}

esm_status check_train_call(const esm_encoder* e, const esm_layer_weights* w, int32_t layer_idx, int64_t T,
                            int32_t B) {
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (is_quantised(e)) return fail(ESM_ERR_UNSUPPORTED, "the training layer entries run bf16 encoders");
  esm_status s = check_rows(e, T, B);
  if (s) return s;
  if (layer_idx < 0 || layer_idx >= e->cfg.num_hidden_layers)
    return fail(ESM_ERR_SHAPE, "layer_idx %d outside [0, %d)", layer_idx, e->cfg.num_hidden_layers);
  return check_weights(w, layer_idx);
}

}  // namespace

esm_status esm_layer_saved_size(const esm_encoder* e, int64_t T, size_t* bytes) {
  g_last_error.clear();
  if (!e || !bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (T < 0) return fail(ESM_ERR_SHAPE, "T < 0");
  *bytes = saved_plan(e->cfg, T).total;
  return ok();
}

esm_status esm_layer_saved_region(const esm_encoder* e, int64_t T, int32_t r, size_t* offset, size_t* bytes) {
  g_last_error.clear();
  if (!e || !offset || !bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (T < 0) return fail(ESM_ERR_SHAPE, "T < 0");
  if (r < 0 || r >= ESM_SAVED_COUNT) return fail(ESM_ERR_SHAPE, "saved region %d outside [0, %d)", r, ESM_SAVED_COUNT);
  const SavedPlan sp = saved_plan(e->cfg, T);
  *offset = sp.off[r];
  *bytes = sp.size[r];
  return ok();
}

esm_status esm_layer_bwd_workspace_size(const esm_encoder* e, int64_t T, int32_t B, size_t* bytes) {
  g_last_error.clear();
  if (!e || !bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (T < 0 || B < 0) return fail(ESM_ERR_SHAPE, "negative T or B");
  *bytes = bwd_plan(e->cfg, T, B).total;
  return ok();
}

esm_status esm_layer_fwd_train(esm_encoder* e, const esm_layer_weights* w, int32_t layer_idx, const void* x_in,
                               void* x_out, const int32_t* cu_dev, const int32_t* cu_host, int32_t B, int64_t T,
                               int32_t max_seqlen, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                               esm_stream_t stream) {
  g_last_error.clear();
  esm_status s = check_train_call(e, w, layer_idx, T, B);
  if (s) return s;
  if (!x_in || !x_out || !cu_dev) return fail(ESM_ERR_NULL, "x_in, x_out or cu_seqlens_dev is NULL");
  if (!aligned16(x_in) || !aligned16(x_out)) return fail(ESM_ERR_UNSUPPORTED, "x_in/x_out not 16-byte aligned");
  if ((s = check_cu_host(e, cu_host, B, T, max_seqlen))) return s;
  const SavedPlan sp = saved_plan(e->cfg, T);
  if (!saved || ((uintptr_t)saved & 255u) || saved_bytes < sp.total)
    return fail(ESM_ERR_WORKSPACE, "saved activations: NULL, not 256-byte aligned or %zu bytes < %zu", saved_bytes,
                sp.total);
  if (T == 0 || B == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = run_segments(e, 0, cu_dev, B, T, 0, ws, p, st))) return s;
  const esm_config& c = e->cfg;
  const int H = c.hidden_size, F = c.intermediate_size;
  char* sv = (char*)saved;
  bf16_t* h1 = (bf16_t*)(sv + sp.off[ESM_SAVED_H1]);
  bf16_t* qkv = (bf16_t*)(sv + sp.off[ESM_SAVED_QKV]);
  bf16_t* ctx = (bf16_t*)(sv + sp.off[ESM_SAVED_CTX]);
  float* lse = (float*)(sv + sp.off[ESM_SAVED_LSE]);
  bf16_t* x1 = (bf16_t*)(sv + sp.off[ESM_SAVED_X1]);
  bf16_t* h2 = (bf16_t*)(sv + sp.off[ESM_SAVED_H2]);
  bf16_t* z = (bf16_t*)(sv + sp.off[ESM_SAVED_Z]);
  bf16_t* a = (bf16_t*)(sv + sp.off[ESM_SAVED_A]);
  const E4m3Out none{nullptr, nullptr, nullptr, nullptr};

  s = timed(e, ESM_K_LAYERNORM, st, "layernorm 1", [&] {
    return launch_layernorm((const bf16_t*)x_in, (const bf16_t*)w->ln1_gamma, (const bf16_t*)w->ln1_beta, h1, T, H,
                            c.layer_norm_eps, none, st);
  });
  if (s) return s;
  GemmArgs g{};
  g.dtype = kBF16;
  g.M = T;
  g.pos = region<int32_t>(ws, p, ESM_WS_POS);
  g.rope = e->rope;
  g.max_positions = c.max_position_embeddings;
  g.x = h1; g.w = w->w_qkv; g.bias = (const bf16_t*)w->b_qkv; g.y = qkv;
  g.N = 3 * H; g.K = H;
  s = timed(e, ESM_K_GEMM_QKV, st, "qkv gemm", [&] { return launch_gemm(EPI_QKV_ROPE, g, st); });
  if (s) return s;
  AttnArgs aa{};
  aa.qkv = qkv; aa.ctx = ctx; aa.lse = lse;
  aa.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  aa.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  aa.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  aa.tile_cap = tile_cap(T, B);
  aa.T = T; aa.heads = c.num_attention_heads;
  s = timed(e, ESM_K_ATTENTION, st, "attention", [&] { return launch_attention(aa, st); });
  if (s) return s;
  g.x = ctx; g.w = w->w_out; g.bias = (const bf16_t*)w->b_out; g.res = (const bf16_t*)x_in; g.y = x1;
  g.N = H; g.K = H;
  s = timed(e, ESM_K_GEMM_OUT, st, "out-proj gemm", [&] { return launch_gemm(EPI_BIAS_RESIDUAL, g, st); });
  if (s) return s;
  s = timed(e, ESM_K_LAYERNORM, st, "layernorm 2", [&] {
    return launch_layernorm(x1, (const bf16_t*)w->ln2_gamma, (const bf16_t*)w->ln2_beta, h2, T, H, c.layer_norm_eps,
                            none, st);
  });
  if (s) return s;
  g.x = h2; g.w = w->w_fc1; g.bias = (const bf16_t*)w->b_fc1; g.res = nullptr; g.y = z;
  g.N = F; g.K = H;
  s = timed(e, ESM_K_GEMM_FC1, st, "fc1 gemm", [&] { return launch_gemm(EPI_BIAS, g, st); });
  if (s) return s;
  s = timed(e, ESM_K_OTHER, st, "gelu", [&] { return launch_gelu_fwd(z, a, T * F, st); });
  if (s) return s;
  g.x = a; g.w = w->w_fc2; g.bias = (const bf16_t*)w->b_fc2; g.res = x1; g.y = (bf16_t*)x_out;
  g.N = H; g.K = F;
  return timed(e, ESM_K_GEMM_FC2, st, "fc2 gemm", [&] { return launch_gemm(EPI_BIAS_RESIDUAL, g, st); });
}

esm_status esm_layer_bwd(esm_encoder* e, const esm_layer_weights* w, int32_t layer_idx, const void* x_in,
                         const void* saved, size_t saved_bytes, const void* dy, void* dx, const esm_layer_grads* gr,
                         const int32_t* cu_dev, int32_t B, int64_t T, void* ws, size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  esm_status s = check_train_call(e, w, layer_idx, T, B);
  if (s) return s;
  if (!x_in || !dy || !dx || !gr || !cu_dev) return fail(ESM_ERR_NULL, "x_in, dy, dx, grads or cu_seqlens_dev is NULL");
  void* const gw[4] = {gr->w_qkv, gr->w_out, gr->w_fc1, gr->w_fc2};
  float* const gv[8] = {gr->ln1_gamma, gr->ln1_beta, gr->b_qkv, gr->b_out, gr->ln2_gamma, gr->ln2_beta, gr->b_fc1,
                        gr->b_fc2};
  for (void* q : gw)
    if (!q) return fail(ESM_ERR_NULL, "a weight gradient pointer is NULL");
  for (float* q : gv)
    if (!q) return fail(ESM_ERR_NULL, "a bias or LayerNorm gradient pointer is NULL");
  if (!aligned16(x_in) || !aligned16(dy) || !aligned16(dx)) return fail(ESM_ERR_UNSUPPORTED, "x_in/dy/dx not 16-byte aligned");
  for (void* q : gw)
    if (!aligned16(q)) return fail(ESM_ERR_UNSUPPORTED, "weight gradient not 16-byte aligned");
  for (float* q : gv)
    if ((uintptr_t)q & 3u) return fail(ESM_ERR_UNSUPPORTED, "bias/LayerNorm gradient not 4-byte aligned");
  const SavedPlan sp = saved_plan(e->cfg, T);
  if (!saved || ((uintptr_t)saved & 255u) || saved_bytes < sp.total)
    return fail(ESM_ERR_WORKSPACE, "saved activations: NULL, not 256-byte aligned or %zu bytes < %zu", saved_bytes,
                sp.total);
  const BwdPlan bp = bwd_plan(e->cfg, T, B);
  if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < bp.total)
    return fail(ESM_ERR_WORKSPACE, "workspace: NULL, not 256-byte aligned or %zu bytes < %zu", ws_bytes, bp.total);
  if (T == 0 || B == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = run_segments(e, 0, cu_dev, B, T, 0, ws, bp.fwd, st))) return s;
  const esm_config& c = e->cfg;
  const int32_t H = c.hidden_size, F = c.intermediate_size;
  const char* sv = (const char*)saved;
  auto saved_at = [&](int r) { return (const void*)(sv + sp.off[r]); };
  char* wb = (char*)ws;
  const Plan& p = bp.fwd;
  bf16_t* dz = region<bf16_t>(ws, p, ESM_WS_ACT);      // [T, F]
  bf16_t* dh2 = region<bf16_t>(ws, p, ESM_WS_LN2);     // [T, H]
  bf16_t* dx1 = region<bf16_t>(ws, p, ESM_WS_X1);      // [T, H]
  bf16_t* dctx = region<bf16_t>(ws, p, ESM_WS_CTX);    // [T, H]
  bf16_t* dqkv = region<bf16_t>(ws, p, ESM_WS_QKV);    // [3, heads, T, 64]
  bf16_t* dh1 = region<bf16_t>(ws, p, ESM_WS_LN1);     // [T, H]
  float* delta = (float*)(wb + bp.delta);
  bf16_t* da = (bf16_t*)(wb + bp.da);                  // [T, F], then the QKV output gradient [T, 3H]
  void* lin = wb + bp.lin;
  float* ln_stats = (float*)(wb + bp.ln);
  float* ln_part = (float*)(wb + bp.ln + ln_bwd_stats_bytes(T));

  // fc2: dA = dy W_fc2, dW_fc2 = dy^T A, db_fc2
  if ((s = esm_linear_bwd(e, saved_at(ESM_SAVED_A), w->w_fc2, dy, da, gr->w_fc2, gr->b_fc2, T, H, F, lin, bp.lin_bytes,
                          stream)))
    return s;
  if ((s = esm_gelu_bwd(e, saved_at(ESM_SAVED_Z), da, dz, T * F, stream))) return s;
  if ((s = esm_linear_bwd(e, saved_at(ESM_SAVED_H2), w->w_fc1, dz, dh2, gr->w_fc1, gr->b_fc1, T, F, H, lin,
                          bp.lin_bytes, stream)))
    return s;
  // LN2, and dy through the residual: dX1 = dy + LN2'(dh2)
  s = timed(e, ESM_K_LINEAR_BWD, st, "layernorm backward", [&] {
    return launch_layernorm_bwd((const bf16_t*)saved_at(ESM_SAVED_X1), (const bf16_t*)w->ln2_gamma, dh2,
                                (const bf16_t*)dy, dx1, gr->ln2_gamma, gr->ln2_beta, T, H, c.layer_norm_eps, ln_stats,
                                ln_part, st);
  });
  if (s) return s;
  if ((s = esm_linear_bwd(e, saved_at(ESM_SAVED_CTX), w->w_out, dx1, dctx, gr->w_out, gr->b_out, T, H, H, lin,
                          bp.lin_bytes, stream)))
    return s;
  AttnBwdArgs ab{};
  ab.qkv = (const bf16_t*)saved_at(ESM_SAVED_QKV); ab.out = (const bf16_t*)saved_at(ESM_SAVED_CTX);
  ab.dout = dctx; ab.lse = (const float*)saved_at(ESM_SAVED_LSE); ab.delta = delta; ab.dqkv = dqkv;
  ab.segs = region<int32_t>(ws, p, ESM_WS_SEGS);
  ab.tiles = region<int32_t>(ws, p, ESM_WS_TILES);
  ab.ntiles = region<int32_t>(ws, p, ESM_WS_NTILES);
  ab.tile_cap = tile_cap(T, B);
  ab.T = T; ab.heads = c.num_attention_heads;
  if ((s = timed(e, ESM_K_ATTENTION_BWD, st, "attention_bwd", [&] { return launch_attention_bwd(ab, st); }))) return s;
  bf16_t* dyq = da;   // dA is dead: the QKV linear's output gradient [T, 3H]
  s = timed(e, ESM_K_LINEAR_BWD, st, "qkv rope backward", [&] {
    return launch_qkv_rope_bwd(dqkv, region<int32_t>(ws, p, ESM_WS_POS), e->rope, c.max_position_embeddings, T,
                               c.num_attention_heads, dyq, st);
  });
  if (s) return s;
  if ((s = esm_linear_bwd(e, saved_at(ESM_SAVED_H1), w->w_qkv, dyq, dh1, gr->w_qkv, gr->b_qkv, T, 3 * H, H, lin,
                          bp.lin_bytes, stream)))
    return s;
  // LN1, and dX1 through the residual: dx = dX1 + LN1'(dh1)
  return timed(e, ESM_K_LINEAR_BWD, st, "layernorm backward", [&] {
    return launch_layernorm_bwd((const bf16_t*)x_in, (const bf16_t*)w->ln1_gamma, dh1, dx1, (bf16_t*)dx, gr->ln1_gamma,
                                gr->ln1_beta, T, H, c.layer_norm_eps, ln_stats, ln_part, st);
  });
}

namespace {

// A stack's training activations: per layer, its input X_l (bf16 [T, H]) then
// the layer's saved activations, each 256-byte aligned.
struct StackSavedPlan {
  SavedPlan sp;
  size_t x_size, stride, total;
};
StackSavedPlan stack_saved_plan(const esm_config& c, int64_t T) {
  StackSavedPlan q;
  q.sp = saved_plan(c, T);
  q.x_size = align256((size_t)(T > 0 ? T : 0) * (size_t)c.hidden_size * 2);
  q.stride = q.x_size + q.sp.total;
  q.total = q.stride * (size_t)c.num_hidden_layers;
  return q;
}

// Stack backward workspace: the gradient passed between layers (bf16 [T, H]),
// then the layer backward's workspace, which the embedding gradient's chunk
// sums reuse once the layers are done.
struct StackBwdPlan {
  BwdPlan bp;
  size_t layer, total;
};
StackBwdPlan stack_bwd_plan(const esm_config& c, int64_t T, int32_t B) {
  StackBwdPlan q;
  q.bp = bwd_plan(c, T, B);
  const size_t t = (size_t)(T > 0 ? T : 0);
  q.layer = align256(t * (size_t)c.hidden_size * 2);
  const size_t emb = (size_t)colsum_chunks((int64_t)t) * (size_t)c.vocab_size * (size_t)c.hidden_size * 4;
  q.total = q.layer + align256(q.bp.total > emb ? q.bp.total : emb);
  return q;
}

}  // namespace

esm_status esm_stack_saved_size(const esm_encoder* e, int64_t T, size_t* bytes) {
  g_last_error.clear();
  if (!e || !bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (T < 0) return fail(ESM_ERR_SHAPE, "T < 0");
  *bytes = stack_saved_plan(e->cfg, T).total;
  return ok();
}

esm_status esm_stack_saved_layer(const esm_encoder* e, int64_t T, int32_t l, size_t* x_offset, size_t* saved_offset) {
  g_last_error.clear();
  if (!e || !x_offset || !saved_offset) return fail(ESM_ERR_NULL, "NULL argument");
  if (T < 0) return fail(ESM_ERR_SHAPE, "T < 0");
  if (l < 0 || l >= e->cfg.num_hidden_layers)
    return fail(ESM_ERR_SHAPE, "layer %d outside [0, %d)", l, e->cfg.num_hidden_layers);
  const StackSavedPlan q = stack_saved_plan(e->cfg, T);
  *x_offset = q.stride * (size_t)l;
  *saved_offset = *x_offset + q.x_size;
  return ok();
}

esm_status esm_stack_bwd_workspace_size(const esm_encoder* e, int64_t T, int32_t B, size_t* bytes) {
  g_last_error.clear();
  if (!e || !bytes) return fail(ESM_ERR_NULL, "NULL argument");
  if (T < 0 || B < 0) return fail(ESM_ERR_SHAPE, "negative T or B");
  *bytes = stack_bwd_plan(e->cfg, T, B).total;
  return ok();
}

esm_status esm_stack_fwd_train(esm_encoder* e, const esm_layer_weights* w, const int32_t* ids, const void* emb,
                               const void* x_in, void* x_out, const int32_t* cu_dev, const int32_t* cu_host, int32_t B,
                               int64_t T, int32_t max_seqlen, void* saved, size_t saved_bytes, void* ws,
                               size_t ws_bytes, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (!w) return fail(ESM_ERR_NULL, "weights are NULL");
  const int L = e->cfg.num_hidden_layers, H = e->cfg.hidden_size;
  esm_status s;
  for (int l = 0; l < L; ++l)
    if ((s = check_train_call(e, &w[l], l, T, B))) return s;
  if (!x_out || !cu_dev) return fail(ESM_ERR_NULL, "x_out or cu_seqlens_dev is NULL");
  if (!aligned16(x_out)) return fail(ESM_ERR_UNSUPPORTED, "x_out not 16-byte aligned");
  if (ids) {
    if (!emb) return fail(ESM_ERR_NULL, "token_ids given without an embedding table");
    if (!aligned16(emb)) return fail(ESM_ERR_UNSUPPORTED, "embedding not 16-byte aligned");
  } else {
    if (!x_in) return fail(ESM_ERR_NULL, "x_in is NULL (and no token ids)");
    if (!aligned16(x_in)) return fail(ESM_ERR_UNSUPPORTED, "x_in not 16-byte aligned");
  }
  if ((s = check_cu_host(e, cu_host, B, T, max_seqlen))) return s;
  const StackSavedPlan q = stack_saved_plan(e->cfg, T);
  if (!saved || ((uintptr_t)saved & 255u) || saved_bytes < q.total)
    return fail(ESM_ERR_WORKSPACE, "saved activations: NULL, not 256-byte aligned or %zu bytes < %zu", saved_bytes,
                q.total);
  if (T == 0 || B == 0) return ok();
  Plan p;
  if ((s = check_ws(e, ws, ws_bytes, T, B, &p))) return s;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  char* sv = (char*)saved;
  if (ids) {
    s = timed(e, ESM_K_EMBED, st, "embedding", [&] {
      return launch_embed(ids, (const bf16_t*)emb, e->cfg.vocab_size, (bf16_t*)sv, T, H, st);
    });
    if (s) return s;
  } else {
    HIP_TRY(hipMemcpyAsync(sv, x_in, (size_t)T * H * 2, hipMemcpyDeviceToDevice, st), "hipMemcpyAsync");
  }
  for (int l = 0; l < L; ++l) {
    void* out = l + 1 < L ? (void*)(sv + q.stride * (l + 1)) : x_out;
    if ((s = esm_layer_fwd_train(e, &w[l], l, sv + q.stride * l, out, cu_dev, cu_host, B, T, max_seqlen,
                                 sv + q.stride * l + q.x_size, q.sp.total, ws, ws_bytes, stream)))
      return s;
  }
  return ok();
}

esm_status esm_stack_bwd(esm_encoder* e, const esm_layer_weights* w, const void* saved, size_t saved_bytes,
                         const void* dy, void* dx, const esm_layer_grads* g, const int32_t* ids, float* d_emb,
                         const int32_t* cu_dev, int32_t B, int64_t T, void* ws, size_t ws_bytes,
                         esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (!w || !g) return fail(ESM_ERR_NULL, "weights or gradients are NULL");
  const int L = e->cfg.num_hidden_layers, H = e->cfg.hidden_size, V = e->cfg.vocab_size;
  esm_status s;
  for (int l = 0; l < L; ++l)
    if ((s = check_train_call(e, &w[l], l, T, B))) return s;
  if (!dy || !dx || !cu_dev) return fail(ESM_ERR_NULL, "dy, dx or cu_seqlens_dev is NULL");
  if (!aligned16(dy) || !aligned16(dx)) return fail(ESM_ERR_UNSUPPORTED, "dy/dx not 16-byte aligned");
  if ((ids == nullptr) != (d_emb == nullptr))
    return fail(ESM_ERR_NULL, "token_ids and d_embedding go together (one of them is NULL)");
  if (ids) {
    if (V > kEmbedBwdMaxVocab)
      return fail(ESM_ERR_UNSUPPORTED, "the embedding gradient takes vocab <= %d (vocab %d)", kEmbedBwdMaxVocab, V);
    if ((uintptr_t)d_emb & 3u) return fail(ESM_ERR_UNSUPPORTED, "d_embedding not 4-byte aligned");
  }
  const StackSavedPlan q = stack_saved_plan(e->cfg, T);
  if (!saved || ((uintptr_t)saved & 255u) || saved_bytes < q.total)
    return fail(ESM_ERR_WORKSPACE, "saved activations: NULL, not 256-byte aligned or %zu bytes < %zu", saved_bytes,
                q.total);
  const StackBwdPlan bq = stack_bwd_plan(e->cfg, T, B);
  if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < bq.total)
    return fail(ESM_ERR_WORKSPACE, "workspace: NULL, not 256-byte aligned or %zu bytes < %zu", ws_bytes, bq.total);
  if (T == 0 || B == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  const char* sv = (const char*)saved;
  char* gbuf = (char*)ws;   // the gradient between layers; each middle layer updates it in place
  char* lws = (char*)ws + bq.layer;
  const size_t lws_bytes = ws_bytes - bq.layer;
  const void* cur = dy;
  for (int l = L - 1; l >= 0; --l) {
    void* out = l == 0 ? dx : (void*)gbuf;
    if ((s = esm_layer_bwd(e, &w[l], l, sv + q.stride * l, sv + q.stride * l + q.x_size, q.sp.total, cur, out, &g[l],
                           cu_dev, B, T, lws, lws_bytes, stream)))
      return s;
    cur = out;
  }
  if (!ids) return ok();
  return timed(e, ESM_K_LINEAR_BWD, st, "embedding backward", [&] {
    return launch_embed_bwd(ids, (const bf16_t*)dx, T, H, V, (float*)lws, d_emb, st);
  });
}

esm_status esm_layernorm_fwd(esm_encoder* e, const void* x, const void* gamma, const void* beta, void* y, int64_t M,
                             esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !x || !gamma || !beta || !y) return fail(ESM_ERR_NULL, "NULL argument");
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(beta) || !aligned16(y))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (M < 0) return fail(ESM_ERR_SHAPE, "M < 0");
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  return timed(e, ESM_K_LAYERNORM, (hipStream_t)stream, "layernorm", [&] {
    return launch_layernorm((const bf16_t*)x, (const bf16_t*)gamma, (const bf16_t*)beta, (bf16_t*)y, M,
                            e->cfg.hidden_size, e->cfg.layer_norm_eps, E4m3Out{nullptr, nullptr, nullptr, nullptr},
                            (hipStream_t)stream);
  });
}

esm_status esm_layernorm_e4m3_fwd(esm_encoder* e, const void* x, const void* gamma, const void* beta,
                                  const float* scale, void* y8, uint32_t* amax, int64_t M, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !x || !gamma || !beta || !scale || !y8 || !amax) return fail(ESM_ERR_NULL, "NULL argument");
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(beta) || ((uintptr_t)y8 & 7u))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (M < 0) return fail(ESM_ERR_SHAPE, "M < 0");
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  return timed(e, ESM_K_LAYERNORM, (hipStream_t)stream, "layernorm e4m3", [&] {
    return launch_layernorm((const bf16_t*)x, (const bf16_t*)gamma, (const bf16_t*)beta, nullptr, M,
                            e->cfg.hidden_size, e->cfg.layer_norm_eps, E4m3Out{(uint8_t*)y8, scale, amax, nullptr},
                            (hipStream_t)stream);
  });
}

esm_status esm_linear_e4m3_fwd(esm_encoder* e, const void* x8, const float* x_scale, const void* w8,
                               const float* w_scale, const void* b, const void* res, void* y, const float* y_scale,
                               uint32_t* y_amax, int64_t M, int32_t N, int32_t K, int32_t epi, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !x8 || !w8 || !y || !x_scale || !w_scale) return fail(ESM_ERR_NULL, "NULL argument");
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 128)
    return fail(ESM_ERR_SHAPE, "M %lld N %d K %d: N must be a positive multiple of 64, K of 128", (long long)M, N, K);
  if (epi < ESM_EPI_BIAS || epi > ESM_EPI_BIAS_GELU_E4M3) return fail(ESM_ERR_UNSUPPORTED, "epilogue %d", epi);
  if (epi == ESM_EPI_BIAS_RESIDUAL && !res) return fail(ESM_ERR_NULL, "residual is NULL");
  if (epi == ESM_EPI_BIAS_GELU_E4M3 && (!y_scale || !y_amax)) return fail(ESM_ERR_NULL, "output scale or amax NULL");
  if (!aligned16(x8) || !aligned16(w8) || !aligned16(y) || (res && !aligned16(res)) || (b && ((uintptr_t)b & 7u)))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (M == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  GemmArgs g{};
  g.dtype = kE4M3;
  g.x = x8; g.w = w8; g.x_scale = x_scale; g.w_scale = w_scale;
  g.bias = (const bf16_t*)b; g.res = (const bf16_t*)res;
  g.M = M; g.N = N; g.K = K;
  int kind = EPI_BIAS;
  if (epi == ESM_EPI_BIAS_GELU) kind = EPI_BIAS_GELU;
  if (epi == ESM_EPI_BIAS_RESIDUAL) kind = EPI_BIAS_RESIDUAL;
  if (epi == ESM_EPI_BIAS_GELU_E4M3) {
    kind = EPI_BIAS_GELU_E4M3;
    g.y8 = (uint8_t*)y; g.y8_scale = y_scale; g.y8_amax = y_amax;
  } else {
    g.y = (bf16_t*)y;
  }
  return timed(e, ESM_K_OTHER, (hipStream_t)stream, "linear e4m3", [&] { return launch_gemm(kind, g, (hipStream_t)stream); });
}

esm_status esm_fp8_prepare_layer(esm_encoder* e, int32_t layer_idx, const esm_layer_weights* w, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (!is_quantised(e)) return fail(ESM_ERR_STATE, "encoder was created with bf16 precision");
  if (layer_idx < 0 || layer_idx >= e->cfg.num_hidden_layers)
    return fail(ESM_ERR_SHAPE, "layer_idx %d outside [0, %d)", layer_idx, e->cfg.num_hidden_layers);
  esm_status s = check_weights(w, layer_idx);
  if (s) return s;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = ensure_fp8(e))) return s;
  hipStream_t st = (hipStream_t)stream;
  const esm_config& c = e->cfg;
  const int64_t H = c.hidden_size, F = c.intermediate_size;
  const W8Off wo = w8_offsets(c);
  uint8_t* w8 = e->w8 + (size_t)layer_idx * e->w8_layer;
  uint32_t* wam = e->f8.w_amax + 4 * layer_idx;
  float* wsc = e->f8.w_scale + 4 * layer_idx;
  const bf16_t* src[4] = {(const bf16_t*)w->w_qkv, (const bf16_t*)w->w_out, (const bf16_t*)w->w_fc1,
                          (const bf16_t*)w->w_fc2};
  const int64_t n[4] = {3 * H * H, H * H, F * H, H * F};
  const size_t off[4] = {wo.qkv, wo.out, wo.fc1, wo.fc2};
  HIP_TRY(hipMemsetAsync(wam, 0, 4 * sizeof(uint32_t), st), "hipMemsetAsync");
  for (int i = 0; i < 4; ++i) {
    s = timed(e, ESM_K_FP8, st, "weight amax", [&] { return launch_amax_bf16(src[i], n[i], wam + i, st); });
    if (s) return s;
    s = timed(e, ESM_K_FP8, st, "weight cast",
              [&] { return launch_quantize_weight(src[i], n[i], wam + i, w8 + off[i], wsc + i, st); });
    if (s) return s;
  }
  e->prepared8[(size_t)layer_idx] = 1;
  return ok();
}

esm_status esm_prepare_layer(esm_encoder* e, int32_t layer_idx, const esm_layer_weights* w, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (e->cfg.precision != ESM_PRECISION_BF16)
    return fail(ESM_ERR_STATE, "esm_prepare_layer is for bf16 encoders (FP8: esm_fp8_prepare_layer, MXFP4: "
                               "esm_mxfp4_prepare_layer)");
  if (layer_idx < 0 || layer_idx >= e->cfg.num_hidden_layers)
    return fail(ESM_ERR_SHAPE, "layer_idx %d outside [0, %d)", layer_idx, e->cfg.num_hidden_layers);
  esm_status s = check_weights(w, layer_idx);
  if (s) return s;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  const esm_config& c = e->cfg;
  const FoldOff fo = fold_offsets(c);
  if (!e->fold) {
    const size_t L = (size_t)c.num_hidden_layers;
    e->fold_layer = align256(fo.total);
    HIP_TRY(hipMalloc((void**)&e->fold, L * e->fold_layer), "folded LayerNorm weights");
    e->folded.assign(L, 0);
  }
  hipStream_t st = (hipStream_t)stream;
  unsigned char* fl = e->fold + (size_t)layer_idx * e->fold_layer;
  const int H = c.hidden_size, F = c.intermediate_size;
  s = timed(e, ESM_K_OTHER, st, "fold qkv", [&] {
    return launch_fold_weight((const bf16_t*)w->w_qkv, (const bf16_t*)w->ln1_gamma, (const bf16_t*)w->ln1_beta,
                              (const bf16_t*)w->b_qkv, 3 * H, H, (bf16_t*)(fl + fo.wqkv), (float2*)(fl + fo.cdqkv), st);
  });
  if (s) return s;
  s = timed(e, ESM_K_OTHER, st, "fold fc1", [&] {
    return launch_fold_weight((const bf16_t*)w->w_fc1, (const bf16_t*)w->ln2_gamma, (const bf16_t*)w->ln2_beta,
                              (const bf16_t*)w->b_fc1, F, H, (bf16_t*)(fl + fo.wfc1), (float2*)(fl + fo.cdfc1), st);
  });
  if (s) return s;
  e->folded[(size_t)layer_idx] = 1;
  return ok();
}

esm_status esm_mxfp4_prepare_layer(esm_encoder* e, int32_t layer_idx, const esm_layer_weights* w,
                                   esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (!is_quantised(e)) return fail(ESM_ERR_STATE, "encoder was created with bf16 precision");
  if (layer_idx < 0 || layer_idx >= e->cfg.num_hidden_layers)
    return fail(ESM_ERR_SHAPE, "layer_idx %d outside [0, %d)", layer_idx, e->cfg.num_hidden_layers);
  esm_status s = check_weights(w, layer_idx);
  if (s) return s;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  if ((s = ensure_mx(e))) return s;
  hipStream_t st = (hipStream_t)stream;
  const esm_config& c = e->cfg;
  const int64_t H = c.hidden_size, F = c.intermediate_size;
  const W4Off wo = w4_offsets(c);
  uint8_t* w4 = e->w4 + (size_t)layer_idx * e->w4_layer;
  const bf16_t* src[4] = {(const bf16_t*)w->w_qkv, (const bf16_t*)w->w_out, (const bf16_t*)w->w_fc1,
                          (const bf16_t*)w->w_fc2};
  const int64_t n[4] = {3 * H, H, F, H}, k[4] = {H, H, H, F};
  for (int i = 0; i < 4; ++i) {
    const MxOff o = mx_operand((size_t)n[i], (size_t)k[i]);
    s = timed(e, ESM_K_OTHER, st, "mxfp4 weight", [&] {
      return launch_mx_quantize(src[i], n[i], (int32_t)k[i], w4 + wo.at[i] + o.codes, w4 + wo.at[i] + o.scales, st);
    });
    if (s) return s;
  }
  e->prepared4[(size_t)layer_idx] = 1;
  return ok();
}

static esm_status check_state_arg(const esm_encoder* e, const esm_fp8_state* st) {
  if (!e || !st) return fail(ESM_ERR_NULL, "encoder or state is NULL");
  if (!e->fp8_mem) return fail(ESM_ERR_STATE, "encoder has no FP8 state (bf16, or MXFP4 with no FP8 layer)");
  if (st->num_layers != e->cfg.num_hidden_layers || st->history_len != e->cfg.amax_history_len)
    return fail(ESM_ERR_SHAPE, "state is for %d layers x history %d; the encoder has %d x %d", st->num_layers,
                st->history_len, e->cfg.num_hidden_layers, e->cfg.amax_history_len);
  return ok();
}

esm_status esm_fp8_get_state(esm_encoder* e, esm_fp8_state* st, esm_stream_t stream) {
  g_last_error.clear();
  esm_status s = check_state_arg(e, st);
  if (s) return s;
  if (!st->act_scale || !st->amax_history || !st->steps || !st->weight_scale)
    return fail(ESM_ERR_NULL, "state arrays are NULL");
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  const size_t L = (size_t)st->num_layers, HL = (size_t)st->history_len;
  if (L > 0) {
    HIP_TRY(hipMemcpy(st->act_scale, e->f8.act_scale, L * 4 * sizeof(float), hipMemcpyDeviceToHost), "fp8 state");
    HIP_TRY(hipMemcpy(st->amax_history, e->f8.history, L * 4 * HL * sizeof(float), hipMemcpyDeviceToHost), "fp8 state");
    HIP_TRY(hipMemcpy(st->steps, e->f8.steps, L * sizeof(int64_t), hipMemcpyDeviceToHost), "fp8 state");
    HIP_TRY(hipMemcpy(st->weight_scale, e->f8.w_scale, L * 4 * sizeof(float), hipMemcpyDeviceToHost), "fp8 state");
  }
  uint32_t flags = 0;
  HIP_TRY(hipMemcpy(&flags, e->f8.flags, sizeof flags, hipMemcpyDeviceToHost), "fp8 state");
  st->nonfinite = flags & 1u;
  return ok();
}

esm_status esm_fp8_set_state(esm_encoder* e, const esm_fp8_state* st, esm_stream_t stream) {
  g_last_error.clear();
  esm_status s = check_state_arg(e, st);
  if (s) return s;
  if (!st->act_scale || !st->amax_history || !st->steps) return fail(ESM_ERR_NULL, "state arrays are NULL");
  const size_t L = (size_t)st->num_layers, HL = (size_t)st->history_len;
  for (size_t i = 0; i < L * 4; ++i)
    if (!(st->act_scale[i] > 0.f) || !isfinite(st->act_scale[i]))
      return fail(ESM_ERR_SHAPE, "act_scale[%zu] = %g is not positive and finite", i, (double)st->act_scale[i]);
  for (size_t i = 0; i < L; ++i)
    if (st->steps[i] < 0) return fail(ESM_ERR_SHAPE, "steps[%zu] < 0", i);
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  if (L > 0) {
    HIP_TRY(hipMemcpy(e->f8.act_scale, st->act_scale, L * 4 * sizeof(float), hipMemcpyHostToDevice), "fp8 state");
    HIP_TRY(hipMemcpy(e->f8.history, st->amax_history, L * 4 * HL * sizeof(float), hipMemcpyHostToDevice), "fp8 state");
    HIP_TRY(hipMemcpy(e->f8.steps, st->steps, L * sizeof(int64_t), hipMemcpyHostToDevice), "fp8 state");
    HIP_TRY(hipMemset(e->f8.act_amax, 0, L * 4 * sizeof(uint32_t)), "fp8 state");
  }
  const uint32_t flags = st->nonfinite ? 1u : 0u;
  HIP_TRY(hipMemcpy(e->f8.flags, &flags, sizeof flags, hipMemcpyHostToDevice), "fp8 state");
  return ok();
}

esm_status esm_fp8_reset(esm_encoder* e, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (!e->fp8_mem) return fail(ESM_ERR_STATE, "encoder has no FP8 state (bf16, or MXFP4 with no FP8 layer)");
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  return fp8_reset_state(e);
}

esm_status esm_fp8_grad_quantize(esm_encoder* e, int32_t layer_idx, int32_t slot, const void* g, int64_t n, void* y8,
                                 float* scale_out, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !g || !y8) return fail(ESM_ERR_NULL, "NULL argument");
  if (!e->fp8_mem) return fail(ESM_ERR_STATE, "encoder has no FP8 state (bf16, or MXFP4 with no FP8 layer)");
  if (layer_idx < 0 || layer_idx >= e->cfg.num_hidden_layers || slot < 0 || slot > 3)
    return fail(ESM_ERR_SHAPE, "layer_idx %d / slot %d outside [0, %d) / [0, 4)", layer_idx, slot,
                e->cfg.num_hidden_layers);
  if (n < 0 || n % 8) return fail(ESM_ERR_SHAPE, "n %lld: a non-negative multiple of 8", (long long)n);
  if (!aligned16(g) || ((uintptr_t)y8 & 7u) || ((uintptr_t)scale_out & 3u))
    return fail(ESM_ERR_UNSUPPORTED, "misaligned pointer");
  if (n == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  const int k = 4 * layer_idx + slot;
  return timed(e, ESM_K_FP8, st, "e5m2 gradient cast", [&] {
    return launch_quantize_e5m2((const bf16_t*)g, n, e->f8.g_scale + k, (uint8_t*)y8, e->f8.g_amax + k, st, scale_out);
  });
}

esm_status esm_fp8_grad_step(esm_encoder* e, int32_t layer_idx, esm_stream_t stream) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  if (!e->fp8_mem) return fail(ESM_ERR_STATE, "encoder has no FP8 state (bf16, or MXFP4 with no FP8 layer)");
  if (layer_idx < 0 || layer_idx >= e->cfg.num_hidden_layers)
    return fail(ESM_ERR_SHAPE, "layer_idx %d outside [0, %d)", layer_idx, e->cfg.num_hidden_layers);
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  hipStream_t st = (hipStream_t)stream;
  return timed(e, ESM_K_FP8, st, "gradient scale update", [&] { return launch_grad_scale_update(e->f8, layer_idx, st); });
}

esm_status esm_fp8_grad_get_state(esm_encoder* e, float* scale, float* history, int64_t* steps, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !scale || !history || !steps) return fail(ESM_ERR_NULL, "NULL argument");
  if (!e->fp8_mem) return fail(ESM_ERR_STATE, "encoder has no FP8 state (bf16, or MXFP4 with no FP8 layer)");
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  const size_t L = (size_t)e->cfg.num_hidden_layers, HL = (size_t)e->cfg.amax_history_len;
  if (L > 0) {
    HIP_TRY(hipMemcpy(scale, e->f8.g_scale, L * 4 * sizeof(float), hipMemcpyDeviceToHost), "fp8 gradient state");
    HIP_TRY(hipMemcpy(history, e->f8.g_history, L * 4 * HL * sizeof(float), hipMemcpyDeviceToHost),
            "fp8 gradient state");
    HIP_TRY(hipMemcpy(steps, e->f8.g_steps, L * sizeof(int64_t), hipMemcpyDeviceToHost), "fp8 gradient state");
  }
  return ok();
}

esm_status esm_set_layer_precision(esm_encoder* e, const int32_t* prec, int32_t n, esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !prec) return fail(ESM_ERR_NULL, "NULL argument");
  if (!is_quantised(e)) return fail(ESM_ERR_STATE, "encoder was created with bf16 precision");
  if (n != e->cfg.num_hidden_layers)
    return fail(ESM_ERR_SHAPE, "%d precisions for %d layers", n, e->cfg.num_hidden_layers);
  bool any8 = false, any4 = false;
  for (int32_t l = 0; l < n; ++l) {
    if (prec[l] != ESM_PRECISION_BF16 && prec[l] != ESM_PRECISION_FP8_DELAYED && prec[l] != ESM_PRECISION_MXFP4)
      return fail(ESM_ERR_UNSUPPORTED, "layer %d: precision %d", l, prec[l]);
    any8 |= prec[l] == ESM_PRECISION_FP8_DELAYED;
    any4 |= prec[l] == ESM_PRECISION_MXFP4;
  }
  esm_status s;
  if (any8 && (s = check_fp8_shape(&e->cfg))) return s;
  if (any4 && (s = check_mx_shape(&e->cfg))) return s;
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  e->layer_prec.assign(prec, prec + n);
  // An FP8 layer needs the delayed-scaling state; the state's per-layer flags
  // say which layers record amax and roll their history.
  if (any8 && (s = ensure_fp8(e))) return s;
  if (e->fp8_mem) {
    std::vector<int32_t> on((size_t)n);
    for (int32_t l = 0; l < n; ++l) on[(size_t)l] = prec[l] == ESM_PRECISION_FP8_DELAYED;
    HIP_TRY(hipMemcpy(e->f8.layer_on, on.data(), on.size() * sizeof(int32_t), hipMemcpyHostToDevice),
            "layer flags");
  }
  return ok();
}

esm_status esm_fp8_quantize(esm_encoder* e, const float* x, int64_t n, const float* scale, void* y, uint32_t* amax,
                            esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !x || !scale || !y || !amax) return fail(ESM_ERR_NULL, "NULL argument");
  if (n < 0) return fail(ESM_ERR_SHAPE, "n < 0");
  if (n == 0) return ok();
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  return timed(e, ESM_K_FP8, (hipStream_t)stream, "e4m3 cast",
               [&] { return launch_quantize_f32(x, n, scale, (uint8_t*)y, amax, (hipStream_t)stream); });
}

esm_status esm_mfma_peak(esm_encoder* e, int32_t iters, void* sink, size_t sink_bytes, double* flops,
                         esm_stream_t stream) {
  g_last_error.clear();
  if (!e || !sink || !flops) return fail(ESM_ERR_NULL, "NULL argument");
  if (iters <= 0) return fail(ESM_ERR_SHAPE, "iters %d must be positive", iters);
  HIP_TRY(hipSetDevice(e->device), "hipSetDevice");
  const int32_t blocks = mfma_peak_blocks();
  if (sink_bytes < (size_t)blocks * 4 * sizeof(float))
    return fail(ESM_ERR_WORKSPACE, "sink of %zu bytes, %zu needed", sink_bytes, (size_t)blocks * 4 * sizeof(float));
  *flops = (double)blocks * 4 * 16 * (double)iters * 32768.0;
  hipStream_t st = (hipStream_t)stream;
  return timed(e, ESM_K_OTHER, st, "mfma peak", [&] { return launch_mfma_peak(iters, blocks, (float*)sink, st); });
}

esm_status esm_profile_enable(esm_encoder* e, int32_t on) {
  g_last_error.clear();
  if (!e) return fail(ESM_ERR_NULL, "encoder is NULL");
  e->profiling = on != 0;
  e->recs.clear();
  e->pool_used = 0;
  for (int i = 0; i < ESM_K_COUNT; ++i) {
    e->ms[i] = 0;
    e->launches[i] = 0;
  }
  return ok();
}

esm_status esm_profile_read(esm_encoder* e, double* ms_out, int64_t* launches_out) {
  g_last_error.clear();
  if (!e || !ms_out || !launches_out) return fail(ESM_ERR_NULL, "NULL argument");
  if (!e->recs.empty()) {
    HIP_TRY(hipEventSynchronize(e->pool[e->recs.back().second + 1]), "hipEventSynchronize");
    for (auto& r : e->recs) {
      float ms = 0.f;
      HIP_TRY(hipEventElapsedTime(&ms, e->pool[r.second], e->pool[r.second + 1]), "hipEventElapsedTime");
      e->ms[r.first] += ms;
      e->launches[r.first] += 1;
    }
    e->recs.clear();
    e->pool_used = 0;
  }
  for (int i = 0; i < ESM_K_COUNT; ++i) {
    ms_out[i] = e->ms[i];
    launches_out[i] = e->launches[i];
  }
  return ok();
}

esm_status esm_check_cu_seqlens(const int32_t* cu, int32_t B, int64_t T, int32_t max_seqlen, int32_t max_positions) {
  if (!cu) return fail(ESM_ERR_NULL, "cu_seqlens is NULL");
  if (B < 0 || T < 0) return fail(ESM_ERR_SHAPE, "negative B or T");
  if (max_seqlen < 0 || max_seqlen > max_positions)
    return fail(ESM_ERR_SEQLENS, "max_seqlen %d outside [0, %d]", max_seqlen, max_positions);
  if (cu[0] != 0) return fail(ESM_ERR_SEQLENS, "cu_seqlens[0] = %d, expected 0", cu[0]);
  for (int32_t s = 0; s < B; ++s) {
    const int64_t L = (int64_t)cu[s + 1] - cu[s];
    if (L < 0) return fail(ESM_ERR_SEQLENS, "cu_seqlens decreases at %d (%d -> %d)", s, cu[s], cu[s + 1]);
    if (L > max_seqlen) return fail(ESM_ERR_SEQLENS, "sequence %d has length %lld > max_seqlen %d", s, (long long)L, max_seqlen);
  }
  if ((int64_t)cu[B] != T) return fail(ESM_ERR_SEQLENS, "cu_seqlens[B] = %d, expected T = %lld", cu[B], (long long)T);
  return ESM_OK;
}

esm_status esm_check_seqlens(const int32_t* sl, int32_t B, int32_t S, int32_t max_positions) {
  if (!sl) return fail(ESM_ERR_NULL, "seqlens is NULL");
  if (B < 0 || S < 0) return fail(ESM_ERR_SHAPE, "negative B or S");
  if (S > max_positions) return fail(ESM_ERR_SEQLENS, "S = %d above max positions %d", S, max_positions);
  for (int32_t b = 0; b < B; ++b)
    if (sl[b] < 0 || sl[b] > S) return fail(ESM_ERR_SEQLENS, "seqlens[%d] = %d outside [0, S = %d]", b, sl[b], S);
  return ESM_OK;
}

const char* esm_last_error(void) { return g_last_error.c_str(); }

const char* esm_status_str(esm_status s) {
  switch (s) {
    case ESM_OK: return "ESM_OK";
    case ESM_ERR_NULL: return "ESM_ERR_NULL";
    case ESM_ERR_SHAPE: return "ESM_ERR_SHAPE";
    case ESM_ERR_SEQLENS: return "ESM_ERR_SEQLENS";
    case ESM_ERR_UNSUPPORTED: return "ESM_ERR_UNSUPPORTED";
    case ESM_ERR_WORKSPACE: return "ESM_ERR_WORKSPACE";
    case ESM_ERR_ARCH: return "ESM_ERR_ARCH";
    case ESM_ERR_HIP: return "ESM_ERR_HIP";
    case ESM_ERR_STATE: return "ESM_ERR_STATE";
  }
  return "unknown status";
}

int32_t esm_abi_version(void) { return ESM_ABI_VERSION; }

}  // extern "C"
