/*
 * esm_encoder.h -- C ABI of the MI355X (gfx950) ESM-2 encoder forward.
 *
 * The library runs the forward pass of the ESM-2 BERT-style encoder layer
 * stack over variable-length protein sequences, either packed by cu_seqlens
 * (THD layout, no padding) or padded (bshd layout with per-row valid
 * lengths).  Every step runs in the library's own HIP kernels.
 *
 * Pages that define the operations (title, section):
 *   [TE-ESM2] "深入源码NVIDIA ESM-2 TransformerEngine优化的实现原理与技术细节":
 *             核心技术架构设计 (NVEsmEncoder: a stack of Transformer layers;
 *             config.json 33 layers / hidden 1280 / 20 heads), 旋转位置编码集成
 *             (rotary embedding of size hidden/heads), 注意力掩码优化 (padding mask,
 *             bshd input format), 权重融合技术 (fused, interleaved QKV weight),
 *             序列长度优化 (max_position_embeddings 1026, vocab 33),
 *             自动混合精度训练 (per-layer forward loop).
 *   [BIO-ACC] "生物大模型训练加速实战：基于PyTorch与NVIDIA BioNeMo的Transformer优化指南":
 *             3.1 (EsmLayer: self-attention, LayerNorm, fc1, fc2; TransformerLayer
 *             with hidden / ffn / heads, encoder type, padding mask, bshd or thd),
 *             3.2 (collate_fn: cu_seqlens = cumsum([0] + lengths), max_seqlen =
 *             max(lengths); PackedEsm.forward(input_ids, cu_seqlens, max_seqlen)
 *             = embedding then every layer), 4.1 (DelayedScaling recipe).
 *   [CARD]    "ESM-2" (BioNeMo framework model card): 描述 (bidirectional BERT-style
 *             encoder; 650M and 3B shapes), 输入 (at most 1022 residues), 输出 (one
 *             embedding vector per residue).
 *   [TE-RU]   TransformerEngine tutorial summary (aikraft.ru): fused modules
 *             LayerNormLinear / LayerNormMLP / TransformerLayer; FP8 DelayedScaling
 *             with amax_history_len 16 and the "max" algorithm.
 *
 * Conventions for every call
 *   - All tensors are device pointers to bfloat16 unless stated, row-major,
 *     16-byte aligned.  Linear weights use the [out, in] layout.
 *   - Calls are asynchronous on the given stream (hipStream_t, NULL = the
 *     default stream): they enqueue kernels and return.  The caller keeps every
 *     buffer alive until the stream has passed the call.
 *   - All argument checks happen on the host before anything is enqueued; on
 *     failure nothing is enqueued and esm_last_error() describes the problem.
 *   - One handle must not be used from two host threads or two streams at once.
 *   - The caller owns every tensor passed in, the workspace and the stream.  The
 *     library owns the handle and the rotary table it builds at create time,
 *     and, for the FP8 precision, the delayed-scaling state and the E4M3
 *     copies of the weights.
 */
#ifndef ESM_ENCODER_H
#define ESM_ENCODER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ESM_ABI_VERSION 22

/* Query rows per attention workgroup (the segment table's tile size). */
#define ESM_ATTN_TILE_ROWS 256

typedef struct esm_encoder esm_encoder;
typedef void* esm_stream_t; /* a hipStream_t */

typedef enum {
  ESM_OK = 0,
  ESM_ERR_NULL = 1,        /* a required pointer is NULL */
  ESM_ERR_SHAPE = 2,       /* bad hidden / heads / ffn / layers / vocab / T / B / S */
  ESM_ERR_SEQLENS = 3,     /* host copy of cu_seqlens / seqlens inconsistent */
  ESM_ERR_UNSUPPORTED = 4, /* head_dim != 64, misaligned pointer, unknown option */
  ESM_ERR_WORKSPACE = 5,   /* workspace NULL or too small */
  ESM_ERR_ARCH = 6,        /* device is not gfx950 */
  ESM_ERR_HIP = 7,         /* HIP runtime error */
  ESM_ERR_STATE = 8        /* call not valid in the handle's current state */
} esm_status;

typedef enum { ESM_PRECISION_BF16 = 0, ESM_PRECISION_FP8_DELAYED = 1, ESM_PRECISION_MXFP4 = 2 } esm_precision;
typedef enum { ESM_LAYOUT_THD = 0, ESM_LAYOUT_BSHD = 1 } esm_layout;

/* Model configuration.  Key names follow the config.json keys of [TE-ESM2]. */
typedef struct {
  int32_t hidden_size;          /* H, multiple of 64 */
  int32_t num_attention_heads;  /* H / 64 (head_dim 64 is the only one built) */
  int32_t intermediate_size;    /* F, FFN width, multiple of 64 */
  int32_t num_hidden_layers;    /* layers in a stack call */
  int32_t vocab_size;           /* rows of the embedding table */
  int32_t max_position_embeddings; /* rotary table rows; longest allowed sequence */
  float layer_norm_eps;         /* LayerNorm epsilon (biased variance) */
  float rope_base;              /* rotary base; theta_i = p * base^(-i/32) */
  int32_t precision;            /* esm_precision; FP8 needs H and F multiples of 128 */
  int32_t amax_history_len;     /* FP8 delayed-scaling history, 1..1024 */
} esm_config;

/* Fills the ESM-2 650M configuration: H 1280, 20 heads, F 5120, 33 layers,
 * vocab 33, 1026 positions, eps 1e-5, base 10000, bf16, history 16. */
void esm_config_default(esm_config* cfg);

/* One layer's tensors (bfloat16, device).  Rows of w_qkv [3H, H] are grouped
 * per head as in [TE-ESM2] 权重融合技术 with the interleaved flag: row
 * 192*n + 64*c + j is component c (0 query, 1 key, 2 value) of head n, dim j.
 * Bias pointers may be NULL (treated as zero); gamma/beta may not. */
typedef struct {
  const void* ln1_gamma; /* [H] */
  const void* ln1_beta;  /* [H] */
  const void* w_qkv;     /* [3H, H] */
  const void* b_qkv;     /* [3H] */
  const void* w_out;     /* [H, H] */
  const void* b_out;     /* [H] */
  const void* ln2_gamma; /* [H] */
  const void* ln2_beta;  /* [H] */
  const void* w_fc1;     /* [F, H] */
  const void* b_fc1;     /* [F] */
  const void* w_fc2;     /* [H, F] */
  const void* b_fc2;     /* [H] */
} esm_layer_weights;

/* ---------------------------------------------------------------- lifetime */

/* Validates cfg, checks that `device` is a gfx950 GPU (ESM_ERR_ARCH otherwise),
 * makes it current and builds the rotary cos/sin table [max_positions, 32]
 * (fp32, computed in fp64 on the host).  *out receives the new handle. */
esm_status esm_encoder_create(const esm_config* cfg, int device, esm_encoder** out);

/* Frees the handle and everything it owns.  NULL is a no-op. */
esm_status esm_encoder_destroy(esm_encoder* enc);

/* ---------------------------------------------------------------- workspace */

/* Bytes of device workspace a forward call needs for up to max_tokens rows
 * (T for THD, B*S for bshd) and max_seqs sequences.  The workspace is
 * caller-allocated, 256-byte aligned, and may be reused between calls once the
 * stream has passed the previous one.  Its contents after a layer call hold
 * that layer's intermediates (see esm_workspace_region).  The size includes
 * the few kilobytes esm_stack_fwd's two-group schedule needs beyond the
 * regions (a smaller workspace that holds the regions runs it as one group). */
esm_status esm_workspace_size(const esm_encoder* enc, int64_t max_tokens, int32_t max_seqs,
                              size_t* bytes);

/* With the FP8 precision the four GEMM inputs (LN1, CTX, LN2, ACT) hold E4M3
 * bytes with the same row counts ([T, H] or [T, F] bytes, the region keeps its
 * bf16 size); the code of value v is cast(v * scale) of that tensor. */
typedef enum {
  ESM_WS_LN1 = 0,   /* bf16 [T, H]  LayerNorm-1 output */
  ESM_WS_QKV = 1,   /* bf16 [3, heads, T, 64]  rotated q, rotated k, v (planar) */
  ESM_WS_CTX = 2,   /* bf16 [T, H]  attention output, head-major columns */
  ESM_WS_X1 = 3,    /* bf16 [T, H]  after the attention residual */
  ESM_WS_LN2 = 4,   /* bf16 [T, H]  LayerNorm-2 output */
  ESM_WS_ACT = 5,   /* bf16 [T, F]  GELU(fc1) */
  ESM_WS_POS = 6,   /* int32 [T]    position of each row in its sequence, -1 = padding */
  ESM_WS_TILES = 7, /* int32 [n, 2] attention query tiles (sequence, first row) */
  ESM_WS_NTILES = 8,/* int32 [1]    number of valid tiles */
  ESM_WS_SEGS = 9,  /* int32 [B, 2] (first row, length) of every sequence */
  ESM_WS_STATS = 10 /* float2 [ceil(H / 256), T] LayerNorm statistics of a layer's input rows in
                     * 256-column chunks (mean, sum of squared deviations), used by the layers
                     * prepared with esm_prepare_layer */
} esm_ws_region;

/* Byte offset and size of one region inside a workspace sized for
 * (max_tokens, max_seqs).  Row strides use T = max_tokens. */
esm_status esm_workspace_region(const esm_encoder* enc, int64_t max_tokens, int32_t max_seqs,
                                int32_t region, size_t* offset, size_t* bytes);

/* ---------------------------------------------------------------- forward */

/* One pre-LN encoder layer on a packed batch ([BIO-ACC] 3.1, 3.2):
 *   X1 = X + Attn(RoPE(LN1(X) W_qkv^T + b_qkv)) W_out^T + b_out
 *   Y  = X1 + GELU(LN2(X1) W_fc1^T + b_fc1) W_fc2^T + b_fc2
 * Attention is non-causal and stays inside each sequence; positions restart at
 * 0 in every sequence.
 *   x_in, x_out      [T, H]; x_out may equal x_in (in-place)
 *   cu_seqlens_dev   int32 [B+1] on the device: sequence s owns rows
 *                    cu[s] .. cu[s+1]-1; zero-length sequences allowed
 *   cu_seqlens_host  optional host copy; when given it is checked (cu[0] = 0,
 *                    non-decreasing, cu[B] = T, every length <= max_seqlen <=
 *                    max_positions) and ESM_ERR_SEQLENS returned on failure.
 *                    When NULL the device array is trusted; kernels clamp every
 *                    index, so bad values give wrong numbers, never an
 *                    out-of-bounds access.
 *   max_seqlen       host upper bound on the sequence lengths
 *   layer_idx        0-based index of the layer (FP8 state slot)
 * T = 0 or B = 0 returns ESM_OK without a launch.
 *
 * FP8 precision (ESM_PRECISION_FP8_DELAYED; [BIO-ACC] 2.1 and 4.1, [TE-RU] FP8
 * recipe): each of the four linears computes (Q(a s_a) Q(W s_w)^T) / (s_a s_w)
 * + b, Q = cast to E4M3 (round to nearest even, saturating at +-448), with the
 * per-tensor scales of layer layer_idx; LayerNorm, attention, the residuals and
 * every GEMM output stay in bf16/fp32.  The layer's E4M3 weights come from
 * esm_fp8_prepare_layer (ESM_ERR_STATE if it was never called for layer_idx);
 * the bf16 weight pointers in w must still be valid, LN parameters and biases
 * are read from w.  The call is one delayed-scaling step for that layer: it
 * uses the scales fixed by earlier steps, records this step's amax of the four
 * activations and, at its end, rolls the history and sets the next scales.
 *
 * MXFP4 precision (ESM_PRECISION_MXFP4; the FP4 recipe of [TE-ESM2]
 * FP8与FP4混合精度支持, read as OCP MXFP4, see esm_mxfp4_quantize): each linear
 * computes x_q . W_q^T + b with x_q the GEMM input written straight in MXFP4
 * (32-value blocks along K) by its producer from fp32 values -- LayerNorm,
 * the attention epilogue, fc1's GELU epilogue -- on every call (no state, no
 * bf16 copy of the input) and W_q from esm_mxfp4_prepare_layer
 * (ESM_ERR_STATE if never called for layer_idx); LayerNorm, attention, the
 * residuals and every GEMM output stay in bf16/fp32.  Needs hidden_size and
 * intermediate_size multiples of 256 and intermediate_size <= 8 hidden_size
 * (checked at create).
 *
 * A quantised encoder (FP8 or MXFP4) runs each layer in the precision
 * esm_set_layer_precision gave it -- FP8, MXFP4 or bf16, its own by default --
 * so one stack can mix FP8 and MXFP4 layers. */
esm_status esm_layer_fwd(esm_encoder* enc, const esm_layer_weights* w, int32_t layer_idx,
                         const void* x_in, void* x_out,
                         const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                         int32_t B, int64_t T, int32_t max_seqlen,
                         void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Allocation-free variant of esm_layer_fwd, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, semantics and results (bit for bit)
 * as esm_layer_fwd, without the workspace: the layer's intermediates go to a
 * library scratch array of ESM_NOALLOC_SCRATCH_BYTES per device, held from
 * load until the process ends.  The call allocates nothing and records no
 * esm_profile_* timing.  A batch whose workspace (esm_workspace_size(T, B))
 * exceeds the scratch returns ESM_ERR_WORKSPACE before any launch (at hidden
 * 1280 / FFN 5120 that is about 2,300 rows).  Every call on one device shares
 * that device's scratch: calls whose stream work overlaps on one device race
 * (order them on one stream, or with events).  Nothing in the scratch needs
 * to start at zero: every region a layer reads is written earlier in that
 * same call. */
#define ESM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
esm_status esm_layer_fwd_noalloc(esm_encoder* enc, const esm_layer_weights* w, int32_t layer_idx,
                                 const void* x_in, void* x_out,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                 int32_t B, int64_t T, int32_t max_seqlen, esm_stream_t stream);

/* Embedding lookup (when token_ids != NULL: X0 = E[ids], ids clamped into
 * [0, vocab)) or the given hidden states x_in, then all num_hidden_layers
 * layers in order ([BIO-ACC] 3.2 PackedEsm.forward; [TE-ESM2] 自动混合精度训练).
 * No final LayerNorm.  `w` is a HOST array of num_hidden_layers structs.
 * FP8: layer l uses state slot l; the call is one step for every layer.
 * With cu_seqlens_host given (and per-kernel timing off) the batch may run
 * as two groups of whole sequences, split where esm_stack_split says, the
 * first on `stream` and the second on the encoder's own stream (default
 * priority), forked from and joined back to `stream` inside the call: one
 * group's attention runs beside the other's GEMMs.  Rows do not interact, so
 * the output (and the FP8 state) is the same bit for bit as one group's. */
esm_status esm_stack_fwd(esm_encoder* enc, const esm_layer_weights* w,
                         const int32_t* token_ids, const void* embedding,
                         const void* x_in, void* x_out,
                         const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                         int32_t B, int64_t T, int32_t max_seqlen,
                         void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Where esm_stack_fwd splits a batch into its two groups (host only): the
 * sequence index b written to *split_seq (group 1 = sequences 0 .. b - 1,
 * group 2 = b .. B - 1), or 0 when it runs one group.  A split is taken only
 * where, for each GEMM output width of the layer (3 hidden, hidden,
 * intermediate), the two groups' rounds of workgroups over the device's
 * compute units (the current device's, 256 when none is visible) sum to at
 * most the whole batch's, and among those the one with the most balanced
 * tokens; never below 4096 rows or 2 sequences.  cu_seqlens_host [B + 1]
 * from 0 to T.  Errors: ESM_ERR_NULL, ESM_ERR_SHAPE. */
esm_status esm_stack_split(int32_t hidden_size, int32_t intermediate_size, const int32_t* cu_seqlens_host,
                           int32_t B, int64_t T, int32_t* split_seq);

/* Padded (bshd) variants ([TE-ESM2] 注意力掩码优化; [BIO-ACC] 3.1 bshd format).
 * x_in / x_out are [B, S, H]; row b holds a valid prefix of seqlens[b] <= S
 * tokens (the padding mask, 1 = valid, as lengths).  Keys beyond the prefix
 * are never read; output rows beyond it are written as 0.  The dense layers run
 * over all B*S rows, as padded execution does.  Workspace is sized with
 * max_tokens = B*S, max_seqs = B. */
esm_status esm_layer_fwd_bshd(esm_encoder* enc, const esm_layer_weights* w, int32_t layer_idx,
                              const void* x_in, void* x_out,
                              const int32_t* seqlens_dev, const int32_t* seqlens_host,
                              int32_t B, int32_t S,
                              void* workspace, size_t workspace_bytes, esm_stream_t stream);

esm_status esm_stack_fwd_bshd(esm_encoder* enc, const esm_layer_weights* w,
                              const int32_t* token_ids, const void* embedding,
                              const void* x_in, void* x_out,
                              const int32_t* seqlens_dev, const int32_t* seqlens_host,
                              int32_t B, int32_t S,
                              void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* ---------------------------------------------------------------- after the stack */

/* Weights of the final LayerNorm and of the masked-LM head (device bf16,
 * row-major [out, in] like the layer weights). */
typedef struct {
  const void* final_ln_gamma;  /* [H] LayerNorm after the last layer */
  const void* final_ln_beta;   /* [H] */
  const void* lm_dense_w;      /* [H, H] LM head dense layer */
  const void* lm_dense_b;      /* [H] or NULL (zero) */
  const void* lm_ln_gamma;     /* [H] LM head LayerNorm */
  const void* lm_ln_beta;      /* [H] */
  const void* lm_decoder_w;    /* [vocab, H] decoder weight: the token embedding (tied) */
  const void* lm_decoder_b;    /* [vocab] or NULL (zero) */
} esm_head_weights;

/* The outputs after the stack ([CARD] 输出: per-residue and sequence-level
 * embeddings; [TE-ESM2] 快速开始使用: the model as a masked LM; the layouts of
 * the final LayerNorm and the head are ESM-2's, which the pages do not spell
 * out):
 *   x_final    = LayerNorm(x; final_ln)                  bf16 [T, H]; may alias x
 *   logits     = LN(GELU(x_final W_d^T + b_d); lm_ln) E^T + b_e
 *                                                         bf16 [T, vocab]; skipped when NULL
 *   seq_emb[s] = mean of x_final over sequence s's rows   fp32 [B, H], 0 for an empty
 *                                                         sequence; skipped when NULL
 * x, cu_seqlens, B, T, max_seqlen and the workspace as for esm_stack_fwd (the
 * workspace of esm_workspace_size(T, B) suffices); cu_seqlens_dev may be NULL
 * when seq_emb is.  Runs in bf16 with fp32 accumulation for both precisions.
 * x, x_final and the weights must be 16-byte aligned (x and x_final may be
 * NULL when T = 0); the LM head takes vocab <= min(4096, 3 H). */
esm_status esm_head_fwd(esm_encoder* enc, const esm_head_weights* w, const void* x, void* x_final,
                        void* logits, float* seq_emb, const int32_t* cu_seqlens_dev,
                        const int32_t* cu_seqlens_host, int32_t B, int64_t T, int32_t max_seqlen,
                        void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* ---------------------------------------------------------------- kernel-level entries */

/* Segment table ([BIO-ACC] 3.2 cu_seqlens contract): writes into the workspace
 * the per-row positions (ESM_WS_POS), the sequence extents (ESM_WS_SEGS) and the
 * attention query tiles of ESM_ATTN_TILE_ROWS rows, longest sequence first
 * (ESM_WS_TILES, count in ESM_WS_NTILES).  layout selects cu_seqlens (THD,
 * `lens` = cu [B+1], S ignored) or seqlens (bshd, `lens` = [B], rows b*S + p). */
esm_status esm_segment_table(esm_encoder* enc, int32_t layout, const int32_t* lens_dev,
                             int32_t B, int64_t T, int32_t S,
                             void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Attention alone on a packed batch: qkv is [3, heads, T, 64] (q and k
 * already rotated), ctx is [T, H].  Runs the segment table first. */
esm_status esm_attention_fwd(esm_encoder* enc, const void* qkv, void* ctx,
                             const int32_t* cu_seqlens_dev, int32_t B, int64_t T,
                             void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Attention with its softmax normaliser, for a backward pass: as
 * esm_attention_fwd, and also lse[n * T + t] = log sum_j exp(q_t . k_j / 8)
 * over the keys j of t's sequence (natural log, fp32, head-major [heads, T]).
 * lse: device, 4-byte aligned, written for every row of every sequence.
 * Errors as esm_attention_fwd; ESM_ERR_NULL for lse NULL. */
esm_status esm_attention_fwd_lse(esm_encoder* enc, const void* qkv, void* ctx, float* lse,
                                 const int32_t* cu_seqlens_dev, int32_t B, int64_t T,
                                 void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Attention backward (the gradient of the forward above; the pages time
 * training, [BIO-ACC] 3.2 and 6, [CARD] 训练性能).  For each sequence and head,
 * with S = q k^T / 8, P = exp(S - lse) and dO = the gradient of the context:
 *   dv = P^T dO,  dP = dO v^T,  dS = P * (dP - rowsum(dO * O)),
 *   dq = dS k / 8,  dk = dS^T q / 8.
 * qkv:   bf16 [3, heads, T, 64], the forward's input (q and k rotated).
 * ctx:   bf16 [T, H], the forward's context O; dctx: bf16 [T, H], dO.
 * lse:   fp32 [heads, T] from esm_attention_fwd_lse on the same qkv.
 * delta: fp32 [heads, T] device scratch, overwritten (rowsum(dO * O)).
 * dqkv:  bf16 [3, heads, T, 64] out (dq, dk, dv in qkv's layout); must not
 *        overlap the inputs.
 * Tensors 16-byte aligned, lse and delta 4-byte aligned.  P is recomputed from
 * lse (never stored); P and dS enter their products as bf16 with fp32
 * accumulation.  Runs the segment table first (workspace as
 * esm_attention_fwd).  Errors: ESM_ERR_NULL, ESM_ERR_UNSUPPORTED (alignment),
 * ESM_ERR_SHAPE / ESM_ERR_WORKSPACE as esm_attention_fwd.  Asynchronous. */
esm_status esm_attention_bwd(esm_encoder* enc, const void* qkv, const void* ctx, const void* dctx,
                             const float* lse, float* delta, void* dqkv,
                             const int32_t* cu_seqlens_dev, int32_t B, int64_t T,
                             void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Biased attention ([DS4SCI] 3.2 and 5.3: the Evoformer attention kernel,
 * which takes Q, K, V shaped [B, N, L, heads, D] and up to two additive
 * biases, a per-key mask bias [B, N, 1, 1, L] and a pair bias
 * [B, 1, heads, L, L] shared by the N rows).  For every (b, n, h):
 *   out[b, n, i, h, :] = sum_j P_ij v[b, n, j, h, :],
 *   P_ij = softmax_j( q_i . k_j / sqrt(64) + mask[b, n, j] + pair[b, h, i, j] ).
 * q, k, v, out: bf16, contiguous [B, N, L, heads, 64], 16-byte aligned (the
 *   head size is 64 only).  out must not overlap q, k or v.
 * mask_bias: bf16 [B, N, L] (the [B, N, 1, 1, L] tensor) or NULL (no mask).
 * pair_bias: bf16 [B, heads, L, L] (the [B, 1, heads, L, L] tensor) or NULL.
 * Both biases are read as stored (e.g. -inf or a large negative value for
 * masked keys); they need 8-byte alignment when L % 4 == 0.  A row whose
 * scores are all -inf has no softmax and yields NaN, as the definition does.
 * enc selects the device and the profiling timers; no workspace is used.
 * Errors: ESM_ERR_NULL (enc NULL; q, k, v or out NULL with no size 0),
 * ESM_ERR_SHAPE (B, N, heads < 0, L < 0 or L > 65536, or more than 2^31 - 1
 * workgroups), ESM_ERR_UNSUPPORTED (misaligned pointer).  Any size 0 returns
 * ESM_OK with no launch.  Asynchronous on stream. */
esm_status esm_biased_attention_fwd(esm_encoder* enc, const void* q, const void* k, const void* v,
                                    const void* mask_bias, const void* pair_bias, void* out,
                                    int32_t B, int32_t N, int32_t L, int32_t heads,
                                    esm_stream_t stream);

/* MXFP4 quantisation (the FP4 recipe, [TE-ESM2] FP8与FP4混合精度支持, read as
 * OCP MXFP4: E2M1 values in blocks of 32 along K, one E8M0 scale per block).
 * Per block: e = floor(log2 max|v|) - 2, clamped to [-127, 127] (-127 for an
 * all-zero block), scale byte e + 127, and each value v / 2^e rounded to the
 * nearest E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6 with sign), ties to even,
 * saturating at 6.
 *   x      bf16 [M, K] row-major, K a positive multiple of 256, finite values
 *          (subnormal inputs may be flushed to zero).
 *   codes  uint8 [M, K / 2]: value 2j of a row in the low nibble of byte j,
 *          value 2j + 1 in the high nibble (bit 3 of a nibble is the sign).
 *   scales uint8 [K / 256][M2][8], M2 = M rounded up to even: the 8 bytes of
 *          (K step s, row m) are the scales of blocks 8s + 0, 2, 4, 6, 1, 3, 5,
 *          7 (the order the MXFP4 GEMM reads them in); the pad row of an odd
 *          M holds 127.
 * x and codes 16-byte aligned, scales 16-byte aligned.  Errors: ESM_ERR_NULL,
 * ESM_ERR_SHAPE (M < 0, K not a positive multiple of 256),
 * ESM_ERR_UNSUPPORTED (alignment).  M = 0 launches nothing. */
esm_status esm_mxfp4_quantize(esm_encoder* enc, const void* x, int64_t M, int32_t K, void* codes,
                              void* scales, esm_stream_t stream);

typedef enum {
  ESM_EPI_BIAS = 0,          /* y = x W^T + b */
  ESM_EPI_BIAS_GELU = 1,     /* y = GELU(x W^T + b) */
  ESM_EPI_BIAS_RESIDUAL = 2, /* y = r + x W^T + b */
  ESM_EPI_BIAS_GELU_E4M3 = 3 /* y = cast(GELU(x W^T + b) * s_y) to E4M3, amax recorded (E4M3 GEMM only) */
} esm_epilogue;

/* y[M, N] = epilogue(x[M, K] W[N, K]^T + b) on the library's MFMA GEMM.
 * N and K must be multiples of 64; residual r is [M, N] (may equal y). */
esm_status esm_linear_fwd(esm_encoder* enc, const void* x, const void* w, const void* b,
                          const void* residual, void* y, int64_t M, int32_t N, int32_t K,
                          int32_t epilogue, esm_stream_t stream);

/* E4M3 GEMM of the FP8 path ([BIO-ACC] 4.1, [TE-RU] FP8 recipe):
 *   z = (x8 . w8^T) / (x_scale[0] * w_scale[0]) + b,  then the epilogue on z.
 *   x8 [M, K], w8 [N, K]: E4M3 codes (uint8); x_scale, w_scale: device float[1]
 *   y: bf16 [M, N], or E4M3 [M, N] for ESM_EPI_BIAS_GELU_E4M3, which casts
 *      GELU(z) * y_scale[0] and atomically maxes max|GELU(z)| into *y_amax
 *      (device uint32 holding float bits; the caller clears it).
 * N must be a multiple of 64 and K of 128. */
esm_status esm_linear_e4m3_fwd(esm_encoder* enc, const void* x8, const float* x_scale,
                               const void* w8, const float* w_scale, const void* b,
                               const void* residual, void* y, const float* y_scale,
                               uint32_t* y_amax, int64_t M, int32_t N, int32_t K,
                               int32_t epilogue, esm_stream_t stream);

/* MXFP4 GEMM (the FP4 recipe reading, [TE-ESM2] FP8与FP4混合精度支持):
 *   y = epilogue(x_q . w_q^T + b),  x_q[m, k] = 2^(xs - 127) * E2M1(code)
 * with the codes and block scales of esm_mxfp4_quantize for x [M, K] and
 * w [N, K] (w's scale array has N rows: N is even).  Products of the
 * dequantised values accumulate in fp32 on the scaled MFMA; y is bf16 [M, N].
 * Epilogues ESM_EPI_BIAS, ESM_EPI_BIAS_GELU and ESM_EPI_BIAS_RESIDUAL (r may
 * equal y).  N must be a multiple of 64 and K of 256; pointers 16-byte
 * aligned, b 8-byte aligned.  Errors: ESM_ERR_NULL, ESM_ERR_SHAPE,
 * ESM_ERR_UNSUPPORTED (epilogue, alignment). */
esm_status esm_linear_mxfp4_fwd(esm_encoder* enc, const void* x_codes, const void* x_scales,
                                const void* w_codes, const void* w_scales, const void* b,
                                const void* residual, void* y, int64_t M, int32_t N, int32_t K,
                                int32_t epilogue, esm_stream_t stream);

/* Row LayerNorm y = (x - mean) / sqrt(var + eps) * gamma + beta over [M, H]. */
/* Backward of a linear layer y = x W^T + b (the encoder's four linears; the
 * pages time training, [BIO-ACC] 3.2 and 6, [CARD] 训练性能):
 *   dx = dy W        [M, K]  (written when dx is not NULL; needs w)
 *   dW = dy^T x      [N, K]  (written when dw is not NULL; needs x)
 *   db = sum_m dy[m] [N]     (fp32, written when db is not NULL)
 * x bf16 [M, K], w bf16 [N, K] (as in esm_linear_fwd), dy bf16 [M, N]; dx and
 * dw bf16.  N and K multiples of 64, any M >= 0.  The two products run on the
 * library's MFMA GEMM with fp32 accumulation (dW over all M rows in fp32: for
 * large M the contraction is cut into up to 16 slices whose fp32 products are
 * summed in slice order, then rounded once);
 * W^T is written into the workspace first; the dW product reads dy and x as
 * they are (contraction-major, through gfx950's transposing LDS reads), with
 * M cut into slices of ceil(M / (64 S)) * 64 rows (rows past M count as zero);
 * db by a fixed-order two-pass column sum, so results are deterministic.  dW
 * needs M < 2^31 - 1024.  The dW path runs on a stream of the encoder's own
 * (created on first use, default priority), forked from and joined back to
 * `stream` within the call, so the call stays ordered on `stream` alone.
 * workspace: device, 256-byte aligned, at least
 * esm_linear_bwd_workspace_size(M, N, K) bytes, overwritten.  Outputs must not
 * overlap inputs or workspace.  Errors: ESM_ERR_NULL, ESM_ERR_SHAPE,
 * ESM_ERR_UNSUPPORTED (alignment: tensors 16 bytes, db 4), ESM_ERR_WORKSPACE.
 * M = 0 launches nothing and writes nothing.  Asynchronous on stream. */
esm_status esm_linear_bwd(esm_encoder* enc, const void* x, const void* w, const void* dy,
                          void* dx, void* dw, float* db, int64_t M, int32_t N, int32_t K,
                          void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Workspace bytes esm_linear_bwd needs for these sizes (host only). */
esm_status esm_linear_bwd_workspace_size(int64_t M, int32_t N, int32_t K, size_t* bytes);

/* Backward of the encoder's LayerNorm y = gamma (x - mu) r + beta per row of
 * H = hidden_size values (mu the row mean, r = 1 / sqrt(var + eps) with the
 * biased variance; the pre-LN placement of [TE-RU] and [BIO-ACC] 3.1; the
 * pages time training, [BIO-ACC] 3.2 and 6).  With xh = (x - mu) r and
 * g = dy gamma:
 *   dx = r (g - mean(g) - xh mean(g xh))   bf16 [M, H]
 *   dgamma = sum over rows of dy xh         fp32 [H]
 *   dbeta  = sum over rows of dy            fp32 [H]
 * mu and r are recomputed from x (fp32, as the forward).  x, dy bf16 [M, H],
 * gamma bf16 [H]; tensors 16-byte aligned, dgamma/dbeta 4-byte aligned.
 * workspace: device, 256-byte aligned, at least
 * esm_layernorm_bwd_workspace_size(M, H) bytes, overwritten.  Column sums in
 * a fixed order (deterministic).  dx must not overlap x or dy.  H must be a
 * multiple of 64 up to 4096 (ESM_ERR_UNSUPPORTED otherwise).  Errors:
 * ESM_ERR_NULL, ESM_ERR_SHAPE (M < 0), ESM_ERR_UNSUPPORTED, ESM_ERR_WORKSPACE.
 * M = 0 launches nothing.  Asynchronous on stream. */
esm_status esm_layernorm_bwd(esm_encoder* enc, const void* x, const void* gamma, const void* dy,
                             void* dx, float* dgamma, float* dbeta, int64_t M,
                             void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Workspace bytes esm_layernorm_bwd needs for M rows of H values (host only). */
esm_status esm_layernorm_bwd_workspace_size(int64_t M, int32_t H, size_t* bytes);

/* FP8 backward of the HYBRID recipe ([BIO-ACC] 4.1: E4M3 in the forward, E5M2
 * for the gradients).  E5M2 is the OCP format (1 sign, 5 exponent bits with
 * bias 15, 2 mantissa bits, largest finite value 57344).
 * esm_e5m2_quantize: y8[i] = cast_e5m2(x[i] * scale[0]), round to nearest
 * even, saturating at +-57344; the max of |x| is folded into *amax (fp32 bits,
 * caller-initialised).  x bf16 [n], n a multiple of 8, 16-byte aligned; y8
 * 8-byte aligned; finite inputs.
 * esm_linear_e5m2_dgrad: dx [M, K] bf16 = (dy8 / dy_scale) . (wt8 / w_scale)^T
 * for dy8 E5M2 [M, N] (the gradient of y = x W^T) and wt8 E4M3 [K, N] (W^T
 * cast with its scale): the data gradient dx = dy W on the scaled MFMA with the
 * two operands in their own FP8 formats, fp32 accumulation.  N a multiple of
 * 128, K of 64.  Errors: ESM_ERR_NULL, ESM_ERR_SHAPE, ESM_ERR_UNSUPPORTED
 * (alignment).  Asynchronous on stream. */
esm_status esm_e5m2_quantize(esm_encoder* enc, const void* x, int64_t n, const float* scale, void* y8,
                             uint32_t* amax, esm_stream_t stream);
esm_status esm_linear_e5m2_dgrad(esm_encoder* enc, const void* dy8, const float* dy_scale, const void* wt8,
                                 const float* w_scale, void* dx, int64_t M, int32_t N, int32_t K,
                                 esm_stream_t stream);

/* Weight gradient of the HYBRID recipe's backward ([BIO-ACC] 4.1: E5M2
 * gradients, E4M3 activations): dW = (dy8 / s_dy)^T (x8 / s_x), dW bf16
 * [N, K], from dy8 E5M2 codes [M, N] (esm_e5m2_quantize with scale
 * dy_scale[0]) and x8 E4M3 codes [M, K], the linear's input as the forward
 * cast it (scale x_scale[0]); both scales device fp32.  The contraction over
 * the M rows runs on the scaled MFMA (E5M2 x E4M3, fp32 accumulation) after
 * byte transposes of both operands with rows past M zero; for large M it is
 * cut into up to 16 slices whose fp32 products are summed in slice order and
 * dequantised once (deterministic).  N and K multiples of 64, any M >= 0.
 * Workspace: esm_linear_e5m2_wgrad_workspace_size bytes, 256-byte aligned.
 * ESM_ERR_NULL, ESM_ERR_SHAPE, ESM_ERR_UNSUPPORTED (alignment: tensors 16
 * bytes, scales 4), ESM_ERR_WORKSPACE.  Asynchronous on stream. */
esm_status esm_linear_e5m2_wgrad(esm_encoder* enc, const void* dy8, const float* dy_scale, const void* x8,
                                 const float* x_scale, void* dw, int64_t M, int32_t N, int32_t K,
                                 void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* Workspace bytes esm_linear_e5m2_wgrad needs for these sizes (host only). */
esm_status esm_linear_e5m2_wgrad_workspace_size(int64_t M, int32_t N, int32_t K, size_t* bytes);

/* Backward of the exact-erf GELU of fc1's epilogue ([BIO-ACC] 3.1; training
 * timed in [BIO-ACC] 3.2 and 6): dz[i] = dy[i] (Phi(z[i]) + z[i] phi(z[i]))
 * with Phi, phi the standard normal distribution and density.  z is the
 * pre-activation (x W1^T + b1, e.g. from esm_linear_fwd with ESM_EPI_BIAS),
 * dy the gradient of GELU(z); all bf16, n values, n a multiple of 8, 16-byte
 * aligned; dz may alias dy.  Errors: ESM_ERR_NULL, ESM_ERR_SHAPE,
 * ESM_ERR_UNSUPPORTED.  Asynchronous on stream. */
esm_status esm_gelu_bwd(esm_encoder* enc, const void* z, const void* dy, void* dz, int64_t n,
                        esm_stream_t stream);

/* Backward of the QKV split and the rotary embedding ([TE-ESM2] 旋转位置编码集成
 * and 权重融合技术): from dqkv, bf16 [3, heads, T, 64] (the gradients of the
 * rotated q, k and of v, as esm_attention_bwd writes them), writes dy, bf16
 * [T, 3H], the gradient of the fused QKV linear's output in its interleaved
 * column order 192 n + 64 c + j: v copied, q and k turned back by each row's
 * angle p theta_i (p the row's position in its sequence, from cu_seqlens;
 * pairs (j, j + 32): a = a' cos + b' sin, b = b' cos - a' sin), with the
 * forward's rotary table.  Runs the segment table first (workspace as
 * esm_attention_fwd).  dy must not overlap dqkv.  Errors as
 * esm_attention_fwd.  Asynchronous on stream. */
esm_status esm_qkv_rope_bwd(esm_encoder* enc, const void* dqkv, void* dy,
                            const int32_t* cu_seqlens_dev, int32_t B, int64_t T,
                            void* workspace, size_t workspace_bytes, esm_stream_t stream);

/* ------------------------------------------------------------ training layer
 *
 * One layer's forward for training and its backward from the activations the
 * forward keeps (the pages time training: [BIO-ACC] 3.2 and 6, [CARD] 训练性能;
 * the steps are those of the per-step backward entries above, chained in
 * reverse order of the forward).  bf16 encoders only (ESM_ERR_UNSUPPORTED for
 * an FP8 or MXFP4 encoder).
 *
 * Saved activations, one caller-owned device buffer of esm_layer_saved_size
 * bytes (256-byte aligned); region r starts at the offset
 * esm_layer_saved_region gives:
 *   ESM_SAVED_H1   bf16 [T, H]              LN1 output
 *   ESM_SAVED_QKV  bf16 [3, heads, T, 64]   rotated q, rotated k, v (planar)
 *   ESM_SAVED_CTX  bf16 [T, H]              attention context
 *   ESM_SAVED_LSE  fp32 [heads, T]          softmax normaliser (as esm_attention_fwd_lse)
 *   ESM_SAVED_X1   bf16 [T, H]              residual stream after the attention block
 *   ESM_SAVED_H2   bf16 [T, H]              LN2 output
 *   ESM_SAVED_Z    bf16 [T, F]              fc1 output before GELU
 *   ESM_SAVED_A    bf16 [T, F]              GELU(z), fc2's input
 * (650M widths: 38,400 bytes per residue plus 80 of lse.) */
typedef enum {
  ESM_SAVED_H1 = 0, ESM_SAVED_QKV = 1, ESM_SAVED_CTX = 2, ESM_SAVED_LSE = 3, ESM_SAVED_X1 = 4,
  ESM_SAVED_H2 = 5, ESM_SAVED_Z = 6, ESM_SAVED_A = 7, ESM_SAVED_COUNT = 8
} esm_saved_region;

/* Bytes of the saved activations of one layer for T rows (host only). */
esm_status esm_layer_saved_size(const esm_encoder* enc, int64_t T, size_t* bytes);
/* Offset and size of region r inside them (host only); ESM_ERR_SHAPE for r
 * outside [0, ESM_SAVED_COUNT). */
esm_status esm_layer_saved_region(const esm_encoder* enc, int64_t T, int32_t r, size_t* offset, size_t* bytes);

/* Training forward of layer layer_idx: x_out as esm_layer_fwd computes it,
 * except that the GELU is applied to z as stored in bf16 (the value the
 * backward differentiates at), and the activations listed above written to
 * saved.  Arguments and workspace (esm_workspace_size(T, B)) as
 * esm_layer_fwd; a layer prepared by esm_prepare_layer still runs its
 * LayerNorms as separate passes here (their outputs are saved).  The
 * backward takes x_in again: x_out may alias x_in only if the caller keeps a
 * copy.  ESM_ERR_WORKSPACE when saved is NULL, misaligned or smaller than
 * esm_layer_saved_size(T).  Asynchronous on stream. */
esm_status esm_layer_fwd_train(esm_encoder* enc, const esm_layer_weights* w, int32_t layer_idx,
                               const void* x_in, void* x_out, const int32_t* cu_seqlens_dev,
                               const int32_t* cu_seqlens_host, int32_t B, int64_t T, int32_t max_seqlen,
                               void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                               esm_stream_t stream);

/* Gradients of one layer's parameters: weights bf16 in the weights' own
 * layouts ([out, in]), biases and LayerNorm vectors fp32.  All required. */
typedef struct {
  float* ln1_gamma; float* ln1_beta;   /* [H] */
  void* w_qkv; float* b_qkv;           /* [3H, H], [3H] */
  void* w_out; float* b_out;           /* [H, H], [H] */
  float* ln2_gamma; float* ln2_beta;   /* [H] */
  void* w_fc1; float* b_fc1;           /* [F, H], [F] */
  void* w_fc2; float* b_fc2;           /* [H, F], [H] */
} esm_layer_grads;

/* Workspace bytes esm_layer_bwd needs for T rows in B sequences (host only). */
esm_status esm_layer_bwd_workspace_size(const esm_encoder* enc, int64_t T, int32_t B, size_t* bytes);

/* Backward of layer layer_idx from esm_layer_fwd_train's saved activations
 * (same T, B and cu_seqlens) and its input x_in: given dy = dL/dx_out (bf16
 * [T, H]) writes dx = dL/dx_in (bf16 [T, H]) and every parameter gradient in
 * g.  Order: fc2 (dA, dW_fc2, db_fc2), GELU (dZ at the saved z), fc1, LN2
 * (plus dy through the residual: dX1), out-projection, attention (from the
 * saved lse), the QKV split and rotary embedding, the QKV linear, LN1 (plus
 * dX1 through the residual: dx).  The residual gradients join the LayerNorm
 * gradients in fp32 and are rounded to bf16 once.  dx may alias dy.
 * Workspace: esm_layer_bwd_workspace_size(T, B) bytes, 256-byte aligned.
 * Deterministic (fixed-order sums, no atomics).  Errors as esm_layer_fwd_train
 * (ESM_ERR_NULL for a NULL gradient pointer).  Asynchronous on stream. */
esm_status esm_layer_bwd(esm_encoder* enc, const esm_layer_weights* w, int32_t layer_idx, const void* x_in,
                         const void* saved, size_t saved_bytes, const void* dy, void* dx, const esm_layer_grads* g,
                         const int32_t* cu_seqlens_dev, int32_t B, int64_t T, void* workspace,
                         size_t workspace_bytes, esm_stream_t stream);

/* ------------------------------------------------------------ training stack
 *
 * The whole stack's training forward and backward ([BIO-ACC] 6: the training
 * loop runs the model forward, then the loss's backward through every layer;
 * [BIO-ACC] 3.2 PackedEsm: the stack starts from the embedding of the packed
 * ids), built from the layer entries above: the forward keeps every layer's
 * input and saved activations (650M widths: 41,040 bytes per residue per
 * layer, 43.7 GB for 33 layers at T = 32,293: resident in HBM, no
 * recomputation), the backward runs the layers' backward in reverse and then,
 * for a stack that started from token ids, the embedding table's gradient.
 * bf16 encoders only.
 *
 * Saved activations: one caller-owned device buffer of esm_stack_saved_size
 * bytes (256-byte aligned); esm_stack_saved_layer gives, for layer l, the
 * offset of its input X_l (bf16 [T, H]) and of its saved activations (the
 * layout of esm_layer_saved_region). */
esm_status esm_stack_saved_size(const esm_encoder* enc, int64_t T, size_t* bytes);
/* ESM_ERR_SHAPE for l outside [0, num_hidden_layers). Host only. */
esm_status esm_stack_saved_layer(const esm_encoder* enc, int64_t T, int32_t l, size_t* x_offset,
                                 size_t* saved_offset);

/* Training forward of the whole stack: x_out as esm_stack_fwd computes it
 * through unprepared layers (each layer as esm_layer_fwd_train), from token
 * ids and the embedding table, or from x_in when token_ids is NULL (x_in is
 * copied into the saved buffer as X_0).  w holds num_hidden_layers weight
 * sets; workspace esm_workspace_size(T, B).  Errors as esm_layer_fwd_train.
 * Asynchronous on stream. */
esm_status esm_stack_fwd_train(esm_encoder* enc, const esm_layer_weights* w, const int32_t* token_ids,
                               const void* embedding, const void* x_in, void* x_out,
                               const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int32_t B,
                               int64_t T, int32_t max_seqlen, void* saved, size_t saved_bytes, void* workspace,
                               size_t workspace_bytes, esm_stream_t stream);

/* Workspace bytes esm_stack_bwd needs for T rows in B sequences (host only). */
esm_status esm_stack_bwd_workspace_size(const esm_encoder* enc, int64_t T, int32_t B, size_t* bytes);

/* Backward of the whole stack from esm_stack_fwd_train's saved activations
 * (same T, B, cu_seqlens): given dy = dL/dx_out (bf16 [T, H]) writes
 * dx = dL/dX_0 (bf16 [T, H]; may alias dy), the gradients of layer l into
 * g[l] (num_hidden_layers entries, as esm_layer_bwd writes them), and, when
 * token_ids is given (the forward's ids), d_embedding (fp32 [vocab, H],
 * overwritten): row v is the sum of dX_0 over the residues whose id is v
 * (ids clamped to [0, vocab) as the gather clamps them; zero for tokens
 * absent from the batch).  token_ids and d_embedding are both given or both
 * NULL (ESM_ERR_NULL otherwise); the table gradient takes vocab <= 64
 * (ESM_ERR_UNSUPPORTED above).  Deterministic.  T = 0 or B = 0: returns
 * without writing.  Errors as esm_layer_bwd.  Asynchronous on stream. */
esm_status esm_stack_bwd(esm_encoder* enc, const esm_layer_weights* w, const void* saved, size_t saved_bytes,
                         const void* dy, void* dx, const esm_layer_grads* g, const int32_t* token_ids,
                         float* d_embedding, const int32_t* cu_seqlens_dev, int32_t B, int64_t T,
                         void* workspace, size_t workspace_bytes, esm_stream_t stream);

esm_status esm_layernorm_fwd(esm_encoder* enc, const void* x, const void* gamma,
                             const void* beta, void* y, int64_t M, esm_stream_t stream);

/* The same LayerNorm with the E4M3 output that feeds an FP8 GEMM ([BIO-ACC]
 * 2.1: the LN output is an FP8 GEMM input), as a test entry: y8[m, h] =
 * cast(LN(x)[m, h] * scale[0]) (uint8 codes, [M, H]); max |LN(x)| over all M
 * rows, before the cast, is atomically maxed into *amax (device uint32, float
 * bits, caller-cleared).  x, gamma, beta bf16 as above; scale device float. */
esm_status esm_layernorm_e4m3_fwd(esm_encoder* enc, const void* x, const void* gamma,
                                  const void* beta, const float* scale, void* y8, uint32_t* amax,
                                  int64_t M, esm_stream_t stream);

/* ---------------------------------------------------------------- FP8 delayed scaling */

/* Per-tensor delayed scaling ([BIO-ACC] 2.1 and 4.1: DelayedScaling, amax
 * history, "max" algorithm; [TE-RU] FP8 recipe: history length 16).  Per layer
 * four activation tensors are tracked, in this order: LN1 output, attention
 * context, LN2 output, GELU output.  Each has a scale s (initially 1) and a
 * ring buffer of the amax (max |value| before the cast) of the last
 * amax_history_len steps (initially 0).  At the end of every step the step's
 * amax enters slot steps % history_len, steps increases, and
 * s = 448 / max(history) when that maximum is positive and finite (otherwise s
 * is kept and, if the step's amax was Inf or NaN, the sticky nonfinite flag is
 * set).  Weight scales are 448 / amax(W), fixed when the layer is prepared
 * (1 for an all-zero or non-finite weight). */
typedef struct {
  int32_t num_layers;    /* must equal the config's num_hidden_layers */
  int32_t history_len;   /* must equal the config's amax_history_len */
  float* act_scale;      /* host [num_layers, 4] */
  float* amax_history;   /* host [num_layers, 4, history_len] */
  int64_t* steps;        /* host [num_layers] */
  float* weight_scale;   /* host [num_layers, 4] (qkv, out, fc1, fc2); read by get, ignored by set */
  uint32_t nonfinite;    /* sticky flag */
} esm_fp8_state;

/* bf16 encoders: folds layer layer_idx's two LayerNorms into the linears that
 * consume them ([TE-RU] LayerNormLinear / LayerNormMLP; [BIO-ACC] 2.1, the
 * LayerNorm fused with the projection).  With h = (x - mu) r gamma + beta,
 * r = 1 / sqrt(var + eps), a linear of h is
 *   h W^T + b = r (x W'^T) - r mu c + d,  W' = gamma (.) W (per input column),
 *   c_n = sum_k W'_nk,  d_n = b_n + sum_k beta_k W_nk,
 * so the QKV and fc1 GEMMs read the raw residual stream and apply each row's
 * (mu, r) and the columns' (c, d) in their epilogue, and no LayerNorm output
 * is written.  This call computes, on the device into library-owned memory,
 * W'_qkv and W'_fc1 (bf16, the fp32 product gamma_k W_nk rounded once) and
 * (c, d) of both (fp32 from fp64 sums).  Afterwards layer layer_idx's forward
 * takes w_qkv, b_qkv, w_fc1, b_fc1 and the four LayerNorm vectors from this
 * copy (the pointers in w are still checked); call again whenever any of
 * them changes.  Layers never prepared run LayerNorm as a separate pass.
 * Enqueued on stream.  ESM_ERR_STATE for an FP8 or MXFP4 encoder (their
 * LayerNorms write the quantised GEMM input). */
esm_status esm_prepare_layer(esm_encoder* enc, int32_t layer_idx, const esm_layer_weights* w,
                             esm_stream_t stream);

/* Casts layer layer_idx's four linear weights (bf16 in w) to E4M3 copies owned
 * by the library, each with scale 448 / amax(W) computed on the device.
 * Enqueued on stream; call again whenever the weights change.  In an MXFP4
 * encoder the first call creates the FP8 state and E4M3 weight store
 * (synchronous allocation; ESM_ERR_UNSUPPORTED unless hidden_size and
 * intermediate_size are multiples of 128).  ESM_ERR_STATE for a bf16
 * encoder. */
esm_status esm_fp8_prepare_layer(esm_encoder* enc, int32_t layer_idx, const esm_layer_weights* w,
                                 esm_stream_t stream);

/* The FP8 state functions below need an encoder holding the delayed-scaling
 * state: an FP8 encoder, or an MXFP4 encoder given an FP8 layer (by
 * esm_set_layer_precision or esm_fp8_prepare_layer); ESM_ERR_STATE otherwise.
 *
 * Copies the state into the caller's host arrays after waiting for stream. */
esm_status esm_fp8_get_state(esm_encoder* enc, esm_fp8_state* state, esm_stream_t stream);

/* Replaces the state (scales must be positive and finite; steps >= 0) after
 * waiting for stream, and clears the amax of the current step. */
esm_status esm_fp8_set_state(esm_encoder* enc, const esm_fp8_state* state, esm_stream_t stream);

/* Back to the initial state (scales 1, empty histories, steps 0, flag clear);
 * prepared weights and per-layer precisions are kept. */
esm_status esm_fp8_reset(esm_encoder* enc, esm_stream_t stream);

/* Gradient scaling of the HYBRID recipe ([BIO-ACC] 4.1: E5M2 for the
 * backward's gradients; [TE-RU] Рецепт FP8: Delayed Scaling).  Beside the
 * forward's state each layer keeps, for four gradient tensors -- slot 0 the
 * output gradient of the QKV linear, 1 of the out-projection, 2 of fc1, 3 of
 * fc2 (the layer's output gradient) -- a scale (initially 1), the amax of the
 * current backward step and a history of history_len steps, with the
 * forward's window rule and E5M2's largest finite value: at the end of a step
 * the step's amax enters slot steps % history_len and the scale becomes
 * 57344 / max(history) when that is positive and finite (else it is kept; a
 * non-finite amax sets the state's sticky flag).  esm_fp8_reset clears it with
 * the rest of the state.  All need an encoder holding the FP8 state
 * (ESM_ERR_STATE otherwise); layer_idx outside [0, num_hidden_layers) or slot
 * outside [0, 4): ESM_ERR_SHAPE.
 *
 * esm_fp8_grad_quantize: y8 = cast_e5m2(g * scale) with the slot's current
 * scale (g bf16, n values, a multiple of 8; y8 uint8 codes, 8-byte aligned);
 * max |g| is folded into the slot's amax of this step; the scale used is also
 * written to *scale_out (device fp32, may be NULL), the dy_scale that
 * esm_linear_e5m2_dgrad and esm_linear_e5m2_wgrad take.  Asynchronous. */
esm_status esm_fp8_grad_quantize(esm_encoder* enc, int32_t layer_idx, int32_t slot, const void* g, int64_t n,
                                 void* y8, float* scale_out, esm_stream_t stream);

/* End of layer layer_idx's backward step: rolls its four gradient histories
 * and sets their next scales.  Asynchronous. */
esm_status esm_fp8_grad_step(esm_encoder* enc, int32_t layer_idx, esm_stream_t stream);

/* Copies the gradient state into host arrays after waiting for stream: scale
 * [num_layers, 4], history [num_layers, 4, history_len] (ring order: step s in
 * slot s % history_len), steps [num_layers]. */
esm_status esm_fp8_grad_get_state(esm_encoder* enc, float* scale, float* history, int64_t* steps,
                                  esm_stream_t stream);

/* MXFP4 weights of layer layer_idx ([TE-ESM2] FP8与FP4混合精度支持, read as
 * OCP MXFP4): the four linear weights of w quantised per 32-value block along
 * K (esm_mxfp4_quantize) into library-owned memory, asynchronously on stream.
 * In an FP8 encoder the first call creates the MXFP4 weight store
 * (synchronous allocation; ESM_ERR_UNSUPPORTED unless the MXFP4 shape rule of
 * esm_layer_fwd holds).  ESM_ERR_STATE for a bf16 encoder; ESM_ERR_SHAPE for
 * layer_idx outside [0, num_hidden_layers). */
esm_status esm_mxfp4_prepare_layer(esm_encoder* enc, int32_t layer_idx, const esm_layer_weights* w,
                                   esm_stream_t stream);

/* Per-layer precision of an FP8 or MXFP4 encoder ([TE-ESM2] FP8与FP4混合精度支持:
 * the encoder takes an FP8 and an FP4 recipe and a per-layer precision list):
 * precision[l] (host, num_layers entries) is ESM_PRECISION_FP8_DELAYED,
 * ESM_PRECISION_MXFP4 or ESM_PRECISION_BF16, in any mix; the default of every
 * layer is the encoder's own precision.  A layer needs weights prepared in its
 * format (esm_fp8_prepare_layer / esm_mxfp4_prepare_layer) before it runs,
 * else the forward returns ESM_ERR_STATE; a bf16 layer runs the bf16 kernels
 * and needs none.  Only FP8 layers record amax and step their delayed-scaling
 * state; a layer that is not FP8 keeps its FP8 state (scales, history, step
 * count) as it is until it runs FP8 again.  The first FP8 layer of an MXFP4
 * encoder creates the FP8 state.  Waits for stream.  ESM_ERR_STATE for an
 * encoder created with bf16 precision; ESM_ERR_SHAPE when num_layers is not
 * the config's; ESM_ERR_UNSUPPORTED for another precision code or when the
 * shape rule of a requested format (esm_layer_fwd) does not hold. */
esm_status esm_set_layer_precision(esm_encoder* enc, const int32_t* precision, int32_t num_layers,
                                   esm_stream_t stream);

/* The E4M3 cast the producers use, as a test entry: y[i] = cast(x[i] *
 * scale[0]) for fp32 x (device, n values), y uint8 codes; max |x| is
 * atomically maxed into *amax (device uint32, float bits, caller-cleared). */
esm_status esm_fp8_quantize(esm_encoder* enc, const float* x, int64_t n, const float* scale,
                            void* y, uint32_t* amax, esm_stream_t stream);

/* ---------------------------------------------------------------- timing */

/* Kernel classes timed when profiling is on. */
typedef enum {
  ESM_K_SEGMENT = 0, ESM_K_EMBED = 1, ESM_K_LAYERNORM = 2, ESM_K_GEMM_QKV = 3,
  ESM_K_ATTENTION = 4, ESM_K_GEMM_OUT = 5, ESM_K_GEMM_FC1 = 6, ESM_K_GEMM_FC2 = 7,
  ESM_K_OTHER = 8, ESM_K_FP8 = 9 /* weight casts, scale updates */,
  ESM_K_HEAD = 10 /* final LayerNorm, LM head, sequence means */,
  ESM_K_BIASED_ATTENTION = 11 /* esm_biased_attention_fwd */,
  ESM_K_ATTENTION_BWD = 12 /* esm_attention_bwd */,
  ESM_K_LINEAR_BWD = 13 /* esm_linear_bwd, esm_layernorm_bwd, esm_gelu_bwd, esm_qkv_rope_bwd */,
  ESM_K_COUNT = 14
} esm_kernel_class;

/* Matrix-core rate probe, for measuring the achievable bf16 MFMA rate of the
 * device beside the spec peak: two workgroups of four waves per compute unit,
 * each wave issuing 16 * iters v_mfma_f32_32x32x16_bf16 on register operands
 * that change every instruction (pseudo-random bf16 in [-2, 2)), nothing
 * else in the loop.  *flops receives the flop count of the launch (time it
 * with events on stream).  sink: device buffer of at least
 * 16 * (compute units) * 2 floats; ESM_ERR_WORKSPACE if smaller. */
esm_status esm_mfma_peak(esm_encoder* enc, int32_t iters, void* sink, size_t sink_bytes, double* flops,
                         esm_stream_t stream);

/* When on, every launch is bracketed by HIP events recorded on the launch
 * stream, and durations are summed per kernel class.  Turning it on clears the
 * sums.  Adds two event records per launch. */
esm_status esm_profile_enable(esm_encoder* enc, int32_t on);

/* Waits for the recorded events and returns, per class, the summed kernel time
 * in milliseconds and the number of launches (arrays of ESM_K_COUNT). */
esm_status esm_profile_read(esm_encoder* enc, double* ms_out, int64_t* launches_out);

/* ---------------------------------------------------------------- host-only helpers */

/* Host check of a cu_seqlens array (no device work): cu[0] = 0, non-decreasing,
 * cu[B] = T, every length <= max_seqlen, max_seqlen <= max_positions. */
esm_status esm_check_cu_seqlens(const int32_t* cu_host, int32_t B, int64_t T,
                                int32_t max_seqlen, int32_t max_positions);

/* Host check of padded lengths: 0 <= seqlens[b] <= S <= max_positions. */
esm_status esm_check_seqlens(const int32_t* seqlens_host, int32_t B, int32_t S,
                             int32_t max_positions);

/* Message of the last failing call on this host thread ("" if none). */
const char* esm_last_error(void);
const char* esm_status_str(esm_status s);
int32_t esm_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ESM_ENCODER_H */
