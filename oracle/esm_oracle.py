"""Plain fp64 CPU oracle of the ESM-2 encoder forward.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module.  It shares no code with the HIP path and
imports nothing from the product package: every input arrives as an array.

What is computed, and where the pages define it
-----------------------------------------------
Pages cited (title, section):
  [TE-ESM2]  "深入源码NVIDIA ESM-2 TransformerEngine优化的实现原理与技术细节"
             (mlqm.cn), sections 核心技术架构设计, 旋转位置编码集成, 注意力掩码优化,
             权重融合技术, 序列长度优化, 自动混合精度训练
  [BIO-ACC]  "生物大模型训练加速实战：基于PyTorch与NVIDIA BioNeMo的Transformer优化指南"
             (hotelren.com), sections 2.1, 3.1, 3.2
  [CARD]     "ESM-2", BioNeMo framework model card (docs.nvda.net.cn), sections
             模型概述/描述, 输入, 输出
  [TE-RU]    Russian summary of the TransformerEngine tutorial (aikraft.ru),
             section "Ключевые компоненты и Fused Kernels"
  [DS4SCI]   "DeepSpeed4Science 深度解读以 AI 系统优化技术驱动大规模科学发现"
             (mhpn.cn), sections 3.2 and 5.3 (biased attention only)

* Encoder = stack of BERT-style bidirectional Transformer layers ([CARD] 描述;
  [TE-ESM2] 核心技术架构设计).  Each layer has self-attention, LayerNorm and two
  linears fc1/fc2 ([BIO-ACC] 3.1); LayerNorm is applied to the input of the
  QKV linear and of the MLP (LayerNormLinear / LayerNormMLP, [TE-RU]), i.e.
  pre-LN, with a residual add after attention and after the MLP.
* The packed (THD) batch is described by cu_seqlens = cumsum([0] + lengths);
  sequence s owns rows cu[s] .. cu[s+1]-1 ([BIO-ACC] 3.2, collate_fn and
  PackedEsm.forward).  Attention never crosses a sequence boundary.
* Rotary position embedding on head_dim = hidden / heads ([TE-ESM2]
  旋转位置编码集成).  Positions restart at 0 in every sequence.
* Q, K, V come from one fused, per-head interleaved weight ([TE-ESM2] 权重融合技术).
* Padded layout: bshd rows with a padding mask ([TE-ESM2] 注意力掩码优化).

Readings where the pages are silent (each is listed in the design notes):
  pre-LN; LayerNorm eps 1e-5 with the biased (1/H) variance; FFN width 4H with
  biases on all four linears; interleaved rows 192*n + 64*c + j (c = q, k, v);
  RoPE base 10000 with rotate-half pairing (i, i+32), applied after the QKV
  bias to q and k only; softmax scale 1/sqrt(64) = 1/8; exact-erf GELU; no
  dropout; no final LayerNorm inside the stack; X0 = E[ids].  After the
  stack (head_forward): final LayerNorm, the ESM-2 masked-LM head with the
  decoder tied to the embedding, and per-sequence mean embeddings.

linear_bwd and layer_norm_bwd give the gradients of a linear layer (dx, dW,
db) and of a LayerNorm (dx, dgamma, dbeta); gelu_bwd, rope_bwd and
qkv_rope_bwd those of GELU, of the rotary embedding and of the QKV split;
layer_backward chains them through one whole layer.
attention_lse and attention_bwd give the softmax normaliser a backward pass
keeps and the gradients of the attention with respect to q, k and v: the
backward of the training runs the pages time ([BIO-ACC] 3.2 and 6, [CARD]
训练性能).

A second, separate function, biased_attention, is the Evoformer attention of
[DS4SCI]: softmax(q k^T / sqrt(D) + mask bias + pair bias) v per (b, n, h) on
[B, N, L, H, D] tensors (the scale is a reading; the page does not state it).

Everything is evaluated densely in float64 on bf16-valued inputs, per sequence
and per head, with an exact max-subtracted softmax.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

HEAD_DIM = 64
LN_EPS = 1e-5
ROPE_BASE = 10000.0
SOFTMAX_SCALE = 1.0 / math.sqrt(HEAD_DIM)   # = 0.125 exactly


def bf16_to_f64(bits) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def weights_to_f64(w: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """bf16 bit-pattern dict -> float64 dict (missing biases become zeros)."""
    out = {k: (bf16_to_f64(v) if np.asarray(v).dtype == np.uint16 else np.asarray(v, np.float64))
           for k, v in w.items() if v is not None}
    return out


# --------------------------------------------------------------------------
# Segments ([BIO-ACC] 3.2)
# --------------------------------------------------------------------------

def segments(cu_seqlens) -> List[tuple]:
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    return [(cu[s], cu[s + 1]) for s in range(len(cu) - 1)]


def positions(cu_seqlens) -> np.ndarray:
    """Position of every packed row inside its own sequence: p = t - cu[s]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    pos = np.empty(T, dtype=np.int64)
    for a, b in segments(cu):
        pos[a:b] = np.arange(b - a)
    return pos


# --------------------------------------------------------------------------
# Elementwise pieces
# --------------------------------------------------------------------------

def layer_norm(x, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """Row LayerNorm: (x - mean) / sqrt(var + eps) * gamma + beta, biased var."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def gelu(z) -> np.ndarray:
    """Exact GELU: z * Phi(z) = 0.5 * z * (1 + erf(z / sqrt(2)))."""
    z = np.asarray(z, np.float64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def rope_angles(pos, dim: int = HEAD_DIM, base: float = ROPE_BASE) -> np.ndarray:
    """theta[p, i] = p * base^(-i/(dim/2)) for i < dim/2."""
    half = dim // 2
    inv = base ** (-np.arange(half, dtype=np.float64) / half)
    return np.asarray(pos, np.float64)[:, None] * inv[None, :]


def apply_rope(u, pos, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate-half RoPE on the last axis (size 64) of u[T, ..., 64].

    For each pair (a, b) = (u_i, u_{i+32}):  a' = a cos - b sin,  b' = b cos + a sin."""
    u = np.asarray(u, np.float64)
    dim = u.shape[-1]
    half = dim // 2
    th = rope_angles(pos, dim, base)
    shape = (u.shape[0],) + (1,) * (u.ndim - 2) + (half,)
    c = np.cos(th).reshape(shape)
    s = np.sin(th).reshape(shape)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def split_qkv(y, heads: int):
    """Interleaved fused QKV output y[T, 3H] -> q, k, v each [T, heads, 64].

    Column 192*n + 64*c + j is component c (q, k, v) of head n, dim j."""
    T = y.shape[0]
    y = np.asarray(y).reshape(T, heads, 3, HEAD_DIM)
    return y[:, :, 0, :], y[:, :, 1, :], y[:, :, 2, :]


def pack_qkv_weight(wq, wk, wv, heads: int) -> np.ndarray:
    """Separate [H, H] query/key/value weights -> the interleaved [3H, H] fused weight."""
    H = wq.shape[1]
    parts = [w.reshape(heads, HEAD_DIM, H) for w in (wq, wk, wv)]
    return np.stack(parts, axis=1).reshape(3 * heads * HEAD_DIM, H)


# --------------------------------------------------------------------------
# Attention ([CARD] bidirectional encoder; [BIO-ACC] 3.2 segments)
# --------------------------------------------------------------------------

def softmax_rows(S) -> np.ndarray:
    S = np.asarray(S, np.float64)
    m = S.max(axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_probs(q, k, scale: float = SOFTMAX_SCALE) -> np.ndarray:
    """P = softmax(q k^T * scale) for one (sequence, head): q, k are [L, 64]."""
    return softmax_rows((np.asarray(q) @ np.asarray(k).T) * scale)


def attention(q, k, v, cu_seqlens, scale: float = SOFTMAX_SCALE) -> np.ndarray:
    """Non-causal attention inside each segment; q, k, v are [T, heads, 64] -> ctx [T, heads*64]."""
    T, heads, d = q.shape
    ctx = np.zeros((T, heads, d), np.float64)
    for a, b in segments(cu_seqlens):
        if b == a:
            continue
        for n in range(heads):
            P = attention_probs(q[a:b, n], k[a:b, n], scale)
            ctx[a:b, n] = P @ v[a:b, n]
    return ctx.reshape(T, heads * d)


def attention_lse(q, k, cu_seqlens, scale: float = SOFTMAX_SCALE) -> np.ndarray:
    """Natural-log softmax normaliser of every row: lse[n, t] =
    log sum_j exp(scale q_t . k_j) over the keys j of t's sequence; q, k
    [T, heads, 64] -> [heads, T].  Evaluated as max + log(sum exp(s - max))."""
    T, heads, _ = q.shape
    lse = np.zeros((heads, T), np.float64)
    for a, b in segments(cu_seqlens):
        if b == a:          # an empty sequence has no rows
            continue
        for n in range(heads):
            S = (q[a:b, n] @ k[a:b, n].T) * scale
            m = S.max(axis=1)
            lse[n, a:b] = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    return lse


def attention_bwd(q, k, v, dctx, cu_seqlens, scale: float = SOFTMAX_SCALE):
    """Gradients of sum(dctx * attention(q, k, v)) with respect to q, k and v
    (the backward pass of the training runs the pages time: [BIO-ACC] 3.2 and 6,
    [CARD] 训练性能; written
    out by the chain rule on the forward above).  Per (sequence, head), with
    S = scale q k^T, P = softmax_rows(S), O = P v and dO the incoming gradient:
        dv = P^T dO
        dP = dO v^T
        dS = P * (dP - rowsum(P * dP))          (softmax Jacobian, row by row)
        dq = scale dS k,   dk = scale dS^T q.
    q, k, v [T, heads, 64], dctx [T, heads * 64] -> dq, dk, dv [T, heads, 64]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, heads, d = q.shape
    dO = np.asarray(dctx, np.float64).reshape(T, heads, d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for a, b in segments(cu_seqlens):
        if b == a:          # an empty sequence has no rows
            continue
        for n in range(heads):
            P = attention_probs(q[a:b, n], k[a:b, n], scale)
            g = dO[a:b, n]
            dv[a:b, n] = P.T @ g
            dP = g @ v[a:b, n].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[a:b, n] = scale * (dS @ k[a:b, n])
            dk[a:b, n] = scale * (dS.T @ q[a:b, n])
    return dq, dk, dv


def layer_norm_bwd(x, gamma, dy, eps: float = LN_EPS):
    """Gradients of sum(dy * layer_norm(x, gamma, beta)) with respect to x,
    gamma and beta (the backward of the pre-LN LayerNorms, [TE-RU] and
    [BIO-ACC] 3.1; training timed in [BIO-ACC] 3.2 and 6).  Per row, with the
    forward's mean mu, biased variance var, r = 1 / sqrt(var + eps),
    xh = (x - mu) r and g = dy * gamma:
        dx = r (g - mean(g) - xh mean(g xh)),
        dgamma = sum over rows of dy xh,   dbeta = sum over rows of dy."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    gamma = np.asarray(gamma, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    xh = (x - mu) * r
    g = dy * gamma
    dx = r * (g - g.mean(axis=-1, keepdims=True) - xh * (g * xh).mean(axis=-1, keepdims=True))
    return dx, (dy * xh).sum(axis=0), dy.sum(axis=0)


def gelu_bwd(z, dy) -> np.ndarray:
    """dz = dy * GELU'(z) with GELU'(z) = Phi(z) + z phi(z) (the derivative of
    the exact-erf GELU above; phi the standard normal density)."""
    z = np.asarray(z, np.float64)
    phi = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return np.asarray(dy, np.float64) * (0.5 * (1.0 + _erf(z / math.sqrt(2.0))) + z * phi)


def rope_bwd(du, pos, base: float = ROPE_BASE) -> np.ndarray:
    """Gradient through apply_rope: each pair is rotated by -theta (the
    rotation's transpose): a = a' cos + b' sin, b = b' cos - a' sin."""
    return apply_rope(du, -np.asarray(pos, np.float64), base)


def qkv_rope_bwd(dq, dk, dv, cu_seqlens, base: float = ROPE_BASE) -> np.ndarray:
    """Gradient of the QKV linear's output y [T, 3H] (interleaved columns
    192 n + 64 c + j, c = q, k, v) from the gradients of the rotated q, k
    and of v, each [T, heads, 64]: the inverse of split_qkv after undoing the
    rotation of q and k at every row's position."""
    pos = positions(cu_seqlens)
    parts = [rope_bwd(dq, pos, base), rope_bwd(dk, pos, base), np.asarray(dv, np.float64)]
    T, heads, d = parts[0].shape
    return np.stack(parts, axis=2).reshape(T, heads * 3 * d)


def linear_bwd(x, w, dy):
    """Gradients of sum(dy * (x w^T + b)) for x [M, K], w [N, K], dy [M, N]
    (the backward of the encoder's linears, [BIO-ACC] 3.1; training timed in
    [BIO-ACC] 3.2 and 6): dx = dy w [M, K], dw = dy^T x [N, K], db = the
    column sums of dy [N]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    dy = np.asarray(dy, np.float64)
    return dy @ w, dy.T @ x, dy.sum(axis=0)


# --------------------------------------------------------------------------
# One layer, stack
# --------------------------------------------------------------------------

def _bias(w, name, n):
    b = w.get(name)
    return np.zeros(n) if b is None else b


def layer_forward(x, cu_seqlens, w: Dict[str, np.ndarray], heads: int,
                  eps: float = LN_EPS, base: float = ROPE_BASE,
                  return_intermediates: bool = False):
    """One pre-LN encoder layer over a packed [T, H] batch (float64 weights)."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    assert H == heads * HEAD_DIM
    F = w["w_fc1"].shape[0]
    h1 = layer_norm(x, w["ln1_gamma"], w["ln1_beta"], eps)
    y = h1 @ w["w_qkv"].T + _bias(w, "b_qkv", 3 * H)
    q, k, v = split_qkv(y, heads)
    pos = positions(cu_seqlens)
    qr = apply_rope(q, pos, base)
    kr = apply_rope(k, pos, base)
    ctx = attention(qr, kr, v, cu_seqlens)
    x1 = x + ctx @ w["w_out"].T + _bias(w, "b_out", H)
    h2 = layer_norm(x1, w["ln2_gamma"], w["ln2_beta"], eps)
    a = gelu(h2 @ w["w_fc1"].T + _bias(w, "b_fc1", F))
    x2 = x1 + a @ w["w_fc2"].T + _bias(w, "b_fc2", H)
    if return_intermediates:
        return x2, dict(h1=h1, q=qr, k=kr, v=v, ctx=ctx, x1=x1, h2=h2, a=a)
    return x2


def layer_backward(x, cu_seqlens, w: Dict[str, np.ndarray], heads: int, dout,
                   eps: float = LN_EPS, base: float = ROPE_BASE):
    """Gradients of sum(dout * layer_forward(x)) with respect to x and every
    weight, by the chain rule through the layer's steps in reverse, each step
    the backward above (linear_bwd, gelu_bwd, layer_norm_bwd, attention_bwd,
    qkv_rope_bwd; the residual adds pass the gradient through).  Returns
    (dx [T, H], {name: gradient} with the names of w)."""
    x = np.asarray(x, np.float64)
    dout = np.asarray(dout, np.float64)
    T, H = x.shape
    F = w["w_fc1"].shape[0]
    _, im = layer_forward(x, cu_seqlens, w, heads, eps, base, return_intermediates=True)
    z = im["h2"] @ w["w_fc1"].T + _bias(w, "b_fc1", F)
    g = {}
    da, g["w_fc2"], g["b_fc2"] = linear_bwd(im["a"], w["w_fc2"], dout)
    dh2, g["w_fc1"], g["b_fc1"] = linear_bwd(im["h2"], w["w_fc1"], gelu_bwd(z, da))
    dx1_ln, g["ln2_gamma"], g["ln2_beta"] = layer_norm_bwd(im["x1"], w["ln2_gamma"], dh2, eps)
    dx1 = dout + dx1_ln
    dctx, g["w_out"], g["b_out"] = linear_bwd(im["ctx"], w["w_out"], dx1)
    dq, dk, dv = attention_bwd(im["q"], im["k"], im["v"], dctx, cu_seqlens)
    dh1, g["w_qkv"], g["b_qkv"] = linear_bwd(im["h1"], w["w_qkv"], qkv_rope_bwd(dq, dk, dv, cu_seqlens, base))
    dx_ln, g["ln1_gamma"], g["ln1_beta"] = layer_norm_bwd(x, w["ln1_gamma"], dh1, eps)
    return dx1 + dx_ln, g


def layer_forward_seqs(x, cu_seqlens, w, heads: int, seqs: Sequence[int], **kw):
    """Layer output for a subset of sequences only (rows of those sequences, in order).

    Sequences are independent, so this equals the matching rows of the full
    layer_forward; it lets large batches be checked on a sample."""
    cu = np.asarray(cu_seqlens, np.int64)
    parts, lens = [], []
    for s in seqs:
        a, b = int(cu[s]), int(cu[s + 1])
        parts.append(np.asarray(x[a:b], np.float64))
        lens.append(b - a)
    sub_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return layer_forward(np.concatenate(parts, axis=0), sub_cu, w, heads, **kw), sub_cu


def embed(ids, table) -> np.ndarray:
    """X0 = E[ids] ([BIO-ACC] 3.2, PackedEsm.forward)."""
    return np.asarray(table, np.float64)[np.asarray(ids, np.int64)]


def stack_forward(cu_seqlens, layers: List[Dict[str, np.ndarray]], heads: int,
                  ids=None, table=None, x=None, **kw) -> np.ndarray:
    """Embedding (when ids are given) then every layer in order; no final LayerNorm."""
    h = embed(ids, table) if ids is not None else np.asarray(x, np.float64)
    for w in layers:
        h = layer_forward(h, cu_seqlens, w, heads, **kw)
    return h


def embed_backward(ids, dx0, vocab: int) -> np.ndarray:
    """Gradient of the embedding table under X0 = E[ids]: each table row
    collects the gradients of the residues that gathered it, zero for tokens
    the batch does not hold."""
    d = np.zeros((vocab, np.asarray(dx0).shape[1]))
    np.add.at(d, np.asarray(ids, np.int64), np.asarray(dx0, np.float64))
    return d


def stack_backward(cu_seqlens, layers: List[Dict[str, np.ndarray]], heads: int, dout,
                   ids=None, table=None, x=None, **kw):
    """Gradients of sum(dout * stack_forward(...)) by the chain rule: the
    layers' backward in reverse order, each at the input the forward gave it,
    then the embedding's when the stack starts from token ids.  Returns
    (gradient of the stack input X0, [per-layer gradients as layer_backward
    names them], table gradient or None)."""
    h = embed(ids, table) if ids is not None else np.asarray(x, np.float64)
    inputs = []
    for w in layers:
        inputs.append(h)
        h = layer_forward(h, cu_seqlens, w, heads, **kw)
    g = np.asarray(dout, np.float64)
    grads = [None] * len(layers)
    for l in reversed(range(len(layers))):
        g, grads[l] = layer_backward(inputs[l], cu_seqlens, layers[l], heads, g, **kw)
    d_table = embed_backward(ids, g, np.asarray(table).shape[0]) if ids is not None else None
    return g, grads, d_table


# --------------------------------------------------------------------------
# After the stack: final LayerNorm, masked-LM head, sequence-level embedding
# --------------------------------------------------------------------------
# The model card lists per-residue and sequence-level embeddings as the outputs
# ([CARD] 输出), and the usage section loads the model as a masked-LM
# ([TE-ESM2] 快速开始使用).  The pages define neither head; the readings used
# here are ESM-2's published ones: a final LayerNorm after the last layer; the
# LM head dense(H -> H) + bias, exact GELU, LayerNorm, then a decoder whose
# weight is the token embedding [vocab, H] plus a bias; the sequence-level
# embedding is the mean of the sequence's final representations (zeros for an
# empty sequence).

def lm_head(x, w: Dict[str, np.ndarray], eps: float = LN_EPS) -> np.ndarray:
    """Masked-LM logits [T, vocab] of final representations x [T, H]."""
    x = np.asarray(x, np.float64)
    h = gelu(x @ np.asarray(w["lm_dense_w"], np.float64).T + np.asarray(w["lm_dense_b"], np.float64))
    h = layer_norm(h, w["lm_ln_gamma"], w["lm_ln_beta"], eps)
    return h @ np.asarray(w["embedding"], np.float64).T + np.asarray(w["lm_decoder_b"], np.float64)


def sequence_means(x, cu_seqlens) -> np.ndarray:
    """Mean over each sequence's rows of x [T, H] -> [B, H]; zeros for an empty sequence."""
    x = np.asarray(x, np.float64)
    segs = segments(cu_seqlens)
    out = np.zeros((len(segs), x.shape[1]))
    for s, (a, b) in enumerate(segs):
        if b > a:
            out[s] = x[a:b].mean(axis=0)
    return out


def head_forward(x, cu_seqlens, w: Dict[str, np.ndarray], eps: float = LN_EPS):
    """Stack output x [T, H] -> (final representations [T, H], logits [T, vocab],
    sequence embeddings [B, H])."""
    final = layer_norm(x, w["final_ln_gamma"], w["final_ln_beta"], eps)
    return final, lm_head(final, w, eps), sequence_means(final, cu_seqlens)


def layer_forward_bshd(x, seqlens, w, heads: int, **kw) -> np.ndarray:
    """Padded layout x[B, S, H] with right-padded valid prefixes of length seqlens[b].

    Rows at or beyond seqlens[b] are unspecified: they are returned as NaN so a
    comparison can never count them."""
    x = np.asarray(x, np.float64)
    B, S, H = x.shape
    out = np.full_like(x, np.nan)
    for b in range(B):
        L = int(seqlens[b])
        if L == 0:
            continue
        out[b, :L] = layer_forward(x[b, :L], np.array([0, L]), w, heads, **kw)
    return out


# --------------------------------------------------------------------------
# Segment table (integer work): which attention query tiles exist
# --------------------------------------------------------------------------

def query_tiles(lengths, tile_rows: int) -> List[tuple]:
    """All (sequence, first query row) pairs of a sequence cut into tiles of
    tile_rows rows, longest sequence first and, among equal lengths, in
    sequence order (any order of equal lengths is equally valid)."""
    lengths = [int(L) for L in lengths]
    order = sorted(range(len(lengths)), key=lambda s: (-lengths[s], s))
    out = []
    for s in order:
        for q0 in range(0, lengths[s], tile_rows):
            out.append((s, q0))
    return out


# --------------------------------------------------------------------------
# Metrics
# --------------------------------------------------------------------------

def rel_max_err(got, ref) -> float:
    """max|got - ref| / max|ref| over finite reference entries."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.isfinite(ref)
    den = np.abs(ref[m]).max()
    return float(np.abs(got[m] - ref[m]).max() / den) if den > 0 else float(np.abs(got[m]).max())


def param_count(hidden: int, ffn: int, layers: int, vocab: int = 33) -> int:
    """Parameters of the layer definition used here: per layer 4 linears with
    biases (QKV 3H*H, out H*H, fc1 F*H, fc2 H*F) and two LayerNorms, plus the
    embedding table."""
    H, F = hidden, ffn
    per_layer = (3 * H * H + 3 * H) + (H * H + H) + (F * H + F) + (H * F + H) + 4 * H
    return layers * per_layer + vocab * H


# --------------------------------------------------------------------------
# Biased attention (the Evoformer-style kernel of the DeepSpeed4Science page)
# --------------------------------------------------------------------------
# [DS4SCI] "DeepSpeed4Science 深度解读以 AI 系统优化技术驱动大规模科学发现"
# (mhpn.cn), sections 3.2 and 5.3: Q, K, V are [B, N, L, H, D]; up to two
# additive biases shaped [B, N, 1, 1, L] (a per-key mask bias) and
# [B, 1, H, L, L] (a pair bias shared by the N rows) are added to the scores
# before the softmax.  The page leaves the score scale unstated; the reading
# used is 1/sqrt(D), as in the encoder.

def biased_attention(q, k, v, biases=(), scale: Optional[float] = None) -> np.ndarray:
    """softmax(q k^T * scale + sum(biases)) v per (b, n, h); q, k, v [B, N, L, H, D]."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    s = np.einsum("bnqhd,bnkhd->bnhqk", q, k) * scale
    for b in biases:
        s = s + np.asarray(b, np.float64)          # broadcast [B,N,1,1,L] or [B,1,H,L,L]
    m = s.max(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        p = np.exp(s - m)
        p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("bnhqk,bnkhd->bnqhd", p, v)
