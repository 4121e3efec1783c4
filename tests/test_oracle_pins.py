"""Pins of the oracle pieces every stack, sampled-layer, FP8 and MXFP4 parity
test relies on, each against something other than the function's own
formula:

* bf16_to_f64 against torch's independent bfloat16 decode;
* embed against a one-hot matrix product;
* layer_forward_seqs against the matching rows of layer_forward;
* stack_forward against two layers composed by hand;
* the FP8-emulating layer (fp8_ref.layer_forward_fp8): every one of the
  eight casts (four GEMM inputs, four weights) is shown to be applied, to
  the right tensor and with the right scale -- a dropped or misplaced cast
  fails one of these checks;
* the MXFP4-emulating layer (fp4_ref.layer_forward_mxfp4): the same for its
  eight block quantisations, and one MXFP4 block product worked by hand.

Quantisation readings (the pages name the recipes only): [BIO-ACC] 4.1 and
[TE-RU] "Рецепт FP8: Delayed Scaling" for E4M3 with per-tensor scales;
[TE-ESM2] FP8与FP4混合精度支持 for the FP4 recipe, read as OCP MXFP4.
"""
import math

import numpy as np
import pytest

from oracle import esm_oracle as O
from oracle import fp4_ref as F4
from oracle import fp8_ref as F8


# ---------------------------------------------------------------- plain pieces

def test_bf16_to_f64_matches_torch_on_every_pattern():
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities come through as such
    assert math.copysign(1.0, O.bf16_to_f64([0x8000])[0]) == -1.0
    assert O.bf16_to_f64([0x7F80, 0xFF80]).tolist() == [math.inf, -math.inf]


def test_embed_is_a_one_hot_product():
    r = np.random.default_rng(3)
    vocab, H, T = 33, 48, 200
    table = r.standard_normal((vocab, H))
    ids = r.integers(0, vocab, T)
    onehot = np.zeros((T, vocab))
    onehot[np.arange(T), ids] = 1.0
    assert np.array_equal(O.embed(ids, table), onehot @ table)


def _plain_weights(r, H, F, scale=0.08, random_ln=True):
    w = {"w_qkv": r.standard_normal((3 * H, H)) * scale, "b_qkv": r.standard_normal(3 * H) * scale,
         "w_out": r.standard_normal((H, H)) * scale, "b_out": r.standard_normal(H) * scale,
         "w_fc1": r.standard_normal((F, H)) * scale, "b_fc1": r.standard_normal(F) * scale,
         "w_fc2": r.standard_normal((H, F)) * scale, "b_fc2": r.standard_normal(H) * scale}
    if random_ln:
        w.update(ln1_gamma=1 + 0.2 * r.standard_normal(H), ln1_beta=0.1 * r.standard_normal(H),
                 ln2_gamma=1 + 0.2 * r.standard_normal(H), ln2_beta=0.1 * r.standard_normal(H))
    else:
        w.update(ln1_gamma=np.ones(H), ln1_beta=np.zeros(H), ln2_gamma=np.ones(H), ln2_beta=np.zeros(H))
    return w


def test_layer_forward_seqs_equals_rows_of_the_full_layer():
    r = np.random.default_rng(4)
    H, F, heads = 128, 512, 2
    w = _plain_weights(r, H, F)
    lengths = np.array([5, 0, 17, 1, 30, 9])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    x = r.standard_normal((int(cu[-1]), H))
    full = O.layer_forward(x, cu, w, heads)
    for seqs in ([0], [2, 4], [5, 3, 0], [1, 2], [4, 2]):
        got, sub_cu = O.layer_forward_seqs(x, cu, w, heads, seqs)
        rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
        assert np.array_equal(sub_cu, np.concatenate([[0], np.cumsum(lengths[seqs])]))
        assert np.allclose(got, full[rows], rtol=0, atol=1e-12), seqs


def test_stack_forward_is_two_layers_composed_by_hand():
    r = np.random.default_rng(5)
    H, F, heads, vocab = 128, 512, 2, 33
    layers = [_plain_weights(r, H, F), _plain_weights(r, H, F)]
    table = r.standard_normal((vocab, H)) * 0.5
    cu = np.array([0, 11, 11, 40])
    ids = r.integers(0, vocab, 40)
    x0 = table[ids]
    by_hand = O.layer_forward(O.layer_forward(x0, cu, layers[0], heads), cu, layers[1], heads)
    assert np.array_equal(O.stack_forward(cu, layers, heads, ids=ids, table=table), by_hand)
    assert np.array_equal(O.stack_forward(cu, layers, heads, x=x0), by_hand)
    # the order of the layers matters (the stack is not symmetric in them)
    swapped = O.layer_forward(O.layer_forward(x0, cu, layers[1], heads), cu, layers[0], heads)
    assert not np.allclose(swapped, by_hand)
    # no layers: the embedding itself (no final LayerNorm inside the stack)
    assert np.array_equal(O.stack_forward(cu, [], heads, ids=ids, table=table), x0)


# ---------------------------------------------------------------- FP8 layer

def _e4m3_q(a, s):
    """Value of the E4M3 cast of a * s, divided back by s (the pinned codec)."""
    return F8.quantize(a, s) / s


def _routing_weights(H, F, part, c):
    """Weights that reduce the layer's GEMMs to column selections scaled by c
    (c exact in both formats): part "attn" routes LN1's output to v and v
    back to the residual (q = k = 0, FFN zero); part "ffn" zeroes the
    attention branch and routes LN2's output through fc1 (times c) and the
    first H GELU columns back through fc2."""
    heads = H // 64
    w = {"ln1_gamma": np.ones(H), "ln1_beta": np.zeros(H), "ln2_gamma": np.ones(H), "ln2_beta": np.zeros(H),
         "w_qkv": np.zeros((3 * H, H)), "b_qkv": np.zeros(3 * H), "w_out": np.zeros((H, H)), "b_out": np.zeros(H),
         "w_fc1": np.zeros((F, H)), "b_fc1": np.zeros(F), "w_fc2": np.zeros((H, F)), "b_fc2": np.zeros(H)}
    if part == "attn":
        for n in range(heads):
            for j in range(64):
                w["w_qkv"][192 * n + 128 + j, 64 * n + j] = c       # v of head n, dim j <- h1 column 64 n + j
        w["w_out"] = np.eye(H)
    else:
        w["w_fc1"][np.arange(H), np.arange(H)] = c
        w["w_fc2"][np.arange(H), np.arange(H)] = 1.0
    return w


def _fp8_scales(s1=37.0, s2=53.0, s3=29.0, s4=61.0):
    return {"ln1": s1, "ctx": s2, "ln2": s3, "act": s4}


def test_fp8_layer_casts_ln1_output_and_context():
    """Length-1 sequences at position 0 (RoPE the identity, attention returns
    v), v = 1.5 Q(h1), out-projection the identity: x2 = x + Q(1.5 Q(h1)) with
    each Q the cast at its own scale.  Without the LN1 cast the result is
    x + Q(1.5 h1); without the context cast x + 1.5 Q(h1)."""
    r = np.random.default_rng(6)
    H, F, T = 128, 512, 24
    w = _routing_weights(H, F, "attn", 1.5)
    x = r.standard_normal((T, H)) * 2 + 0.3
    cu = np.arange(T + 1)
    sc = _fp8_scales()
    got = F8.layer_forward_fp8(x, cu, w, H // 64, sc)
    h1 = O.layer_norm(x, w["ln1_gamma"], w["ln1_beta"])
    want = x + _e4m3_q(1.5 * _e4m3_q(h1, sc["ln1"]), sc["ctx"])
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    for wrong in (x + _e4m3_q(1.5 * h1, sc["ctx"]), x + 1.5 * _e4m3_q(h1, sc["ln1"]),
                  x + _e4m3_q(1.5 * _e4m3_q(h1, sc["ctx"]), sc["ln1"])):      # scales swapped
        assert np.abs(got - wrong).max() > 1e-3


def test_fp8_layer_casts_ln2_output_and_gelu_output():
    """Zero attention branch (x1 = x); fc1 = 1.5 I on the first H columns, fc2
    picks them back: x2 = x + Q(GELU(1.5 Q(h2)))."""
    r = np.random.default_rng(7)
    H, F, T = 128, 512, 40
    w = _routing_weights(H, F, "ffn", 1.5)
    x = r.standard_normal((T, H)) * 3 - 0.2
    cu = np.array([0, 13, 13, 40])
    sc = _fp8_scales()
    got = F8.layer_forward_fp8(x, cu, w, H // 64, sc)
    h2 = O.layer_norm(x, w["ln2_gamma"], w["ln2_beta"])
    want = x + _e4m3_q(O.gelu(1.5 * _e4m3_q(h2, sc["ln2"])), sc["act"])
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    for wrong in (x + _e4m3_q(O.gelu(1.5 * h2), sc["act"]), x + O.gelu(1.5 * _e4m3_q(h2, sc["ln2"])),
                  x + _e4m3_q(O.gelu(1.5 * _e4m3_q(h2, sc["act"])), sc["ln2"])):
        assert np.abs(got - wrong).max() > 1e-3


def test_fp8_layer_tiny_activation_scales_leave_only_the_biases():
    """An activation scale so small that every scaled value rounds to the
    E4M3 zero makes that GEMM return its bias alone: context and GELU
    scales tiny give x2 = x + b_out + b_fc2 exactly."""
    r = np.random.default_rng(8)
    H, F, heads = 128, 512, 2
    w = _plain_weights(r, H, F)
    x = r.standard_normal((30, H))
    cu = np.array([0, 12, 30])
    got = F8.layer_forward_fp8(x, cu, w, heads, _fp8_scales(s2=1e-30, s4=1e-30))
    assert np.array_equal(got, (x + w["b_out"]) + w["b_fc2"])
    # LN1 tiny: q, k, v are the bias rows for every token, so the context
    # (and everything added to the residual) is the same for every row; LN2
    # tiny likewise makes the FFN branch row-independent.
    y = F8.layer_forward_fp8(x, cu, w, heads, _fp8_scales(s1=1e-30, s3=1e-30))
    d = y - x
    assert np.allclose(d, d[:1], rtol=0, atol=1e-12)
    assert np.abs(d).max() > 1e-3


@pytest.mark.parametrize("wname", ["w_qkv", "w_out", "w_fc1", "w_fc2"])
def test_fp8_layer_casts_every_weight(wname):
    """Moving a weight element (not the tensor's amax) halfway towards the
    value its cast gives leaves the cast, hence the FP8 layer's output,
    unchanged bit for bit, while the plain layer moves: each weight passes
    through its own cast with s = 448 / amax(W)."""
    r = np.random.default_rng(9)
    H, F, heads = 128, 512, 2
    w = _plain_weights(r, H, F)
    x = r.standard_normal((30, H))
    cu = np.array([0, 7, 30])
    sc = _fp8_scales()
    base = F8.layer_forward_fp8(x, cu, w, heads, sc)
    W = w[wname]
    s = 448.0 / np.abs(W).max()
    flat = np.abs(W).ravel()
    moved = 0
    for idx in r.choice(W.size, 40, replace=False):
        if flat[idx] == flat.max():
            continue
        i = np.unravel_index(idx, W.shape)
        qv = _e4m3_q(W[i], s)
        if qv == W[i]:
            continue
        w2 = dict(w)
        w2[wname] = W.copy()
        w2[wname][i] = W[i] + (qv - W[i]) / 2
        assert np.array_equal(F8.layer_forward_fp8(x, cu, w2, heads, sc), base), (wname, i)
        assert not np.array_equal(O.layer_forward(x, cu, w2, heads), O.layer_forward(x, cu, w, heads))
        moved += 1
        if moved == 3:
            break
    assert moved == 3


# ---------------------------------------------------------------- MXFP4 layer

def _mx_q(a):
    """Dequantised MXFP4 of a [rows, K] (the pinned block quantiser)."""
    return F4.mx_dequantize(*F4.mx_quantize(a))


def test_mxfp4_block_product_worked_by_hand():
    """One 32-value block each.  x: max 7 -> shared exponent
    floor(log2 7) - 2 = 0 (scale 1); 5 is the midpoint of 4 and 6 and goes to
    4 (even mantissa), 2.6 -> 3, 0.74 -> 0.5, -1.25 (midpoint of 1 and 1.5)
    -> -1, 7 saturates to 6.  w: max 1 -> exponent -2 (scale 1/4); 1 -> 4/4,
    0.3 -> 1.2 quarters -> 1 quarter.  y = 4*1 + 3*0.25 + 0.5*1 - 1*1 + 6*1."""
    x = np.zeros((1, 32))
    x[0, :5] = [5.0, 2.6, 0.74, -1.25, 7.0]
    w = np.zeros((1, 32))
    w[0, :5] = [1.0, 0.3, 1.0, 1.0, 1.0]
    xc, xe = F4.mx_quantize(x)
    wc, we = F4.mx_quantize(w)
    assert xe.tolist() == [[0]] and we.tolist() == [[-2]]
    assert F4.mx_dequantize(xc, xe)[0, :5].tolist() == [4.0, 3.0, 0.5, -1.0, 6.0]
    assert F4.mx_dequantize(wc, we)[0, :5].tolist() == [1.0, 0.25, 1.0, 1.0, 1.0]
    assert F4.mx_matmul(xc, xe, wc, we).tolist() == [[10.25]]


def test_mxfp4_layer_quantises_ln1_output_and_context():
    """As the FP8 check: x2 = x + Q(1.5 Q(h1)), Q the MXFP4 block quantiser
    (blocks of 32 along each GEMM's K).  Without the LN1 quantisation
    x + Q(1.5 h1); without the context's x + 1.5 Q(h1)."""
    r = np.random.default_rng(10)
    H, F, T = 128, 512, 24
    w = _routing_weights(H, F, "attn", 1.5)
    x = r.standard_normal((T, H)) * 2 + 0.3
    cu = np.arange(T + 1)
    got = F4.layer_forward_mxfp4(x, cu, w, H // 64)
    h1 = O.layer_norm(x, w["ln1_gamma"], w["ln1_beta"])
    assert np.array_equal(got, x + _mx_q(1.5 * _mx_q(h1)))
    for wrong in (x + _mx_q(1.5 * h1), x + 1.5 * _mx_q(h1)):
        assert np.abs(got - wrong).max() > 1e-3


def test_mxfp4_layer_quantises_ln2_output_and_gelu_output():
    r = np.random.default_rng(11)
    H, F, T = 128, 512, 40
    w = _routing_weights(H, F, "ffn", 1.5)
    x = r.standard_normal((T, H)) * 3 - 0.2
    cu = np.array([0, 13, 13, 40])
    got = F4.layer_forward_mxfp4(x, cu, w, H // 64)
    h2 = O.layer_norm(x, w["ln2_gamma"], w["ln2_beta"])
    # GELU output [T, F]: only its first H columns are nonzero; blocks of 32
    # along F never mix them with the zero columns
    a = O.gelu(1.5 * _mx_q(h2))
    assert np.array_equal(got, x + _mx_q(a))
    for wrong in (x + _mx_q(O.gelu(1.5 * h2)), x + a):
        assert np.abs(got - wrong).max() > 1e-3


@pytest.mark.parametrize("wname", ["w_qkv", "w_out", "w_fc1", "w_fc2"])
def test_mxfp4_layer_quantises_every_weight(wname):
    """Moving a weight element (not its block's maximum) halfway towards its
    quantised value keeps the block's exponent and every code: the MXFP4
    layer's output is unchanged bit for bit while the plain layer moves."""
    r = np.random.default_rng(12)
    H, F, heads = 128, 512, 2
    w = _plain_weights(r, H, F)
    x = r.standard_normal((30, H))
    cu = np.array([0, 7, 30])
    base = F4.layer_forward_mxfp4(x, cu, w, heads)
    W = w[wname]
    Wq = _mx_q(W)
    moved = 0
    for idx in r.choice(W.size, 40, replace=False):
        i = np.unravel_index(idx, W.shape)
        b0 = (i[1] // 32) * 32
        blk = np.abs(W[i[0], b0:b0 + 32])
        if abs(W[i]) == blk.max() or Wq[i] == W[i]:
            continue
        w2 = dict(w)
        w2[wname] = W.copy()
        w2[wname][i] = W[i] + (Wq[i] - W[i]) / 2
        assert np.array_equal(_mx_q(w2[wname]), Wq)
        assert np.array_equal(F4.layer_forward_mxfp4(x, cu, w2, heads), base), (wname, i)
        assert not np.array_equal(O.layer_forward(x, cu, w2, heads), O.layer_forward(x, cu, w, heads))
        moved += 1
        if moved == 3:
            break
    assert moved == 3
