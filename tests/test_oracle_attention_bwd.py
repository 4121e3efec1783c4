"""Pins of the oracle's attention backward, softmax normaliser and linear backward
(oracle/esm_oracle.py: attention_bwd, attention_lse, linear_bwd, layer_norm_bwd, gelu_bwd, rope_bwd, qkv_rope_bwd), against things other
than the oracle's own formulas:

* central finite differences of the forward loss sum(dO * attention(q, k, v))
  (the definition of the gradient), on tiny ragged batches;
* exact identities of the softmax Jacobian: every row of dS sums to zero, so
  the keys' dk of one (sequence, head) sum to zero; every row of P sums to
  one, so the keys' dv sum to the queries' dO;
* special cases: a one-residue sequence (P = 1: dq = dk = 0, dv = dO), equal
  keys (uniform P), and no coupling across sequences;
* the normaliser by a brute-force exact sum (math.fsum of exp) on tiny rows.
"""
import math

import numpy as np
import pytest

from oracle import esm_oracle as O

D = 64


def _inputs(lens, heads, seed):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    q = rng.standard_normal((T, heads, D))
    k = rng.standard_normal((T, heads, D))
    v = rng.standard_normal((T, heads, D))
    g = rng.standard_normal((T, heads * D))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, g, cu


def _loss(q, k, v, g, cu):
    return float(np.sum(g * O.attention(q, k, v, cu)))


@pytest.mark.parametrize("lens,heads,seed", [([3, 5], 2, 0), ([1, 4, 2], 1, 1), ([6], 3, 2)])
def test_bwd_matches_finite_differences(lens, heads, seed):
    q, k, v, g, cu = _inputs(lens, heads, seed)
    dq, dk, dv = O.attention_bwd(q, k, v, g, cu)
    rng = np.random.default_rng(100 + seed)
    h = 1e-5
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        flat = x.reshape(-1)
        for i in rng.choice(flat.size, size=24, replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = _loss(q, k, v, g, cu)
            flat[i] = old - h
            lm = _loss(q, k, v, g, cu)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            # central difference error O(h^2 |f'''|) plus rounding eps |f| / h
            assert abs(fd - dx.reshape(-1)[i]) <= 1e-7 * max(1.0, abs(fd)), (i, fd, dx.reshape(-1)[i])


def test_bwd_key_sums():
    lens, heads = [7, 1, 12], 3
    q, k, v, g, cu = _inputs(lens, heads, 3)
    dq, dk, dv = O.attention_bwd(q, k, v, g, cu)
    dO = g.reshape(-1, heads, D)
    for a, b in O.segments(cu):
        np.testing.assert_allclose(dk[a:b].sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv[a:b].sum(axis=0), dO[a:b].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_bwd_single_residue_and_equal_keys():
    # one residue: P = [[1]], the softmax Jacobian vanishes
    q, k, v, g, cu = _inputs([1], 2, 4)
    dq, dk, dv = O.attention_bwd(q, k, v, g, cu)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv, g.reshape(1, 2, D))
    # all keys equal: P uniform (1 / L), so dq = scale * rowsum(dS) k = 0 and
    # every dv[j] = mean over the queries of dO
    L = 5
    q, k, v, g, cu = _inputs([L], 1, 5)
    k[:] = k[0]
    dq, dk, dv = O.attention_bwd(q, k, v, g, cu)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv[:, 0], np.repeat(g.mean(axis=0, keepdims=True), L, 0), rtol=1e-12, atol=1e-12)


def test_bwd_no_coupling_across_sequences():
    lens, heads = [4, 6], 2
    q, k, v, g, cu = _inputs(lens, heads, 6)
    base = O.attention_bwd(q, k, v, g, cu)
    q2, k2, v2, g2 = q.copy(), k.copy(), v.copy(), g.copy()
    rng = np.random.default_rng(7)
    for x in (q2, k2, v2):
        x[4:] = rng.standard_normal(x[4:].shape)
    g2[4:] = rng.standard_normal(g2[4:].shape)
    moved = O.attention_bwd(q2, k2, v2, g2, cu)
    for a, b in zip(base, moved):
        np.testing.assert_array_equal(a[:4], b[:4])


def test_lse_brute_force():
    lens, heads = [3, 5], 2
    q, k, _, _, cu = _inputs(lens, heads, 8)
    lse = O.attention_lse(q, k, cu)
    for a, b in O.segments(cu):
        for n in range(heads):
            for t in range(a, b):
                terms = [math.exp(O.SOFTMAX_SCALE * sum(q[t, n, i] * k[j, n, i] for i in range(D)))
                         for j in range(a, b)]
                assert abs(lse[n, t] - math.log(math.fsum(terms))) <= 1e-12 * max(1.0, abs(lse[n, t]))
    # exp(S - lse) is the attention's P
    a, b = 3, 8
    S = q[a:b, 1] @ k[a:b, 1].T * O.SOFTMAX_SCALE
    np.testing.assert_allclose(np.exp(S - lse[1, a:b, None]), O.attention_probs(q[a:b, 1], k[a:b, 1]),
                               rtol=1e-12)


def test_empty_sequences_change_nothing():
    """Empty sequences (zero-length segments) add no rows: the results equal
    those of the batch without them."""
    q, k, v, g, cu = _inputs([3, 4], 2, 9)
    cu_e = np.array([0, 0, 3, 3, 7, 7])
    for a, b in zip(O.attention_bwd(q, k, v, g, cu), O.attention_bwd(q, k, v, g, cu_e)):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(O.attention_lse(q, k, cu), O.attention_lse(q, k, cu_e))


# ---------------------------------------------------------------- linear backward

def test_linear_bwd_matches_finite_differences():
    """The loss sum(dy * (x w^T + b)) is linear in each of x, w, b, so central
    differences are exact up to rounding."""
    rng = np.random.default_rng(30)
    M, N, K = 5, 3, 4
    x, w, b, dy = (rng.standard_normal(s) for s in ((M, K), (N, K), (N,), (M, N)))
    dx, dw, db = O.linear_bwd(x, w, dy)

    def loss():
        return float(np.sum(dy * (x @ w.T + b)))
    h = 1e-3
    for a, da in ((x, dx), (w, dw), (b, db)):
        flat, g = a.reshape(-1), da.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            lp = loss()
            flat[i] = old - h
            lm = loss()
            flat[i] = old
            assert abs((lp - lm) / (2 * h) - g[i]) <= 1e-9 * max(1.0, abs(g[i]))


def test_linear_bwd_adjoint_identity():
    """<dy, x w^T> = <dx, x> = <dw, w>: each gradient pairs with its operand to
    the same number, which fails for a transposed or swapped operand."""
    rng = np.random.default_rng(31)
    M, N, K = 37, 64, 128
    x, w, dy = (rng.standard_normal(s) for s in ((M, K), (N, K), (M, N)))
    dx, dw, db = O.linear_bwd(x, w, dy)
    ref = float(np.sum(dy * (x @ w.T)))
    assert abs(float(np.sum(dx * x)) - ref) <= 1e-9 * abs(ref)
    assert abs(float(np.sum(dw * w)) - ref) <= 1e-9 * abs(ref)
    assert abs(float(db.sum()) - float(dy.sum())) <= 1e-9 * max(1.0, abs(float(dy.sum())))


# ---------------------------------------------------------------- LayerNorm backward

def test_layer_norm_bwd_matches_finite_differences():
    rng = np.random.default_rng(32)
    M, H = 3, 16
    x = rng.standard_normal((M, H)) * 2 + 0.5
    gamma, beta = rng.standard_normal(H), rng.standard_normal(H)
    dy = rng.standard_normal((M, H))
    dx, dg, db = O.layer_norm_bwd(x, gamma, dy)

    def loss():
        return float(np.sum(dy * O.layer_norm(x, gamma, beta)))
    h = 1e-6
    for a, da in ((x, dx), (gamma, dg), (beta, db)):
        flat, g = a.reshape(-1), da.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            lp = loss()
            flat[i] = old - h
            lm = loss()
            flat[i] = old
            assert abs((lp - lm) / (2 * h) - g[i]) <= 1e-7 * max(1.0, abs(g[i])), (i, g[i])


def test_layer_norm_bwd_row_sums_and_shift():
    """Every row of dx sums to zero (the output does not change when a constant
    is added to a row), and dx does not change when the row is shifted."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal((7, 64))
    gamma, dy = rng.standard_normal(64), rng.standard_normal((7, 64))
    dx, _, _ = O.layer_norm_bwd(x, gamma, dy)
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-12)
    dx2, _, _ = O.layer_norm_bwd(x + 3.0, gamma, dy)
    np.testing.assert_allclose(dx2, dx, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- GELU and RoPE backward

def test_gelu_bwd_finite_differences_and_closed_forms():
    rng = np.random.default_rng(34)
    z = np.concatenate([rng.standard_normal(40) * 3, [0.0, -8.0, 8.0, 1.0]])
    dy = rng.standard_normal(z.size)
    got = O.gelu_bwd(z, dy)
    h = 1e-6
    fd = (O.gelu(z + h) - O.gelu(z - h)) / (2 * h) * dy
    np.testing.assert_allclose(got, fd, rtol=1e-7, atol=1e-8)
    one = np.ones_like(z)
    # GELU(z) - GELU(-z) = z, so GELU'(z) + GELU'(-z) = 1; GELU'(0) = 1/2
    np.testing.assert_allclose(O.gelu_bwd(z, one) + O.gelu_bwd(-z, one), 1.0, atol=1e-14)
    assert O.gelu_bwd(np.array([0.0]), np.array([1.0]))[0] == 0.5


def test_rope_bwd_is_the_transpose():
    rng = np.random.default_rng(35)
    T, heads = 9, 3
    pos = rng.integers(0, 1000, T)
    u, du = rng.standard_normal((T, heads, 64)), rng.standard_normal((T, heads, 64))
    # adjoint: <du, R u> = <R^T du, u>; orthogonal: R^T R u = u
    lhs = float(np.sum(du * O.apply_rope(u, pos)))
    assert abs(lhs - float(np.sum(O.rope_bwd(du, pos) * u))) <= 1e-10 * max(1.0, abs(lhs))
    np.testing.assert_allclose(O.rope_bwd(O.apply_rope(u, pos), pos), u, atol=1e-12)


def test_qkv_rope_bwd_adjoint_of_split_and_rotate():
    """f(y) = (rope(q(y)), rope(k(y)), v(y)) with (q, k, v) = split_qkv(y) is
    linear in y; its backward g satisfies <(dq, dk, dv), f(y)> = <g(dq, dk, dv), y>
    for every y, and must undo the per-sequence positions."""
    rng = np.random.default_rng(36)
    lens, heads = [5, 1, 7], 2
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    pos = O.positions(cu)
    for _ in range(3):
        y = rng.standard_normal((T, 3 * heads * 64))
        dq, dk, dv = (rng.standard_normal((T, heads, 64)) for _ in range(3))
        q, k, v = O.split_qkv(y, heads)
        lhs = float(np.sum(dq * O.apply_rope(q, pos)) + np.sum(dk * O.apply_rope(k, pos)) + np.sum(dv * v))
        rhs = float(np.sum(O.qkv_rope_bwd(dq, dk, dv, cu) * y))
        assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


# ---------------------------------------------------------------- whole layer

def test_layer_backward_matches_finite_differences():
    """The chained layer backward against central differences of the whole
    layer forward (H = 128, 2 heads, F = 256, two sequences), at random
    coordinates of x and of every weight."""
    rng = np.random.default_rng(37)
    H, heads, F = 128, 2, 256
    lens = [4, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    w = {"ln1_gamma": 1 + 0.1 * rng.standard_normal(H), "ln1_beta": 0.1 * rng.standard_normal(H),
         "w_qkv": 0.1 * rng.standard_normal((3 * H, H)), "b_qkv": 0.1 * rng.standard_normal(3 * H),
         "w_out": 0.1 * rng.standard_normal((H, H)), "b_out": 0.1 * rng.standard_normal(H),
         "ln2_gamma": 1 + 0.1 * rng.standard_normal(H), "ln2_beta": 0.1 * rng.standard_normal(H),
         "w_fc1": 0.1 * rng.standard_normal((F, H)), "b_fc1": 0.1 * rng.standard_normal(F),
         "w_fc2": 0.1 * rng.standard_normal((H, F)), "b_fc2": 0.1 * rng.standard_normal(H)}
    x = rng.standard_normal((T, H))
    dout = rng.standard_normal((T, H))
    dx, g = O.layer_backward(x, cu, w, heads, dout)

    def loss():
        return float(np.sum(dout * O.layer_forward(x, cu, w, heads)))
    h = 1e-5
    for name, a, da in [("x", x, dx)] + [(k, w[k], g[k]) for k in w]:
        flat, gf = a.reshape(-1), da.reshape(-1)
        for i in rng.choice(flat.size, size=6, replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = loss()
            flat[i] = old - h
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - gf[i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, gf[i])


# ---------------------------------------------------------------- stack

def _layer_w(rng, H, F):
    return {"ln1_gamma": 1 + 0.1 * rng.standard_normal(H), "ln1_beta": 0.1 * rng.standard_normal(H),
            "w_qkv": 0.1 * rng.standard_normal((3 * H, H)), "b_qkv": 0.1 * rng.standard_normal(3 * H),
            "w_out": 0.1 * rng.standard_normal((H, H)), "b_out": 0.1 * rng.standard_normal(H),
            "ln2_gamma": 1 + 0.1 * rng.standard_normal(H), "ln2_beta": 0.1 * rng.standard_normal(H),
            "w_fc1": 0.1 * rng.standard_normal((F, H)), "b_fc1": 0.1 * rng.standard_normal(F),
            "w_fc2": 0.1 * rng.standard_normal((H, F)), "b_fc2": 0.1 * rng.standard_normal(H)}


def _check_fd(loss, pairs, rng, n=4, h=1e-5, rtol=1e-6):
    for name, a, da in pairs:
        flat, gf = a.reshape(-1), da.reshape(-1)
        for i in rng.choice(flat.size, size=min(n, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = loss()
            flat[i] = old - h
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - gf[i]) <= rtol * max(1.0, abs(fd)), (name, i, fd, gf[i])


def test_stack_backward_from_ids_matches_finite_differences():
    """Two layers on top of the embedding gather (vocab 7, token 6 absent from
    the batch): central differences of the stack forward from token ids, at
    random coordinates of every weight of both layers and of the table rows;
    the absent token's table row gets exactly zero."""
    rng = np.random.default_rng(38)
    H, heads, F, V = 128, 2, 256, 7
    lens = [4, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    ids = np.array([0, 3, 3, 5, 1, 2, 3])
    table = rng.standard_normal((V, H))
    layers = [_layer_w(rng, H, F) for _ in range(2)]
    dout = rng.standard_normal((int(cu[-1]), H))
    dx0, grads, dtab = O.stack_backward(cu, layers, heads, dout, ids=ids, table=table)
    assert np.all(dtab[6] == 0) and np.all(dtab[4] == 0)

    def loss():
        return float(np.sum(dout * O.stack_forward(cu, layers, heads, ids=ids, table=table)))
    pairs = [("table", table, dtab)]
    for l, (w, g) in enumerate(zip(layers, grads)):
        pairs += [(f"{k}[{l}]", w[k], g[k]) for k in w]
    _check_fd(loss, pairs, rng, n=3)
    # the table gradient is the sum of the input gradient over the rows of each token
    _check_fd(loss, [("table row 3", table[3], dtab[3])], rng, n=8)


def test_stack_backward_from_hidden_states_matches_finite_differences():
    """Three layers from given hidden states, one-residue sequence included:
    central differences at random coordinates of the input and of the first
    and last layers' weights; with one layer the stack backward is the layer
    backward."""
    rng = np.random.default_rng(39)
    H, heads, F = 128, 2, 256
    lens = [1, 5, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    layers = [_layer_w(rng, H, F) for _ in range(3)]
    x = rng.standard_normal((T, H))
    dout = rng.standard_normal((T, H))
    dx0, grads, dtab = O.stack_backward(cu, layers, heads, dout, x=x)
    assert dtab is None

    def loss():
        return float(np.sum(dout * O.stack_forward(cu, layers, heads, x=x)))
    _check_fd(loss, [("x", x, dx0)] + [(f"{k}[0]", layers[0][k], grads[0][k]) for k in ("w_qkv", "ln1_gamma", "b_fc2")]
              + [(f"{k}[2]", layers[2][k], grads[2][k]) for k in ("w_fc1", "ln2_beta", "w_out")], rng, n=4)
    d1, g1, _ = O.stack_backward(cu, layers[:1], heads, dout, x=x)
    d_ref, g_ref = O.layer_backward(x, cu, layers[0], heads, dout)
    assert np.array_equal(d1, d_ref) and all(np.array_equal(g1[0][k], g_ref[k]) for k in g_ref)
