"""Pins of the MXFP4 reference (oracle/fp4_ref.py) against the format's own
definition: the E2M1 value set, rounding at every midpoint, the shared-scale
rule, exact round trips and the error bound of one block."""
import numpy as np

from oracle import fp4_ref as F


def test_e2m1_values():
    t = F.e2m1_decode_table()
    assert list(t[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(t[8:], -t[:8])
    assert np.signbit(t[8]) and t[8] == 0.0          # code 8 is -0
    assert F.E2M1_MAX == t.max() == 1.5 * 2.0 ** F.E2M1_EMAX


def test_e2m1_encode_midpoints_and_saturation():
    # each midpoint between neighbours goes to the one with mantissa bit 0
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             0.2499: 0.0, 0.2501: 0.5, 0.7499: 0.5, 1.2501: 1.5, 1.7499: 1.5, 2.5001: 3.0, 3.4999: 3.0,
             4.9999: 4.0, 5.0001: 6.0, 6.0: 6.0, 7.9: 6.0, 1e30: 6.0, 0.0: 0.0}
    t = F.e2m1_decode_table()
    for v, want in cases.items():
        assert t[F.e2m1_encode(v)] == want, v
        assert t[F.e2m1_encode(-v)] == -want, -v
    assert F.e2m1_encode(-0.1) == 8 and F.e2m1_encode(-0.0) == 8


def test_e2m1_encode_is_nearest():
    rng = np.random.default_rng(3)
    v = rng.uniform(-7, 7, 20000)
    got = F.e2m1_decode_table()[F.e2m1_encode(v)]
    clipped = np.clip(v, -6, 6)
    d_best = np.min(np.abs(clipped[:, None] - F.e2m1_decode_table()[None, :]), axis=1)
    assert np.allclose(np.abs(clipped - got), d_best, rtol=0, atol=0)


def test_block_exponent_rule():
    assert F.block_exponent(np.zeros(32)) == -127
    for amax, e in [(6.0, 0), (4.0, 0), (7.99, 0), (8.0, 1), (1.0, -2), (0.75, -3), (2.0 ** -140, -127),
                    (2.0 ** 200, 127), (3.0 * 2.0 ** 10, 9)]:
        b = np.zeros(32)
        b[5] = -amax
        assert F.block_exponent(b) == e, amax
    # the largest magnitude lands in [4, 8) times 2^e unless clamped
    rng = np.random.default_rng(4)
    for _ in range(200):
        b = rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20)
        e = F.block_exponent(b)
        assert 4.0 <= np.abs(b).max() / 2.0 ** e < 8.0


def test_representable_blocks_round_trip_exactly():
    rng = np.random.default_rng(5)
    t = F.e2m1_decode_table()
    codes = rng.integers(0, 16, (6, 128))
    codes[:, ::32] = 7                                   # each block holds a 6
    e = rng.integers(-30, 30, (6, 4))
    x = t[codes] * np.exp2(np.repeat(e, 32, axis=1))
    q, ex = F.mx_quantize(x)
    assert np.array_equal(ex, e)
    assert np.array_equal(F.mx_dequantize(q, ex), x)


def test_quantisation_error_bound():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 256)) * np.exp2(rng.integers(-8, 8, (8, 1)))
    q, ex = F.mx_quantize(x)
    X = np.exp2(np.repeat(ex, 32, axis=1).astype(np.float64))
    v = np.abs(x) / X
    half_step = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    bound = np.where(v <= 6, half_step, v - 6) * X
    assert np.all(np.abs(F.mx_dequantize(q, ex) - x) <= bound)


def test_mx_matmul():
    rng = np.random.default_rng(7)
    t = F.e2m1_decode_table()
    # representable operands: the MXFP4 product is the plain product
    xc, wc = rng.integers(0, 16, (5, 96)), rng.integers(0, 16, (3, 96))
    xc[:, ::32] = 7
    wc[:, ::32] = 15
    xe, we = rng.integers(-5, 5, (5, 3)), rng.integers(-5, 5, (3, 3))
    x = t[xc] * np.exp2(np.repeat(xe, 32, axis=1))
    w = t[wc] * np.exp2(np.repeat(we, 32, axis=1))
    qx, ex = F.mx_quantize(x)
    qw, ew = F.mx_quantize(w)
    assert np.array_equal(F.mx_matmul(qx, ex, qw, ew), x @ w.T)
    # scaling an operand by 2^k moves only its exponents, so y scales exactly
    qx2, ex2 = F.mx_quantize(x * 8.0)
    assert np.array_equal(qx2, qx) and np.array_equal(ex2, ex + 3)
    assert np.array_equal(F.mx_matmul(qx2, ex2, qw, ew), 8.0 * (x @ w.T))


def test_vectorised_quantiser_follows_the_block_rule():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((16, 256)) * np.exp2(rng.integers(-60, 60, (16, 8)).repeat(32, axis=1))
    x[3, 64:96] = 0.0
    codes, exps = F.mx_quantize(x)
    for r in range(16):
        for b in range(8):
            blk = x[r, 32 * b: 32 * b + 32]
            e = F.block_exponent(blk)
            assert exps[r, b] == e
            assert np.array_equal(codes[r, 32 * b: 32 * b + 32], F.e2m1_encode(blk / 2.0 ** e))


def test_bf16_round():
    # exactly representable values stay; midpoints go to the even neighbour
    assert F.bf16_round(1.0) == 1.0 and F.bf16_round(-3.5) == -3.5
    assert F.bf16_round(1.0 + 2.0 ** -8) == 1.0                 # midpoint, even below
    assert F.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # midpoint, even above
    assert F.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7


def test_mxfp4_layer_with_representable_operands_is_the_plain_layer():
    """Zero weights in the two GEMMs that feed the residuals make the MXFP4
    layer the identity, as the plain one (the quantised zero is exact)."""
    from oracle import esm_oracle as O
    rng = np.random.default_rng(9)
    H, F_, heads = 256, 512, 4
    w = {"ln1_gamma": np.ones(H), "ln1_beta": np.zeros(H), "ln2_gamma": np.ones(H), "ln2_beta": np.zeros(H),
         "w_qkv": F.bf16_round(rng.standard_normal((3 * H, H)) * 0.02), "b_qkv": np.zeros(3 * H),
         "w_out": np.zeros((H, H)), "b_out": np.zeros(H), "w_fc1": F.bf16_round(rng.standard_normal((F_, H)) * 0.02),
         "b_fc1": np.zeros(F_), "w_fc2": np.zeros((H, F_)), "b_fc2": np.zeros(H)}
    x = rng.standard_normal((40, H))
    cu = np.array([0, 15, 40])
    assert np.array_equal(F.layer_forward_mxfp4(x, cu, w, heads), x)
    assert np.array_equal(O.layer_forward(x, cu, w, heads), x)
