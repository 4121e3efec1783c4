"""MXFP4 (the FP4 recipe reading: OCP microscaling E2M1 with one E8M0 scale
per 32 values along K) through the C ABI, against oracle/fp4_ref.py."""
import numpy as np
import pytest
import torch

from oracle import fp4_ref as F
from protein_language_model_amd import datagen as D
from protein_language_model_amd import esm

pytestmark = pytest.mark.gpu

ORDER = [0, 2, 4, 6, 1, 3, 5, 7]   # blocks of one K step in the scale layout


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


@pytest.fixture(scope="module")
def enc():
    e = esm.Encoder(num_hidden_layers=1)
    yield e
    e.close()


def pack_reference(codes, exps):
    """Oracle codes / exponents in the library's MXFP4 layout."""
    M, K = codes.shape
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    M2 = M + (M & 1)
    sc = np.full((K // 256, M2, 8), 127, np.uint8)
    for s in range(K // 256):
        for p, j in enumerate(ORDER):
            sc[s, :M, p] = (exps[:, 8 * s + j] + 127).astype(np.uint8)
    return packed, sc


def _inputs(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp2(rng.integers(-12, 12, (M, 1)))
    x[0, :32] = 0.0                                            # an all-zero block
    if M > 1 and K >= 64:                                      # every rounding midpoint, scale 2^3
        mids = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.2, 0.3, 4.9, 5.1, 7.5, 0.5, 1, 1.5])
        x[1, 32:64] = np.concatenate([mids, -mids]) * 8.0
    return D.to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("M,K", [(1, 256), (7, 512), (130, 1280), (1000, 5120)])
def test_mxfp4_quantize_bit_exact(enc, gu, M, K):
    bits = _inputs(M, K, seed=M + K)
    codes, scales = enc.mxfp4_quantize(gu.to_dev_bf16(bits))
    torch.cuda.synchronize()
    ref_codes, ref_exps = F.mx_quantize(D.bf16_bits_to_f64(bits))
    want_codes, want_scales = pack_reference(ref_codes, ref_exps)
    assert np.array_equal(codes.cpu().numpy(), want_codes)
    assert np.array_equal(scales.cpu().numpy(), want_scales)


@pytest.mark.parametrize("M,N,K,epi", [(1, 64, 256, esm.EPI_BIAS), (300, 320, 1280, esm.EPI_BIAS_GELU),
                                       (1000, 1280, 512, esm.EPI_BIAS_RESIDUAL), (2049, 512, 1280, esm.EPI_BIAS)])
def test_mxfp4_linear_matches_oracle(enc, gu, M, N, K, epi):
    """MXFP4 GEMM on the library's own quantisation of x and w against the
    oracle's quantisation and exact product: the dequantised products are
    exact, the sums run in fp32 and y is rounded to bf16."""
    from oracle import esm_oracle as O
    rng = np.random.default_rng(M + N + K)
    xb = D.to_bf16_bits((rng.standard_normal((M, K)) * np.exp2(rng.integers(-4, 4, (M, 1)))).astype(np.float32))
    wb = D.to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    bb = D.to_bf16_bits((rng.standard_normal(N) * 0.02).astype(np.float32))
    rb = D.to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    xq = enc.mxfp4_quantize(gu.to_dev_bf16(xb))
    wq = enc.mxfp4_quantize(gu.to_dev_bf16(wb))
    res = gu.to_dev_bf16(rb) if epi == esm.EPI_BIAS_RESIDUAL else None
    got = gu.from_dev(enc.linear_mxfp4_fwd(xq, wq, gu.to_dev_bf16(bb), residual=res, epilogue=epi))
    ref = F.mx_matmul(*F.mx_quantize(D.bf16_bits_to_f64(xb)), *F.mx_quantize(D.bf16_bits_to_f64(wb)))
    ref = ref + D.bf16_bits_to_f64(bb)
    if epi == esm.EPI_BIAS_GELU:
        ref = O.gelu(ref)
    if epi == esm.EPI_BIAS_RESIDUAL:
        ref = ref + D.bf16_bits_to_f64(rb)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max()
    assert np.all(np.abs(got - ref) <= bound), np.abs(got - ref).max()


# ------------------------------------------------------------ MXFP4 layers

# vs the MXFP4-emulating oracle: the library computes the quantiser inputs (LN
# outputs, context, GELU output) in fp32 and the emulation in fp64; where the
# two land on different sides of an E2M1 midpoint the code moves by one step
# (up to a third of the value), and attention and the FFN carry such flips on
# (measured 5.3e-2 on this layer).
TOL_MX_EMU = 8e-2
# vs the plain fp64 layer: the recipe's own error (emulation vs fp64, measured
# 1.3e-1 here) plus 2e-2, the rule of the FP8 stack.
TOL_MX_OVER_RECIPE = 2e-2


@pytest.fixture(scope="module")
def l650_mx(gu):
    """650M-shaped single layer (hidden 1280, 20 heads, FFN 5120), MXFP4
    encoder, three packed sequences, random LayerNorm parameters."""
    H, F, heads = 1280, 5120, 20
    lengths = np.array([17, 100, 333])
    cu = D.cu_from_lengths(lengths)
    T = int(cu[-1])
    enc = esm.Encoder(hidden_size=H, num_attention_heads=heads, intermediate_size=F, num_hidden_layers=1,
                      precision="mxfp4")
    wd, wr, _ = gu.layer_weights(H, F, layer=0, seed=3, random_ln=True)
    enc.mxfp4_prepare([wd])
    xb = D.make_hidden(T, H, seed=3)
    yield {"enc": enc, "wd": wd, "wr": wr, "xb": xb, "cu": cu, "lengths": lengths, "T": T, "H": H, "heads": heads}
    enc.close()


def _mx_layer(t, gu, xbits, cu):
    T = int(cu[-1])
    return t["enc"].layer_fwd(t["wd"], gu.to_dev_bf16(xbits), gu.to_dev_i32(cu), len(cu) - 1, T,
                              int(np.max(np.diff(cu))))


def test_mxfp4_layer_matches_the_oracles(gu, l650_mx):
    t = l650_mx
    y = gu.from_dev(_mx_layer(t, gu, t["xb"], t["cu"]))
    x = D.bf16_bits_to_f64(t["xb"])
    emu = F.layer_forward_mxfp4(x, t["cu"], t["wr"], t["heads"])
    from oracle import esm_oracle as O
    ref = O.layer_forward(x, t["cu"], t["wr"], t["heads"])
    e_emu, e_plain = gu.rel_err(y, emu), gu.rel_err(y, ref)
    print(f"650M MXFP4 layer: rel err vs MXFP4 emulation {e_emu:.2e}, vs fp64 {e_plain:.2e}, "
          f"emulation vs fp64 {gu.rel_err(emu, ref):.2e}")
    assert np.isfinite(y).all()
    assert e_emu < TOL_MX_EMU
    assert e_plain < gu.rel_err(emu, ref) + TOL_MX_OVER_RECIPE


def test_mxfp4_layer_packed_equals_alone(gu, l650_mx):
    t = l650_mx
    y = gu.bits_of(_mx_layer(t, gu, t["xb"], t["cu"]))
    for s in range(len(t["lengths"])):
        a, e = int(t["cu"][s]), int(t["cu"][s + 1])
        ya = gu.bits_of(_mx_layer(t, gu, t["xb"][a:e], np.array([0, e - a])))
        assert np.array_equal(ya, y[a:e]), s


def test_mxfp4_layer_thd_equals_bshd_with_nan_padding(gu, l650_mx):
    t = l650_mx
    y = gu.bits_of(_mx_layer(t, gu, t["xb"], t["cu"]))
    S, B = int(t["lengths"].max()), len(t["lengths"])
    xp = np.full((B, S, t["H"]), 0x7FC0, np.uint16)            # NaN padding
    for i in range(B):
        xp[i, :t["lengths"][i]] = t["xb"][t["cu"][i]:t["cu"][i + 1]]
    yp = gu.bits_of(t["enc"].layer_fwd_bshd(t["wd"], gu.to_dev_bf16(xp), gu.to_dev_i32(t["lengths"]), B, S))
    for i in range(B):
        L = int(t["lengths"][i])
        assert np.array_equal(yp[i, :L], y[t["cu"][i]:t["cu"][i + 1]]), i
        assert not np.any(yp[i, L:]), i


def test_mxfp4_layer_precision_bf16_equals_the_bf16_encoder(gu, l650_mx):
    t = l650_mx
    t["enc"].set_layer_precision(["bf16"])
    try:
        y = gu.bits_of(_mx_layer(t, gu, t["xb"], t["cu"]))
    finally:
        t["enc"].set_layer_precision(["mxfp4"])
    e16 = esm.Encoder(hidden_size=t["H"], num_attention_heads=t["heads"], intermediate_size=4 * t["H"],
                      num_hidden_layers=1)
    try:
        y16 = gu.bits_of(e16.layer_fwd(t["wd"], gu.to_dev_bf16(t["xb"]), gu.to_dev_i32(t["cu"]), 3, t["T"],
                                       int(t["lengths"].max())))
    finally:
        e16.close()
    assert np.array_equal(y, y16)


def test_mxfp4_encoder_rejects_unprepared_layers_and_bad_shapes(gu):
    enc = esm.Encoder(hidden_size=512, num_attention_heads=8, intermediate_size=2048, num_hidden_layers=2,
                      precision="mxfp4")
    try:
        w = [gu.layer_weights(512, 2048, layer=l)[0] for l in range(2)]
        x = gu.to_dev_bf16(D.make_hidden(40, 512))
        with pytest.raises(esm.EsmError, match="MXFP4 weights of layer 0 not prepared"):
            enc.layer_fwd(w[0], x, gu.to_dev_i32([0, 40]), 1, 40, 40)
    finally:
        enc.close()
    with pytest.raises(esm.EsmError):   # 320 is not a multiple of 256
        esm.Encoder(hidden_size=320, num_attention_heads=5, intermediate_size=1280, num_hidden_layers=1,
                    precision="mxfp4")


@pytest.mark.parametrize("epi", [esm.EPI_BIAS_RESIDUAL, esm.EPI_BIAS_GELU])
def test_mxfp4_linear_tall_tiles_sampled(enc, gu, epi):
    """M = 32293, N = 1280: the GEMM takes 320-row tiles (fewer rounds of
    workgroups); sampled rows, the last partial tile included, against the
    oracle on the same rows (rows are independent)."""
    from oracle import esm_oracle as O
    M, N, K = 32293, 1280, 512
    rng = np.random.default_rng(17)
    xb = D.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wb = D.to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    bb = D.to_bf16_bits((rng.standard_normal(N) * 0.02).astype(np.float32))
    rb = D.to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    res = gu.to_dev_bf16(rb) if epi == esm.EPI_BIAS_RESIDUAL else None
    got = gu.from_dev(enc.linear_mxfp4_fwd(enc.mxfp4_quantize(gu.to_dev_bf16(xb)), enc.mxfp4_quantize(gu.to_dev_bf16(wb)),
                                           gu.to_dev_bf16(bb), residual=res, epilogue=epi))
    rows = np.unique(np.concatenate([np.arange(0, 640), rng.integers(0, M, 1500), np.arange(M - 400, M)]))
    ref = F.mx_matmul(*F.mx_quantize(D.bf16_bits_to_f64(xb[rows])), *F.mx_quantize(D.bf16_bits_to_f64(wb)))
    ref = ref + D.bf16_bits_to_f64(bb)
    if epi == esm.EPI_BIAS_GELU:
        ref = O.gelu(ref)
    else:
        ref = ref + D.bf16_bits_to_f64(rb[rows])
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max()
    assert np.all(np.abs(got[rows] - ref) <= bound), np.abs(got[rows] - ref).max()
