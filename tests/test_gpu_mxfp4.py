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
