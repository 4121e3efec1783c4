"""FP8 backward pieces of the HYBRID recipe through the C ABI: the E5M2 cast
of a gradient (esm_e5m2_quantize) bit-exact against the oracle's codec
(oracle/fp8_ref.py: e5m2_encode, with x * scale formed in float32 on both
sides), and the E5M2 x E4M3 data-gradient GEMM (esm_linear_e5m2_dgrad)
against the exact fp64 product of the decoded operands (bf16 output:
max|err| / max|ref| <= 4e-3)."""
import numpy as np
import pytest
import torch

from oracle import fp8_ref as F8
from protein_language_model_amd import datagen as D
from protein_language_model_amd import esm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


@pytest.fixture(scope="module")
def enc():
    e = esm.Encoder(hidden_size=320, num_attention_heads=5, intermediate_size=1280, num_hidden_layers=1)
    yield e
    e.close()


@pytest.mark.parametrize("n,scale", [(8, 1.0), (4096, 3.7), (262144, 4096.0)])
def test_e5m2_quantize_bitexact(gu, enc, n, scale):
    r = np.random.default_rng(n)
    x = r.standard_normal(n) * 20
    x[:4] = [0.0, -1e-9, 30.0, -25.0]           # zero, deep underflow, saturation at large scales
    xb = D.to_bf16_bits(x.astype(np.float32))
    s = torch.tensor([scale], dtype=torch.float32, device="cuda:0")
    y8, amax = enc.e5m2_quantize(gu.to_dev_bf16(xb), s)
    torch.cuda.synchronize()
    xf = D.bf16_bits_to_f64(xb).astype(np.float32)
    ref = F8.e5m2_encode((xf * np.float32(scale)).astype(np.float64))
    assert np.array_equal(y8.cpu().numpy(), ref)
    assert amax.cpu().numpy().view(np.float32)[0] == np.abs(xf).max()


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (381, 1280, 320), (1000, 5120, 1280)])
def test_linear_e5m2_dgrad(gu, enc, M, N, K):
    r = np.random.default_rng(M + N)
    s_dy, s_w = 64.0, 448.0 / 0.1
    dy8 = F8.e5m2_encode(r.standard_normal((M, N)) * s_dy)
    wt8 = F8.e4m3_encode(np.clip(r.standard_normal((K, N)) * 0.02, -0.1, 0.1) * s_w)
    dev = "cuda:0"
    dx = enc.linear_e5m2_dgrad(torch.from_numpy(dy8).to(dev), torch.tensor([s_dy], device=dev),
                               torch.from_numpy(wt8).to(dev), torch.tensor([s_w], dtype=torch.float32, device=dev))
    ref = (F8.e5m2_to_f64(dy8) / s_dy) @ (F8.e4m3_to_f64(wt8) / np.float64(np.float32(s_w))).T
    assert gu.rel_err(gu.from_dev(dx), ref) < 4e-3
