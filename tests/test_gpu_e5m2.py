"""FP8 backward pieces of the HYBRID recipe through the C ABI: the E5M2 cast
of a gradient (esm_e5m2_quantize) bit-exact against the oracle's codec
(oracle/fp8_ref.py: e5m2_encode, with x * scale formed in float32 on both
sides), and the E5M2 x E4M3 data-gradient and weight-gradient GEMMs
(esm_linear_e5m2_dgrad, esm_linear_e5m2_wgrad) against the exact fp64
product of the decoded operands (bf16 output: max|err| / max|ref| <= 4e-3,
a bf16 rounding of 2^-9 plus fp32 accumulation)."""
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


def _e5m2_edge_inputs():
    """bf16 inputs around every decision the cast makes: every finite E5M2
    value, every midpoint between neighbours (3 mantissa bits: exact in
    bf16) and the bf16 values either side of it, subnormals (|x| < 2^-14)
    down to the deepest underflow, the saturation edge (57344, the midpoint
    61440 towards the next binade, and beyond), infinities, NaN of both
    signs, signed zero."""
    vals = F8.e5m2_decode_table()[:0x7C]
    mids = (vals[:-1] + vals[1:]) / 2
    mb = D.to_bf16_bits(mids.astype(np.float32)).astype(np.int64)
    assert np.array_equal(D.bf16_bits_to_f64(mb.astype(np.uint16)), mids)        # midpoints are bf16 values
    pos = np.concatenate([D.to_bf16_bits(vals.astype(np.float32)).astype(np.int64), mb, mb - 1, mb + 1,
                          D.to_bf16_bits(np.array([57344, 61440, 61184, 61696, 65536, 1e6, 3e38, 2.0 ** -17,
                                                   2.0 ** -17 * 1.5, 2.0 ** -18, 1e-30, 2.0 ** -14 * 0.875],
                                                  np.float32)).astype(np.int64),
                          np.array([0x7F80, 0x7FC0, 0x7F81, 0x0001], np.int64)])     # +inf, NaNs, tiniest bf16
    bits = np.concatenate([pos, pos | 0x8000, [0x8000]]).astype(np.uint16)
    pad = (-bits.size) % 8
    return np.concatenate([bits, np.zeros(pad, np.uint16)])


@pytest.mark.parametrize("scale", [1.0, 0.25, 8.0])
def test_e5m2_quantize_edges_bitexact(gu, enc, scale):
    """Power-of-two scales keep x * s exact, so every input sits exactly where
    the edge set put it (relative to the scaled grid)."""
    xb = _e5m2_edge_inputs()
    s = torch.tensor([scale], dtype=torch.float32, device="cuda:0")
    y8, amax = enc.e5m2_quantize(gu.to_dev_bf16(xb), s)
    torch.cuda.synchronize()
    got = y8.cpu().numpy()
    xf = D.bf16_bits_to_f64(xb).astype(np.float32)
    ref = F8.e5m2_encode((xf * np.float32(scale)).astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(int(xb[i])), int(got[i]), int(ref[i])) for i in bad[:12]]
    nan = np.isnan(xf)
    assert nan.any() and np.all(got[nan] == 0x7F)
    # amax over the non-NaN inputs (infinities included)
    assert amax.cpu().numpy().view(np.float32)[0] == np.abs(xf[~nan]).max()


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


def test_linear_e5m2_dgrad_320_row_tiles_at_the_650m_shape(gu, enc):
    """At M = 32293 rows, 1280 outputs and a 5120-long contraction the
    dispatch takes the 320-row tiles (fewer rounds over the compute units);
    the last tile is ragged (32293 = 100 * 320 + 293).  Sampled rows,
    including the first and last of every kind of tile, against the exact
    product of the decoded operands."""
    M, N, K = 32293, 5120, 1280
    r = np.random.default_rng(11)
    s_dy, s_w = 32.0, 448.0 / 0.1
    dy8 = F8.e5m2_encode(r.standard_normal((M, N)) * s_dy)
    wt8 = F8.e4m3_encode(np.clip(r.standard_normal((K, N)) * 0.02, -0.1, 0.1) * s_w)
    dev = "cuda:0"
    dx = enc.linear_e5m2_dgrad(torch.from_numpy(dy8).to(dev), torch.tensor([s_dy], device=dev),
                               torch.from_numpy(wt8).to(dev), torch.tensor([s_w], dtype=torch.float32, device=dev))
    rows = np.unique(np.concatenate([[0, 1, 319, 320, 639, 31999, 32000, 32292],
                                     r.choice(M, 120, replace=False)]))
    ref = (F8.e5m2_to_f64(dy8[rows]) / s_dy) @ (F8.e4m3_to_f64(wt8) / np.float64(np.float32(s_w))).T
    assert gu.rel_err(gu.from_dev(dx)[rows], ref) < 4e-3


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (381, 1280, 320), (1000, 5120, 1280), (4097, 320, 1280)])
def test_linear_e5m2_wgrad(gu, enc, M, N, K):
    """dW = (dy8 / s_dy)^T (x8 / s_x) against the exact product of the decoded
    operands; M = 4097 takes the split-K path (slices summed, then
    dequantised once)."""
    r = np.random.default_rng(M + 3 * N + K)
    s_dy, s_x = 64.0, 448.0 / 4.0
    dy8 = F8.e5m2_encode(r.standard_normal((M, N)) * s_dy)
    x8 = F8.e4m3_encode(np.clip(r.standard_normal((M, K)), -4, 4) * s_x)
    dev = "cuda:0"
    dw = enc.linear_e5m2_wgrad(torch.from_numpy(dy8).to(dev), torch.tensor([s_dy], device=dev),
                               torch.from_numpy(x8).to(dev), torch.tensor([s_x], dtype=torch.float32, device=dev))
    ref = (F8.e5m2_to_f64(dy8) / s_dy).T @ (F8.e4m3_to_f64(x8) / np.float64(np.float32(s_x)))
    assert gu.rel_err(gu.from_dev(dw), ref) < 4e-3


def test_linear_e5m2_wgrad_at_the_650m_fc1_shape(gu, enc):
    """fc1's weight gradient at T = 32293 (dW [5120, 1280], contraction over
    all rows in K slices); sampled rows of dW, all columns, against the exact
    product of the decoded operands."""
    M, N, K = 32293, 5120, 1280
    r = np.random.default_rng(17)
    s_dy, s_x = 8.0, 448.0 / 4.0
    dy8 = F8.e5m2_encode(r.standard_normal((M, N)) * s_dy)
    x8 = F8.e4m3_encode(np.clip(r.standard_normal((M, K)), -4, 4) * s_x)
    dev = "cuda:0"
    dw = enc.linear_e5m2_wgrad(torch.from_numpy(dy8).to(dev), torch.tensor([s_dy], device=dev),
                               torch.from_numpy(x8).to(dev), torch.tensor([s_x], dtype=torch.float32, device=dev))
    rows = np.unique(np.concatenate([[0, 255, 256, 5119], r.choice(N, 60, replace=False)]))
    ref = (F8.e5m2_to_f64(dy8[:, rows]) / s_dy).T @ (F8.e4m3_to_f64(x8) / np.float64(np.float32(s_x)))
    assert gu.rel_err(gu.from_dev(dw)[rows], ref) < 4e-3
