"""Kernel-level parity of the HIP path (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

from oracle import esm_oracle as O
from protein_language_model_amd import datagen as D
from protein_language_model_amd import esm

pytestmark = pytest.mark.gpu

TOL = 1e-2  # max|gpu - ref| / max|ref|


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


@pytest.fixture(scope="module")
def enc_tiny():
    e = esm.Encoder(hidden_size=320, num_attention_heads=5, intermediate_size=1280, num_hidden_layers=1)
    yield e
    e.close()


@pytest.fixture(scope="module")
def enc_650m():
    e = esm.Encoder(num_hidden_layers=1)
    yield e
    e.close()


def _rand_bits(shape, seed, scale=1.0):
    return D.to_bf16_bits((np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (381, 960, 320), (257, 320, 1280), (300, 1280, 320),
                                   (5000, 1280, 1280)])
@pytest.mark.parametrize("epi", [esm.EPI_BIAS, esm.EPI_BIAS_GELU, esm.EPI_BIAS_RESIDUAL])
def test_linear(gu, enc_tiny, M, N, K, epi):
    xb, wb, bb, rb = _rand_bits((M, K), 1), _rand_bits((N, K), 2, 0.05), _rand_bits((N,), 3), _rand_bits((M, N), 4)
    x, w, b, r = (gu.to_dev_bf16(a) for a in (xb, wb, bb, rb))
    y = enc_tiny.linear_fwd(x, w, b, residual=r if epi == esm.EPI_BIAS_RESIDUAL else None, epilogue=epi)
    z = D.bf16_bits_to_f64(xb) @ D.bf16_bits_to_f64(wb).T + D.bf16_bits_to_f64(bb)
    if epi == esm.EPI_BIAS_GELU:
        z = O.gelu(z)
    if epi == esm.EPI_BIAS_RESIDUAL:
        z = z + D.bf16_bits_to_f64(rb)
    err = gu.rel_err(gu.from_dev(y), z)
    assert err < 4e-3, err


def test_gelu_epilogue_elementwise(gu, enc_650m):
    """GELU epilogue on pre-activations known exactly: W picks one input column
    per output (z[m, n] = x[m, n % 64], no bias), so z spans [-12, 12] with no
    GEMM rounding.  Each output must be the exact z Phi(z) up to one bf16
    rounding (2^-8 relative) plus the epilogue's tail error (1e-7 |z|), and
    carry the sign of z."""
    M, N, K = 4096, 256, 64
    rng = np.random.default_rng(21)
    z = np.concatenate([rng.uniform(-12, 12, M * K // 2), rng.standard_normal(M * K // 2) * 3]).reshape(M, K)
    xb = D.to_bf16_bits(z.astype(np.float32))
    wf = np.zeros((N, K), np.float32)
    wf[np.arange(N), np.arange(N) % K] = 1.0
    y = enc_650m.linear_fwd(gu.to_dev_bf16(xb), gu.to_dev_bf16(D.to_bf16_bits(wf)), gu.to_dev_bf16(D.to_bf16_bits(np.zeros(N, np.float32))),
                            epilogue=esm.EPI_BIAS_GELU)
    got = gu.from_dev(y)
    zz = D.bf16_bits_to_f64(xb)[:, np.arange(N) % K]
    ref = O.gelu(zz)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-7 * np.abs(zz) + 1e-38
    excess = np.abs(got - ref) / bound
    assert excess.max() <= 1.0, (excess.max(), zz.flat[excess.argmax()])
    neg = (zz < 0) & (np.abs(ref) > 1e-30)
    assert np.all(np.signbit(got[zz < 0])) and np.all(got[neg] < 0)


def test_linear_large_tiles_and_in_place_residual(gu, enc_650m):
    # Enough tiles for the 256x256 configuration; residual aliases the output.
    M, N, K = 4200, 5120, 1280
    xb, wb, rb = _rand_bits((M, K), 5), _rand_bits((N, K), 6, 0.05), _rand_bits((M, N), 7)
    x, w, r = gu.to_dev_bf16(xb), gu.to_dev_bf16(wb), gu.to_dev_bf16(rb)
    y = enc_650m.linear_fwd(x, w, None, residual=r, epilogue=esm.EPI_BIAS_RESIDUAL, y=r)
    rows = np.random.default_rng(0).choice(M, 64, replace=False)
    z = D.bf16_bits_to_f64(xb[rows]) @ D.bf16_bits_to_f64(wb).T + D.bf16_bits_to_f64(rb[rows])
    assert gu.rel_err(gu.from_dev(y)[rows], z) < 4e-3


@pytest.mark.parametrize("epi", [esm.EPI_BIAS, esm.EPI_BIAS_GELU, esm.EPI_BIAS_RESIDUAL])
def test_linear_tile_shape_does_not_change_rows(gu, enc_650m, epi):
    """At M = 15530, N = 1280 the 320-row tiles take fewer rounds and are used;
    a 1000-row slice takes 256-row tiles.  Every row must come out bit for bit
    the same, and match the fp64 product on a sample."""
    M, N, K, Ms = 15530, 1280, 1280, 1000
    xb, wb, bb, rb = _rand_bits((M, K), 11), _rand_bits((N, K), 12, 0.05), _rand_bits((N,), 13), _rand_bits((M, N), 14)
    x, w, b, r = (gu.to_dev_bf16(a) for a in (xb, wb, bb, rb))
    res = epi == esm.EPI_BIAS_RESIDUAL
    y = gu.bits_of(enc_650m.linear_fwd(x, w, b, residual=r if res else None, epilogue=epi))
    ys = gu.bits_of(enc_650m.linear_fwd(x[:Ms].contiguous(), w, b, residual=r[:Ms].contiguous() if res else None,
                                        epilogue=epi))
    assert np.array_equal(y[:Ms], ys)
    rows = np.random.default_rng(1).choice(M, 96, replace=False)
    z = D.bf16_bits_to_f64(xb[rows]) @ D.bf16_bits_to_f64(wb).T + D.bf16_bits_to_f64(bb)
    if epi == esm.EPI_BIAS_GELU:
        z = O.gelu(z)
    if res:
        z = z + D.bf16_bits_to_f64(rb[rows])
    assert gu.rel_err(D.bf16_bits_to_f64(y[rows]), z) < 4e-3


@pytest.mark.parametrize("H,M", [(320, 381), (1280, 1000), (2560, 77)])
def test_layernorm(gu, H, M):
    e = esm.Encoder(hidden_size=H, num_attention_heads=H // 64, intermediate_size=4 * H, num_hidden_layers=1)
    xb = D.to_bf16_bits((np.random.default_rng(1).standard_normal((M, H)) * 3 + 0.5).astype(np.float32))
    ln = D.random_layernorm_params(H, 2)
    y = e.layernorm_fwd(gu.to_dev_bf16(xb), gu.to_dev_bf16(ln["ln1_gamma"]), gu.to_dev_bf16(ln["ln1_beta"]))
    ref = O.layer_norm(D.bf16_bits_to_f64(xb), D.bf16_bits_to_f64(ln["ln1_gamma"]),
                       D.bf16_bits_to_f64(ln["ln1_beta"]), 1e-5)
    assert gu.rel_err(gu.from_dev(y), ref) < 4e-3
    e.close()


@pytest.mark.parametrize("lens", [[17, 64, 100, 200], [0, 5, 0, 1026, 1, 128, 129, 0], [1], [300] * 40,
                                  [255, 256, 257, 512, 513]])
def test_segment_table_thd(gu, enc_tiny, lens):
    cu = D.cu_from_lengths(lens)
    T, B = int(cu[-1]), len(lens)
    ws = enc_tiny.segment_table(esm.LAYOUT_THD, gu.to_dev_i32(cu), B, T)
    torch.cuda.synchronize()
    pos = enc_tiny.workspace_region(ws, T, B, "pos").cpu().numpy()
    assert np.array_equal(pos, O.positions(cu))
    segs = enc_tiny.workspace_region(ws, T, B, "segs").cpu().numpy().reshape(B, 2)
    assert np.array_equal(segs[:, 0], cu[:-1]) and np.array_equal(segs[:, 1], lens)
    n = int(enc_tiny.workspace_region(ws, T, B, "ntiles").cpu().numpy()[0])
    tiles = enc_tiny.workspace_region(ws, T, B, "tiles").cpu().numpy().reshape(-1, 2)[:n]
    ref = O.query_tiles(lens, esm.ATTN_TILE_ROWS)
    # unique: the set of tiles; valid: lengths non-increasing along the list
    assert sorted(map(tuple, tiles.tolist())) == sorted(ref)
    L = [lens[s] for s, _ in tiles]
    assert L == sorted(L, reverse=True)


def test_segment_table_bshd(gu, enc_tiny):
    lens, S = [3, 0, 8, 5], 8
    ws = enc_tiny.segment_table(esm.LAYOUT_BSHD, gu.to_dev_i32(lens), 4, 0, S)
    torch.cuda.synchronize()
    pos = enc_tiny.workspace_region(ws, 32, 4, "pos").cpu().numpy().reshape(4, S)
    ref = np.array([[p if p < L else -1 for p in range(S)] for L in lens])
    assert np.array_equal(pos, ref)


def _attention_case(gu, enc, lens, seed, qscale=1.0):
    H = enc.hidden
    heads = H // 64
    cu = D.cu_from_lengths(lens)
    T = int(cu[-1])
    r = np.random.default_rng(seed)
    q = D.to_bf16_bits((r.standard_normal((T, heads, 64)) * qscale).astype(np.float32))
    k = D.to_bf16_bits(r.standard_normal((T, heads, 64)).astype(np.float32))
    v = D.to_bf16_bits(r.standard_normal((T, heads, 64)).astype(np.float32))
    planar = np.stack([a.transpose(1, 0, 2) for a in (q, k, v)])  # [3, heads, T, 64]
    ctx = enc.attention_fwd(gu.to_dev_bf16(planar), gu.to_dev_i32(cu), len(lens), T)
    ref = O.attention(D.bf16_bits_to_f64(q), D.bf16_bits_to_f64(k), D.bf16_bits_to_f64(v), cu)
    return gu.from_dev(ctx), ref


@pytest.mark.parametrize("lens", [[17, 64, 100, 200], [1, 2, 63, 64, 65, 127, 128, 129], [1026, 0, 3], [700, 5],
                                  [255, 256, 257, 31, 33, 224, 225]])
def test_attention(gu, enc_tiny, lens):
    got, ref = _attention_case(gu, enc_tiny, lens, 11)
    assert gu.rel_err(got, ref) < TOL


def test_attention_large_logits(gu, enc_tiny):
    got, ref = _attention_case(gu, enc_tiny, [300, 41], 12, qscale=30.0)
    assert gu.rel_err(got, ref) < TOL


def test_attention_packed_equals_alone_bitexact(gu, enc_tiny):
    lens = [130, 7, 64, 250]
    H, heads = 320, 5
    cu = D.cu_from_lengths(lens)
    T = int(cu[-1])
    r = np.random.default_rng(3)
    planar = D.to_bf16_bits(r.standard_normal((3, heads, T, 64)).astype(np.float32))
    full = gu.bits_of(enc_tiny.attention_fwd(gu.to_dev_bf16(planar), gu.to_dev_i32(cu), len(lens), T))
    for s, L in enumerate(lens):
        a = int(cu[s])
        one = gu.bits_of(enc_tiny.attention_fwd(gu.to_dev_bf16(np.ascontiguousarray(planar[:, :, a:a + L])),
                                                gu.to_dev_i32([0, L]), 1, L))
        assert np.array_equal(one, full[a:a + L])
