"""Parity of the GELU backward (esm_gelu_bwd) and of the QKV-split / RoPE
backward (esm_qkv_rope_bwd) against the fp64 oracle (oracle/esm_oracle.py:
gelu_bwd, qkv_rope_bwd), through the C ABI.

Tolerances.  GELU: fp32 erf and exp (a few ulp) and one bf16 rounding of the
product: |err| <= 2^-8 |ref| + 1e-6 |dy| per element.  RoPE: a rotation of
bf16 values by fp32 cos/sin from the forward's table, one bf16 rounding:
max|err| / max|ref| <= 4e-3; v is copied bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import esm_oracle as O
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


@pytest.mark.parametrize("n,scale", [(8, 1.0), (4096, 3.0), (32293 * 64, 2.0)])
def test_gelu_bwd(gu, enc, n, scale):
    r = np.random.default_rng(n)
    z = r.standard_normal(n) * scale
    z[:8] = [0.0, -0.7518, 1.0, -1.0, 9.5, -9.5, 30.0, -30.0][:min(8, n)]
    zb = D.to_bf16_bits(z.astype(np.float32))
    db = D.to_bf16_bits(r.standard_normal(n).astype(np.float32))
    dz = enc.gelu_bwd(gu.to_dev_bf16(zb), gu.to_dev_bf16(db))
    got = gu.from_dev(dz)
    dyf = D.bf16_bits_to_f64(db)
    ref = O.gelu_bwd(D.bf16_bits_to_f64(zb), dyf)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(dyf))


@pytest.mark.parametrize("lens", [[17, 64, 100, 200], [1, 1026, 3], [255, 256, 257]])
def test_qkv_rope_bwd(gu, enc, lens):
    heads = 5
    cu = D.cu_from_lengths(lens)
    T = int(cu[-1])
    r = np.random.default_rng(sum(lens))
    planar = D.to_bf16_bits(r.standard_normal((3, heads, T, 64)).astype(np.float32))
    dy = enc.qkv_rope_bwd(gu.to_dev_bf16(planar), gu.to_dev_i32(cu), len(lens), T)
    got = gu.from_dev(dy)
    f = D.bf16_bits_to_f64(planar).transpose(0, 2, 1, 3)   # [3, T, heads, 64]
    ref = O.qkv_rope_bwd(f[0], f[1], f[2], cu)
    assert gu.rel_err(got, ref) < 4e-3
    # v columns (c = 2) are the planar v, bit for bit
    gv = gu.bits_of(dy).reshape(T, heads, 3, 64)[:, :, 2, :]
    assert np.array_equal(gv, planar[2].transpose(1, 0, 2))


def test_qkv_rope_bwd_after_attention_bwd(gu, enc):
    """The two compose: attention backward's dqkv through esm_qkv_rope_bwd
    equals the oracle's qkv_rope_bwd of the oracle's attention gradients."""
    lens, heads = [130, 7, 300], 5
    cu = D.cu_from_lengths(lens)
    T = int(cu[-1])
    r = np.random.default_rng(77)
    planar = D.to_bf16_bits(r.standard_normal((3, heads, T, 64)).astype(np.float32))
    g = D.to_bf16_bits(r.standard_normal((T, heads * 64)).astype(np.float32))
    qkv, cu_d = gu.to_dev_bf16(planar), gu.to_dev_i32(cu)
    ctx, lse = enc.attention_fwd_lse(qkv, cu_d, len(lens), T)
    dqkv = enc.attention_bwd(qkv, ctx, gu.to_dev_bf16(g), lse, cu_d, len(lens), T)
    dy = gu.from_dev(enc.qkv_rope_bwd(dqkv, cu_d, len(lens), T))
    f = D.bf16_bits_to_f64(planar).transpose(0, 2, 1, 3)
    dq, dk, dv = O.attention_bwd(f[0], f[1], f[2], D.bf16_bits_to_f64(g), cu)
    assert gu.rel_err(dy, O.qkv_rope_bwd(dq, dk, dv, cu)) < 1e-2
