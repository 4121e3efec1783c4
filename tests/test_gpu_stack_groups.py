"""The stack forward as two groups of whole sequences on two streams
(esm_stack_fwd with host cu_seqlens, split where esm_stack_split says): every
row's arithmetic is that of the single-stream run, so the output is the same
bit for bit, for bf16 (LayerNorm folded and not), FP8 (outputs and the
delayed-scaling state after the steps) and MXFP4 encoders, from token ids and
from hidden states, on the 650M batch (its widths, two layers: the batch
splits) and on batches whose split falls after the first or before the last
sequence.
"""
import numpy as np
import pytest
import torch

from protein_language_model_amd import datagen as D
from protein_language_model_amd import esm

pytestmark = pytest.mark.gpu

H, HEADS, F, L = 1280, 20, 5120, 2


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


def _batch(lens, seed):
    cu = D.cu_from_lengths(lens)
    T = int(cu[-1])
    ids = np.random.default_rng(seed).integers(0, 33, T).astype(np.int32)
    return cu, T, len(lens), ids


def _run(gu, enc, wd, cu, B, T, ms, ids, emb, x, host, steps=1):
    cu_d = gu.to_dev_i32(cu)
    y = None
    for _ in range(steps):
        if ids is not None:
            y = enc.stack_fwd(wd, cu_d, B, T, ms, token_ids=gu.to_dev_i32(ids), embedding=emb,
                              cu_seqlens_host=cu if host else None)
        else:
            y = enc.stack_fwd(wd, cu_d, B, T, ms, x_in=gu.to_dev_bf16(x), cu_seqlens_host=cu if host else None)
    torch.cuda.synchronize()
    return gu.bits_of(y)


@pytest.mark.parametrize("prec,fold,from_ids", [("bf16", True, True), ("bf16", False, False), ("fp8", False, True),
                                                ("mxfp4", False, False)])
def test_two_group_stack_equals_one_stream(gu, prec, fold, from_ids):
    b = D.make_batch(D.WORKLOADS["650m"])
    cu, T, B, lens = b.cu_seqlens, b.T, b.B, b.lengths
    assert esm.stack_split(H, F, cu) > 0
    ids = b.ids
    wd = [gu.layer_weights(H, F, l, seed=11, random_ln=True)[0] for l in range(L)]
    emb = gu.to_dev_bf16(D.make_embedding(33, H))
    x = D.make_hidden(T, H, 5)
    outs, states = [], []
    for host in (False, True):
        enc = esm.Encoder(hidden_size=H, num_attention_heads=HEADS, intermediate_size=F, num_hidden_layers=L,
                          precision=prec)
        try:
            if prec == "bf16" and fold:
                enc.prepare(wd)
            elif prec == "fp8":
                enc.fp8_prepare(wd)
            elif prec == "mxfp4":
                enc.mxfp4_prepare(wd)
            outs.append(_run(gu, enc, wd, cu, B, T, int(max(lens)), ids if from_ids else None, emb, x, host,
                             steps=3 if prec == "fp8" else 1))
            if prec == "fp8":
                states.append(enc.fp8_get_state())
        finally:
            enc.close()
    assert np.array_equal(outs[0], outs[1])
    if prec == "fp8":
        for k in states[0]:
            assert np.array_equal(states[0][k], states[1][k]), k


def test_group_boundary_positions(gu):
    """Batches whose split falls after the first sequence and before the last
    (one long sequence among short ones)."""
    wd = [gu.layer_weights(H, F, l, seed=2)[0] for l in range(L)]
    emb = gu.to_dev_bf16(D.make_embedding(33, H))
    short = [100] * 161 + [47]
    for lens, at in (([16146] + short, 1), (short + [16146], len(short))):
        cu, T, B, ids = _batch(lens, 7)
        assert esm.stack_split(H, F, cu) == at
        outs = []
        for host in (False, True):
            enc = esm.Encoder(hidden_size=H, num_attention_heads=HEADS, intermediate_size=F, num_hidden_layers=L,
                              max_position_embeddings=16200)
            try:
                enc.prepare(wd)
                outs.append(_run(gu, enc, wd, cu, B, T, max(lens), ids, emb, None, host))
            finally:
                enc.close()
        assert np.array_equal(outs[0], outs[1]), at
