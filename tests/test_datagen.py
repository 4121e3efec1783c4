"""Seed-0 workloads reproduce the documented batches, and the bf16 rounding
used for every input agrees with torch's float32 -> bfloat16 conversion."""
import numpy as np
import torch

from protein_language_model_amd import datagen as D


def test_seed0_batches():
    b1 = D.make_batch(D.WORKLOADS["tiny"])
    assert b1.lengths.tolist() == [17, 64, 100, 200] and b1.T == 381
    assert b1.ids[:8].tolist() == [17, 29, 32, 18, 9, 26, 7, 31]
    b2 = D.make_batch(D.WORKLOADS["650m_layer"])
    L = b2.lengths
    assert (b2.B, b2.T, L.min(), L.max()) == (46, 15530, 74, 744)
    assert L[:5].tolist() == [324, 277, 441, 319, 218]
    assert int((L.astype(np.int64) ** 2).sum()) == 6522882
    assert b2.hidden.shape == (15530, 1280) and b2.hidden.dtype == np.uint16
    b3 = D.make_batch(D.WORKLOADS["650m"])
    L = b3.lengths
    assert (b3.B, b3.T, L.min(), L.max(), L[-1]) == (87, 32293, 74, 997, 425)
    assert int((L.astype(np.int64) ** 2).sum()) == 16024465
    assert b3.cu_seqlens[0] == 0 and b3.cu_seqlens[-1] == 32293 and b3.cu_seqlens.dtype == np.int32
    L4 = D.draw_lengths(0, 400, budget=16384)
    assert (len(L4), sum(L4), min(L4), max(L4)) == (39, 16208, 99, 908)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32) * 3,
        ((r.integers(0, 2**32, 5000, dtype=np.uint64) & 0xFFFF0000) | 0x8000).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(D.to_bf16_bits(x), ref)
    assert np.array_equal(D.bf16_bits_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_weights_shapes_and_determinism():
    w = D.make_layer_weights(320, 1280, 0)
    assert w["w_qkv"].shape == (960, 320) and w["w_fc2"].shape == (320, 1280)
    w2 = D.make_layer_weights(320, 1280, 0)
    assert all(np.array_equal(w[k], w2[k]) for k in w)
    assert not np.array_equal(w["w_qkv"], D.make_layer_weights(320, 1280, 1)["w_qkv"])
    std = D.bf16_bits_to_f64(w["w_fc1"]).std()
    assert abs(std - 0.02) < 5e-4
