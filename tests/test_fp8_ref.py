"""Pins of the FP8 reference: the E4M3 codec against torch's float8_e4m3fn
(an independent implementation) and the OCP format's published constants,
the delayed-scaling state machine on a scripted amax sequence, and the
FP8-emulating layer against the plain layer."""
import math

import numpy as np
import pytest
import torch

from oracle import esm_oracle as O
from oracle import fp8_ref as F8


def test_decode_table_matches_torch_and_the_format_constants():
    tab = F8.e4m3_decode_table()
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(tab[ok], ref[ok])
    assert np.isnan(tab).sum() == 2 and np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert tab[0x7E] == 448.0 and tab[0x38] == 1.0
    assert tab[0x08] == 2.0 ** -6 and tab[0x01] == 2.0 ** -9
    pos = tab[:0x7F]
    assert (np.diff(pos) > 0).all()
    assert np.array_equal(tab[0x80:0xFF], -tab[:0x7F])


def _midpoints():
    pos = F8.e4m3_decode_table()[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    f32 = mids.astype(np.float32)
    return np.concatenate([f32, np.nextafter(f32, np.float32(0)), np.nextafter(f32, np.float32(1e9)), pos])


def test_encode_matches_torch_in_range():
    r = np.random.default_rng(0)
    x = np.concatenate([_midpoints(), r.standard_normal(20000) * 30, r.standard_normal(2000) * 1e-3]).astype(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F8.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_encode_saturates_and_handles_nan_and_signed_zero():
    got = F8.e4m3_encode(np.array([448.0, 463.9, 464.0, 500.0, 1e30, -1e30, np.nan, -0.0, 0.0]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F, 0x80, 0x00]


def test_encode_is_nearest_by_brute_force():
    tab = F8.e4m3_decode_table()
    fin = np.array([c for c in range(256) if not np.isnan(tab[c])])
    xs = np.random.default_rng(1).uniform(-450, 450, 3000)
    for x in xs:
        got = F8.e4m3_encode(x)
        best = np.min(np.abs(tab[fin] - min(max(x, -448), 448)))
        assert abs(tab[got] - min(max(x, -448), 448)) == best


def test_quantize_is_exact_on_the_grid():
    tab = F8.e4m3_decode_table()
    vals = tab[~np.isnan(tab)]
    s = 0.375
    assert np.array_equal(F8.quantize(vals / s, s), vals)


def test_delayed_scaling_state_machine():
    st = F8.DelayedScaling(history_len=3)
    assert st.scale == 1.0
    st.record(0.0)
    assert st.scale == 1.0          # max(history) = 0: keep the previous scale
    st.record(2.0)
    assert st.scale == 224.0
    st.record(4.0)
    assert st.scale == 112.0
    st.record(1.0)                  # history [1, 2, 4]
    assert st.scale == 112.0
    st.record(1.0)                  # history [1, 1, 4]
    assert st.scale == 112.0
    st.record(1.0)                  # history [1, 1, 1]: the 4 left the window
    assert st.scale == 448.0
    st.record(float("nan"))         # non-finite amax: keep the previous scale
    assert st.scale == 448.0
    assert F8.weight_scale(np.array([0.5, -2.0])) == 224.0


def test_delayed_scaling_of_e5m2_gradients_targets_57344():
    """The gradient state of the HYBRID recipe: the same window rule with
    E5M2's largest value (57344 = 1.75 * 2^15), so a window maximum of 2^k
    gives the scale 1.75 * 2^(15 - k), exact."""
    st = F8.DelayedScaling(history_len=2, fp8_max=F8.E5M2_MAX)
    assert st.scale == 1.0
    st.record(4.0)
    assert st.scale == 14336.0                  # 57344 / 4
    st.record(0.25)
    assert st.scale == 14336.0                  # history [4, 0.25]
    st.record(0.25)                             # history [0.25, 0.25]: the 4 left the window
    assert st.scale == 229376.0                 # 57344 / 0.25
    st.record(float("inf"))                     # non-finite: keep the scale
    assert st.scale == 229376.0
    # the scaled window maximum lands exactly on the format's largest value
    assert F8.e5m2_encode(np.array([0.25 * st.scale]))[0] == 0x7B


def _tiny(seed=0):
    r = np.random.default_rng(seed)
    H, F, heads = 128, 512, 2
    w = {"w_qkv": r.standard_normal((3 * H, H)) * 0.05, "b_qkv": r.standard_normal(3 * H) * 0.05,
         "w_out": r.standard_normal((H, H)) * 0.05, "b_out": r.standard_normal(H) * 0.05,
         "w_fc1": r.standard_normal((F, H)) * 0.05, "b_fc1": r.standard_normal(F) * 0.05,
         "w_fc2": r.standard_normal((H, F)) * 0.05, "b_fc2": r.standard_normal(H) * 0.05,
         "ln1_gamma": np.ones(H), "ln1_beta": np.zeros(H), "ln2_gamma": np.ones(H), "ln2_beta": np.zeros(H)}
    x = r.standard_normal((20, H))
    return x, np.array([0, 7, 20]), w, heads


def test_fp8_layer_is_close_to_the_plain_layer_and_scales_settle():
    x, cu, w, heads = _tiny()
    states, out = F8.run_delayed_scaling(x, cu, w, heads, steps=3, history_len=16)
    ref = O.layer_forward(x, cu, w, heads)
    err = O.rel_max_err(out, ref)
    assert 1e-4 < err < 6e-2, err       # really quantised, and within the FP8 gate
    # after the first step every activation scale is 448 / amax of that tensor
    _, amax = F8.layer_forward_fp8(x, cu, w, heads, {n: s.scale for n, s in states.items()}, return_amax=True)
    for n in F8.ACT_NAMES:
        assert math.isclose(states[n].scale, 448.0 / max(states[n].history), rel_tol=0)
        assert abs(states[n].scale * amax[n] / 448.0 - 1) < 0.05


def test_fp8_layer_first_step_uses_unit_scales():
    x, cu, w, heads = _tiny(1)
    y = F8.layer_forward_fp8(x, cu, w, heads, {n: 1.0 for n in F8.ACT_NAMES})
    assert np.isfinite(y).all()


# ---------------------------------------------------------------- E5M2

def test_e5m2_decode_table_matches_torch():
    import torch
    codes = torch.arange(256, dtype=torch.int16).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    got = F8.e5m2_decode_table()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    assert F8.e5m2_to_f64([0x7B])[0] == 57344.0 and F8.e5m2_to_f64([0x01])[0] == 2.0 ** -16
    assert np.isinf(F8.e5m2_to_f64([0x7C])[0])


def test_e5m2_encode_matches_torch_in_range_and_saturates():
    import torch
    # float32 inputs (exact in both; torch casts float64 through float32, which
    # would move a value just below a midpoint onto it): every value, every
    # midpoint and its float32 neighbours, random values
    vals = F8.e5m2_decode_table()[:0x7C].astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([vals, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
                        (np.random.default_rng(5).standard_normal(4000) * 300).astype(np.float32)])
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 57344.0]
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(F8.e5m2_encode(x.astype(np.float64)), ref)
    # saturation (the reading): beyond the largest finite value -> +-57344
    assert list(F8.e5m2_encode([1e6, -61440.0, 60000.0])) == [0x7B, 0xFB, 0x7B]
    # nearest by brute force
    r = np.random.default_rng(6).uniform(-6e4, 6e4, 500)
    fin = F8.e5m2_decode_table()[np.r_[0:0x7C, 0x80:0xFC]]
    best = fin[np.argmin(np.abs(np.minimum(np.abs(r), 57344.0)[:, None] * np.sign(r)[:, None] - fin[None, :]), axis=1)]
    assert np.all(np.abs(F8.e5m2_to_f64(F8.e5m2_encode(r)) - np.clip(r, -57344, 57344))
                  <= np.abs(best - np.clip(r, -57344, 57344)) + 0.0)
