"""FP8 reference for the ESM-2 encoder: E4M3 codec, per-tensor delayed
scaling, an FP8-emulating layer, and the E5M2 codec of the gradients.

TEST INFRASTRUCTURE.  Only the test suite and the benchmark's CPU-baseline leg
use this module; it shares no code with the HIP path.

Pages cited (title, section):
  [BIO-ACC] "生物大模型训练加速实战：基于PyTorch与NVIDIA BioNeMo的Transformer优化指南",
            2.1 (dynamic FP8 managed by the DelayedScaling algorithm) and 4.1
            (DelayedScaling with the HYBRID format: E4M3 in the forward pass;
            amax history; "max" as the amax algorithm).
  [TE-RU]   TransformerEngine tutorial summary (aikraft.ru), "Рецепт FP8: Delayed
            Scaling" (history length 16, algorithm "max").
  [TE-ESM2] "深入源码NVIDIA ESM-2 TransformerEngine优化的实现原理与技术细节",
            FP8与FP4混合精度支持 (model-level FP8 recipe).

Readings (the pages give names, not formulas):
  * E4M3 is the OCP 8-bit format: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    exponent 0 is subnormal (m/8 * 2^-6); the all-ones pattern S.1111.111 is
    NaN; there is no infinity; the largest finite value is 448.
  * Casting to E4M3 rounds to nearest, ties to even, and saturates to +-448.
  * Per-tensor scaling: q = cast(x * s), dequantised x ~ q / s, with
    s = 448 / max(amax history) (margin 0).  The history holds the amax of the
    previous steps (zero-initialised, length 16); while its maximum is 0 or not
    finite the previous scale is kept (initial scale 1).  Step n quantises with
    the scale computed from steps < n and then records its own amax.
  * Weights use s = 448 / amax(W) from the start.
  * The FP8 tensors are the inputs of the four GEMMs of a layer (LayerNorm-1
    output, attention context, LayerNorm-2 output, GELU output, and the four
    weights); attention, LayerNorm and every GEMM output stay in higher
    precision.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

from . import esm_oracle as O

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 E4M3 codes (NaN for the two NaN codes)."""
    vals = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()
# Non-negative finite codes in increasing value: 0x00 .. 0x7E.
_POS_CODES = np.arange(0x7F)
_POS_VALS = _TABLE[_POS_CODES]


def e4m3_encode(x) -> np.ndarray:
    """Round each value (float64) to the nearest E4M3 code, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    a_sat = np.minimum(a, E4M3_MAX)
    # index of the largest representable value <= a
    lo = np.clip(np.searchsorted(_POS_VALS, a_sat, side="right") - 1, 0, len(_POS_VALS) - 1)
    hi = np.minimum(lo + 1, len(_POS_VALS) - 1)
    vlo, vhi = _POS_VALS[lo], _POS_VALS[hi]
    dlo, dhi = a_sat - vlo, vhi - a_sat
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    out[...] = code | sign
    nan = np.isnan(x)
    out[nan] = 0x7F
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def quantize(x, scale: float) -> np.ndarray:
    """Value of cast_e4m3(x * scale), as float64 (still scaled)."""
    return e4m3_to_f64(e4m3_encode(np.asarray(x, np.float64) * scale))


# ---------------------------------------------------------------- E5M2
# The HYBRID format of [BIO-ACC] 4.1 keeps E4M3 for the forward and uses E5M2
# for gradients.  Reading: OCP E5M2, 1 sign, 5 exponent (bias 15), 2 mantissa
# bits; exponent 0 is subnormal (m/4 * 2^-14); exponent 31 holds +-inf
# (mantissa 0) and NaN; the largest finite value is 57344.  Casting rounds to
# nearest, ties to even, and saturates to +-57344 (as the E4M3 cast does).
E5M2_MAX = 57344.0


def e5m2_decode_table() -> np.ndarray:
    """float64 value of each of the 256 E5M2 codes."""
    vals = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 2) & 0x1F
        m = c & 0x3
        if e == 0x1F:
            vals[c] = s * np.inf if m == 0 else np.nan
        elif e == 0:
            vals[c] = s * (m / 4.0) * 2.0 ** -14
        else:
            vals[c] = s * (1.0 + m / 4.0) * 2.0 ** (e - 15)
    return vals


_TABLE52 = e5m2_decode_table()
_POS_CODES52 = np.arange(0x7C)          # 0 .. 57344, increasing
_POS_VALS52 = _TABLE52[_POS_CODES52]


def e5m2_encode(x) -> np.ndarray:
    """Nearest E5M2 code of each value (ties to the even code), saturating at
    +-57344; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a_sat = np.minimum(np.abs(x), E5M2_MAX)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    lo = np.clip(np.searchsorted(_POS_VALS52, a_sat, side="right") - 1, 0, len(_POS_VALS52) - 1)
    hi = np.minimum(lo + 1, len(_POS_VALS52) - 1)
    dlo, dhi = a_sat - _POS_VALS52[lo], _POS_VALS52[hi] - a_sat
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((_POS_CODES52[hi] & 1) == 0))
    out = (np.where(pick_hi, _POS_CODES52[hi], _POS_CODES52[lo]).astype(np.uint8) | sign).astype(np.uint8)
    out[np.isnan(x)] = 0x7F
    return out


def e5m2_to_f64(codes) -> np.ndarray:
    return _TABLE52[np.asarray(codes, dtype=np.uint8)]


class DelayedScaling:
    """Per-tensor delayed scaling with an amax history and the max algorithm.

    fp8_max is the largest finite value of the tensor's format: E4M3's 448 for
    the forward's activations, E5M2's 57344 for the HYBRID recipe's gradients
    ([BIO-ACC] 4.1: E4M3 forward, E5M2 backward), so that the scaled amax of
    the window lands on the format's largest value."""

    def __init__(self, history_len: int = 16, fp8_max: float = E4M3_MAX):
        self.history = np.zeros(history_len)
        self.pos = 0
        self.scale = 1.0
        self.fp8_max = fp8_max

    def record(self, amax: float) -> None:
        """End of a step: push its amax and recompute the scale for the next."""
        self.history[self.pos] = amax
        self.pos = (self.pos + 1) % len(self.history)
        m = float(np.max(self.history))
        if m > 0 and math.isfinite(m):
            self.scale = self.fp8_max / m


def weight_scale(w) -> float:
    amax = float(np.max(np.abs(w)))
    return E4M3_MAX / amax if amax > 0 else 1.0


ACT_NAMES = ("ln1", "ctx", "ln2", "act")


def layer_forward_fp8(x, cu_seqlens, w: Dict[str, np.ndarray], heads: int, act_scales: Dict[str, float],
                      return_amax: bool = False):
    """One pre-LN layer with the four GEMM inputs and weights cast to E4M3.

    Y = (Q(a s_a) . Q(W s_w)^T) / (s_a s_w) + b for each linear; everything
    else as in the plain layer.  Returns the output and, when asked, the amax
    of each activation tensor before quantisation."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    F = w["w_fc1"].shape[0]
    amax = {}

    def lin(a, name_a, wname, bname, n_out):
        s_a = act_scales[name_a]
        s_w = weight_scale(w[wname])
        amax[name_a] = float(np.max(np.abs(a))) if a.size else 0.0
        qa = quantize(a, s_a)
        qw = quantize(w[wname], s_w)
        b = w.get(bname)
        return qa @ qw.T / (s_a * s_w) + (np.zeros(n_out) if b is None else b)

    h1 = O.layer_norm(x, w["ln1_gamma"], w["ln1_beta"])
    y = lin(h1, "ln1", "w_qkv", "b_qkv", 3 * H)
    q, k, v = O.split_qkv(y, heads)
    pos = O.positions(cu_seqlens)
    ctx = O.attention(O.apply_rope(q, pos), O.apply_rope(k, pos), v, cu_seqlens)
    x1 = x + lin(ctx, "ctx", "w_out", "b_out", H)
    h2 = O.layer_norm(x1, w["ln2_gamma"], w["ln2_beta"])
    a = O.gelu(lin(h2, "ln2", "w_fc1", "b_fc1", F))
    x2 = x1 + lin(a, "act", "w_fc2", "b_fc2", H)
    return (x2, amax) if return_amax else x2


def run_delayed_scaling(x, cu_seqlens, w, heads: int, steps: int, history_len: int = 16):
    """Repeat the same layer forward `steps` times under delayed scaling (each
    step uses the scales from the previous steps, then records its amax).
    Returns the states and the output of the last step."""
    states = {n: DelayedScaling(history_len) for n in ACT_NAMES}
    out = None
    for _ in range(steps):
        scales = {n: states[n].scale for n in ACT_NAMES}
        out, amax = layer_forward_fp8(x, cu_seqlens, w, heads, scales, return_amax=True)
        for n in ACT_NAMES:
            states[n].record(amax[n])
    return states, out
