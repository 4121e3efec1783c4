"""FP4 reference: the MXFP4 block format (E2M1 values, one E8M0 scale per 32
consecutive values) and an MXFP4 GEMM.

TEST INFRASTRUCTURE.  Only the test suite uses this module; it shares no code
with the HIP path.

Pages cited (title, section):
  [TE-ESM2] "深入源码NVIDIA ESM-2 TransformerEngine优化的实现原理与技术细节",
            FP8与FP4混合精度支持 (the encoder takes an fp4_recipe beside the fp8
            recipe) and 精度配置建议 (FP8 or FP4 for inference, by hardware).

The pages name an FP4 recipe but give no format, block size or scale rule.
Reading used (the plainest one on CDNA4, whose matrix cores take this format
natively): the OCP Microscaling (MX) format MXFP4, as the OCP MX
specification v1.0 defines it --
  * elements are E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0
    is subnormal (m/2); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no inf or NaN;
  * a block is 32 consecutive values along the contraction (K) dimension with
    one shared scale X = 2^e stored as E8M0 (the byte e + 127; 255 = NaN);
  * quantisation of a block: e = floor(log2(max |v|)) - 2 (2 = the largest
    E2M1 exponent), clamped to [-127, 127], e = -127 for an all-zero block;
    each element is v / X rounded to the nearest E2M1 value, ties to even,
    magnitudes beyond 6 saturating to 6;
  * a block holding a NaN gets the NaN scale; inputs here are finite.
The MXFP4 GEMM multiplies the dequantised values exactly: y = x_q . w_q^T with
x_q[m, k] = X_x[m, k // 32] * E2M1(code), likewise for w.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 32
E2M1_EMAX = 2          # largest exponent of an E2M1 normal value (6 = 1.5 * 2^2)
E2M1_MAX = 6.0


def e2m1_decode_table() -> np.ndarray:
    """float64 value of each of the 16 E2M1 codes (bit 3 sign, bits 2..1
    exponent with bias 1, bit 0 mantissa)."""
    vals = np.empty(16)
    for c in range(16):
        s = -1.0 if c & 0x8 else 1.0
        e = (c >> 1) & 0x3
        m = c & 0x1
        vals[c] = s * (m / 2.0) if e == 0 else s * (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return vals


_MAGS = e2m1_decode_table()[:8]          # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def e2m1_encode(v) -> np.ndarray:
    """Nearest E2M1 code of each value (ties to the even code, i.e. mantissa
    bit 0), saturating beyond 6; the sign of zero is kept."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    d = np.abs(a[..., None] - _MAGS)                     # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among the nearest magnitudes prefer an even code (mantissa bit 0)
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return (pick | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def block_exponent(block) -> int:
    """Shared exponent e of one block (X = 2^e), per the MX rule above."""
    amax = float(np.max(np.abs(np.asarray(block, np.float64))))
    if amax == 0.0:
        return -127
    e = math.floor(math.log2(amax)) - E2M1_EMAX
    # log2 of an exact power of two is exact; guard the floor against rounding
    if 2.0 ** (e + E2M1_EMAX) > amax:
        e -= 1
    elif 2.0 ** (e + E2M1_EMAX + 1) <= amax:
        e += 1
    return max(-127, min(127, e))


def mx_quantize(x):
    """x [rows, K] (K a multiple of 32) -> (codes uint8 [rows, K], exponents
    int32 [rows, K // 32]).  Every block at once: frexp writes max|v| as
    m 2^E with m in [0.5, 1), so floor(log2 max|v|) = E - 1 exactly (the same
    rule as block_exponent, checked against it in the tests)."""
    x = np.asarray(x, np.float64)
    rows, K = x.shape
    assert K % BLOCK == 0
    xb = x.reshape(rows, K // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=-1)
    _, E = np.frexp(amax)
    exps = np.where(amax == 0.0, -127, np.clip(E - 1 - E2M1_EMAX, -127, 127)).astype(np.int32)
    codes = e2m1_encode(xb / np.exp2(exps.astype(np.float64))[..., None])
    return codes.reshape(rows, K), exps


def bf16_round(x) -> np.ndarray:
    """float64 -> nearest bfloat16 value (through float32, ties to even), the
    rounding of a bf16 tensor written by a float32 computation."""
    f = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def layer_forward_mxfp4(x, cu_seqlens, w, heads: int):
    """One pre-LN layer with MXFP4 GEMMs: each linear is mx(a) . mx(W)^T + b,
    the input a quantised as computed, per 32-value block along K, and W (bf16
    values) likewise.  Everything else as in the plain fp64 layer."""
    from . import esm_oracle as O
    x = np.asarray(x, np.float64)
    T, H = x.shape
    F = w["w_fc1"].shape[0]

    def lin(a, wname, bname, n_out):
        y = mx_matmul(*mx_quantize(a), *mx_quantize(w[wname]))
        b = w.get(bname)
        return y + (np.zeros(n_out) if b is None else b)

    h1 = O.layer_norm(x, w["ln1_gamma"], w["ln1_beta"])
    q, k, v = O.split_qkv(lin(h1, "w_qkv", "b_qkv", 3 * H), heads)
    pos = O.positions(cu_seqlens)
    ctx = O.attention(O.apply_rope(q, pos), O.apply_rope(k, pos), v, cu_seqlens)
    x1 = x + lin(ctx, "w_out", "b_out", H)
    h2 = O.layer_norm(x1, w["ln2_gamma"], w["ln2_beta"])
    a = O.gelu(lin(h2, "w_fc1", "b_fc1", F))
    return x1 + lin(a, "w_fc2", "b_fc2", H)


def mx_dequantize(codes, exps) -> np.ndarray:
    codes = np.asarray(codes)
    rows, K = codes.shape
    vals = e2m1_decode_table()[codes].reshape(rows, K // BLOCK, BLOCK)
    return (vals * np.exp2(np.asarray(exps, np.float64))[..., None]).reshape(rows, K)


def mx_matmul(x_codes, x_exps, w_codes, w_exps) -> np.ndarray:
    """y[m, n] = sum_k x_q[m, k] w_q[n, k] in float64."""
    return mx_dequantize(x_codes, x_exps) @ mx_dequantize(w_codes, w_exps).T
