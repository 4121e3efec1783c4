"""Throughput of the ESM-2 encoder forward on one MI355X.

One step = one esm_stack_fwd call: embedding lookup plus all layers of the
650M (33-layer, bf16) encoder over one packed THD batch of ~32768 residues
(87 sequences, lognormal lengths, seed 0), inputs already resident in HBM;
the LayerNorms are folded into the QKV and fc1 linears once before timing
(esm_prepare_layer, like the FP8 weight casts).  Beside it: the same batch
padded to bshd [87, 1024] ("padded", the packing gain), the same stack with
the LayerNorms as separate passes ("bf16_unfolded"), the 3B-shaped 36-layer
stack on its own packed batch ("stack_3b"), the device's achievable bf16
MFMA rate from a register-only probe ("mfma_peak") and memory use.
Timing follows the TransformerEngine tutorial's protocol: warm-up steps, then
timed steps bracketed by device synchronisation, HIP events on the library
stream; a second pass over the same steps times every kernel launch with HIP
events for the roofline of the dominant kernel.  The same batch is then run
through the FP8 (E4M3, delayed scaling) encoder, whose scales come from at
least 10 warm-up steps, and reported under "fp8"; what follows the stack
(final LayerNorm, masked-LM logits, per-sequence means) is timed on its own
under "head".  The biased attention kernel (the DeepSpeed4Science page's
Evoformer attention with a mask bias and a pair bias) is timed on its own
synthetic MSA-row shape under "biased_attention", the MXFP4 quantiser and
GEMM (the FP4 recipe) on the layer's four GEMM shapes under "mxfp4", the
whole stack with MXFP4 GEMMs under "mxfp4_stack", the stack with FP8 and
MXFP4 layers alternating in one encoder under "mixed_fp8_mxfp4_stack", the
attention backward on the batch's sequences under "attention_bwd", the
linear backward on the layer's four shapes under "linear_bwd", the
LayerNorm backward on [T, H] under "layernorm_bwd", and one 650M layer's
training forward and backward (esm_layer_fwd_train, esm_layer_bwd) on the
batch under "layer_train", and the whole 33-layer training step
(esm_stack_fwd_train, esm_stack_bwd) under "stack_train".
Prints one JSON line.

    python bench.py [--steps 30] [--warmup 10] [--workload 650m|3b|650m_fp8] [--no-cpu-baseline]
                    [--no-padded] [--no-unfolded] [--no-3b] [--no-mfma-peak] [--no-fp8]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA (vendor figure)
PEAK_FP8_TFLOPS = 5033.2     # MI355X dense fp8 MFMA (vendor figure)
FP8_MIN_WARMUP = 10          # delayed scales settle over the warm-up steps
PEAK_HBM_GBS = 8000.0
PEAK_FP4_TFLOPS = 10066.3    # MI355X dense fp4 MFMA (vendor figure)
# Exponentials per second: the transcendental unit issues a quarter of the 32
# fp32 lanes per cycle per SIMD that make the 157.3 TFLOP/s vector peak, i.e.
# 8 lanes per cycle (a wave-wide v_exp_f32 in 8 cycles), on 4 SIMDs x 256
# compute units at 2.4 GHz.
PEAK_EXP_GPS = 256 * 4 * 8 * 2.4


def layer_flops(H: int, F: int, T: int, sum_L2: int) -> dict:
    """Algorithmic flops per launch of each kernel class for one layer."""
    return {
        "gemm_qkv": 2.0 * T * H * 3 * H,
        "gemm_out": 2.0 * T * H * H,
        "gemm_fc1": 2.0 * T * H * F,
        "gemm_fc2": 2.0 * T * F * H,
        "attention": 4.0 * H * sum_L2,   # q k^T and p v, 2 flops per multiply-add
    }


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="650m", choices=["650m", "3b", "650m_fp8"])
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 leg of a bf16 workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-padded", action="store_true", help="skip the padded bshd layout of the same batch")
    ap.add_argument("--no-unfolded", action="store_true",
                    help="skip the bf16 stack with the LayerNorms as separate passes")
    ap.add_argument("--no-3b", action="store_true", help="skip the 3B-shaped 36-layer stack leg")
    ap.add_argument("--no-mfma-peak", action="store_true", help="skip the matrix-core rate probe")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-head", action="store_true", help="skip timing the final LayerNorm / LM head / means")
    ap.add_argument("--no-linear-bwd", action="store_true",
                    help="skip timing the linear and LayerNorm backward on the layer's shapes")
    ap.add_argument("--no-attention-bwd", action="store_true",
                    help="skip timing the attention backward on the batch")
    ap.add_argument("--no-biased-attention", action="store_true",
                    help="skip timing the biased (Evoformer MSA-row) attention kernel")
    ap.add_argument("--no-mxfp4", action="store_true", help="skip timing the MXFP4 GEMMs on the layer shapes")
    ap.add_argument("--no-layer-train", action="store_true",
                    help="skip one layer's training forward and backward (esm_layer_fwd_train, esm_layer_bwd)")
    ap.add_argument("--no-stack-train", action="store_true",
                    help="skip the whole stack's training forward and backward (esm_stack_fwd_train, esm_stack_bwd)")
    ap.add_argument("--no-vendor-gemm", action="store_true", help="skip the hipBLASLt fc1-shape reference timing")
    ap.add_argument("--one-group", action="store_true",
                    help="run the stacks as one group (no host lengths, so no two-stream split): the per-kernel "
                         "timing pass's launches, for counter runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device copy first (reference dispatch for HBM byte counters)")
    return ap.parse_args()


def traffic_record(kernel: str, rows: int, hidden: int, ffn: int):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when the summary is missing, was taken on a different GEMM source or
    on another shape (rows x hidden x ffn) than the one being measured."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    csrc = os.path.join(ROOT, "protein_language_model_amd", "csrc")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for f in ("gemm.hip", "common.h"):     # the GEMM kernel and the device helpers it inlines
            h.update(open(os.path.join(csrc, f), "rb").read())
        sha = h.hexdigest()
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("gemm_source_sha256") != sha:
        return None
    if (ent.get("rows"), ent.get("hidden"), ent.get("ffn")) != (rows, hidden, ffn):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(wl, batch, emb_bits, weights_dev, budget_residues: int = 12288, layers: int = 8) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    the first sequences of the batch up to `budget_residues` residues, through
    `layers` layers; scaled to residues/s of the full-depth forward."""
    from oracle import esm_oracle as O
    from protein_language_model_amd import datagen as D
    m = wl.model
    n, tot = 0, 0
    while n < batch.B and tot + int(batch.lengths[n]) <= budget_residues:
        tot += int(batch.lengths[n])
        n += 1
    n = max(n, 1)
    seqs = list(range(n))
    tot = int(sum(batch.lengths[:n]))
    cu = D.cu_from_lengths(batch.lengths[:n])
    x = D.bf16_bits_to_f64(emb_bits)[batch.ids[:tot]]
    ws = [O.weights_to_f64({k: D.tensor_bits(v) for k, v in weights_dev[l].items()}) for l in range(layers)]
    threads, blas = None, None
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max((i.get("num_threads") or 0) for i in info) or None
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info})) or None
    except Exception:
        pass
    fp8 = wl.precision == "fp8"
    if fp8:
        from oracle import fp8_ref as F8
        unit_scales = {n: 1.0 for n in F8.ACT_NAMES}   # the cost does not depend on the scale values
    t0 = time.perf_counter()
    for l in range(layers):
        if fp8:
            x = F8.layer_forward_fp8(x, cu, ws[l], m.heads, unit_scales)
        else:
            x = O.layer_forward(x, cu, ws[l], m.heads)
    dt = time.perf_counter() - t0
    per_layer = dt / layers
    return {
        "value": tot / (per_layer * m.layers),
        "unit": "residues/s",
        "cores": threads or os.cpu_count(),
        "blas": blas,
        "kind": "oracle",
        "sample": f"first {n} sequences ({tot} residues) of the batch through {layers} of {m.layers} layers "
                  f"({'FP8-emulating ' if fp8 else ''}fp64 numpy/scipy), {dt:.1f} s; scaled to the "
                  f"{m.layers}-layer forward",
    }


def roofline_of(prof, fl, peaks):
    """Roofline record of the kernel class with the largest total time."""
    cand = {k: v for k, v in prof.items() if k in fl and v[1]}
    dom = max(cand, key=lambda k: cand[k][0])
    avg_ms = cand[dom][0] / cand[dom][1]
    achieved = fl[dom] / (avg_ms * 1e-3) / 1e12
    peak = peaks.get(dom, PEAK_BF16_TFLOPS)
    return {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None, "avg_launch_ms": round(avg_ms, 4),
            "flops_per_launch": fl[dom]}


def rooflines_all(prof, fl, peaks, T: int, H: int, fp8: bool) -> dict:
    """Achieved rate of every kernel class against the bound that applies to it:
    MFMA flops for the GEMMs and attention (attention also reports its exp rate),
    HBM bytes for LayerNorm and the embedding gather (algorithmic bytes: each
    input read once, each output written once)."""
    out = {}
    for k, (ms_tot, n) in prof.items():
        if not n:
            continue
        avg_s = ms_tot / n * 1e-3
        if k in fl:
            peak = peaks.get(k, PEAK_BF16_TFLOPS)
            a = fl[k] / avg_s / 1e12
            out[k] = {"bound": "mfma", "achieved": round(a, 1), "peak": peak, "unit": "TFLOP/s",
                      "frac": round(a / peak, 4)}
            if k == "attention":
                # one exponential per score: 4 * 64 * heads * sum L^2 flops -> heads * sum L^2 exponentials
                exps = fl[k] / 256.0
                r = exps / avg_s / 1e9
                out[k]["exp"] = {"bound": "alu", "achieved": round(r, 1), "peak": PEAK_EXP_GPS, "unit": "Gexp/s",
                                 "frac": round(r / PEAK_EXP_GPS, 4), "exps_per_launch": exps}
        elif k in ("layernorm", "embed"):
            # LN: x in (bf16) + y out (bf16, or E4M3 in an FP8 encoder); embed: y out (the table is tiny)
            nbytes = (T * H * 2 + T * H * (1 if fp8 else 2)) if k == "layernorm" else T * H * 2
            a = nbytes / avg_s / 1e9
            out[k] = {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(a / PEAK_HBM_GBS, 4), "bytes_per_launch": nbytes}
    return out


def bench_biased_attention(enc, steps: int, dev: str, stream) -> dict:
    """The biased attention kernel alone on the synthetic MSA-row shape
    [1, 128, 512, 8, 64] with a mask bias and a pair bias: time per call
    (one launch) from HIP events on the library stream, against both bounds
    (MFMA flops 4 L^2 64 per (b, n, h); HBM bytes: q, k, v read and out
    written once, mask and pair bias read once); the fp64 oracle is timed on
    one row n and scaled to the call."""
    import torch
    from oracle import esm_oracle as O
    from protein_language_model_amd import datagen as D
    w = D.BIASED_ATTN_WORKLOADS["msa_row_512"]
    bits = D.make_biased_attention_inputs(w.B, w.N, w.L, w.heads, seed=0)
    t = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
         for k, v in bits.items()}
    out = torch.empty_like(t["q"])

    def call():
        enc.biased_attention_fwd(t["q"], t["k"], t["v"], t["mask"], t["pair"], out=out, stream=stream)

    for _ in range(3):
        call()
    n = max(10, steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 4.0 * w.B * w.N * w.heads * w.L * w.L * 64
    nbytes = 4 * (w.B * w.N * w.L * w.heads * 64 * 2) + w.B * w.N * w.L * 2 + w.B * w.heads * w.L * w.L * 2
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    t_mfma, t_hbm = flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": None, "flops_per_launch": flops, "bytes_per_launch": nbytes})
    f = {k: D.bf16_bits_to_f64(v[:, :1]) if k != "pair" else D.bf16_bits_to_f64(v) for k, v in bits.items()}
    t0 = time.perf_counter()
    O.biased_attention(f["q"], f["k"], f["v"], [f["mask"], f["pair"]])
    dt_row = time.perf_counter() - t0
    del t, out
    return {"shape": f"q, k, v, out [{w.B}, {w.N}, {w.L}, {w.heads}, 64] bf16; mask [{w.B}, {w.N}, 1, 1, {w.L}], "
                     f"pair [{w.B}, 1, {w.heads}, {w.L}, {w.L}] bf16",
            "ms_per_call": round(ms, 4), "calls": n, "tflops": round(tf, 1), "hbm_gbs": round(gbs, 1),
            "roofline": roof,
            "oracle": {"ms_per_call": round(dt_row * w.B * w.N * 1e3, 1), "kind": "oracle",
                       "sample": f"one of the {w.B * w.N} rows n (fp64 numpy), {dt_row:.2f} s, scaled to the call"}}


def bench_attention_bwd(enc, batch, cu, ws, heads: int, steps: int, dev: str, stream) -> dict:
    """The attention backward (esm_attention_bwd: row dot, dK/dV kernel, dQ
    kernel) on this batch's packed sequences at the layer's width: q, k, v and
    the context gradient N(0, 1) bf16, context and lse from one
    esm_attention_fwd_lse.  HIP events on the library stream around back-to-
    back calls.  Algorithmic flops: 2.5x the forward's 4 * 64 * sum(L^2) per
    head (dV, dP, dQ, dK and one S), the usual count for a backward that
    recomputes P (the kernels form S and dP twice, once per kernel, which is
    not counted).  The fp64 oracle is timed on the longest sequence (all
    heads) and scaled by sum(L^2) / L_max^2."""
    import torch
    from oracle import esm_oracle as O
    from protein_language_model_amd import datagen as D
    T, B = batch.T, len(batch.lengths)
    g = torch.Generator(device=dev).manual_seed(29)
    qkv = torch.randn((3, heads, T, 64), generator=g, device=dev).to(torch.bfloat16)
    dctx = torch.randn((T, heads * 64), generator=g, device=dev).to(torch.bfloat16)
    ctx = torch.empty((T, heads * 64), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((heads, T), dtype=torch.float32, device=dev)
    delta = torch.empty((heads, T), dtype=torch.float32, device=dev)
    dqkv = torch.empty_like(qkv)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = max(10, steps)
    ms_f = timed(lambda: enc.attention_fwd_lse(qkv, cu, B, T, ctx=ctx, lse=lse, workspace=ws, stream=stream), n)
    ms_b = timed(lambda: enc.attention_bwd(qkv, ctx, dctx, lse, cu, B, T, dqkv=dqkv, delta=delta, workspace=ws,
                                           stream=stream), n)
    sum_L2 = int((batch.lengths.astype(np.int64) ** 2).sum())
    fl_f = 4.0 * 64 * heads * sum_L2
    fl_b = 2.5 * fl_f
    tf = fl_b / (ms_b * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "flops_per_launch": fl_b}
    s = int(np.argmax(batch.lengths))
    a, L = int(batch.cu_seqlens[s]), int(batch.lengths[s])
    sl = slice(a, a + L)
    f = D.bf16_bits_to_f64
    host = qkv[:, :, sl].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    gq, gk, gv = (f(host[i]).transpose(1, 0, 2) for i in range(3))
    gd = f(dctx[sl].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    t0 = time.perf_counter()
    O.attention_bwd(gq, gk, gv, gd, np.array([0, L]))
    dt = time.perf_counter() - t0
    del qkv, dctx, ctx, lse, delta, dqkv
    return {"what": f"esm_attention_bwd on the batch's {B} packed sequences, {heads} heads of 64; inputs N(0, 1) bf16",
            "ms_per_call": round(ms_b, 4), "calls": n, "tflops": round(tf, 1),
            "fwd_lse_ms_per_call": round(ms_f, 4), "fwd_tflops": round(fl_f / (ms_f * 1e-3) / 1e12, 1),
            "bwd_over_fwd": round(ms_b / ms_f, 3), "roofline": roof,
            "oracle": {"ms_per_call": round(dt * sum_L2 / (L * L) * 1e3, 1), "kind": "oracle",
                       "sample": f"the longest sequence (L = {L}, all heads; fp64 numpy), {dt:.2f} s, "
                                 f"scaled by sum(L^2) / L^2"}}


def bench_linear_bwd(enc, T: int, H: int, F: int, steps: int, dev: str, stream) -> dict:
    """esm_linear_bwd (dx, dW and db) on the layer's four linear shapes at this
    batch's T: bf16 x, dy N(0, 1) and W N(0, 0.02); HIP events on the library
    stream around back-to-back calls.  Algorithmic flops 4 M N K per call (the
    two products); the W^T copy, the column sum and the slice sum are counted
    as time, not flops."""
    import torch
    out = {}
    g = torch.Generator(device=dev).manual_seed(12)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(10, steps)
    for name, N, K in (("qkv", 3 * H, H), ("out", H, H), ("fc1", F, H), ("fc2", H, F)):
        x = torch.randn((T, K), device=dev, generator=g).to(torch.bfloat16)
        w = (torch.randn((N, K), device=dev, generator=g) * 0.02).to(torch.bfloat16)
        dy = torch.randn((T, N), device=dev, generator=g).to(torch.bfloat16)
        dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        db = torch.empty((N,), dtype=torch.float32, device=dev)
        ws = torch.empty((enc.linear_bwd_workspace_size(T, N, K),), dtype=torch.uint8, device=dev)

        def call():
            enc.linear_bwd(x, w, dy, dx=dx, dw=dw, db=db, workspace=ws, stream=stream)

        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        fl = 4.0 * T * N * K
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"us_per_call": round(ms * 1e3, 1), "tflops": round(tf, 1),
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                                  "flops_per_launch": fl}}
        del x, w, dy, dx, dw, db, ws
    # the HYBRID recipe's FP8 weight gradient on fc1's shape: E5M2 dy [T, F],
    # E4M3 x [T, H] (codes drawn uniformly over finite values), dW [F, H]
    f8 = torch.randint(0, 0x7B, (T, F), device=dev, generator=g, dtype=torch.int32).to(torch.uint8)
    x8 = torch.randint(0, 0x7E, (T, H), device=dev, generator=g, dtype=torch.int32).to(torch.uint8)
    one = torch.ones((1,), dtype=torch.float32, device=dev)
    dw8 = torch.empty((F, H), dtype=torch.bfloat16, device=dev)

    def call8():
        enc.linear_e5m2_wgrad(f8, one, x8, one, dw=dw8, stream=stream)

    for _ in range(3):
        call8()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        call8()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    fl = 2.0 * T * F * H
    tf = fl / (ms * 1e-3) / 1e12
    out["e5m2_wgrad_fc1"] = {"us_per_call": round(ms * 1e3, 1), "tflops": round(tf, 1),
                             "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
                                          "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": None,
                                          "flops_per_launch": fl}}
    del f8, x8, dw8
    return out


def bench_layer_train(enc, batch, cu, weights, m, steps: int, dev: str, stream) -> dict:
    """One layer's training forward (esm_layer_fwd_train: the forward keeping
    the activations its backward takes) and backward (esm_layer_bwd: dx and
    the 12 parameter gradients) on the batch, the 650M layer's widths and
    layer 0's weights, x and dy N(0, 1) bf16; HIP events on the library stream
    around back-to-back calls.  Algorithmic flops: the forward's (linears
    2 T (4 H^2 + 2 H F), attention 4 H sum L^2), the backward's twice the
    linears' and 2.5 times the attention's; a 33-layer training step is
    projected as 33 times forward plus backward."""
    import torch
    T, B, H, F = batch.T, batch.B, m.hidden, m.ffn
    g = torch.Generator(device=dev).manual_seed(13)
    x = torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)
    dy = torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    saved = torch.empty((enc.saved_size(T),), dtype=torch.uint8, device=dev)
    ws = enc.workspace(T, B)
    bws = enc.layer_bwd_workspace(T, B)
    grads = None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(10, steps)

    def fwd():
        enc.layer_fwd_train(weights, x, cu, B, T, batch.max_seqlen, x_out=y, saved=saved, workspace=ws, stream=stream)

    def bwd():
        nonlocal grads
        _, grads = enc.layer_bwd(weights, x, saved, dy, cu, B, T, dx=dx, grads=grads, workspace=bws, stream=stream)

    res = {}
    for name, call in (("fwd_train", fwd), ("bwd", bwd)):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / n
    lin = 2.0 * T * (4 * H * H + 2 * H * F)
    att = 4.0 * H * int((batch.lengths.astype(np.int64) ** 2).sum())
    fl_f, fl_b = lin + att, 2.0 * lin + 2.5 * att
    tf_f = fl_f / (res["fwd_train"] * 1e-3) / 1e12
    tf_b = fl_b / (res["bwd"] * 1e-3) / 1e12
    per_layer = res["fwd_train"] + res["bwd"]
    tf_t = (fl_f + fl_b) / (per_layer * 1e-3) / 1e12
    del x, dy, y, dx, saved, ws, bws, grads
    return {"what": "esm_layer_fwd_train then esm_layer_bwd, one 650M-width layer on the batch, inputs N(0, 1) bf16",
            "fwd_train_ms": round(res["fwd_train"], 4), "bwd_ms": round(res["bwd"], 4),
            "fwd_tflops": round(tf_f, 1), "bwd_tflops": round(tf_b, 1), "tflops": round(tf_t, 1),
            "bwd_over_fwd": round(res["bwd"] / res["fwd_train"], 3),
            "projected_33_layer_train_step_ms": round(33 * per_layer, 2),
            "projected_residues_per_s": round(T / (33 * per_layer * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf_t, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf_t / PEAK_BF16_TFLOPS, 4), "traffic": None,
                         "flops_per_launch": fl_f + fl_b}}


def bench_stack_train(enc, batch, cu, ids, emb, weights, m, steps: int, dev: str, stream) -> dict:
    """The whole stack's training step on the batch: esm_stack_fwd_train from
    the token ids (every layer's input and activations kept in HBM) then
    esm_stack_bwd from dy N(0, 1) bf16 down to the embedding table's gradient;
    HIP events on the library stream around back-to-back steps.  Algorithmic
    flops per step: the layers' forward and backward flops of
    bench_layer_train, times the depth (the embedding's gather and gradient
    are not counted)."""
    import torch
    T, B, H, F, L = batch.T, batch.B, m.hidden, m.ffn, m.layers
    g = torch.Generator(device=dev).manual_seed(17)
    dy = torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)
    y = torch.empty_like(dy)
    dx = torch.empty_like(dy)
    saved = torch.empty((enc.stack_saved_size(T),), dtype=torch.uint8, device=dev)
    ws = enc.workspace(T, B)
    bws = enc.stack_bwd_workspace(T, B)
    grads = None
    demb = torch.empty((m.vocab, H), dtype=torch.float32, device=dev)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    n = max(3, steps // 10)

    def fwd():
        enc.stack_fwd_train(weights, cu, B, T, batch.max_seqlen, token_ids=ids, embedding=emb, x_out=y, saved=saved,
                            workspace=ws, stream=stream)

    def bwd():
        nonlocal grads
        _, grads, _ = enc.stack_bwd(weights, saved, dy, cu, B, T, dx=dx, grads=grads, token_ids=ids,
                                    d_embedding=demb, workspace=bws, stream=stream)

    fwd()
    bwd()
    torch.cuda.synchronize()
    f_ms = b_ms = 0.0
    for _ in range(n):
        e0.record(stream)
        fwd()
        e1.record(stream)
        bwd()
        e2.record(stream)
        torch.cuda.synchronize()
        f_ms += e0.elapsed_time(e1) / n
        b_ms += e1.elapsed_time(e2) / n
    lin = 2.0 * T * (4 * H * H + 2 * H * F)
    att = 4.0 * H * int((batch.lengths.astype(np.int64) ** 2).sum())
    fl = L * (3.0 * lin + 3.5 * att)
    step = f_ms + b_ms
    tf = fl / (step * 1e-3) / 1e12
    saved_gb = saved.numel() / 1e9
    del dy, y, dx, saved, ws, bws, grads, demb
    return {"what": f"esm_stack_fwd_train (from token ids) then esm_stack_bwd (to the embedding table's gradient), "
                    f"{L} layers of the 650M widths on the batch, dy N(0, 1) bf16, {n} timed steps",
            "fwd_train_ms": round(f_ms, 3), "bwd_ms": round(b_ms, 3), "ms_per_step": round(step, 3),
            "residues_per_s": round(T / (step * 1e-3), 1), "tflops": round(tf, 1),
            "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "saved_activation_gb": round(saved_gb, 2),
            "flops_per_step": fl}


def bench_layernorm_bwd(enc, T: int, H: int, steps: int, dev: str, stream) -> dict:
    """esm_layernorm_bwd on [T, H] (x N(0, 1), gamma 1 + N(0, 0.04), dy N(0, 1)
    bf16); HIP events over back-to-back calls.  HBM roofline on the
    algorithmic bytes: x and dy read once, dx written (the column pass reads
    x and dy a second time, which is counted as time, not bytes)."""
    import torch
    g = torch.Generator(device=dev).manual_seed(13)
    x = torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)
    gamma = (1 + 0.2 * torch.randn((H,), device=dev, generator=g)).to(torch.bfloat16)
    dy = torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)
    dx = torch.empty_like(x)
    dgamma = torch.empty((H,), dtype=torch.float32, device=dev)
    dbeta = torch.empty((H,), dtype=torch.float32, device=dev)
    ws = torch.empty((64 << 20,), dtype=torch.uint8, device=dev)

    def call():
        enc.layernorm_bwd(x, gamma, dy, dx=dx, dgamma=dgamma, dbeta=dbeta, workspace=ws, stream=stream)

    for _ in range(3):
        call()
    n = max(10, steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    nbytes = 3 * T * H * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    del x, gamma, dy, dx, dgamma, dbeta, ws
    return {"shape": f"x, dy, dx [{T}, {H}] bf16; dgamma, dbeta [{H}] fp32", "us_per_call": round(ms * 1e3, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "bytes_per_launch": nbytes}}


def bench_mxfp4(enc, T: int, H: int, F: int, steps: int, dev: str, stream) -> dict:
    """The MXFP4 (FP4 recipe) quantiser and GEMM alone on the four linears'
    shapes of one layer of this batch: bf16 activations and weights N(0, 1) /
    N(0, 0.02), quantised by the library, GEMM with a bias epilogue; HIP
    events on the library stream.  GEMMs against the dense fp4 MFMA peak,
    the quantiser against HBM (bf16 read, codes and scales written)."""
    import torch
    out = {}
    g = torch.Generator(device=dev).manual_seed(11)

    def timeit(fn, n):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = max(10, steps)
    for name, N, K in (("qkv", 3 * H, H), ("out", H, H), ("fc1", F, H), ("fc2", H, F)):
        x = torch.randn((T, K), device=dev, generator=g).to(torch.bfloat16)
        w = (torch.randn((N, K), device=dev, generator=g) * 0.02).to(torch.bfloat16)
        b = (torch.randn((N,), device=dev, generator=g) * 0.02).to(torch.bfloat16)
        y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        xq = enc.mxfp4_quantize(x, stream=stream)
        wq = enc.mxfp4_quantize(w, stream=stream)
        ms_q = timeit(lambda: enc.mxfp4_quantize(x, codes=xq[0], scales=xq[1], stream=stream), n)
        ms_g = timeit(lambda: enc.linear_mxfp4_fwd(xq, wq, b, y=y, stream=stream), n)
        fl = 2.0 * T * N * K
        qbytes = T * K * 2 + T * K // 2 + T * K // 32
        tf = fl / (ms_g * 1e-3) / 1e12
        out[name] = {"gemm_us": round(ms_g * 1e3, 1), "tflops": round(tf, 1),
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP4_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_FP4_TFLOPS, 4), "traffic": None,
                                  "flops_per_launch": fl},
                     "quantize_us": round(ms_q * 1e3, 1),
                     "quantize_gbs": round(qbytes / (ms_q * 1e-3) / 1e9, 1)}
        del x, w, b, y, xq, wq
    out["shape"] = f"T = {T} rows; x bf16 [T, K] and W bf16 [N, K] quantised to MXFP4 (E2M1, E8M0 per 32)"
    return out


def bench_stack_leg(name: str, steps: int, warmup: int, dev: str, stream) -> dict:
    """Another packed workload's bf16 stack (LayerNorms folded), timed the
    same way as the main leg: warm-up steps, then HIP events around `steps`
    steps on the library stream."""
    import torch
    from protein_language_model_amd import datagen as D
    from protein_language_model_amd import esm
    wl = D.WORKLOADS[name]
    m = wl.model
    b = D.make_batch(wl)
    emb_d = torch.from_numpy(D.make_embedding(m.vocab, m.hidden).view(np.int16)).view(torch.bfloat16).to(dev)
    wts = [D.make_layer_weights_device(m.hidden, m.ffn, l) for l in range(m.layers)]
    enc = esm.Encoder(hidden_size=m.hidden, num_attention_heads=m.heads, intermediate_size=m.ffn,
                      num_hidden_layers=m.layers)
    enc.prepare(wts, stream=stream)
    cu = torch.from_numpy(b.cu_seqlens).to(dev)
    ids = torch.from_numpy(b.ids).to(dev)
    out = torch.empty((b.T, m.hidden), dtype=torch.bfloat16, device=dev)
    ws = enc.workspace(b.T, b.B)

    def step():
        enc.stack_fwd(wts, cu, b.B, b.T, b.max_seqlen, token_ids=ids, embedding=emb_d, x_out=out,
                      cu_seqlens_host=b.cu_seqlens, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    sum_L2 = int((b.lengths.astype(np.int64) ** 2).sum())
    flops = m.layers * sum(layer_flops(m.hidden, m.ffn, b.T, sum_L2).values())
    tf = flops / (ms * 1e-3) / 1e12
    enc.close()
    del ws, wts, out
    return {"workload": f"ESM-2 {m.hidden}x{m.layers} ({name}) packed THD forward, bf16",
            "sequences": b.B, "residues": b.T, "max_seqlen": b.max_seqlen, "sum_L2": sum_L2,
            "hidden": m.hidden, "heads": m.heads, "ffn": m.ffn, "layers": m.layers, "steps": steps,
            "ms_per_step": round(ms, 4), "value": round(b.T / (ms * 1e-3), 1), "unit": "residues/s",
            "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def bench_mfma_peak(dev: str, stream) -> dict:
    """The library's matrix-core rate probe (bf16 32x32x16 MFMAs on changing
    register operands, nothing else in the loop), two workgroups of four
    waves per compute unit: the achievable bf16 MFMA rate of this device under
    load, beside the spec peak."""
    import torch
    from protein_language_model_amd import esm
    enc = esm.Encoder(hidden_size=320, num_attention_heads=5, intermediate_size=1280, num_hidden_layers=1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(16 * cus * 2, dtype=torch.float32, device=dev)
    iters = 20000
    for _ in range(2):
        enc.mfma_peak(iters, sink, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    n = 5
    e0.record(stream)
    flops = 0.0
    for _ in range(n):
        flops += enc.mfma_peak(iters, sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    enc.close()
    tf = flops / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "frac_of_spec_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "ms_per_launch": round(ms / n, 4), "launches": n,
            "what": "bf16 v_mfma_f32_32x32x16 chains on register operands that change every instruction, "
                    "2 workgroups x 4 waves per CU, nothing else in the loop (esm_mfma_peak)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the forward needs no "
              "cross-GPU exchange: a batch would be split by whole sequences, one process per GPU)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from protein_language_model_amd import datagen as D
    from protein_language_model_amd import esm

    wl = D.WORKLOADS[args.workload]
    m = wl.model
    batch = D.make_batch(wl)
    dev = "cuda:0"
    emb = D.make_embedding(m.vocab, m.hidden)
    weights = [D.make_layer_weights_device(m.hidden, m.ffn, l) for l in range(m.layers)]

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    T, B = batch.T, batch.B
    cu = torch.from_numpy(batch.cu_seqlens).to(dev)
    ids = torch.from_numpy(batch.ids).to(dev)
    emb_d = up_bf16(emb)
    out = torch.empty((T, m.hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    if args.copy_calibration:
        src_c = torch.ones(128 * 1024 * 1024, dtype=torch.bfloat16, device=dev)
        dst_c = torch.empty_like(src_c)
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    sum_L2 = int((batch.lengths.astype(np.int64) ** 2).sum())
    fl = layer_flops(m.hidden, m.ffn, T, sum_L2)
    total_flops = m.layers * sum(fl.values())

    def measure(precision: str, warmup: int, fold: bool = True, layer_prec=None):
        """Clean timed region (the throughput), then the same steps with every
        launch bracketed by HIP events (per-kernel durations).  bf16: the
        LayerNorms are folded into the QKV and fc1 linears (esm_prepare_layer,
        once, like the FP8 and MXFP4 weight preparation) unless fold is off.
        layer_prec: per-layer precisions of a quantised encoder (each layer's
        weights prepared in its own format)."""
        enc = esm.Encoder(hidden_size=m.hidden, num_attention_heads=m.heads, intermediate_size=m.ffn,
                          num_hidden_layers=m.layers, precision=precision)
        if precision == "bf16" and fold:
            enc.prepare(weights, stream=stream)
        if layer_prec is not None:
            enc.set_layer_precision(layer_prec, stream=stream)
            for l, p in enumerate(layer_prec):
                if p == "fp8":
                    enc.fp8_prepare_layer(l, weights[l], stream=stream)
                elif p == "mxfp4":
                    enc.mxfp4_prepare_layer(l, weights[l], stream=stream)
        elif precision == "fp8":
            enc.fp8_prepare(weights, stream=stream)
        elif precision == "mxfp4":
            enc.mxfp4_prepare(weights, stream=stream)
        ws = enc.workspace(T, B)

        host_cu = None if args.one_group else batch.cu_seqlens

        def step():
            enc.stack_fwd(weights, cu, B, T, batch.max_seqlen, token_ids=ids, embedding=emb_d, x_out=out,
                          cu_seqlens_host=host_cu, workspace=ws, stream=stream)

        def timed_steps(n: int, per_step: list = None) -> float:
            """Mean ms per step over n steps; per_step (if given) receives each
            step's own duration from an event recorded after it."""
            marks = [torch.cuda.Event(enable_timing=True) for _ in range(n)] if per_step is not None else None
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(n):
                step()
                if marks:
                    marks[i].record(stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if marks:
                per_step[:] = [e0.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i]) for i in range(1, n)]
            return e0.elapsed_time(e1) / n

        for _ in range(warmup):
            step()
        steps_ms = []
        ms = timed_steps(args.steps, steps_ms)
        prof = ms_instr = None
        if not args.no_kernel_timing:
            enc.profile_enable(True)
            ms_instr = timed_steps(args.steps)
            prof = enc.profile_read()
            enc.profile_enable(False)
        measure.steps_ms = steps_ms
        return enc, ws, ms, prof, ms_instr

    def kernel_table(prof):
        return {k: {"ms_per_launch": (v[0] / v[1]) if v[1] else None, "launches_per_step": v[1] / args.steps,
                    "ms_per_step": v[0] / args.steps} for k, v in prof.items() if v[1]}

    fp8_main = wl.precision == "fp8"
    gemm_peak = PEAK_FP8_TFLOPS if fp8_main else PEAK_BF16_TFLOPS
    peaks = {k: gemm_peak for k in fl if k.startswith("gemm")}
    enc, ws, ms, prof, ms_instrumented = measure(wl.precision, max(args.warmup, FP8_MIN_WARMUP) if fp8_main
                                                 else args.warmup)
    tflops = total_flops / (ms * 1e-3) / 1e12
    value = T / (ms * 1e-3)
    sm = sorted(measure.steps_ms)
    step_stats = {"median": round(sm[len(sm) // 2], 4), "min": round(sm[0], 4), "max": round(sm[-1], 4)} if sm else None
    roofline = kernels = rooflines = None
    if prof:
        kernels = kernel_table(prof)
        roofline = roofline_of(prof, fl, peaks)
        roofline["traffic"] = traffic_record(("fp8_" if fp8_main else "") + roofline["kernel"], T, m.hidden, m.ffn)
        rooflines = rooflines_all(prof, fl, peaks, T, m.hidden, fp8_main)

    # Context for the dominant kernel: the vendor GEMM library (hipBLASLt via
    # torch.matmul, plain bf16, no epilogue) on the fc1 shape of this batch.
    vendor = None
    if not args.no_vendor_gemm:
        xa = torch.randn((T, m.hidden), device=dev).to(torch.bfloat16)
        wa = torch.randn((m.hidden, m.ffn), device=dev).to(torch.bfloat16)   # W^T, contiguous
        for _ in range(3):
            torch.matmul(xa, wa)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(20):
            torch.matmul(xa, wa)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_v = e0.elapsed_time(e1) / 20
        vendor = {"what": "torch.matmul (hipBLASLt) bf16 [T,H] x [H,F], no bias/GELU epilogue",
                  "us_per_call": round(ms_v * 1e3, 1), "tflops": round(fl["gemm_fc1"] / (ms_v * 1e-3) / 1e12, 1)}
        del xa, wa

    # After the stack (final LayerNorm, masked-LM logits, per-sequence means):
    # timed on its own, on the stack output of the last timed step.
    head = None
    if not args.no_head:
        hw = {k: up_bf16(v) for k, v in D.make_head_weights(m.hidden, emb).items()}
        xf = torch.empty_like(out)
        lg = torch.empty((T, m.vocab), dtype=torch.bfloat16, device=dev)
        pe = torch.empty((B, m.hidden), dtype=torch.float32, device=dev)

        def head_call():
            enc.head_fwd(hw, out, cu, B, T, batch.max_seqlen, x_final=xf, logits=lg, seq_emb=pe, workspace=ws,
                         stream=stream)

        for _ in range(3):
            head_call()
        n_h = max(5, args.steps)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n_h):
            head_call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_h = e0.elapsed_time(e1) / n_h
        fl_h = 2.0 * T * m.hidden * (m.hidden + m.vocab)
        head = {"ms_per_call": round(ms_h, 4), "calls": n_h, "tflops": round(fl_h / (ms_h * 1e-3) / 1e12, 1),
                "outputs": f"final LayerNorm [T,{m.hidden}] bf16, logits [T,{m.vocab}] bf16, sequence means "
                           f"[{B},{m.hidden}] fp32",
                "share_of_step": round(ms_h / ms, 4)}

    biased = None
    if not args.no_biased_attention:
        biased = bench_biased_attention(enc, args.steps, dev, stream)

    attn_bwd = None
    if not args.no_attention_bwd:
        attn_bwd = bench_attention_bwd(enc, batch, cu, ws, m.heads, args.steps, dev, stream)

    lin_bwd = ln_bwd = None
    if not args.no_linear_bwd:
        lin_bwd = bench_linear_bwd(enc, T, m.hidden, m.ffn, args.steps, dev, stream)
        ln_bwd = bench_layernorm_bwd(enc, T, m.hidden, args.steps, dev, stream)

    layer_train = None
    if not args.no_layer_train and m.hidden == 1280:
        layer_train = bench_layer_train(enc, batch, cu, weights[0], m, args.steps, dev, stream)
    stack_train = None
    if not args.no_stack_train and m.hidden == 1280:
        stack_train = bench_stack_train(enc, batch, cu, ids, emb_d, weights, m, args.steps, dev, stream)
        torch.cuda.empty_cache()

    mxfp4 = None
    if not args.no_mxfp4:
        mxfp4 = bench_mxfp4(enc, T, m.hidden, m.ffn, args.steps, dev, stream)

    padded = None
    if not args.no_padded:
        S = 1024
        sl = torch.from_numpy(batch.lengths).to(dev)
        ids_p = np.zeros((B, S), np.int32)
        for i in range(B):
            ids_p[i, :batch.lengths[i]] = batch.ids[batch.cu_seqlens[i]:batch.cu_seqlens[i + 1]]
        ids_pd = torch.from_numpy(ids_p).to(dev)
        ws_p = enc.workspace(B * S, B)
        out_p = torch.empty((B, S, m.hidden), dtype=torch.bfloat16, device=dev)
        for _ in range(2):
            enc.stack_fwd_bshd(weights, sl, B, S, token_ids=ids_pd, embedding=emb_d, x_out=out_p, workspace=ws_p)
        n_p = max(3, args.steps // 6)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n_p):
            enc.stack_fwd_bshd(weights, sl, B, S, token_ids=ids_pd, embedding=emb_d, x_out=out_p, workspace=ws_p,
                               stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_p = e0.elapsed_time(e1) / n_p
        padded = {"layout": f"bshd [{B}, {S}]", "ms_per_step": round(ms_p, 3), "steps": n_p,
                  "valid_fraction": round(T / (B * S), 4), "packing_gain": round(ms_p / ms, 3),
                  "what": "the same sequences right-padded to S = 1024 (esm_stack_fwd_bshd, every GEMM over all "
                          "B * S rows, attention skipping padded keys); packing_gain = padded / packed step time"}
        del ws_p, out_p
    enc.close()
    del ws
    peak_mem = {"torch_max_allocated_bytes": int(torch.cuda.max_memory_allocated()),
                "device_used_bytes": int(torch.cuda.mem_get_info()[1] - torch.cuda.mem_get_info()[0]),
                "what": "torch allocator high-water mark of the run so far (weights, batch, workspaces: the bf16 "
                        "and padded legs) and device memory in use after them (adds the library's own "
                        "allocations: folded weights, RoPE table)"}

    unfolded = None
    if not fp8_main and not args.no_unfolded:
        encu, wsu, msu, profu, _ = measure("bf16", args.warmup, fold=False)
        unfolded = {"ms_per_step": round(msu, 4), "value": round(T / (msu * 1e-3), 1),
                    "fold_gain": round(msu / ms, 4),
                    "what": "the same bf16 stack without esm_prepare_layer: both LayerNorms as separate passes "
                            "writing their bf16 output, plain bias epilogues"}
        if profu:
            unfolded["kernels"] = kernel_table(profu)
        encu.close()
        del wsu

    stack_3b = None
    if args.workload == "650m" and not args.no_3b:
        stack_3b = bench_stack_leg("3b", args.steps, args.warmup, dev, stream)

    mfma_peak = None
    if not args.no_mfma_peak:
        mfma_peak = bench_mfma_peak(dev, stream)

    fp8 = None
    if not fp8_main and not args.no_fp8 and m.hidden % 128 == 0 and m.ffn % 128 == 0:
        enc8, ws8, ms8, prof8, _ = measure("fp8", max(args.warmup, FP8_MIN_WARMUP))
        fp8 = {"ms_per_step": round(ms8, 4), "value": round(T / (ms8 * 1e-3), 1), "unit": "residues/s",
               "tflops": round(total_flops / (ms8 * 1e-3) / 1e12, 1), "speedup_vs_bf16": round(ms / ms8, 3),
               "warmup": max(args.warmup, FP8_MIN_WARMUP),
               "recipe": "E4M3 QKV/out/fc1/fc2 GEMMs, per-tensor delayed scaling, amax history 16, max"}
        if prof8:
            fp8["kernels"] = kernel_table(prof8)
            fp8["roofline"] = roofline_of(prof8, fl, {k: PEAK_FP8_TFLOPS for k in fl if k.startswith("gemm")})
            fp8["roofline"]["traffic"] = traffic_record("fp8_" + fp8["roofline"]["kernel"], T, m.hidden, m.ffn)
            fp8["rooflines"] = rooflines_all(prof8, fl, {k: PEAK_FP8_TFLOPS for k in fl if k.startswith("gemm")}, T,
                                             m.hidden, True)
        enc8.close()
        del ws8

    mx_stack = None
    if not fp8_main and not args.no_mxfp4 and m.hidden % 256 == 0 and m.ffn % 256 == 0 and m.ffn <= 8 * m.hidden:
        encm, wsm, msm, profm, _ = measure("mxfp4", args.warmup)
        mx_stack = {"ms_per_step": round(msm, 4), "value": round(T / (msm * 1e-3), 1), "unit": "residues/s",
                    "tflops": round(total_flops / (msm * 1e-3) / 1e12, 1), "speedup_vs_bf16": round(ms / msm, 3),
                    "recipe": "MXFP4 (E2M1, E8M0 scale per 32 values along K) QKV/out/fc1/fc2 GEMMs; each GEMM "
                              "input quantised after its producer"}
        if profm:
            mx_stack["kernels"] = kernel_table(profm)
            mx_stack["rooflines"] = rooflines_all(profm, fl, {k: PEAK_FP4_TFLOPS for k in fl if k.startswith("gemm")},
                                                  T, m.hidden, False)
        encm.close()
        del wsm

    mixed = None
    if (not fp8_main and not args.no_mxfp4 and not args.no_fp8 and m.hidden % 256 == 0 and m.ffn % 256 == 0
            and m.ffn <= 8 * m.hidden):
        # the per-layer precision setting: FP8 and MXFP4 layers alternating in one encoder
        lp = ["fp8" if l % 2 == 0 else "mxfp4" for l in range(m.layers)]
        encx, wsx, msx, profx, _ = measure("fp8", max(args.warmup, FP8_MIN_WARMUP), layer_prec=lp)
        mixed = {"ms_per_step": round(msx, 4), "value": round(T / (msx * 1e-3), 1), "unit": "residues/s",
                 "tflops": round(total_flops / (msx * 1e-3) / 1e12, 1), "speedup_vs_bf16": round(ms / msx, 3),
                 "layers": "even layers FP8 (E4M3, delayed scaling), odd layers MXFP4, one encoder"}
        if profx:
            mixed["kernels"] = kernel_table(profx)
        encx.close()
        del wsx

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, batch, emb, weights)

    prec = "FP8 E4M3 delayed scaling" if fp8_main else "bf16"
    shape = "650M 33-layer" if m.layers == 33 else "3B-shaped 36-layer"
    rec = {
        "metric": f"packed residues/s, ESM-2 {shape} fwd {prec}; % of MFMA peak",
        "value": round(value, 1),
        "unit": "residues/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": max(args.warmup, FP8_MIN_WARMUP) if fp8_main else args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if fp8_main else "bf16",
        "data": "synthetic",
        "config": {"workload": f"ESM-2 {m.hidden}x{m.layers} ({args.workload}) packed THD forward",
                   "sequences": B, "residues": T, "max_seqlen": batch.max_seqlen, "sum_L2": sum_L2,
                   "hidden": m.hidden, "heads": m.heads, "ffn": m.ffn, "layers": m.layers},
        "tflops": round(tflops, 1),
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "rooflines": rooflines,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "step_ms": step_stats,
        "ms_per_step_with_kernel_events": round(ms_instrumented, 4) if ms_instrumented else None,
        "frac_measured_mfma_peak": round(tflops / mfma_peak["tflops"], 4) if mfma_peak else None,
        "mfma_peak": mfma_peak,
        "peak_memory": peak_mem,
        "padded": padded,
        "bf16_unfolded": unfolded,
        "stack_3b": stack_3b,
        "head": head,
        "biased_attention": biased,
        "mxfp4": mxfp4,
        "attention_bwd": attn_bwd,
        "linear_bwd": lin_bwd,
        "layernorm_bwd": ln_bwd,
        "layer_train": layer_train,
        "stack_train": stack_train,
        "mxfp4_stack": mx_stack,
        "mixed_fp8_mxfp4_stack": mixed,
        "vendor_gemm_fc1": vendor,
        "fp8": fp8,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
