"""Layer- and stack-level parity of the HIP path against the fp64 oracle, and
the bit-exact index invariants (packed == alone, THD == bshd on valid rows,
permutation, NaN padding, determinism)."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import esm_oracle as O
from protein_language_model_amd import datagen as D
from protein_language_model_amd import esm

pytestmark = pytest.mark.gpu

TOL = 1e-2  # per-layer max|gpu - ref| / max|ref| for bf16


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


def _encoder(shape, layers=1):
    return esm.Encoder(hidden_size=shape.hidden, num_attention_heads=shape.heads, intermediate_size=shape.ffn,
                       num_hidden_layers=layers)


@pytest.fixture(scope="module")
def tiny(gu):
    w = D.WORKLOADS["tiny"]
    m = w.model
    enc = _encoder(m)
    batch = D.make_batch(w)
    emb = D.make_embedding(m.vocab, m.hidden)
    wd, wr, _ = gu.layer_weights(m.hidden, m.ffn, 0)
    yield dict(enc=enc, batch=batch, emb=emb, wd=wd, wr=wr, m=m)
    enc.close()


def test_tiny_layer_matches_oracle_with_intermediates(gu, tiny):
    enc, b, m = tiny["enc"], tiny["batch"], tiny["m"]
    x0 = D.bf16_bits_to_f64(tiny["emb"])[b.ids]
    xb = D.to_bf16_bits(x0.astype(np.float32))
    ws = enc.workspace(b.T, b.B)
    y = enc.layer_fwd(tiny["wd"], gu.to_dev_bf16(xb), gu.to_dev_i32(b.cu_seqlens), b.B, b.T, b.max_seqlen,
                      cu_seqlens_host=b.cu_seqlens, workspace=ws)
    ref, it = O.layer_forward(D.bf16_bits_to_f64(xb), b.cu_seqlens, tiny["wr"], m.heads, return_intermediates=True)
    qkv = gu.from_dev(enc.workspace_region(ws, b.T, b.B, "qkv")).reshape(3, m.heads, b.T, 64)
    assert gu.rel_err(qkv[0].transpose(1, 0, 2), it["q"]) < TOL
    assert gu.rel_err(qkv[1].transpose(1, 0, 2), it["k"]) < TOL
    assert gu.rel_err(qkv[2].transpose(1, 0, 2), it["v"]) < TOL
    assert gu.rel_err(gu.from_dev(enc.workspace_region(ws, b.T, b.B, "ctx")).reshape(b.T, -1), it["ctx"]) < TOL
    assert gu.rel_err(gu.from_dev(enc.workspace_region(ws, b.T, b.B, "x1")).reshape(b.T, -1), it["x1"]) < TOL
    assert gu.rel_err(gu.from_dev(enc.workspace_region(ws, b.T, b.B, "act")).reshape(b.T, -1), it["a"]) < TOL
    err = gu.rel_err(gu.from_dev(y), ref)
    print(f"tiny layer rel err {err:.2e}")
    assert err < TOL


def test_tiny_stack_with_embedding(gu, tiny):
    enc, b, m = tiny["enc"], tiny["batch"], tiny["m"]
    y = enc.stack_fwd([tiny["wd"]], gu.to_dev_i32(b.cu_seqlens), b.B, b.T, b.max_seqlen,
                      token_ids=gu.to_dev_i32(b.ids), embedding=gu.to_dev_bf16(tiny["emb"]),
                      cu_seqlens_host=b.cu_seqlens)
    ref = O.stack_forward(b.cu_seqlens, [tiny["wr"]], m.heads, ids=b.ids, table=D.bf16_bits_to_f64(tiny["emb"]))
    assert gu.rel_err(gu.from_dev(y), ref) < TOL


def test_random_layernorm_params(gu, tiny):
    enc, b, m = tiny["enc"], tiny["batch"], tiny["m"]
    wd, wr, _ = gu.layer_weights(m.hidden, m.ffn, 3, random_ln=True)
    xb = D.make_hidden(b.T, m.hidden, seed=5)
    y = enc.layer_fwd(wd, gu.to_dev_bf16(xb), gu.to_dev_i32(b.cu_seqlens), b.B, b.T, b.max_seqlen)
    ref = O.layer_forward(D.bf16_bits_to_f64(xb), b.cu_seqlens, wr, m.heads)
    assert gu.rel_err(gu.from_dev(y), ref) < TOL


def test_zero_output_weights_make_the_layer_the_identity_bitexact(gu, tiny):
    enc, b, m = tiny["enc"], tiny["batch"], tiny["m"]
    wd = dict(tiny["wd"])
    for k in ("w_out", "b_out", "w_fc2", "b_fc2"):
        wd[k] = torch.zeros_like(wd[k])
    xb = D.make_hidden(b.T, m.hidden, seed=6)
    y = enc.layer_fwd(wd, gu.to_dev_bf16(xb), gu.to_dev_i32(b.cu_seqlens), b.B, b.T, b.max_seqlen)
    assert np.array_equal(gu.bits_of(y), xb)


def test_empty_batch_is_a_no_op(gu, tiny):
    enc = tiny["enc"]
    x = torch.zeros((0, 320), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda:0")
    enc.layer_fwd(tiny["wd"], x, gu.to_dev_i32([0]), 0, 0, 0, x_out=x, workspace=ws)


def test_workspace_too_small_is_rejected(gu, tiny):
    enc, b = tiny["enc"], tiny["batch"]
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda:0")
    x = gu.to_dev_bf16(D.make_hidden(b.T, 320))
    with pytest.raises(esm.EsmError) as ei:
        enc.layer_fwd(tiny["wd"], x, gu.to_dev_i32(b.cu_seqlens), b.B, b.T, b.max_seqlen, workspace=ws)
    assert ei.value.status == 5


def test_bad_host_cu_seqlens_is_rejected_before_launch(gu, tiny):
    enc, b = tiny["enc"], tiny["batch"]
    x = gu.to_dev_bf16(D.make_hidden(b.T, 320))
    bad = b.cu_seqlens.copy()
    bad[2] = bad[1] - 1
    with pytest.raises(esm.EsmError) as ei:
        enc.layer_fwd(tiny["wd"], x, gu.to_dev_i32(bad), b.B, b.T, b.max_seqlen, cu_seqlens_host=bad)
    assert ei.value.status == 3


def _bshd_stack_case(gu, m, lengths, layers, S, seed, fold=False):
    """Token ids [B, S] right-padded with out-of-range garbage ids (the
    library clamps ids, so they are still read), and the same sequences
    packed; returns (bshd output bits [B, S, H], THD output bits [T, H],
    weights, embedding bits, ids [B, S])."""
    enc = _encoder(m, layers)
    lengths = np.asarray(lengths, np.int32)
    B = len(lengths)
    r = np.random.default_rng(seed)
    ids = r.integers(0, m.vocab, (B, S)).astype(np.int32)
    for i in range(B):
        ids[i, lengths[i]:] = r.integers(-5, m.vocab + 40, S - lengths[i])
    emb = D.make_embedding(m.vocab, m.hidden, seed=seed)
    wd = [D.make_layer_weights_device(m.hidden, m.ffn, l, seed=seed) for l in range(layers)]
    if fold:
        enc.prepare(wd)
    yb = enc.stack_fwd_bshd(wd, gu.to_dev_i32(lengths), B, S, token_ids=gu.to_dev_i32(ids),
                            embedding=gu.to_dev_bf16(emb), seqlens_host=lengths)
    packed = np.concatenate([ids[i, :lengths[i]] for i in range(B)])
    cu = D.cu_from_lengths(lengths)
    T = int(cu[-1])
    yt = enc.stack_fwd(wd, gu.to_dev_i32(cu), B, T, int(lengths.max()), token_ids=gu.to_dev_i32(packed),
                       embedding=gu.to_dev_bf16(emb), cu_seqlens_host=cu)
    out = gu.bits_of(yb).reshape(B, S, m.hidden), gu.bits_of(yt), wd, emb, ids
    enc.close()
    return out


@pytest.mark.parametrize("fold", [False, True])
def test_stack_bshd_from_ids_matches_thd_and_the_oracle(gu, fold):
    """esm_stack_fwd_bshd from padded token ids (3 layers, hidden 320): valid
    rows bit-equal to the packed stack, padded rows written as 0, and the
    valid rows against the oracle's padded layers chained (free-running,
    within the depth tolerance)."""
    m = D.WORKLOADS["tiny"].model
    lengths = [17, 64, 0, 100, 200, 1]
    S, layers = 224, 3
    yb, yt, wd, emb, ids = _bshd_stack_case(gu, m, lengths, layers, S, seed=3, fold=fold)
    cu = D.cu_from_lengths(lengths)
    for i, L in enumerate(lengths):
        assert np.array_equal(yb[i, :L], yt[cu[i]:cu[i + 1]]), i
        assert not np.any(yb[i, L:]), i
    # oracle: padded rows NaN (they must never reach a valid row)
    e0 = D.bf16_bits_to_f64(emb)
    x = np.full((len(lengths), S, m.hidden), np.nan)
    for i, L in enumerate(lengths):
        x[i, :L] = e0[ids[i, :L]]
    for l in range(layers):
        wr = O.weights_to_f64({k: D.tensor_bits(v) for k, v in wd[l].items()})
        x = O.layer_forward_bshd(x, lengths, wr, m.heads)
    got = D.bf16_bits_to_f64(yb)
    for i, L in enumerate(lengths):
        if L:
            assert gu.rel_err(got[i, :L], x[i, :L]) < _depth_tol(layers - 1), i


@pytest.mark.parametrize("fold", [False, True])
def test_650m_stack_bshd_equals_thd_bitexact(gu, fold):
    """Two 650M-width layers on twelve sequences of the 650M batch padded to
    S = 1024 (the padded benchmark's S): valid rows bit-equal to the packed
    stack, padded rows 0."""
    wl = D.WORKLOADS["650m"]
    lengths = D.make_batch(wl).lengths[:12]
    yb, yt, *_ = _bshd_stack_case(gu, dataclasses.replace(wl.model, layers=2), lengths, 2, 1024, seed=0, fold=fold)
    cu = D.cu_from_lengths(lengths)
    for i, L in enumerate(lengths):
        assert np.array_equal(yb[i, :L], yt[cu[i]:cu[i + 1]]), i
        assert not np.any(yb[i, L:]), i


# ------------------------------------------------------------- LayerNorm folded into the linears

def _chunk_stats_f64(x):
    """Exact (fp64) 256-column chunk (mean, M2) of every row of x [T, H]."""
    T, H = x.shape
    out = []
    for c0 in range(0, H, 256):
        blk = x[:, c0:c0 + 256]
        m = blk.mean(axis=1)
        out.append(np.stack([m, ((blk - m[:, None]) ** 2).sum(axis=1)], axis=1))
    return np.stack(out)          # [chunks, T, 2]


@pytest.mark.parametrize("random_ln", [False, True])
def test_tiny_folded_layer_matches_oracle_and_writes_exact_statistics(gu, tiny, random_ln):
    """esm_prepare_layer folds gamma, beta into W_qkv, W_fc1: the layer against
    the oracle (random gamma, beta included), and the LayerNorm partials its
    fc2 epilogue leaves in the workspace (those of the output rows) against
    fp64 chunk statistics of the output's stored values."""
    b, m = tiny["batch"], tiny["m"]
    enc = _encoder(m)
    wd, wr, _ = gu.layer_weights(m.hidden, m.ffn, 4, random_ln=random_ln)
    enc.prepare_layer(0, wd)
    xb = D.make_hidden(b.T, m.hidden, seed=7)
    ws = enc.workspace(b.T, b.B)
    y = enc.layer_fwd(wd, gu.to_dev_bf16(xb), gu.to_dev_i32(b.cu_seqlens), b.B, b.T, b.max_seqlen,
                      cu_seqlens_host=b.cu_seqlens, workspace=ws)
    got = gu.from_dev(y)
    err = gu.rel_err(got, O.layer_forward(D.bf16_bits_to_f64(xb), b.cu_seqlens, wr, m.heads))
    print(f"tiny folded layer (random LN {random_ln}) rel err {err:.2e}")
    assert err < TOL
    st = enc.workspace_region(ws, b.T, b.B, "stats")
    torch.cuda.synchronize()
    chunks = (m.hidden + 255) // 256
    st = st.cpu().numpy()[:chunks * b.T * 2].reshape(chunks, b.T, 2).astype(np.float64)
    ref = _chunk_stats_f64(got)
    assert np.allclose(st[..., 0], ref[..., 0], rtol=1e-5, atol=1e-6 * np.abs(got).max())
    assert np.allclose(st[..., 1], ref[..., 1], rtol=1e-4, atol=1e-6 * ref[..., 1].max())
    enc.close()


def test_650m_folded_layer_matches_oracle_and_index_invariants(gu, l650):
    """The 650M layer with folded LayerNorms: oracle gate; packed == alone,
    THD == bshd on valid rows with NaN padding, bit for bit."""
    b, m = l650["b"], l650["m"]
    enc = _encoder(m)
    enc.prepare_layer(0, l650["wd"])
    cu = b.cu_seqlens
    y = gu.bits_of(enc.layer_fwd(l650["wd"], gu.to_dev_bf16(b.hidden), gu.to_dev_i32(cu), b.B, b.T, b.max_seqlen))
    err = gu.rel_err(D.bf16_bits_to_f64(y), O.layer_forward(D.bf16_bits_to_f64(b.hidden), cu, l650["wr"], m.heads))
    print(f"650M folded layer rel err {err:.2e}")
    assert err < TOL
    for s in (0, int(np.argmax(b.lengths)), b.B - 1):
        a, L = int(cu[s]), int(b.lengths[s])
        one = enc.layer_fwd(l650["wd"], gu.to_dev_bf16(b.hidden[a:a + L]), gu.to_dev_i32([0, L]), 1, L, L)
        assert np.array_equal(gu.bits_of(one), y[a:a + L]), s
    sel = list(range(10))
    lens = b.lengths[sel]
    S = int(lens.max())
    xb = np.full((len(sel), S, m.hidden), 0x7FC0, dtype=np.uint16)
    for i in sel:
        xb[i, :lens[i]] = b.hidden[cu[i]:cu[i + 1]]
    yb = gu.bits_of(enc.layer_fwd_bshd(l650["wd"], gu.to_dev_bf16(xb), gu.to_dev_i32(lens), len(sel), S,
                                       seqlens_host=lens)).reshape(len(sel), S, m.hidden)
    for i in sel:
        assert np.array_equal(yb[i, :lens[i]], y[cu[i]:cu[i + 1]]), i
        assert not np.any(yb[i, lens[i]:]), i
    enc.close()


def test_prepare_is_rejected_by_quantised_encoders(gu):
    m = D.WORKLOADS["tiny"].model
    enc = esm.Encoder(hidden_size=256, num_attention_heads=4, intermediate_size=1024, num_hidden_layers=1,
                      precision="fp8")
    wd, _, _ = gu.layer_weights(256, 1024, 0)
    with pytest.raises(esm.EsmError) as ei:
        enc.prepare_layer(0, wd)
    assert ei.value.status == 8   # ESM_ERR_STATE
    enc.close()


# ------------------------------------------------------------- 650M single layer

@pytest.fixture(scope="module")
def l650(gu):
    w = D.WORKLOADS["650m_layer"]
    m = w.model
    enc = _encoder(m)
    b = D.make_batch(w)
    wd, wr, _ = gu.layer_weights(m.hidden, m.ffn, 0)
    yield dict(enc=enc, b=b, wd=wd, wr=wr, m=m)
    enc.close()


def test_650m_layer_matches_oracle(gu, l650):
    enc, b, m = l650["enc"], l650["b"], l650["m"]
    y = enc.layer_fwd(l650["wd"], gu.to_dev_bf16(b.hidden), gu.to_dev_i32(b.cu_seqlens), b.B, b.T, b.max_seqlen,
                      cu_seqlens_host=b.cu_seqlens)
    ref = O.layer_forward(D.bf16_bits_to_f64(b.hidden), b.cu_seqlens, l650["wr"], m.heads)
    err = gu.rel_err(gu.from_dev(y), ref)
    print(f"650M layer rel err {err:.2e}")
    assert err < TOL


def test_650m_packed_equals_alone_and_permuted_bitexact(gu, l650):
    enc, b = l650["enc"], l650["b"]
    x = gu.to_dev_bf16(b.hidden)
    full = gu.bits_of(enc.layer_fwd(l650["wd"], x, gu.to_dev_i32(b.cu_seqlens), b.B, b.T, b.max_seqlen))
    cu = b.cu_seqlens
    for s in (0, 7, int(np.argmax(b.lengths)), b.B - 1):
        a, L = int(cu[s]), int(b.lengths[s])
        one = enc.layer_fwd(l650["wd"], gu.to_dev_bf16(b.hidden[a:a + L]), gu.to_dev_i32([0, L]), 1, L, L)
        assert np.array_equal(gu.bits_of(one), full[a:a + L]), s
    perm = D.permutation(b.B)
    hp = np.concatenate([b.hidden[cu[s]:cu[s + 1]] for s in perm])
    cup = D.cu_from_lengths(b.lengths[perm])
    yp = gu.bits_of(enc.layer_fwd(l650["wd"], gu.to_dev_bf16(hp), gu.to_dev_i32(cup), b.B, b.T, b.max_seqlen))
    for i, s in enumerate(perm):
        assert np.array_equal(yp[cup[i]:cup[i + 1]], full[cu[s]:cu[s + 1]])


def test_650m_thd_equals_bshd_valid_rows_and_nan_padding(gu, l650):
    enc, b = l650["enc"], l650["b"]
    sel = list(range(12))
    lens = b.lengths[sel]
    S = int(lens.max())
    cu = b.cu_seqlens
    H = 1280
    xb = np.full((len(sel), S, H), 0x7FC0, dtype=np.uint16)  # NaN padding
    for i, s in enumerate(sel):
        xb[i, :lens[i]] = b.hidden[cu[s]:cu[s + 1]]
    thd_in = np.concatenate([b.hidden[cu[s]:cu[s + 1]] for s in sel])
    cut = D.cu_from_lengths(lens)
    y_thd = gu.bits_of(enc.layer_fwd(l650["wd"], gu.to_dev_bf16(thd_in), gu.to_dev_i32(cut), len(sel),
                                     int(cut[-1]), S))
    y_b = gu.bits_of(enc.layer_fwd_bshd(l650["wd"], gu.to_dev_bf16(xb), gu.to_dev_i32(lens), len(sel), S,
                                        seqlens_host=lens))
    y_b = y_b.reshape(len(sel), S, H)
    for i in range(len(sel)):
        assert np.array_equal(y_b[i, :lens[i]], y_thd[cut[i]:cut[i + 1]]), i
        assert (y_b[i, lens[i]:] == 0).all()


def test_650m_deterministic(gu, l650):
    enc, b = l650["enc"], l650["b"]
    x = gu.to_dev_bf16(b.hidden)
    cu = gu.to_dev_i32(b.cu_seqlens)
    ws = enc.workspace(b.T, b.B)
    y0 = gu.bits_of(enc.layer_fwd(l650["wd"], x, cu, b.B, b.T, b.max_seqlen, workspace=ws))
    for _ in range(2):
        assert np.array_equal(gu.bits_of(enc.layer_fwd(l650["wd"], x, cu, b.B, b.T, b.max_seqlen, workspace=ws)), y0)


# ------------------------------------------------------------- full stacks, sampled

def _stack_layers(gu, wl, tf_seqs, fr_seqs, fold=True):
    """Chained esm_layer_fwd calls over the whole batch from token ids; the
    final output must equal one esm_stack_fwd call bit for bit (with the
    LayerNorms folded, the chained calls take each layer's statistics from a
    statistics pass, the stack from the previous GEMM's epilogue: the bits
    agree only if both give the same partials).  Each layer's
    output is checked on sampled sequences (sequences are independent, so a
    sample can be computed alone) in two ways:
      * teacher-forced (the gate): the oracle layer l is fed the library's
        own layer-(l-1) output on the tf_seqs rows, upcast exactly, so every
        layer is judged on its real activations;
      * free-running (reported): the oracle runs the whole stack from the
        same embedding on the fr_seqs rows.
    Returns (teacher-forced errors, free-running errors) per layer."""
    m = wl.model
    enc = _encoder(m, m.layers)
    b = D.make_batch(wl)
    emb = D.make_embedding(m.vocab, m.hidden)
    wd_all = [D.make_layer_weights_device(m.hidden, m.ffn, l) for l in range(m.layers)]
    if fold:
        enc.prepare(wd_all)
    cu_d = gu.to_dev_i32(b.cu_seqlens)
    ws = enc.workspace(b.T, b.B)
    stack = enc.stack_fwd(wd_all, cu_d, b.B, b.T, b.max_seqlen, token_ids=gu.to_dev_i32(b.ids),
                          embedding=gu.to_dev_bf16(emb), cu_seqlens_host=b.cu_seqlens, workspace=ws)
    stack_bits = gu.bits_of(stack)

    def rows_of(seqs):
        return (np.concatenate([np.arange(b.cu_seqlens[s], b.cu_seqlens[s + 1]) for s in seqs]),
                D.cu_from_lengths(b.lengths[seqs]))

    tf_rows, tf_cu = rows_of(tf_seqs)
    fr_rows, fr_cu = rows_of(fr_seqs)
    e0 = D.bf16_bits_to_f64(emb)
    tf_in, fr_ref = e0[b.ids[tf_rows]], e0[b.ids[fr_rows]]
    cur = gu.to_dev_bf16(emb[b.ids])
    e_tf, e_fr = [], []
    for l in range(m.layers):
        cur = enc.layer_fwd(wd_all[l], cur, cu_d, b.B, b.T, b.max_seqlen, layer_idx=l, workspace=ws)
        y = gu.from_dev(cur)
        wr = O.weights_to_f64({k: D.tensor_bits(v) for k, v in wd_all[l].items()})
        e_tf.append(gu.rel_err(y[tf_rows], O.layer_forward(tf_in, tf_cu, wr, m.heads)))
        tf_in = y[tf_rows]
        fr_ref = O.layer_forward(fr_ref, fr_cu, wr, m.heads)
        e_fr.append(gu.rel_err(y[fr_rows], fr_ref))
    assert np.array_equal(gu.bits_of(cur), stack_bits), "stack differs from chained layer calls"
    enc.close()
    return e_tf, e_fr


def _depth_tol(l: int) -> float:
    """Free-running tolerance after l+1 layers: every layer adds independent
    bf16 rounding of the same relative size, so the stack error grows as the
    square root of depth times the single-layer gate."""
    return TOL * float(np.sqrt(l + 1))


def _short_median_long(b):
    order = np.argsort(b.lengths, kind="stable")
    return sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})


def test_650m_stack_33_layers_every_layer_teacher_forced(gu):
    """cfg 650M: 87 packed sequences (T = 32293), 33 layers from token ids;
    the per-layer gate on the shortest, median and longest (997 residues)
    sequences."""
    wl = D.WORKLOADS["650m"]
    b = D.make_batch(wl)
    sample = _short_median_long(b)
    assert int(b.lengths.max()) in b.lengths[sample]
    e_tf, e_fr = _stack_layers(gu, wl, sample, sample)
    print("650M per-layer errors, teacher-forced:", " ".join(f"{e:.1e}" for e in e_tf))
    print("650M per-layer errors, free-running:", " ".join(f"{e:.1e}" for e in e_fr))
    assert max(e_tf) < TOL, e_tf
    assert all(e < _depth_tol(l) for l, e in enumerate(e_fr)), e_fr


def test_3b_stack_36_layers_every_layer_teacher_forced(gu):
    """cfg 3B-shaped: 39 packed sequences (T = 16208), 36 layers of hidden
    2560; the per-layer gate on the shortest and the longest (908 residues)
    sequences, free-running reported on the shortest."""
    wl = D.WORKLOADS["3b"]
    b = D.make_batch(wl)
    sample = sorted({int(np.argmin(b.lengths)), int(np.argmax(b.lengths))})
    e_tf, e_fr = _stack_layers(gu, wl, sample, [int(np.argmin(b.lengths))])
    print("3B per-layer errors, teacher-forced:", " ".join(f"{e:.1e}" for e in e_tf))
    print("3B per-layer errors, free-running:", " ".join(f"{e:.1e}" for e in e_fr))
    assert max(e_tf) < TOL, e_tf
    assert all(e < _depth_tol(l) for l, e in enumerate(e_fr)), e_fr


@pytest.mark.parametrize("name", ["650m", "3b"])
def test_every_layer_of_the_stack_on_seeded_input(gu, name):
    """Per-layer gate: each layer of the full-depth model, with its own weights,
    on a seeded N(0,1) input batch at the full batch shape; the oracle sees
    the same seeded input (sampled sequences)."""
    wl = D.WORKLOADS[name]
    m = wl.model
    b = D.make_batch(wl)
    enc = _encoder(m)
    order = np.argsort(b.lengths, kind="stable")
    sample = sorted({int(order[0]), int(order[len(order) // 2])}) if name == "650m" else [int(order[0])]
    rows = np.concatenate([np.arange(b.cu_seqlens[s], b.cu_seqlens[s + 1]) for s in sample])
    cu_d = gu.to_dev_i32(b.cu_seqlens)
    ws = enc.workspace(b.T, b.B)
    errs = []
    for l in range(m.layers):
        xb = D.make_hidden(b.T, m.hidden, seed=0, stream=100 + l)
        wd = D.make_layer_weights_device(m.hidden, m.ffn, l)
        y = enc.layer_fwd(wd, gu.to_dev_bf16(xb), cu_d, b.B, b.T, b.max_seqlen, layer_idx=l, workspace=ws)
        wr = O.weights_to_f64({k: D.tensor_bits(v) for k, v in wd.items()})
        ref, _ = O.layer_forward_seqs(D.bf16_bits_to_f64(xb), b.cu_seqlens, wr, m.heads, sample)
        errs.append(gu.rel_err(gu.from_dev(y)[rows], ref))
    enc.close()
    print(f"{name} per-layer errors on seeded inputs: max {max(errs):.2e}")
    assert max(errs) < TOL, errs
