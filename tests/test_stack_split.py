"""esm_stack_split, the host rule that decides where esm_stack_fwd runs a batch
as two groups of whole sequences on two streams (host only, no GPU needed:
with no device visible the rule counts 256 compute units, the MI355X's).

A split must not add rounds of workgroups to any of the layer's GEMMs: for
each output width (3H, H, F) the two groups' rounds, with the dispatch's tile
choice (320-row tiles when rounds x 320 <= rounds x 256 of the 256-row
tiles), sum to at most the whole batch's; among qualifying sequence
boundaries the most balanced is taken; 0 means one group."""
import numpy as np
import pytest

from protein_language_model_amd import datagen as D
from protein_language_model_amd import esm

CUS = 256


def _rounds(rows, n):
    tn = -(-n // 256)
    r256 = -(-(-(-rows // 256) * tn) // CUS)
    r320 = -(-(-(-rows // 320) * tn) // CUS)
    return r320 if r320 * 320 <= r256 * 256 else r256


def _rule(H, F, cu):
    cu = np.asarray(cu, dtype=np.int64)
    B, T = len(cu) - 1, int(cu[-1])
    if B < 2 or T < 4096:
        return 0
    widths = (3 * H, H, F)
    best, bs = T, 0
    for b in range(1, B):
        t1, t2 = int(cu[b]), T - int(cu[b])
        if t1 <= 0 or t2 <= 0:
            continue
        if all(_rounds(t1, w) + _rounds(t2, w) <= _rounds(T, w) for w in widths) and abs(2 * t1 - T) < best:
            best, bs = abs(2 * t1 - T), b
    return bs


def test_650m_batch_splits_into_two_whole_round_groups():
    wl = D.WORKLOADS["650m"]
    b = D.make_batch(wl)
    m = wl.model
    bs = esm.stack_split(m.hidden, m.ffn, b.cu_seqlens)
    assert bs > 0
    t1 = int(b.cu_seqlens[bs])
    T = b.T
    # per group: 255 out-proj / fc2 tiles (one round), 765 qkv (three), 1020 fc1 (four)
    for w, whole in ((3 * m.hidden, 6), (m.hidden, 2), (m.ffn, 8)):
        assert _rounds(T, w) == whole
        assert _rounds(t1, w) + _rounds(T - t1, w) <= whole
    assert bs == _rule(m.hidden, m.ffn, b.cu_seqlens)


def test_3b_batch_runs_as_one_group():
    wl = D.WORKLOADS["3b"]
    b = D.make_batch(wl)
    assert esm.stack_split(wl.model.hidden, wl.model.ffn, b.cu_seqlens) == 0
    # no boundary qualifies: 51 row tiles can never split into two single rounds at 10 column tiles
    assert _rule(wl.model.hidden, wl.model.ffn, b.cu_seqlens) == 0


@pytest.mark.parametrize("seed", range(6))
def test_rule_on_random_batches(seed):
    r = np.random.default_rng(seed)
    H, F = [(256, 1024), (1280, 5120), (640, 2560)][seed % 3]
    lens = r.integers(0, 1025, size=int(r.integers(2, 200)))
    cu = D.cu_from_lengths(lens)
    assert esm.stack_split(H, F, cu) == _rule(H, F, cu)


def test_small_batches_and_bad_arguments():
    assert esm.stack_split(1280, 5120, [0, 2000, 4000]) == 0      # below 4096 rows
    assert esm.stack_split(1280, 5120, [0, 40000]) == 0           # one sequence
    with pytest.raises(esm.EsmError) as ei:
        esm.stack_split(1280, 5120, [1, 2, 3])
    assert ei.value.status == 2
    with pytest.raises(esm.EsmError) as ei:
        esm.stack_split(0, 5120, [0, 5000, 10000])
    assert ei.value.status == 2
