"""Pins of the oracle's Cache-Craft selection (CSDN article §2.1-§2.2; KVCache reuse 01 §2.3):
attention statistics against closed forms, invariants and an independent softmax; CCI, prefix
overlap and the recompute count against hand-worked values. No GPU is involved.
"""
import math

import numpy as np
import torch

import oracle as O
from workloads import make_custom


def _rope_fwd(x, pos, base):
    """R(p) x per pair written with cos/sin (independent of the oracle's rope)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    out = np.empty_like(x)
    pos = np.asarray(pos, dtype=np.float64)
    for i in range(h):
        th = base ** (-(2.0 * i) / d)
        c, s = np.cos(pos * th), np.sin(pos * th)
        out[..., i] = x[..., i] * c - x[..., i + h] * s
        out[..., i + h] = x[..., i] * s + x[..., i + h] * c
    return out


def _setup(dtype="f32"):
    w = make_custom(dtype=dtype, n_q_heads=4, n_kv_heads=2, head_dim=16, chunk_lens=[11, 7, 9],
                    orig_pos=[0, 0, 0], query_len=2, seed=61)
    lay = w.layer(0)
    L_ctx = 27
    kc = O.round_to_storage(_rope_fwd(O.to_f64(lay["k_new"][0][:L_ctx], dtype), np.arange(L_ctx)[:, None], 10000.0),
                            dtype)
    return w, lay, kc


def test_stats_rows_sum_to_heads_and_respect_causality():
    w, lay, kc = _setup()
    inter = O.chunk_attention_stats(lay["q_new"][0], kc, w.chunks[0], 2, "f32", 10000.0)
    assert inter.shape == (27, 3)
    np.testing.assert_allclose(inter.sum(axis=1), 4.0, rtol=1e-12)
    assert np.all(inter[:11, 1:] == 0.0)                  # the first chunk sees no later chunk
    assert np.all(inter[11:18, 2] == 0.0)
    np.testing.assert_allclose(inter[0], [4.0, 0.0, 0.0], rtol=1e-15)


def test_stats_uniform_attention_closed_form():
    w, lay, kc = _setup()
    q0 = np.zeros_like(lay["q_new"][0])                   # all logits 0: uniform over s <= t
    inter = O.chunk_attention_stats(q0, kc, w.chunks[0], 2, "f32", 10000.0)
    starts = [0, 11, 18, 27]
    for t in range(27):
        for j in range(3):
            seen = max(0, min(t + 1, starts[j + 1]) - starts[j])
            assert abs(inter[t, j] - 4.0 * seen / (t + 1)) < 1e-12


def test_stats_match_independent_softmax():
    w, lay, kc = _setup()
    rows = [0, 5, 11, 12, 20, 26]
    inter = O.chunk_attention_stats(lay["q_new"][0], kc, w.chunks[0], 2, "f32", 10000.0, rows=rows)
    q = _rope_fwd(O.to_f64(lay["q_new"][0][:27], "f32"), np.arange(27)[:, None], 10000.0)
    starts = [0, 11, 18, 27]
    for i, t in enumerate(rows):
        for j in range(3):
            tot = 0.0
            for h in range(4):
                x = torch.from_numpy(kc[:t + 1, h // 2] @ q[t, h] / 4.0)
                p = torch.softmax(x, dim=0).numpy()
                tot += p[starts[j]:min(starts[j + 1], t + 1)].sum()
            assert abs(inter[i, j] - tot) < 1e-12


def test_preceding_scores_and_cci_hand_example():
    chunks = np.array([[0, 2, 0, 0], [2, 2, 2, 0]])
    inter = np.array([[2.0, 0.0], [2.0, 0.0], [0.5, 1.5], [1.0, 1.0]])   # two heads
    np.testing.assert_array_equal(O.preceding_chunk_scores(inter, chunks), [0.0, 0.0, 0.5, 1.0])
    cci = O.cache_context_impact(inter, chunks)
    assert cci[0] == 0.5                                   # nothing before the first chunk: sigmoid(0)
    assert abs(cci[1] - 1.0 / (1.0 + math.exp(-1.5 / 2.5))) < 1e-15


def test_prefix_overlap_hand_examples():
    att = {10: 3.0, 11: 1.0, 12: 4.0}
    assert O.prefix_overlap(att, [10, 11, 12], [10, 11, 12]) == 1.0              # same prefix
    assert O.prefix_overlap(att, [10, 11, 12], [12, 11, 10]) == 0.0              # reversed: gamma = 1
    assert abs(O.prefix_overlap(att, [10, 11, 12], [10, 12]) - 7.0 / 8.0) < 1e-15   # chunk 11 dropped
    # one swap among three shared: gamma = 1/3
    assert abs(O.prefix_overlap(att, [10, 11, 12], [11, 10, 12]) - (2.0 / 3.0)) < 1e-15
    assert O.prefix_overlap(att, [], [10]) == 0.0
    assert O.prefix_overlap(att, [10, 11], [99]) == 0.0


def test_cachecraft_count():
    assert O.cachecraft_count(0.4, 0.5, 0.0, 100) == 20
    assert O.cachecraft_count(0.4, 0.5, 0.5, 101) == 11            # 10.1 rounds up
    assert O.cachecraft_count(0.3, 0.9, 1.0, 512) == 0             # full overlap: nothing to fix
    assert O.cachecraft_count(2.0, 0.9, 0.0, 50) == 50             # clamped to the chunk
    assert O.cachecraft_count(0.4, 0.0, 0.0, 64) == 0
