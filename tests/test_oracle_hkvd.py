"""Pins of the oracle's gradual-filtering part (KV deviation and the nested per-layer selection,
KVCache reuse 01, §1.3.2-§1.3.4) against hand-worked values, brute force and planted structure.
No GPU is involved.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
from workloads import make_custom


def _rope_inverse(x, pos, base):
    """R(-p) x written out per pair with cos/sin (independent of the oracle's rope)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    out = np.empty_like(x)
    pos = np.asarray(pos, dtype=np.float64)
    for i in range(h):
        th = base ** (-(2.0 * i) / d)
        c, s = np.cos(-pos * th), np.sin(-pos * th)
        out[..., i] = x[..., i] * c - x[..., i + h] * s
        out[..., i + h] = x[..., i] * s + x[..., i + h] * c
    return out


def test_kv_deviation_hand_example():
    # one KV head, d = 2 (theta_0 = 1): rows are listed out of position order on purpose
    kf = np.array([[[3.0, 0.0]], [[math.cos(1.0), math.sin(1.0)]], [[0.0, 0.0]]])
    vf = np.array([[[0.0, 4.0]], [[1.0, 1.0]], [[4.0, 6.0]]])
    kf = O.round_to_storage(kf, "f32")
    row_pos = np.array([2, 0, 1], dtype=np.int32)
    k_new = np.float32([[[0.0, 0.0]], [[0.0, 0.0]], [[1.0, 0.0]]])   # row 2 at p = 1: R(1)(1, 0) = kf[1]
    v_new = np.float32([[[1.0, 2.0]], [[0.0, 0.0]], [[1.0, 1.0]]])
    dev = O.kv_deviation(kf, vf, k_new, v_new, row_pos, 3, "f32", 10000.0)
    # row 0 at p = 2: |V diff| = |(1,2) - (4,6)| = 5; row 1 at p = 0: |(0,0)-(3,0), (0,0)-(0,4)| = 5;
    # row 2 at p = 1: K matches after rotation, V matches: 0
    assert dev[0] == 5.0 and dev[1] == 5.0 and dev[2] == 0.0
    # only the first n_rows rows are measured
    assert O.kv_deviation(kf, vf, k_new, v_new, row_pos, 2, "f32", 10000.0).shape == (2,)


def test_kv_deviation_vanishes_for_unrotated_reused_rows():
    w = make_custom(dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=16, chunk_lens=[9, 7],
                    orig_pos=[0, 5], query_len=2, seed=11)
    lay = w.layer(0)
    L = 18
    kf, vf = O.fuse_rerotate(lay["k_store"], lay["v_store"], w.chunks[0], L, "f32", 10000.0)
    rp = np.array([1, 4, 8, 13, 15], dtype=np.int32)
    k_new = np.float32(_rope_inverse(kf[rp], rp[:, None], 10000.0))   # fresh K equal to the reused one
    v_new = np.float32(vf[rp])
    dev = O.kv_deviation(kf, vf, k_new, v_new, rp, len(rp), "f32", 10000.0)
    scale = np.sqrt((kf[rp] ** 2).sum(axis=(1, 2)))
    assert np.all(dev <= 1e-6 * scale), dev
    # the same fresh rows measured at other context positions deviate by about the key's size
    dev_wrong = O.kv_deviation(kf, vf, k_new, v_new, np.roll(rp, 1), len(rp), "f32", 10000.0)
    assert np.all(dev_wrong > 1e-2 * scale)


def test_hkvd_filter_brute_force_and_ties():
    rng = np.random.default_rng(5)
    for trial in range(40):
        n_prev = int(rng.integers(0, 8))
        dev = rng.integers(0, 4, n_prev).astype(np.float64)       # many ties
        ctx = np.sort(rng.choice(100, n_prev, replace=False)).astype(np.int32)
        rows = np.concatenate([ctx, [100, 101]]).astype(np.int32)   # two query rows
        for n_keep in range(n_prev + 1):
            got = O.hkvd_filter(dev, rows, n_prev, n_keep)
            assert list(got[n_keep:]) == [100, 101]
            # brute force: the unique subset where every kept row beats every dropped row
            # (higher deviation, or equal deviation and lower row)
            good = []
            for sub in itertools.combinations(range(n_prev), n_keep):
                s = set(sub)
                if all(dev[i] > dev[j] or (dev[i] == dev[j] and i < j)
                       for i in s for j in range(n_prev) if j not in s):
                    good.append(sub)
            assert len(good) == 1
            assert list(got[:n_keep]) == [int(ctx[i]) for i in good[0]]


def test_hkvd_filter_ranks_in_float64():
    # equal as float32, different as float64: the plain definition ranks the larger value first
    # (the device ranks float32 deviations; the GPU tests allow swaps inside the 1e-5 window)
    dev = np.array([1.0, 1.0 + 1e-12, 0.5])
    rows = np.array([3, 7, 9, 20], dtype=np.int32)
    assert list(O.hkvd_filter(dev, rows, 3, 1)) == [7, 20]
    # an exact tie keeps the lower row
    assert list(O.hkvd_filter(np.array([2.0, 2.0, 0.5]), rows, 3, 1)) == [3, 20]


def _taper_workload():
    return make_custom(dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=16, chunk_lens=[11, 13, 8],
                       orig_pos=[0, 3, 0], query_len=3, seed=23)


def test_gradual_filtering_keeps_the_planted_deviating_rows():
    w = _taper_workload()
    base = 10000.0
    L_ctx, Lq = 32, 3
    L = L_ctx + Lq
    counts = [12, 7, 4]
    lay0 = w.layer(0)
    # layers 1 and 2 reuse layer 0's stores; their fresh K/V equal the reused rows except for a
    # planted set of tokens with a large change, so deviation ranking must recover that set
    kf, vf = O.fuse_rerotate(lay0["k_store"], lay0["v_store"], w.chunks[0], L, "f32", base)
    pos = np.arange(L)
    k_same = np.float32(_rope_inverse(kf, pos[:, None], base))
    r0 = O.row_positions(np.array([0, 2, 3, 5, 8, 9, 14, 17, 20, 25, 29, 31]), L_ctx, Lq)
    planted = {1: [3, 9, 14, 20, 25, 31, 0], 2: [9, 20, 31, 3]}
    layers = [{"k_store": lay0["k_store"], "v_store": lay0["v_store"], "q_new": lay0["q_new"][0],
               "k_new": lay0["k_new"][0], "v_new": lay0["v_new"][0]}]
    for l in (1, 2):
        kn = np.broadcast_to(k_same, k_same.shape).copy()
        vn = np.float32(vf).copy()
        for j, p in enumerate(planted[l]):
            kn[p] += np.float32(3.0 + j)   # distinct deviations, the first planted row largest
        layers.append({"k_store": lay0["k_store"], "v_store": lay0["v_store"], "q_new": lay0["q_new"][0],
                       "k_new": kn, "v_new": vn})
    res = O.gradual_filter_layers(layers=layers, chunks=w.chunks[0], L=L, dtype="f32", base=base,
                                  n_kv_heads=2, counts=counts, row_pos0=r0, attn_rows=[0])
    assert list(res[0]["row_pos"]) == list(r0)
    for l in (1, 2):
        rp = res[l]["row_pos"]
        assert list(rp[:counts[l]]) == sorted(planted[l][:counts[l]])
        assert list(rp[counts[l]:]) == list(range(L_ctx, L))
        assert set(rp[:counts[l]]) <= set(res[l - 1]["row_pos"][:counts[l - 1]])
    with pytest.raises(ValueError):
        O.gradual_filter_layers(layers=layers[:2], chunks=w.chunks[0], L=L, dtype="f32", base=base,
                                n_kv_heads=2, counts=[4, 6], row_pos0=O.row_positions(np.arange(4), L_ctx, Lq))


def test_keeping_every_row_equals_the_given_rows():
    w = _taper_workload()
    lay = w.layer(0)
    L = 35
    prev = O.row_positions(np.array([1, 4, 6, 10, 22, 30]), 32, 3)
    kw = dict(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=L, q_new=lay["q_new"][0],
              k_new=lay["k_new"][0], v_new=lay["v_new"][0], dtype="f32", base=10000.0, n_kv_heads=2,
              attn_rows=[0, 3, 6])
    a = O.fused_layer(row_pos=prev, **kw)
    b = O.fused_layer(hkvd_prev=prev, hkvd_n_prev=6, n_select=6, **kw)
    assert list(a["row_pos"]) == list(b["row_pos"])
    np.testing.assert_array_equal(a["out"], b["out"])
    assert b["dev"].shape == (6,) and np.all(b["dev"] > 0)
