"""Pins of the oracle's anchor probe prefix and the query-centric layer baselines (QCFuse summary
(zh) §2.A anchors as a lightweight prefix; §4 QCAll / QCLast) against library routines, brute
construction and special cases. No GPU is involved.
"""
import numpy as np
import torch

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


def _rope_fwd(x, pos, base):
    return _rope_inverse(x, -np.asarray(pos, dtype=np.float64), base)


def _workload():
    return make_custom(dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=16, chunk_lens=[20, 13, 17],
                       orig_pos=[0, 40, 7], query_len=5, seed=41)


def test_prefix_order_rows_and_rotation():
    w = _workload()
    lay = w.layer(0)
    anchors = np.array([[9, 2, 15], [12, 0, 5], [3, 16, 8]], dtype=np.int32)   # not in token order
    kp, vp = O.anchor_prefix(lay["k_store"], lay["v_store"], w.chunks[0], anchors, "f32", 10000.0)
    assert kp.shape == (9, 2, 16) and vp.shape == (9, 2, 16)
    ks, vs = O.to_f64(lay["k_store"], "f32"), O.to_f64(lay["v_store"], "f32")
    a = 0
    for (src, _T, _dst, orig), anc in zip(w.chunks[0].tolist(), anchors.tolist()):
        for t in sorted(anc):
            np.testing.assert_array_equal(vp[a], vs[src + t])                  # V copied, token order
            # the key's content without rotation is the cached key's without rotation
            np.testing.assert_allclose(_rope_inverse(kp[a], a, 10000.0),
                                       _rope_inverse(ks[src + t], orig + t, 10000.0), rtol=0, atol=2e-6)
            a += 1


def test_prefix_with_zero_shift_copies_bits():
    w = make_custom(dtype="bf16", n_q_heads=2, n_kv_heads=1, head_dim=16, chunk_lens=[12], orig_pos=[0],
                    query_len=2, seed=42)
    lay = w.layer(0)
    kp, vp = O.anchor_prefix(lay["k_store"], lay["v_store"], w.chunks[0], np.array([[3, 0, 1, 2]]), "bf16", 10000.0)
    # anchors 0..3 at orig 0 land on rows 0..3: no rotation, bit-exact copies
    np.testing.assert_array_equal(kp, O.to_f64(lay["k_store"], "bf16")[:4])
    np.testing.assert_array_equal(vp, O.to_f64(lay["v_store"], "bf16")[:4])


def _sdpa_causal(q, k, v):
    Hq, Hkv = q.shape[1], k.shape[1]
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).repeat_interleave(Hq // Hkv, 0)[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).repeat_interleave(Hq // Hkv, 0)[None]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].numpy().transpose(1, 0, 2)


def test_probe_equals_causal_prefill_over_anchors_then_query():
    w = _workload()
    base = 10000.0
    lay = w.layer(0)
    anchors = O.extract_anchors(w.k_crit, w.chunks[0], 3, "f32")
    kp, vp = O.anchor_prefix(lay["k_store"], lay["v_store"], w.chunks[0], anchors, "f32", base)
    A, Lq = kp.shape[0], 5
    qn, kn, vn = (lay[n][0][50:55] for n in ("q_new", "k_new", "v_new"))   # the query rows' projections
    out, _lse = O.anchor_probe(kp, vp, qn, kn, vn, "f32", base)
    # the same computation as one causal prefill of A + Lq tokens: anchors carry their un-rotated
    # cached content, then the query; every token rotated at its own row
    ks, vs = O.to_f64(lay["k_store"], "f32"), O.to_f64(lay["v_store"], "f32")
    k_raw, v_raw = [], []
    for (src, _T, _dst, orig), anc in zip(w.chunks[0].tolist(), anchors.tolist()):
        for t in sorted(anc):
            k_raw.append(_rope_inverse(ks[src + t], orig + t, base))
            v_raw.append(vs[src + t])
    k_all = np.concatenate([np.asarray(k_raw), O.to_f64(kn, "f32")])
    v_all = np.concatenate([np.asarray(v_raw), O.to_f64(vn, "f32")])
    q_all = np.concatenate([np.zeros((A,) + qn.shape[1:]), O.to_f64(qn, "f32")])
    pos = np.arange(A + Lq)[:, None]
    ref = _sdpa_causal(_rope_fwd(q_all, pos, base), _rope_fwd(k_all, pos, base), v_all)[A:]
    # the probe rounds keys to the storage type (float32 here)
    np.testing.assert_allclose(out, ref, rtol=0, atol=2e-6)


def test_probe_without_prefix_is_plain_causal_attention():
    w = _workload()
    lay = w.layer(0)
    qn, kn, vn = (lay[n][0][:4] for n in ("q_new", "k_new", "v_new"))
    empty = np.zeros((0, 2, 16))
    out, _ = O.anchor_probe(empty, empty, qn, kn, vn, "f32", 10000.0)
    pos = np.arange(4)[:, None]
    ref = _sdpa_causal(_rope_fwd(O.to_f64(qn, "f32"), pos, 10000.0),
                       _rope_fwd(O.to_f64(kn, "f32"), pos, 10000.0), O.to_f64(vn, "f32"))
    np.testing.assert_allclose(out, ref, rtol=0, atol=2e-6)


def test_query_centric_layer_modes():
    w = _workload()
    lays = [w.layer(0)]
    w2 = make_custom(dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=16, chunk_lens=[20, 13, 17],
                     orig_pos=[0, 40, 7], query_len=5, seed=43)
    lays.append(w2.layer(0))
    qs = [w.q_crit[0], w2.q_crit[0]]
    ks = [lays[0]["k_store"], lays[1]["k_store"]]
    sc_all, sel_all = O.query_centric_layers(qs, ks, w.chunks[0], 2, "f32", 10000.0, 9, "all")
    sc_last, sel_last = O.query_centric_layers(qs, ks, w.chunks[0], 2, "f32", 10000.0, 9, "last")
    assert sc_all.shape == (2, 50) and sc_last.shape == (1, 50)
    # every layer's scores sum to Lq * Hq (softmax rows over the context)
    np.testing.assert_allclose(sc_all.sum(axis=1), 5 * 4, rtol=1e-12)
    np.testing.assert_array_equal(sc_last[0], sc_all[1])               # the last layer's own scores
    assert all(list(s) == list(sel_last[1]) for s in sel_last)          # one selection for every layer
    assert list(sel_all[1]) == list(sel_last[1])
    assert list(sel_all[0]) != list(sel_all[1])                         # the layers see different keys
