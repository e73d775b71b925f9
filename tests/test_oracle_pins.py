"""Pins of the fp64 oracle against things other than itself.

Each test ties one part of the oracle to a library routine, a closed form, an
invariant the method guarantees, or brute force on tiny inputs, chosen so that a
plausible slip (a dropped term, a wrong sign or index, a transposed operand, a
wrong tie-break or rounding) fails at least one of them. No GPU is involved.
"""
import cmath
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle as O
from workloads import make_custom, make_workload
from workloads.gen import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers (independent formulations)

def rope_complex(x, pos, base):
    """Rotary embedding written as a complex product: (x_i + j x_{i+d/2}) * exp(j pos theta_i)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    theta = np.array([base ** (-(2.0 * i) / d) for i in range(h)])
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def sdpa_causal(q, k, v):
    """torch SDPA (CPU, float64) with a causal mask; q [L,Hq,d], k/v [L,Hkv,d]; GQA by repeat."""
    Hq, Hkv = q.shape[1], k.shape[1]
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).repeat_interleave(Hq // Hkv, 0)[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).repeat_interleave(Hq // Hkv, 0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return o[0].numpy().transpose(1, 0, 2)


def store_round_torch(x, dtype):
    t = torch.from_numpy(np.asarray(x, dtype=np.float64))
    return t.float().double().numpy() if dtype == "f32" else None


# ----------------------------------------------------------------------------- storage rounding

def test_bf16_round_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 8, 20000),
                        np.float32([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.5, 0.0])])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(O.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour is 1.
    assert O.bf16_round(np.float64(1.0 + 2.0 ** -8)) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: the even neighbour is 1 + 2^-6.
    assert O.bf16_round(np.float64(1.0 + 3 * 2.0 ** -8)) == 1.0 + 2.0 ** -6
    # just above a tie rounds up
    assert O.bf16_round(np.float64(1.0 + 2.0 ** -8 + 2.0 ** -30)) == 1.0 + 2.0 ** -7


def test_storage_bits_roundtrip_generator_bits():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4096).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    np.testing.assert_array_equal(O.storage_bits(O.to_f64(bits, "bf16"), "bf16"), bits)


# ----------------------------------------------------------------------------- rotary embedding

def test_rope_theta_closed_form():
    th = O.rope_theta(128, 10000.0)
    assert th[0] == 1.0
    assert math.isclose(th[1], 10000.0 ** (-1 / 64), rel_tol=1e-15)
    ratios = th[1:] / th[:-1]
    np.testing.assert_allclose(ratios, 10000.0 ** (-2 / 128), rtol=1e-13)
    assert math.isclose(th[-1] * 10000.0 ** (-2 / 128), 1 / 10000.0, rel_tol=1e-12)  # theta_{d/2} would be 1/base


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_rope_equals_complex_rotation(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((7, 3, d))
    pos = rng.integers(-40000, 40000, size=(7, 3))
    np.testing.assert_allclose(O.rope(x, pos, 10000.0), rope_complex(x, pos, 10000.0), rtol=0, atol=1e-9)


def test_rope_direction_on_a_2d_vector():
    # d = 2: theta_0 = 1, so position p rotates (1, 0) counter-clockwise by p radians.
    for p in [0, 1, 2, -3, 31]:
        np.testing.assert_allclose(O.rope(np.array([1.0, 0.0]), p, 10000.0), [math.cos(p), math.sin(p)], atol=1e-14)


def test_rope_composition_and_inverse():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 2, 64))
    for a, b in [(3, 5), (-700, 1200), (32000, -31999), (0, 0)]:
        np.testing.assert_allclose(O.rope(O.rope(x, a, 10000.0), b, 10000.0), O.rope(x, a + b, 10000.0),
                                   rtol=0, atol=1e-10)
        np.testing.assert_allclose(O.rope(O.rope(x, a, 10000.0), -a, 10000.0), x, rtol=0, atol=1e-10)
    assert np.array_equal(O.rope(x, 0, 10000.0), x)


def test_rope_relative_position_property():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    base = np.dot(O.rope(q, 100, 10000.0), O.rope(k, 37, 10000.0))
    for shift in [1, 513, 17920, -90]:
        assert math.isclose(np.dot(O.rope(q, 100 + shift, 10000.0), O.rope(k, 37 + shift, 10000.0)), base,
                            rel_tol=1e-10, abs_tol=1e-10)


# ----------------------------------------------------------------------------- S1 re-rotation

def test_rerotate_zero_delta_is_bit_exact_copy():
    w = make_custom(dtype="bf16", chunk_lens=(8, 8), orig_pos=(0, 8), query_len=2)  # deltas 0, 0
    lay = w.layer(0)
    kf, vf = O.fuse_rerotate(lay["k_store"], lay["v_store"], w.chunks[0], 18, "bf16", 10000.0)
    np.testing.assert_array_equal(O.storage_bits(kf[:16], "bf16"), lay["k_store"][:16])
    np.testing.assert_array_equal(O.storage_bits(vf[:16], "bf16"), lay["v_store"][:16])
    assert np.isnan(kf[16:]).all()


def test_rerotate_matches_complex_rotation_then_rounding():
    w = make_custom(dtype="f32", chunk_lens=(5, 9, 3), orig_pos=(4, 0, 100), query_len=1)
    lay = w.layer(0)
    kf, vf = O.fuse_rerotate(lay["k_store"], lay["v_store"], w.chunks[0], 18, "f32", 10000.0)
    n = 0
    for (src, T, dst, orig) in w.chunks[0].tolist():
        delta = dst - orig
        ref = store_round_torch(rope_complex(lay["k_store"][src:src + T].astype(np.float64), delta, 10000.0), "f32")
        np.testing.assert_allclose(kf[n:n + T], ref, rtol=2e-7, atol=0)
        np.testing.assert_array_equal(vf[n:n + T], lay["v_store"][src:src + T])
        n += T


def test_orig_pos_shift_gives_same_fused_keys():
    # A chunk cached at original position P holds keys rotated by P more; moving it to the same
    # fused row must rotate it back by P more, landing on the same keys (f32 store, 1 rounding).
    w = make_custom(dtype="f32", chunk_lens=(6, 10), orig_pos=(0, 0), query_len=1)
    lay = w.layer(0)
    ks = lay["k_store"].astype(np.float64)
    P = 2345
    ks_shift = O.rope(ks, P, 10000.0).astype(np.float32)
    ch = w.chunks[0].copy()
    ch[:, 3] += P
    a, _ = O.fuse_rerotate(lay["k_store"], lay["v_store"], w.chunks[0], 17, "f32", 10000.0)
    b, _ = O.fuse_rerotate(ks_shift, lay["v_store"], ch, 17, "f32", 10000.0)
    np.testing.assert_allclose(a[:16], b[:16], rtol=0, atol=2e-6)


# ----------------------------------------------------------------------------- anchors

def test_anchor_brute_force_and_tie_break():
    k = np.zeros((6, 1, 2), dtype=np.float32)
    k[:, 0, 0] = [1.0, 3.0, 2.0, 3.0, 0.5, 2.0]
    chunks = np.array([[0, 6, 0, 0]], dtype=np.int32)
    # norms 1,3,2,3,.5,2: order (3 at t=1), (3 at t=3), (2 at t=2), (2 at t=5)
    np.testing.assert_array_equal(O.extract_anchors(k, chunks, 4, "f32"), [[1, 3, 2, 5]])


def test_anchor_norm_spans_every_kv_head():
    # Three KV heads, d = 2. Full-row L2 norms: t0 3, t1 sqrt(13) = 3.61, t2 3.5, t3 sqrt(12) = 3.46,
    # so the anchors in order are 1, 2, 3, 0. A norm of head 0 alone would rank 0 first, of the last
    # head alone 2 first, the largest per-head norm 2, 0, 1, 3, and a sum of per-head norms 3 first.
    k = np.zeros((4, 3, 2), dtype=np.float32)
    k[0, 0] = (3.0, 0.0)
    k[1, 0], k[1, 1], k[1, 2] = (1.0, 0.0), (2.0, 2.0), (2.0, 0.0)
    k[2, 2] = (0.0, 3.5)
    k[3, :, 0] = 2.0
    chunks = np.array([[0, 4, 0, 0]], dtype=np.int32)
    np.testing.assert_array_equal(O.extract_anchors(k, chunks, 4, "f32"), [[1, 2, 3, 0]])
    np.testing.assert_allclose(O.key_norms(k, "f32"), [3.0, np.sqrt(13.0), 3.5, np.sqrt(12.0)], rtol=1e-15)


def test_key_norms_equal_library_norm_of_flattened_rows():
    # eight KV heads x 128 dims, bf16 with the x4 outliers: numpy's own vector norm of each stored row
    w = make_workload(1)
    rows = O.to_f64(w.k_crit[:2048], "bf16").reshape(2048, -1)
    np.testing.assert_allclose(O.key_norms(w.k_crit[:2048], "bf16"), np.linalg.norm(rows, axis=1), rtol=1e-13)
    # a per-head norm would differ from it on these rows
    assert not np.allclose(np.linalg.norm(O.to_f64(w.k_crit[:2048], "bf16")[:, 0, :], axis=1),
                           O.key_norms(w.k_crit[:2048], "bf16"), rtol=1e-3)


def test_anchors_pick_outliers_and_ignore_rotation():
    w = make_workload(1)
    norms = O.key_norms(w.k_crit, "bf16")
    for c, (src, T, _d, _o) in enumerate(w.chunks[0].tolist()[:2]):
        out = np.flatnonzero(w.outlier_rows[src:src + T])
        anchors = O.extract_anchors(w.k_crit, w.chunks[0][c:c + 1], 4, "bf16")[0]
        if len(out) >= 4:
            assert set(anchors.tolist()) <= set(out.tolist())
            best = sorted(out.tolist(), key=lambda t: -norms[src + t])[:4]
            assert sorted(best) == sorted(anchors.tolist())
    # rotating every key by an arbitrary angle set keeps norms (rotation is orthogonal)
    kc = O.to_f64(w.k_crit[:1024], "bf16")
    np.testing.assert_allclose(np.linalg.norm(O.rope(kc, 777, 10000.0).reshape(1024, -1), axis=1),
                               np.linalg.norm(kc.reshape(1024, -1), axis=1), rtol=1e-13)


# ----------------------------------------------------------------------------- scoring

def test_scores_closed_form_two_dims():
    # d = 2, one head, one query row, two context chunks of one token each.
    # q_stored = (1, 0) at position L_ctx = 2; key j stored as (cos a_j, sin a_j) cached at orig 0,
    # moved to row j (delta_j = j). Logit_j = cos((2 - j) - a_j) / sqrt(2); s = softmax.
    a = [0.3, -1.1]
    k = np.array([[[math.cos(a[0]), math.sin(a[0])]], [[math.cos(a[1]), math.sin(a[1])]]], dtype=np.float32)
    k64 = k.astype(np.float64)
    q = np.array([[[1.0, 0.0]]], dtype=np.float32)
    chunks = np.array([[0, 1, 0, 0], [1, 1, 1, 0]], dtype=np.int32)
    s = O.critical_scores(q, k, chunks, 1, "f32", 10000.0)
    ang = [math.atan2(k64[j, 0, 1], k64[j, 0, 0]) for j in range(2)]
    nk = [math.hypot(k64[j, 0, 0], k64[j, 0, 1]) for j in range(2)]
    x = [nk[j] * math.cos((2 - j) - ang[j]) / math.sqrt(2) for j in range(2)]
    e = [math.exp(v) for v in x]
    np.testing.assert_allclose(s, [e[0] / sum(e), e[1] / sum(e)], rtol=1e-13)


def test_scores_sum_to_query_rows_times_heads():
    for idx in [0]:
        w = make_workload(idx)
        s = O.critical_scores(w.q_crit[0], w.k_crit, w.chunks[0], w.cfg.n_kv_heads, w.cfg.dtype, w.cfg.rope_base)
        assert math.isclose(s.sum(), w.cfg.query_len * w.cfg.n_q_heads, rel_tol=1e-12)
        assert (s > 0).all()


def test_zero_query_gives_uniform_scores_and_first_indices():
    w = make_custom(dtype="bf16", chunk_lens=(10, 6), query_len=3, n_q_heads=4, n_kv_heads=2, head_dim=64)
    q0 = np.zeros_like(w.q_crit[0])
    s = O.critical_scores(q0, w.k_crit, w.chunks[0], 2, "bf16", 10000.0)
    np.testing.assert_allclose(s, 3 * 4 / 16, rtol=1e-14)
    np.testing.assert_array_equal(O.select_topn(s, 5), [0, 1, 2, 3, 4])


def test_select_topn_signed_zeros_are_equal_scores():
    # -0 and +0 compare equal, so among zero scores the lower index wins whatever the sign
    np.testing.assert_array_equal(O.select_topn([0.0, -0.0, 1.0, -0.0], 2), [0, 2])
    np.testing.assert_array_equal(O.select_topn([-0.0, 0.0, 1.0, 0.0], 3), [0, 1, 2])
    np.testing.assert_array_equal(O.select_topn([-1.0, 0.0, -0.0, 2.0], 3), [1, 2, 3])


def test_scores_use_group_kv_head():
    # Zeroing KV head 1 makes every Q head of group 1 uniform over the context; group 0 is untouched.
    w = make_custom(dtype="f32", chunk_lens=(12,), query_len=2, n_q_heads=4, n_kv_heads=2, head_dim=8)
    k = w.k_crit.copy()
    k[:, 1, :] = 0
    s = O.critical_scores(w.q_crit[0], k, w.chunks[0], 2, "f32", 10000.0)
    q_only_g0 = w.q_crit[0].copy()
    q_only_g0[:, 2:, :] = 0    # heads 2,3 (group 1) zero: their softmax is uniform anyway
    s0 = O.critical_scores(q_only_g0, k, w.chunks[0], 2, "f32", 10000.0)
    np.testing.assert_allclose(s, s0, rtol=1e-13)


def test_scores_invariant_to_cached_orig_pos():
    w = make_custom(dtype="f32", chunk_lens=(9, 7), query_len=3, head_dim=16)
    P = [40, -17]
    kc = w.k_crit.astype(np.float64).copy()
    ch = w.chunks[0].copy()
    for c, (src, T, _d, _o) in enumerate(ch.tolist()):
        kc[src:src + T] = O.rope(kc[src:src + T], P[c], 10000.0)
        ch[c, 3] = P[c]
    s_a = O.critical_scores(w.q_crit[0], w.k_crit, w.chunks[0], 2, "f32", 10000.0)
    s_b = O.critical_scores(w.q_crit[0], kc.astype(np.float32), ch, 2, "f32", 10000.0)
    np.testing.assert_allclose(s_a, s_b, rtol=1e-5)


# ----------------------------------------------------------------------------- selection

def test_select_count_exact_ceil_golden():
    with open(os.path.join(GOLDEN, "select_counts.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert O.select_count(c["num"], c["den"], c["L_ctx"]) == c["N"], c


@given(st.integers(0, 200), st.integers(1, 200), st.integers(0, 40000))
@settings(max_examples=300, deadline=None)
def test_select_count_matches_fraction_ceiling(num, den, L):
    assert O.select_count(num, den, L) == math.ceil(Fraction(num * L, den))


@given(st.lists(st.integers(0, 6), min_size=1, max_size=60), st.data())
@settings(max_examples=200, deadline=None)
def test_topn_matches_stable_argsort_with_ties(vals, data):
    s = np.asarray(vals, dtype=np.float64) / 7.0
    N = data.draw(st.integers(0, len(s)))
    ref = np.sort(np.argsort(-s, kind="stable")[:N])
    np.testing.assert_array_equal(O.select_topn(s, N), ref)


def test_topn_quota_brute_force():
    rng = np.random.default_rng(5)
    chunks = np.array([[0, 5, 0, 0], [5, 3, 5, 0], [8, 6, 8, 0]], dtype=np.int32)
    s = rng.integers(0, 4, 14).astype(np.float64)
    quotas = [2, 0, 6]
    got = O.select_topn_quota(s, chunks, quotas)
    ref = []
    for (src, T, n, _o), qc in zip(chunks.tolist(), quotas):
        idx = list(range(n, n + T))
        idx.sort(key=lambda j: (-s[j], j))
        ref += sorted(idx[:qc])
    np.testing.assert_array_equal(got, ref)
    assert len(got) == sum(quotas)


def test_taper_selections_nest():
    rng = np.random.default_rng(6)
    s = rng.random(17920)
    s[::7] = s[3]   # plenty of ties
    prev = None
    for l in range(8):
        N = O.select_count(14 - l, 70, 17920)
        sel = set(O.select_topn(s, N).tolist())
        assert len(sel) == N
        if prev is not None:
            assert sel <= prev
        prev = sel


# ----------------------------------------------------------------------------- scatter

def test_scatter_writes_exactly_the_rows():
    w = make_custom(dtype="bf16", chunk_lens=(7, 5), query_len=3)
    lay = w.layer(0)
    kf, vf = O.fuse_rerotate(lay["k_store"], lay["v_store"], w.chunks[0], 15, "bf16", 10000.0)
    rp = np.array([1, 4, 11, 12, 13, 14])
    kf2, vf2 = O.scatter_kv(kf, vf, lay["k_new"][0][rp], lay["v_new"][0][rp], rp, "bf16", 10000.0)
    untouched = [j for j in range(12) if j not in rp]
    np.testing.assert_array_equal(kf2[untouched], kf[untouched])
    np.testing.assert_array_equal(vf2[untouched], vf[untouched])
    np.testing.assert_array_equal(vf2[rp], O.to_f64(lay["v_new"][0][rp], "bf16"))
    ref = O.bf16_round(rope_complex(O.to_f64(lay["k_new"][0][rp], "bf16"), rp[:, None], 10000.0))
    np.testing.assert_allclose(kf2[rp], ref, rtol=2 ** -7, atol=0)


# ----------------------------------------------------------------------------- attention and the fused layer

def _fresh_full(w):
    lay = w.layer(0)
    return lay["q_new"][0], lay["k_new"][0], lay["v_new"][0]


def test_full_selection_equals_causal_prefill_f32():
    w = make_custom(dtype="f32", chunk_lens=(11, 9, 6), orig_pos=(0, 3, 50), query_len=5,
                    n_q_heads=6, n_kv_heads=2, head_dim=16)
    lay = w.layer(0)
    L_ctx, L = 26, 31
    qn, kn, vn = _fresh_full(w)
    r = O.fused_layer(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=L,
                      q_new=qn, k_new=kn, v_new=vn, dtype="f32", base=10000.0, n_kv_heads=2,
                      q_crit=w.q_crit[0], k_crit_store=w.k_crit, n_select=L_ctx)
    np.testing.assert_array_equal(r["row_pos"], np.arange(L))
    pos = np.arange(L)[:, None]
    q = rope_complex(qn.astype(np.float64), pos, 10000.0)
    k = store_round_torch(rope_complex(kn.astype(np.float64), pos, 10000.0), "f32")
    ref = sdpa_causal(q, k, vn.astype(np.float64))
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-9)


def test_full_selection_equals_causal_prefill_bf16():
    w = make_custom(dtype="bf16", chunk_lens=(16, 16), query_len=4, n_q_heads=4, n_kv_heads=1, head_dim=32)
    lay = w.layer(0)
    qn, kn, vn = _fresh_full(w)
    r = O.fused_layer(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=36,
                      q_new=qn, k_new=kn, v_new=vn, dtype="bf16", base=10000.0, n_kv_heads=1,
                      q_crit=w.q_crit[0], k_crit_store=w.k_crit, n_select=32)
    pos = np.arange(36)[:, None]
    q = rope_complex(O.to_f64(qn, "bf16"), pos, 10000.0)
    k = torch.from_numpy(rope_complex(O.to_f64(kn, "bf16"), pos, 10000.0)).to(torch.bfloat16).double().numpy()
    ref = sdpa_causal(q, k, O.to_f64(vn, "bf16"))
    # torch rounds through float32 on the way to bfloat16; a rare double rounding moves one key by 1 ulp
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=2e-3)
    assert np.mean(np.abs(r["out"] - ref)) < 1e-6


def test_zero_selection_prefix_case():
    # One chunk at its own position (delta 0), nothing selected: the query rows attend to the cached
    # chunk and to themselves exactly as a prefix-cached prefill would.
    w = make_custom(dtype="f32", chunk_lens=(20,), query_len=6, n_q_heads=4, n_kv_heads=2, head_dim=16)
    lay = w.layer(0)
    qn, kn, vn = _fresh_full(w)
    r = O.fused_layer(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=26,
                      q_new=qn, k_new=kn, v_new=vn, dtype="f32", base=10000.0, n_kv_heads=2,
                      q_crit=w.q_crit[0], k_crit_store=w.k_crit, n_select=0)
    np.testing.assert_array_equal(r["row_pos"], np.arange(20, 26))
    np.testing.assert_array_equal(r["k_fused"][:20], lay["k_store"][:20].astype(np.float64))
    pos = np.arange(26)[:, None]
    k_all = np.concatenate([lay["k_store"][:20].astype(np.float64),
                            store_round_torch(rope_complex(kn[20:].astype(np.float64), pos[20:], 10000.0), "f32")])
    v_all = np.concatenate([lay["v_store"][:20], vn[20:]]).astype(np.float64)
    q_all = rope_complex(qn.astype(np.float64), pos, 10000.0)
    ref = sdpa_causal(q_all, k_all, v_all)[20:]
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-9)


def test_sparse_rows_equal_dense_rows_and_are_convex():
    w = make_custom(dtype="bf16", chunk_lens=(13, 8, 11), orig_pos=(5, 0, 2), query_len=4,
                    n_q_heads=8, n_kv_heads=2, head_dim=32)
    lay = w.layer(0)
    qn, kn, vn = _fresh_full(w)
    r = O.fused_layer(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=36,
                      q_new=qn, k_new=kn, v_new=vn, dtype="bf16", base=10000.0, n_kv_heads=2,
                      q_crit=w.q_crit[0], k_crit_store=w.k_crit, n_select=9)
    rp = r["row_pos"]
    pos = np.arange(36)[:, None]
    q_all = rope_complex(O.to_f64(qn, "bf16"), pos, 10000.0)
    dense = sdpa_causal(q_all, r["k_fused"], r["v_fused"])
    np.testing.assert_allclose(r["out"], dense[rp], rtol=0, atol=1e-12)
    for i, p in enumerate(rp):
        vis = r["v_fused"][:p + 1]                  # [p+1, Hkv, d]
        for h in range(8):
            lo, hi = vis[:, h // 4].min(axis=0), vis[:, h // 4].max(axis=0)
            assert np.all(r["out"][i, h] >= lo - 1e-12) and np.all(r["out"][i, h] <= hi + 1e-12)
    # LSE: logsumexp of the visible logits, recomputed with torch
    i, h = 3, 5
    p = int(rp[i])
    logits = torch.from_numpy(r["k_fused"][:p + 1, h // 4] @ q_all[p, h] / math.sqrt(32))
    assert math.isclose(float(torch.logsumexp(logits, 0)), r["lse"][i, h], rel_tol=1e-12)


def test_golden_tiny_fingerprint():
    """Regression anchor: the tiny workload's selection and output digest, written by
    tests/golden/make_golden.py (which calls only the oracle)."""
    with open(os.path.join(GOLDEN, "tiny_f32_fingerprint.json")) as f:
        g = json.load(f)
    w = make_workload(0)
    lay = w.layer(0)
    c = w.cfg
    r = O.fused_layer(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=c.total_len,
                      q_new=lay["q_new"][0], k_new=lay["k_new"][0], v_new=lay["v_new"][0], dtype="f32",
                      base=c.rope_base, n_kv_heads=c.n_kv_heads, q_crit=w.q_crit[0], k_crit_store=w.k_crit,
                      n_select=O.select_count(15, 100, c.ctx_len))
    assert r["row_pos"].tolist() == g["row_pos"]
    assert O.extract_anchors(w.k_crit, w.chunks[0], 4, "f32").tolist() == g["anchors"]
    np.testing.assert_allclose(r["scores"][:8], g["scores_head"], rtol=1e-12)
    np.testing.assert_allclose(float(np.sum(r["out"])), g["out_sum"], rtol=1e-10)
