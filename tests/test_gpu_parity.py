"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Small workloads compare every output; the full-size workloads compare every score, the selection,
every fused K/V row, and the attention output of sampled rows (the oracle evaluates rows one by
one). Tolerances are those stated in tests/gpu_helpers.py.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
import selective_recompute_attention_amd as sra
from workloads import make_custom, make_workload

from gpu_helpers import (assert_out_close, assert_scores_close, assert_storage_close, bits, check_selection,
                         decode, dev, empty, host, run_fused, sample_rows, say, shape_of, workspace)

pytestmark = pytest.mark.gpu


def oracle_compare(w, res, layer=0, rows=None, quotas=None, check_scores=True):
    """Compare one run_fused result with the oracle for every request of the workload."""
    cfg, dt, base = w.cfg, w.cfg.dtype, w.cfg.rope_base
    lay = w.layer(layer)
    Lctx, L, N, R = res["Lctx"], res["L"], res["N"], res["R"]
    Lq = L - Lctx
    stats = {}
    for q in range(w.chunks.shape[0]):
        rp = res["row_pos"][q].astype(np.int64)
        np.testing.assert_array_equal(rp[N:], Lctx + np.arange(Lq))
        if check_scores and "scores" in res:
            s_ref = O.critical_scores(w.q_crit[q], w.k_crit, w.chunks[q], cfg.n_kv_heads, dt, base)
            stats["score_rel"] = max(stats.get("score_rel", 0.0), assert_scores_close(res["scores"][q], s_ref))
            if quotas is None:
                stats["swaps"] = stats.get("swaps", 0) + check_selection(rp[:N], s_ref, N)
            else:
                off = 0
                for c, (src, T, n, _o) in enumerate(w.chunks[q].tolist()):
                    qc = int(quotas[q][c])
                    part = rp[off:off + qc]
                    assert np.all((part >= n) & (part < n + T)), f"chunk {c}: selection leaves the chunk"
                    check_selection(part, s_ref[n:n + T], qc, offset=n)
                    off += qc
        kf, vf = O.fuse_rerotate(lay["k_store"], lay["v_store"], w.chunks[q], L, dt, base)
        kf, vf = O.scatter_kv(kf, vf, lay["k_new"][q][rp], lay["v_new"][q][rp], rp, dt, base)
        # V everywhere and K of unmoved chunks' untouched rows: bit-exact
        np.testing.assert_array_equal(bits(res["v_fused"][q], dt), O.storage_bits(vf, dt))
        still = np.ones(L, bool)
        still[rp] = False
        for (src, T, n, orig) in w.chunks[q].tolist():
            if n - orig != 0:
                still[n:n + T] = False
        still[Lctx:] = False
        np.testing.assert_array_equal(bits(res["k_fused"][q], dt)[still], O.storage_bits(kf[still], dt))
        assert_storage_close(decode(res["k_fused"][q], dt), kf, dt, f"fused K (request {q})")
        sel_rows = list(range(R)) if rows is None else (rows(q) if callable(rows) else rows)
        o_ref, lse_ref = O.sparse_causal_attn(lay["q_new"][q][rp], rp, kf, vf, dt, base, rows=sel_rows)
        o_gpu = decode(res["out"][q][sel_rows], dt)
        mx, mean = assert_out_close(o_gpu, o_ref, dt)
        stats["out_max"] = max(stats.get("out_max", 0.0), mx)
        stats["rows"] = stats.get("rows", 0) + len(sel_rows)
        if dt == "bf16":   # values past the plain 1.5e-2 (allowed only where |O| >= 4, see assert_out_close)
            stats["over_1.5e-2"] = stats.get("over_1.5e-2", 0) + int((np.abs(o_gpu - o_ref) > 1.5e-2).sum())
        lse_tol = 2e-2 if dt == "bf16" else 1e-4
        np.testing.assert_allclose(res["lse"][q][sel_rows], lse_ref, rtol=0, atol=lse_tol)
    say(f"    parity stats: {stats}")
    return stats


# ------------------------------------------------------------------------------ named workloads

def test_tiny_f32_fused_all_rows():
    w = make_workload(0)
    N = O.select_count(15, 100, w.cfg.ctx_len)
    say(f"case tiny_f32 fused N={N}")
    res = run_fused(w, n_select=N)
    oracle_compare(w, res)


def test_mistral_fused_all_rows():
    w = make_workload(1)
    N = O.select_count(15, 100, w.cfg.ctx_len)
    say(f"case mistral7b_layer fused N={N}")
    res = run_fused(w, n_select=N)
    oracle_compare(w, res)


def wide_rows(res, dtype, Lq, k, top, seed=0):
    """Rows of request q to check at full size: a seeded spread (sample_rows), every query row, and the
    `top` rows with the largest GPU |O| (where the output's own bf16 rounding is coarsest)."""
    def pick(q):
        R = res["R"]
        big = np.abs(decode(res["out"][q], dtype)).reshape(R, -1).max(axis=1)
        rows = set(sample_rows(R, Lq, k, seed=seed + q)) | set(range(R - Lq, R))
        rows |= set(np.argsort(-big, kind="stable")[:top].tolist())
        return sorted(rows)
    return pick


def test_yi_batch_of_four_sampled_rows():
    w = make_workload(2)
    N = O.select_count(10, 100, w.cfg.ctx_len)
    say(f"case yi34b_layer_x4req fused N={N}")
    res = run_fused(w, n_select=N)
    oracle_compare(w, res, rows=wide_rows(res, "bf16", w.cfg.query_len, 96, 16))


def test_llama70b_tapered_layers():
    w = make_workload(3)
    Lctx, Lq = w.cfg.ctx_len, w.cfg.query_len
    N0 = O.select_count(14, 70, Lctx)
    say(f"case llama70b_8layers layer 0 (scoring) N={N0}")
    res0 = run_fused(w, 0, n_select=N0)
    oracle_compare(w, res0, 0, rows=wide_rows(res0, "bf16", Lq, 128, 16))
    scores = torch.from_numpy(res0["scores"]).cuda()
    prev = set(res0["row_pos"][0][:N0].tolist())
    for l in (5, 7):
        a, b = w.cfg.select[1][l]
        Nl = O.select_count(a, b, Lctx)
        say(f"case llama70b_8layers layer {l} N={Nl}")
        rp = torch.empty((1, Nl + Lq), dtype=torch.int32, device="cuda")
        sra.select_topn(scores, Nl, None, None, Lq, rp)
        torch.cuda.synchronize()
        rp_h = rp.cpu().numpy()
        np.testing.assert_array_equal(rp_h[0][:Nl], O.select_topn(res0["scores"][0], Nl))  # same fp32 scores
        cur = set(rp_h[0][:Nl].tolist())
        assert cur <= prev, "tapered selections must nest"
        prev = cur
        res = run_fused(w, l, score=False, row_pos_in=rp_h)
        # at least 256 spread rows, every query row and the 32 rows of largest |O|
        oracle_compare(w, res, l, rows=wide_rows(res, "bf16", Lq, 256, 32, seed=l), check_scores=False)


def test_llama7b_per_chunk_quotas():
    w = make_workload(4)
    say(f"case llama7b_mha_quota fused N={int(w.quotas.sum())}")
    res = run_fused(w, quotas=w.quotas)
    oracle_compare(w, res, rows=wide_rows(res, "bf16", w.cfg.query_len, 48, 16), quotas=w.quotas)


# ------------------------------------------------------------------------------ edge cases

EDGE = [
    # (id, make_custom kwargs, selection)
    ("bf16_ragged_orig", dict(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=(37, 100, 5, 64),
                              orig_pos=(3, 0, 999, -20), query_len=7), ("pct", 30)),
    ("bf16_d64_gqa7", dict(dtype="bf16", n_q_heads=14, n_kv_heads=2, head_dim=64, chunk_lens=(130, 129),
                           orig_pos=(0, 5), query_len=5), ("pct", 20)),
    ("bf16_mha_two_req", dict(dtype="bf16", n_q_heads=4, n_kv_heads=4, head_dim=128, chunk_lens=(64, 200),
                              query_len=3, n_req=2), ("pct", 11)),
    ("bf16_zero_select", dict(dtype="bf16", n_q_heads=8, n_kv_heads=8, head_dim=128, chunk_lens=(96,),
                              query_len=16), ("pct", 0)),
    ("bf16_full_select", dict(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=64, chunk_lens=(50, 45),
                              orig_pos=(10, 0), query_len=9), ("pct", 100)),
    ("bf16_long_split", dict(dtype="bf16", n_q_heads=16, n_kv_heads=4, head_dim=128, chunk_lens=(700, 1333),
                             orig_pos=(0, 7), query_len=12), ("pct", 5)),
    ("bf16_quota_ragged", dict(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=(33, 64, 1, 90),
                               query_len=4), ("quota", 0.6)),
    ("bf16_single_query_row", dict(dtype="bf16", n_q_heads=2, n_kv_heads=1, head_dim=128, chunk_lens=(17,),
                                   query_len=1), ("pct", 50)),
    # re-rotation inside scoring pass 1: KV-head shares of 86 rows (256 / 3 rounded up), spans cut by
    # the chunk's end, a one-token chunk, and five heads with a chunk just past one span
    ("bf16_hkv3_s1_shares", dict(dtype="bf16", n_q_heads=6, n_kv_heads=3, head_dim=64, chunk_lens=(300, 129, 1),
                                 orig_pos=(5, 0, 200), query_len=4), ("pct", 12)),
    ("bf16_hkv5_s1_span", dict(dtype="bf16", n_q_heads=10, n_kv_heads=5, head_dim=128, chunk_lens=(257, 40),
                               orig_pos=(0, 3), query_len=6), ("pct", 25)),
    ("f32_ragged", dict(dtype="f32", n_q_heads=6, n_kv_heads=3, head_dim=64, chunk_lens=(31, 7, 66),
                        orig_pos=(0, 2, 40), query_len=6), ("pct", 20)),
    ("f32_d128_quota", dict(dtype="f32", n_q_heads=4, n_kv_heads=1, head_dim=128, chunk_lens=(40, 40),
                            query_len=3), ("quota", 0.5)),
]


@pytest.mark.parametrize("name,kw,sel", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, kw, sel):
    seed = zlib.crc32(name.encode()) % 1000   # fixed per case (str hashes change between processes)
    w = make_custom(select=sel, seed=seed, **kw)
    Lctx = int(w.chunks[0, :, 1].sum())
    say(f"case edge {name} seed={seed}")
    if sel[0] == "quota":
        res = run_fused(w, quotas=w.quotas)
        oracle_compare(w, res, quotas=w.quotas)
    else:
        N = O.select_count(sel[1], 100, Lctx)
        res = run_fused(w, n_select=N)
        oracle_compare(w, res)


# ------------------------------------------------------------------------------ standalone entry points

def _custom_inputs(dtype="bf16"):
    return make_custom(dtype=dtype, n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=(90, 70, 33),
                       orig_pos=(4, 0, 11), query_len=6, n_req=2, seed=77)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_standalone_stages_match_oracle(dtype):
    w = _custom_inputs(dtype)
    cfg, dt, base = w.cfg, dtype, w.cfg.rope_base
    lay = w.layer(0)
    n_req, n_chunks = w.chunks.shape[:2]
    Lctx, Lq = 193, 6
    L = Lctx + Lq
    N = O.select_count(25, 100, Lctx)
    R = N + Lq
    shape = shape_of(cfg)
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    say(f"case standalone stages {dtype}")
    ks, vs = dev(lay["k_store"], dt), dev(lay["v_store"], dt)
    kf, vf = empty((n_req, L, Hkv, D), dt, 0x7F01), empty((n_req, L, Hkv, D), dt, 0x7F01)
    sra.fuse_rerotate(shape, ks, vs, w.chunks, kf, vf)
    # scoring + selection
    ws = workspace(shape, n_req, n_chunks, L, R, Lq)
    scores = torch.empty((n_req, Lctx), dtype=torch.float32, device="cuda")
    rp = torch.empty((n_req, R), dtype=torch.int32, device="cuda")
    sra.score_select(shape, dev(w.q_crit, dt), dev(w.k_crit, dt), w.chunks, N, None, scores, rp, ws)
    # selection alone on the same scores must give the same rows
    rp2 = torch.empty_like(rp)
    sra.select_topn(scores, N, None, None, Lq, rp2)
    torch.cuda.synchronize()
    assert sra.check_rows(rp, L) == -1
    np.testing.assert_array_equal(rp.cpu().numpy(), rp2.cpu().numpy())
    rp_h = rp.cpu().numpy().astype(np.int64)
    sc_h = scores.cpu().numpy()
    # scatter of compact rows, then attention of compact rows
    kn = dev(np.stack([lay["k_new"][q][rp_h[q]] for q in range(n_req)]), dt)
    vn = dev(np.stack([lay["v_new"][q][rp_h[q]] for q in range(n_req)]), dt)
    qn = dev(np.stack([lay["q_new"][q][rp_h[q]] for q in range(n_req)]), dt)
    sra.scatter_kv(shape, kn, vn, rp, kf, vf)
    out = empty((n_req, R, Hq, D), dt)
    lse = torch.empty((n_req, R, Hq), dtype=torch.float32, device="cuda")
    ws2 = workspace(shape, n_req, 1, L, R, 1)
    sra.sparse_causal_attn(shape, qn, rp, kf, vf, out, lse, ws2)
    torch.cuda.synchronize()
    res = {"k_fused": host(kf), "v_fused": host(vf), "out": host(out), "lse": lse.cpu().numpy(),
           "row_pos": rp_h.astype(np.int32), "N": N, "R": R, "L": L, "Lctx": Lctx, "scores": sc_h}
    oracle_compare(w, res)
    # the fused entry produces the same bits as the stage-by-stage calls
    resf = run_fused(w, n_select=N)
    for k in ("k_fused", "v_fused", "out", "row_pos"):
        np.testing.assert_array_equal(resf[k], res[k], err_msg=k)
    np.testing.assert_array_equal(resf["scores"], sc_h)


def test_select_topn_bit_exact_on_given_scores():
    # Ties everywhere: integer-valued float scores; the GPU decision must equal the stable sort exactly.
    rng = np.random.default_rng(11)
    for Lctx, N in [(1, 1), (7, 3), (1000, 0), (1000, 1000), (4097, 1234), (32768, 5767)]:
        s = rng.integers(0, 50, size=(3, Lctx)).astype(np.float32) / 8
        st = torch.from_numpy(s).cuda()
        rp = torch.empty((3, N + 2), dtype=torch.int32, device="cuda")
        say(f"case select_topn L={Lctx} N={N}")
        sra.select_topn(st, N, None, None, 2, rp)
        torch.cuda.synchronize()
        got = rp.cpu().numpy()
        for q in range(3):
            np.testing.assert_array_equal(got[q][:N], O.select_topn(s[q], N))
            np.testing.assert_array_equal(got[q][N:], [Lctx, Lctx + 1])


def test_select_topn_quotas_bit_exact():
    rng = np.random.default_rng(12)
    lens = [512, 3, 200, 1, 77]
    chunks = np.array([[[0, 0, 0, 0]] * len(lens)], dtype=np.int32)
    n = 0
    for c, T in enumerate(lens):
        chunks[0, c] = (n, T, n, 0)
        n += T
    quotas = np.array([[100, 3, 0, 1, 40]], dtype=np.int32)
    s = rng.integers(0, 9, size=(1, n)).astype(np.float32)
    rp = torch.empty((1, int(quotas.sum()) + 4), dtype=torch.int32, device="cuda")
    sra.select_topn(torch.from_numpy(s).cuda(), None, quotas, chunks, 4, rp)
    torch.cuda.synchronize()
    ref = O.select_topn_quota(s[0], chunks[0], quotas[0])
    np.testing.assert_array_equal(rp.cpu().numpy()[0][:len(ref)], ref)


@pytest.mark.parametrize("idx", [0, 1])
def test_anchors_match_oracle(idx):
    w = make_workload(idx)
    cfg = w.cfg
    shape = shape_of(cfg)
    ch = w.chunks[0]
    k = cfg.anchors_k
    say(f"case anchors config {idx}")
    anchors = torch.empty((len(ch), k), dtype=torch.int32, device="cuda")
    norms = torch.zeros((w.store_rows,), dtype=torch.float32, device="cuda")
    ws = torch.empty(sra.anchor_workspace_size(ch), dtype=torch.uint8, device="cuda")
    sra.extract_anchors(shape, dev(w.k_crit, cfg.dtype), ch, k, anchors, ws, norms)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(anchors.cpu().numpy(), O.extract_anchors(w.k_crit, ch, k, cfg.dtype))
    np.testing.assert_allclose(norms.cpu().numpy(), O.key_norms(w.k_crit, cfg.dtype), rtol=1e-6)
    if w.outlier_rows is not None:
        for c, (src, T, _d, _o) in enumerate(ch.tolist()):
            outl = np.flatnonzero(w.outlier_rows[src:src + T])
            if len(outl) >= k:
                assert set(anchors.cpu().numpy()[c].tolist()) <= set(outl.tolist())



FUSED_ANCHOR_CASES = {
    # name: (workload builder, anchors k)
    "mistral7b_layer": (lambda: make_workload(1), 4),                       # bf16: in the scoring passes
    "tiny_f32": (lambda: make_workload(0), 4),                              # float32: standalone kernels
    "two_requests_ragged_bf16": (lambda: make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128,
                                                     chunk_lens=(200, 37, 301), orig_pos=(0, 5, 0), query_len=7,
                                                     n_req=2, seed=11), 6),
    # chunks past 512 tokens: the selection rounds read the totals from LDS instead of registers
    "chunks_past_register_bf16": (lambda: make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=4, head_dim=64,
                                                      chunk_lens=(1000, 513, 64), orig_pos=(0, 0, 9), query_len=4,
                                                      seed=13), 7),
    "chunk_longer_than_lds_bf16": (lambda: make_custom(dtype="bf16", n_q_heads=2, n_kv_heads=1, head_dim=64,
                                                       chunk_lens=(4500, 100), query_len=3, seed=12), 5),
}


@pytest.mark.parametrize("name", list(FUSED_ANCHOR_CASES))
def test_fused_anchors_match_standalone_and_oracle(name):
    build, k = FUSED_ANCHOR_CASES[name]
    w = build()
    cfg = w.cfg
    shape = shape_of(cfg)
    n_req, n_chunks = w.chunks.shape[0], w.chunks.shape[1]
    lay = w.layer(0)
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = cfg.query_len
    L = Lctx + Lq
    N = sra.select_count(15, 100, Lctx)
    R = N + Lq
    dt = cfg.dtype
    say(f"case fused anchors {name}: n_req {n_req}, chunks {n_chunks}, k {k}")
    t = {kk: dev(v, dt) for kk, v in lay.items()}
    kc = dev(w.k_crit, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    kf = torch.empty((n_req, L, cfg.n_kv_heads, cfg.head_dim), dtype=tdt, device="cuda")
    vf = torch.empty_like(kf)
    out = torch.empty((n_req, R, cfg.n_q_heads, cfg.head_dim), dtype=tdt, device="cuda")
    rp = torch.empty((n_req, R), dtype=torch.int32, device="cuda")
    anchors = torch.full((n_req, n_chunks, k), -7, dtype=torch.int32, device="cuda")
    norms = torch.zeros((w.k_crit.shape[0],), dtype=torch.float32, device="cuda")
    ws = torch.empty(sra.workspace_size(shape, n_req, n_chunks, L, R, Lq), dtype=torch.uint8, device="cuda")
    sra.fused_layer(shape, chunks=w.chunks, k_store=t["k_store"], v_store=t["v_store"], q_fresh=t["q_new"],
                    k_fresh=t["k_new"], v_fresh=t["v_new"], row_pos=rp, k_fused=kf, v_fused=vf, out=out, ws=ws,
                    q_crit=dev(w.q_crit, dt), k_crit_store=kc, n_select=N, anchors_k=k, anchor_rows=anchors,
                    anchor_norms=norms)
    torch.cuda.synchronize()
    got = anchors.cpu().numpy()
    for q in range(n_req):
        ch = w.chunks[q]
        a1 = torch.empty((n_chunks, k), dtype=torch.int32, device="cuda")
        n1 = torch.zeros_like(norms)
        aws = torch.empty(sra.anchor_workspace_size(ch), dtype=torch.uint8, device="cuda")
        sra.extract_anchors(shape, kc, ch, k, a1, aws, n1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got[q], a1.cpu().numpy())           # same bits as the standalone call
        np.testing.assert_array_equal(got[q], O.extract_anchors(w.k_crit, ch, k, dt))
        rows = np.concatenate([np.arange(s0, s0 + T) for s0, T, _d, _o in ch.tolist()])
        np.testing.assert_array_equal(norms.cpu().numpy()[rows], n1.cpu().numpy()[rows])
    np.testing.assert_allclose(norms.cpu().numpy()[rows], O.key_norms(w.k_crit, dt)[rows], rtol=1e-6)


# ------------------------------------------------------------------------------ invariants on the GPU

def test_zero_selection_zero_delta_keeps_cache_bits():
    w = make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=(64, 48),
                    orig_pos=(0, 64), query_len=5, select=("pct", 0))
    say("case V2 zero selection, zero delta")
    res = run_fused(w, n_select=0)
    lay = w.layer(0)
    np.testing.assert_array_equal(res["k_fused"][0][:112], lay["k_store"][:112])
    np.testing.assert_array_equal(res["v_fused"][0][:112], lay["v_store"][:112])
    oracle_compare(w, res)


def test_double_rotation_equals_single():
    w = make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=(128,), query_len=1)
    lay = w.layer(0)
    shape = shape_of(w.cfg)
    say("case V3 double rotation")
    ks, vs = dev(lay["k_store"], "bf16"), dev(lay["v_store"], "bf16")
    a_k, a_v = empty((1, 129, 2, 128), "bf16"), empty((1, 129, 2, 128), "bf16")
    b_k, b_v = empty((1, 129, 2, 128), "bf16"), empty((1, 129, 2, 128), "bf16")
    c_k, c_v = empty((1, 129, 2, 128), "bf16"), empty((1, 129, 2, 128), "bf16")
    d1, d2 = 1234, -456
    sra.fuse_rerotate(shape, ks, vs, [[[0, 128, 0, -d1]]], a_k, a_v)               # rotate by d1
    sra.fuse_rerotate(shape, a_k[0], a_v[0], [[[0, 128, 0, -d2]]], b_k, b_v)     # then by d2
    sra.fuse_rerotate(shape, ks, vs, [[[0, 128, 0, -(d1 + d2)]]], c_k, c_v)       # once by d1 + d2
    torch.cuda.synchronize()
    two, one = decode(host(b_k)[0][:128], "bf16"), decode(host(c_k)[0][:128], "bf16")
    from gpu_helpers import bf16_ulp, pair_norm
    # the intermediate rounding moves each pair by at most 0.71 ulp of its norm, the two final
    # roundings by 0.5 ulp each: within 2 ulps of the pair norm
    assert np.all(np.abs(two - one) <= 2 * bf16_ulp(pair_norm(one)) + 1e-30)
    np.testing.assert_array_equal(host(b_v)[0][:128], lay["v_store"][:128])


@pytest.mark.parametrize("wid", [1, 2])
def test_runs_are_deterministic(wid):
    """Mistral-7B layer: static split with merged partial tiles; Yi-34B x 4 requests: whole tiles taken
    from the KV heads' queues, so which work group computes a tile varies from run to run."""
    w = make_workload(wid)
    N = O.select_count(15, 100, w.cfg.ctx_len)
    say(f"case determinism workload {wid}")
    a = run_fused(w, n_select=N)
    b = run_fused(w, n_select=N)
    for k in ("k_fused", "v_fused", "out", "lse", "row_pos", "scores"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_check_rows_reports_bad_rows():
    good = torch.tensor([[0, 3, 9], [1, 2, 9]], dtype=torch.int32, device="cuda")
    assert sra.check_rows(good, 10) == -1
    for bad, idx in [([[0, 3, 3], [1, 2, 9]], 2), ([[0, 3, 9], [1, 2, 10]], 5), ([[-1, 3, 9], [1, 2, 4]], 0),
                     ([[0, 3, 9], [5, 2, 7]], 4)]:
        with pytest.raises(sra.SRAError) as e:
            sra.check_rows(torch.tensor(bad, dtype=torch.int32, device="cuda"), 10)
        assert e.value.status == 7 and f"row_pos[{idx}]" in str(e.value)


# ------------------------------------------------------------------------------ fp16 operand range

def test_fp16_range_fallback_matches_oracle():
    """Keys of magnitude 1e5 have no fp16 value: their (request, KV head) group is recomputed exactly in
    float32, reported as 1 in the fallback array, and the outputs still match the oracle (the other
    group stays on the fp16 path and reports 0)."""
    w = make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=(100, 60), orig_pos=(0, 9),
                    query_len=6, seed=41, select=("pct", 25))
    lay = w.layer(0)
    big = np.array([1e5, -1e5, 1.5e5], dtype=np.float32)
    bits = O.storage_bits(O.bf16_round(big.astype(np.float64)), "bf16")
    # KV head 1 only: two cached keys and one fresh query-row key
    lay["k_store"][10, 1, 3] = bits[0]
    lay["k_store"][130, 1, 70] = bits[1]
    Lctx = int(w.chunks[0, :, 1].sum())
    lay["k_new"][0, Lctx + 2, 1, 5] = bits[2]
    N = O.select_count(25, 100, Lctx)
    say(f"case fp16 range: keys {big.tolist()} on KV head 1, N={N}")
    res = run_fused(w, n_select=N, fallback=True)
    say(f"    fallback report {res['fallback'].tolist()}")
    np.testing.assert_array_equal(res["fallback"], [[0, 1]])
    stats = oracle_compare(w, res)
    say(f"    fallback {res['fallback'].tolist()}, out max {stats['out_max']:.3g}")


def test_fp16_range_fallback_whole_tile_mode():
    """The same exact recomputation where the attention takes whole tiles from per-group queues (four
    requests, 40 tiles per group over 16 work groups, d = 64): one fresh key of magnitude 1e5 on a query
    row of request 2, KV head 1 flags that group alone, and every sampled row still matches the
    oracle."""
    w = make_custom(dtype="bf16", n_q_heads=32, n_kv_heads=8, head_dim=64, chunk_lens=(700, 700),
                    orig_pos=(0, 40), query_len=8, n_req=4, seed=43, select=("pct", 90))
    lay = w.layer(0)
    Lctx = int(w.chunks[0, :, 1].sum())
    big = O.storage_bits(O.bf16_round(np.array([1e5], dtype=np.float64)), "bf16")
    lay["k_new"][2, Lctx + 2, 1, 5] = big[0]
    N = O.select_count(90, 100, Lctx)
    R, g = N + w.cfg.query_len, w.cfg.n_q_heads // w.cfg.n_kv_heads
    tiles, pieces = -(-R * g // 128), 512 // (w.cfg.n_req * w.cfg.n_kv_heads)
    assert 4 * tiles >= 9 * pieces, "the shape must take whole tiles from the queues"
    say(f"case fp16 range, whole tiles: {tiles} tiles per group over {pieces} work groups, N={N}")
    res = run_fused(w, n_select=N, fallback=True)
    want = np.zeros((w.cfg.n_req, w.cfg.n_kv_heads), np.int32)
    want[2, 1] = 1
    np.testing.assert_array_equal(res["fallback"], want)
    stats = oracle_compare(w, res, rows=wide_rows(res, "bf16", w.cfg.query_len, 64, 16))
    say(f"    fallback {res['fallback'].tolist()}, out max {stats['out_max']:.3g}")


def test_fp16_range_query_fallback_standalone():
    """A rotated query whose scaled value reaches fp16's infinity (|q| ~ 6e5) flags its group in the
    standalone attention entry; the group is recomputed exactly and matches the oracle (log-sum-exp
    within 2e-2 + 1e-6 |lse|: float32 logits of magnitude ~1e5 carry ~1e-6 relative error)."""
    w = _custom_inputs("bf16")
    cfg, dt, base = w.cfg, "bf16", w.cfg.rope_base
    lay = w.layer(0)
    n_req = w.chunks.shape[0]
    Lctx, Lq = 193, 6
    L = Lctx + Lq
    shape = shape_of(cfg)
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    rng = np.random.default_rng(3)
    rows = np.stack([O.row_positions(np.sort(rng.choice(Lctx, 40, replace=False)), Lctx, Lq) for _ in range(n_req)])
    R = rows.shape[1]
    kf_ref, vf_ref = [], []
    for q in range(n_req):
        kf, vf = O.fuse_rerotate(lay["k_store"], lay["v_store"], w.chunks[q], L, dt, base)
        kf, vf = O.scatter_kv(kf, vf, lay["k_new"][q][rows[q]], lay["v_new"][q][rows[q]], rows[q], dt, base)
        kf_ref.append(kf)
        vf_ref.append(vf)
    qn = np.stack([lay["q_new"][q][rows[q]] for q in range(n_req)]).copy()
    # request 1, row 7, query head 5 (KV head 1): every element 6e5
    qn[1, 7, 5, :] = O.storage_bits(O.bf16_round(np.full(D, 6e5)), "bf16")
    say("case fp16 range: scaled query beyond 65520 in request 1, KV head 1")
    kd = dev(np.stack([O.storage_bits(k, dt) for k in kf_ref]), dt)
    vd = dev(np.stack([O.storage_bits(v, dt) for v in vf_ref]), dt)
    out = empty((n_req, R, Hq, D), dt)
    lse = torch.empty((n_req, R, Hq), dtype=torch.float32, device="cuda")
    fb = torch.full((n_req, Hkv), -1, dtype=torch.int32, device="cuda")
    ws = workspace(shape, n_req, 1, L, R, 1)
    sra.sparse_causal_attn(shape, dev(qn, dt), torch.from_numpy(rows.astype(np.int32)).cuda(), kd, vd, out, lse, ws,
                           fallback=fb)
    torch.cuda.synchronize()
    say(f"    fallback report {fb.cpu().numpy().tolist()}")
    np.testing.assert_array_equal(fb.cpu().numpy(), [[0, 0], [0, 1]])
    o_h, l_h = host(out), lse.cpu().numpy()
    for q in range(n_req):
        o_ref, l_ref = O.sparse_causal_attn(qn[q], rows[q], kf_ref[q], vf_ref[q], dt, base)
        mx, _ = assert_out_close(decode(o_h[q], dt), o_ref, dt)
        assert np.all(np.abs(l_h[q] - l_ref) <= 2e-2 + 1e-6 * np.abs(l_ref)), "log-sum-exp"
        say(f"    request {q}: out max err {mx:.3g}, largest |lse| {np.abs(l_ref).max():.3g}")
