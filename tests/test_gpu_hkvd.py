"""Gradual filtering on the GPU against the oracle (KVCache reuse 01, §1.3.2-§1.3.4): the KV
deviation of the previous layer's rows and the next layer's rows (sra_hkvd_select), the fused layer
in filtering mode, and a three-layer taper driven by it.

Bars: deviations within 1e-4 relative of the oracle's; kept rows identical to the oracle's except
for swaps among rows whose (float64) deviation lies within 1e-5 relative of the n_keep-th one; query
rows unchanged; outputs of the fused layer as in the parity tests (oracle run on the GPU's rows).
"""
import numpy as np
import pytest
import torch

import oracle as O
import selective_recompute_attention_amd as sra
from workloads import make_custom, make_workload

from gpu_helpers import (assert_out_close, assert_storage_close, check_selection, dev, empty, host,
                         sample_rows, say, shape_of, workspace)

pytestmark = pytest.mark.gpu


def _workload(name):
    if name == "tiny_f32":
        return make_workload(0)
    if name == "mistral7b_layer":
        return make_workload(1)
    if name == "two_requests_bf16":
        return make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=[200, 97, 300],
                           orig_pos=[0, 0, 50], query_len=24, n_req=2, seed=31)
    if name == "d64_bf16":
        return make_custom(dtype="bf16", n_q_heads=6, n_kv_heads=3, head_dim=64, chunk_lens=[70, 45],
                           orig_pos=[10, 0], query_len=5, n_req=1, seed=32)
    raise KeyError(name)


def _prev_rows(w, n_prev, seed):
    """A previous layer's selection per request: seeded ascending context rows, then the query rows."""
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = w.cfg.query_len
    rng = np.random.default_rng(seed)
    rows = [O.row_positions(np.sort(rng.choice(Lctx, n_prev, replace=False)), Lctx, Lq)
            for _ in range(w.chunks.shape[0])]
    return np.asarray(rows, dtype=np.int32).reshape(w.chunks.shape[0], n_prev + Lq)


def _check_kept(rows_gpu, prev, n_prev, n_keep, d_ref, what):
    """Kept rows by the window rule on the oracle's float64 deviations (the device ranks float32
    values: their rounding, 6e-8 relative, stays inside the 1e-5 window); query rows unchanged."""
    assert list(rows_gpu[n_keep:]) == list(prev[n_prev:]), f"{what}: query rows changed"
    idx = np.searchsorted(prev[:n_prev], rows_gpu[:n_keep])
    assert np.all(prev[:n_prev][np.minimum(idx, n_prev - 1)] == rows_gpu[:n_keep]) if n_keep else True, \
        f"{what}: a kept row is not among the previous rows"
    return check_selection(idx, np.asarray(d_ref, dtype=np.float64), n_keep)


HKVD_CASES = [("tiny_f32", 58, 40), ("two_requests_bf16", 120, 77), ("mistral7b_layer", 384, 341),
              ("d64_bf16", 30, 17), ("tiny_f32", 58, 0), ("tiny_f32", 58, 58), ("two_requests_bf16", 0, 0),
              ("tiny_f32", 1, 1)]


@pytest.mark.parametrize("name,n_prev,n_keep", HKVD_CASES)
def test_hkvd_select_matches_oracle(name, n_prev, n_keep):
    w = _workload(name)
    cfg, dt = w.cfg, w.cfg.dtype
    base = cfg.rope_base
    lay = w.layer(0)
    n_req = w.chunks.shape[0]
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = cfg.query_len
    L = Lctx + Lq
    say(f"hkvd_select: {name}, n_req={n_req}, n_prev={n_prev}, n_keep={n_keep}")
    prev = _prev_rows(w, n_prev, seed=7)
    kf_ref, vf_ref = [], []
    for q in range(n_req):
        kf, vf = O.fuse_rerotate(lay["k_store"], lay["v_store"], w.chunks[q], L, dt, base)
        kf[Lctx:] = 0.0   # the query rows are never read here
        vf[Lctx:] = 0.0
        kf_ref.append(kf)
        vf_ref.append(vf)
    up = (lambda x: O.storage_bits(x, dt)) if dt == "bf16" else (lambda x: x.astype(np.float32))
    kf_d = dev(np.stack([up(k) for k in kf_ref]), dt)
    vf_d = dev(np.stack([up(v) for v in vf_ref]), dt)
    kn_c = np.stack([lay["k_new"][q][prev[q]] for q in range(n_req)])   # compact rows of the previous layer
    vn_c = np.stack([lay["v_new"][q][prev[q]] for q in range(n_req)])
    dev_t = torch.full((n_req, max(n_prev, 1)), -1.0, dtype=torch.float32, device="cuda")
    rows_t = torch.full((n_req, n_keep + Lq), -1, dtype=torch.int32, device="cuda")
    sra.hkvd_select(shape_of(cfg), kf_d, vf_d, dev(kn_c, dt), dev(vn_c, dt),
                    torch.from_numpy(prev).cuda(), n_prev, n_keep, dev_t, rows_t)
    torch.cuda.synchronize()
    d_gpu, rows = dev_t.cpu().numpy()[:, :n_prev], rows_t.cpu().numpy()
    for q in range(n_req):
        d_ref = O.kv_deviation(kf_ref[q], vf_ref[q], kn_c[q], vn_c[q], prev[q], n_prev, dt, base)
        if n_prev:
            rel = np.abs(d_gpu[q].astype(np.float64) - d_ref) / np.abs(d_ref)
            assert rel.max() <= 1e-4, f"deviation: max relative error {rel.max():.3g}"
            say(f"  request {q}: deviation max rel err {rel.max():.3g}")
        swaps = _check_kept(rows[q], prev[q], n_prev, n_keep, d_ref, f"request {q}")
        say(f"  request {q}: kept rows ok (window swaps {swaps})")


@pytest.mark.parametrize("name,n_prev,n_keep", [("tiny_f32", 58, 47), ("two_requests_bf16", 120, 90),
                                                ("mistral7b_layer", 384, 341)])
def test_fused_layer_filtering_matches_oracle(name, n_prev, n_keep):
    w = _workload(name)
    cfg, dt = w.cfg, w.cfg.dtype
    base = cfg.rope_base
    lay = w.layer(0)
    n_req, n_chunks = w.chunks.shape[0], w.chunks.shape[1]
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = cfg.query_len
    L, R = Lctx + Lq, n_keep + Lq
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    shape = shape_of(cfg)
    say(f"fused filtering: {name}, n_prev={n_prev}, n_keep={n_keep}")
    prev = _prev_rows(w, n_prev, seed=9)
    t = {k: dev(v, dt) for k, v in lay.items()}
    kf = empty((n_req, L, Hkv, D), dt, fill_bits=0x7F01)
    vf = empty((n_req, L, Hkv, D), dt, fill_bits=0x7F01)
    out = empty((n_req, R, Hq, D), dt)
    lse = torch.empty((n_req, R, Hq), dtype=torch.float32, device="cuda")
    row_pos = torch.full((n_req, R), -1, dtype=torch.int32, device="cuda")
    dev_t = torch.empty((n_req, n_prev), dtype=torch.float32, device="cuda")
    ws = workspace(shape, n_req, n_chunks, L, R, Lq)
    sra.fused_layer(shape, chunks=w.chunks, k_store=t["k_store"], v_store=t["v_store"], q_fresh=t["q_new"],
                    k_fresh=t["k_new"], v_fresh=t["v_new"], row_pos=row_pos, k_fused=kf, v_fused=vf, out=out,
                    lse=lse, ws=ws, n_select=n_keep, hkvd_prev=torch.from_numpy(prev).cuda(),
                    hkvd_prev_ctx=n_prev, hkvd_dev=dev_t)
    torch.cuda.synchronize()
    rows, d_gpu = row_pos.cpu().numpy(), dev_t.cpu().numpy()
    o_gpu, kf_h, vf_h = host(out), host(kf), host(vf)
    for q in range(n_req):
        kw = dict(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[q], L=L, q_new=lay["q_new"][q],
                  k_new=lay["k_new"][q], v_new=lay["v_new"][q], dtype=dt, base=base, n_kv_heads=Hkv)
        ref = O.fused_layer(hkvd_prev=prev[q], hkvd_n_prev=n_prev, n_select=n_keep, attn_rows=[], **kw)
        rel = np.abs(d_gpu[q].astype(np.float64) - ref["dev"]) / np.abs(ref["dev"])
        assert rel.max() <= 1e-4, f"deviation: max relative error {rel.max():.3g}"
        swaps = _check_kept(rows[q], prev[q], n_prev, n_keep, ref["dev"], f"request {q}")
        # the rest of the layer, by the oracle on the rows the GPU kept
        srows = sample_rows(R, Lq, 24, seed=q)
        ref2 = O.fused_layer(row_pos=rows[q], attn_rows=srows, **kw)
        assert_storage_close(O.to_f64(kf_h[q], dt), ref2["k_fused"], dt, "fused K")
        np.testing.assert_array_equal(O.to_f64(vf_h[q], dt), ref2["v_fused"])
        mx, mean = assert_out_close(O.to_f64(o_gpu[q][srows], dt), ref2["out"], dt)
        say(f"  request {q}: dev rel err {rel.max():.3g}, window swaps {swaps}, out max err {mx:.3g}")


def test_three_layer_taper_by_gradual_filtering():
    """Layer 0 selects by the critical-layer score, layers 1 and 2 keep the rows of highest KV
    deviation among the previous layer's (15% -> 12% -> 9% of the context)."""
    w = make_workload(0)
    cfg, dt = w.cfg, w.cfg.dtype
    base = cfg.rope_base
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = cfg.query_len
    L = Lctx + Lq
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    shape = shape_of(cfg)
    counts = [O.select_count(p, 100, Lctx) for p in (15, 12, 9)]
    say(f"three-layer taper: counts {counts}")
    prev = None
    for l, n in enumerate(counts):
        lay = w.layer(l)
        t = {k: dev(v, dt) for k, v in lay.items()}
        R = n + Lq
        kf, vf = empty((1, L, Hkv, D), dt), empty((1, L, Hkv, D), dt)
        out = empty((1, R, Hq, D), dt)
        row_pos = torch.full((1, R), -1, dtype=torch.int32, device="cuda")
        ws = workspace(shape, 1, w.chunks.shape[1], L, R, Lq)
        kw = dict(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=L, q_new=lay["q_new"][0],
                  k_new=lay["k_new"][0], v_new=lay["v_new"][0], dtype=dt, base=base, n_kv_heads=Hkv)
        if l == 0:
            sc = torch.empty((1, Lctx), dtype=torch.float32, device="cuda")
            sra.fused_layer(shape, chunks=w.chunks, k_store=t["k_store"], v_store=t["v_store"], q_fresh=t["q_new"],
                            k_fresh=t["k_new"], v_fresh=t["v_new"], row_pos=row_pos, k_fused=kf, v_fused=vf,
                            out=out, ws=ws, q_crit=dev(w.q_crit, dt), k_crit_store=dev(w.k_crit, dt), n_select=n,
                            scores=sc)
            torch.cuda.synchronize()
            ref = O.fused_layer(q_crit=w.q_crit[0], k_crit_store=w.k_crit, n_select=n, attn_rows=[], **kw)
            swaps = check_selection(row_pos.cpu().numpy()[0][:n], ref["scores"], n)
        else:
            d_t = torch.empty((1, counts[l - 1]), dtype=torch.float32, device="cuda")
            sra.fused_layer(shape, chunks=w.chunks, k_store=t["k_store"], v_store=t["v_store"], q_fresh=t["q_new"],
                            k_fresh=t["k_new"], v_fresh=t["v_new"], row_pos=row_pos, k_fused=kf, v_fused=vf,
                            out=out, ws=ws, n_select=n, hkvd_prev=torch.from_numpy(prev).cuda(),
                            hkvd_prev_ctx=counts[l - 1], hkvd_dev=d_t)
            torch.cuda.synchronize()
            ref = O.fused_layer(hkvd_prev=prev[0], hkvd_n_prev=counts[l - 1], n_select=n, attn_rows=[], **kw)
            swaps = _check_kept(row_pos.cpu().numpy()[0], prev[0], counts[l - 1], n, ref["dev"], f"layer {l}")
            assert set(row_pos.cpu().numpy()[0][:n]) <= set(prev[0][:counts[l - 1]])
        rows = row_pos.cpu().numpy()
        srows = sample_rows(R, Lq, 16, seed=l)
        ref2 = O.fused_layer(row_pos=rows[0], attn_rows=srows, **kw)
        mx, _ = assert_out_close(O.to_f64(host(out)[0][srows], dt), ref2["out"], dt)
        say(f"  layer {l}: {n} rows, window swaps {swaps}, out max err {mx:.3g}")
        prev = rows
