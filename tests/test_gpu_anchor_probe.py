"""The anchor probe prefix and the query-centric layer baselines on the GPU against the oracle
(QCFuse summary (zh) §2.A anchors as a lightweight prefix; §4 QCAll / QCLast).

Bars: prefix keys within one bfloat16 ulp of the oracle's rounded value (float32: 1e-6 of the pair
norm), values bit-exact, rows past the prefix untouched; probe outputs as the attention parity
bar; scores 1e-4 relative and selections by the 1e-5 window rule.
"""
import numpy as np
import pytest
import torch

import oracle as O
import selective_recompute_attention_amd as sra
from workloads import make_custom, make_workload

from gpu_helpers import (assert_out_close, assert_scores_close, assert_storage_close, check_selection, dev,
                         empty, host, say, shape_of)

pytestmark = pytest.mark.gpu


def _workload(name):
    if name == "tiny_f32":
        return make_workload(0)
    if name == "mistral7b_layer":
        return make_workload(1)
    if name == "ragged_bf16":
        return make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=[200, 97, 300],
                           orig_pos=[0, 17, 50], query_len=24, n_req=2, seed=51, anchors_k=5)
    if name == "d64_bf16":
        return make_custom(dtype="bf16", n_q_heads=6, n_kv_heads=3, head_dim=64, chunk_lens=[70, 45],
                           orig_pos=[10, 0], query_len=5, n_req=1, seed=52, anchors_k=3)
    raise KeyError(name)


@pytest.mark.parametrize("name", ["tiny_f32", "ragged_bf16", "mistral7b_layer", "d64_bf16"])
def test_anchor_prefix_and_probe_match_oracle(name):
    w = _workload(name)
    cfg, dt = w.cfg, w.cfg.dtype
    base, k = cfg.rope_base, cfg.anchors_k
    lay = w.layer(0)
    n_req, n_chunks = w.chunks.shape[0], w.chunks.shape[1]
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = cfg.query_len
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    A = n_chunks * k
    Lp = A + Lq
    shape = shape_of(cfg)
    say(f"anchor probe: {name}, A={A}, Lq={Lq}, n_req={n_req}")
    anchors = np.stack([O.extract_anchors(w.k_crit, w.chunks[q], k, dt) for q in range(n_req)])
    kp = empty((n_req, Lp, Hkv, D), dt, fill_bits=0x7F01)
    vp = empty((n_req, Lp, Hkv, D), dt, fill_bits=0x7F01)
    t = {n: dev(lay[n], dt) for n in ("k_store", "v_store")}
    sra.anchor_prefix(shape, t["k_store"], t["v_store"], w.chunks, torch.from_numpy(anchors).cuda(), kp, vp)
    torch.cuda.synchronize()
    kp_h, vp_h = host(kp), host(vp)
    fill = np.uint16(0x7F01) if dt == "bf16" else np.int32(0x7F01).view(np.float32)
    for q in range(n_req):
        kref, vref = O.anchor_prefix(lay["k_store"], lay["v_store"], w.chunks[q], anchors[q], dt, base)
        assert_storage_close(O.to_f64(kp_h[q][:A], dt), kref, dt, f"prefix K (request {q})")
        np.testing.assert_array_equal(O.to_f64(vp_h[q][:A], dt), vref)
        assert np.all(kp_h[q][A:].view(np.uint16 if dt == "bf16" else np.uint32) ==
                      np.asarray(fill).view(np.uint16 if dt == "bf16" else np.uint32)), "rows past the prefix changed"
    # the probe pass: the query's rows after the prefix, every query row attending to all before it
    qn = np.stack([lay["q_new"][q][Lctx:] for q in range(n_req)])
    kn = np.stack([lay["k_new"][q][Lctx:] for q in range(n_req)])
    vn = np.stack([lay["v_new"][q][Lctx:] for q in range(n_req)])
    rows = torch.from_numpy(np.tile(np.arange(A, Lp, dtype=np.int32), (n_req, 1))).cuda()
    sra.scatter_kv(shape, dev(kn, dt), dev(vn, dt), rows, kp, vp)
    out = empty((n_req, Lq, Hq, D), dt)
    lse = torch.empty((n_req, Lq, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(sra.workspace_size(shape, n_req, 1, Lp, Lq, 1), dtype=torch.uint8, device="cuda")
    sra.sparse_causal_attn(shape, dev(qn, dt), rows, kp, vp, out, lse, ws)
    torch.cuda.synchronize()
    o_h, lse_h = host(out), lse.cpu().numpy()
    for q in range(n_req):
        kref, vref = O.anchor_prefix(lay["k_store"], lay["v_store"], w.chunks[q], anchors[q], dt, base)
        o_ref, lse_ref = O.anchor_probe(kref, vref, qn[q], kn[q], vn[q], dt, base)
        mx, mean = assert_out_close(O.to_f64(o_h[q], dt), o_ref, dt, "probe output")
        np.testing.assert_allclose(lse_h[q], lse_ref, rtol=0, atol=2e-2 if dt == "bf16" else 1e-4)
        say(f"  request {q}: probe out max err {mx:.3g}, mean {mean:.3g}")


@pytest.mark.parametrize("mode", ["all", "last"])
def test_query_centric_layer_baselines_match_oracle(mode):
    w = make_workload(0)
    cfg, dt = w.cfg, w.cfg.dtype
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq, n_layers = cfg.query_len, 3
    N = O.select_count(15, 100, Lctx)
    shape = shape_of(cfg)
    lays = [w.layer(l) for l in range(n_layers)]
    qs = [lays[l]["q_new"][0][Lctx:] for l in range(n_layers)]   # each layer's own query projections
    ks = [lays[l]["k_store"] for l in range(n_layers)]
    sc_ref, sel_ref = O.query_centric_layers(qs, ks, w.chunks[0], cfg.n_kv_heads, dt, cfg.rope_base, N, mode)
    say(f"query-centric layers ({mode}): {n_layers} layers, N={N}")
    layers = range(n_layers) if mode == "all" else [n_layers - 1]
    ws = torch.empty(sra.workspace_size(shape, 1, w.chunks.shape[1], Lctx + Lq, N + Lq, Lq), dtype=torch.uint8,
                     device="cuda")
    for i, l in enumerate(layers):
        scores = torch.empty((1, Lctx), dtype=torch.float32, device="cuda")
        row_pos = torch.empty((1, N + Lq), dtype=torch.int32, device="cuda")
        sra.score_select(shape, dev(qs[l][None], dt), dev(ks[l], dt), w.chunks, N, None, scores, row_pos, ws)
        torch.cuda.synchronize()
        rel = assert_scores_close(scores.cpu().numpy()[0], sc_ref[i])
        swaps = check_selection(row_pos.cpu().numpy()[0][:N], sc_ref[i], N)
        if mode == "all":
            assert swaps or list(row_pos.cpu().numpy()[0][:N]) == list(sel_ref[l])
        say(f"  layer {l}: scores rel err {rel:.3g}, window swaps {swaps}")
