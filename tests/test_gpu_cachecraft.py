"""Cache-Craft selection on the GPU against the oracle (CSDN article §2.1-§2.2; KVCache reuse 01
§2.3): per-token chunk attention statistics of a full causal prefill, token scores, CCI, and the
per-chunk recompute selection built from them.

Bars: statistics and token scores within 1e-4 relative + 1e-6 absolute of the oracle's (float32
probabilities summed exactly); CCI within 1e-5 relative; counts equal; selections by the 1e-5
window rule per chunk.
"""
import numpy as np
import pytest
import torch

import oracle as O
import selective_recompute_attention_amd as sra
from workloads import make_custom, make_workload

from gpu_helpers import check_selection, dev, say, shape_of

pytestmark = pytest.mark.gpu


def _workload(name):
    if name == "mistral7b_layer":
        return make_workload(1)
    if name == "ragged_bf16":
        return make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=[200, 97, 300],
                           orig_pos=[0, 0, 0], query_len=4, n_req=2, seed=71)
    if name == "d64_bf16":
        return make_custom(dtype="bf16", n_q_heads=6, n_kv_heads=3, head_dim=64, chunk_lens=[70, 45, 1, 30],
                           orig_pos=[0, 0, 0, 0], query_len=3, n_req=1, seed=72)
    raise KeyError(name)


def _close(gpu, ref, what):
    err = np.abs(gpu.astype(np.float64) - ref)
    bound = 1e-4 * np.abs(ref) + 1e-6
    assert (err <= bound).all(), f"{what}: max err {err.max():.3g} (worst ratio {(err / bound).max():.3g})"
    return float(err.max())


@pytest.mark.parametrize("name,rows", [("ragged_bf16", None), ("d64_bf16", None), ("mistral7b_layer", 48)])
def test_chunk_stats_and_selection_match_oracle(name, rows):
    w = _workload(name)
    cfg, dt = w.cfg, w.cfg.dtype
    base = cfg.rope_base
    lay = w.layer(0)
    n_req, n_chunks = w.chunks.shape[0], w.chunks.shape[1]
    Lctx = int(w.chunks[0, :, 1].sum())
    Hkv = cfg.n_kv_heads
    shape = shape_of(cfg)
    say(f"chunk stats: {name}, n_req={n_req}, chunks={n_chunks}, L_ctx={Lctx}")
    # the prefill's cached keys (rotated at their positions, stored as bf16) from the oracle
    kc = [O.round_to_storage(O.rope(O.to_f64(lay["k_new"][q][:Lctx], dt), np.arange(Lctx)[:, None], base), dt)
          for q in range(n_req)]
    kc = [O.storage_bits(k, dt) for k in kc]   # stored bit patterns, as the oracle takes them
    kc_d = dev(np.stack(kc), dt)
    q_d = dev(lay["q_new"], dt)
    inter = torch.empty((n_req, Lctx, n_chunks), dtype=torch.float32, device="cuda")
    score = torch.empty((n_req, Lctx), dtype=torch.float32, device="cuda")
    cci = torch.empty((n_req, n_chunks), dtype=torch.float32, device="cuda")
    ws = torch.empty(sra.stats_workspace_size(shape, n_req, Lctx, n_chunks), dtype=torch.uint8, device="cuda")
    sra.chunk_attention_stats(shape, q_d, kc_d, w.chunks, ws, inter, score, cci)
    torch.cuda.synchronize()
    inter_h, score_h, cci_h = inter.cpu().numpy(), score.cpu().numpy(), cci.cpu().numpy()
    alpha, beta = 0.4, 0.25
    for q in range(n_req):
        np.testing.assert_allclose(inter_h[q].sum(axis=1), cfg.n_q_heads, rtol=1e-5)
        if rows is None:
            ref = O.chunk_attention_stats(lay["q_new"][q], kc[q], w.chunks[q], Hkv, dt, base)
            e1 = _close(inter_h[q], ref, "inter")
            sref = O.preceding_chunk_scores(ref, w.chunks[q])
            e2 = _close(score_h[q], sref, "token scores")
            cref = O.cache_context_impact(ref, w.chunks[q])
            rel = np.abs(cci_h[q].astype(np.float64) - cref) / cref
            assert rel.max() <= 1e-5, f"CCI: max relative error {rel.max():.3g}"
            # the recompute selection: per-chunk counts from CCI, argtop_N of the token scores
            lens = w.chunks[q][:, 1]
            counts = [sra.cachecraft_count(alpha, float(cci_h[q][c]), beta, int(lens[c])) for c in range(n_chunks)]
            cref_n = [O.cachecraft_count(alpha, float(cref[c]), beta, int(lens[c])) for c in range(n_chunks)]
            assert counts == cref_n, f"counts {counts} != {cref_n}"
            N = int(sum(counts))
            rp = torch.empty((1, N), dtype=torch.int32, device="cuda")
            sra.select_topn(score[q:q + 1].contiguous(), None, np.asarray([counts], dtype=np.int32), w.chunks[q:q + 1],
                            0, rp)
            torch.cuda.synchronize()
            sel = rp.cpu().numpy()[0]
            start = 0
            for c in range(n_chunks):
                n0, T = int(w.chunks[q][c][2]), int(lens[c])
                swaps = check_selection(sel[start:start + counts[c]], sref[n0:n0 + T], counts[c], offset=n0)
                start += counts[c]
            say(f"  request {q}: inter err {e1:.3g}, score err {e2:.3g}, CCI rel {rel.max():.3g}, counts {counts}")
        else:
            rng = np.random.default_rng(3)
            sample = np.unique(np.concatenate([[0, Lctx - 1, 511, 512, 1023, 1024], rng.choice(Lctx, rows)]))
            ref = O.chunk_attention_stats(lay["q_new"][q], kc[q], w.chunks[q], Hkv, dt, base, rows=sample)
            e1 = _close(inter_h[q][sample], ref, "inter (sampled tokens)")
            say(f"  request {q}: {len(sample)} sampled tokens, inter err {e1:.3g}")
