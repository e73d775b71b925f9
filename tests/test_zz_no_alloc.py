"""The allocation-free fused layer (sra_fused_layer_static) against the workspace entry (sra_fused_layer).

Both run the same kernels on the same inputs, so every output must match bit for bit (stronger than the
parity bar: selection indices exact, floats identical). The static entry is called twice in a row, the
second call with a smaller layer, so the second runs on scratch that still holds the first call's data.
A layer needing more than the 64 MiB scratch is rejected on the host before anything runs.
"""
import numpy as np
import pytest
import torch

import oracle as O
import selective_recompute_attention_amd as sra
from workloads import make_custom, make_workload

from gpu_helpers import dev, empty, host, say, shape_of, workspace

pytestmark = pytest.mark.gpu


def _inputs(w, pct):
    cfg, dt = w.cfg, w.cfg.dtype
    lay = w.layer(0)
    n_req, n_chunks = w.chunks.shape[:2]
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = cfg.query_len
    N = O.select_count(pct, 100, Lctx)
    t = {k: dev(v, dt) for k, v in lay.items()}
    t["q_crit"], t["k_crit"] = dev(w.q_crit, dt), dev(w.k_crit, dt)
    return dict(w=w, t=t, n_req=n_req, n_chunks=n_chunks, Lctx=Lctx, Lq=Lq, L=Lctx + Lq, N=N, R=N + Lq)


def _run(inp, static):
    w, t = inp["w"], inp["t"]
    cfg, dt = w.cfg, w.cfg.dtype
    n_req, L, R, Lctx = inp["n_req"], inp["L"], inp["R"], inp["Lctx"]
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    shape = shape_of(cfg)
    outs = {"k_fused": empty((n_req, L, Hkv, D), dt, 0x7F01), "v_fused": empty((n_req, L, Hkv, D), dt, 0x7F01),
            "out": empty((n_req, R, Hq, D), dt), "lse": torch.empty((n_req, R, Hq), dtype=torch.float32, device="cuda"),
            "row_pos": torch.empty((n_req, R), dtype=torch.int32, device="cuda"),
            "scores": torch.empty((n_req, Lctx), dtype=torch.float32, device="cuda"),
            "anchors": torch.empty((n_req, inp["n_chunks"], 4), dtype=torch.int32, device="cuda")}
    kw = dict(chunks=w.chunks, k_store=t["k_store"], v_store=t["v_store"], q_fresh=t["q_new"], k_fresh=t["k_new"],
              v_fresh=t["v_new"], row_pos=outs["row_pos"], k_fused=outs["k_fused"], v_fused=outs["v_fused"],
              out=outs["out"], lse=outs["lse"], q_crit=t["q_crit"], k_crit_store=t["k_crit"], n_select=inp["N"],
              scores=outs["scores"], anchors_k=4, anchor_rows=outs["anchors"])
    if static:
        sra.fused_layer_static(shape, **kw)
    else:
        ws = workspace(shape, n_req, inp["n_chunks"], L, R, inp["Lq"])
        sra.fused_layer(shape, ws=ws, **kw)
        torch.cuda.synchronize()
        del ws
    return outs


def _host(outs):
    return {k: (host(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in outs.items()}


def test_static_scratch_matches_workspace_entry_twice():
    big = _inputs(make_workload(1), 15)   # Mistral-7B-shaped layer: about 46 MiB of scratch
    small = _inputs(make_custom(dtype="bf16", n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_lens=(90, 70, 33),
                                orig_pos=(4, 0, 11), query_len=6, n_req=2, seed=77), 25)
    ref = [_host(_run(big, False)), _host(_run(small, False))]
    say("static entry: Mistral-7B-shaped layer, then a two-request ragged layer, back to back")
    got = [_run(big, True), _run(small, True)]
    torch.cuda.synchronize()
    for name, r, g in zip(("mistral7b_layer", "two_request_ragged"), ref, got):
        g = _host(g)
        for k in r:
            a, b = r[k], g[k]
            if a.dtype == np.float32:
                a, b = a.view(np.uint32), b.view(np.uint32)
            np.testing.assert_array_equal(b, a, err_msg=f"{name}: {k} differs from the workspace entry")
        say(f"  {name}: every output bit-identical to sra_fused_layer")


def test_static_scratch_rejects_layers_beyond_it():
    w = make_custom(dtype="bf16", n_q_heads=32, n_kv_heads=8, head_dim=128, chunk_lens=(8192, 8192), query_len=32,
                    seed=3)
    inp = _inputs(w, 20)
    need = sra.workspace_size(shape_of(w.cfg), 1, 2, inp["L"], inp["R"], inp["Lq"])
    assert need > (64 << 20)
    say(f"static entry: a layer needing {need / 2**20:.1f} MiB is rejected")
    with pytest.raises(sra.SRAError) as ei:
        _run(inp, True)
    assert ei.value.status == 9 and "static scratch" in str(ei.value)
