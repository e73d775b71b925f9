"""Layer-pipelined reconstruction (QCFuse summary (zh) §2.A; KVCache reuse 01 §1.3.5): each
layer's chunk store is copied from pinned host memory on a second stream while the previous layer
runs. Every layer's outputs must equal, bit for bit, those of plain sequential calls with the
stores already on the device (those calls are checked against the oracle by the parity tests);
the last layer is also checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

import oracle as O
import selective_recompute_attention_amd as sra
from workloads import make_workload

from gpu_helpers import assert_out_close, dev, empty, host, sample_rows, say, shape_of, workspace

pytestmark = pytest.mark.gpu


def _pinned(a: np.ndarray, dtype: str) -> torch.Tensor:
    src = dev(a, dtype).cpu()
    t = torch.empty(src.shape, dtype=src.dtype, pin_memory=True)
    t.copy_(src)
    return t


@pytest.mark.parametrize("wid,n_layers,n_buf", [(0, 4, 2), (1, 3, 2), (0, 5, 3), (1, 3, 3)])
def test_pipelined_layers_equal_sequential_layers(wid, n_layers, n_buf):
    w = make_workload(wid)
    cfg, dt = w.cfg, w.cfg.dtype
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = cfg.query_len
    L = Lctx + Lq
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    shape = shape_of(cfg)
    counts = [O.select_count(15 - 2 * l, 100, Lctx) for l in range(n_layers)]
    say(f"pipelined layers: workload {wid}, counts {counts}, {n_buf} buffer pairs")
    lays = [w.layer(l) for l in range(n_layers)]
    fresh = [{k: dev(lays[l][k], dt) for k in ("q_new", "k_new", "v_new")} for l in range(n_layers)]
    S = w.store_rows

    def outputs():
        o = []
        for l, n in enumerate(counts):
            R = n + Lq
            o.append({"k_fused": empty((1, L, Hkv, D), dt), "v_fused": empty((1, L, Hkv, D), dt),
                      "out": empty((1, R, Hq, D), dt),
                      "row_pos": torch.full((1, R), -1, dtype=torch.int32, device="cuda"),
                      "dev": torch.empty((1, counts[l - 1] if l else 1), dtype=torch.float32, device="cuda"),
                      "scores": torch.empty((1, Lctx), dtype=torch.float32, device="cuda")})
        return o

    def layer_kw(l, o):
        kw = dict(chunks=w.chunks, q_fresh=fresh[l]["q_new"], k_fresh=fresh[l]["k_new"], v_fresh=fresh[l]["v_new"],
                  row_pos=o[l]["row_pos"], k_fused=o[l]["k_fused"], v_fused=o[l]["v_fused"], out=o[l]["out"],
                  n_select=counts[l])
        if l == 0:
            kw.update(q_crit=dev(w.q_crit, dt), k_crit_store=dev(w.k_crit, dt), scores=o[l]["scores"])
        else:
            kw.update(hkvd_prev=o[l - 1]["row_pos"], hkvd_prev_ctx=counts[l - 1], hkvd_dev=o[l]["dev"])
        return kw

    ws = workspace(shape, 1, w.chunks.shape[1], L, counts[0] + Lq, Lq)
    # sequential reference: stores resident on the device
    ref = outputs()
    for l in range(n_layers):
        sra.fused_layer(shape, ws=ws, k_store=dev(lays[l]["k_store"], dt), v_store=dev(lays[l]["v_store"], dt),
                        **layer_kw(l, ref))
    torch.cuda.synchronize()
    # pipelined: stores from pinned host memory through two device buffer pairs
    hk = [_pinned(lays[l]["k_store"], dt) for l in range(n_layers)]
    hv = [_pinned(lays[l]["v_store"], dt) for l in range(n_layers)]
    k_buf = [empty((S, Hkv, D), dt, fill_bits=0x7F01) for _ in range(n_buf)]
    v_buf = [empty((S, Hkv, D), dt, fill_bits=0x7F01) for _ in range(n_buf)]
    got = outputs()
    layers = []
    for l in range(n_layers):
        kw = layer_kw(l, got)
        kw["store_rows"] = S
        layers.append(kw)
    ev = sra.create_events(2 * n_buf)
    copy_stream = torch.cuda.Stream()
    try:
        for rep in range(2):   # the second pass reuses buffers that still hold the last layers' stores
            for o in got:
                o["out"].view(torch.int16 if dt == "bf16" else torch.int32).fill_(0x7F01 + rep)
            sra.pipelined_layers(shape, layers, hk, hv, k_buf, v_buf, ev, ws, copy_stream=copy_stream)
            torch.cuda.synchronize()
            for l in range(n_layers):
                for k in ("row_pos", "k_fused", "v_fused", "out"):
                    assert torch.equal(got[l][k], ref[l][k]), f"pass {rep}, layer {l}: {k} differs"
                if l:
                    assert torch.equal(got[l]["dev"], ref[l]["dev"])
            say(f"  pass {rep}: all {n_layers} layers equal the sequential run")
    finally:
        sra.destroy_events(ev)
    # the last layer against the oracle, on the rows the GPU chose
    l = n_layers - 1
    R = counts[l] + Lq
    rows = got[l]["row_pos"].cpu().numpy()[0]
    srows = sample_rows(R, Lq, 12, seed=l)
    r = O.fused_layer(k_store=lays[l]["k_store"], v_store=lays[l]["v_store"], chunks=w.chunks[0], L=L,
                      q_new=lays[l]["q_new"][0], k_new=lays[l]["k_new"][0], v_new=lays[l]["v_new"][0], dtype=dt,
                      base=cfg.rope_base, n_kv_heads=Hkv, row_pos=rows, attn_rows=srows)
    mx, _ = assert_out_close(O.to_f64(host(got[l]["out"])[0][srows], dt), r["out"], dt)
    say(f"  last layer vs oracle: out max err {mx:.3g}")
