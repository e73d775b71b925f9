"""Benchmark of the KV-cache fusion step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input. The timed step is the
Llama-70B-shaped eight-layer step (64 Q / 8 KV heads, head_dim 128, 35 chunks x 512 tokens + a 64-token
query, 17984 tokens): one critical-layer scoring with the chunks' key-norm anchors picks the ranking,
and each of the eight layers re-rotates its own chunk store, takes the first N_l = ceil((14 - l) L_ctx
/ 70) tokens of that ranking (20% tapering to 10%), scatters their fresh K/V and runs the sparse causal
attention of those rows (Sum N_l = 21504 selected rows per step). Seeded synthetic data from the
workload generators (per-KV-head scales U(0.5, 2)); every call goes through the C ABI on one stream.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu] [--no-legs] [--workload N]

Prints one JSON line. `value` = selected context rows per second of the whole step. Inputs are
resident in HBM; one step touches about 1.5 GB, far more than the 256 MB last-level cache. Side legs
time the same fused step at the Mistral-7B, Yi-34B (4 requests) and Llama-7B (per-chunk quotas)
shapes and the next rows (gradual filtering, pipelined layers, anchor probe, query-centric layers,
chunk statistics) at the Mistral-7B shape.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
HEADLINE = 3            # Llama-70B-shaped, eight tapered layers
# every source the attention stage's kernels and their launch are built from (a change to any of
# them invalidates the committed counter figures)
ATTN_SOURCES = ["selective_recompute_attention_amd/csrc/attn.hip",
                "selective_recompute_attention_amd/csrc/common.h",
                "selective_recompute_attention_amd/csrc/api.cpp"]
REPLICAS = {1: 8, 2: 3, 3: 1, 4: 1}   # input copies rotated between steps (footprint above 256 MB)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=HEADLINE, help="workload timed as the step (1-4)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the side measurements: profiler runs then see only the step's kernels")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only plain device copies of known size (for scaling memory counters)")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls the benchmark needs for events on the library's stream."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.h.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b):
        assert self.h.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


def hbm_copy_gbs():
    """Read+write bandwidth of a plain 1 GiB device copy (torch), timed with events: the practical
    ceiling of a streaming kernel on this GPU, reported beside the stages' figures."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    e1.synchronize()
    gbs = 2.0 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


def copy_probe():
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}))


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key):
    """HBM bytes per launch from committed counter runs, only while the attention sources are unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    ent = t.get(kernel_key)
    if not ent or ent.get("source_digest") != source_digest(ATTN_SOURCES):
        return None
    return ent.get("bytes_per_launch")


def timed_calls(hip, sp, fn, n):
    """Mean duration of n back-to-back calls of fn on the stream, from HIP events on it."""
    import torch
    a, b = hip.event(), hip.event()
    fn()
    torch.cuda._sleep(int(2e7))   # everything below is queued before the GPU reaches it
    hip.record(a, sp)
    for _ in range(n):
        fn()
    hip.record(b, sp)
    return hip.elapsed_ms(a, b) / n


def gen_layers(w, n_layers):
    """All layers' host tensors from the workload generators (numpy releases the GIL while drawing)."""
    from workloads.gen import _make_layer
    with ThreadPoolExecutor(max_workers=min(8, n_layers)) as ex:
        return list(ex.map(lambda l: _make_layer(w, l), range(n_layers)))


def bf16_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


class FusedStep:
    """Device inputs and outputs of one workload's fusion step, and the step itself.

    Layer 0 runs sra_fused_layer with the critical-layer scoring (and the chunks' anchors); a later
    layer l takes the first N_l of the same ranking and runs sra_fused_layer on those rows. The later
    layers' rows come from one sra_select_topn_nested launch among layer 0's rows, issued before layer
    1 (the sets nest: each is the Top-N_l of the same scores). `replicas` copies of every input rotate
    between steps."""

    def __init__(self, sra, w, replicas):
        import torch
        cfg = w.cfg
        self.sra, self.w, self.cfg = sra, w, cfg
        self.n_layers, self.n_req = cfg.n_layers, cfg.n_req
        self.Lq, self.Lctx, self.L = cfg.query_len, cfg.ctx_len, cfg.total_len
        self.Hq, self.Hkv, self.D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        self.shape = sra.make_shape(self.Hq, self.Hkv, self.D, "bf16", cfg.rope_base)
        self.n_chunks = w.chunks.shape[1]
        spec = w.selection_spec(0)
        self.quotas = w.quotas if spec[0] == "quota" else None
        if self.quotas is not None:
            self.counts = [int(self.quotas[0].sum())]
        else:
            self.counts = [sra.select_count(*w.selection_spec(l)[1:], self.Lctx) for l in range(self.n_layers)]
        host = gen_layers(w, self.n_layers)
        self.host0 = host[0]
        qc, kc = bf16_dev(w.q_crit), bf16_dev(w.k_crit)
        self.reps = []
        nr, L, Hkv, D = self.n_req, self.L, self.Hkv, self.D
        for i in range(replicas):
            layers = []
            for l in range(self.n_layers):
                R = self.counts[l] + self.Lq
                ins = {k: bf16_dev(v) for k, v in host[l].items()}
                outs = {"k_fused": torch.empty((nr, L, Hkv, D), dtype=torch.bfloat16, device="cuda"),
                        "v_fused": torch.empty((nr, L, Hkv, D), dtype=torch.bfloat16, device="cuda"),
                        "out": torch.empty((nr, R, self.Hq, D), dtype=torch.bfloat16, device="cuda"),
                        "lse": torch.empty((nr, R, self.Hq), dtype=torch.float32, device="cuda"),
                        "row_pos": torch.empty((nr, R), dtype=torch.int32, device="cuda")}
                layers.append((ins, outs))
            extra = {"q_crit": qc if i == 0 else qc.clone(), "k_crit": kc if i == 0 else kc.clone(),
                     "scores": torch.empty((nr, self.Lctx), dtype=torch.float32, device="cuda"),
                     "anchors": torch.empty((nr, self.n_chunks, cfg.anchors_k), dtype=torch.int32, device="cuda")}
            self.reps.append((layers, extra))
        del host
        R0 = self.counts[0] + self.Lq
        self.ws = torch.empty(sra.workspace_size(self.shape, nr, self.n_chunks, L, R0, self.Lq), dtype=torch.uint8,
                              device="cuda")

    def run(self, i, events=None, sel_events=None, hip=None, sp=None):
        layers, extra = self.reps[i % len(self.reps)]
        sra, w, cfg = self.sra, self.w, self.cfg
        for l, (ins, outs) in enumerate(layers):
            kw = dict(chunks=w.chunks, k_store=ins["k_store"], v_store=ins["v_store"], q_fresh=ins["q_new"],
                      k_fresh=ins["k_new"], v_fresh=ins["v_new"], row_pos=outs["row_pos"], k_fused=outs["k_fused"],
                      v_fused=outs["v_fused"], out=outs["out"], lse=outs["lse"], ws=self.ws,
                      stage_events=None if events is None else events[l])
            if l == 0:
                sra.fused_layer(self.shape, q_crit=extra["q_crit"], k_crit_store=extra["k_crit"],
                                n_select=None if self.quotas is not None else self.counts[0], quotas=self.quotas,
                                scores=extra["scores"], anchors_k=cfg.anchors_k, anchor_rows=extra["anchors"], **kw)
            else:
                if l == 1:   # every later layer's rows, in one launch
                    if sel_events is not None:
                        hip.record(ctypes.c_void_p(sel_events[l][0]), sp)
                    sra.select_topn_nested(extra["scores"], layers[0][1]["row_pos"], self.counts[0], self.Lq,
                                           self.counts[1:], [o["row_pos"] for _, o in layers[1:]])
                    if sel_events is not None:
                        hip.record(ctypes.c_void_p(sel_events[l][1]), sp)
                sra.fused_layer(self.shape, **kw)

    # ------------------------------------------------------------------ algorithmic work
    def row_positions(self):
        layers, _ = self.reps[0]
        return [outs["row_pos"].cpu().numpy().astype(np.int64) for _, outs in layers]

    def attn_flops(self, rps):
        return [4.0 * self.Hq * self.D * float(np.sum(rp + 1)) for rp in rps]

    def kv_row_bytes(self):
        return self.Hkv * self.D * 2

    def s1_bytes(self):
        """Read every distinct stored row's K and V once, write K and V of every request's context."""
        distinct = len({(int(s), int(n)) for s, n, _d, _o in self.w.chunks.reshape(-1, 4).tolist()})
        stored = distinct * self.cfg.chunk_tokens if self.cfg.shared_chunks else self.n_req * self.Lctx
        return 2 * self.kv_row_bytes() * (stored + self.n_req * self.Lctx)

    def s2_bytes(self):
        return self.kv_row_bytes() * self.w.store_rows            # the critical layer's K, once

    def s2_flops(self):
        return 2.0 * self.Lq * self.Hq * self.D * self.Lctx * self.n_req

    def s3_bytes(self, l):
        """Fresh K and V of the layer's rows read, the fused rows written."""
        return 4 * self.kv_row_bytes() * self.n_req * (self.counts[l] + self.Lq)

    def s1_launch_bytes(self):
        """Everything the re-rotation launch moves: the algorithmic bytes plus the fp16 copy of every
        fused key row that the attention reads its S operand from."""
        return self.s1_bytes() + self.kv_row_bytes() * self.n_req * self.Lctx

    def s3_launch_bytes(self, l):
        """Everything the scatter launch moves: fresh K/V read and fused K/V written, the fp16 key copy
        of the rows, and each row's fresh query read and written back as the attention's fp16 query
        operand (rotated and scaled in the same launch)."""
        rows = self.n_req * (self.counts[l] + self.Lq)
        q_row = self.Hq * self.D * 2
        return rows * (5 * self.kv_row_bytes() + 2 * q_row)

    def measure(self, hip, sp, steps, warmup):
        """Wall clock of `steps` steps (synchronised on both sides), then a separate pass with stage
        events queued behind a spin kernel; returns a dict of times and throughputs."""
        import torch
        for i in range(warmup):
            self.run(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.run(i)
        torch.cuda.synchronize()
        ms_per_step = 1e3 * (time.perf_counter() - t0) / steps
        n_ev = max(3, min(steps, 10))
        ev = [[(ctypes.c_void_p * 8)(*[hip.event() for _ in range(8)]) for _ in range(self.n_layers)]
              for _ in range(n_ev)]
        sev = [[(hip.event().value, hip.event().value) for _ in range(self.n_layers)] for _ in range(n_ev)]
        torch.cuda._sleep(int(4e7))   # every stage below is queued before the GPU reaches it
        for i in range(n_ev):
            self.run(i, ev[i], sev[i], hip, sp)
        torch.cuda.synchronize()

        def span(i, l, a, b):
            return hip.elapsed_ms(ctypes.c_void_p(ev[i][l][a]), ctypes.c_void_p(ev[i][l][b]))
        st = {"s1": [], "s2": [], "s3": [], "s4": [], "sel": []}
        for l in range(self.n_layers):
            st["s1"].append(float(np.mean([span(i, l, 0, 1) for i in range(n_ev)])))
            st["s2"].append(float(np.mean([span(i, l, 2, 3) for i in range(n_ev)])))
            st["s3"].append(float(np.mean([span(i, l, 4, 5) for i in range(n_ev)])))
            st["s4"].append(float(np.mean([span(i, l, 6, 7) for i in range(n_ev)])))
            st["sel"].append(float(np.mean([hip.elapsed_ms(ctypes.c_void_p(sev[i][l][0]), ctypes.c_void_p(sev[i][l][1]))
                                             for i in range(n_ev)])) if l == 1 else 0.0)
        # layer 0's stage 0 is empty when S1 runs inside the scoring launch (bf16): S1+S2 as one span
        s12_0 = float(np.mean([span(i, 0, 0, 3) for i in range(n_ev)]))
        rps = self.row_positions()
        flops = self.attn_flops(rps)
        t_attn = float(np.sum(st["s4"]))
        res = {"ms_per_step": ms_per_step, "rows": int(sum(self.counts)) * self.n_req,
               "rows_per_s": sum(self.counts) * self.n_req / (ms_per_step * 1e-3),
               "stage_ms": {k: [round(x, 5) for x in v] for k, v in st.items()},
               "layer0_rerotate_score_select_ms": s12_0,
               "attn_flops": flops, "attn_ms_total": t_attn,
               "attn_tflops": float(np.sum(flops)) / (t_attn * 1e-3) / 1e12}
        res["attn_mfma_frac"] = res["attn_tflops"] / BF16_PEAK_TFLOPS
        s1 = self.s1_bytes()
        later = [st["s1"][l] for l in range(1, self.n_layers)]
        if later:   # standalone re-rotation launches (layers without scoring)
            res["s1_hbm_gbs"] = s1 / (float(np.mean(later)) * 1e-3) / 1e9
        res["s1_bytes_per_layer"] = s1
        res["s2_bytes"] = self.s2_bytes()
        res["s2_gflop"] = self.s2_flops() / 1e9
        res["rerotate_score_hbm_gbs"] = (s1 + self.s2_bytes()) / (s12_0 * 1e-3) / 1e9
        s3b = [self.s3_bytes(l) for l in range(self.n_layers)]
        s3l = [self.s3_launch_bytes(l) for l in range(self.n_layers)]
        t3 = float(np.sum(st["s3"])) * 1e-3
        res["s3_hbm_gbs"] = float(np.sum(s3b)) / t3 / 1e9
        res["s3_launch_hbm_gbs"] = float(np.sum(s3l)) / t3 / 1e9
        res["s3_bytes"] = s3b
        res["s3_launch_bytes"] = s3l
        if later:
            res["s1_launch_hbm_gbs"] = self.s1_launch_bytes() / (float(np.mean(later)) * 1e-3) / 1e9
        res["s1_launch_bytes_per_layer"] = self.s1_launch_bytes()
        # the scoring alone at layer 0: the layer-0 span less a standalone re-rotation
        if later:
            t2 = s12_0 - float(np.mean(later))
            res["s2_ms_est"] = t2
            res["s2_tflops"] = self.s2_flops() / (t2 * 1e-3) / 1e12
        self.rps = rps
        return res


# ---------------------------------------------------------------------------------------- side legs
def hkvd_leg(sra, fs, hip, sp):
    """Gradual filtering at this layer's shape: deviation of the N recomputed context rows against
    the reused cache, then the rows of the next (13%) layer. Algorithmic bytes: fresh and reused K
    and V of every measured row."""
    import torch
    (ins, outs), = fs.reps[0][0][:1]
    N, Lq, Lctx = fs.counts[0], fs.Lq, fs.Lctx
    prev = outs["row_pos"].clone()
    rp = prev.long()[0]
    kn = ins["k_new"][0][rp].unsqueeze(0).contiguous()
    vn = ins["v_new"][0][rp].unsqueeze(0).contiguous()
    keep = sra.select_count(13, 100, Lctx)
    dev = torch.empty((1, N), dtype=torch.float32, device="cuda")
    nxt = torch.empty((1, keep + Lq), dtype=torch.int32, device="cuda")
    ms = timed_calls(hip, sp, lambda: sra.hkvd_select(fs.shape, outs["k_fused"], outs["v_fused"], kn, vn, prev, N,
                                                       keep, dev, nxt), 50)
    byts = 4.0 * fs.kv_row_bytes() * N
    return {"rows": N, "keep": keep, "ms_per_call": ms, "hbm_gbs": byts / (ms * 1e-3) / 1e9,
            "algorithmic_bytes": byts, "kernels": "k_kv_deviation + k_select"}


def pipeline_leg(sra, fs, hip, sp, n_layers=8):
    """Eight layers of this shape with the CacheBlend-style taper N_l = ceil((14 - l) L_ctx / 70)
    (layer 0 by the critical-layer score, later layers by gradual filtering), each layer's chunk
    store (K and V) coming from pinned host memory. Timed three ways on HIP events: the host-to-
    device copies alone, the layers alone (stores already on the device), and the pipelined run
    where layer l+1's copy overlaps layer l's step."""
    import torch
    w = fs.w
    (ins, _o), = fs.reps[0][0][:1]
    extra = fs.reps[0][1]
    Lq, Lctx = fs.Lq, fs.Lctx
    L, Hq, Hkv, D = Lctx + Lq, fs.Hq, fs.Hkv, fs.D
    counts = [sra.select_count(14 - l, 70, Lctx) for l in range(n_layers)]
    ws = torch.empty(sra.workspace_size(fs.shape, 1, fs.n_chunks, L, counts[0] + Lq, Lq), dtype=torch.uint8,
                     device="cuda")   # sized for the largest layer
    S = ins["k_store"].shape[0]
    store_bytes = ins["k_store"].numel() * 2
    hk = torch.empty(ins["k_store"].shape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(ins["v_store"].shape, dtype=torch.bfloat16, pin_memory=True)
    hk.copy_(ins["k_store"])
    hv.copy_(ins["v_store"])
    # one device buffer pair per layer: the copy stream never waits for compute
    k_buf = [torch.empty_like(ins["k_store"]) for _ in range(n_layers)]
    v_buf = [torch.empty_like(ins["v_store"]) for _ in range(n_layers)]
    outs = []
    for l, n in enumerate(counts):
        R = n + Lq
        outs.append({"k_fused": torch.empty((1, L, Hkv, D), dtype=torch.bfloat16, device="cuda"),
                     "v_fused": torch.empty((1, L, Hkv, D), dtype=torch.bfloat16, device="cuda"),
                     "out": torch.empty((1, R, Hq, D), dtype=torch.bfloat16, device="cuda"),
                     "row_pos": torch.empty((1, R), dtype=torch.int32, device="cuda"),
                     "dev": torch.empty((1, counts[l - 1] if l else 1), dtype=torch.float32, device="cuda"),
                     "scores": torch.empty((1, Lctx), dtype=torch.float32, device="cuda")})
    layers = []
    for l in range(n_layers):
        kw = dict(chunks=w.chunks, q_fresh=ins["q_new"], k_fresh=ins["k_new"], v_fresh=ins["v_new"],
                  row_pos=outs[l]["row_pos"], k_fused=outs[l]["k_fused"], v_fused=outs[l]["v_fused"],
                  out=outs[l]["out"], n_select=counts[l], store_rows=S)
        if l == 0:
            kw.update(q_crit=extra["q_crit"], k_crit_store=extra["k_crit"], scores=outs[l]["scores"])
        else:
            kw.update(hkvd_prev=outs[l - 1]["row_pos"], hkvd_prev_ctx=counts[l - 1], hkvd_dev=outs[l]["dev"])
        layers.append(kw)
    copy_stream = torch.cuda.Stream()
    cp = ctypes.c_void_p(copy_stream.cuda_stream)
    ev = sra.create_events(2 * n_layers)
    stream = torch.cuda.current_stream()

    def span(fn, st, reps=5):
        a, b = hip.event(), hip.event()
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            hip.record(a, st)
            fn()
            hip.record(b, st)
            ms.append(hip.elapsed_ms(a, b))
            torch.cuda.synchronize()
        return float(np.median(ms))

    def copies():
        with torch.cuda.stream(copy_stream):
            for l in range(n_layers):
                k_buf[l].copy_(hk, non_blocking=True)
                v_buf[l].copy_(hv, non_blocking=True)

    def compute():
        for l in range(n_layers):
            sra.fused_layer(fs.shape, ws=ws, k_store=ins["k_store"], v_store=ins["v_store"],
                            **{k: v for k, v in layers[l].items() if k != "store_rows"})

    def pipelined():
        sra.pipelined_layers(fs.shape, layers, [hk] * n_layers, [hv] * n_layers, k_buf, v_buf, ev, ws,
                             copy_stream=copy_stream)

    try:
        t_copy = span(copies, cp)
        t_comp = span(compute, sp)
        # the pipelined run starts with the first copy on the copy stream: bracket it on both
        a, b = hip.event(), hip.event()
        pipelined()
        torch.cuda.synchronize()
        ms = []
        for _ in range(5):
            hip.record(a, cp)
            copy_stream.wait_stream(stream)
            pipelined()
            hip.record(b, sp)
            ms.append(hip.elapsed_ms(a, b))
            torch.cuda.synchronize()
        t_pipe = float(np.median(ms))
    finally:
        torch.cuda.synchronize()
        sra.destroy_events(ev)
    hidden = (t_copy + t_comp - t_pipe) / min(t_copy, t_comp)
    return {"layers": n_layers, "counts": counts, "store_mb_per_layer": 2 * store_bytes / 1e6,
            "copy_ms": t_copy, "compute_ms": t_comp, "pipelined_ms": t_pipe,
            "h2d_gbs": n_layers * 2 * store_bytes / (t_copy * 1e-3) / 1e9,
            "overlap_of_shorter": hidden,
            "note": "pipelined_ms near max(copy_ms, compute_ms) means the recompute hides under the load"}


def probe_leg(sra, fs, hip, sp):
    """The query's anchor-grounded probe pass: gather the chunks' anchors into a compact prefix
    (keys re-rotated to their prefix rows), store the query's K/V after it and attend every query
    row over prefix and query."""
    import torch
    (ins, _o), = fs.reps[0][0][:1]
    extra = fs.reps[0][1]
    Lq, Lctx, Hq, Hkv, D = fs.Lq, fs.Lctx, fs.Hq, fs.Hkv, fs.D
    A = fs.n_chunks * fs.cfg.anchors_k
    Lp = A + Lq
    kp = torch.empty((1, Lp, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    qn = ins["q_new"][:, Lctx:].contiguous()
    kn = ins["k_new"][:, Lctx:].contiguous()
    vn = ins["v_new"][:, Lctx:].contiguous()
    rows = torch.arange(A, Lp, dtype=torch.int32, device="cuda")[None].contiguous()
    out = torch.empty((1, Lq, Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(sra.workspace_size(fs.shape, 1, 1, Lp, Lq, 1), dtype=torch.uint8, device="cuda")

    def probe():
        sra.anchor_prefix(fs.shape, ins["k_store"], ins["v_store"], fs.w.chunks, extra["anchors"], kp, vp)
        sra.scatter_kv(fs.shape, kn, vn, rows, kp, vp)
        sra.sparse_causal_attn(fs.shape, qn, rows, kp, vp, out, None, ws)

    ms = timed_calls(hip, sp, probe, 50)
    return {"prefix_rows": A, "query_rows": Lq, "ms_per_probe": ms,
            "kernels": "k_anchor_prefix + k_scatter + k_attn_mfma + k_attn_combine"}


def qc_layers_leg(sra, fs, hip, sp, n_layers=8):
    """Scoring cost of the query-centric baselines at this shape: QCAll scores every layer with
    its own query and keys (8 layers here), against the one critical layer QCFuse scores; QCLast
    costs one layer like the critical one."""
    import torch
    extra = fs.reps[0][1]
    N, Lq, Lctx = fs.counts[0], fs.Lq, fs.Lctx
    ws = torch.empty(sra.workspace_size(fs.shape, 1, fs.n_chunks, Lctx + Lq, N + Lq, Lq), dtype=torch.uint8,
                     device="cuda")
    sc = torch.empty((1, Lctx), dtype=torch.float32, device="cuda")
    rp = torch.empty((1, N + Lq), dtype=torch.int32, device="cuda")

    def one():
        sra.score_select(fs.shape, extra["q_crit"], extra["k_crit"], fs.w.chunks, N, None, sc, rp, ws)

    t_one = timed_calls(hip, sp, one, 50)

    def all_layers():
        for _ in range(n_layers):
            one()

    qc_all = timed_calls(hip, sp, all_layers, 10)
    return {"critical_layer_ms": t_one, "qcall_ms": qc_all, "layers": n_layers, "qcall_over_critical": qc_all / t_one}


def stats_leg(sra, fs, hip, sp):
    """Cache-Craft attention statistics of this layer's full causal prefill (every context token
    over the keys before it, per chunk). Algorithmic flops: 2 Hq d per (token, visible key) for the
    logits (the two passes and the hi/lo split are the implementation's extra work)."""
    import torch
    (ins, _o), = fs.reps[0][0][:1]
    Lctx = fs.Lctx
    kc = ins["k_new"]   # any bf16 keys of the right shape: the timing does not depend on values
    inter = torch.empty((1, Lctx, fs.n_chunks), dtype=torch.float32, device="cuda")
    score = torch.empty((1, Lctx), dtype=torch.float32, device="cuda")
    cci = torch.empty((1, fs.n_chunks), dtype=torch.float32, device="cuda")
    ws = torch.empty(sra.stats_workspace_size(fs.shape, 1, Lctx, fs.n_chunks), dtype=torch.uint8, device="cuda")
    ms = timed_calls(hip, sp, lambda: sra.chunk_attention_stats(fs.shape, ins["q_new"], kc, fs.w.chunks, ws, inter,
                                                                 score, cci), 10)
    flops = 2.0 * fs.Hq * fs.D * Lctx * (Lctx + 1) / 2.0
    return {"tokens": Lctx, "ms_per_call": ms, "algorithmic_tflops": flops / (ms * 1e-3) / 1e12,
            "kernels": "k_scatter (query operand) + k_chunk_stats + k_stats_finish"}


def summary(res):
    keep = ["ms_per_step", "rows", "rows_per_s", "attn_tflops", "attn_mfma_frac", "s1_hbm_gbs",
            "s1_launch_hbm_gbs", "rerotate_score_hbm_gbs", "s3_hbm_gbs", "s3_launch_hbm_gbs", "s2_tflops",
            "stage_ms", "layer0_rerotate_score_select_ms"]
    return {k: res[k] for k in keep if k in res}


# ---------------------------------------------------------------------------------------- CPU baseline
def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return None


def cpu_baseline(w, counts, budget_s):
    """The fp64 oracle (as it stands) on a bounded sample of the same eight-layer step, scaled to rows/s:
    S1 and S3 of layer 0 in full, the critical-layer scoring, anchors and ranking once, and S4 on a
    spread of layer 0's rows until about half the budget is used. The step's time is estimated as
    scoring + anchors + 8 x S1 + S3 scaled by each layer's rows + S4 scaled by each layer's algorithmic
    flops (4 Hq d (p+1) per row)."""
    import oracle as O
    cfg = w.cfg
    lay = w.layer(0)
    ch = w.chunks[0]
    Lctx, Lq, L = cfg.ctx_len, cfg.query_len, cfg.total_len
    t0 = time.perf_counter()
    kf, vf = O.fuse_rerotate(lay["k_store"], lay["v_store"], ch, L, cfg.dtype, cfg.rope_base)
    t_s1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.extract_anchors(w.k_crit, ch, cfg.anchors_k, cfg.dtype)
    t_anc = time.perf_counter() - t0
    t0 = time.perf_counter()
    s = O.critical_scores(w.q_crit[0], w.k_crit, ch, cfg.n_kv_heads, cfg.dtype, cfg.rope_base)
    order_rows = O.select_topn(s, counts[0])
    t_s2 = time.perf_counter() - t0
    rps = [O.row_positions(O.select_topn(s, n), Lctx, Lq).astype(np.int64) for n in counts]
    rp = rps[0]
    t0 = time.perf_counter()
    kf, vf = O.scatter_kv(kf, vf, lay["k_new"][0][rp], lay["v_new"][0][rp], rp, cfg.dtype, cfg.rope_base)
    t_s3 = time.perf_counter() - t0
    qn = lay["q_new"][0][rp]
    # S4 on a seeded spread of rows, in batches, until about half the budget is spent
    rng = np.random.default_rng(0)
    order = rng.permutation(len(rp))
    done, t_s4 = [], 0.0
    while t_s4 < 0.5 * budget_s and len(done) < len(rp):
        batch = order[len(done):len(done) + 8].tolist()
        t0 = time.perf_counter()
        O.sparse_causal_attn(qn, rp, kf, vf, cfg.dtype, cfg.rope_base, rows=batch)
        t_s4 += time.perf_counter() - t0
        done += batch
    f_sample = float(np.sum(rp[done] + 1))
    est = t_s2 + t_anc
    for l, rpl in enumerate(rps):
        est += t_s1 + t_s3 * len(rpl) / len(rp) + t_s4 * float(np.sum(rpl + 1)) / f_sample
    del order_rows
    return {"value": sum(counts) / est, "unit": "rows/s", "cores": blas_threads(), "kind": "oracle",
            "sample": (f"oracle on the Llama-70B-shaped step: S1 and S3 of layer 0 in full ({t_s1:.2f} s, {t_s3:.2f} s), "
                       f"scoring + ranking + anchors once ({t_s2 + t_anc:.2f} s), S4 on {len(done)} spread rows of "
                       f"layer 0 ({t_s4:.2f} s); step estimated as 8 x S1 + S3 per layer's rows + S4 per layer's "
                       f"flops = {est:.1f} s for {sum(counts)} rows; fp64 numpy"),
            "host_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_threads": blas_threads()}


def cpu_single_thread(budget_s=15.0):
    """The oracle's whole Mistral-7B-shaped step (anchors + fused layer) with one BLAS thread."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    from workloads import make_workload
    w = make_workload(1)
    cfg = w.cfg
    lay = w.layer(0)
    N = O.select_count(15, 100, cfg.ctx_len)
    steps, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            O.extract_anchors(w.k_crit, w.chunks[0], cfg.anchors_k, cfg.dtype)
            O.fused_layer(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=cfg.total_len,
                          q_new=lay["q_new"][0], k_new=lay["k_new"][0], v_new=lay["v_new"][0], dtype=cfg.dtype,
                          base=cfg.rope_base, n_kv_heads=cfg.n_kv_heads, q_crit=w.q_crit[0],
                          k_crit_store=w.k_crit, n_select=N)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or steps >= 5:
                break
    return {"value": N * steps / el, "unit": "rows/s", "cores": 1,
            "sample": f"{steps} whole Mistral-7B-shaped step(s) (anchors + fused layer, all {N + cfg.query_len} "
                      f"rows) with one BLAS thread, {el:.1f} s"}


# ---------------------------------------------------------------------------------------- main
def describe(cfg, counts):
    names = {1: "mistral7b_layer: 32 Q / 8 KV heads, d 128, 5 x 512-token chunks + 32-token query, 15% recompute",
             2: "yi34b_layer_x4req: 56 Q / 8 KV heads, d 128, 4 requests x 15 x 512-token chunks (11 shared) + "
                "48-token query, 10% recompute",
             3: "llama70b_8layers: 64 Q / 8 KV heads, d 128, 35 x 512-token chunks + 64-token query, 8 layers "
                "with N_l = ceil((14-l) L_ctx/70) (20% -> 10%), one critical-layer scoring",
             4: "llama7b_mha_quota: 32 Q / 32 KV heads, d 128, 64 x 512-token chunks + 64-token query, per-chunk "
                "quotas ceil(0.35 u 512)"}
    return f"{names[cfg.index]} (selected rows per step {sum(counts) * cfg.n_req})"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the fusion step is measured on one GPU's share at its real shape)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    import selective_recompute_attention_amd as sra
    from workloads import make_workload

    hip = Hip()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    w = make_workload(args.workload)
    cfg = w.cfg
    fs = FusedStep(sra, w, REPLICAS[args.workload])
    res = fs.measure(hip, sp, args.steps, args.warmup)
    rps = fs.rps
    for l, rp in enumerate(rps):   # the parity of these outputs against the oracle is covered by the GPU tests
        for q in range(cfg.n_req):
            n = fs.counts[l]
            assert (np.diff(rp[q][:n]) > 0).all() and rp[q][n] == fs.Lctx
    flops = res["attn_flops"]
    avg_flops = float(np.mean(flops))
    avg_ms = res["attn_ms_total"] / len(flops)
    achieved = avg_flops / (avg_ms * 1e-3) / 1e12
    key = f"attention_{cfg.name}"
    result = {
        "metric": "fused-layer selected rows/s (whole step); attention MFMA TFLOP/s; re-rotate+score HBM GB/s",
        "value": res["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded workload generators: N(0,1) bf16 caches and projections, per-KV-head scales "
                "U(0.5, 2); no weights or datasets)",
        "config": {"workload": describe(cfg, fs.counts), "global_batch": cfg.n_req, "seq_len": fs.L,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic_for(key),
                     "kernel": "sparse causal attention stage (k_attn_mfma + split merge), mean over the step's "
                               f"{len(flops)} launches",
                     "algorithmic_flops_per_launch": avg_flops, "avg_launch_ms": avg_ms},
        "stages_ms": res["stage_ms"],
        "layer0_rerotate_score_select_ms": res["layer0_rerotate_score_select_ms"],
        "s1_hbm_gbs": res.get("s1_hbm_gbs"),
        "rerotate_score_hbm_gbs": res["rerotate_score_hbm_gbs"],
        "s3_hbm_gbs": res["s3_hbm_gbs"],
        "streaming_stages": {
            "hbm_peak_gbs": HBM_PEAK_GBS,
            "plain_copy_gbs": hbm_copy_gbs(),
            "s1": {"ms": float(np.mean(res["stage_ms"]["s1"][1:])) if fs.n_layers > 1 else None,
                   "algorithmic_bytes": res["s1_bytes_per_layer"], "launch_bytes": res["s1_launch_bytes_per_layer"],
                   "algorithmic_gbs": res.get("s1_hbm_gbs"), "launch_gbs": res.get("s1_launch_hbm_gbs")},
            "s3": {"ms": res["stage_ms"]["s3"], "algorithmic_bytes": res["s3_bytes"],
                   "launch_bytes": res["s3_launch_bytes"], "algorithmic_gbs": res["s3_hbm_gbs"],
                   "launch_gbs": res["s3_launch_hbm_gbs"]},
            "s2_layer0": {"ms_est": res.get("s2_ms_est"), "gflop": res["s2_gflop"], "tflops": res.get("s2_tflops"),
                          "note": "compute-bound (two passes over the critical layer's K with float32-exact "
                                  "products); its time is the layer-0 span less a standalone re-rotation"},
            "note": "algorithmic bytes: what the method reads and writes (stored K/V, fused K/V, fresh K/V); "
                    "launch bytes add what the launch also moves for the attention (the fp16 key copy, and in "
                    "S3 the rows' fresh Q read and fp16 query operand written); plain_copy_gbs is a device "
                    "copy of 1 GiB timed here, the practical ceiling of a read+write stream"},
        "algorithmic": {"s1_bytes_per_layer": res["s1_bytes_per_layer"], "s2_bytes": res["s2_bytes"],
                        "s2_gflop": res["s2_gflop"], "attn_flops_per_layer": flops},
    }
    if not args.no_legs:
        legs = {}
        for wl in (1, 2, 4):
            if wl == args.workload:
                continue
            print(f"leg: fused step of workload {wl}", file=sys.stderr, flush=True)
            fl = FusedStep(sra, make_workload(wl), REPLICAS[wl])
            r = fl.measure(hip, sp, 20, 5)
            legs[fl.cfg.name] = dict(summary(r), workload=describe(fl.cfg, fl.counts))
            if wl == 1:
                mistral = fl
            else:
                del fl
                torch.cuda.empty_cache()
        result["fused_step_legs"] = legs
        if args.workload != 1:
            result["mistral7b_next_rows"] = {
                "hkvd": hkvd_leg(sra, mistral, hip, sp),
                "pipeline": pipeline_leg(sra, mistral, hip, sp),
                "anchor_probe": probe_leg(sra, mistral, hip, sp),
                "query_centric_layers": qc_layers_leg(sra, mistral, hip, sp),
                "chunk_stats": stats_leg(sra, mistral, hip, sp)}
    if not args.no_cpu:
        if args.workload == HEADLINE:
            w._layers[0] = fs.host0   # the same layer-0 inputs, not drawn again
            result["cpu_baseline"] = cpu_baseline(w, fs.counts, args.cpu_seconds)
        result["cpu_single_thread"] = cpu_single_thread()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
