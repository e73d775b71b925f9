"""Helpers of the GPU parity tests: moving workload arrays to the device, running the HIP path
through the C ABI binding, and the comparison rules of the parity bar.

Comparison rules (float outputs):
  * fused K rows: within 1 bfloat16 ulp of the oracle's rounded value (float32: 2e-6 relative);
    V rows and K rows of chunks that do not move (delta 0): bit-exact;
  * scores: 1e-4 relative to the oracle;
  * selected indices: bit-exact, except that swaps are allowed among tokens whose oracle score is
    within 1e-5 relative of the N-th score (per chunk with quotas);
  * attention output: bfloat16 max |err| <= 1.5e-2 where |ref| < 4, and half a bfloat16 ulp of
    |ref| plus 5e-3 where |ref| >= 4 (the output's own rounding to bfloat16 reaches 1.56e-2 there);
    mean |err| <= 2e-3; float32 |err| <= 1e-4 * max(1, |ref|); log-sum-exp: 2e-2 (bf16) / 1e-4 (f32)
    absolute.
"""
import sys

import numpy as np
import torch

import oracle as O
import selective_recompute_attention_amd as sra


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def empty(shape, dtype: str, fill_bits=None) -> torch.Tensor:
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = torch.empty(shape, dtype=tdt, device="cuda")
    if fill_bits is not None:   # a recognisable pattern to catch rows that are never written
        if dtype == "bf16":
            t.view(torch.int16).fill_(fill_bits)
        else:
            t.view(torch.int32).fill_(fill_bits)
    return t


def shape_of(cfg):
    return sra.make_shape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype, cfg.rope_base)


def workspace(shape, n_req, n_chunks, L, R, Lq) -> torch.Tensor:
    n = sra.workspace_size(shape, n_req, n_chunks, L, R, Lq)
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    _m, e = np.frexp(np.abs(ref))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def pair_norm(x: np.ndarray) -> np.ndarray:
    """Norm of each rotary pair (x_i, x_{i+d/2}), broadcast back to both members (rotation-invariant)."""
    h = x.shape[-1] // 2
    r = np.sqrt(x[..., :h] ** 2 + x[..., h:] ** 2)
    return np.concatenate([r, r], axis=-1)


def assert_storage_close(gpu_vals: np.ndarray, ref: np.ndarray, dtype: str, what: str, ulps: float = 1.0):
    """gpu_vals: float64 values decoded from the device; ref: oracle values (on the storage grid).

    A rotated pair is computed in float32 on the device, so each component carries an absolute error of
    a few float32 ulps of the pair's norm before it is stored. bf16: within `ulps` bfloat16 ulps of the
    oracle's rounded value plus 4 * 2^-24 * pair norm (the second term only matters where the pair's
    components cancel to a value far below the norm). f32: 1e-6 * max(1, pair norm)."""
    if dtype == "bf16":
        tol = ulps * bf16_ulp(ref) + 4 * 2.0 ** -24 * pair_norm(ref) + 1e-30
    else:
        tol = 1e-6 * np.maximum(1.0, pair_norm(ref))
    err = np.abs(gpu_vals - ref)
    bad = err > tol
    if bad.any():
        idx = [tuple(int(v) for v in i) for i in np.argwhere(bad)[:5]]
        detail = "; ".join(f"{i}: gpu {gpu_vals[i]!r} ref {ref[i]!r} bound {tol[i]:.3g}" for i in idx)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} values off by more than the bound; "
                             f"first: {detail}")


def assert_out_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "attention output"):
    """bf16: max |err| <= 1.5e-2 and mean |err| <= 2e-3. Where |ref| >= 4, half a bfloat16 ulp of the
    stored output alone is 1.56e-2 (a correctly rounded output can miss 1.5e-2 there), so the bound is
    half an ulp of |ref| plus 5e-3 of arithmetic error: 2.06e-2 on [4, 8), 3.6e-2 on [8, 16)."""
    err = np.abs(gpu - ref)
    if dtype == "bf16":
        bound = np.maximum(1.5e-2, 0.5 * bf16_ulp(ref) + 5e-3)
        bad = err > bound
        if bad.any():
            i = tuple(int(v) for v in np.argwhere(bad)[0])
            raise AssertionError(f"{what}: {bad.sum()} values beyond the bound (max |err| {err.max():.4g}); "
                                 f"first {i}: gpu {gpu[i]!r} ref {ref[i]!r}")
        assert err.mean() <= 2e-3, f"{what}: mean |err| {err.mean():.4g} > 2e-3"
    else:
        tol = 1e-4 * np.maximum(1.0, np.abs(ref))
        assert (err <= tol).all(), f"{what}: max |err| {err.max():.4g} (f32 bound 1e-4 * max(1, |ref|))"
    return float(err.max()), float(err.mean())


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, what: str = "scores"):
    rel = np.abs(gpu.astype(np.float64) - ref) / np.abs(ref)
    assert rel.max() <= 1e-4, f"{what}: max relative error {rel.max():.3g} > 1e-4"
    return float(rel.max())


def check_selection(sel_gpu, scores_ref, N: int, offset: int = 0, rel: float = 1e-5):
    """Window rule: same count; identical outside the 1e-5 window around the N-th score."""
    sel_gpu = np.asarray(sel_gpu, dtype=np.int64) - offset
    assert len(sel_gpu) == N
    assert np.all(np.diff(sel_gpu) > 0), "selection must be strictly ascending"
    if N == 0:
        return 0
    s = np.asarray(scores_ref, dtype=np.float64)
    assert sel_gpu.min() >= 0 and sel_gpu.max() < len(s)
    ref = O.select_topn(s, N)
    order = sorted(range(len(s)), key=lambda j: (-s[j], j))
    s_star = s[order[N - 1]]
    window = set(np.flatnonzero(np.abs(s - s_star) <= rel * abs(s_star)).tolist())
    a = set(sel_gpu.tolist()) - window
    b = set(ref.tolist()) - window
    assert a == b, f"selection differs outside the tie window: gpu-only {sorted(a - b)[:8]}, ref-only {sorted(b - a)[:8]}"
    return len(set(sel_gpu.tolist()) ^ set(ref.tolist())) // 2


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    return O.to_f64(a, dtype)


def bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage bits of a host copy (uint16 for bf16, uint32 for f32)."""
    return a if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def sample_rows(R: int, Lq: int, k: int, seed: int = 0) -> list:
    """Rows the oracle evaluates one by one at full size: first/last selected rows, every query row
    (bounded), and a seeded spread of the rest."""
    if R <= k:
        return list(range(R))
    rng = np.random.default_rng(seed)
    base = {0, 1, R - Lq - 1, R - Lq, R - 1}
    base |= set(range(max(R - Lq, 0), R, max(1, Lq // 8)))
    rest = sorted(set(range(R)) - base)
    pick = rng.choice(len(rest), size=max(0, k - len(base)), replace=False)
    return sorted(base | {rest[i] for i in pick})


def run_fused(w, layer: int = 0, *, score: bool = True, row_pos_in=None, n_select=None, quotas=None,
              fallback: bool = False):
    """Runs sra_fused_layer for all requests of workload w; returns host arrays (with fallback, also
    the [n_req][Hkv] report of groups recomputed exactly because of fp16's range)."""
    cfg = w.cfg
    dt = cfg.dtype
    lay = w.layer(layer)
    n_req, n_chunks = w.chunks.shape[0], w.chunks.shape[1]
    Lctx = int(w.chunks[0, :, 1].sum())
    Lq = cfg.query_len
    L = Lctx + Lq
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    shape = shape_of(cfg)
    if score:
        if quotas is not None:
            N = int(np.asarray(quotas)[0].sum())
        else:
            N = int(n_select)
    else:
        N = row_pos_in.shape[1] - Lq
    R = N + Lq
    t = {k: dev(v, dt) for k, v in lay.items()}
    kf = empty((n_req, L, Hkv, D), dt, fill_bits=0x7F01)
    vf = empty((n_req, L, Hkv, D), dt, fill_bits=0x7F01)
    out = empty((n_req, R, Hq, D), dt)
    lse = torch.empty((n_req, R, Hq), dtype=torch.float32, device="cuda")
    scores = torch.empty((n_req, Lctx), dtype=torch.float32, device="cuda") if score else None
    if score:
        row_pos = torch.empty((n_req, R), dtype=torch.int32, device="cuda")
    else:
        row_pos = torch.from_numpy(np.ascontiguousarray(row_pos_in, dtype=np.int32)).cuda()
    ws = workspace(shape, n_req, n_chunks, L, R, Lq)
    kw = {}
    fb = None
    if fallback:
        fb = torch.full((n_req, Hkv), -1, dtype=torch.int32, device="cuda")
        kw["attn_fallback"] = fb
    if score:
        kw.update(q_crit=dev(w.q_crit, dt), k_crit_store=dev(w.k_crit, dt), n_select=n_select,
                  quotas=quotas, scores=scores)
    sra.fused_layer(shape, chunks=w.chunks, k_store=t["k_store"], v_store=t["v_store"], q_fresh=t["q_new"],
                    k_fresh=t["k_new"], v_fresh=t["v_new"], row_pos=row_pos, k_fused=kf, v_fused=vf, out=out,
                    lse=lse, ws=ws, **kw)
    torch.cuda.synchronize()
    res = {"k_fused": host(kf), "v_fused": host(vf), "out": host(out), "lse": lse.cpu().numpy(),
           "row_pos": row_pos.cpu().numpy(), "N": N, "R": R, "L": L, "Lctx": Lctx}
    if score:
        res["scores"] = scores.cpu().numpy()
    if fb is not None:
        res["fallback"] = fb.cpu().numpy()
    return res
