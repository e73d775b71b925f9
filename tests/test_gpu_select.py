"""Top-N selection on the GPU against the oracle's definition (the N best indices by (-score, index),
ascending), at unit lengths that take each of the kernel's key paths: registers (up to 4096 keys), LDS
(up to 32768) and global memory (beyond). Scores are quantised so that many ties straddle the N-th
score, and the lowest index must win them."""
import numpy as np
import pytest
import torch

import oracle as O
import selective_recompute_attention_amd as sra

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ctx_len", [3000, 4096, 17920, 32768, 40000])
def test_select_topn_key_paths_match_oracle(ctx_len):
    print(f"case select_topn ctx_len={ctx_len}", flush=True)
    rng = np.random.default_rng(ctx_len)
    n_req, Lq = 2, 5
    scores = (np.round(rng.standard_normal((n_req, ctx_len)) * 16) / 16).astype(np.float32)
    scores[1, ::7] = scores[1, 3]   # a long run of equal scores in the second request
    N = O.select_count(15, 100, ctx_len)
    dev = torch.from_numpy(scores).cuda()
    rp = torch.full((n_req, N + Lq), -7, dtype=torch.int32, device="cuda")
    sra.select_topn(dev, N, None, None, Lq, rp)
    got = rp.cpu().numpy()
    for q in range(n_req):
        np.testing.assert_array_equal(got[q][:N], O.select_topn(scores[q], N), err_msg=f"request {q}")
        np.testing.assert_array_equal(got[q][N:], ctx_len + np.arange(Lq))


@pytest.mark.parametrize("ctx_len", [3000, 20000])
def test_select_topn_signed_zeros_tie(ctx_len):
    """-0 and +0 are equal scores: with the N-th score at zero, the lowest positions among zeros of
    either sign are taken."""
    print(f"case select_topn signed zeros ctx_len={ctx_len}", flush=True)
    rng = np.random.default_rng(ctx_len + 1)
    n_req, Lq = 2, 3
    scores = rng.choice(np.array([-1.0, -0.0, 0.0, 1.0], dtype=np.float32), size=(n_req, ctx_len))
    N = int((scores[0] > 0).sum()) + ctx_len // 20   # the N-th score of request 0 is a zero
    dev = torch.from_numpy(scores).cuda()
    rp = torch.full((n_req, N + Lq), -7, dtype=torch.int32, device="cuda")
    sra.select_topn(dev, N, None, None, Lq, rp)
    got = rp.cpu().numpy()
    for q in range(n_req):
        np.testing.assert_array_equal(got[q][:N], O.select_topn(scores[q], N), err_msg=f"request {q}")


@pytest.mark.parametrize("ctx_len,n_prev", [(17920, 3584), (17920, 9000), (40000, 36000)])
def test_select_topn_nested_matches_oracle(ctx_len, n_prev):
    """Levels selected among an earlier Top-n_prev (from the oracle) equal the oracle's Top-N_l of the
    whole context; among an arbitrary ascending subset they are the subset's own Top-N_l. n_prev spans
    the kernel's register, LDS and global-memory key paths."""
    print(f"case select_topn_nested ctx_len={ctx_len} n_prev={n_prev}", flush=True)
    rng = np.random.default_rng(ctx_len + n_prev)
    n_req, Lq = 2, 5
    scores = (np.round(rng.standard_normal((n_req, ctx_len)) * 16) / 16).astype(np.float32)
    scores[1, ::7] = scores[1, 3]
    levels = [n_prev, n_prev - 1, (3 * n_prev) // 4, n_prev // 2 + 1, 1, 0]
    dev = torch.from_numpy(scores).cuda()
    qrows = ctx_len + np.arange(Lq)
    for kind in ("top", "subset"):
        if kind == "top":
            prev = np.stack([O.select_topn(scores[q], n_prev) for q in range(n_req)])
        else:
            prev = np.stack([np.sort(rng.choice(ctx_len, n_prev, replace=False)) for _ in range(n_req)])
        prev_full = np.concatenate([prev, np.tile(qrows, (n_req, 1))], axis=1).astype(np.int32)
        prev_dev = torch.from_numpy(prev_full).cuda()
        outs = [torch.full((n_req, n + Lq), -7, dtype=torch.int32, device="cuda") for n in levels]
        sra.select_topn_nested(dev, prev_dev, n_prev, Lq, levels, outs)
        for n, o in zip(levels, outs):
            got = o.cpu().numpy()
            for q in range(n_req):
                if kind == "top":
                    want = O.select_topn(scores[q], n)
                else:
                    want = prev[q][O.select_topn(scores[q][prev[q]], n)]
                np.testing.assert_array_equal(got[q][:n], want, err_msg=f"{kind} level N={n} request {q}")
                np.testing.assert_array_equal(got[q][n:], qrows)
