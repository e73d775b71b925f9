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
