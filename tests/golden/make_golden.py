"""Writes tests/golden/tiny_f32_fingerprint.json from the oracle alone (no HIP code involved).

Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from workloads import make_workload  # noqa: E402


def main():
    w = make_workload(0)
    lay = w.layer(0)
    c = w.cfg
    r = O.fused_layer(k_store=lay["k_store"], v_store=lay["v_store"], chunks=w.chunks[0], L=c.total_len,
                      q_new=lay["q_new"][0], k_new=lay["k_new"][0], v_new=lay["v_new"][0], dtype="f32",
                      base=c.rope_base, n_kv_heads=c.n_kv_heads, q_crit=w.q_crit[0], k_crit_store=w.k_crit,
                      n_select=O.select_count(15, 100, c.ctx_len))
    out = {
        "workload": "tiny_f32 (4 Q / 2 KV heads, d 64, 3 x 128 context + 16 query, 15% selected), seed 0",
        "row_pos": r["row_pos"].tolist(),
        "anchors": O.extract_anchors(w.k_crit, w.chunks[0], 4, "f32").tolist(),
        "scores_head": r["scores"][:8].tolist(),
        "out_sum": float(np.sum(r["out"])),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_fingerprint.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
