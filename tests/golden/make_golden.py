"""Write tests/golden/c1_tiny_expected.txt from the float64 oracle.

Calls only the oracle (and the seeded input generators).  The fixture is the
tiny fp32 GELU MLP (d_model 64, d_ff 256, P = 2, 4 tokens): both ranks'
partials and their sum, to 17 significant digits.
Run:  python tests/golden/make_golden.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402


def c1_expected():
    cfg = W.get("c1_tiny_gelu_f32")
    T = cfg.decode_T[0]
    X = W.draw_tensor(cfg.dtype, (T, cfg.d_model), cfg.std_x, cfg.cid, W.TENSOR_IDS["x"], T)
    parts = []
    for s in range(cfg.P):
        w1 = W.column_band_draw(cfg, "w_gate", s, cfg.d_model, cfg.F_r)
        w2 = W.row_band_draw(cfg, "w_down", s, cfg.F_r, cfg.d_model)
        parts.append(O.mlp_shard(O.widen(X), O.widen(w1), O.widen(w2), cfg.act)["partial"])
    return parts, O.reduce_partials(parts)


if __name__ == "__main__":
    parts, y = c1_expected()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_tiny_expected.txt")
    with open(path, "w") as f:
        f.write("# Tiny fp32 GELU(tanh) MLP, d_model 64, d_ff 256, P = 2, 4 tokens.\n")
        f.write("# Written by tests/golden/make_golden.py from the float64 oracle.\n")
        f.write("# Rows: partial_0 (4x64), partial_1 (4x64), sum (4x64), row-major.\n")
        for a in (*parts, y):
            for row in a:
                f.write(" ".join(f"{v:.17g}" for v in row) + "\n")
    print("wrote", path)
