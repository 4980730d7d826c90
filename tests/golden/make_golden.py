"""Write oracle_tiny_mha.json from the CPU oracle only (run from the repository root)."""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from bit_quantized_exact_amd.inputs import WORKLOADS, make_qkv  # noqa: E402
from oracle import oracle as O  # noqa: E402

ROWS = [0, 1, 63, 64, 127]


def main():
    w = WORKLOADS["tiny_mha"]
    q, k, v = make_qkv(w)
    out, lse = O.attention(q, k, v, causal=w.causal, rows=ROWS, with_lse=True)
    qz = O.quantize_qk(q, k)
    doc = {
        "workload": "tiny_mha: batch 1, 2 heads, seq 128, head_dim 64, non-causal, seed 0",
        "rows": ROWS,
        "input_sha256": hashlib.sha256(q.tobytes() + k.tobytes() + v.tobytes()).hexdigest(),
        "out": out.tolist(),
        "lse": lse.tolist(),
        "k_mean": qz["k_mean"].tolist(),
        "q_scale": qz["q_scale"].tolist(),
        "k_scale": qz["k_scale"].tolist(),
        "q_i8_row0": qz["q_i8"][0, 0, 0].tolist(),
        "k_i8_row0": qz["k_i8"][0, 0, 0].tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_mha.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
