"""Write tests/golden/tiny_f32_oracle.json: the oracle's output on the seeded
tiny fp32 workload (4 query / 1 KV head, head_dim 64, rotary_dim 16, theta 1e4,
32 cached tokens).  Calls only the oracle and the seeded input generators; the
pages print no numeric example, so this fixture is a regression pin on the
oracle itself (any later change to its arithmetic shows up here).

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gated_gqa_attention_amd.workloads import WORKLOADS, make_inputs  # noqa: E402


def compute():
    w = WORKLOADS["tiny_f32"]
    g = oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                        w.rotary_dim, w.rope_theta, w.rms_eps, 0.0, w.dtype)
    out, kr, vr = oracle.gated_attention(g, make_inputs(w))
    return out, kr, vr


if __name__ == "__main__":
    out, kr, vr = compute()
    doc = {
        "_about": "oracle output for workload tiny_f32 (seed 1), fp32 storage; written by make_golden.py",
        "out": [float(x).hex() for x in out.reshape(-1)],
        "k_row": [float(x).hex() for x in kr.reshape(-1)],
        "v_row": [float(x).hex() for x in vr.reshape(-1)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", path)
