"""Golden fixtures (no GPU): the pages' printed constants and the oracle regression pin."""
import json
import os

import numpy as np

from gated_gqa_attention_amd.workloads import WORKLOADS
from test_oracle import head_chunk_plan

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_workloads_use_the_pages_geometry():
    g = _load("geometry.json")
    c4b = g["qwen3_5_4b"]
    assert c4b["head_dim"] * c4b["partial_rotary_factor"] == c4b["rotary_dim"]
    assert c4b["q_total"] == c4b["num_heads"] * c4b["head_dim"] * 2
    assert c4b["kv_dim"] == c4b["num_kv_heads"] * c4b["head_dim"]
    for name in ("decode_4b", "ragged_4b", "prefill_4b"):
        w = WORKLOADS[name]
        assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.rotary_dim) == (
            c4b["num_heads"], c4b["num_kv_heads"], c4b["head_dim"], c4b["rotary_dim"])
        assert w.rope_theta == c4b["rope_theta"] and w.rms_eps == c4b["rms_eps"]
    v = g["verify_24x2"]
    w = WORKLOADS["verify_24x2"]
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.q_len) == (
        v["num_heads"], v["num_kv_heads"], v["head_dim"], v["q_len"])
    # the page's verify shape is the chunked case: 4 * 12 > 32 with chunks of 32 // 4 = 8
    assert [len(c) for c in head_chunk_plan(w.q_len, w.num_q_heads, w.num_kv_heads,
                                            g["head_chunk_plan"]["limit"])] == [8, 4, 8, 4]
    rd = g["rope_dims_rule"]
    assert int(rd["head_dim"] * rd["partial_rotary_factor"]) == rd["dims"]


def test_oracle_regression_fixture():
    import sys
    sys.path.insert(0, GOLDEN)
    from make_golden import compute
    out, kr, vr = compute()
    doc = _load("tiny_f32_oracle.json")
    for key, arr in (("out", out), ("k_row", kr), ("v_row", vr)):
        ref = np.array([float.fromhex(x) for x in doc[key]])
        assert ref.shape == arr.reshape(-1).shape
        assert np.max(np.abs(arr.reshape(-1) - ref)) <= 1e-14 * np.max(np.abs(ref))
