"""GatedDeltaNet decode on the GPU (qsa_gdn_decode) against the CPU oracle
(oracle/gdn.py), element by element.

Bars: y (fp32 arithmetic, one rounding to bf16) element by element within
2^-8 |y_ref| + 1e-4 (the rounding's bound, bf16 keeping 8 significant bits,
plus fp32 arithmetic) and rel-L2 5e-3 overall.  The gated norm puts |y| up to
about 15 (o / rms(o) times norm_weight times silu(z)), where one bf16 ulp is
0.0625, so the attention core's absolute 2e-2 bar does not carry over.  The
updated fp32 state within rel-L2 1e-5 and max-abs 1e-5 of its largest
magnitude; the updated conv state bit-exact (it only moves stored values and
the new bf16 input, which fp32 holds exactly).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gated_gqa_attention_amd import binding
from gated_gqa_attention_amd.workloads import GDN_WORKLOADS, GdnWorkload, make_gdn_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _oracle():
    from oracle import gdn
    return gdn


def run_gpu(w: GdnWorkload, x: dict) -> dict:
    d = {k: v.to(DEV).contiguous() for k, v in x.items()}
    y = torch.full((w.batch, w.num_v_heads, w.v_head_dim), float("nan"), dtype=torch.bfloat16, device=DEV)
    cfg = binding.make_gdn_cfg(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads,
                               k_head_dim=w.k_head_dim, v_head_dim=w.v_head_dim, conv_kernel=w.conv_kernel,
                               rms_eps=w.rms_eps)
    binding.gdn_decode(cfg, d["qkv"], d["z"], d["a"], d["b"], d["conv_w"], d["a_log"], d["dt_bias"], d["norm_w"],
                       d["conv_state"], d["state"], y)
    torch.cuda.synchronize()
    return {"y": y.float().cpu().numpy().astype(np.float64), "conv_state": d["conv_state"].cpu().numpy(),
            "state": d["state"].cpu().numpy().astype(np.float64)}


def check(w: GdnWorkload, got: dict, ref: dict, tag: str):
    y, ry = got["y"], ref["y"]
    assert np.isfinite(y).all(), f"{tag}: non-finite y"
    rel = np.linalg.norm(y - ry) / np.linalg.norm(ry)
    mab = np.abs(y - ry).max()
    excess = (np.abs(y - ry) - (2.0 ** -8 * np.abs(ry) + 1e-4)).max()
    s, rs = got["state"], ref["state"]
    srel = np.linalg.norm(s - rs) / np.linalg.norm(rs)
    smab = np.abs(s - rs).max() / np.abs(rs).max()
    print(f"  {tag}: y max_abs={mab:.3g} rel_l2={rel:.3g} bound_excess={excess:.3g}; "
          f"state rel_l2={srel:.3g} max_rel={smab:.3g}", flush=True)
    assert excess <= 0 and rel <= 5e-3, tag
    assert srel <= 1e-5 and smab <= 1e-5, tag
    np.testing.assert_array_equal(got["conv_state"], ref["conv_state"].astype(np.float32), err_msg=tag)


CASES = [
    GDN_WORKLOADS["gdn_small"],
    GdnWorkload("r1_k3", batch=2, num_k_heads=3, num_v_heads=3, conv_kernel=3, seed=51),
    GdnWorkload("r4_k1", batch=2, num_k_heads=1, num_v_heads=4, conv_kernel=1, seed=52),
    GdnWorkload("r2_k2_b5", batch=5, num_k_heads=2, num_v_heads=4, conv_kernel=2, seed=53),
    GDN_WORKLOADS["gdn_decode_4b_b1"],
    GDN_WORKLOADS["gdn_decode_4b"],
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_gdn_decode_matches_the_oracle(w):
    print(f"case gdn {w.name} B={w.batch} Hk={w.num_k_heads} Hv={w.num_v_heads} K={w.conv_kernel}", flush=True)
    x = make_gdn_inputs(w)
    ref = _oracle().gdn_decode(x, w.num_k_heads, w.num_v_heads, w.k_head_dim, w.v_head_dim, w.rms_eps)
    check(w, run_gpu(w, x), ref, w.name)


def test_gdn_three_steps_carry_the_states():
    """Three tokens in a row: each call's updated states are the next call's."""
    w = GDN_WORKLOADS["gdn_small"]
    print("case gdn three steps", flush=True)
    x = make_gdn_inputs(w)
    cur_gpu = {k: v.clone() for k, v in x.items()}
    cur_ref = {k: v.clone() for k, v in x.items()}
    for step in range(3):
        fresh = make_gdn_inputs(w, seed=100 + step)
        for k in ("qkv", "z", "a", "b"):
            cur_gpu[k] = fresh[k]
            cur_ref[k] = fresh[k]
        got = run_gpu(w, cur_gpu)
        ref = _oracle().gdn_decode(cur_ref, w.num_k_heads, w.num_v_heads, w.k_head_dim, w.v_head_dim, w.rms_eps)
        check(w, got, ref, f"step {step}")
        cur_gpu["conv_state"] = torch.from_numpy(got["conv_state"])
        cur_gpu["state"] = torch.from_numpy(got["state"].astype(np.float32))
        cur_ref["conv_state"] = torch.from_numpy(ref["conv_state"].astype(np.float32))
        cur_ref["state"] = torch.from_numpy(ref["state"].astype(np.float32))


def test_gdn_degenerate_inputs():
    """Zero state (first token), a gate that empties the state (strong decay), and
    beta near 1 and near 0."""
    w = GDN_WORKLOADS["gdn_small"]
    print("case gdn degenerate", flush=True)
    x = make_gdn_inputs(w)
    x["state"] = torch.zeros_like(x["state"])
    x["conv_state"] = torch.zeros_like(x["conv_state"])
    ref = _oracle().gdn_decode(x, w.num_k_heads, w.num_v_heads, w.k_head_dim, w.v_head_dim, w.rms_eps)
    check(w, run_gpu(w, x), ref, "zero states")
    x = make_gdn_inputs(w)
    a = x["a"].float()
    a[:, 0] = 30.0                                     # softplus ~ 30: exp(g) underflows to 0
    bb = x["b"].float()
    bb[:, 1] = 40.0                                    # beta = 1
    bb[:, 2] = -40.0                                   # beta ~ 0
    x["a"], x["b"] = a.to(torch.bfloat16), bb.to(torch.bfloat16)
    ref = _oracle().gdn_decode(x, w.num_k_heads, w.num_v_heads, w.k_head_dim, w.v_head_dim, w.rms_eps)
    check(w, run_gpu(w, x), ref, "extreme gates")


def test_gdn_empty_batch_is_a_no_op():
    w = GDN_WORKLOADS["gdn_small"].with_(batch=0)
    x = make_gdn_inputs(GDN_WORKLOADS["gdn_small"])
    d = {k: v.to(DEV) for k, v in x.items()}
    y = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    cfg = binding.make_gdn_cfg(batch=0, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads,
                               k_head_dim=128, v_head_dim=128, conv_kernel=4)
    before = d["state"].clone()
    binding.gdn_decode(cfg, d["qkv"], d["z"], d["a"], d["b"], d["conv_w"], d["a_log"], d["dt_bias"], d["norm_w"],
                       d["conv_state"], d["state"], y)
    torch.cuda.synchronize()
    assert torch.equal(before, d["state"])
