"""Pins for the oracle's projections around the core (no GPU).

The fused q/k/v projection and o_proj are plain linear layers; what is
particular is the layout: the doubled q_proj output holds per head the query
half and then the gate half, and the fused weight stacks q_proj, k_proj and
v_proj (mlxd PR #99 Summary; Atlas FullAttentionLayer and Qwen35Kernels
qkv_split).  Pinned against a library matmul, against exact selections, and
end to end against transformers' Qwen3.5 attention layer with random
projection weights.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_gqa_attention_amd.workloads import WORKLOADS, Workload, make_inputs, make_proj_inputs


def geo(w, dtype=None):
    return oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rotary_dim, w.rope_theta, w.rms_eps, 0.0, dtype or w.dtype)


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


def test_linear_matches_library_matmul():
    rng = np.random.default_rng(3)
    x, w = rng.standard_normal((5, 96)), rng.standard_normal((40, 96))
    assert np.max(np.abs(oracle.linear(x, w) - x @ w.T)) < 1e-12
    # rounding to bf16 is the oracle's round to nearest even of the double result
    assert np.array_equal(oracle.linear(x, w, "bf16"), oracle.round_to(x @ w.T, "bf16"))


def test_qkv_split_routes_each_feature():
    """With a weight that selects input feature perm[n] for output feature n, the
    three outputs are exact slices of x: q_gate[.., h, :D] the query rows of head
    h, q_gate[.., h, D:] its gate rows, then k_new, then v_new."""
    w = Workload("route", batch=2, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=8, rotary_dim=0,
                 rope_theta=1e4, dtype="f32", prior=0, seed=1)
    D, Hq, Hkv = 8, 4, 2
    n = 2 * Hq * D + 2 * Hkv * D
    hidden = n + 5
    rng = np.random.default_rng(4)
    perm = rng.permutation(hidden)[:n]
    wq = np.zeros((n, hidden))
    wq[np.arange(n), perm] = 1.0
    x = rng.standard_normal((4, hidden))
    qg, kn, vn = oracle.qkv_proj(geo(w, "f64"), hidden, x, wq)
    sel = x[:, perm]
    for h in range(Hq):
        assert np.array_equal(qg.reshape(4, Hq, 2 * D)[:, h, :D], sel[:, h * 2 * D:h * 2 * D + D])
        assert np.array_equal(qg.reshape(4, Hq, 2 * D)[:, h, D:], sel[:, h * 2 * D + D:(h + 1) * 2 * D])
    assert np.array_equal(kn.reshape(4, -1), sel[:, 2 * Hq * D:2 * Hq * D + Hkv * D])
    assert np.array_equal(vn.reshape(4, -1), sel[:, 2 * Hq * D + Hkv * D:])


def _hf_block(w: Workload, inp: dict, proj: dict, hidden: int):
    """transformers' Qwen3_5Attention (float64) with the given projection weights."""
    from transformers import DynamicCache
    from transformers.models.qwen3_5 import modeling_qwen3_5 as M
    from transformers.models.qwen3_5.configuration_qwen3_5 import Qwen3_5TextConfig

    B, L, Hq, Hkv, D, r = w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim, w.rotary_dim
    half = r // 2
    sec = [half - 2 * (half // 3), half // 3, half // 3]
    cfg = Qwen3_5TextConfig(
        hidden_size=hidden, num_attention_heads=Hq, num_key_value_heads=Hkv, head_dim=D,
        rope_parameters={"rope_type": "default", "rope_theta": w.rope_theta,
                         "partial_rotary_factor": r / D, "mrope_section": sec},
        rms_norm_eps=w.rms_eps, attention_bias=False, num_hidden_layers=1, layer_types=["full_attention"])
    cfg._attn_implementation = "eager"
    att = M.Qwen3_5Attention(cfg, 0).double()
    wqkv = proj["w_qkv"].double()
    nq, nk = Hq * 2 * D, Hkv * D
    with torch.no_grad():
        att.q_proj.weight.copy_(wqkv[:nq])
        att.k_proj.weight.copy_(wqkv[nq:nq + nk])
        att.v_proj.weight.copy_(wqkv[nq + nk:])
        att.o_proj.weight.copy_(proj["w_o"].double())
        att.q_norm.weight.copy_(inp["w_q"].double() - 1)
        att.k_norm.weight.copy_(inp["w_k"].double() - 1)
    rot = M.Qwen3_5TextRotaryEmbedding(cfg)
    outs = []
    xs = proj["x"].double().reshape(B, L, hidden)
    for b in range(B):
        n, off = int(inp["seq_lens"][b]), int(inp["seq_offset"][b])
        pos = inp["positions"][b:b + 1].long()
        cos, sin = rot(xs[b:b + 1], pos)
        cache = DynamicCache()
        if n:
            cache.update(inp["k_cache"][off:off + n].double().permute(1, 0, 2)[None],
                         inp["v_cache"][off:off + n].double().permute(1, 0, 2)[None], 0)
        mask = torch.full((L, n + L), float("-inf"), dtype=torch.float64)
        for l in range(L):
            mask[l, :n + l + 1] = 0.0
        with torch.no_grad():
            o, _ = att(xs[b:b + 1], (cos, sin), mask[None, None], past_key_values=cache)
        outs.append(o.reshape(L, hidden).numpy())
    return np.concatenate(outs)


@pytest.mark.parametrize("w", [
    Workload("block_gqa", batch=2, q_len=3, num_q_heads=6, num_kv_heads=2, head_dim=64, rotary_dim=16,
             rope_theta=1e4, dtype="f32", prior=9, seed=41),
    Workload("block_4b_heads", batch=1, q_len=2, num_q_heads=16, num_kv_heads=4, head_dim=256, rotary_dim=64,
             rope_theta=1e7, dtype="f32", prior=5, seed=42),
], ids=lambda w: w.name)
def test_projection_attention_block_matches_transformers(w):
    """x -> fused q/k/v projection (and its split) -> gated attention -> o_proj,
    all in the oracle, equals transformers' Qwen3_5Attention forward with the
    same q_proj / k_proj / v_proj / o_proj weights."""
    hidden = 128
    inp = make_inputs(w)
    proj = make_proj_inputs(w, hidden=hidden)
    g = geo(w, "f64")
    qg, kn, vn = oracle.qkv_proj(g, hidden, proj["x"], proj["w_qkv"])
    x = dict(inp, q_gate=torch.from_numpy(qg), k_new=torch.from_numpy(kn), v_new=torch.from_numpy(vn))
    out, _, _ = oracle.gated_attention(g, x)
    y = oracle.o_proj(g, hidden, out, proj["w_o"])
    ref = _hf_block(w, inp, proj, hidden)
    assert rel_l2(y, ref) < 2e-6                  # transformers keeps its norm and rotary tables in fp32


def test_gate_swapped_in_the_weight_layout_is_caught():
    """Swapping the query and gate rows of each head in w_qkv (a plausible
    layout slip) moves the block output far past the bf16 tolerance."""
    w = WORKLOADS["tiny_f32"].with_(q_len=2, prior=6)
    hidden = 128
    inp = make_inputs(w)
    proj = make_proj_inputs(w, hidden=hidden)
    g = geo(w, "f64")
    D, Hq = w.head_dim, w.num_q_heads
    wq = proj["w_qkv"].double().clone()
    swapped = wq.clone()
    for h in range(Hq):
        a, b = h * 2 * D, h * 2 * D + D
        swapped[a:a + D], swapped[b:b + D] = wq[b:b + D].clone(), wq[a:a + D].clone()
    outs = []
    for ww in (wq, swapped):
        qg, kn, vn = oracle.qkv_proj(g, hidden, proj["x"], ww)
        x = dict(inp, q_gate=torch.from_numpy(qg), k_new=torch.from_numpy(kn), v_new=torch.from_numpy(vn))
        out, _, _ = oracle.gated_attention(g, x)
        outs.append(oracle.o_proj(g, hidden, out, proj["w_o"]))
    assert rel_l2(outs[1], outs[0]) > 10 * 5e-3
