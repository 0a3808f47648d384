"""GPU parity of the projections around the core (qsa_qkv_proj, qsa_o_proj)
through the C ABI against the oracle.

Both round a sum of K products once to bf16: the GPU sums in fp32 (in its own
order), the oracle in double.  So every GPU output is the bf16 rounding of a
value within K 2^-24 sum_k |x_k w_k| (the fp32 summation error bound) of the
exact sum: it lies within half a bf16 unit in the last place of itself plus
that bound from the oracle's unrounded sum.  The graded bf16 bar holds over all
outputs as well.  Outputs are preset to NaN and written into larger buffers,
so that a missed or stray store shows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_gqa_attention_amd import binding
from gated_gqa_attention_amd.workloads import HIDDEN_4B, WORKLOADS, Workload, make_proj_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def geo(w):
    return oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rotary_dim, w.rope_theta, w.rms_eps, 0.0, w.dtype)


def cfg_of(w):
    return binding.make_cfg(batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads,
                            num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, rotary_dim=w.rotary_dim,
                            rope_theta=w.rope_theta, rms_eps=w.rms_eps, dtype=torch.bfloat16,
                            max_seq_len=w.q_len, q_norm_w=1, k_norm_w=1)


def check(got, ref, exact, absum, K, what):
    """ref: the oracle's bf16 outputs; exact: its unrounded sums; absum: sum_k |x_k w_k|."""
    got = got.float().cpu().double().numpy().reshape(ref.shape)
    exact, absum = exact.reshape(ref.shape), absum.reshape(ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: unwritten (NaN) outputs"
    diff = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    say(f"  {what}: max_abs={diff.max():.3g} rel_l2={rel:.3g} exact={np.mean(diff == 0):.4f}")
    mag = np.maximum(np.abs(got), 1e-38)
    half_ulp = np.exp2(np.floor(np.log2(mag)) - 8)
    assert np.all(np.abs(got - exact) <= half_ulp + K * 2.0 ** -24 * absum), what
    assert diff.max() <= 2e-2 and rel <= 5e-3, what


def padded(shape, dev, pad=4096):
    """A NaN-filled tensor of `shape` at the front of a larger NaN buffer."""
    n = int(np.prod(shape))
    buf = torch.full((n + pad,), float("nan"), dtype=torch.bfloat16, device=dev)
    return buf, buf[:n].view(shape)


CASES = [
    (WORKLOADS["decode_4b"], HIDDEN_4B),                 # 1 row, 4B geometry (one wavefront per feature)
    (WORKLOADS["decode_4b"].with_(batch=2), HIDDEN_4B),  # 2 rows
    (WORKLOADS["decode_4b"].with_(batch=4), 8192),       # 4 rows, 16 pieces of 512 per weight row
    (WORKLOADS["decode_4b"].with_(batch=3), 1536),       # 3 rows, 3 pieces: registers sized for 4, one unused
    (WORKLOADS["decode_4b"].with_(batch=5), 512),        # 5 rows: the MFMA kernel
    (WORKLOADS["verify_24x2"], 2048),                    # 32 rows, 24 / 2 heads
    (WORKLOADS["decode_4b"].with_(batch=2, q_len=3), 1024),  # 6 rows
    (WORKLOADS["decode_4b"].with_(batch=16, q_len=4), 512),  # 64 rows, the most a call takes
    (Workload("proj_d64", batch=3, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=64, rotary_dim=16,
              rope_theta=1e4, dtype="bf16", prior=0, seed=61), 256),
    (Workload("proj_d128", batch=1, q_len=17, num_q_heads=6, num_kv_heads=1, head_dim=128, rotary_dim=32,
              rope_theta=1e6, dtype="bf16", prior=0, seed=62), 768),
]


@pytest.mark.parametrize("w,hidden", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_qkv_and_o_projections_match_the_oracle(w, hidden):
    dev = torch.device("cuda")
    say(f"case projections {w.name} rows={w.batch * w.q_len} hidden={hidden}")
    p = make_proj_inputs(w, hidden=hidden)
    g = geo(w)
    cfg = cfg_of(w)
    B, L, Hq, Hkv, D = w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim
    x, wqkv, wo = p["x"].to(dev), p["w_qkv"].to(dev), p["w_o"].to(dev)
    bq, q_gate = padded((B, L, Hq, 2 * D), dev)
    bk, k_new = padded((B, L, Hkv, D), dev)
    bv, v_new = padded((B, L, Hkv, D), dev)
    binding.qkv_proj(cfg, x, wqkv, hidden, q_gate, k_new, v_new)
    attn = torch.randn((B * L, Hq * D), generator=torch.Generator().manual_seed(w.seed)).to(torch.bfloat16)
    by, y = padded((B * L, hidden), dev)
    binding.o_proj(cfg, attn.to(dev), wo, hidden, y)
    torch.cuda.synchronize()
    g64 = geo(w.with_(dtype="f64"))
    rq, rk, rv = oracle.qkv_proj(g, hidden, p["x"], p["w_qkv"])
    eq, ek, ev = oracle.qkv_proj(g64, hidden, p["x"], p["w_qkv"])
    aq, ak, av = oracle.qkv_proj(g64, hidden, p["x"].double().abs(), p["w_qkv"].double().abs())
    check(q_gate, rq, eq, aq, hidden, "q_gate")
    check(k_new, rk, ek, ak, hidden, "k_new")
    check(v_new, rv, ev, av, hidden, "v_new")
    K = Hq * D
    check(y, oracle.o_proj(g, hidden, attn, p["w_o"]), oracle.o_proj(g64, hidden, attn, p["w_o"]),
          oracle.o_proj(g64, hidden, attn.double().abs(), p["w_o"].double().abs()), K, "o_proj")
    for buf, out in ((bq, q_gate), (bk, k_new), (bv, v_new), (by, y)):
        assert torch.isnan(buf[out.numel():]).all(), "store past the output"


def test_projection_limits_are_refused():
    w = WORKLOADS["decode_4b"].with_(batch=65)
    cfg = cfg_of(w)
    dev = torch.device("cuda")
    t = torch.zeros(16, dtype=torch.bfloat16, device=dev)
    with pytest.raises(binding.QSAError) as e:
        binding.qkv_proj(cfg, t, t, 2560, t, t, t)
    assert e.value.code == binding.QSA_ERR_UNSUPPORTED
    with pytest.raises(binding.QSAError) as e:
        binding.o_proj(cfg_of(WORKLOADS["decode_4b"]), t, t, 2500, t)
    assert e.value.code == binding.QSA_ERR_UNSUPPORTED
