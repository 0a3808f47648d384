"""GPU parity of the Turbo8 KV path (qsa_gated_attention and qsa_append_kv on
a Turbo8 cache) through the C ABI against the oracle's Turbo8 path.

Outputs: the bf16 bar (max-abs 2e-2, rel-L2 5e-3).  Appended rows: the GPU
quantizes its own fp32 row (norm, rotation and WHT in fp32) with the same rule
as the oracle, which quantizes the exact row rounded to fp32, so a code or a
scale can land one step apart where the two sit on either side of a rounding
boundary: every decoded value is within one E4M3 step (times its scale) plus
one bf16 step of the scale of the oracle's, and nearly all codes are equal.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_gqa_attention_amd import binding
from gated_gqa_attention_amd.session import Session
from gated_gqa_attention_amd.workloads import WORKLOADS, Workload, make_turbo8_inputs, to_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def geo(w):
    return oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rotary_dim, w.rope_theta, w.rms_eps, 0.0, w.dtype)


def check_out(got, ref, what):
    got = got.float().cpu().double().numpy()
    assert np.all(np.isfinite(got)), what
    err = float(np.max(np.abs(got - ref)))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    say(f"  {what}: max_abs={err:.3g} rel_l2={rel:.3g}")
    assert err <= 2e-2 and rel <= 5e-3, what


def check_new_rows(sess, inp, new, w):
    """The appended rows (codes x scales) against the oracle's quantized new rows."""
    kc, ks, vc, vs = new
    same = total = 0
    for b in range(w.batch):
        s0 = int(inp["seq_offset"][b]) + int(inp["seq_lens"][b])
        for name, oc, osc in (("k", kc, ks), ("v", vc, vs)):
            gc = sess.dev[f"{name}_codes"][s0:s0 + w.q_len].cpu().numpy()
            gs = sess.dev[f"{name}_scales"][s0:s0 + w.q_len].cpu().view(torch.int16).numpy().view(np.uint16)
            gd = oracle.turbo8_dequantize(gc, gs)
            od = oracle.turbo8_dequantize(oc[b], osc[b])
            s = np.repeat((osc[b].astype(np.uint32) << 16).view(np.float32).astype(np.float64), 16, axis=-1)
            q = np.abs(od / np.where(s > 0, s, 1))
            step = np.where(q >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(q, 1e-300))) - 3), 2.0 ** -9) * s
            assert np.all(np.abs(gd - od) <= step + 2.0 ** -7 * np.abs(od) + 1e-30), f"{name} rows of sequence {b}"
            same += int(np.sum(gc == oc[b]))
            total += gc.size
    say(f"  appended codes equal to the oracle's: {same / total:.4f}")
    assert same >= 0.97 * total


CASES = [
    (WORKLOADS["decode_4b"], 0),
    (WORKLOADS["verify_24x2"].with_(prior=600), 0),
    (Workload("t8_ragged", batch=5, q_len=1, num_q_heads=16, num_kv_heads=4, head_dim=256, rotary_dim=64,
              rope_theta=1e7, dtype="bf16", prior=0, seed=151, ragged=(100, 5000)), 0),
    (Workload("t8_d128_l16", batch=2, q_len=16, num_q_heads=3, num_kv_heads=1, head_dim=128, rotary_dim=32,
              rope_theta=1e6, dtype="bf16", prior=150, seed=152), 3),
    (Workload("t8_d64", batch=3, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=64, rotary_dim=16,
              rope_theta=1e4, dtype="bf16", prior=0, seed=153, ragged=(0, 300)), 1),
    (WORKLOADS["decode_4b"].with_(prior=700, batch=2), 1),   # one chunk of 11 stages
]


@pytest.mark.parametrize("w,splits", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_turbo8_attention_matches_the_oracle(w, splits):
    for variant in ("graded", "stress"):
        inp = make_turbo8_inputs(w, variant=variant)
        say(f"case turbo8 {w.name} splits={splits} {variant}")
        sess = Session(w, inp, force_splits=splits)
        say(f"  plan {sess.plan()}")
        out = sess.run()
        torch.cuda.synchronize()
        assert sess.device_error() == 0
        ref, new = oracle.turbo8_gated_attention(geo(w), inp)
        check_out(out, ref, f"{w.name}/{variant}")
        check_new_rows(sess, inp, new, w)


@pytest.mark.parametrize("w", [WORKLOADS["verify_24x2"].with_(prior=300), WORKLOADS["decode_4b"]],
                         ids=lambda w: w.name)
def test_turbo8_append_then_attend_equals_fused(w):
    """qsa_append_kv quantizes the new rows exactly as the fused call does, and
    the unfused call attends them the same way: bitwise equal caches and outputs."""
    inp = make_turbo8_inputs(w, variant="stress")
    say(f"case turbo8 append+attend {w.name}")
    fused = Session(w, inp)
    a = fused.run().clone()
    split = Session(w, inp)
    split.append()
    b = split.run(fused=False).clone()
    torch.cuda.synchronize()
    for k in ("k_codes", "k_scales", "v_codes", "v_scales"):
        assert torch.equal(fused.dev[k], split.dev[k]), k
    assert torch.equal(a, b)


def test_turbo8_unsupported_combinations_are_refused():
    w = WORKLOADS["decode_4b"].with_(q_len=40, prior=64)       # tile route
    inp = make_turbo8_inputs(w)
    with pytest.raises(binding.QSAError) as e:
        Session(w, inp).run()
    assert e.value.code == binding.QSA_ERR_UNSUPPORTED
