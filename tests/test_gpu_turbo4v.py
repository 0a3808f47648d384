"""GPU parity of the bf16-K / Turbo4-V cache path (qsa_gated_attention and
qsa_append_kv with kv_dtype QSA_KV_BF16K_TURBO4V) through the C ABI against the
oracle's path.

Outputs: the bf16 bar (max-abs 2e-2, rel-L2 5e-3), the oracle reading the same
stored rows.  Appended rows: K is the bf16 cache's row, within one bf16 ulp of
the oracle's (fp32 norm and rotation against double, each rounded once).  V is
quantized by the GPU from its own fp32 WHT of the row with the same rule as the
oracle, which works in double: an index or a scale can land one step apart
where the two sit on either side of a decision threshold, so nearly all (not
all) indices and scales must be equal, and the decoded rows close.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_gqa_attention_amd import binding
from gated_gqa_attention_amd.session import Session
from gated_gqa_attention_amd.workloads import WORKLOADS, Workload, make_turbo4v_inputs

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
    kr, vc, vs = new
    same_c = same_s = total_c = total_s = 0
    for b in range(w.batch):
        s0 = int(inp["seq_offset"][b]) + int(inp["seq_lens"][b])
        gk = sess.dev["k_cache"][s0:s0 + w.q_len].float().cpu().double().numpy()
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(kr[b]), 1e-30))) - 7)
        assert np.all(np.abs(gk - kr[b]) <= ulp), f"K rows of sequence {b}"
        gc = sess.dev["v_codes"][s0:s0 + w.q_len].cpu().numpy()
        gs = sess.dev["v_scales"][s0:s0 + w.q_len].cpu().numpy()
        same_c += int(np.sum((gc & 15) == (vc[b] & 15)) + np.sum((gc >> 4) == (vc[b] >> 4)))
        total_c += 2 * gc.size
        same_s += int(np.sum(gs == vs[b]))
        total_s += gs.size
        gd, od = oracle.turbo4_dequantize(gc, gs), oracle.turbo4_dequantize(vc[b], vs[b])
        assert np.linalg.norm(gd - od) <= 2e-2 * np.linalg.norm(od), f"V rows of sequence {b}"
    say(f"  appended V indices equal to the oracle's: {same_c / total_c:.4f}, scales: {same_s / total_s:.4f}")
    assert same_c >= 0.99 * total_c and same_s >= 0.97 * total_s


CASES = [
    (WORKLOADS["decode_4b"], 0),
    (WORKLOADS["verify_24x2"].with_(prior=600), 0),
    (Workload("t4_ragged", batch=5, q_len=1, num_q_heads=16, num_kv_heads=4, head_dim=256, rotary_dim=64,
              rope_theta=1e7, dtype="bf16", prior=0, seed=161, ragged=(100, 5000)), 0),
    (Workload("t4_l16", batch=2, q_len=16, num_q_heads=2, num_kv_heads=2, head_dim=256, rotary_dim=64,
              rope_theta=1e6, dtype="bf16", prior=150, seed=162), 3),
    (WORKLOADS["decode_4b"].with_(prior=700, batch=2), 1),   # one chunk of 11 stages
]


@pytest.mark.parametrize("w,splits", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_turbo4v_attention_matches_the_oracle(w, splits):
    for variant in ("graded", "stress"):
        inp = make_turbo4v_inputs(w, variant=variant)
        say(f"case bf16k_turbo4v {w.name} splits={splits} {variant}")
        sess = Session(w, inp, force_splits=splits)
        say(f"  plan {sess.plan()}")
        out = sess.run()
        torch.cuda.synchronize()
        assert sess.device_error() == 0
        # the oracle reads the same cached rows; its new rows are its own
        ref, new = oracle.bf16k_turbo4v_gated_attention(geo(w), inp)
        check_out(out, ref, f"{w.name}/{variant}")
        check_new_rows(sess, inp, new, w)


@pytest.mark.parametrize("w", [WORKLOADS["verify_24x2"].with_(prior=300), WORKLOADS["decode_4b"]],
                         ids=lambda w: w.name)
def test_turbo4v_append_then_attend_equals_fused(w):
    """qsa_append_kv writes the new rows exactly as the fused call does, and the
    unfused call attends them the same way: bitwise equal caches and outputs."""
    inp = make_turbo4v_inputs(w, variant="stress")
    say(f"case bf16k_turbo4v append+attend {w.name}")
    fused = Session(w, inp)
    a = fused.run().clone()
    split = Session(w, inp)
    split.append()
    b = split.run(fused=False).clone()
    torch.cuda.synchronize()
    for k in ("k_cache", "v_codes", "v_scales"):
        assert torch.equal(fused.dev[k], split.dev[k]), k
    assert torch.equal(a, b)


def test_turbo4v_unsupported_combinations_are_refused():
    for w in (WORKLOADS["decode_4b"].with_(q_len=40, prior=64),                     # tile route
              WORKLOADS["decode_4b"].with_(head_dim=128, rotary_dim=32, prior=64)):  # head_dim 256 only
        inp = make_turbo4v_inputs(w)
        with pytest.raises(binding.QSAError) as e:
            Session(w, inp).run()
        assert e.value.code == binding.QSA_ERR_UNSUPPORTED
