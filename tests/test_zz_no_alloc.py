"""The allocation-free entry point (qsa_gated_attention_noalloc) against
qsa_gated_attention with a caller workspace, through the C ABI: two calls in a
row on the library's per-GPU scratch, the second with a smaller input.  Both
calls take the same kernels and plan, so the outputs and the appended cache
rows must be bitwise equal; each is also checked against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_gqa_attention_amd import binding
from gated_gqa_attention_amd.session import Session
from gated_gqa_attention_amd.workloads import WORKLOADS, make_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def geo(w):
    return oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rotary_dim, w.rope_theta, w.rms_eps, 0.0, w.dtype)


def noalloc_call(w, inp):
    """The same call as Session.run, through the allocation-free entry point, on
    fresh device copies of the inputs (so that both paths append to their own cache)."""
    sess = Session(w, inp)
    d = sess.dev
    out = torch.full_like(sess.out, float("nan"))
    cfg = sess.cfg
    cfg.workspace, cfg.workspace_bytes = None, 0       # ignored by this entry point
    binding.gated_attention_noalloc(cfg, sess.kv, d["q_gate"], d["k_new"], d["v_new"], d["seq_lens"],
                                    d["positions"], out)
    return out, sess


def test_noalloc_matches_workspace_call_twice_second_smaller():
    first = WORKLOADS["verify_24x2"]                    # 12 MiB of split-K partials
    second = WORKLOADS["decode_4b"].with_(prior=1500)   # smaller: 1 MiB, other plan
    for w in (first, second):
        say(f"case noalloc {w.name} prior={w.prior}")
        inp = make_inputs(w)
        ref_sess = Session(w, inp)
        say(f"  plan {ref_sess.plan()}")
        ref = ref_sess.run().clone()
        out, sess = noalloc_call(w, inp)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(sess.dev["k_cache"], ref_sess.dev["k_cache"])
        assert torch.equal(sess.dev["v_cache"], ref_sess.dev["v_cache"])
        want, _, _ = oracle.gated_attention(geo(w), inp)
        got = out.float().cpu().double().numpy()
        assert np.all(np.isfinite(got))
        assert float(np.max(np.abs(got - want))) <= 2e-2 and rel_l2(got, want) <= 5e-3


def test_noalloc_rejects_a_plan_larger_than_its_scratch():
    w = WORKLOADS["prefill_4b"].with_(q_len=12288)     # 96 MiB of prepared queries
    inp = make_inputs(w.with_(prior=64))                 # a short cache; only the plan's size matters here
    sess = Session(w.with_(prior=64), inp, max_seq_len=w.prior + w.q_len)
    need = binding.workspace_size(sess.cfg)
    say(f"case noalloc too large: needs {need} bytes")
    if need <= binding.NOALLOC_SCRATCH_BYTES:
        pytest.skip("this shape fits the scratch")
    out = torch.empty_like(sess.out)
    with pytest.raises(binding.QSAError) as e:
        binding.gated_attention_noalloc(sess.cfg, sess.kv, sess.dev["q_gate"], sess.dev["k_new"],
                                        sess.dev["v_new"], sess.dev["seq_lens"], sess.dev["positions"], out)
    assert e.value.code == binding.QSA_ERR_WORKSPACE
