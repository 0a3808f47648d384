"""Paged KV caches (block table) on the GPU, through the C ABI.

A paged cache holds the same rows as a contiguous one, in blocks placed at
shuffled physical positions (TensorFold issue #503: grow-as-used K/V; Atlas
qwen3_5/mod.rs module doc: paged KV).  The method's result does not depend on
where rows live, and the kernels take the same chunks either way, so a paged
call must equal the contiguous call bitwise: outputs, and every cache row
after the append.  The contiguous call itself is checked against the oracle by
test_gpu_parity; here each paged case is also checked against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_gqa_attention_amd import binding
from gated_gqa_attention_amd.session import Session
from gated_gqa_attention_amd.workloads import WORKLOADS, Workload, make_inputs, paged_rows, to_paged

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def geo(w):
    return oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rotary_dim, w.rope_theta, w.rms_eps, 0.0, w.dtype)


def same_rows(paged_cache, table, bs, contig_cache, inp):
    for b in range(len(inp["seq_lens"])):
        c, o = int(inp["capacity"][b]), int(inp["seq_offset"][b])
        got = paged_rows(paged_cache, table, bs, b, c)
        assert torch.equal(got, contig_cache[o:o + c]), f"cache rows of sequence {b}"


CASES = [
    (WORKLOADS["decode_4b"], 64, 0),                    # one new key in a free ring slot, 64 chunks
    (WORKLOADS["decode_4b"].with_(prior=700, batch=2), 128, 1),   # new rows after 11 cached stages
    (WORKLOADS["verify_24x2"].with_(prior=500), 64, 0),  # three row tiles, new rows from the arena
    (Workload("paged_ragged", batch=6, q_len=1, num_q_heads=16, num_kv_heads=4, head_dim=256, rotary_dim=64,
              rope_theta=1e7, dtype="bf16", prior=0, seed=141, ragged=(3000, 9000)), 64, 0),  # equal-length chunks
    (Workload("paged_l16", batch=2, q_len=16, num_q_heads=3, num_kv_heads=1, head_dim=128, rotary_dim=32,
              rope_theta=1e6, dtype="bf16", prior=250, seed=142), 64, 7),
    (Workload("paged_d64", batch=3, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=64, rotary_dim=16,
              rope_theta=1e4, dtype="bf16", prior=0, seed=143, ragged=(60, 700)), 256, 3),
]


@pytest.mark.parametrize("w,bs,splits", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_paged_equals_contiguous(w, bs, splits):
    inp = make_inputs(w)
    pin = to_paged(inp, bs, seed=w.seed)
    say(f"case paged {w.name} block_size={bs} splits={splits}")
    contig = Session(w, inp, force_splits=splits)
    say(f"  plan {contig.plan()}")
    a = contig.run().clone()
    paged = Session(w, pin, force_splits=splits, block_size=bs)
    b = paged.run().clone()
    torch.cuda.synchronize()
    assert paged.device_error() == 0 and contig.device_error() == 0
    assert torch.equal(a, b)
    same_rows(paged.dev["k_cache"], pin["block_table"], bs, contig.dev["k_cache"], inp)
    same_rows(paged.dev["v_cache"], pin["block_table"], bs, contig.dev["v_cache"], inp)
    ref, _, _ = oracle.gated_attention(geo(w), inp)
    got = b.float().cpu().double().numpy()
    assert np.max(np.abs(got - ref)) <= 2e-2
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 5e-3


@pytest.mark.parametrize("w,bs", [(WORKLOADS["verify_24x2"].with_(prior=300), 64),
                                  (WORKLOADS["decode_4b"].with_(batch=3, prior=900), 128)],
                         ids=lambda c: getattr(c, "name", str(c)))
def test_paged_append_then_attend_equals_contiguous_fused(w, bs):
    """qsa_append_kv into the paged cache, then attention on the appended rows
    (k_new = v_new = NULL), equals the fused call on the contiguous cache."""
    inp = make_inputs(w, variant="stress")
    say(f"case paged append+attend {w.name} block_size={bs}")
    contig = Session(w, inp)
    a = contig.run().clone()
    paged = Session(w, to_paged(inp, bs, seed=3), block_size=bs)
    paged.append()
    b = paged.run(fused=False).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    same_rows(paged.dev["k_cache"], paged.dev["block_table"].cpu(), bs, contig.dev["k_cache"], inp)
    assert paged.device_error() == 0


def test_paged_block_outside_the_cache_is_reported_not_read():
    """A block id past the allocated rows: that sequence's outputs are NaN and
    the error bit is set; the other sequence is exact and its rows unchanged
    apart from its own appended row."""
    w = WORKLOADS["decode_4b"].with_(batch=2, prior=500)
    inp = make_inputs(w)
    pin = to_paged(inp, 64, seed=9)
    good = Session(w, to_paged(inp, 64, seed=9), block_size=64).run().clone()
    pin["block_table"][1, 2] = 10 ** 6                  # past num_rows / block_size
    sess = Session(w, pin, block_size=64)
    before = sess.dev["k_cache"].clone()
    say("case paged bad block")
    out = sess.run()
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all()
    assert torch.equal(out[0], good[0])
    assert sess.device_error() & 1
    assert torch.equal(paged_rows(before, pin["block_table"], 64, 0, 500),
                       paged_rows(sess.dev["k_cache"], pin["block_table"], 64, 0, 500))


def test_paged_prefill_is_refused():
    w = WORKLOADS["decode_4b"].with_(q_len=40, prior=100)
    inp = make_inputs(w)
    sess = Session(w, to_paged(inp, 64), block_size=64)
    with pytest.raises(binding.QSAError) as e:
        sess.run()
    assert e.value.code == binding.QSA_ERR_UNSUPPORTED
