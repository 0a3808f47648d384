"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerances: bf16 storage with fp32 accumulation -- max-abs <= 2e-2 and
relative L2 <= 5e-3 over the compared outputs; fp32 -- relative L2 <= 1e-5.
Appended cache rows must match the oracle's rounded rows to one unit in the
last place of the storage dtype.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import twin
from gated_gqa_attention_amd.session import Session
from gated_gqa_attention_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = {"bf16": dict(max_abs=2e-2, rel_l2=5e-3), "f32": dict(max_abs=1e-3, rel_l2=1e-5)}
ULP_BITS = {"bf16": 8, "f32": 24}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def geo(w):
    return oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rotary_dim, w.rope_theta, w.rms_eps, 0.0, w.dtype)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    err, rl2 = float(np.max(np.abs(got - ref))), rel_l2(got, ref)
    say(f"  {what}: max_abs={err:.3g} rel_l2={rl2:.3g}")
    assert err <= TOL[dtype]["max_abs"], (what, err)
    assert rl2 <= TOL[dtype]["rel_l2"], (what, rl2)


def check_rows(sess, inp, kr, vr, w):
    """Cache rows n_b .. n_b+L-1 written by the GPU vs the oracle's rounded rows."""
    kc = sess.dev["k_cache"].float().cpu().double().numpy()
    vc = sess.dev["v_cache"].float().cpu().double().numpy()
    ulp = 2.0 ** (1 - ULP_BITS[w.dtype])
    for b in range(w.batch):
        s = int(inp["seq_offset"][b]) + int(inp["seq_lens"][b])
        gk, gv = kc[s:s + w.q_len], vc[s:s + w.q_len]
        # the GPU normalises and rotates in fp32: its value before rounding is within a few
        # fp32 ulps of the row's scale, so the stored element is within one storage ulp of
        # the oracle's, or within that fp32 error for elements far below the row's scale
        row_scale = np.max(np.abs(kr[b]), axis=-1, keepdims=True)
        bound = np.maximum(np.abs(kr[b]) * ulp, 8 * 2.0 ** -24 * row_scale)
        assert np.all(np.abs(gk - kr[b]) <= bound), f"K rows of sequence {b}"
        assert np.array_equal(gv, vr[b]), f"V rows of sequence {b}"


def to_np(t):
    return t.float().cpu().double().numpy()


SMALL = [
    WORKLOADS["tiny_f32"],
    Workload("f32_gqa_causal", batch=2, q_len=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
             rotary_dim=32, rope_theta=1e6, dtype="f32", prior=70, seed=101),
    Workload("f32_ragged", batch=3, q_len=1, num_q_heads=4, num_kv_heads=4, head_dim=64,
             rotary_dim=64, rope_theta=1e4, dtype="f32", prior=0, seed=102, ragged=(0, 200)),
    Workload("bf16_decode_ragged", batch=3, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=0, seed=103, ragged=(1, 300)),
    Workload("bf16_d64_mha", batch=2, q_len=2, num_q_heads=4, num_kv_heads=4, head_dim=64,
             rotary_dim=0, rope_theta=1e4, dtype="bf16", prior=129, seed=104),
    Workload("bf16_d128_full_rope", batch=2, q_len=1, num_q_heads=6, num_kv_heads=1, head_dim=128,
             rotary_dim=128, rope_theta=1e6, dtype="bf16", prior=191, seed=105),
    Workload("bf16_verify_small", batch=2, q_len=4, num_q_heads=24, num_kv_heads=2, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=130, seed=106),
    # short-query route in two row tiles of unequal size: 3 new rows x 11 heads
    # per KV group = 33 rows, tiles of 17 and 16
    Workload("bf16_row_tiles_33", batch=3, q_len=3, num_q_heads=22, num_kv_heads=2, head_dim=128,
             rotary_dim=32, rope_theta=1e6, dtype="bf16", prior=150, seed=117),
    Workload("bf16_fused_l16", batch=1, q_len=16, num_q_heads=4, num_kv_heads=1, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=77, seed=107),
    Workload("bf16_no_prior", batch=2, q_len=5, num_q_heads=16, num_kv_heads=4, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=0, seed=108),
    Workload("bf16_prefill_tiles", batch=2, q_len=40, num_q_heads=16, num_kv_heads=4, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=100, seed=109),
    Workload("bf16_prefill_l17", batch=1, q_len=17, num_q_heads=4, num_kv_heads=2, head_dim=128,
             rotary_dim=32, rope_theta=1e7, dtype="bf16", prior=33, seed=110),
    # 64 cached + 16 new keys in one chunk: one full stage plus the new-key block
    Workload("bf16_new_rows_fold", batch=2, q_len=16, num_q_heads=4, num_kv_heads=1, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=64, seed=112),
    # tile route at head_dim 64 (half of the workgroup issues no stage copies):
    # 132 rows = one ragged 256-row tile, 183 keys = 5 full 32-key stages + a ragged one
    Workload("bf16_prefill_d64", batch=2, q_len=33, num_q_heads=8, num_kv_heads=2, head_dim=64,
             rotary_dim=32, rope_theta=1e4, dtype="bf16", prior=150, seed=113),
    # tile route at head_dim 128: 280 rows = a full 256-row tile and a ragged one (a pair when split)
    Workload("bf16_prefill_d128_tiles", batch=1, q_len=70, num_q_heads=8, num_kv_heads=2, head_dim=128,
             rotary_dim=64, rope_theta=1e6, dtype="bf16", prior=200, seed=114),
    # tile route with an odd tile count: 600 rows = tiles 0 and 2 as a pair plus tile 1
    # alone; with split key chunks one range per pair crosses from tile 0 into tile 2
    Workload("bf16_prefill_tile_pairs", batch=2, q_len=150, num_q_heads=8, num_kv_heads=2, head_dim=128,
             rotary_dim=32, rope_theta=1e6, dtype="bf16", prior=300, seed=135),
    # tile route over sequences of unequal cached lengths: each (sequence, KV head)
    # cuts its pair's keys by its own length; 400 rows = two tiles
    Workload("bf16_prefill_ragged_pairs", batch=3, q_len=100, num_q_heads=8, num_kv_heads=2, head_dim=128,
             rotary_dim=32, rope_theta=1e6, dtype="bf16", prior=0, seed=136, ragged=(0, 600)),
    # tile route with no cached keys: the pair's first tile sees 64 keys, the second 100
    Workload("bf16_prefill_no_prior_pairs", batch=1, q_len=100, num_q_heads=8, num_kv_heads=2, head_dim=128,
             rotary_dim=32, rope_theta=1e6, dtype="bf16", prior=0, seed=137),
    # short-query route, smallest rotation by whole lanes: r/2 = D/16 at head_dim 64 and 128
    Workload("bf16_d64_r8", batch=2, q_len=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
             rotary_dim=8, rope_theta=1e4, dtype="bf16", prior=90, seed=118),
    Workload("bf16_d128_r16_rows48", batch=2, q_len=4, num_q_heads=12, num_kv_heads=1, head_dim=128,
             rotary_dim=16, rope_theta=1e6, dtype="bf16", prior=150, seed=119),
    # short-query route with more stages than ring slots when unsplit (refills):
    # head_dim 64 (8 slots), 700 + 2 keys = 11 stages; head_dim 128 (4 slots), 380 + 3 keys = 6 stages
    Workload("bf16_d64_refills", batch=1, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
             rotary_dim=16, rope_theta=1e4, dtype="bf16", prior=700, seed=122),
    Workload("bf16_d128_refills", batch=1, q_len=3, num_q_heads=6, num_kv_heads=2, head_dim=128,
             rotary_dim=32, rope_theta=1e6, dtype="bf16", prior=380, seed=123),
    # short-query route with many new rows (keys 4 .. 15 of the first-attended new block,
    # causal among themselves): 16 x 3 rows at head_dim 128, 12 x 4 rows at head_dim 256
    Workload("bf16_fused_new16_d128", batch=2, q_len=16, num_q_heads=6, num_kv_heads=2, head_dim=128,
             rotary_dim=32, rope_theta=1e6, dtype="bf16", prior=200, seed=124),
    Workload("bf16_fused_new12_d256", batch=1, q_len=12, num_q_heads=4, num_kv_heads=1, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=100, seed=125),
    # decode shapes outside the short-query route: r/2 not a multiple of D/16, and 49 rows
    Workload("bf16_decode_r16_prepared", batch=2, q_len=1, num_q_heads=16, num_kv_heads=4, head_dim=256,
             rotary_dim=16, rope_theta=1e7, dtype="bf16", prior=200, seed=120),
    Workload("bf16_rows49_prepared", batch=1, q_len=7, num_q_heads=7, num_kv_heads=1, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=60, seed=121),
]


@pytest.mark.parametrize("splits", [0, 1, 2, 7])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_parity_small(w, splits):
    for variant in ("graded", "stress"):
        say(f"case {w.name} splits={splits} variant={variant}")
        inp = make_inputs(w, variant=variant)
        sess = Session(w, inp, force_splits=splits)
        say(f"  plan {sess.plan()}")
        out = to_np(sess.run())
        torch.cuda.synchronize()
        ref, kr, vr = oracle.gated_attention(geo(w), inp)
        check(out, ref, w.dtype, f"{w.name}/{variant}")
        check_rows(sess, inp, kr, vr, w)
        assert sess.device_error() == 0


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("w", [
    # short-query route (one new row per sequence)
    Workload("bf16_dominant_decode", batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=400, seed=116),
    # short-query route at three row tiles (verify shape): with 3 splits a chunk holds
    # several stages, so a later stage moves a reference max that is already set
    Workload("bf16_dominant_verify", batch=2, q_len=4, num_q_heads=24, num_kv_heads=2, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=400, seed=126),
    # tile route (160 rows)
    Workload("bf16_dominant_prefill", batch=1, q_len=40, num_q_heads=8, num_kv_heads=2, head_dim=256,
             rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=300, seed=115),
], ids=lambda w: w.name)
def test_late_dominant_keys_move_the_running_max(w, splits):
    """Three cached keys late in each sequence point along the prepared query of
    one row per KV head (last new row, first head of the group) with scores 6,
    14 and 24, so that row's maximum jumps by more than 8 log2 units (the tile
    kernel's lazy-max headroom) at each of them and the output rescaling runs;
    the earlier keys' weights must shrink exactly as in the oracle's softmax.
    (Keys along the query keep one key dominant per row: random huge keys would
    instead make two keys compete, where the bf16 rounding of q, about 1.1e-3 of
    the score, is amplified past the bf16 tolerance.)"""
    inp = make_inputs(w)
    B, L, Hq, Hkv, D = w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    qg = twin._f64(inp["q_gate"])
    wq = twin._f64(inp["w_q"])
    pos = np.asarray(inp["positions"]).astype(np.float64)
    kc = inp["k_cache"]
    for b in range(B):
        o, nb = int(inp["seq_offset"][b]), int(inp["seq_lens"][b])
        rot = twin.rotation_matrix(pos[b, L - 1], w.rotary_dim, w.rope_theta, D)
        for g in range(Hkv):
            qh = twin._norm(qg[b, L - 1, g * G, :D], wq, w.rms_eps) @ rot.T
            for frac, score in ((0.15, 6.0), (0.45, 14.0), (0.9, 24.0)):
                kc[o + int(frac * nb), g] = torch.from_numpy(score * np.sqrt(D) / (qh @ qh) * qh).to(kc.dtype)
    say(f"case {w.name} splits={splits}")
    sess = Session(w, inp, force_splits=splits)
    say(f"  plan {sess.plan()}")
    out = to_np(sess.run())
    torch.cuda.synchronize()
    ref, kr, vr = oracle.gated_attention(geo(w), inp)
    check(out, ref, w.dtype, w.name)
    check_rows(sess, inp, kr, vr, w)
    assert sess.device_error() == 0


def test_long_decode_equal_chunks():
    """Enough keys that the short-query route cuts each sequence into
    equal-length chunks of ~2048 keys (rounded count) instead of fixed ones."""
    w = Workload("bf16_long_even", batch=8, q_len=1, num_q_heads=8, num_kv_heads=4, head_dim=128,
                 rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=0, seed=117, ragged=(17000, 23000))
    inp = make_inputs(w)
    sess = Session(w, inp)
    plan = sess.plan()
    say(f"case {w.name} plan {plan}")
    fields = dict(kv.split("=") for kv in plan.split())
    assert fields["route"] == "fused_splitk" and int(fields["chunk_keys"]) >= 1024
    out = to_np(sess.run())
    torch.cuda.synchronize()
    ref, kr, vr = oracle.gated_attention(geo(w), inp)
    check(out, ref, w.dtype, w.name)
    check_rows(sess, inp, kr, vr, w)
    assert sess.device_error() == 0


@pytest.mark.parametrize("name", ["decode_4b", "verify_24x2"])
def test_parity_full_workload(name):
    w = WORKLOADS[name]
    say(f"case {name} full")
    inp = make_inputs(w)
    sess = Session(w, inp)
    say(f"  plan {sess.plan()}")
    out = to_np(sess.run())
    ref, kr, vr = oracle.gated_attention(geo(w), inp)
    check(out, ref, w.dtype, name)
    check_rows(sess, inp, kr, vr, w)
    # worst (sequence, head) slice as a diagnostic
    worst = max(rel_l2(out[b, :, h], ref[b, :, h]) for b in range(w.batch) for h in range(w.num_q_heads))
    say(f"  worst per-(b,h) rel_l2={worst:.3g}")


def per_row_worst(out, ref, D):
    """Worst relative L2 over (b, l, h) head rows: a diagnostic beside the graded figures."""
    a, b = out.reshape(-1, D), ref.reshape(-1, D)
    num = np.linalg.norm(a - b, axis=1)
    den = np.maximum(np.linalg.norm(b, axis=1), 1e-300)
    return float(np.max(num / den))


@pytest.mark.parametrize("name", ["ragged_4b", "prefill_4b"])
def test_parity_full_size_every_output(name):
    """Every output of the ragged batch (1,024 head rows over 4.36 GB of cache)
    and of the prefill chunk (32,768 head rows, 8.4 M values) against the
    oracle, in the launch configuration the benchmark times."""
    w = WORKLOADS[name]
    say(f"case {name} full size, every output")
    inp = make_inputs(w)
    say(f"  sum of cached lengths {int(inp['seq_lens'].sum())}")
    sess = Session(w, inp)
    say(f"  plan {sess.plan()}")
    out = to_np(sess.run())
    torch.cuda.synchronize()
    assert sess.device_error() == 0
    say("  oracle ...")
    ref, kr, vr = oracle.gated_attention(geo(w), inp)
    check(out, ref, w.dtype, f"{name} every output")
    say(f"  worst per-(b,l,h) rel_l2={per_row_worst(out, ref, w.head_dim):.3g}")
    check_rows(sess, inp, kr, vr, w)


APPEND_CASES = [
    # short-query route, three row tiles: new rows attended first from the arena, split keys
    (WORKLOADS["verify_24x2"].with_(prior=300), 0),
    # short-query route, one new key in the free ring slot (decode), split keys
    (WORKLOADS["decode_4b"].with_(prior=1000), 0),
    # short-query route, one row tile and no free slot: the new rows follow 11 cached stages
    (WORKLOADS["decode_4b"].with_(prior=700, batch=2), 1),
    # tile route (prepared queries), two row tiles and split keys
    (Workload("append_tiles", batch=2, q_len=40, num_q_heads=16, num_kv_heads=4, head_dim=256,
              rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=100, seed=127), 2),
    # tile route because r/2 = 8 is not a multiple of D/16 = 16 (the prologue's LDS rotation)
    (Workload("append_r16", batch=2, q_len=1, num_q_heads=16, num_kv_heads=4, head_dim=256,
              rotary_dim=16, rope_theta=1e7, dtype="bf16", prior=200, seed=128), 0),
    # fp32 route
    (Workload("append_f32", batch=2, q_len=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
              rotary_dim=32, rope_theta=1e6, dtype="f32", prior=70, seed=129), 0),
]


@pytest.mark.parametrize("w,splits", APPEND_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_append_then_attend_equals_fused(w, splits):
    """qsa_gated_attention with k_new / v_new equals qsa_append_kv followed by
    qsa_gated_attention on the appended rows (k_new = v_new = NULL), bitwise:
    the same cache rows and the same outputs, on every route."""
    inp = make_inputs(w, variant="stress")
    say(f"case append+attend vs fused {w.name} splits={splits}")
    fused = Session(w, inp, force_splits=splits)
    say(f"  plan {fused.plan()}")
    a = fused.run().clone()
    split = Session(w, inp, force_splits=splits)
    split.append()
    b = split.run(fused=False).clone()
    torch.cuda.synchronize()
    assert torch.equal(fused.dev["k_cache"], split.dev["k_cache"])
    assert torch.equal(fused.dev["v_cache"], split.dev["v_cache"])
    assert torch.equal(a, b)
    out, kr, vr = oracle.gated_attention(geo(w), inp)
    check(to_np(a), out, w.dtype, "fused")
    check_rows(split, inp, kr, vr, w)
    assert fused.device_error() == 0 and split.device_error() == 0


SCALE_CASES = [
    (WORKLOADS["tiny_f32"], 0.3),
    (WORKLOADS["decode_4b"].with_(prior=1500), 0.09),
    (Workload("scale_verify", batch=2, q_len=4, num_q_heads=24, num_kv_heads=2, head_dim=256,
              rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=700, seed=130), 0.045),
    (Workload("scale_tiles", batch=1, q_len=40, num_q_heads=16, num_kv_heads=4, head_dim=128,
              rotary_dim=32, rope_theta=1e6, dtype="bf16", prior=300, seed=131), 0.15),
]


@pytest.mark.parametrize("w,scale", SCALE_CASES, ids=lambda c: getattr(c, "name", str(c)))
@pytest.mark.parametrize("splits", [0, 3])
def test_parity_explicit_softmax_scale(w, scale, splits):
    """softmax_scale > 0 replaces 1/sqrt(head_dim) on every route."""
    inp = make_inputs(w)
    say(f"case {w.name} softmax_scale={scale} splits={splits}")
    sess = Session(w, inp, force_splits=splits, softmax_scale=scale)
    say(f"  plan {sess.plan()}")
    out = to_np(sess.run())
    torch.cuda.synchronize()
    g = geo(w)
    g.softmax_scale = scale
    ref, kr, vr = oracle.gated_attention(g, inp)
    check(out, ref, w.dtype, f"{w.name} scale {scale}")
    # and the scale matters: the default scale's result is far from this one
    ref0, _, _ = oracle.gated_attention(geo(w), inp)
    assert rel_l2(ref0, ref) > 20 * TOL[w.dtype]["rel_l2"]
    assert sess.device_error() == 0


def test_consecutive_calls_on_one_workspace():
    """Two calls with different inputs, one after the other on the same
    workspace and output: the second result must not carry anything of the
    first (split-K partials, counters)."""
    w = WORKLOADS["decode_4b"].with_(prior=3000)
    inp_a = make_inputs(w)
    inp_b = make_inputs(w, seed=77)
    sess = Session(w, inp_a)
    say(f"case consecutive calls, plan {sess.plan()}")
    sess.run()
    for k, v in inp_b.items():
        sess.dev[k].copy_(v)
    out = to_np(sess.run())
    torch.cuda.synchronize()
    ref, _, _ = oracle.gated_attention(geo(w), inp_b)
    check(out, ref, w.dtype, "second call")
    assert sess.device_error() == 0


def test_split_count_invariance():
    w = WORKLOADS["decode_4b"]
    inp = make_inputs(w)
    outs = {}
    for k in (0, 1, 2, 7, 65):
        say(f"case decode_4b force_splits={k}")
        outs[k] = to_np(Session(w, inp, force_splits=k).run())
    for k, o in outs.items():
        assert rel_l2(o, outs[1]) < 5e-3, k


def test_repeat_calls_are_idempotent():
    w = WORKLOADS["decode_4b"]
    inp = make_inputs(w)
    sess = Session(w, inp)
    first = sess.run().clone()
    kc = sess.dev["k_cache"].clone()
    for _ in range(3):
        again = sess.run()
    torch.cuda.synchronize()
    assert torch.equal(first, again)
    assert torch.equal(kc, sess.dev["k_cache"])
    assert sess.device_error() == 0


@pytest.mark.parametrize("case", ["capacity_one_chunk", "capacity_split", "length_past_bound"])
def test_device_side_range_error_is_reported_not_faulted(case):
    """A sequence whose rows would pass its capacity (or the call's max_seq_len)
    gets NaN outputs and a workspace flag; its cache rows are not written; the
    other sequence is unaffected.  Every case stays inside the buffers."""
    w = Workload("range", batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=256,
                 rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=50, seed=111)
    inp = make_inputs(w)
    sess = Session(w, inp, max_seq_len=64, force_splits=3 if case == "capacity_split" else 0)
    if case == "length_past_bound":
        sess.dev["seq_lens"][1] = 70       # n + L exceeds max_seq_len (and the sequence's rows)
    else:
        sess.dev["capacity"][1] = 40       # sequence 1 claims fewer rows than n + L
    kc = sess.dev["k_cache"].clone()
    print(f"range case {case}", flush=True)
    out = to_np(sess.run())
    torch.cuda.synchronize()
    assert np.all(np.isnan(out[1]))
    assert np.all(np.isfinite(out[0]))
    assert sess.device_error() & 1
    s1 = int(inp["seq_offset"][1]) + 50
    assert torch.equal(kc[s1], sess.dev["k_cache"][s1])
