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
    # 132 rows = one full and one ragged 128-row tile, 183 keys = 5 full 32-key stages + a ragged one
    Workload("bf16_prefill_d64", batch=2, q_len=33, num_q_heads=8, num_kv_heads=2, head_dim=64,
             rotary_dim=32, rope_theta=1e4, dtype="bf16", prior=150, seed=113),
    # tile route at head_dim 128: 280 rows = three tiles
    Workload("bf16_prefill_d128_tiles", batch=1, q_len=70, num_q_heads=8, num_kv_heads=2, head_dim=128,
             rotary_dim=64, rope_theta=1e6, dtype="bf16", prior=200, seed=114),
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


def sampled_rows(w, count, seed):
    rng = np.random.default_rng(seed)
    B, L, Hq = w.batch, w.q_len, w.num_q_heads
    fixed = [0, Hq - 1, (L - 1) * Hq, ((B - 1) * L + L - 1) * Hq + Hq - 1]
    rand = rng.choice(B * L * Hq, size=count, replace=False)
    return np.unique(np.concatenate([fixed, rand]).astype(np.int64))


@pytest.mark.parametrize("name,count", [("ragged_4b", 96), ("prefill_4b", 96)])
def test_parity_full_size_sampled(name, count):
    w = WORKLOADS[name]
    say(f"case {name} full size, {count} sampled rows")
    inp = make_inputs(w)
    say(f"  sum of cached lengths {int(inp['seq_lens'].sum())}")
    sess = Session(w, inp)
    say(f"  plan {sess.plan()}")
    out = to_np(sess.run()).reshape(-1, w.head_dim)
    rows = sampled_rows(w, count, seed=w.seed)
    g = geo(w)
    kr, vr = oracle.new_kv(g, inp["k_new"], inp["v_new"], inp["w_k"], inp["positions"])
    ref = oracle.attention(g, inp["q_gate"], inp["w_q"], inp["k_cache"], inp["v_cache"],
                           inp["seq_offset"], inp["seq_lens"], inp["positions"], kr, vr, rows=rows)
    check(out[rows], ref, w.dtype, f"{name} sampled")
    check_rows(sess, inp, kr, vr, w)
    assert np.all(np.isfinite(out))
    assert sess.device_error() == 0


def test_append_then_attend_equals_fused():
    w = WORKLOADS["verify_24x2"].with_(prior=300)
    inp = make_inputs(w)
    say("case append+attend vs fused")
    fused = Session(w, inp)
    a = to_np(fused.run())
    split = Session(w, inp)
    split.append()
    b = to_np(split.run(fused=False))
    # Both equal the oracle.  Between themselves they differ by rounding only:
    # the fused call attends the new keys from its own LDS copy, and first when
    # they fit beside the cached stages, so its lazy reference max, and with it
    # each probability's bf16 rounding, can differ from the unfused call's.  So
    # A probability's rounding moves an output element by an amount that scales
    # with its head row, so every element agrees to two bf16 ulps of the largest
    # magnitude in its row.
    out, _, _ = oracle.gated_attention(geo(w), inp)
    check(a, out, w.dtype, "fused")
    check(b, out, w.dtype, "append then attend")
    ra, rb = a.reshape(-1, w.head_dim), b.reshape(-1, w.head_dim)
    row_mag = np.maximum(np.abs(ra), np.abs(rb)).max(axis=1).astype(np.float32)
    row_ulp = np.spacing(row_mag) * 2.0 ** 16             # bf16 keeps 8 of float32's 24 significand bits
    diff = np.abs(ra - rb)
    say(f"  fused vs append+attend: max_abs={float(diff.max()):.3g} "
        f"max_row_ulps={float((diff / row_ulp[:, None]).max()):.3g} rel_l2={rel_l2(a, b):.3g}")
    assert np.all(diff <= 2 * row_ulp[:, None])
    assert rel_l2(a, b) <= 5e-3
    ulp = 2.0 ** -7                                      # one bf16 ulp, relative
    # appended rows: V is copied exactly; K is an fp32 norm and rotation rounded
    # once, so the two kernels' roundings agree to one bf16 ulp
    assert torch.equal(fused.dev["v_cache"], split.dev["v_cache"])
    ka, kb = to_np(fused.dev["k_cache"]), to_np(split.dev["k_cache"])
    assert np.all(np.abs(ka - kb) <= ulp * np.maximum(np.abs(ka), np.abs(kb)))


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
