"""Pins for the oracle's Turbo8 KV path (no GPU).

Turbo8 (Atlas docs, spark_model/forward/qwen3_5/mod.rs: MetalKvDtype::Turbo8,
LayerKvCache::alloc, Qwen35Kernels' quantizing appends, dequantizing decode
attention and WHT bookends) stores K and V as FP8 E4M3 codes with a bf16
scale per 16 elements, in the Walsh-Hadamard rotated basis.  Pinned here:

* E4M3 decoding and rounding against torch's float8_e4m3fn casts (a library
  implementation of the OCP format);
* the transform against scipy's Hadamard matrix, and its inverse;
* the quantizer's error bound, exact round trips and saturation;
* the attention: on a cache whose rows are exactly Turbo8 values, the Turbo8
  attention equals the plain attention on the rows rotated back, to rounding;
  a missing bookend breaks that by far;
* the fused call equals append-then-attend.

Parity unpinned (no page fixes them, so both sides follow one reading): the
group scale rule amax / 448 in bf16 and the orthonormal Sylvester-order WHT.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import twin
from gated_gqa_attention_amd.workloads import WORKLOADS, Workload, make_turbo8_inputs


def geo(w, dtype=None):
    return oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.rotary_dim, w.rope_theta, w.rms_eps, 0.0, dtype or w.dtype)


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


def test_e4m3_values_match_library_decoding():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_value(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], lib[~nan])
    assert oracle.e4m3_value(np.array([0x7E], dtype=np.uint8))[0] == 448.0


def test_e4m3_rounding_matches_library_cast():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 9, 20000))
    grid = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[np.isfinite(grid)])
    ties = (grid[1:] + grid[:-1]) / 2                    # exact midpoints: ties to even
    x = np.clip(np.concatenate([x, ties, -ties, [0.0, 1e-30, 447.9, 448.0]]), -448.0, 448.0)
    ours = oracle.e4m3_code(x)
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, lib)
    # saturation beyond the largest value (the library cast gives NaN there)
    assert list(oracle.e4m3_code(np.array([449.0, 1e6, -500.0]))) == [0x7E, 0x7E, 0xFE]


@pytest.mark.parametrize("n", [16, 64, 256])
def test_wht_is_the_orthonormal_hadamard_transform(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((3, n))
    H = scipy.linalg.hadamard(n) / np.sqrt(n)
    y = oracle.wht(x)
    assert np.max(np.abs(y - x @ H.T)) < 1e-12
    assert np.max(np.abs(oracle.wht(y) - x)) < 1e-12      # its own inverse
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_quantizer_error_bound_round_trip_and_saturation():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((50, 256)) * np.exp(rng.standard_normal((50, 256 // 16)).repeat(16, axis=1))
    codes, sb = oracle.turbo8_quantize(x)
    deq = oracle.turbo8_dequantize(codes, sb)
    s = np.repeat((sb.astype(np.uint32) << 16).view(np.float32).astype(np.float64), 16, axis=-1)
    # each value is within half an E4M3 step of x/s, times s (steps: 2^-3 relative, 2^-9 below 2^-6)
    q = x.astype(np.float32).astype(np.float64) / s
    step = np.where(np.abs(q) >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(np.abs(q), 1e-300))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - x) <= (0.5 * step + 1e-7 * np.abs(q)) * s + 1e-12 * np.abs(x))
    # the scale is the group's largest magnitude over 448, in bf16
    amax = np.abs(x.astype(np.float32)).reshape(50, 16, 16).max(axis=-1).astype(np.float32)
    assert np.array_equal(sb, torch.from_numpy(amax / np.float32(448)).to(torch.bfloat16).view(torch.int16)
                          .numpy().view(np.uint16))
    # groups already on the grid come back exactly; a zero group has a zero scale
    grid_vals = oracle.e4m3_value(np.array([0x7E, 0x30, 0xB5, 0x01, 0x00, 0x44, 0xC0, 0x3C] * 2, dtype=np.uint8))
    exact = np.concatenate([grid_vals * 2.0 ** -5, np.zeros(16)])
    c2, s2 = oracle.turbo8_quantize(exact)
    assert np.array_equal(oracle.turbo8_dequantize(c2, s2), exact)
    assert s2[1] == 0 and np.all(c2[16:] == 0)
    # a scale rounded down below amax / 448 saturates the largest element at 448 * s
    sat = np.full(16, 0.1)
    sat[0] = 448.0 * (1 + 2.0 ** -8) * 2.0 ** -3      # amax / 448 = 2^-3 (1 + 2^-8): the bf16 scale rounds down
    c3, s3 = oracle.turbo8_quantize(sat)
    assert c3[0] == 0x7E


def _plain_equivalent(w, inp):
    """The same attention on the rows rotated back: K_plain = WHT(decoded K), likewise V."""
    kd = oracle.turbo8_dequantize(inp["k_codes"].numpy(), inp["k_scales"].view(torch.int16).numpy())
    vd = oracle.turbo8_dequantize(inp["v_codes"].numpy(), inp["v_scales"].view(torch.int16).numpy())
    return oracle.wht(kd), oracle.wht(vd), kd, vd


@pytest.mark.parametrize("w", [
    Workload("t8_gqa", batch=2, q_len=3, num_q_heads=8, num_kv_heads=2, head_dim=64, rotary_dim=16,
             rope_theta=1e4, dtype="bf16", prior=9, seed=71),
    Workload("t8_4b", batch=1, q_len=1, num_q_heads=16, num_kv_heads=4, head_dim=256, rotary_dim=64,
             rope_theta=1e7, dtype="bf16", prior=40, seed=72),
], ids=lambda w: w.name)
def test_turbo8_attention_equals_plain_attention_on_rotated_back_rows(w):
    """With every key and value read from the Turbo8 cache (the new rows already
    in it), scores (H q).k = q.(H k) and H sum p v = sum p H v, so the Turbo8
    attention is the plain attention on K = H(decoded K), V = H(decoded V)."""
    inp = make_turbo8_inputs(w.with_(prior=w.prior))
    # put the new rows into the cache, as an append would
    cap_fill = {k: inp[k] for k in ("k_codes", "k_scales", "v_codes", "v_scales")}
    new = oracle.turbo8_new_kv(geo(w), inp["k_new"], inp["v_new"], inp["w_k"], inp["positions"])
    for b in range(w.batch):
        s0 = int(inp["seq_offset"][b]) + int(inp["seq_lens"][b])
        cap_fill["k_codes"][s0:s0 + w.q_len] = torch.from_numpy(new[0][b])
        cap_fill["k_scales"][s0:s0 + w.q_len] = torch.from_numpy(new[1][b].view(np.int16)).view(torch.bfloat16)
        cap_fill["v_codes"][s0:s0 + w.q_len] = torch.from_numpy(new[2][b])
        cap_fill["v_scales"][s0:s0 + w.q_len] = torch.from_numpy(new[3][b].view(np.int16)).view(torch.bfloat16)
    inp.update(cap_fill)
    g = geo(w, "f64")
    t8 = oracle.turbo8_attention(g, inp["q_gate"], inp["w_q"], inp["k_codes"], inp["k_scales"], inp["v_codes"],
                                 inp["v_scales"], inp["seq_offset"], inp["seq_lens"], inp["positions"])
    kp, vp, kd, vd = _plain_equivalent(w, inp)
    plain = oracle.attention(g, inp["q_gate"], inp["w_q"], kp, vp, inp["seq_offset"], inp["seq_lens"],
                             inp["positions"])
    assert rel_l2(t8, plain) < 1e-12
    # a missing bookend is far off: the unrotated rows attended directly (neither
    # WHT(q) nor iWHT(out)), or the output left in the rotated basis
    no_bookends = oracle.attention(g, inp["q_gate"], inp["w_q"], kd, vd, inp["seq_offset"], inp["seq_lens"],
                                   inp["positions"])
    assert rel_l2(no_bookends, t8) > 0.1
    left_rotated = oracle.wht(t8)
    assert rel_l2(left_rotated, t8) > 0.1


def test_turbo8_new_rows_follow_their_definition():
    """New K rows: quantize(WHT(rope(rmsnorm(k) w))) with the twin's norm and
    rotation and scipy's Hadamard matrix; new V rows: quantize(WHT(v))."""
    w = Workload("t8_new", batch=2, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=128, rotary_dim=32,
                 rope_theta=1e6, dtype="bf16", prior=3, seed=73)
    inp = make_turbo8_inputs(w, variant="stress")
    kc, ks, vc, vs = oracle.turbo8_new_kv(geo(w), inp["k_new"], inp["v_new"], inp["w_k"], inp["positions"])
    H = scipy.linalg.hadamard(128) / np.sqrt(128)
    kn, wk = twin._f64(inp["k_new"]), twin._f64(inp["w_k"])
    for b in range(2):
        for l in range(2):
            rot = twin.rotation_matrix(float(inp["positions"][b, l]), 32, 1e6, 128)
            for g in range(2):
                k = H @ (rot @ twin._norm(kn[b, l, g], wk, w.rms_eps))
                deq = oracle.turbo8_dequantize(kc[b, l, g], ks[b, l, g])
                s = np.repeat((ks[b, l, g].astype(np.uint32) << 16).view(np.float32), 16).astype(np.float64)
                assert np.all(np.abs(deq - k) <= s * np.maximum(np.abs(k / s), 2.0 ** -6) * 2.0 ** -4 + 1e-9)
                v = H @ twin._f64(inp["v_new"])[b, l, g]
                codes, sc = oracle.turbo8_quantize(v)
                assert np.array_equal(codes, vc[b, l, g]) and np.array_equal(sc, vs[b, l, g])


def test_turbo8_fused_equals_append_then_attend():
    w = WORKLOADS["verify_24x2"].with_(prior=30, head_dim=64, rotary_dim=16, batch=2)
    inp = make_turbo8_inputs(w)
    g = geo(w)
    fused, new = oracle.turbo8_gated_attention(g, inp)
    for b in range(w.batch):
        s0 = int(inp["seq_offset"][b]) + int(inp["seq_lens"][b])
        inp["k_codes"][s0:s0 + w.q_len] = torch.from_numpy(new[0][b])
        inp["k_scales"][s0:s0 + w.q_len] = torch.from_numpy(new[1][b].view(np.int16)).view(torch.bfloat16)
        inp["v_codes"][s0:s0 + w.q_len] = torch.from_numpy(new[2][b])
        inp["v_scales"][s0:s0 + w.q_len] = torch.from_numpy(new[3][b].view(np.int16)).view(torch.bfloat16)
    unfused, _ = oracle.turbo8_gated_attention(g, inp, fused=False)
    assert np.array_equal(fused, unfused)


def test_turbo8_tracks_the_unquantized_attention():
    """Quantization noise only: against the plain attention on the decoded rows
    rotated back (the same values unquantized) the difference is zero; against
    the plain attention on bf16 keys the Turbo8 result stays close (E4M3 keeps
    3 mantissa bits, the rotation spreads outliers)."""
    w = WORKLOADS["decode_4b"].with_(prior=200)
    inp = make_turbo8_inputs(w)
    g = geo(w)
    out, _ = oracle.turbo8_gated_attention(g, inp, fused=False)
    kp, vp, _, _ = _plain_equivalent(w, inp)
    # quantizing the rotated-back rows again (bf16 storage) changes the result only a little
    plain = oracle.attention(g, inp["q_gate"], inp["w_q"], torch.from_numpy(kp).to(torch.bfloat16),
                             torch.from_numpy(vp).to(torch.bfloat16), inp["seq_offset"], inp["seq_lens"],
                             inp["positions"])
    assert rel_l2(out, plain) < 2e-2
