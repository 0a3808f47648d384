"""Pins of the bf16-K / Turbo4-V oracle (CPU only).

Atlas docs, spark_model/forward/qwen3_5/mod.rs: MetalKvDtype::Bf16KTurbo4V
(K raw bf16, V Turbo4: 4-bit Lloyd-Max indices and FP8 scales per 16,
matched-norm L2, WHT-rotated basis) and LayerKvCache::alloc.  The codebook
and the index/scale rules are readings (parity against the page unpinned);
their arithmetic is pinned here by the published Lloyd-Max table for the
normal distribution, quadrature and Monte Carlo, brute-force nearest levels,
library E4M3 casts, the plain attention oracle on rotated-back rows, and the
quantization error of the whole path against unquantized attention.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gated_gqa_attention_amd.workloads import WORKLOADS, make_inputs, make_turbo4v_inputs


def geo_of(w, dtype="bf16"):
    return oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim, w.rotary_dim,
                           w.rope_theta, w.rms_eps, 0.0, dtype)


def e4m3_cast(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_codebook_matches_the_published_lloyd_max_table():
    """J. Max, "Quantizing for minimum distortion" (1960), the 16-level normal
    quantizer: output levels +-0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618,
    2.069, 2.733 and mean squared error 0.009497."""
    c = oracle.lloyd_max_normal(16)
    pub = np.array([0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733])
    np.testing.assert_allclose(c[8:], pub, atol=6e-4)
    np.testing.assert_array_equal(c[:8], -c[8:][::-1])
    assert np.all(np.diff(c) > 0)


def test_codebook_is_a_fixed_point_and_its_distortion():
    from scipy import integrate, stats
    c = oracle.lloyd_max_normal(16)
    t = np.concatenate([[-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]])
    for i in range(16):
        mass = stats.norm.cdf(t[i + 1]) - stats.norm.cdf(t[i])
        mean = integrate.quad(lambda x: x * stats.norm.pdf(x), t[i], t[i + 1])[0] / mass
        assert mean == pytest.approx(c[i], abs=1e-8)
    rng = np.random.default_rng(0)
    x = rng.standard_normal(2_000_000)
    mse = np.mean((x - c[np.abs(x[:, None] - c[None, :]).argmin(axis=1)]) ** 2)
    assert mse == pytest.approx(0.009497, abs=1.5e-4)


def test_turbo4_quantizer_definition():
    c = oracle.lloyd_max_normal(16)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)))
    codes, scales = oracle.turbo4_quantize(x)
    assert codes.shape == (64, 128) and scales.shape == (64, 16)
    g = x.reshape(64, 16, 16)
    sigma = np.sqrt((g * g).mean(axis=-1, keepdims=True))
    idx = np.abs(g[..., None] / sigma[..., None] - c).argmin(axis=-1)       # brute-force nearest level
    got = np.stack([codes & 15, codes >> 4], axis=-1).reshape(64, 16, 16)
    np.testing.assert_array_equal(got, idx)
    s = np.sqrt((g * g).sum(-1) / (c[idx] ** 2).sum(-1))
    np.testing.assert_array_equal(scales, e4m3_cast(s))
    deq = oracle.turbo4_dequantize(codes, scales).reshape(64, 16, 16)
    ratio = np.linalg.norm(deq, axis=-1) / np.linalg.norm(g, axis=-1)       # matched norm, up to the E4M3 scale
    assert np.all(np.abs(ratio - 1) <= 1 / 16 + 1e-12)


def test_turbo4_packing_and_zero_group():
    c = oracle.lloyd_max_normal(16)
    x = np.zeros(32)
    x[16:] = c[5]
    x[16], x[17] = c[3], c[12]
    codes, scales = oracle.turbo4_quantize(x)
    assert list(codes[:8]) == [0] * 8 and scales[0] == 0
    assert oracle.turbo4_dequantize(codes, scales)[:16].tolist() == [0.0] * 16
    sigma = np.sqrt(np.mean(x[16:] ** 2))
    i0 = np.abs(c - c[3] / sigma).argmin()
    i1 = np.abs(c - c[12] / sigma).argmin()
    assert codes[8] == i0 | (i1 << 4)


@pytest.mark.parametrize("name", ["decode_4b", "verify_24x2"])
def test_attention_equals_plain_attention_on_rotated_back_values(name):
    """With every key and value read from the cache (the new rows appended), the
    attention on Turbo4 values rotated back equals the plain attention on the
    bf16 K rows and the decoded V rows passed through the WHT (H sum p v =
    sum p H v); leaving out the iWHT bookend is far off."""
    w = WORKLOADS[name].with_(prior=96, batch=min(WORKLOADS[name].batch, 2))
    x = make_turbo4v_inputs(w)
    g = geo_of(w, "f64")
    kr, vc, vs = oracle.bf16k_turbo4v_new_kv(g, x["k_new"], x["v_new"], x["w_k"], x["positions"])
    for b in range(w.batch):
        s0 = int(x["seq_offset"][b]) + int(x["seq_lens"][b])
        x["k_cache"][s0:s0 + w.q_len] = torch.from_numpy(kr[b]).to(torch.bfloat16)
        x["v_codes"][s0:s0 + w.q_len] = torch.from_numpy(vc[b])
        x["v_scales"][s0:s0 + w.q_len] = torch.from_numpy(vs[b])
    got = oracle.bf16k_turbo4v_attention(g, x["q_gate"], x["w_q"], x["k_cache"], x["v_codes"], x["v_scales"],
                                         x["seq_offset"], x["seq_lens"], x["positions"])
    vd = oracle.turbo4_dequantize(x["v_codes"], x["v_scales"])
    plain = oracle.attention(g, x["q_gate"], x["w_q"], x["k_cache"].double().numpy(), oracle.wht(vd),
                             x["seq_offset"], x["seq_lens"], x["positions"])
    rel = np.linalg.norm(got - plain) / np.linalg.norm(plain)
    assert rel < 1e-12
    no_bookend = oracle.attention(g, x["q_gate"], x["w_q"], x["k_cache"].double().numpy(), vd,
                                  x["seq_offset"], x["seq_lens"], x["positions"])
    assert np.linalg.norm(no_bookend - got) / np.linalg.norm(got) > 0.1


def test_new_rows_follow_their_definition():
    w = WORKLOADS["verify_24x2"].with_(prior=16, batch=2)
    x = make_inputs(w)
    geo = geo_of(w)
    kr, vc, vs = oracle.bf16k_turbo4v_new_kv(geo, x["k_new"], x["v_new"], x["w_k"], x["positions"])
    kref, _ = oracle.new_kv(geo, x["k_new"], x["v_new"], x["w_k"], x["positions"])    # bf16 storage
    np.testing.assert_array_equal(kr, kref)
    c2, s2 = oracle.turbo4_quantize(oracle.wht(x["v_new"].double().numpy()))
    np.testing.assert_array_equal(vc, c2)
    np.testing.assert_array_equal(vs, s2)


def test_fused_equals_append_then_attend():
    w = WORKLOADS["verify_24x2"].with_(prior=40, batch=2)
    x = make_turbo4v_inputs(w)
    geo = geo_of(w)
    out_f, (kr, vc, vs) = oracle.bf16k_turbo4v_gated_attention(geo, x)
    k = x["k_cache"].clone()
    v_codes, v_scales = x["v_codes"].clone(), x["v_scales"].clone()
    for b in range(w.batch):
        o, n = int(x["seq_offset"][b]), int(x["seq_lens"][b])
        for l in range(w.q_len):
            k[o + n + l] = torch.from_numpy(kr[b, l]).to(torch.bfloat16)
            v_codes[o + n + l] = torch.from_numpy(vc[b, l])
            v_scales[o + n + l] = torch.from_numpy(vs[b, l])
    y = dict(x, k_cache=k, v_codes=v_codes, v_scales=v_scales)
    out_u, _ = oracle.bf16k_turbo4v_gated_attention(geo, y, fused=False)
    np.testing.assert_array_equal(out_f, out_u)


def test_tracks_unquantized_attention():
    """Quantizing real V rows with the rotation: the output stays within the
    4-bit quantization noise of plain attention on the same bf16 rows, and is
    far from it without the rotation bookend."""
    w = WORKLOADS["decode_4b"].with_(prior=512)
    x = make_inputs(w)
    g = geo_of(w, "f64")
    kr, vr = oracle.new_kv(geo_of(w), x["k_new"], x["v_new"], x["w_k"], x["positions"])
    ref = oracle.attention(g, x["q_gate"], x["w_q"], x["k_cache"], x["v_cache"], x["seq_offset"], x["seq_lens"],
                           x["positions"], k_rows=kr, v_rows=vr)
    vc, vs = oracle.turbo4_quantize(oracle.wht(x["v_cache"].double().numpy()))
    y = dict(x, v_codes=torch.from_numpy(vc), v_scales=torch.from_numpy(vs))
    out, _ = oracle.bf16k_turbo4v_gated_attention(g, y)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 0.005 < rel < 0.2, rel
