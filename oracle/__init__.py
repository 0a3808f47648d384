"""CPU oracle for the gated grouped-query attention core.

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product library
(``gated_gqa_attention_amd``) never imports this package, and this package
never imports the product library.

The arithmetic lives in ``qsa_oracle.c`` (plain C, IEEE double, one row at a
time).  This module only builds it with gcc, loads it with ctypes and marshals
arrays.  The steps it follows, with the pages they come from:

* split of the doubled q_proj output per head into ``[query | gate]`` --
  mlxd PR #99 "stage D6", Summary and the second review (``mlx_split`` index 0
  = queries, index 1 = gate); Atlas ``qwen3_5/mod.rs``, ``q_total``;
* per-head RMS QK-norm -- mlxd PR #99, config audit table (``has_qk_norm``);
  Atlas ``FullAttentionLayer`` (``q_norm``, ``k_norm``);
* partial RoPE on the first ``rotary_dim`` dims -- mlxd PR #99 Summary
  (``partial_rotary_factor``); Atlas ``Qwen35ForwardConfig::rotary_dim``;
* KV append at slot ``n_b + l`` then attention over ``n_b + l + 1`` keys --
  Atlas ``qwen3_5/mod.rs`` module doc;
* grouped-query attention with contiguous head groups -- DS4Server issue #113,
  Reproduction; Atlas ``Qwen35ForwardConfig`` (16 query / 4 KV heads);
* ``attn * sigmoid(gate)`` -- mlxd PR #99 Summary; Atlas ``sigmoid_gate``;
* the projections either side (fused q/k/v with the query/gate split in its
  output layout, and o_proj) -- mlxd PR #99 Summary; Atlas
  ``FullAttentionLayer`` q/k/v/o_proj and ``Qwen35Kernels`` ``qkv_split``.

Readings where the pages are silent are listed with each function below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "libqsa_oracle.so")

F64, F32, BF16 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("rotary_dim", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double),
        ("softmax_scale", ctypes.c_double), ("store_bits", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        lib.qsa_oracle_round.restype = ctypes.c_double
        lib.qsa_oracle_round.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.qsa_oracle_new_kv.restype = ctypes.c_int
        lib.qsa_oracle_new_kv.argtypes = [ctypes.POINTER(_Cfg), p, p, p, p, p, p]
        lib.qsa_oracle_attention.restype = ctypes.c_int
        lib.qsa_oracle_attention.argtypes = [
            ctypes.POINTER(_Cfg), p, p, p, p, ctypes.c_int32, p, p, p, p, p, p,
            ctypes.c_int64, p, p]
        lib.qsa_oracle_linear.restype = ctypes.c_int
        lib.qsa_oracle_linear.argtypes = [p, p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, p]
        lib.qsa_oracle_qkv_proj.restype = ctypes.c_int
        lib.qsa_oracle_qkv_proj.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int32, p, p, p, p, p]
        lib.qsa_oracle_e4m3_value.restype = ctypes.c_double
        lib.qsa_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.qsa_oracle_e4m3_code.restype = ctypes.c_uint8
        lib.qsa_oracle_e4m3_code.argtypes = [ctypes.c_double]
        lib.qsa_oracle_wht.restype = ctypes.c_int
        lib.qsa_oracle_wht.argtypes = [p, ctypes.c_int, p]
        lib.qsa_oracle_turbo8_quantize.restype = ctypes.c_int
        lib.qsa_oracle_turbo8_quantize.argtypes = [p, ctypes.c_int, p, p]
        lib.qsa_oracle_turbo8_new_kv.restype = ctypes.c_int
        lib.qsa_oracle_turbo8_new_kv.argtypes = [ctypes.POINTER(_Cfg), p, p, p, p, p, p, p, p]
        lib.qsa_oracle_turbo8_attention.restype = ctypes.c_int
        lib.qsa_oracle_turbo8_attention.argtypes = [ctypes.POINTER(_Cfg), p, p, p, p, p, p, p, p, p, p, p, p, p,
                                                    p, ctypes.c_int64, p]
        lib.qsa_oracle_lloyd_max_normal.restype = ctypes.c_int
        lib.qsa_oracle_lloyd_max_normal.argtypes = [ctypes.c_int, p]
        lib.qsa_oracle_turbo4_quantize.restype = ctypes.c_int
        lib.qsa_oracle_turbo4_quantize.argtypes = [p, ctypes.c_int, p, p, p]
        lib.qsa_oracle_turbo4_dequantize.restype = ctypes.c_int
        lib.qsa_oracle_turbo4_dequantize.argtypes = [p, p, ctypes.c_int, p, p]
        lib.qsa_oracle_bf16k_turbo4v_new_kv.restype = ctypes.c_int
        lib.qsa_oracle_bf16k_turbo4v_new_kv.argtypes = [ctypes.POINTER(_Cfg), p, p, p, p, p, p, p, p]
        lib.qsa_oracle_bf16k_turbo4v_attention.restype = ctypes.c_int
        lib.qsa_oracle_bf16k_turbo4v_attention.argtypes = [ctypes.POINTER(_Cfg)] + [p] * 13 + [ctypes.c_int64, p]
        lib.qsa_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


@dataclass
class Geometry:
    """Shape and numeric parameters of one call (plain values, no arrays)."""
    batch: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rotary_dim: int
    rope_theta: float
    rms_eps: float = 1e-6
    softmax_scale: float = 0.0          # 0 selects 1/sqrt(head_dim)
    dtype: str = "bf16"                  # storage dtype: "bf16" | "f32" | "f64"

    def _c(self) -> _Cfg:
        bits = {"bf16": 8, "f32": 24, "f64": 53}[self.dtype]
        return _Cfg(self.batch, self.q_len, self.num_q_heads, self.num_kv_heads,
                    self.head_dim, self.rotary_dim, float(self.rope_theta),
                    float(self.rms_eps), float(self.softmax_scale), bits)


def _f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.float64))


def _i32(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.int32))


def _i64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.int64))


def _cache(t):
    """Raw storage of a cache buffer and its dtype code (no copy of bf16 data)."""
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), BF16
        if t.dtype == torch.float32:
            return t.numpy(), F32
        return t.to(torch.float64).numpy(), F64
    a = np.ascontiguousarray(t)
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.float32:
        return a, F32
    return a.astype(np.float64), F64


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def round_to(x, dtype: str):
    """Round doubles to a storage dtype (ties to even) with the oracle's rounding."""
    lib = _load()
    bits = {"bf16": 8, "f32": 24, "f64": 53}[dtype]
    a = _f64(x)
    return np.vectorize(lambda v: lib.qsa_oracle_round(float(v), bits))(a)


def new_kv(geo: Geometry, k_new, v_new, w_k, positions):
    """Roped, normalized K rows and V rows of the new tokens, rounded to storage.

    Reading: the cache holds K after norm and rotation and V as given
    (mlxd PR #99 first review, issue 2: KV-shared layers take K "pre-rotated"
    from the source layer's cache); both rounded to nearest-even.
    """
    lib = _load()
    kn, vn, wk, pos = _f64(k_new), _f64(v_new), _f64(w_k), _i32(positions)
    kr = np.empty_like(kn)
    vr = np.empty_like(vn)
    rc = lib.qsa_oracle_new_kv(ctypes.byref(geo._c()), _ptr(kn), _ptr(vn), _ptr(wk),
                               _ptr(pos), _ptr(kr), _ptr(vr))
    if rc != 0:
        raise ValueError("oracle rejected the configuration")
    return kr, vr


def attention(geo: Geometry, q_gate, w_q, k_cache, v_cache, seq_offset, seq_lens, positions,
              k_rows=None, v_rows=None, rows=None, want_attn=False):
    """Gated attention of the new rows (see qsa_oracle.h for layouts).

    ``k_rows``/``v_rows`` (from :func:`new_kv`) supply keys n_b..n_b+L-1; pass
    ``None`` for both when those rows are already in the cache.  ``rows`` is an
    optional array of flat ``(b*L + l)*Hq + h`` indices.  Returns ``out`` (and
    the ungated ``attn`` when ``want_attn``) as float64 arrays, shape
    ``[B, L, Hq, D]`` or ``[n_rows, D]``.
    """
    lib = _load()
    qg, wq = _f64(q_gate), _f64(w_q)
    kc, kdt = _cache(k_cache)
    vc, vdt = _cache(v_cache)
    if kdt != vdt:
        raise ValueError("K and V caches must share a storage dtype")
    off, sl, pos = _i64(seq_offset), _i32(seq_lens), _i32(positions)
    kr = None if k_rows is None else _f64(k_rows)
    vr = None if v_rows is None else _f64(v_rows)
    D = geo.head_dim
    if rows is None:
        shape = (geo.batch, geo.q_len, geo.num_q_heads, D)
        r = None
        n = 0
    else:
        r = _i64(rows)
        n = r.size
        shape = (n, D)
    out = np.empty(shape, dtype=np.float64)
    att = np.empty(shape, dtype=np.float64) if want_attn else None
    rc = lib.qsa_oracle_attention(ctypes.byref(geo._c()), _ptr(qg), _ptr(wq), _ptr(kc),
                                  _ptr(vc), kdt, _ptr(off), _ptr(sl), _ptr(pos), _ptr(kr),
                                  _ptr(vr), _ptr(r), n, _ptr(out), _ptr(att))
    if rc != 0:
        raise ValueError("oracle rejected the configuration or a row index")
    return (out, att) if want_attn else out


def gated_attention(geo: Geometry, inputs: dict, rows=None, want_attn=False, fused=True):
    """Whole call: append the new rows (when ``fused``), then gated attention.

    ``inputs`` holds ``q_gate, k_new, v_new, k_cache, v_cache, w_q, w_k,
    seq_offset, seq_lens, positions`` (CPU tensors or arrays).  Returns
    ``(out, k_rows, v_rows)`` plus ``attn`` when requested.
    """
    kr = vr = None
    if fused:
        kr, vr = new_kv(geo, inputs["k_new"], inputs["v_new"], inputs["w_k"],
                        inputs["positions"])
    res = attention(geo, inputs["q_gate"], inputs["w_q"], inputs["k_cache"], inputs["v_cache"],
                    inputs["seq_offset"], inputs["seq_lens"], inputs["positions"], kr, vr,
                    rows=rows, want_attn=want_attn)
    if want_attn:
        out, att = res
        return out, kr, vr, att
    return res, kr, vr


def linear(x, w, dtype: str = "f64"):
    """y = x w^T for x [M, K] and w [N, K] in double, rounded to `dtype`."""
    lib = _load()
    xa, wa = _f64(x), _f64(w)
    M, K = xa.shape
    N = wa.shape[0]
    if wa.shape[1] != K:
        raise ValueError("x and w disagree on the inner size")
    y = np.empty((M, N), dtype=np.float64)
    bits = {"bf16": 8, "f32": 24, "f64": 53}[dtype]
    if lib.qsa_oracle_linear(_ptr(xa), _ptr(wa), M, N, K, bits, _ptr(y)) != 0:
        raise ValueError("oracle rejected the sizes")
    return y


def qkv_proj(geo: Geometry, hidden: int, x, w_qkv):
    """Fused q/k/v projection of x [B*L, hidden] and its split (see qsa_oracle.h).
    Returns q_gate [B, L, Hq, 2D], k_new and v_new [B, L, Hkv, D], rounded to
    the geometry's storage dtype."""
    lib = _load()
    xa, wa = _f64(x), _f64(w_qkv)
    B, L, Hq, Hkv, D = geo.batch, geo.q_len, geo.num_q_heads, geo.num_kv_heads, geo.head_dim
    if xa.shape != (B * L, hidden) or wa.shape != (2 * Hq * D + 2 * Hkv * D, hidden):
        raise ValueError("x or w_qkv has the wrong shape")
    qg = np.empty((B, L, Hq, 2 * D))
    kn = np.empty((B, L, Hkv, D))
    vn = np.empty((B, L, Hkv, D))
    if lib.qsa_oracle_qkv_proj(ctypes.byref(geo._c()), hidden, _ptr(xa), _ptr(wa), _ptr(qg), _ptr(kn),
                               _ptr(vn)) != 0:
        raise ValueError("oracle rejected the configuration")
    return qg, kn, vn


def o_proj(geo: Geometry, hidden: int, attn, w_o):
    """y [B*L, hidden] = attn [B*L, Hq*D] w_o^T, rounded to the storage dtype."""
    a = _f64(attn).reshape(geo.batch * geo.q_len, geo.num_q_heads * geo.head_dim)
    if _f64(w_o).shape != (hidden, geo.num_q_heads * geo.head_dim):
        raise ValueError("w_o has the wrong shape")
    return linear(a, w_o, geo.dtype)


# ------------------------------------------------------------------ Turbo8
# Turbo8 KV cache (Atlas docs, spark_model/forward/qwen3_5/mod.rs, MetalKvDtype::
# Turbo8 and LayerKvCache::alloc): FP8 E4M3 codes, one per element, and bf16
# scales, one per group of 16 elements, in the Walsh-Hadamard rotated basis,
# with WHT(Q) / iWHT(out) bookends around the attention.  The readings where the
# page is silent (scale rule, rounding, WHT normalisation) are in qsa_oracle.h.

def _u8(t):
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        t = t.view(torch.uint8) if t.dtype != torch.uint8 else t
        t = t.numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.uint8))


def _u16(t):
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        t = t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.int16) else t
        t = t.numpy()
    return np.ascontiguousarray(np.asarray(t).view(np.uint16) if np.asarray(t).dtype == np.int16
                                else np.asarray(t, dtype=np.uint16))


def e4m3_value(codes) -> np.ndarray:
    """Values of E4M3 codes (uint8 array)."""
    lib = _load()
    c = _u8(codes)
    return np.vectorize(lambda v: lib.qsa_oracle_e4m3_value(int(v)), otypes=[np.float64])(c)


def e4m3_code(x) -> np.ndarray:
    """E4M3 codes of x (nearest, ties to even, saturating)."""
    lib = _load()
    return np.vectorize(lambda v: lib.qsa_oracle_e4m3_code(float(v)), otypes=[np.uint8])(_f64(x))


def wht(x) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform along the last axis."""
    lib = _load()
    a = _f64(x)
    flat = a.reshape(-1, a.shape[-1])
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[i])
        res = np.empty_like(row)
        if lib.qsa_oracle_wht(_ptr(row), row.size, _ptr(res)) != 0:
            raise ValueError("the transform length must be a power of two")
        out[i] = res
    return out.reshape(a.shape)


def turbo8_quantize(x):
    """Turbo8 codes (uint8, same shape) and scale bits (uint16, last axis / 16) of x."""
    lib = _load()
    a = _f64(x)
    flat = a.reshape(-1, a.shape[-1])
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty((flat.shape[0], flat.shape[1] // 16), dtype=np.uint16)
    for i in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[i])
        cr = np.empty(row.size, dtype=np.uint8)
        sr = np.empty(row.size // 16, dtype=np.uint16)
        if lib.qsa_oracle_turbo8_quantize(_ptr(row), row.size, _ptr(cr), _ptr(sr)) != 0:
            raise ValueError("Turbo8 rows need a multiple of 16 elements")
        codes[i], scales[i] = cr, sr
    return codes.reshape(a.shape), scales.reshape(a.shape[:-1] + (a.shape[-1] // 16,))


def turbo8_dequantize(codes, scale_bits) -> np.ndarray:
    """codes x scales in double (the cache rows a Turbo8 attention reads)."""
    c = e4m3_value(codes)
    sb = _u16(scale_bits).astype(np.uint32) << 16
    s = sb.view(np.float32).astype(np.float64)
    return c * np.repeat(s, 16, axis=-1)


def turbo8_new_kv(geo: Geometry, k_new, v_new, w_k, positions):
    """Turbo8 rows of the new tokens: (k_codes, k_scales, v_codes, v_scales)."""
    lib = _load()
    kn, vn, wk, pos = _f64(k_new), _f64(v_new), _f64(w_k), _i32(positions)
    D = geo.head_dim
    kc = np.empty(kn.shape, dtype=np.uint8)
    vc = np.empty(kn.shape, dtype=np.uint8)
    ks = np.empty(kn.shape[:-1] + (D // 16,), dtype=np.uint16)
    vs = np.empty_like(ks)
    if lib.qsa_oracle_turbo8_new_kv(ctypes.byref(geo._c()), _ptr(kn), _ptr(vn), _ptr(wk), _ptr(pos), _ptr(kc),
                                    _ptr(ks), _ptr(vc), _ptr(vs)) != 0:
        raise ValueError("oracle rejected the configuration")
    return kc, ks, vc, vs


def turbo8_attention(geo: Geometry, q_gate, w_q, k_codes, k_scales, v_codes, v_scales, seq_offset, seq_lens,
                     positions, new=None, rows=None):
    """Gated attention over a Turbo8 cache; `new` = turbo8_new_kv(...) output for
    keys n_b .. n_b+L-1, or None when those rows are in the cache."""
    lib = _load()
    qg, wq = _f64(q_gate), _f64(w_q)
    kc, ks, vc, vs = _u8(k_codes), _u16(k_scales), _u8(v_codes), _u16(v_scales)
    off, sl, pos = _i64(seq_offset), _i32(seq_lens), _i32(positions)
    nk = [None] * 4 if new is None else [_u8(new[0]), _u16(new[1]), _u8(new[2]), _u16(new[3])]
    D = geo.head_dim
    if rows is None:
        out = np.empty((geo.batch, geo.q_len, geo.num_q_heads, D))
        r, n = None, 0
    else:
        r = _i64(rows)
        n = r.size
        out = np.empty((n, D))
    rc = lib.qsa_oracle_turbo8_attention(ctypes.byref(geo._c()), _ptr(qg), _ptr(wq), _ptr(kc), _ptr(ks), _ptr(vc),
                                         _ptr(vs), _ptr(off), _ptr(sl), _ptr(pos), _ptr(nk[0]), _ptr(nk[1]),
                                         _ptr(nk[2]), _ptr(nk[3]), _ptr(r), n, _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the configuration or a row index")
    return out


def turbo8_gated_attention(geo: Geometry, inputs: dict, rows=None, fused=True):
    """Whole call on a Turbo8 cache (inputs from make_turbo8_inputs): quantize and
    append the new rows (when fused), then attend.  Returns (out, new rows)."""
    new = turbo8_new_kv(geo, inputs["k_new"], inputs["v_new"], inputs["w_k"], inputs["positions"]) if fused else None
    out = turbo8_attention(geo, inputs["q_gate"], inputs["w_q"], inputs["k_codes"], inputs["k_scales"],
                           inputs["v_codes"], inputs["v_scales"], inputs["seq_offset"], inputs["seq_lens"],
                           inputs["positions"], new=new, rows=rows)
    return out, new


# ------------------------------------------------------------------ bf16 K + Turbo4 V
# Atlas docs, spark_model/forward/qwen3_5/mod.rs, MetalKvDtype::Bf16KTurbo4V and
# LayerKvCache::alloc: K stays a bf16 cache (not rotated); V is Turbo4 -- 4-bit
# Lloyd-Max codebook indices and an FP8 scale per group of 16 (matched-norm L2)
# in the WHT basis -- with the iWHT(out) bookend.  Readings (codebook, index
# rule, scale rule, packing) are in qsa_oracle.h.

def lloyd_max_normal(levels: int = 16) -> np.ndarray:
    """The Lloyd-Max quantizer levels of N(0, 1), ascending."""
    c = np.empty(levels)
    if _load().qsa_oracle_lloyd_max_normal(levels, _ptr(c)) != 0:
        raise ValueError("levels must be in 2 .. 256")
    return c


def turbo4_quantize(x, cb=None):
    """Turbo4 codes (uint8, last axis / 2, two per byte) and E4M3 scales (uint8,
    last axis / 16) of x."""
    lib = _load()
    cb = lloyd_max_normal() if cb is None else np.ascontiguousarray(cb, dtype=np.float64)
    a = _f64(x)
    flat = a.reshape(-1, a.shape[-1])
    n = flat.shape[1]
    codes = np.empty((flat.shape[0], n // 2), dtype=np.uint8)
    scales = np.empty((flat.shape[0], n // 16), dtype=np.uint8)
    for i in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[i])
        cr, sr = np.empty(n // 2, dtype=np.uint8), np.empty(n // 16, dtype=np.uint8)
        if lib.qsa_oracle_turbo4_quantize(_ptr(row), n, _ptr(cb), _ptr(cr), _ptr(sr)) != 0:
            raise ValueError("Turbo4 rows need a multiple of 16 elements")
        codes[i], scales[i] = cr, sr
    return codes.reshape(a.shape[:-1] + (n // 2,)), scales.reshape(a.shape[:-1] + (n // 16,))


def turbo4_dequantize(codes, scales, cb=None) -> np.ndarray:
    """codebook level times group scale, in double."""
    lib = _load()
    cb = lloyd_max_normal() if cb is None else np.ascontiguousarray(cb, dtype=np.float64)
    c, s = _u8(codes), _u8(scales)
    n = c.shape[-1] * 2
    cf, sf = c.reshape(-1, n // 2), s.reshape(-1, n // 16)
    out = np.empty((cf.shape[0], n))
    for i in range(cf.shape[0]):
        row = np.empty(n)
        lib.qsa_oracle_turbo4_dequantize(_ptr(np.ascontiguousarray(cf[i])), _ptr(np.ascontiguousarray(sf[i])), n,
                                         _ptr(cb), _ptr(row))
        out[i] = row
    return out.reshape(c.shape[:-1] + (n,))


def bf16k_turbo4v_new_kv(geo: Geometry, k_new, v_new, w_k, positions, cb=None):
    """New rows: (K rows as bf16 values in double, V codes, V scales)."""
    lib = _load()
    cb = lloyd_max_normal() if cb is None else np.ascontiguousarray(cb, dtype=np.float64)
    kn, vn, wk, pos = _f64(k_new), _f64(v_new), _f64(w_k), _i32(positions)
    D = geo.head_dim
    kr = np.empty(kn.shape)
    vc = np.empty(kn.shape[:-1] + (D // 2,), dtype=np.uint8)
    vs = np.empty(kn.shape[:-1] + (D // 16,), dtype=np.uint8)
    if lib.qsa_oracle_bf16k_turbo4v_new_kv(ctypes.byref(geo._c()), _ptr(kn), _ptr(vn), _ptr(wk), _ptr(pos), _ptr(cb),
                                           _ptr(kr), _ptr(vc), _ptr(vs)) != 0:
        raise ValueError("oracle rejected the configuration")
    return kr, vc, vs


def bf16k_turbo4v_attention(geo: Geometry, q_gate, w_q, k_cache, v_codes, v_scales, seq_offset, seq_lens, positions,
                            new=None, rows=None, cb=None):
    """Gated attention with K from a bf16 cache and V from Turbo4 rows; `new` =
    bf16k_turbo4v_new_kv(...) output for keys n_b .. n_b+L-1, or None when those
    rows are in the cache."""
    lib = _load()
    cb = lloyd_max_normal() if cb is None else np.ascontiguousarray(cb, dtype=np.float64)
    qg, wq = _f64(q_gate), _f64(w_q)
    kc, vc, vs = _u16(k_cache), _u8(v_codes), _u8(v_scales)
    off, sl, pos = _i64(seq_offset), _i32(seq_lens), _i32(positions)
    nk = [None] * 3 if new is None else [np.ascontiguousarray(new[0], dtype=np.float64), _u8(new[1]), _u8(new[2])]
    D = geo.head_dim
    if rows is None:
        out = np.empty((geo.batch, geo.q_len, geo.num_q_heads, D))
        r, n = None, 0
    else:
        r = _i64(rows)
        n = r.size
        out = np.empty((n, D))
    rc = lib.qsa_oracle_bf16k_turbo4v_attention(ctypes.byref(geo._c()), _ptr(qg), _ptr(wq), _ptr(kc), _ptr(vc),
                                                _ptr(vs), _ptr(off), _ptr(sl), _ptr(pos), _ptr(cb), _ptr(nk[0]),
                                                _ptr(nk[1]), _ptr(nk[2]), _ptr(r), n, _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the configuration or a row index")
    return out


def bf16k_turbo4v_gated_attention(geo: Geometry, inputs: dict, rows=None, fused=True):
    """Whole call on a bf16-K / Turbo4-V cache (inputs from make_turbo4v_inputs):
    the new rows (when fused), then attention.  Returns (out, new rows)."""
    new = (bf16k_turbo4v_new_kv(geo, inputs["k_new"], inputs["v_new"], inputs["w_k"], inputs["positions"])
           if fused else None)
    out = bf16k_turbo4v_attention(geo, inputs["q_gate"], inputs["w_q"], inputs["k_cache"], inputs["v_codes"],
                                  inputs["v_scales"], inputs["seq_offset"], inputs["seq_lens"], inputs["positions"],
                                  new=new, rows=rows)
    return out, new


def threads() -> int:
    return int(_load().qsa_oracle_threads())
