"""ctypes binding of libqsa.so (declared in include/qsa.h).

Argument marshalling only: tensors become device pointers, the configuration
becomes a ``qsa_cfg`` struct, negative status codes become ``QSAError``.  Every
step of the computation runs in the library's HIP kernels; there is no other
path.  Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsa.so")

QSA_OK, QSA_ERR_INVALID, QSA_ERR_UNSUPPORTED, QSA_ERR_WORKSPACE, QSA_ERR_DEVICE = 0, -1, -2, -3, -4
QSA_BF16, QSA_F32 = 0, 1
QSA_KV_NATIVE, QSA_KV_TURBO8, QSA_KV_BF16K_TURBO4V = 0, 1, 2
_DT = {torch.bfloat16: QSA_BF16, torch.float32: QSA_F32}

EXPORTS = ("qsa_workspace_size", "qsa_append_kv", "qsa_gated_attention", "qsa_gated_attention_noalloc",
           "qsa_qkv_proj", "qsa_o_proj", "qsa_gdn_decode", "qsa_describe_plan", "qsa_last_error")
NOALLOC_SCRATCH_BYTES = 64 << 20     # QSA_NOALLOC_SCRATCH_BYTES


class QSAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"qsa status {code}: {msg}")
        self.code = code


class Cfg(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("rotary_dim", ctypes.c_int32),
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32), ("force_splits", ctypes.c_int32),
        ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("timing_begin", ctypes.c_void_p), ("timing_end", ctypes.c_void_p),
    ]


class KVCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("seq_offset", ctypes.c_void_p), ("capacity", ctypes.c_void_p),
        ("num_rows", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
    ]


class GdnCfg(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
        ("k_head_dim", ctypes.c_int32), ("v_head_dim", ctypes.c_int32), ("conv_kernel", ctypes.c_int32),
        ("rms_eps", ctypes.c_float), ("stream", ctypes.c_void_p),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libqsa.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m gated_gqa_attention_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        lib.qsa_workspace_size.restype = ctypes.c_size_t
        lib.qsa_workspace_size.argtypes = [ctypes.POINTER(Cfg)]
        lib.qsa_append_kv.restype = ctypes.c_int
        lib.qsa_append_kv.argtypes = [p, p, ctypes.POINTER(KVCache), p, p, ctypes.POINTER(Cfg)]
        lib.qsa_gated_attention.restype = ctypes.c_int
        lib.qsa_gated_attention.argtypes = [p, p, p, ctypes.POINTER(KVCache), p, p,
                                            ctypes.POINTER(Cfg), p]
        lib.qsa_gated_attention_noalloc.restype = ctypes.c_int
        lib.qsa_gated_attention_noalloc.argtypes = [p, p, p, ctypes.POINTER(KVCache), p, p,
                                                    ctypes.POINTER(Cfg), p]
        lib.qsa_qkv_proj.restype = ctypes.c_int
        lib.qsa_qkv_proj.argtypes = [p, p, ctypes.c_int32, ctypes.POINTER(Cfg), p, p, p]
        lib.qsa_o_proj.restype = ctypes.c_int
        lib.qsa_o_proj.argtypes = [p, p, ctypes.c_int32, ctypes.POINTER(Cfg), p]
        lib.qsa_gdn_decode.restype = ctypes.c_int
        lib.qsa_gdn_decode.argtypes = [p] * 11 + [ctypes.POINTER(GdnCfg)]
        lib.qsa_describe_plan.restype = ctypes.c_int
        lib.qsa_describe_plan.argtypes = [ctypes.POINTER(Cfg), ctypes.c_char_p, ctypes.c_size_t]
        lib.qsa_last_error.restype = ctypes.c_char_p
        lib.qsa_last_error.argtypes = []
        _lib = lib
    return _lib


def last_error() -> str:
    return load().qsa_last_error().decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(rc: int):
    if rc != QSA_OK:
        raise QSAError(rc, last_error())


def make_cfg(*, batch, q_len, num_q_heads, num_kv_heads, head_dim, rotary_dim, rope_theta,
             rms_eps, dtype, max_seq_len, q_norm_w=None, k_norm_w=None, workspace=None,
             softmax_scale=0.0, force_splits=0, stream=None) -> Cfg:
    """Build a qsa_cfg.  ``dtype`` is a torch dtype; tensors are passed as device pointers."""
    if stream is None and torch.cuda.is_available():
        stream = torch.cuda.current_stream()
    stream_handle = None if stream is None else (stream if isinstance(stream, int) else stream.cuda_stream)
    return Cfg(batch, q_len, num_q_heads, num_kv_heads, head_dim, rotary_dim, float(rope_theta),
               float(rms_eps), float(softmax_scale), _DT[dtype] if not isinstance(dtype, int) else dtype,
               max_seq_len, force_splits, _ptr(q_norm_w), _ptr(k_norm_w), _ptr(workspace),
               0 if workspace is None else workspace.numel() * workspace.element_size(),
               stream_handle)


def make_kv(k_cache, v_cache, seq_offset, capacity=None, block_table=None, block_size=0,
            k_scales=None, v_scales=None) -> KVCache:
    """Describe a token-major cache: k/v ``[rows, Hkv, D]``; contiguous with
    seq_offset int64 ``[B]``, or paged with block_table int32 ``[B, max_blocks]``.
    With k_scales and v_scales ``[rows, Hkv, D/16]`` (bf16) the cache is Turbo8
    (k/v hold E4M3 codes); with v_scales only (E4M3 bytes) it is bf16 K + Turbo4
    V (k bf16 rows, v ``[rows, Hkv, D/2]`` 4-bit indices)."""
    max_blocks = 0 if block_table is None else int(block_table.shape[1])
    kind = QSA_KV_NATIVE if v_scales is None else QSA_KV_TURBO8 if k_scales is not None else QSA_KV_BF16K_TURBO4V
    return KVCache(_ptr(k_cache), _ptr(v_cache), _ptr(seq_offset), _ptr(capacity),
                   int(k_cache.shape[0]), _ptr(block_table), int(block_size), max_blocks,
                   kind, _ptr(k_scales), _ptr(v_scales))


def workspace_size(cfg: Cfg) -> int:
    n = load().qsa_workspace_size(ctypes.byref(cfg))
    if n == 0:
        raise QSAError(QSA_ERR_INVALID, last_error())
    return int(n)


def describe_plan(cfg: Cfg) -> str:
    buf = ctypes.create_string_buffer(512)
    rc = load().qsa_describe_plan(ctypes.byref(cfg), buf, len(buf))
    if rc < 0:
        raise QSAError(rc, last_error())
    return buf.value.decode()


def append_kv(cfg: Cfg, kv: KVCache, k_new, v_new, seq_lens, positions) -> None:
    _check(load().qsa_append_kv(_ptr(k_new), _ptr(v_new), ctypes.byref(kv), _ptr(seq_lens),
                                _ptr(positions), ctypes.byref(cfg)))


def gated_attention(cfg: Cfg, kv: KVCache, q_gate, k_new, v_new, seq_lens, positions, out) -> None:
    _check(load().qsa_gated_attention(_ptr(q_gate), _ptr(k_new), _ptr(v_new), ctypes.byref(kv),
                                      _ptr(seq_lens), _ptr(positions), ctypes.byref(cfg), _ptr(out)))


def gated_attention_noalloc(cfg: Cfg, kv: KVCache, q_gate, k_new, v_new, seq_lens, positions, out) -> None:
    """qsa_gated_attention_noalloc: the library's own per-GPU scratch instead of
    ``cfg.workspace`` (which is ignored)."""
    _check(load().qsa_gated_attention_noalloc(_ptr(q_gate), _ptr(k_new), _ptr(v_new), ctypes.byref(kv),
                                              _ptr(seq_lens), _ptr(positions), ctypes.byref(cfg),
                                              _ptr(out)))


def qkv_proj(cfg: Cfg, x, w_qkv, hidden: int, q_gate, k_new, v_new) -> None:
    """qsa_qkv_proj: x [rows, hidden] times the fused q/k/v weight, split into q_gate, k_new, v_new."""
    _check(load().qsa_qkv_proj(_ptr(x), _ptr(w_qkv), int(hidden), ctypes.byref(cfg), _ptr(q_gate), _ptr(k_new),
                               _ptr(v_new)))


def o_proj(cfg: Cfg, attn, w_o, hidden: int, y) -> None:
    """qsa_o_proj: y [rows, hidden] = attn [rows, Hq*D] times w_o^T."""
    _check(load().qsa_o_proj(_ptr(attn), _ptr(w_o), int(hidden), ctypes.byref(cfg), _ptr(y)))


def make_gdn_cfg(*, batch, num_k_heads, num_v_heads, k_head_dim, v_head_dim, conv_kernel, rms_eps=1e-6,
                 stream=None) -> GdnCfg:
    return GdnCfg(batch, num_k_heads, num_v_heads, k_head_dim, v_head_dim, conv_kernel, rms_eps,
                  stream if stream is not None else torch.cuda.current_stream().cuda_stream
                  if torch.cuda.is_available() else None)


def gdn_decode(cfg: GdnCfg, qkv, z, a, b, conv_w, a_log, dt_bias, norm_w, conv_state, state, y) -> None:
    """qsa_gdn_decode: one GatedDeltaNet decode step; conv_state and state are updated in place."""
    _check(load().qsa_gdn_decode(_ptr(qkv), _ptr(z), _ptr(a), _ptr(b), _ptr(conv_w), _ptr(a_log), _ptr(dt_bias),
                                 _ptr(norm_w), _ptr(conv_state), _ptr(state), _ptr(y), ctypes.byref(cfg)))
