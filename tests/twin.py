"""A second, independent CPU derivation of the gated GQA attention core (NumPy, float64).

Written differently from the C oracle on purpose so that a slip in either one
shows up as a disagreement:

* the rotation is an explicit r x r block-rotation matrix per position,
* grouped-query attention is plain multi-head attention after repeating each
  KV head G times (``np.repeat`` along the head axis),
* scores, masking and softmax are whole-matrix operations.

It also carries *mutants*: single plausible mistakes (a dropped gate, a
swapped split, a shifted position, the wrong head map, ...).  The mutation
tests check that each mutant moves the result far past the parity tolerance,
i.e. that the inputs and tolerances used for parity would catch that mistake.
"""
from __future__ import annotations

import numpy as np
import torch

MUTANTS = (
    "no_gate",          # out = attn (sigmoid gate dropped)
    "swap_split",       # query and gate halves exchanged
    "pos_plus1",        # rotary position off by one
    "head_mod",         # query head h uses KV head h % Hkv instead of h // G
    "no_causal",        # new rows see every new row
    "no_qnorm",         # query RMS norm dropped (weight still applied)
    "no_knorm",         # key RMS norm dropped (weight still applied)
    "freq_over_D",      # theta^(-2i/D) instead of theta^(-2i/r)
    "rope_interleaved", # pairs (2i, 2i+1) instead of (i, i + r/2)
    "scale_r",          # 1/sqrt(r) instead of 1/sqrt(D)
    "exclude_self",     # row l does not see its own key
)


def _f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def round_bits(x: np.ndarray, bits: int) -> np.ndarray:
    """Round to `bits` significand bits, ties to even (np.rint rounds half to even)."""
    if bits >= 53:
        return x
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, bits)), e - bits)


def rotation_matrix(p: float, r: int, theta: float, D: int, mutant=None) -> np.ndarray:
    """Full D x D matrix applying the partial rotation at position p."""
    R = np.eye(D)
    h = r // 2
    denom = D if mutant == "freq_over_D" else r
    for i in range(h):
        a = p * theta ** (-2.0 * i / denom)
        c, s = np.cos(a), np.sin(a)
        if mutant == "rope_interleaved":
            u, v = 2 * i, 2 * i + 1
        else:
            u, v = i, i + h
        R[u, u], R[u, v], R[v, u], R[v, v] = c, -s, s, c
    return R


def _norm(x, w, eps, skip=False):
    if skip:
        return x * w
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def twin(w, inputs: dict, store_bits: int, mutant: str | None = None, fused: bool = True):
    """Return (out_rounded, attn) of shape [B, L, Hq, D] for workload-like `w`.

    `w` needs batch, q_len, num_q_heads, num_kv_heads, head_dim, rotary_dim,
    rope_theta, rms_eps attributes.  `store_bits` is 8 for bf16, 24 for fp32.
    """
    if mutant is not None and mutant not in MUTANTS:
        raise ValueError(mutant)
    B, L, Hq, Hkv, D = w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    r, theta, eps = w.rotary_dim, w.rope_theta, w.rms_eps
    qg = _f64(inputs["q_gate"])
    kn, vn = _f64(inputs["k_new"]), _f64(inputs["v_new"])
    kc, vc = _f64(inputs["k_cache"]), _f64(inputs["v_cache"])
    wq, wk = _f64(inputs["w_q"]), _f64(inputs["w_k"])
    n_all = np.asarray(inputs["seq_lens"]).astype(np.int64)
    off = np.asarray(inputs["seq_offset"]).astype(np.int64)
    pos = np.asarray(inputs["positions"]).astype(np.float64)
    if mutant == "pos_plus1":
        pos = pos + 1.0

    q, z = qg[..., :D], qg[..., D:]
    if mutant == "swap_split":
        q, z = z, q
    scale = 1.0 / np.sqrt(r if mutant == "scale_r" else D)

    out = np.zeros((B, L, Hq, D))
    attn = np.zeros((B, L, Hq, D))
    for b in range(B):
        n = int(n_all[b])
        rots = [rotation_matrix(pos[b, l], r, theta, D, mutant) for l in range(L)]
        qt = _norm(q[b], wq, eps, skip=(mutant == "no_qnorm"))          # [L, Hq, D]
        qt = np.stack([qt[l] @ rots[l].T for l in range(L)])
        keys = kc[off[b]:off[b] + n + L].copy()                          # [n+L, Hkv, D]
        vals = vc[off[b]:off[b] + n + L].copy()
        if fused:
            kt = _norm(kn[b], wk, eps, skip=(mutant == "no_knorm"))      # [L, Hkv, D]
            kt = np.stack([kt[l] @ rots[l].T for l in range(L)])
            keys[n:n + L] = round_bits(kt, store_bits)
            vals[n:n + L] = round_bits(vn[b], store_bits)
        if mutant == "head_mod":
            kh, vh = np.tile(keys, (1, G, 1)), np.tile(vals, (1, G, 1))
        else:
            kh, vh = np.repeat(keys, G, axis=1), np.repeat(vals, G, axis=1)   # [n+L, Hq, D]
        s = np.einsum("lhd,jhd->hlj", qt, kh) * scale                    # [Hq, L, n+L]
        j = np.arange(n + L)[None, :]
        lim = n + np.arange(L)[:, None]
        if mutant == "no_causal":
            mask = np.ones((L, n + L), dtype=bool)
        elif mutant == "exclude_self":
            mask = j < lim
            mask[:, 0] = True
        else:
            mask = j <= lim
        s = np.where(mask[None], s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        a = np.einsum("hlj,jhd->lhd", p, vh)                               # [L, Hq, D]
        attn[b] = a
        g = 1.0 / (1.0 + np.exp(-z[b]))
        o = a if mutant == "no_gate" else a * g
        out[b] = round_bits(o, store_bits)
    return out, attn
