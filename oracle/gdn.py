"""CPU oracle for one GatedDeltaNet decode step (the linear-attention layer type
of hybrid Qwen3.5).

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product library
never imports this module, and this module never imports the product library.

Plain NumPy in IEEE double, one sequence and one state head at a time, in the
order the steps are listed here.

What the pages fix (Atlas docs, ``spark_model/forward/qwen3_5/mod.rs``):

* sizes -- ``Qwen35ForwardConfig``: num_k_heads_lin, num_v_heads_lin,
  k_head_dim_lin, v_head_dim_lin, conv_kernel_size;
  ``qkv_total_lin() = 2 Hk Dk + Hv Dv`` channels (queries, keys, values, in that
  order); ``num_state_heads() = Hv`` (gate, beta, dt_bias and A_log run over
  the value heads);
* tensors -- ``LinearAttentionLayer``: a_log FP32 [Hv], dt_bias BF16 [Hv],
  conv1d_weight BF16 [C, K, 1], norm_weight BF16 [Dv];
  ``LinearAttentionState``: conv1d_state FP32 [C, K], gdn_state FP32
  [Hv, Dk, Dv], kept across tokens; ``LinearAttentionScratch``: gate and beta
  FP32 [Hv], y and y_norm;
* the step's kernels, in order -- ``Qwen35Kernels``:
  causal_conv1d_update_l2norm, gdn_compute_gate, sigmoid_bf16_to_f32,
  gated_delta_rule_decode.

The update rule itself is not printed.  It is taken as the published gated
delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta Networks: Improving
Mamba2 with Delta Rule", 2024) in the form those names and shapes imply.  The
readings (parity of these choices with the pages is unpinned; the tests pin
the arithmetic against closed forms and against an independent implementation
of the same rule):

R1  convolution: per channel, a causal depthwise convolution over the K most
    recent inputs.  The state row holds them oldest first; the step shifts the
    new input in, the output is sum_j w[c, j] state'[c, j], then SiLU.
R2  l2norm: q and k of every key head become x / sqrt(sum x^2 + 1e-6).
R3  the query is scaled by 1 / sqrt(Dk).
R4  gate (log decay): g = -exp(A_log) softplus(a + dt_bias);
    beta = sigmoid(b).
R5  value head h reads key head h // (Hv / Hk).
R6  state step:  S <- exp(g) S;   S <- S + beta k (v - S^T k)^T;   o = S^T q
    (S is [Dk, Dv]).
R7  output: a gated RMS norm per value head,
    y = o / sqrt(mean(o^2) + eps) * norm_weight * silu(z).
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6


def _f64(t) -> np.ndarray:
    """A tensor or array as float64 (bf16 and fp32 values are exact in it)."""
    if hasattr(t, "detach"):
        t = t.detach().cpu().float().numpy()
    return np.asarray(t, dtype=np.float64)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def softplus(x):
    """log(1 + e^x), written so that large x does not overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 30.0, x + np.log1p(np.exp(-np.minimum(x, 700.0))), np.log1p(np.exp(np.minimum(x, 30.0))))


def conv_update(conv_state_row: np.ndarray, x: float, w_row: np.ndarray):
    """R1, one channel: the state holds the K latest inputs oldest first; the new
    input x is shifted in and the output is the dot product with the channel's
    taps, then SiLU (Atlas ``causal_conv1d_update_l2norm``, conv1d_state [C, K])."""
    new_state = np.concatenate([conv_state_row[1:], [x]])
    return silu(float(np.dot(w_row, new_state))), new_state


def l2norm(v: np.ndarray) -> np.ndarray:
    """R2: v / sqrt(sum v^2 + 1e-6)."""
    return v / np.sqrt(np.sum(v * v) + L2_EPS)


def gate(a: float, dt_bias: float, a_log: float) -> float:
    """R4: the log decay g = -exp(A_log) softplus(a + dt_bias) (Atlas
    ``gdn_compute_gate``; a_log FP32, dt_bias BF16)."""
    return float(-np.exp(a_log) * softplus(a + dt_bias))


def beta(b: float) -> float:
    """R4: sigmoid(b) (Atlas ``sigmoid_bf16_to_f32``)."""
    return float(sigmoid(b))


def delta_rule_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, g: float, bt: float):
    """R6 for one state head (S [Dk, Dv], q and k [Dk], v [Dv]): decay, then the
    delta-rule write of v at key k with strength beta, then the read at q
    (Atlas ``gated_delta_rule_decode``, gdn_state FP32 [Hv, Dk, Dv])."""
    S = np.exp(g) * S
    S = S + bt * np.outer(k, v - S.T @ k)
    return S.T @ q, S


def gated_rmsnorm(o: np.ndarray, z: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """R7: o / sqrt(mean(o^2) + eps) * w * silu(z) over one value head."""
    return o / np.sqrt(np.mean(o * o) + eps) * w * silu(z)


def gdn_decode(x: dict, num_k_heads: int, num_v_heads: int, k_head_dim: int, v_head_dim: int,
               rms_eps: float = 1e-6, seqs=None) -> dict:
    """One decode step for every sequence (or those listed in ``seqs``).

    x holds the inputs as laid out by the seeded generator: qkv [B, C],
    z [B, Hv Dv], a and b [B, Hv], conv_w [C, K], a_log [Hv], dt_bias [Hv],
    norm_w [Dv], conv_state [B, C, K], state [B, Hv, Dk, Dv].  Returns float64
    y [B, Hv, Dv] (the gated-norm output), conv_state and state after the step;
    sequences not listed keep zeros in y and their old states."""
    Hk, Hv, Dk, Dv = num_k_heads, num_v_heads, k_head_dim, v_head_dim
    qkv, z, a, b = _f64(x["qkv"]), _f64(x["z"]), _f64(x["a"]), _f64(x["b"])
    conv_w, a_log, dt_bias, norm_w = _f64(x["conv_w"]), _f64(x["a_log"]), _f64(x["dt_bias"]), _f64(x["norm_w"])
    conv_state, state = _f64(x["conv_state"]).copy(), _f64(x["state"]).copy()
    B, C = qkv.shape
    assert C == 2 * Hk * Dk + Hv * Dv and Hv % Hk == 0
    y = np.zeros((B, Hv, Dv))
    for s in (range(B) if seqs is None else seqs):
        conv_out = np.empty(C)
        for c in range(C):
            conv_out[c], conv_state[s, c] = conv_update(conv_state[s, c], qkv[s, c], conv_w[c])
        qs = conv_out[:Hk * Dk].reshape(Hk, Dk)
        ks = conv_out[Hk * Dk:2 * Hk * Dk].reshape(Hk, Dk)
        vs = conv_out[2 * Hk * Dk:].reshape(Hv, Dv)
        for h in range(Hv):
            kh = h // (Hv // Hk)                                           # R5
            q = l2norm(qs[kh]) / np.sqrt(Dk)                               # R2, R3
            k = l2norm(ks[kh])
            o, state[s, h] = delta_rule_step(state[s, h], q, k, vs[h], gate(a[s, h], dt_bias[h], a_log[h]),
                                             beta(b[s, h]))
            y[s, h] = gated_rmsnorm(o, z[s, h * Dv:(h + 1) * Dv], norm_w, rms_eps)
    return {"y": y, "conv_state": conv_state, "state": state}
