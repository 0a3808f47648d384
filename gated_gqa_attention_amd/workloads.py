"""Seeded synthetic inputs for the gated GQA attention core.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no norm, rotation, softmax or gate).  Both the HIP path's
tests/benchmark and the CPU oracle's callers take their inputs from here.

Shapes follow the pages' workloads: the Qwen3.5-4B attention geometry
(16 query / 4 KV heads, head_dim 256, rotary_dim 64, theta 1e7, eps 1e-6 --
Atlas ``qwen3_5/mod.rs``, ``Qwen35ForwardConfig::qwen3_5_4b_mlx_int8``) and the
24-query / 2-KV-head, dim-256, four-row speculative-verify case (DS4Server
issue #113, Reproduction).

Recipe (one ``torch.Generator('cpu')`` per workload, seeded with its seed):

1. ragged workloads only: prior lengths ``randint(lo, hi + 1, (B,))``;
2. ``q_gate`` ``randn(B, L, Hq, 2D)``, then ``k_new``, ``v_new``
   ``randn(B, L, Hkv, D)``;
3. cached K rows, sequence by sequence ``randn(n_b, Hkv, D)``, then cached V
   rows the same way;
4. ``w_q = 1 + 0.1 randn(D)``, ``w_k = 1 + 0.1 randn(D)``;
5. stress variant only: per (b, l, head) scale factors drawn from {0.05, 20}
   (``randint(0, 2)``) for the query half of ``q_gate`` and for ``k_new``;
6. every array is drawn in fp32 and then cast to the storage dtype
   (bf16: round to nearest even, as ``Tensor.to`` does).

Cache layout: token-major rows of ``[Hkv, D]``; sequence b owns rows
``seq_offset[b] .. seq_offset[b] + capacity[b] - 1``; rows past ``n_b`` are
zero.  Uniform batches give every sequence ``capacity = n + L`` rows; ragged
batches pack sequences back to back with ``capacity_b = n_b + L``.  Positions
of the new rows are ``n_b + l``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rotary_dim: int
    rope_theta: float
    dtype: str
    prior: int                      # cached rows per sequence (uniform batches)
    seed: int
    rms_eps: float = 1e-6
    ragged: tuple | None = None     # (lo, hi): prior lengths drawn uniformly in [lo, hi]
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", batch=1, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
        rotary_dim=16, rope_theta=1e4, dtype="f32", prior=32, seed=1,
        description="tiny fp32 check: 4/1 heads, D 64, r 16, 32 cached tokens"),
    "decode_4b": Workload(
        "decode_4b", batch=1, q_len=1, num_q_heads=16, num_kv_heads=4, head_dim=256,
        rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=4096, seed=2,
        description="Qwen3.5-4B single-stream decode, 4096 cached tokens"),
    "verify_24x2": Workload(
        "verify_24x2", batch=8, q_len=4, num_q_heads=24, num_kv_heads=2, head_dim=256,
        rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=2048, seed=3,
        description="speculative verify: 8 sequences x 4 causal rows, 24/2 heads, 2048 cached"),
    "ragged_4b": Workload(
        "ragged_4b", batch=64, q_len=1, num_q_heads=16, num_kv_heads=4, head_dim=256,
        rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=0, seed=4, ragged=(512, 32768),
        description="ragged batched decode: 64 sequences, cached lengths U[512, 32768]"),
    "prefill_4b": Workload(
        "prefill_4b", batch=1, q_len=2048, num_q_heads=16, num_kv_heads=4, head_dim=256,
        rotary_dim=64, rope_theta=1e7, dtype="bf16", prior=30720, seed=5,
        description="long prefill chunk: 2048 causal rows on 30720 cached tokens"),
}


def prior_lengths(w: Workload, gen: torch.Generator | None = None) -> torch.Tensor:
    """Cached length per sequence (draw step 1 for ragged workloads)."""
    if w.ragged is None:
        return torch.full((w.batch,), w.prior, dtype=torch.int32)
    lo, hi = w.ragged
    if gen is None:
        gen = torch.Generator("cpu").manual_seed(w.seed)
    return torch.randint(lo, hi + 1, (w.batch,), generator=gen).to(torch.int32)


def make_inputs(w: Workload, variant: str = "graded", seed: int | None = None) -> dict:
    """Draw one call's inputs on the CPU.  See the module docstring for the recipe."""
    if variant not in ("graded", "stress"):
        raise ValueError(f"unknown variant {variant!r}")
    gen = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    B, L, Hq, Hkv, D = w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim
    dt = DTYPES[w.dtype]

    n = prior_lengths(w, gen)
    cap = (n + L).to(torch.int32)
    offset = torch.zeros(B, dtype=torch.int64)
    if B > 1:
        offset[1:] = torch.cumsum(cap.to(torch.int64), 0)[:-1]
    rows = int(cap.to(torch.int64).sum().item())

    q_gate = torch.randn((B, L, Hq, 2 * D), generator=gen)
    k_new = torch.randn((B, L, Hkv, D), generator=gen)
    v_new = torch.randn((B, L, Hkv, D), generator=gen)
    k_cache = torch.zeros((rows, Hkv, D), dtype=dt)
    v_cache = torch.zeros((rows, Hkv, D), dtype=dt)
    for cache in (k_cache, v_cache):
        for b in range(B):
            nb, o = int(n[b]), int(offset[b])
            if nb:
                cache[o:o + nb] = torch.randn((nb, Hkv, D), generator=gen).to(dt)
    w_q = 1.0 + 0.1 * torch.randn(D, generator=gen)
    w_k = 1.0 + 0.1 * torch.randn(D, generator=gen)
    if variant == "stress":
        levels = torch.tensor([0.05, 20.0])
        sq = levels[torch.randint(0, 2, (B, L, Hq, 1), generator=gen)]
        sk = levels[torch.randint(0, 2, (B, L, Hkv, 1), generator=gen)]
        q_gate[..., :D] *= sq
        k_new *= sk

    positions = (n.view(B, 1) + torch.arange(L, dtype=torch.int32).view(1, L)).to(torch.int32)
    return {
        "q_gate": q_gate.to(dt).contiguous(),
        "k_new": k_new.to(dt).contiguous(),
        "v_new": v_new.to(dt).contiguous(),
        "k_cache": k_cache,
        "v_cache": v_cache,
        "w_q": w_q.to(dt),
        "w_k": w_k.to(dt),
        "seq_lens": n.clone(),
        "positions": positions.contiguous(),
        "seq_offset": offset,
        "capacity": cap,
    }


def to_device(inputs: dict, device) -> dict:
    """Copy every tensor of an input dict to ``device``."""
    return {k: v.to(device) if isinstance(v, torch.Tensor) else v for k, v in inputs.items()}


HIDDEN_4B = 2560   # Atlas qwen3_5_4b_mlx_int8: hidden


def make_proj_inputs(w: Workload, hidden: int = HIDDEN_4B, seed: int | None = None) -> dict:
    """Seeded inputs of the projections around the core: the rows x
    [B*L, hidden] ~ N(0, 1), the fused q/k/v weight [2 Hq D + 2 Hkv D, hidden]
    and the o_proj weight [hidden, Hq D], both N(0, 1) / sqrt(in_features) so
    that outputs are O(1); drawn in fp32 (in that order) and cast to the
    storage dtype."""
    gen = torch.Generator("cpu").manual_seed((w.seed if seed is None else seed) + 1000)
    dt = DTYPES[w.dtype]
    M, D = w.batch * w.q_len, w.head_dim
    nqkv = 2 * w.num_q_heads * D + 2 * w.num_kv_heads * D
    x = torch.randn((M, hidden), generator=gen)
    w_qkv = torch.randn((nqkv, hidden), generator=gen) / hidden ** 0.5
    w_o = torch.randn((hidden, w.num_q_heads * D), generator=gen) / (w.num_q_heads * D) ** 0.5
    return {"x": x.to(dt).contiguous(), "w_qkv": w_qkv.to(dt).contiguous(), "w_o": w_o.to(dt).contiguous()}


def paged_layout(capacity: torch.Tensor, seq_offset: torch.Tensor, block_size: int, seed: int = 0,
                 spare_blocks: int = 3):
    """Placement of a contiguous cache's rows in blocks: sequence b's capacity
    rows are cut into blocks of `block_size` rows placed at physical blocks
    drawn by a seeded permutation (plus a few spare blocks that no sequence
    owns).  Returns (block_table [B, max_blocks] int32 with -1 past each
    sequence's blocks, src rows, dst rows, physical row count)."""
    cap = capacity.to(torch.int64)
    B = cap.numel()
    nblk = (cap + block_size - 1) // block_size
    nphys = int(nblk.sum()) + spare_blocks
    max_blocks = int(nblk.max()) + 1
    perm = torch.randperm(nphys, generator=torch.Generator("cpu").manual_seed(seed)).to(torch.int32)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    first = torch.cumsum(nblk, 0) - nblk
    for b in range(B):
        table[b, :int(nblk[b])] = perm[int(first[b]):int(first[b] + nblk[b])]
    seq = torch.repeat_interleave(torch.arange(B), cap)
    t = torch.arange(int(cap.sum())) - torch.repeat_interleave(torch.cumsum(cap, 0) - cap, cap)
    src = seq_offset.to(torch.int64)[seq] + t
    dst = table[seq, t // block_size].to(torch.int64) * block_size + t % block_size
    return table, src, dst, nphys * block_size


def to_paged(inputs: dict, block_size: int, seed: int = 0, spare_blocks: int = 3) -> dict:
    """The same cache in paged form (see paged_layout); data movement only.
    Returns a copy of `inputs` with k_cache, v_cache and block_table replaced
    or added.  Works on CPU or device tensors."""
    table, src, dst, rows = paged_layout(inputs["capacity"].cpu(), inputs["seq_offset"].cpu(), block_size, seed,
                                         spare_blocks)
    out = dict(inputs)
    for name in ("k_cache", "v_cache"):
        c = inputs[name]
        pc = torch.zeros((rows,) + tuple(c.shape[1:]), dtype=c.dtype, device=c.device)
        pc[dst.to(c.device)] = c[src.to(c.device)]
        out[name] = pc
    out["block_table"] = table.to(inputs["capacity"].device)
    return out


def paged_rows(cache: torch.Tensor, table: torch.Tensor, block_size: int, seq: int, count: int) -> torch.Tensor:
    """Rows 0 .. count-1 of sequence `seq` gathered from a paged cache."""
    t = torch.arange(count)
    blk = table[seq].to(torch.int64)[t // block_size].to(cache.device)
    return cache[blk * block_size + (t % block_size).to(cache.device)]


def make_turbo8_inputs(w: Workload, variant: str = "graded", seed: int | None = None) -> dict:
    """Inputs of a call on a Turbo8 cache: the bf16 inputs of make_inputs (their
    cache replaced) plus cached rows in Turbo8 storage drawn directly: codes
    [rows, Hkv, D] (uint8) as the E4M3 casts of 128 N(0, 1) clamped to +-448, and
    scales [rows, Hkv, D/16] (bf16) as exp(0.25 N(0, 1)) / 128, so that the
    stored rows are about N(0, 1); rows past n_b are zero.  Random draws and
    library casts only (torch's float8_e4m3fn and bfloat16 conversions)."""
    x = make_inputs(w, variant=variant, seed=seed)
    gen = torch.Generator("cpu").manual_seed((w.seed if seed is None else seed) + 2000)
    rows = x["k_cache"].shape[0]
    D, Hkv = w.head_dim, w.num_kv_heads
    n, off = x["seq_lens"], x["seq_offset"]
    out = {k: v for k, v in x.items() if k not in ("k_cache", "v_cache")}
    for t in ("k", "v"):
        codes = torch.zeros((rows, Hkv, D), dtype=torch.uint8)
        scales = torch.zeros((rows, Hkv, D // 16), dtype=torch.bfloat16)
        for b in range(w.batch):
            nb, o = int(n[b]), int(off[b])
            if nb:
                vals = (128.0 * torch.randn((nb, Hkv, D), generator=gen)).clamp(-448.0, 448.0)
                codes[o:o + nb] = vals.to(torch.float8_e4m3fn).view(torch.uint8)
                scales[o:o + nb] = (torch.exp(0.25 * torch.randn((nb, Hkv, D // 16), generator=gen)) / 128.0).to(
                    torch.bfloat16)
        out[f"{t}_codes"], out[f"{t}_scales"] = codes, scales
    return out


# ---------------------------------------------------------------- GatedDeltaNet decode
@dataclass(frozen=True)
class GdnWorkload:
    """One decode step of the GatedDeltaNet (linear-attention) layer for a batch
    of sequences.  Geometry of the 4B checkpoint (Atlas ``qwen3_5/mod.rs``,
    ``Qwen35ForwardConfig::qwen3_5_4b_mlx_int8``: num_k_heads_lin 16,
    num_v_heads_lin 32, k/v_head_dim_lin 128, conv_kernel_size 4, rms_eps 1e-6)."""
    name: str
    batch: int
    num_k_heads: int = 16
    num_v_heads: int = 32
    k_head_dim: int = 128
    v_head_dim: int = 128
    conv_kernel: int = 4
    seed: int = 0
    rms_eps: float = 1e-6
    description: str = ""

    @property
    def channels(self) -> int:        # QKV_TOTAL_LIN = 2 Hk Dk + Hv Dv
        return 2 * self.num_k_heads * self.k_head_dim + self.num_v_heads * self.v_head_dim

    def with_(self, **kw) -> "GdnWorkload":
        return replace(self, **kw)


GDN_WORKLOADS = {
    "gdn_decode_4b": GdnWorkload("gdn_decode_4b", batch=64, seed=41,
                                 description="4B GatedDeltaNet geometry, 64 sequences, one token each"),
    "gdn_decode_4b_b1": GdnWorkload("gdn_decode_4b_b1", batch=1, seed=42,
                                    description="4B GatedDeltaNet geometry, one sequence"),
    "gdn_small": GdnWorkload("gdn_small", batch=3, num_k_heads=2, num_v_heads=4, seed=43,
                             description="small parity case: 3 sequences, 2 key / 4 value heads"),
}


def make_gdn_inputs(w: GdnWorkload, seed: int | None = None, state_scale: float = 0.05) -> dict:
    """Seeded inputs of one GatedDeltaNet decode step (one ``torch.Generator``
    seeded with the workload's seed, drawn in this order, fp32 then cast):

    1. ``qkv`` ``randn(B, C)`` bf16 (the q/k/v projection output, C = QKV_TOTAL_LIN);
    2. ``z`` ``randn(B, Hv * Dv)`` bf16; ``a`` ``randn(B, Hv)`` bf16; ``b`` ``randn(B, Hv)`` bf16;
    3. ``conv_w`` ``randn(C, K) / sqrt(K)`` bf16 ([C, K, 1] in the pages, the last axis dropped);
    4. ``a_log`` ``log(uniform(1, 16))`` fp32 [Hv]; ``dt_bias`` ``1 + 0.1 randn(Hv)`` bf16;
       ``norm_w`` ``1 + 0.1 randn(Dv)`` bf16;
    5. ``conv_state`` ``randn(B, C, K)`` rounded to bf16 and held as fp32 (earlier inputs);
    6. ``state`` ``state_scale * randn(B, Hv, Dk, Dv)`` fp32.

    Shapes and dtypes follow the pages' layer structs (Atlas ``LinearAttentionLayer``:
    a_log FP32, dt_bias BF16, conv1d_weight BF16, norm_weight BF16;
    ``LinearAttentionState``: conv1d_state FP32 [C, K], gdn_state FP32 [Hv, Dk, Dv]
    per sequence)."""
    gen = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    B, C, K = w.batch, w.channels, w.conv_kernel
    Hv, Dk, Dv = w.num_v_heads, w.k_head_dim, w.v_head_dim
    bf = torch.bfloat16
    x = {
        "qkv": torch.randn((B, C), generator=gen).to(bf),
        "z": torch.randn((B, Hv * Dv), generator=gen).to(bf),
        "a": torch.randn((B, Hv), generator=gen).to(bf),
        "b": torch.randn((B, Hv), generator=gen).to(bf),
        "conv_w": (torch.randn((C, K), generator=gen) / K ** 0.5).to(bf),
        "a_log": torch.log(1.0 + 15.0 * torch.rand((Hv,), generator=gen)),
        "dt_bias": (1.0 + 0.1 * torch.randn((Hv,), generator=gen)).to(bf),
        "norm_w": (1.0 + 0.1 * torch.randn((Dv,), generator=gen)).to(bf),
        "conv_state": torch.randn((B, C, K), generator=gen).to(bf).float(),
        "state": state_scale * torch.randn((B, Hv, Dk, Dv), generator=gen),
    }
    return x


def make_turbo4v_inputs(w: Workload, variant: str = "graded", seed: int | None = None) -> dict:
    """Inputs of a call on a bf16-K / Turbo4-V cache: the bf16 inputs of
    make_inputs (their K cache kept, their V cache replaced) plus V rows in
    Turbo4 storage drawn directly: codes [rows, Hkv, D/2] as random bytes (two
    uniform 4-bit indices each) and scales [rows, Hkv, D/16] as the E4M3 casts
    of exp(0.25 N(0, 1)) (torch's float8_e4m3fn); rows past n_b are zero."""
    x = make_inputs(w, variant=variant, seed=seed)
    gen = torch.Generator("cpu").manual_seed((w.seed if seed is None else seed) + 3000)
    rows = x["v_cache"].shape[0]
    D, Hkv = w.head_dim, w.num_kv_heads
    n, off = x["seq_lens"], x["seq_offset"]
    out = {k: v for k, v in x.items() if k != "v_cache"}
    codes = torch.zeros((rows, Hkv, D // 2), dtype=torch.uint8)
    scales = torch.zeros((rows, Hkv, D // 16), dtype=torch.uint8)
    for b in range(w.batch):
        nb, o = int(n[b]), int(off[b])
        if nb:
            codes[o:o + nb] = torch.randint(0, 256, (nb, Hkv, D // 2), generator=gen, dtype=torch.uint8)
            s = torch.exp(0.25 * torch.randn((nb, Hkv, D // 16), generator=gen))
            scales[o:o + nb] = s.to(torch.float8_e4m3fn).view(torch.uint8)
    out["v_codes"], out["v_scales"] = codes, scales
    return out
