"""Device-side set-up for one layer call: inputs on the GPU, workspace, output,
``qsa_cfg`` and ``qsa_kv_cache``.  Plumbing only; the call itself is one
``qsa_gated_attention`` through the C ABI."""
from __future__ import annotations

import torch

from . import binding
from .workloads import DTYPES, Workload


class Session:
    def __init__(self, w: Workload, inputs: dict, device="cuda", force_splits: int = 0,
                 max_seq_len: int | None = None, stream=None, softmax_scale: float = 0.0,
                 block_size: int = 0):
        """block_size > 0: the cache is given in paged form (inputs hold block_table)."""
        self.w = w
        self.softmax_scale = softmax_scale
        self.block_size = block_size
        self.dev = {k: v.to(device) if isinstance(v, torch.Tensor) else v for k, v in inputs.items()}
        d = self.dev
        if max_seq_len is None:
            max_seq_len = int((inputs["seq_lens"].max() + w.q_len).item())
        self.dtype = DTYPES[w.dtype]
        self.max_seq_len = max_seq_len
        self.force_splits = force_splits
        self.stream = stream
        probe = self._cfg(None)
        nbytes = binding.workspace_size(probe)
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.out = torch.empty((w.batch, w.q_len, w.num_q_heads, w.head_dim), dtype=self.dtype,
                               device=device)
        self.cfg = self._cfg(self.workspace)
        if "k_codes" in d:                                 # Turbo8 cache
            self.kv = binding.make_kv(d["k_codes"], d["v_codes"], d["seq_offset"], d["capacity"],
                                      k_scales=d["k_scales"], v_scales=d["v_scales"])
        elif "v_codes" in d:                               # bf16 K + Turbo4 V cache
            self.kv = binding.make_kv(d["k_cache"], d["v_codes"], d["seq_offset"], d["capacity"],
                                      v_scales=d["v_scales"])
        elif block_size:
            self.kv = binding.make_kv(d["k_cache"], d["v_cache"], None, d["capacity"], d["block_table"], block_size)
        else:
            self.kv = binding.make_kv(d["k_cache"], d["v_cache"], d["seq_offset"], d["capacity"])

    def _cfg(self, workspace):
        w, d = self.w, self.dev
        return binding.make_cfg(
            batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
            head_dim=w.head_dim, rotary_dim=w.rotary_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
            dtype=self.dtype, max_seq_len=self.max_seq_len, q_norm_w=d["w_q"], k_norm_w=d["w_k"],
            workspace=workspace, force_splits=self.force_splits, stream=self.stream,
            softmax_scale=self.softmax_scale)

    def plan(self) -> str:
        return binding.describe_plan(self.cfg)

    def run(self, fused: bool = True):
        """One call.  The output buffer is filled with NaN first, so an output
        element that the call fails to write cannot pass for a result."""
        d = self.dev
        if self.stream is None:
            self.out.fill_(float("nan"))
        else:
            with torch.cuda.stream(self.stream):
                self.out.fill_(float("nan"))
        binding.gated_attention(self.cfg, self.kv, d["q_gate"], d["k_new"] if fused else None,
                                d["v_new"] if fused else None, d["seq_lens"], d["positions"], self.out)
        return self.out

    def append(self):
        d = self.dev
        binding.append_kv(self.cfg, self.kv, d["k_new"], d["v_new"], d["seq_lens"], d["positions"])

    def device_error(self) -> int:
        return int(self.workspace[:4].view(torch.int32).item())
