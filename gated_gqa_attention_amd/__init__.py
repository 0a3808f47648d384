"""gated_gqa_attention_amd -- the Qwen3.5 gated full-attention core on MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI (``libqsa.so``,
declared in ``include/qsa.h``).  This package holds the kernels' sources
(``csrc/``), the thin ctypes binding (``binding``), device-buffer plumbing
(``session``) and the seeded input generators (``workloads``).  Importing the
package does not load the library; the first call through ``binding`` does,
and raises if it has not been built.
"""
from . import binding, workloads  # noqa: F401

__all__ = ["binding", "workloads"]
