"""CSA / HCA hybrid-attention hot path for MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(csrc/, header include/csa_attn.h).  `long_context_attention_23_amd.api`
is the thin ctypes binding over it; `synth` draws seeded synthetic inputs.
"""
__all__ = ["api", "synth"]
