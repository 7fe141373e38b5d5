"""CPU fp64 oracle for the quantized MoE decode step (test infrastructure only).

This package is the plain, slow, obviously correct definition of what the GPU
path computes. It exists to check that path and nothing else: only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (the HIP library and its Python binding) never
imports, calls or falls back to anything here, and nothing here imports the
product path.

Modules
-------
``oracle.gen``
    The oracle's own implementation of the seeded synthetic-input generator
    (splitmix64 counter hashing -> codes, bf16 scales/biases, bf16 vectors, x
    rows).  The GPU library implements the same published generator
    separately; the two share no code.
``oracle.moe``
    The method: group-affine dequantisation, RMSNorm, router logits,
    renormalised softmax top-k, SwiGLU experts, sigmoid-gated shared expert,
    weighted combine + residual, and a layer stack that hands bf16 h between
    layers.
``oracle.dense``
    Dense group-affine matrix-vector products of the non-expert projections
    (fused Q/K/V reading one input, attention output, lm_head).
``oracle.attention``
    Grouped-query decode attention of verify rows over a bf16 K/V cache.
``oracle.gdn``
    One decode step of the Gated DeltaNet recurrence (gated delta rule).

Every floating-point step is fp64; bf16 appears only where the workload fixes
it (stored weights' scales/biases, bf16 vectors, the bf16 hidden state handed
between layers).
"""

from . import attention, dense, gdn, gen, moe  # noqa: F401
from .gen import (  # noqa: F401
    MoEShape,
    GeneratedLayer,
    ExplicitLayer,
    bf16_round,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    gen_x,
    mix64,
)
from .moe import (  # noqa: F401
    dequant,
    rmsnorm,
    route,
    expert_ffn,
    shared_gate,
    layer_forward,
    stack_forward,
)
