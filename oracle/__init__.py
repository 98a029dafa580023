"""CPU oracle for the MXFP4 MoE layer: plain, slow, fp64 definitions.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The GPU library never imports it and it never imports the GPU
library; the two share no code.  The only module both sides use is the seeded
input generator ``mxfp4_moe_decode_amd.synth``, which holds none of the
method's arithmetic.

Every function states the passage it follows.  The layer itself is defined by
the pages as: a high-precision router choosing 4 of 128 routed experts per
token plus an always-on shared expert ("MiniMax-M3.1 on AMD Instinct GPUs:
Day-0 support and optimization", section "MiniMax-M3.1 at a glance"); routed
experts with OCP MXFP4 weights (static) and OCP MXFP4 activations (dynamic)
(model card "amd/MiniMax-M3.1-Flash-Quark-MXFP4", section "Model Overview");
the shared expert in MXFP8 (article above, sections "MiniMax-M3.1 at a glance"
and "Serving with vLLM / What we Optimized").  Element and scale formats follow
the OCP Microscaling Formats (MX) v1.0 specification.

Parity status: every function is pinned by tests under ``tests/`` (closed
forms, library dtype conversions, brute force, invariants); none is unpinned.
"""

from . import mx, moe  # noqa: F401
