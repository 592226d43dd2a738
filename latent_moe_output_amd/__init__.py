"""latent_moe_output_amd -- the latent-MoE output tail on MI355X (gfx950).

The compute lives in ``liblatenttail.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/latent_tail.h``).  ``binding`` is the thin ctypes
layer over it; ``synth`` holds the seeded workload generator.  Importing the
package does not load the shared library; the first call through
``binding`` does, and fails loudly if it has not been built.
"""

__all__ = ["binding", "synth"]
