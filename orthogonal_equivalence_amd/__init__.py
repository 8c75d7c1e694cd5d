"""POET-X reparameterized linear layer on AMD Instinct MI355X (gfx950).

The layer z = P^T (W0^T (R^T x)) with permuted block-diagonal Cayley-Neumann
rotations R and P runs in hand-written HIP kernels behind the C ABI declared
in ``include/poetx.h`` (library ``libpoetx.so``). ``poetx`` is the thin ctypes
binding over that ABI; ``synth`` draws seeded synthetic inputs.

Importing this package does not load the HIP library; ``import
orthogonal_equivalence_amd.poetx`` does, and fails loudly if it is not built.
"""

__all__ = ["poetx", "synth"]
