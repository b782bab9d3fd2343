"""FlashAttention forward and split-KV decode for the AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libfa_mi355x.so``, declared in ``include/fa.h``); this package only builds it,
loads it and marshals arguments to it.  ``workloads`` draws seeded inputs.
"""
