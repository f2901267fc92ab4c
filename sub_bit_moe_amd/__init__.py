"""sub_bit_moe_amd: fused decode + matvec of dictionary-coded ternary MoE
expert weights on gfx950 (MI355X).

The compute lives in the HIP library libsbm.so (include/sbm.h); this package
marshals arguments to it.  Import is lazy: `sub_bit_moe_amd.synth` (seeded
inputs) works without the library; everything in `api` needs it and raises if
it is missing.
"""
__all__ = ["api", "synth"]
