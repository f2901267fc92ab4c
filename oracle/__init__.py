"""Plain, slow CPU oracle for dictionary-coded ternary MoE weights.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the graft entry's smoke check
and the benchmark's CPU-baseline leg use it.  It shares no code, tables or
constants with the HIP library under sub_bit_moe_amd/.

Sources (cited by page title and section):
  [QMoE]  "QMoE: Practical Sub-1-Bit Compression of Trillion-Parameter Models"
          (paper-graph-ui summary), section "The Fixed-to-Variable Dictionary
          Code" (Algorithm 1, Figure 4, Eq. 2) and "The GPU Decoding Kernel"
          (row offsets, ternary grid, trie encoder).
  [M8.5]  "M8.5 - Extreme Weight Compression and Representations",
          section 0x08A (QMoE reference decoder semantics).

Arithmetic is fp64 throughout; fp16 inputs convert exactly.

Modules:
  dictionary -- dictionary generation and the Figure-4 entry packing
  codec      -- trie encoder, reference decoder, row/block offset tables
  matvec     -- fp64 matrix-vector products (the symmetric grid -s_r/0/+s_r and the
                page's per-row grid w_min/0/w_max), the MoE layer, stack glue

Parity-pinning status of every function is listed in its docstring.
``matvec.rms_glue`` (harness glue between stacked layers, not part of the
method) is pinned by its defining properties: unit RMS, a positive multiple of
the input, zero rows kept zero.
"""
