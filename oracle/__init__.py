"""CPU oracle for TileShare's shared decoder layer and the TileShare-k stack.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only the tests, the smoke check and the bench's CPU-baseline leg
do.  It shares no code with the HIP library (no kernels, headers, tables or
helpers); the two sides meet only through the seeded inputs of ``synth``.

Sources.  "The pages" below means the TileShare paper page ("TileShare:
Training-Free Acceleration of Overlapping Tiled ViT Decoding") and its
summaries.  The method is given there only as a definition: the abstract,
the Figure 2 caption (inside one shared layer), the Table 1 and Table S7
captions (which operations are shared from layer k on) and Table S1 (each
operation of a block under TileShare).  The oracle writes that definition out
directly in numpy, in float64, with plain loops over tiles and heads and no
blocking or fusion.  Where the pages leave a step open the oracle takes one
reading, named in the docstring of the module or function that takes it.

Modules
-------
plan   tiling, coverage map, blend weights, RoPE tables
model  norms, attention, the per-tile block, the shared layer, the stack
fp8    OCP e4m3 encoding and the per-tensor fake-quantised GEMM
brute  pure-Python per-token loops for tiny grids (a second, independent
       formulation used to pin ``model``)

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against closed forms, brute force, invariants fixed by the pages, or an
independent library routine.  No function is "parity unpinned".
"""
