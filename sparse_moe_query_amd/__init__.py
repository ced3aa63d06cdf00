"""MI355X-native forward (prefill) pass of the Grouped Query Experts (GQE) attention layer.

The compute lives in ``libgqe.so`` (hand-written HIP for gfx950 behind a C ABI declared in
``include/gqe.h``); :mod:`sparse_moe_query_amd.gqe` is the thin ctypes binding and
:mod:`sparse_moe_query_amd.inputs` the seeded synthetic input generator.
"""
