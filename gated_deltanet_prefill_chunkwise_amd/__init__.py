"""Chunkwise Gated DeltaNet (GDN) core prefill for MI355X (gfx950).

Dense operator and the SparseGDN approximate operator, computed by
hand-written HIP kernels behind the C ABI of ``libsgdn.so``
(``include/sgdn.h``).  ``ops`` holds the thin Python binding; ``synth`` the
seeded synthetic inputs.  Importing the package does not load the library;
the first call into ``ops`` does, and raises if it has not been built.
"""
