"""MI355X-native KDA (fine-grained gated delta rule) layer: chunkwise prefill and
single-token decode as hand-written HIP kernels for gfx950 behind a C ABI.

The Python side only marshals arguments: ``kda.kda_chunk_fwd`` and
``kda.kda_recurrent_step`` call the shared library ``libkda.so`` through ctypes.
Importing this package does not load the library; the first call does, and it
raises if the library is missing.
"""
__all__ = ["kda", "inputs"]
