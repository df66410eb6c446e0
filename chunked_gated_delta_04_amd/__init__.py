"""Chunked gated delta rule on MI355X (gfx950): forward, deterministic backward
and the recurrent decode step, as hand-written HIP kernels behind a C ABI
(include/gdn.h, libgdn.so). ``gdn`` is the Python binding; importing it needs
the built library (``python -m chunked_gated_delta_04_amd.build``).
"""
