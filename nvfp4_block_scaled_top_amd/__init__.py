"""NVFP4 routed-expert ("MegaMoE") layer for MI355X (gfx950).

The compute path is libmegamoe.so (hand-written HIP kernels behind a C ABI, declared in
include/megamoe.h).  ``megamoe`` is its ctypes binding, ``layer`` owns the device buffers of one
layer forward, and ``synth`` draws seeded synthetic inputs.  Importing the package does not load
the library; the first call into ``megamoe`` does, and fails loudly if it has not been built.
"""
__all__ = ["megamoe", "layer", "synth", "build_lib"]
