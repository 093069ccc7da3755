"""MI355X-native NVFP4 block-scaled linear and MoE grouped GEMM.

The compute path is the C-ABI library ``libnvfp4.so`` (hand-written HIP for
gfx950, declared in ``include/nvfp4.h``); ``fp4_block_scaled_route_amd.ops``
is a thin ctypes binding with the same entry-point names.  ``synth`` draws
seeded synthetic inputs.  Importing this package does not load the library;
the binding loads it on first use and raises if it is missing.
"""
