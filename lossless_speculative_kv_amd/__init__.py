"""VeriCache draft/verify hot path for AMD MI355X (gfx950).

The compute lives in libvc.so (include/vc.h). ``_lib`` is its ctypes
binding (importing it loads the library and raises ImportError when it has
not been built); ``engine`` drives rounds with device buffers from PyTorch.
Build with ``python -m lossless_speculative_kv_amd.build``.
"""
