"""MI355X (gfx950) sparse-attention step of Mistral Large 4: DSA indexer -> exact top-k ->
sparse MLA, as a C-ABI HIP library (libml4dsa.so) with a thin ctypes binding.

Submodules:
  ml4dsa  -- the binding (loads libml4dsa.so; raises ImportError when it is not built)
  synth   -- seeded synthetic inputs shaped like the pages' workloads
  runner  -- device buffers and the per-layer calls used by the benchmark and tests
  build   -- in-tree hipcc build of the library
Importing the package itself loads nothing.
"""
