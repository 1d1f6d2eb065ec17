"""MI355X-native chunkwise forward of GTR's key-only gated linear attention.

The forward runs in hand-written HIP kernels for gfx950 behind a C-ABI shared
library (include/gla.h); `gla` is the thin ctypes binding over it and
`workloads` draws the seeded synthetic inputs. Importing the package does not
load the library; the first call does, and fails loudly if it is not built.
"""
