"""MI355X-native DiLoCo outer-step merge.

The merge runs in hand-written HIP kernels for gfx950 behind a C ABI
(``libdlmerge.so``, declared in ``include/dlmerge.h``); ``dlmerge`` is the thin
ctypes binding over it.  ``synth`` holds the seeded synthetic inputs (layouts,
globals, worker checkpoints, token counts, arrival orders).

Importing the package loads nothing; ``checkpoint_averaging_amd.dlmerge``
loads the library and raises if it has not been built.
"""
