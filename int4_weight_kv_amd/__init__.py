"""futx: INT4 decode block for AMD Instinct MI355X (gfx950).

Submodules:
  workload  seeded synthetic inputs (no method arithmetic)
  futx      ctypes binding of libfutx.so (the C-ABI in include/futx.h);
            importing it raises if the HIP library is not built.
  _build    compiles libfutx.so with hipcc for gfx950.
"""
