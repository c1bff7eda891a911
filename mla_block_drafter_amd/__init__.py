"""DSpark draft pass on AMD Instinct MI355X (gfx950): HIP kernels behind the C
ABI in include/dspark.h, with a thin ctypes binding (dspark.py).

Importing the package does not load the library; `dspark.lib()` does, and it
raises if libdspark.so has not been built (there is no CPU fallback).
"""
