"""MI355X-native Mixture-of-Experts layer (route, permute, grouped SwiGLU FFN, combine, backward).

The compute lives in ``libmoe_mi355x.so`` (hand-written HIP kernels for gfx950 behind a C ABI,
declared in ``include/moe.h``).  ``binding`` marshals torch tensors into that ABI; ``workloads``
draws the seeded synthetic layer inputs.  Importing this package loads nothing; the library is
loaded on first use and a missing library is an error.
"""
