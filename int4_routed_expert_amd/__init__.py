"""int4 routed-expert MoE layer (GLM-5.2 style) for AMD Instinct MI355X.

The work happens in ``libmoe.so`` (hand-written HIP for gfx950, C ABI declared
in include/moe.h); ``moe`` is its ctypes binding.
"""
