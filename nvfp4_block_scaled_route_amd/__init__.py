"""MI355X-native NVFP4 routed-MoE layer: HIP kernels for gfx950 behind the C-ABI
of include/moe_nvfp4.h (libmoe_nvfp4.so, built in this directory by build.py),
a ctypes binding (native.py), a layer helper that owns the device buffers
(layer.py) and the seeded synthetic workloads (workloads.py).

Importing the package loads nothing; the library loads on first use and its
absence is an error.
"""
