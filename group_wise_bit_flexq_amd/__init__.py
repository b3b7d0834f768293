"""flexq: group-wise 4-bit weight + KV-cache OPT decoder path for MI355X (gfx950).

The computation lives in libflexq.so (HIP kernels behind the C ABI of
include/flexq.h); `flexq` is its ctypes binding, `synth` the seeded input
generators and `workloads` the model/batch shapes.
"""
