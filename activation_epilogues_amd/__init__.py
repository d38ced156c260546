"""libconvt3d: ConvTranspose3d (NCDHW fp32) fused with ReLU+GroupNorm,
channel softmax+sigmoid, or scale+training BatchNorm3d+average pool, as
hand-written HIP kernels for AMD Instinct MI355X (gfx950).

``activation_epilogues_amd.convt3d`` is the ctypes binding of the C ABI in
``include/convt3d.h``; ``activation_epilogues_amd.workloads`` holds the seeded
synthetic workloads.
"""
__all__ = ["convt3d", "workloads"]
