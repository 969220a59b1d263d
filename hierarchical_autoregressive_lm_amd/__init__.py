"""PHOTON recursive-generation decode on AMD Instinct MI355X (gfx950).

The compute path is the C ABI in include/photon.h, implemented by the HIP
kernels under csrc/ and built into libphoton.so; ``photon`` is its ctypes
binding (``from hierarchical_autoregressive_lm_amd.photon import Photon``).
"""
