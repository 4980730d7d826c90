"""ctypes loader of libattn_probe.so (mfma_probe.h): the dense MFMA loop and the
streaming read the benchmark reports beside the published peaks.  Not part of the
attention path or of libattn.so's C ABI."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (its HIP runtime must load first, as for libattn.so)

_HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(_HERE, "libattn_probe.so")
EXPORTED = ("attn_probe_mfma", "attn_probe_hbm_read", "attn_probe_compute_units")

_lib = None


def lib():
    """Load libattn_probe.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_exact_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    L.attn_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.POINTER(ctypes.c_double), P]
    L.attn_probe_mfma.restype = ctypes.c_int
    L.attn_probe_hbm_read.argtypes = [P, ctypes.c_ulonglong, ctypes.c_int, P, P]
    L.attn_probe_hbm_read.restype = ctypes.c_int
    L.attn_probe_compute_units.argtypes = [ctypes.POINTER(ctypes.c_int)]
    L.attn_probe_compute_units.restype = ctypes.c_int
    _lib = L
    return L
