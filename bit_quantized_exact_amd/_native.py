"""ctypes loader of libattn.so (the C ABI declared in include/attn.h).

torch is imported first on purpose: its HIP runtime then satisfies the
library's libamdhip64 dependency, so both share one runtime, one device
context and the same streams.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must load before libattn.so, see above)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_ELAUNCH, ATTN_ERANGE, ATTN_ESCRATCH = 0, -1, -2, -3, -4, -5
ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20
ATTN_MAX_HEADS = 256
ATTN_MAX_SEQ = 1 << 22

EXPORTED = (
    "attn_quant_blocks", "attn_quantize_workspace_bytes", "attn_quantize_qk", "attn_quantize_k",
    "attn_quantize_k_noalloc",
    "attn_fwd_int8", "attn_fwd_int8_fused_q", "attn_fwd_fp16", "attn_debug_qk_int32",
    "attn_debug_qk_int32_fused_q",
    "attn_status_string", "attn_quantize_qk_fp8", "attn_fwd_fp8", "attn_v_fp8_stride",
    "attn_quantize_v_fp8", "attn_fwd_int8_pv8", "attn_decode_workspace_bytes", "attn_decode_int8",
    "attn_decode_fp16", "attn_block_mask_tiles", "attn_block_mask_apb", "attn_block_mask_csr",
    "attn_fwd_fp16_masked", "attn_fwd_int8_masked",
)


class AttnShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seq", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


class AttnKvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seq_q", ctypes.c_int32),
                ("seq_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


ATTN_DECODE_MAX_SEQ_Q = 32

_lib = None


def lib():
    """Load libattn.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m bit_quantized_exact_amd.build`; "
            "this package has no non-HIP fallback")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    SP = ctypes.POINTER(AttnShape)
    L.attn_quant_blocks.argtypes = [ctypes.POINTER(I32), ctypes.POINTER(I32)]
    L.attn_quant_blocks.restype = ctypes.c_int
    L.attn_quantize_workspace_bytes.argtypes = [SP]
    L.attn_quantize_workspace_bytes.restype = ctypes.c_size_t
    L.attn_quantize_qk.argtypes = [SP, P, P, P, P, P, P, P, P, P]
    L.attn_quantize_qk.restype = ctypes.c_int
    L.attn_fwd_int8.argtypes = [SP, P, P, P, P, P, P, P, P, ctypes.c_int, F32, P]
    L.attn_fwd_int8.restype = ctypes.c_int
    L.attn_quantize_k.argtypes = [SP, P, P, P, P, P, P]
    L.attn_quantize_k.restype = ctypes.c_int
    L.attn_quantize_k_noalloc.argtypes = [SP, P, P, P, P, P]
    L.attn_quantize_k_noalloc.restype = ctypes.c_int
    L.attn_fwd_int8_fused_q.argtypes = [SP, P, P, P, P, P, P, P, P, ctypes.c_int, F32, P]
    L.attn_fwd_int8_fused_q.restype = ctypes.c_int
    L.attn_fwd_fp16.argtypes = [SP, P, P, P, P, P, P, ctypes.c_int, F32, P]
    L.attn_fwd_fp16.restype = ctypes.c_int
    L.attn_debug_qk_int32.argtypes = [SP, P, P, P, ctypes.c_int, I32, I32, P, P]
    L.attn_debug_qk_int32.restype = ctypes.c_int
    L.attn_debug_qk_int32_fused_q.argtypes = [SP, P, P, P, ctypes.c_int, I32, I32, P, P, P]
    L.attn_debug_qk_int32_fused_q.restype = ctypes.c_int
    L.attn_quantize_qk_fp8.argtypes = [SP, P, P, P, P, P, P, P, P, P]
    L.attn_quantize_qk_fp8.restype = ctypes.c_int
    L.attn_fwd_fp8.argtypes = [SP, P, P, P, P, P, P, P, P, ctypes.c_int, F32, P]
    L.attn_fwd_fp8.restype = ctypes.c_int
    L.attn_v_fp8_stride.argtypes = [SP]
    L.attn_v_fp8_stride.restype = ctypes.c_int64
    L.attn_quantize_v_fp8.argtypes = [SP, P, P, P, P, P]
    L.attn_quantize_v_fp8.restype = ctypes.c_int
    L.attn_fwd_int8_pv8.argtypes = [SP, P, P, P, P, P, P, P, P, P, ctypes.c_int, F32, P]
    L.attn_fwd_int8_pv8.restype = ctypes.c_int
    KP = ctypes.POINTER(AttnKvShape)
    L.attn_decode_workspace_bytes.argtypes = [KP, P]
    L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.attn_decode_int8.argtypes = [KP, P, P, P, P, P, P, P, P, ctypes.c_int, F32, P, P]
    L.attn_decode_int8.restype = ctypes.c_int
    L.attn_decode_fp16.argtypes = [KP, P, P, P, P, P, P, ctypes.c_int, F32, P, P]
    L.attn_decode_fp16.restype = ctypes.c_int
    L.attn_block_mask_tiles.argtypes = [I32, P, P]
    L.attn_block_mask_tiles.restype = ctypes.c_int
    L.attn_block_mask_apb.argtypes = [I32, I32, I32, P]
    L.attn_block_mask_apb.restype = ctypes.c_int
    L.attn_block_mask_csr.argtypes = [I32, P, P, P, P]
    L.attn_block_mask_csr.restype = ctypes.c_int
    L.attn_fwd_fp16_masked.argtypes = [SP, P, P, P, P, P, P, P, P, I32, F32, P]
    L.attn_fwd_fp16_masked.restype = ctypes.c_int
    L.attn_fwd_int8_masked.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, I32, F32, P]
    L.attn_fwd_int8_masked.restype = ctypes.c_int
    L.attn_status_string.argtypes = [ctypes.c_int]
    L.attn_status_string.restype = ctypes.c_char_p
    _lib = L
    return L
