"""MI355X-native 8-bit (SageAttention-form) attention forward.

Thin Python binding over libattn.so (include/attn.h): every function below
only checks and marshals arguments (device pointers, sizes, the current HIP
stream) and calls the C ABI of the same name; all arithmetic runs in the HIP
kernels.  torch provides device memory and streams.

    attn_quantize_qk -> quantize_qk     K smoothing + per-block INT8 Q/K
    attn_quantize_k  -> quantize_k      K smoothing + per-block INT8 K only
    attn_fwd_int8    -> fwd_int8        INT8 QK^T, FP16 PV, online softmax
    attn_fwd_int8_fused_q -> fwd_int8_fused_q   the same, quantising Q in the kernel
    attn_fwd_fp16    -> fwd_fp16        exact FP16 FlashAttention-style forward
    attn_debug_qk_int32 -> debug_qk_int32   the INT32 score tiles (test hook)
    sageattn(q, k, v, is_causal, scale)     one-call scaled_dot_product_attention
                                            replacement (quantize_k + fwd_int8_fused_q)
    attn_quantize_qk_fp8 -> quantize_qk_fp8 the FP8 (E4M3) alternative for Q/K
    attn_fwd_fp8     -> fwd_fp8         E4M3 QK^T, FP16 PV
    attn_quantize_v_fp8 -> quantize_v_fp8   per-channel E4M3 V (transposed)
    attn_fwd_int8_pv8 -> fwd_int8_pv8   INT8 QK^T with 8-bit P and V (ablation)
    attn_decode_int8 -> decode_int8     KV-cache decode, 8-bit (K from quantize_k on the cache)
    attn_decode_fp16 -> decode_fp16     KV-cache decode, exact FP16
    attn_block_mask_* -> block_mask_tiles / apb_block_mask / block_mask_csr   tile masks
    attn_fwd_fp16_masked / attn_fwd_int8_masked -> fwd_fp16_masked / fwd_int8_masked

Sources: SageAttention article ("又快又准，即插即用！清华8比特量化Attention…"),
技术方案 and its plug-and-play example; "注意力即一切：从 MHA 到 GQA" §2.2-§5.1.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _native
from ._native import AttnKvShape, AttnShape, lib

__all__ = [
    "AttnError", "quant_blocks", "quantize_workspace_bytes", "quantize_qk", "quantize_k",
    "fwd_int8", "fwd_int8_fused_q", "fwd_fp16", "debug_qk_int32", "sageattn", "status_string",
    "quantize_qk_fp8", "fwd_fp8", "v_fp8_stride", "quantize_v_fp8", "fwd_int8_pv8",
    "decode_workspace_bytes", "decode_int8", "decode_fp16", "block_mask_tiles", "apb_block_mask",
    "block_mask_csr", "fwd_fp16_masked", "fwd_int8_masked", "AttnShape", "AttnKvShape", "lib",
]


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != _native.ATTN_OK:
        raise AttnError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(q: torch.Tensor, k: torch.Tensor) -> AttnShape:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, heads, seq, head_dim]")
    B, Hq, S, D = q.shape
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return AttnShape(B, Hq, k.shape[1], S, D)


def _map_arg(kv_head_map):
    if kv_head_map is None:
        return None, None
    arr = (ctypes.c_int32 * len(kv_head_map))(*[int(x) for x in kv_head_map])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def quant_blocks():
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    lib().attn_quant_blocks(ctypes.byref(bq), ctypes.byref(bk))
    return bq.value, bk.value


def quantize_workspace_bytes(shape: AttnShape) -> int:
    return int(lib().attn_quantize_workspace_bytes(ctypes.byref(shape)))


def quantize_qk(q: torch.Tensor, k: torch.Tensor, *, out: Optional[dict] = None,
                workspace: Optional[torch.Tensor] = None, with_mean: bool = True, stream=None):
    """K smoothing + per-block INT8 quantisation.  Returns a dict with q_i8,
    q_scale, k_i8, k_scale, k_mean (None unless with_mean) and workspace."""
    _dev(q, torch.float16, "q")
    _dev(k, torch.float16, "k")
    sh = _shape(q, k)
    bq, bk = quant_blocks()
    B, Hq, Hkv, S, D = sh.batch, sh.heads_q, sh.heads_kv, sh.seq, sh.head_dim
    o = dict(out) if out is not None else {}
    dev = q.device
    if "q_i8" not in o:
        o["q_i8"] = torch.empty((B, Hq, S, D), dtype=torch.int8, device=dev)
        o["q_scale"] = torch.empty((B, Hq, -(-S // bq)), dtype=torch.float32, device=dev)
        o["k_i8"] = torch.empty((B, Hkv, S, D), dtype=torch.int8, device=dev)
        o["k_scale"] = torch.empty((B, Hkv, -(-S // bk)), dtype=torch.float32, device=dev)
    if with_mean and o.get("k_mean") is None:
        o["k_mean"] = torch.empty((B, Hkv, D), dtype=torch.float32, device=dev)
    if not with_mean:
        o["k_mean"] = None
    nbytes = quantize_workspace_bytes(sh)
    if nbytes == 0:
        raise AttnError(_native.ATTN_EINVAL, "attn_quantize_workspace_bytes")
    if workspace is None:
        workspace = o.get("workspace")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    o["workspace"] = workspace
    _check(lib().attn_quantize_qk(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(o["q_i8"]),
                                  _ptr(o["q_scale"]), _ptr(o["k_i8"]), _ptr(o["k_scale"]),
                                  _ptr(o["k_mean"]), _ptr(workspace), _stream(stream)),
           "attn_quantize_qk")
    return o


def quantize_k(k: torch.Tensor, *, out: Optional[dict] = None,
               workspace: Optional[torch.Tensor] = None, with_mean: bool = True, stream=None):
    """K smoothing + per-block INT8 quantisation of K only.  Returns a dict with
    k_i8, k_scale, k_mean (None unless with_mean) and workspace."""
    _dev(k, torch.float16, "k")
    if k.dim() != 4:
        raise ValueError("k must be [batch, heads, seq, head_dim]")
    B, Hkv, S, D = k.shape
    sh = AttnShape(B, Hkv, Hkv, S, D)
    _, bk = quant_blocks()
    o = dict(out) if out is not None else {}
    dev = k.device
    if "k_i8" not in o:
        o["k_i8"] = torch.empty((B, Hkv, S, D), dtype=torch.int8, device=dev)
        o["k_scale"] = torch.empty((B, Hkv, -(-S // bk)), dtype=torch.float32, device=dev)
    if with_mean and o.get("k_mean") is None:
        o["k_mean"] = torch.empty((B, Hkv, D), dtype=torch.float32, device=dev)
    if not with_mean:
        o["k_mean"] = None
    nbytes = quantize_workspace_bytes(sh)
    if nbytes == 0:
        raise AttnError(_native.ATTN_EINVAL, "attn_quantize_workspace_bytes")
    if workspace is None:
        workspace = o.get("workspace")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    o["workspace"] = workspace
    _check(lib().attn_quantize_k(ctypes.byref(sh), _ptr(k), _ptr(o["k_i8"]), _ptr(o["k_scale"]),
                                 _ptr(o["k_mean"]), _ptr(workspace), _stream(stream)),
           "attn_quantize_k")
    return o


def fwd_int8_fused_q(q: torch.Tensor, kz: dict, v: torch.Tensor, *, causal: bool = False,
                     kv_head_map=None, sm_scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     return_lse: bool = False, q_scale_out: Optional[torch.Tensor] = None,
                     stream=None):
    """8-bit attention forward reading fp16 Q and quantising it in the kernel;
    kz is the output of quantize_k (or quantize_qk)."""
    _dev(q, torch.float16, "q")
    k_i8 = _dev(kz["k_i8"], torch.int8, "k_i8")
    ks = _dev(kz["k_scale"], torch.float32, "k_scale")
    _dev(v, torch.float16, "v")
    sh = _shape(q, k_i8)
    if tuple(v.shape) != tuple(k_i8.shape):
        raise ValueError("v must have the shape of k")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if q_scale_out is not None:
        _dev(q_scale_out, torch.float32, "q_scale_out")
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_fwd_int8_fused_q(ctypes.byref(sh), _ptr(q), _ptr(k_i8), _ptr(ks), _ptr(v),
                                       _ptr(out), _ptr(lse), _ptr(q_scale_out), mp,
                                       int(bool(causal)), float(sm_scale or 0.0), _stream(stream)),
           "attn_fwd_int8_fused_q")
    return (out, lse) if (return_lse or lse is not None) else out


def fwd_int8(qz: dict, v: torch.Tensor, *, causal: bool = False, kv_head_map=None,
             sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None):
    """8-bit attention forward on the output of quantize_qk."""
    q_i8 = _dev(qz["q_i8"], torch.int8, "q_i8")
    k_i8 = _dev(qz["k_i8"], torch.int8, "k_i8")
    qs = _dev(qz["q_scale"], torch.float32, "q_scale")
    ks = _dev(qz["k_scale"], torch.float32, "k_scale")
    _dev(v, torch.float16, "v")
    sh = _shape(q_i8, k_i8)
    if tuple(v.shape) != tuple(k_i8.shape):
        raise ValueError("v must have the shape of k")
    if out is None:
        out = torch.empty(q_i8.shape, dtype=torch.float16, device=v.device)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q_i8.shape[:3], dtype=torch.float32, device=v.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_fwd_int8(ctypes.byref(sh), _ptr(q_i8), _ptr(qs), _ptr(k_i8), _ptr(ks),
                               _ptr(v), _ptr(out), _ptr(lse), mp, int(bool(causal)),
                               float(sm_scale or 0.0), _stream(stream)), "attn_fwd_int8")
    return (out, lse) if (return_lse or lse is not None) else out


def fwd_fp16(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
             kv_head_map=None, sm_scale: Optional[float] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             return_lse: bool = False, stream=None):
    """Exact FP16 attention forward (FlashAttention-style baseline)."""
    _dev(q, torch.float16, "q")
    _dev(k, torch.float16, "k")
    _dev(v, torch.float16, "v")
    sh = _shape(q, k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must have the shape of k")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_fwd_fp16(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                               mp, int(bool(causal)), float(sm_scale or 0.0), _stream(stream)),
           "attn_fwd_fp16")
    return (out, lse) if (return_lse or lse is not None) else out


def debug_qk_int32(q_i8: torch.Tensor, k_i8: torch.Tensor, *, causal: bool = False,
                   kv_head_map=None, tile_lo: int = 0, tile_hi: int = 0, fill: int = 0,
                   stream=None) -> torch.Tensor:
    """INT32 score rows of query tiles tile_lo..tile_hi: [B, Hq, ntiles*BQ, S];
    masked entries and rows beyond S keep `fill`."""
    _dev(q_i8, torch.int8, "q_i8")
    _dev(k_i8, torch.int8, "k_i8")
    sh = _shape(q_i8, k_i8)
    bq, _ = quant_blocks()
    rows = (tile_hi - tile_lo + 1) * bq
    s_out = torch.full((sh.batch, sh.heads_q, max(rows, 1), sh.seq), fill, dtype=torch.int32,
                       device=q_i8.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_debug_qk_int32(ctypes.byref(sh), _ptr(q_i8), _ptr(k_i8), mp,
                                     int(bool(causal)), int(tile_lo), int(tile_hi), _ptr(s_out),
                                     _stream(stream)), "attn_debug_qk_int32")
    return s_out


def sageattn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, is_causal: bool = False,
             scale: Optional[float] = None, kv_head_map=None) -> torch.Tensor:
    """Drop-in for torch's scaled_dot_product_attention on fp16 [B, H, S, D]
    tensors (the SageAttention article's plug-and-play use): K smoothing and
    INT8 quantisation of K, then the 8-bit forward that quantises Q itself."""
    kz = quantize_k(k.contiguous(), with_mean=False)
    return fwd_int8_fused_q(q.contiguous(), kz, v.contiguous(), causal=is_causal,
                            kv_head_map=kv_head_map, sm_scale=scale)


# --------------------------------------------------------------------------
# FP8 alternative and the 8-bit P.V ablation
# --------------------------------------------------------------------------
def _workspace(sh: AttnShape, workspace, dev):
    nbytes = quantize_workspace_bytes(sh)
    if nbytes == 0:
        raise AttnError(_native.ATTN_EINVAL, "attn_quantize_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return workspace


def quantize_qk_fp8(q: torch.Tensor, k: torch.Tensor, *, workspace: Optional[torch.Tensor] = None,
                    with_mean: bool = True, stream=None):
    """K smoothing + per-block E4M3 quantisation (the FP8 alternative).  Returns
    a dict with q_f8, q_scale, k_f8, k_scale (codes as uint8), k_mean, workspace."""
    _dev(q, torch.float16, "q")
    _dev(k, torch.float16, "k")
    sh = _shape(q, k)
    bq, bk = quant_blocks()
    B, Hq, Hkv, S, D = sh.batch, sh.heads_q, sh.heads_kv, sh.seq, sh.head_dim
    dev = q.device
    o = dict(q_f8=torch.empty((B, Hq, S, D), dtype=torch.uint8, device=dev),
             q_scale=torch.empty((B, Hq, -(-S // bq)), dtype=torch.float32, device=dev),
             k_f8=torch.empty((B, Hkv, S, D), dtype=torch.uint8, device=dev),
             k_scale=torch.empty((B, Hkv, -(-S // bk)), dtype=torch.float32, device=dev),
             k_mean=torch.empty((B, Hkv, D), dtype=torch.float32, device=dev) if with_mean else None)
    o["workspace"] = _workspace(sh, workspace, dev)
    _check(lib().attn_quantize_qk_fp8(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(o["q_f8"]),
                                      _ptr(o["q_scale"]), _ptr(o["k_f8"]), _ptr(o["k_scale"]),
                                      _ptr(o["k_mean"]), _ptr(o["workspace"]), _stream(stream)),
           "attn_quantize_qk_fp8")
    return o


def fwd_fp8(qz: dict, v: torch.Tensor, *, causal: bool = False, kv_head_map=None,
            sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None):
    """Attention forward on E4M3 Q/K (the output of quantize_qk_fp8), FP16 P.V."""
    q8 = _dev(qz["q_f8"], torch.uint8, "q_f8")
    k8 = _dev(qz["k_f8"], torch.uint8, "k_f8")
    qs = _dev(qz["q_scale"], torch.float32, "q_scale")
    ks = _dev(qz["k_scale"], torch.float32, "k_scale")
    _dev(v, torch.float16, "v")
    sh = _shape(q8, k8)
    if tuple(v.shape) != tuple(k8.shape):
        raise ValueError("v must have the shape of k")
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.float16, device=v.device)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=v.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_fwd_fp8(ctypes.byref(sh), _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(v),
                              _ptr(out), _ptr(lse), mp, int(bool(causal)), float(sm_scale or 0.0),
                              _stream(stream)), "attn_fwd_fp8")
    return (out, lse) if (return_lse or lse is not None) else out


def v_fp8_stride(shape: AttnShape) -> int:
    return int(lib().attn_v_fp8_stride(ctypes.byref(shape)))


def quantize_v_fp8(v: torch.Tensor, *, workspace: Optional[torch.Tensor] = None, stream=None):
    """Per-channel E4M3 V for the 8-bit P.V ablation.  Returns a dict with
    v_f8t (codes, [B, Hkv, D, stride], transposed) and v_scale [B, Hkv, D]."""
    _dev(v, torch.float16, "v")
    if v.dim() != 4:
        raise ValueError("v must be [batch, heads, seq, head_dim]")
    B, Hkv, S, D = v.shape
    sh = AttnShape(B, Hkv, Hkv, S, D)
    stride = v_fp8_stride(sh)
    if stride == 0:
        raise AttnError(_native.ATTN_EINVAL, "attn_v_fp8_stride")
    o = dict(v_f8t=torch.empty((B, Hkv, D, stride), dtype=torch.uint8, device=v.device),
             v_scale=torch.empty((B, Hkv, D), dtype=torch.float32, device=v.device))
    o["workspace"] = _workspace(sh, workspace, v.device)
    _check(lib().attn_quantize_v_fp8(ctypes.byref(sh), _ptr(v), _ptr(o["v_f8t"]), _ptr(o["v_scale"]),
                                     _ptr(o["workspace"]), _stream(stream)), "attn_quantize_v_fp8")
    return o


def fwd_int8_pv8(qz: dict, vz: dict, *, causal: bool = False, kv_head_map=None,
                 sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None):
    """INT8 Q/K (quantize_qk) with 8-bit P and V (quantize_v_fp8): the ablation."""
    q_i8 = _dev(qz["q_i8"], torch.int8, "q_i8")
    k_i8 = _dev(qz["k_i8"], torch.int8, "k_i8")
    qs = _dev(qz["q_scale"], torch.float32, "q_scale")
    ks = _dev(qz["k_scale"], torch.float32, "k_scale")
    vt = _dev(vz["v_f8t"], torch.uint8, "v_f8t")
    vs = _dev(vz["v_scale"], torch.float32, "v_scale")
    sh = _shape(q_i8, k_i8)
    stride = v_fp8_stride(sh)
    if tuple(vt.shape) != (sh.batch, sh.heads_kv, sh.head_dim, stride):
        raise ValueError(f"v_f8t shape {tuple(vt.shape)} does not match k")
    if tuple(vs.shape) != (sh.batch, sh.heads_kv, sh.head_dim):
        raise ValueError("v_scale must be [batch, heads_kv, head_dim]")
    if out is None:
        out = torch.empty(q_i8.shape, dtype=torch.float16, device=q_i8.device)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q_i8.shape[:3], dtype=torch.float32, device=q_i8.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_fwd_int8_pv8(ctypes.byref(sh), _ptr(q_i8), _ptr(qs), _ptr(k_i8), _ptr(ks),
                                   _ptr(vt), _ptr(vs), _ptr(out), _ptr(lse), mp, int(bool(causal)),
                                   float(sm_scale or 0.0), _stream(stream)), "attn_fwd_int8_pv8")
    return (out, lse) if (return_lse or lse is not None) else out


# --------------------------------------------------------------------------
# KV-cache (decode) attention
# --------------------------------------------------------------------------
def _kv_shape(q: torch.Tensor, k: torch.Tensor) -> AttnKvShape:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, heads, seq, head_dim]")
    B, Hq, Sq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return AttnKvShape(B, Hq, k.shape[1], Sq, k.shape[2], D)


def decode_workspace_bytes(shape: AttnKvShape, kv_head_map=None) -> int:
    _keep, mp = _map_arg(kv_head_map)
    return int(lib().attn_decode_workspace_bytes(ctypes.byref(shape), mp))


def _decode_ws(sh, kv_head_map, workspace, dev):
    nbytes = decode_workspace_bytes(sh, kv_head_map)
    if nbytes == 0:
        raise AttnError(_native.ATTN_EINVAL, "attn_decode_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return workspace


def decode_int8(q: torch.Tensor, kz: dict, v: torch.Tensor, *, causal: bool = True,
                kv_head_map=None, sm_scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                return_lse: bool = False, q_scale_out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None):
    """8-bit attention of q [B, Hq, Sq, D] (the last Sq positions) over a KV
    cache: kz = quantize_k(k_cache) (mean over the cached tokens), v the fp16
    V cache [B, Hkv, Sk, D]."""
    _dev(q, torch.float16, "q")
    k_i8 = _dev(kz["k_i8"], torch.int8, "k_i8")
    ks = _dev(kz["k_scale"], torch.float32, "k_scale")
    _dev(v, torch.float16, "v")
    sh = _kv_shape(q, k_i8)
    if tuple(v.shape) != tuple(k_i8.shape):
        raise ValueError("v must have the shape of the K cache")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if q_scale_out is not None:
        _dev(q_scale_out, torch.float32, "q_scale_out")
    workspace = _decode_ws(sh, kv_head_map, workspace, q.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_decode_int8(ctypes.byref(sh), _ptr(q), _ptr(k_i8), _ptr(ks), _ptr(v), _ptr(out),
                                  _ptr(lse), _ptr(q_scale_out), mp, int(bool(causal)),
                                  float(sm_scale or 0.0), _ptr(workspace), _stream(stream)),
           "attn_decode_int8")
    return (out, lse) if (return_lse or lse is not None) else out


def decode_fp16(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = True,
                kv_head_map=None, sm_scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                return_lse: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Exact FP16 attention of q [B, Hq, Sq, D] over a K/V cache [B, Hkv, Sk, D]."""
    _dev(q, torch.float16, "q")
    _dev(k, torch.float16, "k")
    _dev(v, torch.float16, "v")
    sh = _kv_shape(q, k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must have the shape of the K cache")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    workspace = _decode_ws(sh, kv_head_map, workspace, q.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_decode_fp16(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), mp,
                                  int(bool(causal)), float(sm_scale or 0.0), _ptr(workspace),
                                  _stream(stream)), "attn_decode_fp16")
    return (out, lse) if (return_lse or lse is not None) else out


# --------------------------------------------------------------------------
# tile-level attention masks (APB-style anchor / passing / local)
# --------------------------------------------------------------------------
def block_mask_tiles(seq: int):
    nq, nk = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().attn_block_mask_tiles(int(seq), ctypes.byref(nq), ctypes.byref(nk)), "attn_block_mask_tiles")
    return nq.value, nk.value


def apb_block_mask(seq: int, anchor: int, passing: int):
    """Host tile mask (numpy uint8 [q_tiles, k_tiles]) of the APB layout."""
    import numpy as np
    nq, nk = block_mask_tiles(seq)
    m = np.zeros((nq, nk), dtype=np.uint8)
    _check(lib().attn_block_mask_apb(int(seq), int(anchor), int(passing), m.ctypes.data_as(ctypes.c_void_p)),
           "attn_block_mask_apb")
    return m


def block_mask_csr(seq: int, mask, device="cuda"):
    """The tile list of a dense host tile mask, copied to the device:
    dict(row_ptr, cols, nnz)."""
    import numpy as np
    nq, nk = block_mask_tiles(seq)
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    if m.shape != (nq, nk):
        raise ValueError(f"mask must be [{nq}, {nk}] for seq {seq}")
    row_ptr = np.zeros(nq + 1, dtype=np.int32)
    cols = np.zeros(max(1, nq * nk), dtype=np.int32)
    nnz = ctypes.c_int32()
    _check(lib().attn_block_mask_csr(int(seq), m.ctypes.data_as(ctypes.c_void_p),
                                     row_ptr.ctypes.data_as(ctypes.c_void_p),
                                     cols.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nnz)),
           "attn_block_mask_csr")
    return dict(row_ptr=torch.from_numpy(row_ptr).to(device),
                cols=torch.from_numpy(cols[:max(1, nnz.value)].copy()).to(device), nnz=nnz.value, seq=int(seq))


def _csr_args(csr, seq):
    if csr.get("seq") != seq:
        raise ValueError("the mask list was built for another sequence length")
    rp = _dev(csr["row_ptr"], torch.int32, "row_ptr")
    cols = _dev(csr["cols"], torch.int32, "cols")
    return rp, cols, int(csr["nnz"])


def fwd_fp16_masked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, csr: dict, *, kv_head_map=None,
                    sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None):
    """Exact FP16 forward under a tile mask (csr from block_mask_csr)."""
    _dev(q, torch.float16, "q")
    _dev(k, torch.float16, "k")
    _dev(v, torch.float16, "v")
    sh = _shape(q, k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must have the shape of k")
    rp, cols, nnz = _csr_args(csr, sh.seq)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_fwd_fp16_masked(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), mp,
                                      _ptr(rp), _ptr(cols), nnz, float(sm_scale or 0.0), _stream(stream)),
           "attn_fwd_fp16_masked")
    return (out, lse) if (return_lse or lse is not None) else out


def fwd_int8_masked(qz: dict, v: torch.Tensor, csr: dict, *, kv_head_map=None,
                    sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None):
    """8-bit forward (quantize_qk output) under a tile mask."""
    q_i8 = _dev(qz["q_i8"], torch.int8, "q_i8")
    k_i8 = _dev(qz["k_i8"], torch.int8, "k_i8")
    qs = _dev(qz["q_scale"], torch.float32, "q_scale")
    ks = _dev(qz["k_scale"], torch.float32, "k_scale")
    _dev(v, torch.float16, "v")
    sh = _shape(q_i8, k_i8)
    if tuple(v.shape) != tuple(k_i8.shape):
        raise ValueError("v must have the shape of k")
    rp, cols, nnz = _csr_args(csr, sh.seq)
    if out is None:
        out = torch.empty(q_i8.shape, dtype=torch.float16, device=v.device)
    _dev(out, torch.float16, "out")
    if return_lse and lse is None:
        lse = torch.empty(q_i8.shape[:3], dtype=torch.float32, device=v.device)
    _keep, mp = _map_arg(kv_head_map)
    _check(lib().attn_fwd_int8_masked(ctypes.byref(sh), _ptr(q_i8), _ptr(qs), _ptr(k_i8), _ptr(ks), _ptr(v),
                                      _ptr(out), _ptr(lse), mp, _ptr(rp), _ptr(cols), nnz,
                                      float(sm_scale or 0.0), _stream(stream)), "attn_fwd_int8_masked")
    return (out, lse) if (return_lse or lse is not None) else out
