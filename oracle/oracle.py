"""Python wrapper of the CPU oracle (attn_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP path.  Arrays are numpy; fp16
tensors are passed as their raw uint16 bits and decoded by the C code from the
binary16 definition.

Every function here is a direct call into the C oracle; the only arithmetic in
this file is argument preparation (shapes, contiguity, default map and scale).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Block sizes of the quantisation reading (rows per Q block, rows per K block).
BQ, BK = 128, 64

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = D
        L.oracle_round_to_half.argtypes = [D]
        L.oracle_round_to_half.restype = D
        L.oracle_half_array_to_double.argtypes = [P, P, I64]
        L.oracle_half_array_to_float.argtypes = [P, P, I64]
        L.oracle_attention.argtypes = [I32] * 5 + [P, P, P, P, I32, D, P, I32, P, P, I32]
        L.oracle_attention.restype = ctypes.c_int
        L.oracle_k_mean.argtypes = [I32] * 4 + [P, P]
        L.oracle_k_mean.restype = ctypes.c_int
        L.oracle_smooth_k.argtypes = [I32] * 4 + [P, P, P]
        L.oracle_quant_blocks.argtypes = [I64, I32, I32, I32, P, P, P]
        L.oracle_scores_i32.argtypes = [I32] * 5 + [P, P, P, I32, P, I32, P, I32]
        L.oracle_scores_i32.restype = ctypes.c_int
        L.oracle_quant_attention.argtypes = ([I32] * 5 + [P, P, I32, P, P, I32, P, P, I32, D, I32,
                                             P, I32, P, P, I32])
        L.oracle_quant_attention.restype = ctypes.c_int
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = D
        L.oracle_e4m3_round.argtypes = [D]
        L.oracle_e4m3_round.restype = D
        L.oracle_e4m3_encode.argtypes = [D]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_round_array.argtypes = [P, P, I64]
        L.oracle_e4m3_decode_array.argtypes = [P, P, I64]
        L.oracle_quant_blocks_e4m3.argtypes = [I64, I32, I32, I32, P, P, P]
        L.oracle_quant_v_e4m3.argtypes = [I32] * 4 + [P, P, P]
        L.oracle_quant_attention_e4m3.argtypes = L.oracle_quant_attention.argtypes
        L.oracle_quant_attention_e4m3.restype = ctypes.c_int
        L.oracle_pv8_attention.argtypes = ([I32] * 5 + [P, P, I32, P, P, I32, P, P, P, I32, D, I32,
                                           I32, P, I32, P, P, D, P, I32])
        L.oracle_pv8_attention.restype = ctypes.c_int
        L.oracle_attention_kv.argtypes = [I32] * 6 + [P, P, P, P, I32, D, P, P, I32]
        L.oracle_attention_kv.restype = ctypes.c_int
        L.oracle_quant_attention_kv.argtypes = ([I32] * 6 + [P, P, I32, P, P, I32, P, P, I32, D, P, P,
                                                I32])
        L.oracle_quant_attention_kv.restype = ctypes.c_int
        L.oracle_attention_masked.argtypes = [I32] * 5 + [P, P, P, P, P, I32, I32, D, P, P, I32]
        L.oracle_attention_masked.restype = ctypes.c_int
        L.oracle_quant_attention_masked.argtypes = ([I32] * 5 + [P, P, I32, P, P, I32, P, P, P, I32, I32,
                                                    D, P, P, I32])
        L.oracle_quant_attention_masked.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits(x: np.ndarray) -> np.ndarray:
    assert x.dtype == np.float16
    return np.ascontiguousarray(x).view(np.uint16)


def _map(Hq: int, Hkv: int, kv_map):
    if kv_map is None:
        assert Hq % Hkv == 0
        kv_map = np.arange(Hq, dtype=np.int32) // (Hq // Hkv)
    return np.ascontiguousarray(np.asarray(kv_map, dtype=np.int32))


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    return r, int(r.size)


def _check(status: int, what: str):
    if status != 0:
        raise RuntimeError(f"oracle {what} failed with status {status}")


def half_to_double(h16: np.ndarray) -> np.ndarray:
    b = _bits(h16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_half_array_to_double(_ptr(b), _ptr(out), b.size)
    return out


def half_to_float(h16: np.ndarray) -> np.ndarray:
    b = _bits(h16)
    out = np.empty(b.shape, dtype=np.float32)
    lib().oracle_half_array_to_float(_ptr(b), _ptr(out), b.size)
    return out


def round_to_half(x: float) -> float:
    return lib().oracle_round_to_half(float(x))


def attention(q, k, v, causal=False, kv_map=None, sm_scale=None, rows=None,
              with_lse=False, nthreads=0):
    """O1: exact fp64 attention.  q [B,Hq,S,D], k/v [B,Hkv,S,D] fp16.

    Returns out [B,Hq,nrows,D] fp64 (and lse [B,Hq,nrows] when asked)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, S, D) and v.shape == k.shape
    m = _map(Hq, Hkv, kv_map)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    r, nr = _rows(rows)
    n = nr if r is not None else S
    out = np.empty((B, Hq, n, D), dtype=np.float64)
    lse = np.empty((B, Hq, n), dtype=np.float64) if with_lse else None
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    st = lib().oracle_attention(B, Hq, Hkv, S, D, _ptr(qb), _ptr(kb), _ptr(vb), _ptr(m),
                                int(bool(causal)), float(sm_scale),
                                _ptr(r) if r is not None else None, nr,
                                _ptr(out), _ptr(lse) if lse is not None else None, int(nthreads))
    _check(st, "attention")
    return (out, lse) if with_lse else out


def k_mean(k):
    """O2: per-(batch, kv-head) channel mean of K over tokens, fp32 [B,Hkv,D]."""
    B, Hkv, S, D = k.shape
    mu = np.empty((B, Hkv, D), dtype=np.float32)
    kb = _bits(k)
    _check(lib().oracle_k_mean(B, Hkv, S, D, _ptr(kb), _ptr(mu)), "k_mean")
    return mu


def smooth_k(k, mu):
    B, Hkv, S, D = k.shape
    ks = np.empty(k.shape, dtype=np.float32)
    kb = _bits(k)
    mu = np.ascontiguousarray(mu, dtype=np.float32)
    lib().oracle_smooth_k(B, Hkv, S, D, _ptr(kb), _ptr(mu), _ptr(ks))
    return ks


def quant_blocks(x32, block):
    """O3 on a float32 array [..., S, D]: returns (int8 same shape, scale [..., nblk])."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    *lead, S, D = x32.shape
    nmat = int(np.prod(lead)) if lead else 1
    nblk = (S + block - 1) // block
    q = np.empty(x32.shape, dtype=np.int8)
    sc = np.empty((*lead, nblk), dtype=np.float32)
    lib().oracle_quant_blocks(nmat, S, D, block, _ptr(x32), _ptr(q), _ptr(sc))
    return q, sc


def quantize_qk(q, k, bq=BQ, bk=BK):
    """O2 + O3: returns dict with q_i8, q_scale, k_i8, k_scale, k_mean."""
    mu = k_mean(k)
    ks = smooth_k(k, mu)
    qi, qs = quant_blocks(half_to_float(q), bq)
    ki, kscale = quant_blocks(ks, bk)
    return dict(q_i8=qi, q_scale=qs, k_i8=ki, k_scale=kscale, k_mean=mu)


def scores_i32(q_i8, k_i8, causal=False, kv_map=None, rows=None, fill=0):
    B, Hq, S, D = q_i8.shape
    Hkv = k_i8.shape[1]
    m = _map(Hq, Hkv, kv_map)
    r, nr = _rows(rows)
    n = nr if r is not None else S
    out = np.empty((B, Hq, n, S), dtype=np.int32)
    qi = np.ascontiguousarray(q_i8)
    ki = np.ascontiguousarray(k_i8)
    st = lib().oracle_scores_i32(B, Hq, Hkv, S, D, _ptr(qi), _ptr(ki), _ptr(m), int(bool(causal)),
                                 _ptr(r) if r is not None else None, nr, _ptr(out), int(fill))
    _check(st, "scores_i32")
    return out


def quant_attention(qz, v, causal=False, kv_map=None, sm_scale=None, rows=None,
                    with_lse=False, bq=BQ, bk=BK, l_from_rounded=False, nthreads=0):
    """O4: attention on dequantised integer scores with fp16-rounded weights."""
    qi = np.ascontiguousarray(qz["q_i8"])
    ki = np.ascontiguousarray(qz["k_i8"])
    qs = np.ascontiguousarray(qz["q_scale"], dtype=np.float32)
    ks = np.ascontiguousarray(qz["k_scale"], dtype=np.float32)
    B, Hq, S, D = qi.shape
    Hkv = ki.shape[1]
    m = _map(Hq, Hkv, kv_map)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    r, nr = _rows(rows)
    n = nr if r is not None else S
    out = np.empty((B, Hq, n, D), dtype=np.float64)
    lse = np.empty((B, Hq, n), dtype=np.float64) if with_lse else None
    vb = _bits(v)
    st = lib().oracle_quant_attention(B, Hq, Hkv, S, D, _ptr(qi), _ptr(qs), bq, _ptr(ki), _ptr(ks), bk,
                                      _ptr(vb), _ptr(m), int(bool(causal)), float(sm_scale),
                                      int(bool(l_from_rounded)),
                                      _ptr(r) if r is not None else None, nr,
                                      _ptr(out), _ptr(lse) if lse is not None else None, int(nthreads))
    _check(st, "quant_attention")
    return (out, lse) if with_lse else out


# --------------------------------------------------------------------------
# FP8 (E4M3) alternative and the 8-bit P.V ablation
# --------------------------------------------------------------------------
def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 values (ties to even, saturating at 448), as fp64."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty_like(x)
    lib().oracle_e4m3_round_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_encode(x: float) -> int:
    return int(lib().oracle_e4m3_encode(float(x)))


def quant_blocks_e4m3(x32, block):
    """O3 on the E4M3 grid: returns (uint8 codes same shape, scale [..., nblk])."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    *lead, S, D = x32.shape
    nmat = int(np.prod(lead)) if lead else 1
    nblk = (S + block - 1) // block
    q = np.empty(x32.shape, dtype=np.uint8)
    sc = np.empty((*lead, nblk), dtype=np.float32)
    lib().oracle_quant_blocks_e4m3(nmat, S, D, block, _ptr(x32), _ptr(q), _ptr(sc))
    return q, sc


def quantize_qk_fp8(q, k, bq=BQ, bk=BK):
    """O2 + O3 (E4M3): returns dict with q_f8, q_scale, k_f8, k_scale, k_mean."""
    mu = k_mean(k)
    ks = smooth_k(k, mu)
    qf, qs = quant_blocks_e4m3(half_to_float(q), bq)
    kf, kscale = quant_blocks_e4m3(ks, bk)
    return dict(q_f8=qf, q_scale=qs, k_f8=kf, k_scale=kscale, k_mean=mu)


def quant_v_fp8(v):
    """8-bit V of the P.V ablation: codes [B,Hkv,S,D] uint8, scale [B,Hkv,D]."""
    B, Hkv, S, D = v.shape
    codes = np.empty(v.shape, dtype=np.uint8)
    sc = np.empty((B, Hkv, D), dtype=np.float32)
    vb = _bits(v)
    lib().oracle_quant_v_e4m3(B, Hkv, S, D, _ptr(vb), _ptr(codes), _ptr(sc))
    return codes, sc


def quant_attention_fp8(qz, v, causal=False, kv_map=None, sm_scale=None, rows=None,
                        with_lse=False, bq=BQ, bk=BK, l_from_rounded=False, nthreads=0):
    """O4 on E4M3 Q/K codes (qz from quantize_qk_fp8)."""
    qf = np.ascontiguousarray(qz["q_f8"], dtype=np.uint8)
    kf = np.ascontiguousarray(qz["k_f8"], dtype=np.uint8)
    qs = np.ascontiguousarray(qz["q_scale"], dtype=np.float32)
    ks = np.ascontiguousarray(qz["k_scale"], dtype=np.float32)
    B, Hq, S, D = qf.shape
    Hkv = kf.shape[1]
    m = _map(Hq, Hkv, kv_map)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    r, nr = _rows(rows)
    n = nr if r is not None else S
    out = np.empty((B, Hq, n, D), dtype=np.float64)
    lse = np.empty((B, Hq, n), dtype=np.float64) if with_lse else None
    vb = _bits(v)
    st = lib().oracle_quant_attention_e4m3(B, Hq, Hkv, S, D, _ptr(qf), _ptr(qs), bq, _ptr(kf),
                                           _ptr(ks), bk, _ptr(vb), _ptr(m), int(bool(causal)),
                                           float(sm_scale), int(bool(l_from_rounded)),
                                           _ptr(r) if r is not None else None, nr,
                                           _ptr(out), _ptr(lse) if lse is not None else None,
                                           int(nthreads))
    _check(st, "quant_attention_e4m3")
    return (out, lse) if with_lse else out


def pv8_attention(qz, v_codes, v_scale, causal=False, kv_map=None, sm_scale=None, rows=None,
                  with_lse=False, bq=BQ, bk=BK, tile=BK, p_quant=True, tie_rel=None, nthreads=0):
    """O5: INT8 Q/K scores, 8-bit P (against the running maximum of the
    online softmax over key tiles of `tile` keys) and 8-bit V.

    With tie_rel (a relative distance) it also returns, per output row, the
    bound on how far O may move when weights whose 448 p lies within tie_rel
    of an E4M3 half-way point round to the other neighbour: returns
    (out, lse, slack) or (out, slack)."""
    qi = np.ascontiguousarray(qz["q_i8"])
    ki = np.ascontiguousarray(qz["k_i8"])
    qs = np.ascontiguousarray(qz["q_scale"], dtype=np.float32)
    ks = np.ascontiguousarray(qz["k_scale"], dtype=np.float32)
    vc = np.ascontiguousarray(v_codes, dtype=np.uint8)
    vs = np.ascontiguousarray(v_scale, dtype=np.float32)
    B, Hq, S, D = qi.shape
    Hkv = ki.shape[1]
    assert vc.shape == (B, Hkv, S, D) and vs.shape == (B, Hkv, D)
    m = _map(Hq, Hkv, kv_map)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    r, nr = _rows(rows)
    n = nr if r is not None else S
    out = np.empty((B, Hq, n, D), dtype=np.float64)
    lse = np.empty((B, Hq, n), dtype=np.float64) if with_lse else None
    slack = np.empty((B, Hq, n), dtype=np.float64) if tie_rel is not None else None
    st = lib().oracle_pv8_attention(B, Hq, Hkv, S, D, _ptr(qi), _ptr(qs), bq, _ptr(ki), _ptr(ks), bk,
                                    _ptr(vc), _ptr(vs), _ptr(m), int(bool(causal)), float(sm_scale),
                                    int(tile), int(bool(p_quant)),
                                    _ptr(r) if r is not None else None, nr,
                                    _ptr(out), _ptr(lse) if lse is not None else None,
                                    float(tie_rel or 0.0), _ptr(slack) if slack is not None else None,
                                    int(nthreads))
    _check(st, "pv8_attention")
    res = (out,) + ((lse,) if with_lse else ()) + ((slack,) if slack is not None else ())
    return res if len(res) > 1 else out


# --------------------------------------------------------------------------
# KV-cache (decode) case: Sq queries over Sk >= Sq cached keys
# --------------------------------------------------------------------------
def attention_kv(q, k, v, causal=False, kv_map=None, sm_scale=None, with_lse=False, nthreads=0):
    """O1 for Sq queries (the last Sq positions) over Sk cached keys.
    q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D] fp16 -> out [B,Hq,Sq,D] fp64 (and lse)."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    assert k.shape == (B, Hkv, Sk, D) and v.shape == k.shape
    m = _map(Hq, Hkv, kv_map)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.empty((B, Hq, Sq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64) if with_lse else None
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    st = lib().oracle_attention_kv(B, Hq, Hkv, Sq, Sk, D, _ptr(qb), _ptr(kb), _ptr(vb), _ptr(m),
                                   int(bool(causal)), float(sm_scale), _ptr(out),
                                   _ptr(lse) if lse is not None else None, int(nthreads))
    _check(st, "attention_kv")
    return (out, lse) if with_lse else out


def quantize_q(q, bq=BQ):
    """O3 on Q alone: (q_i8, q_scale [B,Hq,ceil(Sq/bq)])."""
    return quant_blocks(half_to_float(q), bq)


def quant_attention_kv(q_i8, q_scale, kz, v, causal=False, kv_map=None, sm_scale=None,
                       with_lse=False, bq=BQ, bk=BK, nthreads=0):
    """O4 for the KV-cache case; kz holds k_i8/k_scale of the Sk cached keys."""
    qi = np.ascontiguousarray(q_i8)
    qs = np.ascontiguousarray(q_scale, dtype=np.float32)
    ki = np.ascontiguousarray(kz["k_i8"])
    ks = np.ascontiguousarray(kz["k_scale"], dtype=np.float32)
    B, Hq, Sq, D = qi.shape
    Hkv, Sk = ki.shape[1], ki.shape[2]
    m = _map(Hq, Hkv, kv_map)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.empty((B, Hq, Sq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64) if with_lse else None
    vb = _bits(v)
    st = lib().oracle_quant_attention_kv(B, Hq, Hkv, Sq, Sk, D, _ptr(qi), _ptr(qs), bq, _ptr(ki),
                                         _ptr(ks), bk, _ptr(vb), _ptr(m), int(bool(causal)),
                                         float(sm_scale), _ptr(out),
                                         _ptr(lse) if lse is not None else None, int(nthreads))
    _check(st, "quant_attention_kv")
    return (out, lse) if with_lse else out


def quantize_k_cache(k, bk=BK):
    """O2 + O3 on the cached keys alone: k_i8, k_scale, k_mean (mean over all Sk tokens)."""
    mu = k_mean(k)
    ki, ks = quant_blocks(smooth_k(k, mu), bk)
    return dict(k_i8=ki, k_scale=ks, k_mean=mu)


# --------------------------------------------------------------------------
# tile-level attention masks (APB-style anchor / passing / local blocks)
# --------------------------------------------------------------------------
TILE_Q, TILE_K = 128, 64   # mask granularity: query rows x keys per mask entry


def attention_masked(q, k, v, mask, kv_map=None, sm_scale=None, with_lse=False, tq=TILE_Q, tk=TILE_K,
                     nthreads=0):
    """O1 under a tile mask (0 invisible, 1 visible, 2 visible iff j <= i),
    mask [ceil(S/tq), ceil(S/tk)] uint8.  Rows with no visible key: O = 0, lse = -inf."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    m = _map(Hq, Hkv, kv_map)
    mk = np.ascontiguousarray(mask, dtype=np.uint8)
    assert mk.shape == (-(-S // tq), -(-S // tk))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.empty((B, Hq, S, D), dtype=np.float64)
    lse = np.empty((B, Hq, S), dtype=np.float64) if with_lse else None
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    st = lib().oracle_attention_masked(B, Hq, Hkv, S, D, _ptr(qb), _ptr(kb), _ptr(vb), _ptr(m), _ptr(mk),
                                       tq, tk, float(sm_scale), _ptr(out),
                                       _ptr(lse) if lse is not None else None, int(nthreads))
    _check(st, "attention_masked")
    return (out, lse) if with_lse else out


def quant_attention_masked(qz, v, mask, kv_map=None, sm_scale=None, with_lse=False, bq=BQ, bk=BK,
                           tq=TILE_Q, tk=TILE_K, nthreads=0):
    """O4 under a tile mask (qz from quantize_qk)."""
    qi = np.ascontiguousarray(qz["q_i8"])
    ki = np.ascontiguousarray(qz["k_i8"])
    qs = np.ascontiguousarray(qz["q_scale"], dtype=np.float32)
    ks = np.ascontiguousarray(qz["k_scale"], dtype=np.float32)
    B, Hq, S, D = qi.shape
    Hkv = ki.shape[1]
    m = _map(Hq, Hkv, kv_map)
    mk = np.ascontiguousarray(mask, dtype=np.uint8)
    assert mk.shape == (-(-S // tq), -(-S // tk))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.empty((B, Hq, S, D), dtype=np.float64)
    lse = np.empty((B, Hq, S), dtype=np.float64) if with_lse else None
    vb = _bits(v)
    st = lib().oracle_quant_attention_masked(B, Hq, Hkv, S, D, _ptr(qi), _ptr(qs), bq, _ptr(ki), _ptr(ks), bk,
                                             _ptr(vb), _ptr(m), _ptr(mk), tq, tk, float(sm_scale), _ptr(out),
                                             _ptr(lse) if lse is not None else None, int(nthreads))
    _check(st, "quant_attention_masked")
    return (out, lse) if with_lse else out


def max_threads() -> int:
    return lib().oracle_max_threads()
