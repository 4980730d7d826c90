"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/attn.h declares, and rejects every invalid argument on the host,
before any HIP call (each call below fails validation, so nothing launches).
The Python wrappers' own checks (buffer shapes, devices, the length of the
kv-head map) are tested here too, on CPU tensors."""
import ctypes
import os
import re

import pytest

import bit_quantized_exact_amd as A
from bit_quantized_exact_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation fails first
MISALIGNED = 0x10008


def _declared(path=os.path.join(ROOT, "include", "attn.h")):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_every_public_header_is_checked():
    """include/ holds the ABI of libattn.so only."""
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["attn.h"]


def test_header_and_binding_agree():
    assert _declared() == sorted(_native.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = A.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_quant_blocks_and_status_strings():
    assert A.quant_blocks() == (128, 64)
    L = A.lib()
    assert L.attn_quant_blocks(None, None) == 0
    for st in (0, -1, -2, -3, -4, -5):
        assert A.status_string(st) and A.status_string(st) != "unknown status"
    assert A.status_string(7) == "unknown status"


def _sh(B=1, Hq=4, Hkv=2, S=256, D=128):
    return A.AttnShape(B, Hq, Hkv, S, D)


def test_workspace_bytes():
    n = A.quantize_workspace_bytes(_sh())
    # partial sums (int64) for 1 chunk of 256 tokens, 2 kv-heads, 128 channels, plus the means
    assert n >= 2 * 1 * 128 * 8 + 2 * 128 * 4 and n % 256 == 0
    assert A.quantize_workspace_bytes(_sh(D=96)) == 0
    assert A.lib().attn_quantize_workspace_bytes(None) == 0
    big = A.quantize_workspace_bytes(_sh(B=2, Hkv=8, Hq=32, S=32768))
    assert big >= 2 * 8 * 128 * 128 * 8


def _fp16(L, sh, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, mp=None, causal=0, scale=0.0):
    return L.attn_fwd_fp16(ctypes.byref(sh) if sh is not None else None, q, k, v, o, lse, mp,
                           causal, scale, None)


def _int8(L, sh, q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, v=FAKE, o=FAKE, lse=None, mp=None, scale=0.0):
    return L.attn_fwd_int8(ctypes.byref(sh) if sh is not None else None, q, qs, k, ks, v, o, lse,
                           mp, 0, scale, None)


def _quant(L, sh, q=FAKE, k=FAKE, qi=FAKE, qs=FAKE, ki=FAKE, ks=FAKE, mean=None, ws=FAKE):
    return L.attn_quantize_qk(ctypes.byref(sh) if sh is not None else None, q, k, qi, qs, ki, ks,
                              mean, ws, None)


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, -1), ("heads_q", -1, -1), ("heads_kv", 0, -1), ("seq", 0, -1),
    ("head_dim", 0, -1), ("head_dim", 96, -2), ("head_dim", 256, -2),
    ("heads_q", 257, -2), ("seq", (1 << 22) + 1, -2)])
def test_shape_validation(field, value, code):
    L = A.lib()
    sh = _sh()
    setattr(sh, field, value)
    assert _fp16(L, sh) == code
    assert _int8(L, sh) == code
    assert _quant(L, sh) == code


def test_null_shape():
    L = A.lib()
    assert _fp16(L, None) == -1
    assert _int8(L, None) == -1
    assert _quant(L, None) == -1
    assert L.attn_debug_qk_int32(None, FAKE, FAKE, None, 0, 0, 0, FAKE, None) == -1


@pytest.mark.parametrize("arg", ["q", "k", "v", "o"])
def test_fp16_null_and_misaligned(arg):
    L = A.lib()
    assert _fp16(L, _sh(), **{arg: None}) == -1
    assert _fp16(L, _sh(), **{arg: MISALIGNED}) == -1


def test_fp16_lse_alignment():
    assert _fp16(A.lib(), _sh(), lse=FAKE + 2) == -1


@pytest.mark.parametrize("arg", ["q", "qs", "k", "ks", "v", "o"])
def test_int8_null(arg):
    assert _int8(A.lib(), _sh(), **{arg: None}) == -1


@pytest.mark.parametrize("arg", ["q", "k", "qi", "qs", "ki", "ks", "ws"])
def test_quant_null(arg):
    assert _quant(A.lib(), _sh(), **{arg: None}) == -1


def test_quant_misaligned():
    L = A.lib()
    assert _quant(L, _sh(), q=MISALIGNED) == -1
    assert _quant(L, _sh(), ws=MISALIGNED) == -1
    assert _quant(L, _sh(), qs=FAKE + 2) == -1


def test_group_divisibility_without_map():
    L = A.lib()
    sh = _sh(Hq=6, Hkv=4)
    assert _fp16(L, sh) == -1
    assert _int8(L, sh) == -1


def test_map_entries_out_of_range():
    L = A.lib()
    sh = _sh(Hq=4, Hkv=2)
    # make the call fail at the map check: map validated before launch, and a
    # NaN scale afterwards would also fail; use both orders to be sure nothing launches
    bad = (ctypes.c_int32 * 4)(0, 1, 2, 0)
    assert _fp16(L, sh, mp=ctypes.cast(bad, ctypes.c_void_p)) == -4
    neg = (ctypes.c_int32 * 4)(0, -1, 1, 0)
    assert _int8(L, sh, mp=ctypes.cast(neg, ctypes.c_void_p)) == -4


def test_nan_scale_rejected():
    L = A.lib()
    assert _fp16(L, _sh(), scale=float("nan")) == -1
    assert _int8(L, _sh(), scale=float("inf")) == -1


@pytest.mark.parametrize("lo,hi", [(-1, 0), (1, 0), (0, 2), (2, 2)])
def test_debug_tile_range(lo, hi):
    L = A.lib()
    sh = _sh(S=256)    # two query tiles
    assert L.attn_debug_qk_int32(ctypes.byref(sh), FAKE, FAKE, None, 0, lo, hi, FAKE, None) == -1


@pytest.mark.parametrize("lo,hi", [(-1, 0), (1, 0), (0, 2), (2, 2)])
def test_debug_fused_q_tile_range(lo, hi):
    L = A.lib()
    sh = _sh(S=256)    # two query tiles
    assert L.attn_debug_qk_int32_fused_q(ctypes.byref(sh), FAKE, FAKE, None, 0, lo, hi, FAKE, None, None) == -1


def test_debug_null_and_alignment():
    L = A.lib()
    sh = _sh()
    assert L.attn_debug_qk_int32(ctypes.byref(sh), None, FAKE, None, 0, 0, 0, FAKE, None) == -1
    assert L.attn_debug_qk_int32(ctypes.byref(sh), FAKE, FAKE, None, 0, 0, 0, FAKE + 2, None) == -1
    F = L.attn_debug_qk_int32_fused_q
    assert F(None, FAKE, FAKE, None, 0, 0, 0, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), None, FAKE, None, 0, 0, 0, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), FAKE, None, None, 0, 0, 0, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), FAKE, FAKE, None, 0, 0, 0, None, None, None) == -1
    assert F(ctypes.byref(sh), MISALIGNED, FAKE, None, 0, 0, 0, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), FAKE, FAKE, None, 0, 0, 0, FAKE, FAKE + 2, None) == -1
    bad = (ctypes.c_int32 * 4)(0, 1, 2, 0)
    assert F(ctypes.byref(sh), FAKE, FAKE, ctypes.cast(bad, ctypes.c_void_p), 0, 0, 0, FAKE, None, None) == -4
    assert F(ctypes.byref(_sh(D=96)), FAKE, FAKE, None, 0, 0, 0, FAKE, None, None) == -2


def test_quantize_k_noalloc_rejects_on_the_host():
    """Argument checks and the scratch limit run before any HIP call."""
    L = A.lib()
    F = L.attn_quantize_k_noalloc
    sh = _sh(Hq=2, Hkv=2)
    assert F(None, FAKE, FAKE, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), None, FAKE, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), FAKE, None, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), FAKE, FAKE, None, None, None) == -1
    assert F(ctypes.byref(sh), MISALIGNED, FAKE, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), FAKE, MISALIGNED, FAKE, None, None) == -1
    assert F(ctypes.byref(sh), FAKE, FAKE, FAKE + 2, None, None) == -1
    assert F(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE + 2, None) == -1
    assert F(ctypes.byref(_sh(D=96)), FAKE, FAKE, FAKE, None, None) == -2
    # the largest shapes that fit, and the smallest that do not
    cap = _native.ATTN_NOALLOC_SCRATCH_BYTES
    fits = A.AttnShape(32, 1, 1, 65536, 128)
    assert 0 < A.quantize_workspace_bytes(fits) <= cap
    too_big = A.AttnShape(64, 1, 1, 65536, 128)
    assert A.quantize_workspace_bytes(too_big) > cap
    assert F(ctypes.byref(too_big), FAKE, FAKE, FAKE, None, None) == -5
    assert "scratch" in A.status_string(-5)


# --------------------------------------------------------------------------
# the Python wrappers' own checks (CPU tensors stand in for device buffers)
# --------------------------------------------------------------------------
def test_map_arg_requires_one_entry_per_query_head():
    arr, ptr = A._map_arg([0, 1, 1, 0], 4)
    assert list(arr) == [0, 1, 1, 0] and ptr is not None
    assert A._map_arg(None, 4) == (None, None)
    for bad in ([0, 1, 1], [0, 1, 1, 0, 1], []):
        with pytest.raises(ValueError):
            A._map_arg(bad, 4)


def test_buffer_checks_reject_wrong_shape_dtype_device_layout():
    import torch
    cpu = torch.device("cpu")
    good = torch.zeros(1, 4, 256, 128, dtype=torch.float16)
    assert A._out_arg(good, (1, 4, 256, 128), cpu) is good
    for bad in (torch.zeros(1, 4, 255, 128, dtype=torch.float16),          # short
                torch.zeros(1, 4, 256, 128, dtype=torch.float32),          # dtype
                torch.zeros(1, 4, 128, 256, dtype=torch.float16).transpose(2, 3)):   # layout
        with pytest.raises(ValueError):
            A._out_arg(bad, (1, 4, 256, 128), cpu)
    with pytest.raises(ValueError):
        A._out_arg(good, (1, 4, 256, 128), torch.device("meta"))           # device
    lse = torch.zeros(1, 4, 256, dtype=torch.float32)
    assert A._lse_arg(lse, False, (1, 4, 256), cpu) is lse
    assert A._lse_arg(None, False, (1, 4, 256), cpu) is None
    assert A._lse_arg(None, True, (1, 4, 256), cpu).shape == (1, 4, 256)
    for bad in (torch.zeros(1, 4, 256, dtype=torch.float16), torch.zeros(1, 4, 200, dtype=torch.float32),
                torch.zeros(4, 256, dtype=torch.float32)):
        with pytest.raises(ValueError):
            A._lse_arg(bad, True, (1, 4, 256), cpu)
    qs = torch.zeros(1, 4, 3, dtype=torch.float32)          # ceil(300 / 128) blocks
    assert A._scales(qs, 1, 4, 300, 128, cpu, "q_scale") is qs
    for bad in (torch.zeros(1, 4, 2, dtype=torch.float32), torch.zeros(1, 2, 3, dtype=torch.float32),
                torch.zeros(1, 4, 3, dtype=torch.float64)):
        with pytest.raises(ValueError):
            A._scales(bad, 1, 4, 300, 128, cpu, "q_scale")
    with pytest.raises(ValueError):
        A._same_device(good, torch.zeros(1, device="meta"))


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        A.fwd_fp16(q, q, q)
    with pytest.raises(ValueError):
        A.quantize_qk(q, q)


def test_quantize_k_validation():
    L = A.lib()
    sh = _sh()
    assert L.attn_quantize_k(None, FAKE, FAKE, FAKE, None, FAKE, None) == -1
    for args in [(None, FAKE, FAKE, None, FAKE), (FAKE, None, FAKE, None, FAKE),
                 (FAKE, FAKE, None, None, FAKE), (FAKE, FAKE, FAKE, None, None),
                 (MISALIGNED, FAKE, FAKE, None, FAKE), (FAKE, FAKE, FAKE + 2, None, FAKE)]:
        assert L.attn_quantize_k(ctypes.byref(sh), *args, None) == -1
    bad = _sh(D=96)
    assert L.attn_quantize_k(ctypes.byref(bad), FAKE, FAKE, FAKE, None, FAKE, None) == -2


def test_fused_q_validation():
    L = A.lib()
    sh = _sh()

    def call(q=FAKE, k=FAKE, ks=FAKE, v=FAKE, o=FAKE, lse=None, qs=None, mp=None, scale=0.0, shape=sh):
        return L.attn_fwd_int8_fused_q(ctypes.byref(shape) if shape is not None else None, q, k, ks,
                                       v, o, lse, qs, mp, 0, scale, None)
    assert call(shape=None) == -1
    for arg in ("q", "k", "ks", "v", "o"):
        assert call(**{arg: None}) == -1
    assert call(q=MISALIGNED) == -1
    assert call(qs=FAKE + 2) == -1
    assert call(scale=float("nan")) == -1
    assert call(shape=_sh(Hq=6, Hkv=4)) == -1
    bad = (ctypes.c_int32 * 4)(0, 1, 2, 0)
    assert call(mp=ctypes.cast(bad, ctypes.c_void_p)) == -4


def test_fp8_entry_points_validation():
    L = A.lib()
    sh = _sh()
    P = ctypes.byref(sh)
    # attn_quantize_qk_fp8: same contract as attn_quantize_qk
    assert L.attn_quantize_qk_fp8(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == -1
    for i in range(7):
        args = [FAKE] * 7
        args[i] = None
        q, k, qf, qs, kf, ks, ws = args
        assert L.attn_quantize_qk_fp8(P, q, k, qf, qs, kf, ks, None, ws, None) == -1
    assert L.attn_quantize_qk_fp8(P, FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE, None, FAKE, None) == -1
    bad = _sh(D=96)
    assert L.attn_quantize_qk_fp8(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                  None) == -2

    # attn_fwd_fp8: as attn_fwd_int8
    def fp8(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, v=FAKE, o=FAKE, lse=None, mp=None, scale=0.0, shape=sh):
        return L.attn_fwd_fp8(ctypes.byref(shape) if shape is not None else None, q, qs, k, ks, v, o,
                              lse, mp, 0, scale, None)
    assert fp8(shape=None) == -1
    for arg in ("q", "qs", "k", "ks", "v", "o"):
        assert fp8(**{arg: None}) == -1
    assert fp8(k=MISALIGNED) == -1 and fp8(ks=FAKE + 2) == -1 and fp8(lse=FAKE + 2) == -1
    assert fp8(scale=float("nan")) == -1
    assert fp8(shape=_sh(Hq=6, Hkv=4)) == -1
    badmap = (ctypes.c_int32 * 4)(0, 1, 2, 0)
    assert fp8(mp=ctypes.cast(badmap, ctypes.c_void_p)) == -4

    # the transposed-V stride and its quantiser
    assert L.attn_v_fp8_stride(ctypes.byref(_sh(S=1))) == 64
    assert L.attn_v_fp8_stride(ctypes.byref(_sh(S=64))) == 64
    assert L.attn_v_fp8_stride(ctypes.byref(_sh(S=65))) == 128
    assert L.attn_v_fp8_stride(ctypes.byref(_sh(D=96))) == 0
    assert L.attn_v_fp8_stride(None) == 0
    assert L.attn_quantize_v_fp8(None, FAKE, FAKE, FAKE, FAKE, None) == -1
    for args in [(None, FAKE, FAKE, FAKE), (FAKE, None, FAKE, FAKE), (FAKE, FAKE, None, FAKE),
                 (FAKE, FAKE, FAKE, None), (MISALIGNED, FAKE, FAKE, FAKE),
                 (FAKE, MISALIGNED, FAKE, FAKE), (FAKE, FAKE, FAKE + 2, FAKE)]:
        assert L.attn_quantize_v_fp8(P, *args, None) == -1
    assert L.attn_quantize_v_fp8(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None) == -2

    # attn_fwd_int8_pv8
    def pv8(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, vt=FAKE, vs=FAKE, o=FAKE, lse=None, mp=None,
            scale=0.0, shape=sh):
        return L.attn_fwd_int8_pv8(ctypes.byref(shape) if shape is not None else None, q, qs, k, ks,
                                   vt, vs, o, lse, mp, 1, scale, None)
    assert pv8(shape=None) == -1
    for arg in ("q", "qs", "k", "ks", "vt", "vs", "o"):
        assert pv8(**{arg: None}) == -1
    assert pv8(vt=MISALIGNED) == -1 and pv8(vs=FAKE + 2) == -1
    assert pv8(scale=float("inf")) == -1
    assert pv8(shape=bad) == -2
    assert pv8(mp=ctypes.cast(badmap, ctypes.c_void_p)) == -4


def _kv(B=1, Hq=4, Hkv=2, Sq=1, Sk=256, D=128):
    return A.AttnKvShape(B, Hq, Hkv, Sq, Sk, D)


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, -1), ("heads_q", 0, -1), ("heads_kv", -2, -1), ("seq_q", 0, -1), ("seq_kv", 0, -1),
    ("head_dim", 0, -1), ("seq_q", 301, -1), ("seq_q", 33, -2), ("head_dim", 80, -2), ("heads_kv", 257, -2),
    ("seq_kv", (1 << 22) + 1, -2)])
def test_decode_shape_validation(field, value, code):
    L = A.lib()
    sh = _kv(Sk=300)
    setattr(sh, field, value)
    assert L.attn_decode_int8(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 1, 0.0,
                              FAKE, None) == code
    assert L.attn_decode_fp16(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, None, 1, 0.0, FAKE,
                              None) == code
    assert L.attn_decode_workspace_bytes(ctypes.byref(sh), None) == 0


def test_decode_seq_q_limit():
    L = A.lib()
    ok, big = _kv(Sq=32, Sk=64), _kv(Sq=33, Sk=64)
    assert L.attn_decode_workspace_bytes(ctypes.byref(ok), None) > 0
    assert L.attn_decode_fp16(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, None, None, 1, 0.0, FAKE,
                              None) == -2


def test_decode_workspace_and_validation():
    L = A.lib()
    sh = _kv(B=2, Hq=32, Hkv=8, Sq=1, Sk=8192)
    n = L.attn_decode_workspace_bytes(ctypes.byref(sh), None)
    # at least one partial row (D floats + max + sum) per (batch, kv-head, split)
    assert n >= 2 * 8 * (128 + 2) * 4 and n % 256 == 0
    assert L.attn_decode_workspace_bytes(None, None) == 0
    bad = (ctypes.c_int32 * 32)(*([0] * 31 + [8]))
    assert L.attn_decode_workspace_bytes(ctypes.byref(sh), ctypes.cast(bad, ctypes.c_void_p)) == 0
    P = ctypes.byref(sh)
    for i in range(6):
        args = [FAKE] * 6
        args[i] = None
        q, k, ks, v, o, ws = args
        assert L.attn_decode_int8(P, q, k, ks, v, o, None, None, None, 1, 0.0, ws, None) == -1
    assert L.attn_decode_int8(P, MISALIGNED, FAKE, FAKE, FAKE, FAKE, None, None, None, 1, 0.0, FAKE,
                              None) == -1
    assert L.attn_decode_int8(P, FAKE, FAKE, FAKE + 2, FAKE, FAKE, None, None, None, 1, 0.0, FAKE,
                              None) == -1
    assert L.attn_decode_int8(P, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 2, None, 1, 0.0, FAKE,
                              None) == -1
    assert L.attn_decode_fp16(P, FAKE, FAKE, FAKE, FAKE, None, None, 1, float("nan"), FAKE, None) == -1
    assert L.attn_decode_fp16(P, FAKE, FAKE, FAKE, FAKE, None, ctypes.cast(bad, ctypes.c_void_p), 1, 0.0,
                              FAKE, None) == -4
    assert L.attn_decode_fp16(P, FAKE, FAKE, FAKE, FAKE, None, None, 1, 0.0, MISALIGNED, None) == -1
    odd = _kv(Hq=6, Hkv=4)
    assert L.attn_decode_fp16(ctypes.byref(odd), FAKE, FAKE, FAKE, FAKE, None, None, 1, 0.0, FAKE,
                              None) == -1


def test_mfma_probe_library_is_separate():
    """The dense MFMA loop lives in libattn_probe.so, not in the attention ABI."""
    from bit_quantized_exact_amd import probe
    hdr = os.path.join(ROOT, "bit_quantized_exact_amd", "probe", "mfma_probe.h")
    assert _declared(hdr) == sorted(probe.EXPORTED)
    L = probe.lib()
    for name in probe.EXPORTED:
        assert hasattr(L, name)
        assert not hasattr(A.lib(), name)


def test_mfma_probe_rejects_bad_arguments():
    from bit_quantized_exact_amd import probe
    L = probe.lib()
    ops = ctypes.c_double(0.0)
    assert L.attn_probe_mfma(4, 1, 1, FAKE, ctypes.byref(ops), None) == -1    # unknown kind
    assert L.attn_probe_mfma(-1, 1, 1, FAKE, ctypes.byref(ops), None) == -1   # unknown kind
    assert L.attn_probe_mfma(0, 0, 1, FAKE, ctypes.byref(ops), None) == -1    # no blocks
    assert L.attn_probe_mfma(1, 1, 0, FAKE, ctypes.byref(ops), None) == -1    # no iterations
    assert L.attn_probe_mfma(0, 1, 1, None, ctypes.byref(ops), None) == -1    # no sink
    assert L.attn_probe_compute_units(None) == -1
    assert L.attn_probe_hbm_read(None, 16, 1, FAKE, None) == -1                # no buffer
    assert L.attn_probe_hbm_read(FAKE, 0, 1, FAKE, None) == -1                 # no bytes
    assert L.attn_probe_hbm_read(FAKE, 24, 1, FAKE, None) == -1                # not whole 16-byte chunks
    assert L.attn_probe_hbm_read(FAKE, 16, 0, FAKE, None) == -1                # no blocks
    assert L.attn_probe_hbm_read(FAKE, 16, 1, None, None) == -1                # no sink
    assert L.attn_probe_hbm_read(MISALIGNED, 16, 1, FAKE, None) == -1          # misaligned
