"""GPU check of attn_quantize_k_noalloc, the entry point that allocates
nothing (its workspace is the library's own device scratch): bit for bit the
outputs of attn_quantize_k with a caller workspace, on consecutive calls of
shrinking and growing shapes (the scratch keeps the previous call's contents,
which must not matter), up to a shape that fills half the scratch."""
import numpy as np
import pytest
import torch

import bit_quantized_exact_amd as A
from bit_quantized_exact_amd import _native
from bit_quantized_exact_amd.inputs import make_qkv

from _util import case, small_workload

pytestmark = pytest.mark.gpu


def _k(B, H, S, D, seed):
    _, k, _ = make_qkv(small_workload(B, H, H, S, D, False, seed, offset_std=4.0))
    return torch.from_numpy(k).cuda()


def _same(kd, with_mean=True):
    ref = A.quantize_k(kd, with_mean=with_mean)
    got = A.quantize_k_noalloc(kd, with_mean=with_mean)
    torch.cuda.synchronize()
    for key in ("k_i8", "k_scale") + (("k_mean",) if with_mean else ()):
        assert torch.equal(got[key], ref[key]), key
    return got


def test_noalloc_matches_quantize_k_on_consecutive_calls():
    shapes = [(1, 8, 32768, 128, 1), (2, 3, 1000, 64, 2), (4, 2, 8193, 128, 3), (1, 1, 5, 64, 4)]
    for B, H, S, D, seed in shapes:      # large, then smaller, larger, smallest
        case(f"quantize_k_noalloc B={B} H={H} S={S} D={D}")
        _same(_k(B, H, S, D, seed))
    case("quantize_k_noalloc without the mean output")
    _same(_k(1, 2, 300, 128, 5), with_mean=False)


def test_noalloc_outputs_given_by_the_caller_and_the_largest_shapes():
    kd = _k(32, 1, 65536, 128, 6)          # 8 MiB of the 16 MiB scratch
    sh = A.AttnShape(32, 1, 1, 65536, 128)
    assert A.quantize_workspace_bytes(sh) <= _native.ATTN_NOALLOC_SCRATCH_BYTES
    case("quantize_k_noalloc 32 x 65536 tokens, caller outputs")
    out = {"k_i8": torch.full(kd.shape, 77, dtype=torch.int8, device="cuda"),
           "k_scale": torch.full((32, 1, 1024), -1.0, dtype=torch.float32, device="cuda"),
           "k_mean": torch.full((32, 1, 128), -1.0, dtype=torch.float32, device="cuda")}
    got = A.quantize_k_noalloc(kd, out=out)
    ref = A.quantize_k(kd)
    torch.cuda.synchronize()
    for key in ("k_i8", "k_scale", "k_mean"):
        assert got[key] is out[key] and torch.equal(got[key], ref[key]), key
    del kd, got, ref, out
    case("quantize_k_noalloc after the largest call: a small one")
    _same(_k(1, 2, 64, 64, 7))


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    kd = torch.zeros((64, 1, 65536, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(A.AttnError, match="scratch"):
        A.quantize_k_noalloc(kd)
