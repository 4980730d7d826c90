"""GPU check that the INT8 path (the allocation-free K quantiser, then the
forward that quantises Q itself) and the FP16 forward can be captured into a
HIP graph and replayed: the outputs are allocated once outside the graph, new
inputs are copied into the captured buffers before each replay, the eager
reference runs between the replays, and every replay must equal the eager
calls on the same inputs bit for bit.  (The library issues no memsets and
allocates nothing inside these calls; the scratch of the allocation-free
quantiser is looked up before the capture, by its first call.)"""
import pytest
import torch

import bit_quantized_exact_amd as A
from bit_quantized_exact_amd.inputs import make_qkv

from _util import case, small_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,D,causal", [(1000, 128, True), (300, 64, False), (4096, 128, True)])
def test_int8_and_fp16_paths_replay_in_a_graph(S, D, causal):
    ws = [small_workload(1, 4, 2, S, D, causal, seed=9000 + 17 * r + S) for r in range(3)]
    inputs = [tuple(torch.from_numpy(x).cuda() for x in make_qkv(w)) for w in ws]
    qd, kd, vd = (x.clone() for x in inputs[0])          # the buffers the graph reads
    kz = A.quantize_k_noalloc(kd)                          # outputs, allocated once
    o8 = torch.empty_like(qd)
    o16 = torch.empty_like(qd)
    lse8 = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    lse16 = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")

    def path():
        A.quantize_k_noalloc(kd, out=kz)
        A.fwd_int8_fused_q(qd, kz, vd, causal=causal, out=o8, lse=lse8)
        A.fwd_fp16(qd, kd, vd, causal=causal, out=o16, lse=lse16)

    # a warm-up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    case(f"graph capture S={S} D={D} causal={causal}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()

    for r, (q, k, v) in enumerate(inputs + inputs[:1]):
        qd.copy_(q)
        kd.copy_(k)
        vd.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        ref_kz = A.quantize_k(k)
        ref8, ref_l8 = A.fwd_int8_fused_q(q, ref_kz, v, causal=causal, return_lse=True)
        ref16, ref_l16 = A.fwd_fp16(q, k, v, causal=causal, return_lse=True)
        torch.cuda.synchronize()
        for key in ("k_i8", "k_scale", "k_mean"):
            assert torch.equal(kz[key], ref_kz[key]), (r, key)
        assert torch.equal(o8, ref8) and torch.equal(lse8, ref_l8), r
        assert torch.equal(o16, ref16) and torch.equal(lse16, ref_l16), r
