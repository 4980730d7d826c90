"""GPU checks of the measurement probes the benchmark reports beside the
published peaks (libattn_probe.so, not part of the attention path): the
streaming read visits every 16-byte chunk of its buffer exactly once, in the
per-thread order its header states, so the bandwidth it reports counts bytes
that were really read."""
import ctypes

import numpy as np
import pytest
import torch

from _util import case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunks,blocks", [(1, 1), (4096, 2), (4096 * 3 + 17, 3), (512 * 4 * 5 + 511, 2)])
def test_hbm_read_visits_every_chunk_once(chunks, blocks):
    from bit_quantized_exact_amd import probe
    L = probe.lib()
    case(f"hbm_read probe chunks={chunks} blocks={blocks}")
    rng = np.random.default_rng(chunks + blocks)
    words = rng.integers(-(1 << 31), 1 << 31, size=(chunks, 4), dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(words.reshape(-1)).cuda()
    T = blocks * 256
    sink = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    assert L.attn_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), chunks * 16, blocks,
                                 ctypes.c_void_p(sink.data_ptr()), None) == 0
    torch.cuda.synchronize()
    # thread t reads chunks t, t + T, t + 2T, ...: the XOR of their four words
    per_chunk = np.bitwise_xor.reduce(words, axis=1)
    want = np.zeros(T, dtype=np.int32)
    for t in range(min(T, chunks)):
        want[t] = np.bitwise_xor.reduce(per_chunk[t::T])
    np.testing.assert_array_equal(sink.cpu().numpy(), want.astype(np.float32))
