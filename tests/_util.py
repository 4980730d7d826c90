"""Helpers shared by the GPU tests (no attention arithmetic here)."""
import sys

import numpy as np
import torch

from bit_quantized_exact_amd.inputs import Workload, make_qkv

# Tolerances (stated where the forward paths are specified):
FP16_MAX_ABS = 2e-3      # FP16 path vs the fp64 oracle
INT8_COS_MIN = 0.999     # INT8 path vs the fp64 oracle (exact attention)
INT8_REL_L1_MAX = 0.02
INT8_VS_MODEL_MAX_ABS = 2e-3   # INT8 path vs the oracle's quantised-attention model


def case(msg: str):
    """Name the case on stdout before any GPU work, so a crash identifies it."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def cos_rel_l1(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    rel = float(np.abs(a - b).sum() / np.abs(b).sum())
    return cos, rel


def small_workload(B, Hq, Hkv, S, D, causal, seed, offset_std=2.0):
    return Workload(f"small_{B}x{Hq}x{Hkv}x{S}x{D}{'c' if causal else ''}", B, Hq, Hkv, S, D,
                    causal, offset_std, seed=seed)


def inputs(w: Workload):
    q, k, v = make_qkv(w)
    return q, k, v
