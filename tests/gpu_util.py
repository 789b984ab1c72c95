"""Helpers shared by the GPU parity tests: host <-> device marshalling and the
output tolerance.

Tolerance for fp32-accumulated outputs against the unrounded fp64 oracle,
per linear over all M x N outputs:
    ||y - y_ref||_2 / ||y_ref||_2 <= 1e-3   and   max |y - y_ref| <= 4e-3 * RMS(y_ref).
The budget: fp16 rounding of the rotated activations (relative 2^-12 RMS per
element, about 2e-4 on the output), fp16 rounding of the output (at most
2^-11 of |y|), fp32 accumulation (about 1e-6).
"""

import sys

import numpy as np
import torch

REL_L2 = 1e-3
MAX_ABS_RMS = 4e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_u32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def host_f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def check_close(y_gpu, y_ref, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    d = y - r
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(d) / nr if nr > 0 else np.linalg.norm(d)
    rms = np.sqrt(np.mean(r * r))
    mx = np.abs(d).max()
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS_RMS * rms + 1e-30, f"{what}: max-abs {mx:.3e} > {MAX_ABS_RMS} * rms {rms:.3e}"
    return rel, mx / rms if rms > 0 else 0.0
