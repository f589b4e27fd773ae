"""Helpers for the GPU tests: move synth/ arrays to the device and back (no attention math)."""
import numpy as np

BF16_TOL = 2e-2  # max-abs vs the fp64 oracle for bf16 outputs
F32_TOL = 1e-4   # max-abs vs the fp64 oracle for fp32 outputs


def torch():
    import torch as t
    return t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).cuda()


def dev(arr: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(arr)).cuda()


def host_f64(x) -> np.ndarray:
    t = torch()
    return x.detach().to(t.float32).cpu().numpy().astype(np.float64)


def host_bits(x) -> np.ndarray:
    t = torch()
    return x.detach().cpu().view(t.int16).numpy().view(np.uint16)


def maxabs(a, b) -> float:
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    assert np.isfinite(d).all(), "non-finite values"
    return float(d.max()) if d.size else 0.0
