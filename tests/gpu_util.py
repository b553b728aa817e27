"""Helpers for the GPU parity tests: device upload of the generators' values,
tolerance checks against the oracle, and a progress line per case."""
import sys

import numpy as np

import workloads as W

# Tolerances fixed for this path: bf16 inputs with fp32 accumulation, and fp32.
BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 5e-3
F32_TOL = 1e-4


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str, device="cuda"):
    """Upload generator values (fp32 numpy holding exact bf16 values for 'bf16')."""
    import torch
    if dtype == "bf16":
        bits = W.bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t) -> np.ndarray:
    """Device tensor -> float64 numpy (exact up-cast)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str = "", max_abs=None, rel_l2=None):
    ma, rl = errors(got, ref)
    if dtype == "bf16":
        max_abs = BF16_MAX_ABS if max_abs is None else max_abs
        rel_l2 = BF16_REL_L2 if rel_l2 is None else rel_l2
    else:
        max_abs = F32_TOL if max_abs is None else max_abs
        rel_l2 = F32_TOL if rel_l2 is None else rel_l2
    say(f"{what}: max-abs {ma:.3e} (<= {max_abs:g}), rel-L2 {rl:.3e} (<= {rel_l2:g})")
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max-abs {ma:.3e}, rel-L2 {rl:.3e}"
    return ma, rl
