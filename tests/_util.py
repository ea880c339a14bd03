"""Shared helpers of the GPU parity tests (no arithmetic of the method)."""
import numpy as np
import torch

# Parity bar for attention outputs against the fp64 oracle.
REL_L2_TOL = 5e-3
MAX_ABS_TOL = 2e-2


def to_dev(bits, device="cuda:0"):
    """uint16 bf16 bit patterns (numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def from_dev_bf16(t):
    """bf16 GPU tensor -> float64 numpy (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


def attn_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    return rel, float(np.abs(got - ref).max())


def assert_attn_close(got, ref, what=""):
    rel, mx = attn_err(got, ref)
    print(f"[parity] {what}: rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert np.isfinite(got).all(), what
    assert rel <= REL_L2_TOL and mx <= MAX_ABS_TOL, (what, rel, mx)
