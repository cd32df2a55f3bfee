"""Helpers shared by the GPU parity tests: moving seeded bf16 bit patterns to the device
and back, the tolerance measures, and one-call wrappers around the library binding."""
import numpy as np
import torch

from synth import bits_to_f64

# Tolerances for floating-point results (bf16 inputs and outputs, fp32 accumulation).
O_MAX_ABS = 2e-2        # forward output and decode output, max |gpu - oracle| over valid rows
GRAD_REL_L2 = 5e-2      # dQ, dK, dV: ||gpu - oracle||_2 / ||oracle||_2 over valid rows
LSE_MAX_ABS = 1e-2      # row log-sum-exp (fp32 output)


TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}


def dev(bits: np.ndarray, dtype: str = "bf16") -> torch.Tensor:
    """uint16 bit patterns of a 16-bit type -> tensor of that type on cuda:0 (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda:0").view(TORCH16[dtype])


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp16 / fp32 device tensor -> float64 numpy (exact)."""
    if t.dtype == torch.bfloat16:
        return bits_to_f64(host_bits(t), "bf16")
    if t.dtype == torch.float16:
        return bits_to_f64(host_bits(t), "f16")
    return t.detach().cpu().double().numpy()


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def rel_l2(a, b) -> float:
    a, b = np.asarray(a), np.asarray(b)
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / den if den > 0 else float(np.linalg.norm(a))


def first_nonfinite(*ts):
    """(argument position, flat index, value) of the first non-finite element, or None."""
    for n, t in enumerate(ts):
        a = t.detach().float().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, dtype=np.float64)
        bad = np.flatnonzero(~np.isfinite(a))
        if bad.size:
            return n, int(bad[0]), float(a.reshape(-1)[bad[0]])
    return None


def all_finite(*ts) -> bool:
    """Every element of every tensor is finite; otherwise prints where the first one is not."""
    nf = first_nonfinite(*ts)
    if nf is not None:
        print(f"first non-finite: tensor #{nf[0]} flat index {nf[1]} value {nf[2]}", flush=True)
    return nf is None
