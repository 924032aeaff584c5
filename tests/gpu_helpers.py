"""Shared helpers for the GPU parity tests (inputs from workloads/, expectations from oracle/)."""
import numpy as np
import torch

# Tolerances (max-abs for O and LSE, relative L2 for gradients) on unit-normal bf16 inputs.
TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def dev():
    return torch.device("cuda:0")


def max_err(a, ref):
    a = f64(a) if isinstance(a, torch.Tensor) else np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(ref) & (np.sign(a) == np.sign(ref))
    d = np.where(both_inf, 0.0, np.abs(a - ref))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def rel_l2(a, ref):
    a = f64(a) if isinstance(a, torch.Tensor) else np.asarray(a, dtype=np.float64)
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))


def rne_bf16(x_f32):
    """Round an fp32 tensor to bf16 on the CPU (round to nearest even), as float64."""
    return f64(x_f32.detach().cpu().to(torch.bfloat16))


def log(msg):
    print(msg, flush=True)
