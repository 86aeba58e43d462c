"""Error metric and tolerances shared by the GPU parity tests.

rel_err(x, ref) = max_i |x_i - ref_i| / max(|ref_i|, rms(ref)): an elementwise
relative error, floored at the RMS of the reference so that outputs near zero
(cancellation) do not make it ill-posed.  Tolerances: 1e-4 for fp32 inputs and
5e-3 for bf16 inputs with fp32 state and accumulation.
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 5e-3}


def rel_err(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    denom = np.maximum(np.abs(ref), rms if rms > 0 else 1e-300)
    return float(np.max(np.abs(x - ref) / denom))


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
