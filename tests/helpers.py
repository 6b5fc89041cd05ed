"""Shared helpers for the GPU tests: device transfer of the seeded inputs and the error metric.

The error metric for every parity check is max|gpu - ref| / max|ref| over the whole tensor.
"""
import numpy as np

TOL_F32 = 1e-5   # fp32 inputs and outputs
TOL_BF16 = 2e-2  # bf16 inputs, fp32 accumulation, bf16 outputs


def tol(dtype: str) -> float:
    return TOL_F32 if dtype == "f32" else TOL_BF16


def to_dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t  # values are already bf16-representable: exact
    return t.cuda()


def empty_out(shape, dtype: str):
    import torch
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / (scale if scale > 0 else 1.0)


def rel_err_per_head(got: np.ndarray, ref: np.ndarray, head_axis: int = 2) -> list:
    """The same metric per head ([B, N, H, d] tensors: axis 2), for the logs of the full-size checks."""
    out = []
    for h in range(ref.shape[head_axis]):
        r = np.take(ref, h, axis=head_axis)
        g = np.take(got, h, axis=head_axis)
        out.append(rel_err(g, r))
    return out
