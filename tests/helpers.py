"""Shared helpers of the GPU tests: device upload and error metrics."""
import numpy as np


def to_device(inp, device="cuda"):
    import torch
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32

    def f(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device).to(dt)

    return dict(q=f(inp.q), k=f(inp.k), v=f(inp.v), beta=f(inp.beta), z=f(inp.z),
                a=torch.from_numpy(np.ascontiguousarray(inp.a)).to(device))


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_max_err(x, ref):
    """max |x - ref| / rms(ref) over the whole tensor."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(x - ref)) / rms) if rms > 0 else float(np.max(np.abs(x)))


TOL = {"bf16": 2e-2, "f32": 1e-4}
