"""Shared helpers for the GPU parity tests: moving the seeded inputs to the
device and comparing with the oracle at the stated tolerances."""
import numpy as np

# Parity bar: fp32 max |err| <= 1e-5; bf16 max |err| <= 2e-2 and mean |err| <= 1e-3.
TOL = {"f32": (1e-5, None), "bf16": (2e-2, 1e-3)}


def to_device(stored, dtype, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).to(device)


def to_host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def errors(got, ref):
    diff = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(diff.max()) if diff.size else 0.0, float(diff.mean()) if diff.size else 0.0


def assert_close(name, got, ref, dtype, tol=None, scaled=False):
    """Max and mean absolute error within the bar. With `scaled`, an element
    whose reference exceeds 1 in magnitude is held to the max bar times that
    magnitude (the output dtype's own rounding grows with it: a bf16 value of
    magnitude 32 is only stored to within 0.125)."""
    max_tol, mean_tol = tol if tol is not None else TOL[dtype]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    mx, mean = errors(got, ref)
    if scaled:
        diff = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
        bound = max_tol * np.maximum(1.0, np.abs(np.asarray(ref, np.float64)))
        worst = float(np.max(diff / bound)) if diff.size else 0.0
        msg = f"{name}: max|err|/bound={worst:.3f} (max|err|={mx:.3e}), mean|err|={mean:.3e}"
        assert worst <= 1.0, msg
        if mean_tol is not None:
            assert mean <= mean_tol, msg
        return mx, mean
    msg = f"{name}: max|err|={mx:.3e} (tol {max_tol}), mean|err|={mean:.3e}"
    assert mx <= max_tol, msg
    if mean_tol is not None:
        assert mean <= mean_tol, msg
    return mx, mean


def device_inputs(inputs, dtype):
    """dict of (stored, values) -> (dict of device tensors, dict of float64 values)."""
    dev = {k: to_device(v[0], dtype) for k, v in inputs.items()}
    val = {k: v[1].astype(np.float64) for k, v in inputs.items()}
    return dev, val
