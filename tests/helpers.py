"""Shared test helpers: host <-> device marshalling and error measures."""
import numpy as np


def to_device(a: np.ndarray, device="cuda"):
    """numpy -> torch on the GPU; uint16 arrays are bfloat16 bit patterns."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t) -> np.ndarray:
    """torch -> numpy; bfloat16 comes back as uint16 bit patterns."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_l2(got, ref) -> float:
    got = as_f64(np.asarray(got))
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)


# tolerances of the outputs against the oracle: relative L2 over the compared tensor
TOL = {"f32": 1e-5, "bf16": 2e-2}
