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


def row_rel_l2(got, ref) -> np.ndarray:
    """Relative L2 error of every row on its own (rows whose reference is all
    zero report their absolute norm)."""
    got = as_f64(np.asarray(got))
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


# (label, whole-tensor rel-L2, worst row rel-L2, worst row, rows) of every
# labelled check in this session, printed at the end of the run
PARITY_LOG = []


def check_outputs(got, ref, tol, label=""):
    """Whole-tensor relative L2 within tol AND every row within tol on its
    own: a single wrong or unwritten row (which adds only about 1/sqrt(rows)
    to the whole-tensor norm) fails the second test.  Returns (whole, worst
    row error, index of the worst row)."""
    whole = rel_l2(got, ref)
    rows = row_rel_l2(got, ref)
    worst = int(np.argmax(rows)) if rows.size else -1
    w = float(rows[worst]) if rows.size else 0.0
    if label:
        print(f"  {label}: out rel_l2={whole:.3e}, worst row {worst} rel_l2={w:.3e} over {rows.size} rows",
              flush=True)
        PARITY_LOG.append((label, whole, w, worst, int(rows.size), tol))
    assert not np.any(np.isnan(as_f64(np.asarray(got)))), f"{label}: NaN in the output"
    assert whole <= tol, f"{label}: whole-tensor rel_l2 {whole:.3e} > {tol}"
    assert w <= tol, f"{label}: row {worst} rel_l2 {w:.3e} > {tol}"
    return whole, w, worst


def workloads_bf16(a) -> np.ndarray:
    """float64 -> bf16 bit patterns (round to nearest even), for tests of the checks."""
    import workloads
    return workloads.bf16_bits(np.asarray(a, dtype=np.float32))
