"""Small helpers shared by the tests (bit views and tolerance reports)."""

import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor on the CPU."""
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


def widen(b: np.ndarray, dtype=np.float64) -> np.ndarray:
    u = np.asarray(b).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(dtype)


def close_report(got: np.ndarray, ref: np.ndarray, atol=1e-2, rtol=1e-2):
    """allclose in the per-element form |got-ref| <= atol + rtol*|ref|,
    plus max-abs, max-rel (over |ref| >= 1e-3) and relative L2."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    ok = bool(np.all(diff <= atol + rtol * np.abs(ref)))
    big = np.abs(ref) >= 1e-3
    max_rel = float((diff[big] / np.abs(ref[big])).max()) if np.any(big) else 0.0
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    return ok, float(diff.max()) if diff.size else 0.0, max_rel, rel_l2
