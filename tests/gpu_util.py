"""Helpers for the GPU parity tests (device transfer, tolerance checks)."""
import numpy as np
import torch


def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def check_tol(got, ref, bound, rel, what=""):
    """|got - ref| <= rel * bound + 1e-6 for every element, all finite.
    Returns max(|err| / tol)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    tol = rel * np.asarray(bound, dtype=np.float64) + 1e-6
    ratio = np.abs(got - ref) / tol
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, f"{what}: max |err|/tol = {worst:.3g} at {np.unravel_index(ratio.argmax(), ratio.shape)}"
    return worst


def guarded(n: int, dtype=torch.float32, guard: int = 64, fill=1234.5):
    """A device buffer of n elements with sentinel guard bands on both sides.
    Returns (full buffer, view of the n middle elements)."""
    full = torch.full((n + 2 * guard,), fill, dtype=dtype, device=dev())
    return full, full[guard:guard + n]


def guards_intact(full: torch.Tensor, n: int, guard: int = 64, fill=1234.5) -> bool:
    h = full.detach().cpu()
    return bool((h[:guard] == fill).all() and (h[guard + n:] == fill).all())
