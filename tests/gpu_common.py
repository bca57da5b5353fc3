"""Shared helpers for the GPU parity tests (libsvq vs the CPU oracle)."""
import numpy as np
import pytest

from oracle import svq_oracle as so

torch = pytest.importorskip("torch")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_spherical_vector_amd import svq  # raises if libsvq.so is missing
    return svq


def to_device_bf16(bits: np.ndarray):
    """uint16 bf16 bit patterns [m, k] -> CUDA bf16 tensor (bit exact)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def out_to_f64(y) -> np.ndarray:
    if y.dtype == torch.bfloat16:
        return so.bf16_bits_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))
    return y.double().cpu().numpy()


def assert_within_tolerance(y_gpu: np.ndarray, y64: np.ndarray, x_bits: np.ndarray, W: np.ndarray,
                            rel: float = 8e-3, label: str = ""):
    """|y - y_ref| <= rel * sum_j |W_ij||x_mj| + 1e-6, element by element."""
    bound = so.tolerance(x_bits, W, rel=rel)
    err = np.abs(y_gpu - y64)
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        worst = float(np.max(err / bound))
        raise AssertionError(f"{label}: {int(bad.sum())} of {bad.size} outside tolerance "
                             f"(worst ratio {worst:.3g}); first at {idx.tolist()}")
    return float(np.max(err / bound)) if err.size else 0.0


def equal_pm0(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Elementwise bit equality of float values, +0 == -0."""
    return (a == b) | ((a == 0) & (b == 0))


def one_hot_bits(k: int, cols) -> np.ndarray:
    x = np.zeros((len(cols), k), dtype=np.uint16)
    for r, j in enumerate(cols):
        x[r, j] = 0x3F80  # bf16 1.0
    return x
