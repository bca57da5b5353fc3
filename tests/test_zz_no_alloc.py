"""svq_linear_noalloc (library-held scratch, no workspace argument) against
svq_linear on the same inputs: bit-identical outputs, and within the stated
tolerance of the CPU oracle.  Calls go through the C ABI, two or more in a
row on one GPU, later calls with smaller inputs than earlier ones (the
scratch keeps the previous call's contents)."""
import numpy as np
import pytest

import synth
from oracle import svq_oracle as so
from tests.gpu_common import assert_within_tolerance, out_to_f64, require_gpu, to_device_bf16, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svq():
    return require_gpu()


def _pair(svq, mat, m, seed, out_dtype):
    pm = svq.pack(mat)
    x_bits = synth.random_activations(m, mat.k, seed=seed)
    x = to_device_bf16(x_bits)
    y_ref = svq.linear(pm, x, out_dtype=out_dtype)
    y = torch.full((m, mat.n), float("nan"), dtype=out_dtype, device="cuda")
    svq.linear_noalloc(pm, x, y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16) if out_dtype == torch.bfloat16 else y.view(torch.int32),
                       y_ref.view(torch.int16) if out_dtype == torch.bfloat16 else y_ref.view(torch.int32)), \
        f"noalloc differs from svq_linear (n={mat.n} k={mat.k} m={m})"
    y64, W = so.linear_from_inputs(mat, x_bits)
    assert_within_tolerance(out_to_f64(y), y64, x_bits, W, label=f"noalloc n={mat.n} k={mat.k} m={m}")


# (n, k, bd, m): each path that takes scratch, largest first, then smaller
SEQUENCE = [
    (2560, 9728, 7, 16),  # small-batch path with K ranges (partials, arrival counters)
    (1024, 2560, 8, 16),  # the same path, fewer units, no K ranges
    (300, 2560, 6, 300),  # dequant-GEMM (prefill kernel)
    (200, 1032, 8, 40),   # dequant-GEMM with K splits (partials + reduce launch)
    (1024, 2560, 7, 4),   # exact path, gathered activations in scratch
    (48, 640, 6, 3),      # the same path, smaller
    (512, 1024, 8, 1),    # m = 1: no scratch used
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_linear_in_sequence(svq, out_dtype):
    for i, (n, k, bd, m) in enumerate(SEQUENCE):
        mat = synth.random_matrix(n, k, bd, seed=(60, n, k))
        _pair(svq, mat, m, (61, i, m), out_dtype)


def test_noalloc_repeated_call_smaller_second(svq):
    """The same matrix twice, the second call with fewer rows: nothing of the
    first call's scratch leaks into the second."""
    mat = synth.random_matrix(2560, 9728, 8, seed=(62, 0, 0))
    _pair(svq, mat, 16, (63, 0, 16), torch.float32)
    _pair(svq, mat, 7, (63, 1, 7), torch.float32)


def test_noalloc_rejects_oversized_call(svq):
    mat = synth.random_matrix(64, 9728, 7, seed=(64, 0, 0))
    pm = svq.pack(mat)
    m = 4096  # fragment-ordered activations alone exceed the scratch
    x = torch.zeros((m, mat.k), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((m, mat.n), dtype=torch.float32, device="cuda")
    st = svq.svq_linear_noalloc(pm.handle, x.data_ptr(), m, x.stride(0), y.data_ptr(), y.stride(0),
                                svq.SVQ_F32, 0)
    assert st == svq.SVQ_ERR_UNSUPPORTED
