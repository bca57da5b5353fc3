"""GPU parity of svq_linear against the CPU oracle (dense matrices).

Bar: decoded weights bit-exact (observed through one-hot activations), every
output within |y - y_ref| <= 8e-3 * sum_j |W_ij||x_j| + 1e-6.  The m <= 16
paths decode exactly in fp32 (one-hot columns reproduce the oracle's W bit
for bit) and are also held to a bound 8x tighter; the m > 16 dequant GEMM's
weights are RNE_bf16 of the exact products and are compared bit-exactly
with the oracle's rounding of them.
"""
import numpy as np
import pytest

import synth
from oracle import svq_oracle as so
from tests.gpu_common import (assert_within_tolerance, equal_pm0, one_hot_bits, out_to_f64,
                              require_gpu, to_device_bf16, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svq():
    return require_gpu()


def _run(svq, pm, x_bits, out_dtype, ldx_pad=0, ldy_pad=0):
    m, k = x_bits.shape
    xp = np.zeros((m, k + ldx_pad), dtype=np.uint16)
    xp[:, :k] = x_bits
    x = to_device_bf16(xp)[:, :k]
    if ldy_pad:
        out = torch.full((m, pm.n + ldy_pad), float("nan"), dtype=out_dtype, device="cuda")
        y = svq.linear(pm, x, out=out[:, :pm.n])
        torch.cuda.synchronize()
        assert torch.isnan(out[:, pm.n:]).all(), "write outside the output rows"
    else:
        y = svq.linear(pm, x, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out_to_f64(y)


def _check_outputs(svq, mat, x_bits, label):
    pm = svq.pack(mat)
    y64, W = so.linear_from_inputs(mat, x_bits)
    m = x_bits.shape[0]
    for dt in (torch.float32, torch.bfloat16):
        y = _run(svq, pm, x_bits, dt)
        assert_within_tolerance(y, y64, x_bits, W, label=f"{label} {dt}")
        if dt == torch.float32 and m <= 16:
            assert_within_tolerance(y, y64, x_bits, W, rel=1e-3, label=f"{label} exact-path")
    return pm, W


def _one_hot_check(svq, pm, W, cols, batch):
    """Decoded weights through one-hot activations, fp32 output."""
    k = W.shape[1]
    for s in range(0, len(cols), batch):
        cs = cols[s:s + batch]
        y = _run(svq, pm, one_hot_bits(k, cs), torch.float32)
        for r, j in enumerate(cs):
            ref = W[:, j] if len(cs) <= 16 else so.round_to_bf16(W[:, j])
            ok = equal_pm0(y[r], ref)
            assert ok.all(), f"column {j}: {int((~ok).sum())} decoded weights differ"


def test_single_matrix_m1(svq):
    mat, x = synth.single_matrix()
    pm, W = _check_outputs(svq, mat, x, "512x1024 m=1")
    # every decoded weight, 4 columns per call through the exact path
    _one_hot_check(svq, pm, W, list(range(mat.k)), 4)
    # and a few through m = 1 itself
    _one_hot_check(svq, pm, W, [0, 1, 511, 1023], 1)


@pytest.mark.parametrize("j", range(7))
def test_dense_layer_m1(svq, j):
    mats, xs = synth.dense_layer()
    mat, x = mats[j], xs[j]
    pm, W = _check_outputs(svq, mat, x, f"layer {mat.name} m=1")
    rng = np.random.default_rng(100 + j)
    cols = sorted(rng.choice(mat.k, 256, replace=False).tolist())
    _one_hot_check(svq, pm, W, cols, 4)
    # and 24 of them through m = 1 itself (its own kernel body)
    _one_hot_check(svq, pm, W, cols[::11], 1)


@pytest.mark.parametrize("m", [4, 16])
@pytest.mark.parametrize("j", range(7))
def test_dense_layer_small_batch(svq, j, m):
    mats, _ = synth.dense_layer()
    mat = mats[j]
    x = synth.dense_layer_activations(m)[j]
    pm, W = _check_outputs(svq, mat, x, f"layer {mat.name} m={m}")
    # decoded weights, exactly, through the m = 16 path (and m = 4 below)
    rng = np.random.default_rng(200 + j)
    cols = sorted(rng.choice(mat.k, 256, replace=False).tolist())
    _one_hot_check(svq, pm, W, cols, m)


@pytest.mark.parametrize("j", range(3))
def test_prefill_m2048(svq, j):
    """All 2048 rows of each prefill matrix against the oracle."""
    mats, xs = synth.prefill_set()
    mat, x = mats[j], xs[j]
    pm = svq.pack(mat)
    W = so.decode_matrix(mat.codes, mat.n, mat.k, mat.bd, mat.codebook, mat.radius, mat.perm)
    y64 = so.linear(x, W)
    for dt in (torch.bfloat16, torch.float32):
        y = _run(svq, pm, x, dt)
        assert y.shape == (2048, mat.n)
        assert_within_tolerance(y, y64, x, W, label=f"prefill {mat.name} {dt}")


EDGE = [
    # n, k, bd, m
    (1, 8, 8, 1),
    (1, 8, 6, 5),
    (37, 104, 6, 3),
    (16, 512, 7, 4),
    (33, 1032, 8, 17),
    (100, 104, 7, 16),
    (2048, 768, 7, 1),
    (2048, 768, 7, 2),
    (17, 520, 6, 64),
    (15, 2048, 8, 65),
    (64, 4096, 6, 1),
    # m = 1 with a row too long for the fused launch's LDS: the two-launch path
    (20, 53248, 8, 1),
    (20, 53248, 7, 3),
]


@pytest.mark.parametrize("n,k,bd,m", EDGE)
def test_edge_shapes(svq, n, k, bd, m):
    mat = synth.random_matrix(n, k, bd, seed=(30, n, k))
    x = synth.random_activations(m, k, seed=(30, m, k))
    pm, W = _check_outputs(svq, mat, x, f"edge n={n} k={k} bd={bd} m={m}")
    cols = sorted(set([0, k - 1] + list(range(0, k, max(1, k // 8)))))
    _one_hot_check(svq, pm, W, cols, 4 if m <= 4 else 16)


SMALL_EDGE = [
    # n, k, bd, m on the 4 < m <= 16 path: 1..19 units (more than 8: K
    # ranges, the last one shorter), blocks of 1..4 row tiles with a partial
    # last group, ragged rows and slots
    (16, 512, 8, 5),
    (40, 1000, 6, 16),
    (70, 1536, 7, 12),
    (64, 2048, 8, 8),
    (100, 2560, 6, 16),
    (260, 3000, 6, 16),
    (33, 3584, 8, 13),
    (130, 4600, 7, 9),
    (50, 5600, 6, 16),
    (70, 9728, 8, 7),
]


@pytest.mark.parametrize("n,k,bd,m", SMALL_EDGE)
def test_small_batch_path_edges(svq, n, k, bd, m):
    mat = synth.random_matrix(n, k, bd, seed=(38, n, k))
    x = synth.random_activations(m, k, seed=(38, m, k))
    pm, W = _check_outputs(svq, mat, x, f"small edge n={n} k={k} bd={bd} m={m}")
    assert pm.handle.xscale_log2 != svq.SVQ_NO_EXACT_SPLIT
    cols = sorted(set([0, k - 1] + list(range(0, k, max(1, k // 30)))))
    _one_hot_check(svq, pm, W, cols, m)


@pytest.mark.parametrize("m", [5, 8, 16])
def test_small_batch_without_exact_split(svq, m):
    """Tables whose products span more binades than two fp16 halves hold
    (a radius of 60000 next to a direction entry of 2^-24) take the m <= 4
    kernels four rows at a time: still exact."""
    n, k, bd = 70, 1536, 7
    mat = synth.random_matrix(n, k, bd, seed=(39, n, k))
    rad = mat.radius.copy()
    rad[0], rad[1] = 0x3C01, 0x7B53
    mat.radius = rad
    cb = mat.codebook.copy()
    cb[0, :] = 0x0001
    mat.codebook = cb
    x = synth.random_activations(m, k, seed=(39, m, k))
    pm, W = _check_outputs(svq, mat, x, f"no split m={m}")
    assert pm.handle.xscale_log2 == svq.SVQ_NO_EXACT_SPLIT
    cols = sorted(set([0, k - 1] + list(range(0, k, 97))))
    _one_hot_check(svq, pm, W, cols, m)


PREFILL_EDGE = [
    # n, k, bd, m: ragged row tiles, a partial last unit, m not a multiple of 256
    (200, 1032, 8, 300),
    (129, 520, 6, 256),
    (16, 8, 7, 257),
    (300, 2560, 7, 511),
]


@pytest.mark.parametrize("n,k,bd,m", PREFILL_EDGE)
def test_prefill_path_edges(svq, n, k, bd, m):
    """m >= 256 takes the LDS-tiled prefill kernel; its decoded weights are
    observed through 256 one-hot rows (one block of activation rows)."""
    mat = synth.random_matrix(n, k, bd, seed=(37, n, k))
    x = synth.random_activations(m, k, seed=(37, m, k))
    pm, W = _check_outputs(svq, mat, x, f"prefill edge n={n} k={k} bd={bd} m={m}")
    cols = [(j * k) // 256 for j in range(256)]
    _one_hot_check(svq, pm, W, cols, 256)


@pytest.mark.parametrize("m", [1, 3, 20])
def test_strided_input_output(svq, m):
    mat = synth.random_matrix(48, 640, 7, seed=(31, m, 0))
    x = synth.random_activations(m, 640, seed=(31, m, 1))
    pm = svq.pack(mat)
    y64, W = so.linear_from_inputs(mat, x)
    y = _run(svq, pm, x, torch.float32, ldx_pad=24, ldy_pad=8)
    assert_within_tolerance(y, y64, x, W, label="strided")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_prefill_full_tiles_strided(svq, dt):
    """The 256-row tile's full output tiles store straight from the
    accumulators: 512 tokens x 512 rows is four full tiles, written through
    a row stride wider than n (padding columns must stay untouched)."""
    mat = synth.random_matrix(512, 1024, 7, seed=(36, 0, 0))
    x = synth.random_activations(512, 1024, seed=(36, 0, 1))
    pm = svq.pack(mat)
    y64, W = so.linear_from_inputs(mat, x)
    y = _run(svq, pm, x, dt, ldx_pad=8, ldy_pad=24)
    assert_within_tolerance(y, y64, x, W, label=f"prefill full tiles, strided {dt}")


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_unaligned_activations(svq, m):
    """Rows that do not start 16-byte aligned (odd row stride, base pointer
    two bytes into the buffer) take the scalar staging path."""
    k = 640
    mat = synth.random_matrix(48, k, 7, seed=(36, m, 0))
    x = synth.random_activations(m, k, seed=(36, m, 1))
    pm = svq.pack(mat)
    y64, W = so.linear_from_inputs(mat, x)
    buf = np.zeros((m, k + 3), dtype=np.uint16)
    buf[:, 1:k + 1] = x
    xd = to_device_bf16(buf)[:, 1:k + 1]
    assert (xd.data_ptr() % 16) != 0 and (xd.stride(0) * 2) % 16 != 0
    y = svq.linear(pm, xd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_within_tolerance(out_to_f64(y), y64, x, W, label=f"unaligned m={m}")


def test_deterministic(svq):
    mat = synth.random_matrix(256, 2560, 8, seed=(32, 0, 0))
    for m in (1, 4, 16, 33):
        x = synth.random_activations(m, 2560, seed=(32, m, 0))
        pm = svq.pack(mat)
        a = _run(svq, pm, x, torch.float32)
        b = _run(svq, pm, x, torch.float32)
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


def test_zero_and_extreme_activations(svq):
    mat = synth.random_matrix(64, 1024, 8, seed=(33, 0, 0))
    pm = svq.pack(mat)
    W = so.decode_matrix(mat.codes, mat.n, mat.k, mat.bd, mat.codebook, mat.radius, mat.perm)
    zero = np.zeros((2, 1024), dtype=np.uint16)
    assert np.all(_run(svq, pm, zero, torch.float32) == 0)
    assert np.all(_run(svq, pm, np.zeros((9, 1024), dtype=np.uint16), torch.float32) == 0)
    # very large and very small magnitudes in one row (fp16 range is far exceeded)
    rng = np.random.default_rng(5)
    for scale in (1e30, 1e-30):
        xf = (rng.standard_normal((3, 1024)) * scale).astype(np.float32)
        xf[0, :5] *= 1e3
        x = synth.bf16_bits_from_f32(xf)
        y64 = so.linear(x, W)
        for m_rows in (x[:1], x):
            y = _run(svq, pm, m_rows, torch.float32)
            assert_within_tolerance(y, y64[:m_rows.shape[0]], m_rows, W, label=f"scale {scale}")


def test_subnormal_codebook_entries_decode_exactly(svq):
    mat = synth.random_matrix(32, 512, 8, seed=(34, 0, 0))
    cb = mat.codebook.copy()
    cb[:, 3] = np.arange(cb.shape[0], dtype=np.uint16) % 0x3FF + 1  # fp16 subnormals
    cb[5, :] = 0x0001  # smallest subnormal
    mat.codebook = cb
    pm = svq.pack(mat)
    W = so.decode_matrix(mat.codes, mat.n, mat.k, mat.bd, mat.codebook, mat.radius, mat.perm)
    _one_hot_check(svq, pm, W, list(range(0, 512, 3)), 4)
    _one_hot_check(svq, pm, W, list(range(0, 512, 37)), 16)
    _one_hot_check(svq, pm, W, list(range(0, 512, 7)), 1)


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_batched_layer_call(svq, m):
    """All seven layer matrices through one svq_linear_batched call."""
    mats, xs1 = synth.dense_layer()
    xs = xs1 if m == 1 else [synth.random_activations(m, w.k, seed=(35, m, j))
                             for j, w in enumerate(mats)]
    pms = [svq.pack(w) for w in mats]
    xd = [to_device_bf16(x) for x in xs]
    outs = svq.linear_batched(pms, xd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for w, x, o in zip(mats, xs, outs):
        y64, W = so.linear_from_inputs(w, x)
        y = out_to_f64(o)
        assert_within_tolerance(y, y64, x, W, label=f"batched {w.name} m={m}")
        if m <= 4:
            assert_within_tolerance(y, y64, x, W, rel=1e-3, label=f"batched exact {w.name}")
