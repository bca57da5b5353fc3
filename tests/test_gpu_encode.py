"""GPU parity of svq_encode against the CPU encoder oracle.

Bar: the canonical code stream is bit-exact (integer output; both sides
take every decision in the same float64 arithmetic, lane-order sums without
fused multiply-adds).  The coding rule is the reading of the SAGE paper's
Fig. 2 caption stated in include/svq.h.
"""
import numpy as np
import pytest

import synth
from oracle import svq_encoder as se
from oracle import svq_oracle as so
from tests.gpu_common import require_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svq():
    return require_gpu()


def _encode_gpu(svq, w: np.ndarray, perm, bd, cb, rad, ld_pad=0):
    n, k = w.shape
    buf = torch.zeros((n, k + ld_pad), dtype=torch.float32)
    buf[:, :k] = torch.from_numpy(w)
    wd = buf.cuda()[:, :k]
    codes = svq.encode(wd, perm, bd, cb, rad)
    torch.cuda.synchronize()
    return codes.cpu().numpy()


@pytest.mark.parametrize("bd", [6, 7, 8])
def test_round_trip_of_decoded_matrix(svq, bd):
    mat = synth.random_matrix(70, 520, bd, seed=(50, bd, 0))
    w = so.decode_matrix(mat.codes, mat.n, mat.k, mat.bd, mat.codebook, mat.radius,
                         mat.perm).astype(np.float32)
    got = _encode_gpu(svq, w, mat.perm, bd, mat.codebook, mat.radius)
    # the synthetic stream's bits past the last code are random; the codes
    # themselves must come back, and the encoder leaves those bits zero
    assert np.array_equal(so.unpack_codes(got, mat.n, mat.k), so.unpack_codes(mat.codes, mat.n, mat.k))
    assert np.array_equal(got, so.pack_codes(so.unpack_codes(mat.codes, mat.n, mat.k)))


SHAPES = [
    # n, k, bd, ld_pad: one code; partial last group of 4 codes (k/8 odd,
    # n*k/8 not a multiple of 4); strided rows; a larger matrix
    (1, 8, 8, 0),
    (3, 24, 6, 5),
    (17, 104, 7, 0),
    (64, 2560, 8, 3),
    (33, 1032, 6, 0),
]


@pytest.mark.parametrize("n,k,bd,ld_pad", SHAPES)
def test_random_weights_match_the_oracle(svq, n, k, bd, ld_pad):
    rng = np.random.default_rng(51 + n + k)
    mat = synth.random_matrix(n, k, bd, seed=(51, n, k))
    R = so.fp16_bits_to_f64(mat.radius)
    # norms across (and beyond) the radius table, exact zeros and -0.0
    w = (rng.standard_normal((n, k)) * rng.uniform(0.05, 3.0) * R[-1] / np.sqrt(8)).astype(np.float32)
    w[rng.random((n, k)) < 0.05] = 0.0
    w[rng.random((n, k)) < 0.05] = -0.0
    expect = se.encode_stream(w, mat.perm, bd, mat.codebook, mat.radius)
    got = _encode_gpu(svq, w, mat.perm, bd, mat.codebook, mat.radius, ld_pad)
    assert got.shape == expect.shape
    assert np.array_equal(got, expect), int((got != expect).sum())


def test_ties_and_zero_subvectors(svq):
    """Duplicated codebook rows (equal scores: the first index wins), an
    all-zero subvector (every score 0: index 0, radius index 0) and norms
    exactly on a radius midpoint (the lower radius wins)."""
    bd, k = 6, 64
    mat = synth.random_matrix(4, k, bd, seed=(52, 0, 0))
    cb = np.asarray(mat.codebook).copy().reshape(64, 8)
    cb[40] = cb[7]
    cb[63] = cb[7]
    R = so.fp16_bits_to_f64(mat.radius)
    w = np.zeros((4, k), dtype=np.float32)
    wp = np.zeros((4, k), dtype=np.float64)
    D = so.fp16_bits_to_f64(cb)
    for c in range(k // 8):
        wp[0, 8 * c:8 * c + 8] = D[7] * R[3]                 # duplicated row 7
        wp[2, 8 * c:8 * c + 8] = np.eye(8)[c] * (R[1] + R[2]) / 2  # norm on a midpoint
    wp[3, :8] = -D[7] * R[5]
    w[:, mat.perm] = wp.astype(np.float32)
    assert np.array_equal(w[:, mat.perm].astype(np.float64), wp)  # exact in float32
    codes_oracle = se.encode_matrix(w, mat.perm, bd, cb, mat.radius)
    s, d, r = so.split_fields(codes_oracle, bd)
    assert np.all(d[0] == 7) and np.all(d[1] == 0) and np.all(r[1] == 0) and np.all(r[2] == 1)
    got = _encode_gpu(svq, w, mat.perm, bd, cb, mat.radius)
    assert np.array_equal(got, se.encode_stream(w, mat.perm, bd, cb, mat.radius))


def test_full_size_matrix_sampled_rows(svq):
    """The 9728 x 2560 gate shape (bd = 7), every row coded on the GPU in one
    call; 48 sampled rows (first and last among them) against the oracle."""
    n, k, bd = 9728, 2560, 7
    mat = synth.random_matrix(64, k, bd, seed=(53, 0, 0))
    gen = torch.Generator(device="cuda").manual_seed(53)
    wd = torch.randn((n, k), device="cuda", generator=gen) * 0.05
    codes = svq.encode(wd, mat.perm, bd, mat.codebook, mat.radius)
    torch.cuda.synchronize()
    all_codes = so.unpack_codes(codes.cpu().numpy(), n, k)
    rows = np.concatenate([[0], np.sort(np.random.default_rng(53).choice(n, 46, replace=False)),
                           [n - 1]])
    w_rows = wd[torch.from_numpy(rows).cuda()].cpu().numpy()
    expect = se.encode_matrix(w_rows, mat.perm, bd, mat.codebook, mat.radius)
    assert np.array_equal(all_codes[rows], expect)


# ---- activation-weighted fit (svq_encode_weighted) --------------------------

def _encode_weighted_gpu(svq, w: np.ndarray, perm, h: np.ndarray, bd, cb, rad, ld_pad=0):
    n, k = w.shape
    buf = torch.zeros((n, k + ld_pad), dtype=torch.float32)
    buf[:, :k] = torch.from_numpy(w)
    wd = buf.cuda()[:, :k]
    codes = svq.encode_weighted(wd, perm, torch.from_numpy(np.ascontiguousarray(h, dtype=np.float64)).cuda(),
                                bd, cb, rad)
    torch.cuda.synchronize()
    return codes.cpu().numpy()


def test_weighted_hand_worked_fixture(svq):
    """The hand-worked fixture of the weighted rule (ties, zero weights, a
    power-of-two scale) on the GPU."""
    from tests.test_weighted_encode_oracle import _golden
    bd, cb, radius, perm, w, cases, _ = _golden()
    for name, code, h in cases:
        got = _encode_weighted_gpu(svq, w, perm, h, bd, cb, radius)
        assert np.array_equal(so.unpack_codes(got, 1, 8), np.array([[code]], dtype=np.uint32)), name


@pytest.mark.parametrize("n,k,bd,ld_pad", SHAPES)
def test_weighted_random_weights_match_the_oracle(svq, n, k, bd, ld_pad):
    """Bit-exact code streams against the weighted oracle: weights across the
    radius table with zeros and -0.0, channel weights lognormal (like
    energies to a power) with 15% exact zeros."""
    rng = np.random.default_rng(91 + n + k)
    mat = synth.random_matrix(n, k, bd, seed=(91, n, k))
    R = so.fp16_bits_to_f64(mat.radius)
    w = (rng.standard_normal((n, k)) * rng.uniform(0.05, 3.0) * R[-1] / np.sqrt(8)).astype(np.float32)
    w[rng.random((n, k)) < 0.05] = 0.0
    w[rng.random((n, k)) < 0.05] = -0.0
    h = rng.lognormal(0.0, 1.5, size=k)
    h[rng.random(k) < 0.15] = 0.0
    expect = se.encode_stream_weighted(w, mat.perm, h, bd, mat.codebook, mat.radius)
    got = _encode_weighted_gpu(svq, w, mat.perm, h, bd, mat.codebook, mat.radius, ld_pad)
    assert got.shape == expect.shape
    assert np.array_equal(got, expect), int((got != expect).sum())
    # the weighting matters on this data
    assert not np.array_equal(expect, se.encode_stream(w, mat.perm, bd, mat.codebook, mat.radius))


def test_weighted_ties_and_degenerate_weights(svq):
    """Duplicated codebook rows (equal errors: the first pair wins), every
    weight zero (every code takes pair (0, 0)), and decoded subvectors with
    positive weights (their own pair is the unique zero-error one)."""
    bd, k = 6, 64
    mat = synth.random_matrix(6, k, bd, seed=(92, 0, 0))
    cb = np.asarray(mat.codebook).copy().reshape(64, 8)
    cb[40] = cb[7]
    cb[63] = cb[7]
    rng = np.random.default_rng(92)
    W = so.decode_matrix(mat.codes, mat.n, mat.k, bd, cb, mat.radius, mat.perm).astype(np.float32)
    for h in (rng.uniform(0.5, 2.0, size=k), np.zeros(k), np.where(rng.random(k) < 0.5, 0.0, 1.0)):
        expect = se.encode_stream_weighted(W, mat.perm, h, bd, cb, mat.radius)
        got = _encode_weighted_gpu(svq, W, mat.perm, h, bd, cb, mat.radius)
        assert np.array_equal(got, expect)
    # with positive weights the decoded matrix comes back (duplicates of row
    # 7 resolve to the first index)
    codes = so.unpack_codes(mat.codes, mat.n, mat.k)
    s, d, r = so.split_fields(codes, bd)
    d = np.where((d == 40) | (d == 63), 7, d)
    got = _encode_weighted_gpu(svq, W, mat.perm, rng.uniform(0.5, 2.0, size=k), bd, cb, mat.radius)
    gs, gd, gr = so.split_fields(so.unpack_codes(got, mat.n, mat.k), bd)
    assert np.array_equal(gs, s) and np.array_equal(gd, d) and np.array_equal(gr, r)


def test_weighted_full_size_matrix_sampled_rows(svq):
    """The 9728 x 2560 gate shape (bd = 7) with the ESG energies of 2048
    calibration tokens as weights, every row coded on the GPU in one call; 24
    sampled rows (first and last among them) against the oracle."""
    n, k, bd = 9728, 2560, 7
    mat = synth.random_matrix(64, k, bd, seed=(93, 0, 0))
    x = synth.random_activations(2048, k, seed=(93, 1, 0))
    from oracle import svq_calib as sc
    h = sc.esg_energy(x)
    perm = sc.esg_perm(h)
    gen = torch.Generator(device="cuda").manual_seed(93)
    wd = torch.randn((n, k), device="cuda", generator=gen) * 0.05
    codes = svq.encode_weighted(wd, perm, torch.from_numpy(h).cuda(), bd, mat.codebook, mat.radius)
    torch.cuda.synchronize()
    all_codes = so.unpack_codes(codes.cpu().numpy(), n, k)
    rows = np.concatenate([[0], np.sort(np.random.default_rng(93).choice(n, 22, replace=False)), [n - 1]])
    w_rows = wd[torch.from_numpy(rows).cuda()].cpu().numpy()
    expect = se.encode_matrix_weighted(w_rows, perm, h, bd, mat.codebook, mat.radius)
    assert np.array_equal(all_codes[rows], expect)


@pytest.mark.parametrize("n,k,pad", [(1, 8, 0), (33, 1032, 3), (130, 512, 0)])
def test_abs_with_weighted_fit_matches_the_oracle(svq, n, k, pad):
    """ABS whose candidates are coded by the weighted fit: errors bit for
    bit, the chosen index and the chosen codes against the oracle."""
    from oracle import svq_calib as sc
    rng = np.random.default_rng(94 + n)
    cands = [(bd, m.codebook, m.radius) for bd, m in
             ((bd, synth.random_matrix(8, k, bd, seed=(94, bd, 0))) for bd in (6, 7, 8))]
    perm = synth.random_matrix(8, k, 7, seed=(94, 0, k)).perm
    R = so.fp16_bits_to_f64(cands[1][2])
    w = (rng.standard_normal((n, k)) * rng.uniform(0.2, 2.0) * R[-1] / np.sqrt(8)).astype(np.float32)
    h = rng.exponential(size=k) ** 0.5
    wbuf = torch.zeros((n, k + pad), dtype=torch.float32)
    wbuf[:, :k] = torch.from_numpy(w)
    chosen, errs, codes = svq.abs_select(wbuf.cuda()[:, :k], perm, torch.from_numpy(h).cuda(), cands,
                                         weighted_fit=True)
    torch.cuda.synchronize()
    c_ref, e_ref, codes_ref = sc.abs_select(w, perm, h, cands, weighted_fit=True)
    assert np.array_equal(errs, e_ref), (errs, e_ref)
    assert chosen == c_ref
    assert np.array_equal(codes.cpu().numpy(), so.pack_codes(codes_ref[c_ref]))
