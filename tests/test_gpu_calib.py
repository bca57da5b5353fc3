"""GPU parity of the calibration entry points against the CPU oracle.

svq_esg_perm: the energies (float64, one token-order chain per channel on
both sides) and the permutation (integer) are compared bit for bit.
svq_abs_select: the per-candidate errors are compared bit for bit (both
sides take the same double-precision operations in the same order: lanes,
then codes of a row, then rows), the chosen index exactly and the chosen
codes bit for bit.  Readings: those stated in include/svq.h.
"""
import numpy as np
import pytest

import synth
from oracle import svq_calib as sc
from oracle import svq_encoder as se
from oracle import svq_oracle as so
from tests.gpu_common import require_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svq():
    return require_gpu()


def _x_dev(bits, pad=0):
    t, k = bits.shape
    buf = np.zeros((t, k + pad), dtype=np.uint16)
    buf[:, :k] = bits
    return torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).cuda()[:, :k]


ESG_SHAPES = [
    # t, k, row padding (tiles of 256 tokens and 32 channels): one token and
    # one subvector; a ragged last token tile (300 = 256 + 44, 257 = 256 + 1)
    # and a ragged channel block (1032 = 32 * 32 + 8); strided rows; the
    # gate/up input width with 2048 calibration tokens (eight full tiles);
    # 1100 = 4 * 256 + 76; twenty tiles of one subvector; the down input
    # width (ranks across 38 spans of 256 channels)
    (1, 8, 0),
    (300, 64, 0),
    (257, 1032, 8),
    (2048, 2560, 0),
    (1100, 520, 0),
    (5000, 8, 0),
    (64, 9728, 0),
]


@pytest.mark.parametrize("t,k,pad", ESG_SHAPES)
def test_esg_matches_the_oracle(svq, t, k, pad):
    x = synth.random_activations(t, k, seed=(70, t, k))
    energy, perm = svq.esg_perm(_x_dev(x, pad))
    torch.cuda.synchronize()
    e_ref = sc.esg_energy(x)
    assert np.array_equal(energy.cpu().numpy(), e_ref)
    assert np.array_equal(perm.cpu().numpy(), sc.esg_perm(e_ref))


def test_esg_ties_and_zero_channels(svq):
    """Small integers (many channels of exactly equal energy: ties go to the
    lower channel index) and all-zero channels."""
    rng = np.random.default_rng(71)
    t, k = 40, 512
    vals = rng.integers(-2, 3, size=(t, k)).astype(np.float32)
    vals[:, rng.choice(k, 50, replace=False)] = 0.0
    x = synth.bf16_bits_from_f32(vals)
    energy, perm = svq.esg_perm(_x_dev(x))
    torch.cuda.synchronize()
    e_ref = sc.esg_energy(x)
    assert len(np.unique(e_ref)) < k // 4  # the case really has ties
    assert np.array_equal(energy.cpu().numpy(), e_ref)
    assert np.array_equal(perm.cpu().numpy(), sc.esg_perm(e_ref))


def _cands(n, k, seed):
    return [(bd, m.codebook, m.radius) for bd, m in
            ((bd, synth.random_matrix(8, k, bd, seed=(seed, bd, 0))) for bd in (6, 7, 8))]


# one row and one code; ragged row blocks (33 rows) and code chunks (129
# codes); 256 full rows; more rows (4100) than the totals kernel stages at
# once (4096)
@pytest.mark.parametrize("n,k,pad", [(1, 8, 0), (33, 1032, 3), (256, 2560, 0), (4100, 64, 0)])
def test_abs_matches_the_oracle(svq, n, k, pad):
    rng = np.random.default_rng(72 + n)
    cands = _cands(n, k, 72)
    perm = synth.random_matrix(8, k, 7, seed=(72, 0, k)).perm
    R = so.fp16_bits_to_f64(cands[1][2])
    w = (rng.standard_normal((n, k)) * rng.uniform(0.2, 2.0) * R[-1] / np.sqrt(8)).astype(np.float32)
    h = rng.exponential(size=k) ** 0.5
    wbuf = torch.zeros((n, k + pad), dtype=torch.float32)
    wbuf[:, :k] = torch.from_numpy(w)
    chosen, errs, codes = svq.abs_select(wbuf.cuda()[:, :k], perm, torch.from_numpy(h).cuda(), cands)
    torch.cuda.synchronize()
    c_ref, e_ref, codes_ref = sc.abs_select(w, perm, h, cands)
    assert np.array_equal(errs, e_ref), (errs, e_ref)
    assert chosen == c_ref
    assert np.array_equal(codes.cpu().numpy(), so.pack_codes(codes_ref[c_ref]))


def test_abs_finds_the_split_that_reproduces_the_weights(svq):
    """Weights decoded from the bd = 8 candidate: zero error, chosen from
    any position in the candidate list."""
    k = 512
    mats = {bd: synth.random_matrix(64, k, bd, seed=(73, bd, 0)) for bd in (6, 7, 8)}
    w = so.decode_matrix(mats[8].codes, 64, k, 8, mats[8].codebook, mats[8].radius,
                         mats[8].perm).astype(np.float32)
    h = torch.from_numpy(np.random.default_rng(73).exponential(size=k)).cuda()
    for order in [(8, 6, 7), (6, 7, 8)]:
        cands = [(bd, mats[bd].codebook, mats[bd].radius) for bd in order]
        chosen, errs, codes = svq.abs_select(torch.from_numpy(w).cuda(), mats[8].perm, h, cands)
        torch.cuda.synchronize()
        assert order[chosen] == 8 and errs[chosen] == 0.0 and np.all(np.delete(errs, chosen) > 0)
        assert np.array_equal(codes.cpu().numpy(), np.asarray(mats[8].codes))


def test_abs_full_size_gate(svq):
    """The 9728 x 2560 gate shape with the ESG permutation of 2048
    calibration tokens and h = energy: the chosen codes equal svq_encode's
    for the chosen split and, on 24 sampled rows, the oracle's; every error
    is finite and positive and the chosen one is the smallest."""
    n, k = 9728, 2560
    x = synth.random_activations(2048, k, seed=(74, 0, 0))
    energy, perm_d = svq.esg_perm(_x_dev(x))
    perm = perm_d.cpu().numpy()
    gen = torch.Generator(device="cuda").manual_seed(74)
    wd = torch.randn((n, k), device="cuda", generator=gen) * 0.05
    cands = _cands(n, k, 74)
    chosen, errs, codes = svq.abs_select(wd, perm, energy, cands)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(errs)) and np.all(errs > 0) and chosen == int(np.argmin(errs))
    bd, cb, rad = cands[chosen]
    again = svq.encode(wd, perm, bd, cb, rad)
    torch.cuda.synchronize()
    assert torch.equal(codes, again)
    rows = np.sort(np.random.default_rng(74).choice(n, 24, replace=False))
    all_codes = so.unpack_codes(codes.cpu().numpy(), n, k)
    w_rows = wd[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(all_codes[rows], se.encode_matrix(w_rows, perm, bd, cb, rad))


def test_abs_equal_candidates_pick_the_first(svq):
    """The same split listed three times: equal errors, index 0 chosen
    (first of equal smallest errors), codes equal to the oracle's."""
    n, k = 16, 256
    mat = synth.random_matrix(8, k, 7, seed=(75, 7, 0))
    w = np.random.default_rng(75).standard_normal((n, k)).astype(np.float32) * 0.05
    h = np.random.default_rng(76).exponential(size=k)
    c = (7, mat.codebook, mat.radius)
    chosen, errs, codes = svq.abs_select(torch.from_numpy(w).cuda(), mat.perm,
                                         torch.from_numpy(h).cuda(), [c, c, c])
    torch.cuda.synchronize()
    c_ref, e_ref, codes_ref = sc.abs_select(w, mat.perm, h, [c, c, c])
    assert chosen == 0 == c_ref and np.array_equal(errs, e_ref) and errs[0] == errs[1] == errs[2]
    assert np.array_equal(codes.cpu().numpy(), so.pack_codes(codes_ref[0]))
