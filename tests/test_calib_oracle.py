"""Pins for the CPU oracle of the calibration steps (ESG energies and
permutation, activation-weighted reconstruction error, ABS split choice).
No GPU.

The oracle is checked against hand-worked fixtures in tests/golden/, the
exactly rounded mean (math.fsum) within the error bound of a sequential sum,
the tier structure the pages ask for, a dense recomputation of the weighted
error through the separately pinned decode oracle (un-permuted matrix, so a
wrong channel index fails it), exactly representable weights (zero error)
and planted mistakes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import svq_calib as sc
from oracle import svq_encoder as se
from oracle import svq_oracle as so
from tests.conftest import load_golden


def _bf16(vals):
    return synth.bf16_bits_from_f32(np.asarray(vals, dtype=np.float32))


def test_golden_esg():
    g = load_golden("esg_sixteen_channels.txt")
    x = _bf16([[float(v) for v in g["x0"][0]], [float(v) for v in g["x1"][0]]])
    energy = sc.esg_energy(x)
    assert np.array_equal(energy, np.array([float(v) for v in g["energy"][0]]))
    assert np.array_equal(sc.esg_perm(energy), np.array([int(v) for v in g["perm"][0]]))


def test_energy_within_the_bound_of_the_exact_mean():
    """|oracle - exact mean| <= (T - 1) * 2^-53 * exact + one division
    rounding, the bound of a sequential sum of non-negative terms."""
    rng = np.random.default_rng(60)
    T, k = 301, 64
    x = _bf16(rng.standard_normal((T, k)) * np.exp(rng.uniform(-8, 8, size=k)))
    xf = so.bf16_bits_to_f64(x)
    e = sc.esg_energy(x)
    for j in range(k):
        exact = Fraction(math.fsum(float(v) * float(v) for v in xf[:, j])) / T
        bound = (T + 1) * 2.0 ** -53 * float(exact)
        assert abs(Fraction(float(e[j])) - exact) <= Fraction(bound)


def test_energy_closed_forms():
    x = _bf16(np.full((1000, 16), 0.5))
    assert np.all(sc.esg_energy(x) == 0.25)          # exact: sums of 0.25 are exact
    x = _bf16(np.vstack([np.full((1, 8), 3.0), np.zeros((2, 8))]))
    assert np.all(sc.esg_energy(x) == 3.0)           # 9 / 3
    with pytest.raises(ValueError):
        sc.esg_energy(np.zeros((0, 8), dtype=np.uint16))


@pytest.mark.parametrize("k", [8, 64, 2560, 1032])
def test_perm_tier_structure(k):
    """A permutation; lane l of every subvector lies in tier l (every
    channel of lane l has at least the energy of every channel of lane
    l + 1); along the subvectors of one lane the energy does not rise; ties
    keep channel order."""
    rng = np.random.default_rng(61 + k)
    e = np.round(rng.exponential(size=k), 1)  # many exact ties
    perm = sc.esg_perm(e)
    assert np.array_equal(np.sort(perm), np.arange(k))
    C = k // 8
    lanes = e[perm].reshape(C, 8)
    for lane in range(7):
        assert lanes[:, lane].min() >= lanes[:, lane + 1].max()
    assert np.all(np.diff(lanes, axis=0) <= 0)
    chan = perm.reshape(C, 8)
    for lane in range(8):
        col_e, col_c = lanes[:, lane], chan[:, lane]
        same = col_e[1:] == col_e[:-1]
        assert np.all(col_c[1:][same] > col_c[:-1][same])
    # the same order as numpy's stable lexicographic sort
    assert np.array_equal(sc.esg_rank_order(e), np.lexsort((np.arange(k), -e)))


def test_golden_weighted_error():
    g = load_golden("encode_two_subvectors.txt")
    bd = int(g["bd"][0][0])
    cb = np.tile(np.array([int(v, 16) for v in g["codebook_fill"][0]], dtype=np.uint16), (1 << bd, 1))
    for row in g["codebook_row"]:
        cb[int(row[0])] = [int(v, 16) for v in row[1:]]
    radius = np.array([int(v, 16) for v in g["radius"][0]], dtype=np.uint16)
    perm = np.array([int(v) for v in g["perm"][0]], dtype=np.int32)
    w = np.array([float(v) for v in g["w"][0]], dtype=np.float32).reshape(1, 16)
    codes = np.array([[int(v, 16) for v in g["codes"][0]]], dtype=np.uint32)
    h = np.arange(1, 17, dtype=np.float64)
    expect = float(load_golden("weighted_error_two_subvectors.txt")["row_error"][0][0])
    assert sc.weighted_error_rows(w, perm, h, codes, bd, cb, radius)[0] == expect


def _dense_weighted_error(w, mat_perm, h, codes, bd, cb, rad):
    """Through the un-permuted dense decode: sum_j h[j] (W - W_hat)^2 per row."""
    n, k = w.shape
    W = so.unpermute(so.decode_permuted(codes, bd, cb, rad), mat_perm)
    return ((w.astype(np.float64) - W) ** 2 * h[None, :]).sum(axis=1)


@pytest.mark.parametrize("bd", [6, 7, 8])
def test_weighted_error_matches_the_dense_form(bd):
    rng = np.random.default_rng(62 + bd)
    mat = synth.random_matrix(12, 128, bd, seed=(62, bd, 0))
    w = (rng.standard_normal((12, 128)) * 0.05).astype(np.float32)
    h = rng.exponential(size=128) ** 0.7
    codes = se.encode_matrix(w, mat.perm, bd, mat.codebook, mat.radius)
    rows = sc.weighted_error_rows(w, mat.perm, h, codes, bd, mat.codebook, mat.radius)
    dense = _dense_weighted_error(w, mat.perm, h, codes, bd, mat.codebook, mat.radius)
    assert np.allclose(rows, dense, rtol=1e-12, atol=0)
    # linear in h, exactly for a power of two
    assert np.array_equal(sc.weighted_error_rows(w, mat.perm, 4 * h, codes, bd, mat.codebook,
                                                 mat.radius), 4 * rows)


def _decodable_weights(mat):
    return so.decode_matrix(mat.codes, mat.n, mat.k, mat.bd, mat.codebook, mat.radius,
                            mat.perm).astype(np.float32)


def test_abs_picks_the_split_that_reproduces_the_weights():
    """Weights decoded from the bd = 7 candidate: its error is exactly 0 and
    the other splits' errors are positive, whatever the candidate order."""
    cands = {bd: synth.random_matrix(8, 64, bd, seed=(63, bd, 0)) for bd in (6, 7, 8)}
    w = _decodable_weights(cands[7])
    perm = cands[7].perm
    h = np.random.default_rng(63).exponential(size=64)
    for order in [(6, 7, 8), (7, 8, 6), (8, 6, 7)]:
        cl = [(bd, cands[bd].codebook, cands[bd].radius) for bd in order]
        chosen, errs, codes = sc.abs_select(w, perm, h, cl)
        assert order[chosen] == 7 and errs[chosen] == 0.0
        assert np.all(np.delete(errs, chosen) > 0)
        assert np.array_equal(codes[chosen], so.unpack_codes(cands[7].codes, 8, 64))


def test_abs_ties_go_to_the_first_candidate():
    mat = synth.random_matrix(4, 32, 6, seed=(64, 6, 0))
    w = np.random.default_rng(64).standard_normal((4, 32)).astype(np.float32)
    c = (6, mat.codebook, mat.radius)
    chosen, errs, _ = sc.abs_select(w, mat.perm, np.ones(32), [c, c, c])
    assert chosen == 0 and errs[0] == errs[1] == errs[2] > 0


# ---- planted mistakes (CPU only): every one must be caught by the pins above

def test_total_in_order_is_sequential():
    """total_in_order adds in index order, one rounding per addition.  The
    values are chosen so that the order decides the result: the ulp of
    1e16 is 2, so 1e16 + 1 rounds (ties to even) back to 1e16."""
    # sixteen values: numpy's eight-way pairwise sum would give 1.0 here
    assert sc.total_in_order(np.array([1e16, 1.0] + [0.0] * 6 + [-1e16] + [0.0] * 7)) == 0.0
    assert sc.total_in_order(np.array([-1e16, 1e16, 1.0])) == 1.0
    assert sc.total_in_order(np.array([1.0, 1e16, -1e16])) == 0.0
    assert sc.total_in_order(np.array([0.25])) == 0.25
    assert sc.total_in_order(np.array([], dtype=np.float64)) == 0.0


def _mut_energy_abs(x_bits):
    x = np.abs(so.bf16_bits_to_f64(x_bits))
    return x.sum(axis=0) / x.shape[0]


def _mut_perm_contiguous(energy):
    return sc.esg_rank_order(energy).astype(np.int32)  # tiers inside a subvector not spread


def _mut_perm_ascending(energy):
    e = np.asarray(energy)
    order = np.array(sorted(range(e.size), key=lambda j: (e[j], j)))
    C = e.size // 8
    return np.array([order[l * C + c] for c in range(C) for l in range(8)], dtype=np.int32)


_orig_rows = sc.weighted_error_rows


def _mut_error_unweighted(w, perm, h, codes, bd, cb, rad):
    return _orig_rows(w, perm, np.ones_like(np.asarray(h, dtype=np.float64)), codes, bd, cb, rad)


def _mut_error_h_slot_order(w, perm, h, codes, bd, cb, rad):
    # weight of slot p taken from channel p instead of channel perm[p]
    return _orig_rows(w, perm, np.asarray(h, dtype=np.float64)[np.argsort(perm)], codes, bd, cb, rad)


def _mut_total_reversed(values):
    tot = 0.0
    for v in np.asarray(values, dtype=np.float64)[::-1]:
        tot = tot + float(v)
    return tot


def _mut_total_pairwise(values):
    return float(np.sum(np.asarray(values, dtype=np.float64)))


def _mut_total_exact(values):
    return math.fsum(np.asarray(values, dtype=np.float64).tolist())


MUTANTS = {
    "total_reversed": ("total_in_order", _mut_total_reversed),
    "total_pairwise": ("total_in_order", _mut_total_pairwise),
    "total_exact": ("total_in_order", _mut_total_exact),
    "energy_abs": ("esg_energy", _mut_energy_abs),
    "perm_contiguous": ("esg_perm", _mut_perm_contiguous),
    "perm_ascending": ("esg_perm", _mut_perm_ascending),
    "error_unweighted": ("weighted_error_rows", _mut_error_unweighted),
    "error_h_slot_order": ("weighted_error_rows", _mut_error_h_slot_order),
    "abs_argmax": ("abs_select", None),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_calib_mutation(monkeypatch, name):
    attr, fn = MUTANTS[name]
    if name == "abs_argmax":
        orig = sc.abs_select

        def fn(w, perm, h, cands):
            chosen, errs, codes = orig(w, perm, h, cands)
            return int(np.argmax(errs)), errs, codes
    monkeypatch.setattr(sc, attr, fn)
    pins = [test_golden_esg, test_energy_closed_forms, test_golden_weighted_error,
            lambda: test_perm_tier_structure(64),
            lambda: test_weighted_error_matches_the_dense_form(7),
            test_abs_picks_the_split_that_reproduces_the_weights,
            test_total_in_order_is_sequential]
    caught = False
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught = True
    assert caught, f"mutation '{name}' slipped through the calibration pins"
