"""Pins for the activation-weighted encoder oracle (no GPU).

The weighted fitting rule (oracle/svq_encoder.py, encode_fields_weighted;
SAGE paper, Abstract and Fig. 2 caption: ESG protects sensitive channels
through activation-weighted fitting) is checked against things other than
itself: a hand-worked fixture with ties and ignored lanes, optimality of
every chosen (direction, radius) pair in exact rational arithmetic over all
pairs, the round trip through the separately pinned decode oracle, and
invariances that the weighted squared error fixes (a power-of-two scale of
h changes nothing, lanes of weight zero do not matter).  Planted mistakes in
each step of the rule must fail at least one of these pins.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import svq_calib as sc
from oracle import svq_encoder as se
from oracle import svq_oracle as so
from tests.conftest import load_golden


def _hex(vals):
    return [int(v, 16) for v in vals]


def _golden():
    g = load_golden("weighted_encode_one_subvector.txt")
    n, k, bd = int(g["n"][0][0]), int(g["k"][0][0]), int(g["bd"][0][0])
    cb = np.tile(np.array(_hex(g["codebook_fill"][0]), dtype=np.uint16), (1 << bd, 1))
    for row in g["codebook_row"]:
        cb[int(row[0])] = _hex(row[1:])
    radius = np.array(_hex(g["radius"][0]), dtype=np.uint16)
    perm = np.array([int(v) for v in g["perm"][0]], dtype=np.int32)
    w = np.array([float(v) for v in g["w"][0]], dtype=np.float32).reshape(n, k)
    cases = [(name, int(code, 16), np.array([float(v) for v in hv])) for name, code, *hv in g["case"]]
    return bd, cb, radius, perm, w, cases, int(g["plain_code"][0][0], 16)


def _golden_ok():
    bd, cb, radius, perm, w, cases, _ = _golden()
    return all(int(se.encode_matrix_weighted(w, perm, h, bd, cb, radius)[0, 0]) == code
               for _, code, h in cases)


def test_golden_hand_worked_weighted_encoding():
    bd, cb, radius, perm, w, cases, plain = _golden()
    for name, code, h in cases:
        got = int(se.encode_matrix_weighted(w, perm, h, bd, cb, radius)[0, 0])
        assert got == code, f"case {name}: {got:#x} != {code:#x}"
    # the weighting changes the answer: the plain rule codes the same
    # subvector differently
    assert int(se.encode_matrix(w, perm, bd, cb, radius)[0, 0]) == plain
    assert plain != cases[0][1]


def _case(bd, n, k, seed):
    """Random matrix of the synthetic recipe, weights spread around the
    radius table, channel weights like energies^gamma with zeros."""
    mat = synth.random_matrix(n, k, bd, seed=(60, bd, seed))
    rng = np.random.default_rng(61 + 7 * bd + seed)
    Rv = so.fp16_bits_to_f64(mat.radius)
    g = np.abs(rng.standard_normal((n, k))) + 0.05
    g *= rng.uniform(0.5 * Rv[0], 1.5 * Rv[-1], size=(n, 1)) / np.sqrt(8.0)
    w = (g * np.where(rng.random((n, k)) < 0.5, -1.0, 1.0)).astype(np.float32)
    h = rng.lognormal(0.0, 1.5, size=k) ** 1.0
    h[rng.random(k) < 0.15] = 0.0
    return mat, w, h


def _exact_ok(mat, w, h, bd):
    """Every chosen pair attains the exact minimum of the weighted error over
    all pairs, up to the rounding of the float64 reduced error; where the
    exact minimum is separated from every other pair by more than that,
    the chosen pair is the exact minimiser."""
    s, d, r = se.encode_fields_weighted(w, mat.perm, h, bd, mat.codebook, mat.radius)
    D = [[Fraction(float(x)) for x in row]
         for row in so.fp16_bits_to_f64(np.asarray(mat.codebook).reshape(-1, 8))]
    R = [Fraction(float(x)) for x in so.fp16_bits_to_f64(mat.radius)]
    v = se.gather_subvectors(w, mat.perm)
    n, C, _ = v.shape
    hp = np.asarray(h, dtype=np.float64)[np.asarray(mat.perm, dtype=np.int64)].reshape(C, 8)
    for i in range(n):
        for c in range(C):
            a = [Fraction(abs(float(x))) for x in v[i, c]]
            hl = [Fraction(float(x)) for x in hp[c]]
            scale = sum(hl[l] * a[l] * a[l] for l in range(8)) + sum(hl) * R[-1] * R[-1]
            errs = []
            for dd in range(len(D)):
                for rr in range(len(R)):
                    errs.append(sum(hl[l] * (a[l] - R[rr] * D[dd][l]) ** 2 for l in range(8)))
            emin = min(errs)
            tol = scale * Fraction(1, 1 << 40)
            got = errs[int(d[i, c]) * len(R) + int(r[i, c])]
            if got - emin > tol:
                return False
            near = [j for j, e in enumerate(errs) if e - emin <= tol]
            if len(near) == 1 and near[0] != int(d[i, c]) * len(R) + int(r[i, c]):
                return False
            sg = sum((1 << l) for l in range(8) if np.signbit(v[i, c, l]))
            if int(s[i, c]) != sg:
                return False
    return True


@pytest.mark.parametrize("bd", [6, 7, 8])
def test_pairs_are_optimal_in_exact_arithmetic(bd):
    mat, w, h = _case(bd, 4, 16, 0)
    assert _exact_ok(mat, w, h, bd)
    # the data exercises the weighting: some codes differ from the plain rule
    plain = se.encode_matrix(w, mat.perm, bd, mat.codebook, mat.radius)
    weighted = se.encode_matrix_weighted(w, mat.perm, h, bd, mat.codebook, mat.radius)
    assert np.any(plain != weighted)


def _round_trip_ok(bd, seed=0):
    """Coding a decoded matrix with positive weights gives back its codes:
    the weighted error of the true pair is zero and, with these tables, no
    other pair reaches zero."""
    mat = synth.random_matrix(24, 128, bd, seed=(62, bd, seed))
    codes = so.unpack_codes(mat.codes, mat.n, mat.k)
    W = so.decode_matrix(mat.codes, mat.n, mat.k, mat.bd, mat.codebook, mat.radius, mat.perm)
    h = np.random.default_rng(63 + bd).uniform(0.25, 4.0, size=mat.k)
    got = se.encode_matrix_weighted(W.astype(np.float32), mat.perm, h, bd, mat.codebook, mat.radius)
    return np.array_equal(got, codes)


@pytest.mark.parametrize("bd", [6, 7, 8])
def test_round_trip_through_the_decode(bd):
    assert _round_trip_ok(bd)


def test_power_of_two_scale_of_h_changes_nothing():
    for bd in (6, 8):
        mat, w, h = _case(bd, 8, 64, 1)
        a = se.encode_matrix_weighted(w, mat.perm, h, bd, mat.codebook, mat.radius)
        b = se.encode_matrix_weighted(w, mat.perm, h * 4.0, bd, mat.codebook, mat.radius)
        c = se.encode_matrix_weighted(w, mat.perm, h * 0.125, bd, mat.codebook, mat.radius)
        assert np.array_equal(a, b) and np.array_equal(a, c)


def test_lanes_of_weight_zero_do_not_matter():
    """Changing the magnitude of a weight whose channel has h = 0 keeps the
    direction and radius (its sign bit is still recorded)."""
    bd = 7
    mat, w, h = _case(bd, 8, 64, 2)
    zero = np.nonzero(h == 0)[0]
    assert zero.size > 0
    w2 = w.copy()
    w2[:, zero] *= np.float32(3.5)
    s1, d1, r1 = se.encode_fields_weighted(w, mat.perm, h, bd, mat.codebook, mat.radius)
    s2, d2, r2 = se.encode_fields_weighted(w2, mat.perm, h, bd, mat.codebook, mat.radius)
    assert np.array_equal(s1, s2) and np.array_equal(d1, d2) and np.array_equal(r1, r2)
    # and with every weight zero, every subvector takes the first pair
    _, d0, r0 = se.encode_fields_weighted(w, mat.perm, np.zeros_like(h), bd, mat.codebook, mat.radius)
    assert not d0.any() and not r0.any()


def test_rejects_bad_weights():
    mat, w, h = _case(6, 2, 16, 3)
    for bad in (h[:-1], np.where(np.arange(h.size) == 3, -1.0, h), np.where(np.arange(h.size) == 0, np.nan, h)):
        with pytest.raises(ValueError):
            se.encode_fields_weighted(w, mat.perm, bad, 6, mat.codebook, mat.radius)


def test_abs_select_with_weighted_fit_scores_the_weighted_codes():
    """ABS on weighted-fit candidates: every candidate's codes are the
    weighted rule's, and its error is the weighted error of those codes,
    never above the plain rule's (both measured by the same pinned error)."""
    mat, w, h = _case(7, 6, 64, 4)
    cands = [(bd, synth.make_codebook(np.random.default_rng(70 + bd), bd),
              synth.make_radius_table(10 - bd)) for bd in (6, 7, 8)]
    ch_w, errs_w, codes_w = sc.abs_select(w, mat.perm, h, cands, weighted_fit=True)
    ch_p, errs_p, codes_p = sc.abs_select(w, mat.perm, h, cands)
    for (bd, cb, rad), cw, ew, ep in zip(cands, codes_w, errs_w, errs_p):
        assert np.array_equal(cw, se.encode_matrix_weighted(w, mat.perm, h, bd, cb, rad))
        assert ew <= ep * (1 + 1e-12)
    assert ch_w == int(np.argmin(errs_w))


# ---- planted mistakes: each must fail one of the pins above -----------------

def _mut_unweighted_A(hp, a):
    return a + 0.0 * hp[None, :, :]


def _mut_B_not_squared(hw, hp, Dd):
    A, _ = ORIG_SUMS(hw, hp, Dd)
    B = hp[:, 0] * Dd[0]
    for l in range(1, 8):
        B = B + hp[:, l] * Dd[l]
    return A, B


def _mut_error_sign(Rr, A, B):
    return (Rr * Rr) * B[None, :] + (Rr + Rr) * A


def _mut_radius_not_squared(Rr, A, B):
    return Rr * B[None, :] - (Rr + Rr) * A


def _mut_last_minimum(E, best):
    return E <= best


def _mut_weights_by_slot(h, perm, C):
    return ORIG_FIT(h, np.arange(8 * C), C)


ORIG_SUMS = se._direction_sums
ORIG_FIT = se._fit_weights

MUTATIONS = {
    "A without the weights": ("_weighted_magnitudes", _mut_unweighted_A),
    "B without the second D": ("_direction_sums", _mut_B_not_squared),
    "error sign": ("_reduced_error", _mut_error_sign),
    "radius not squared": ("_reduced_error", _mut_radius_not_squared),
    "last of equal minima": ("_improves", _mut_last_minimum),
    "weights by slot, not channel": ("_fit_weights", _mut_weights_by_slot),
}


def _pins_pass():
    if not _golden_ok():
        return False
    if not _round_trip_ok(6):
        return False
    mat, w, h = _case(6, 2, 16, 5)
    return _exact_ok(mat, w, h, 6)


def test_pins_pass_unmutated():
    assert _pins_pass()


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_weighted_encoder_mutation(monkeypatch, mutation):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(se, attr, fn)
    assert not _pins_pass(), f"planted mistake '{mutation}' went unnoticed"
