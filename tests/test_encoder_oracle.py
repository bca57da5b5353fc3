"""Pins for the CPU encoder oracle (no GPU).

The encoder oracle is checked against things other than itself: a
hand-worked fixture in tests/golden/, the round trip through the (separately
pinned) decode oracle -- coding a decoded matrix must give back its codes,
since a unit direction is its own best match and a decoded subvector's norm
is its radius (SAGE paper, Fig. 2 caption: signs, direction and radius) --
and the optimality of every chosen field, verified in exact rational
arithmetic over all candidates.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import svq_encoder as se
from oracle import svq_oracle as so
from tests.conftest import load_golden


def _hex(vals):
    return [int(v, 16) for v in vals]


def test_golden_hand_worked_encoding():
    g = load_golden("encode_two_subvectors.txt")
    n, k, bd = int(g["n"][0][0]), int(g["k"][0][0]), int(g["bd"][0][0])
    cb = np.tile(np.array(_hex(g["codebook_fill"][0]), dtype=np.uint16), (1 << bd, 1))
    for row in g["codebook_row"]:
        cb[int(row[0])] = _hex(row[1:])
    radius = np.array(_hex(g["radius"][0]), dtype=np.uint16)
    perm = np.array([int(v) for v in g["perm"][0]], dtype=np.int32)
    w = np.array([float(v) for v in g["w"][0]], dtype=np.float32).reshape(n, k)
    assert np.signbit(w[0, 9])  # the fixture's -0.0 survived parsing
    expect = np.array(_hex(g["codes"][0]), dtype=np.uint32).reshape(n, k // 8)
    got = se.encode_matrix(w, perm, bd, cb, radius)
    assert np.array_equal(got, expect), [hex(v) for v in got.ravel()]


@pytest.mark.parametrize("bd", [6, 7, 8])
def test_round_trip_through_the_decode(bd):
    """encode(decode(codes)) == codes for random codes of the synthetic
    recipe, also as the canonical stream."""
    mat = synth.random_matrix(40, 256, bd, seed=(40, bd, 0))
    codes = so.unpack_codes(mat.codes, mat.n, mat.k)
    w = so.decode_matrix(mat.codes, mat.n, mat.k, mat.bd, mat.codebook, mat.radius, mat.perm)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    got = se.encode_matrix(w.astype(np.float32), mat.perm, bd, mat.codebook, mat.radius)
    assert np.array_equal(got, codes)
    stream = se.encode_stream(w.astype(np.float32), mat.perm, bd, mat.codebook, mat.radius)
    assert np.array_equal(stream, np.asarray(mat.codes, dtype=np.uint8))


def _exact(vals):
    return [Fraction(float(v)) for v in vals]


@pytest.mark.parametrize("bd", [6, 8])
def test_fields_are_optimal_in_exact_arithmetic(bd):
    """Every chosen direction maximises sum_l |v_l| D[j][l] (the first of
    equal maxima) and every radius minimises |norm(v) - R[t]| (the lower of
    two equally near radii), checked over all candidates with rationals."""
    rng = np.random.default_rng(41 + bd)
    n, k = 16, 32
    mat = synth.random_matrix(n, k, bd, seed=(41, bd, 1))
    perm = mat.perm
    # subvector norms spread over (and a little past) the radius table, so
    # that many fall between two radii; a few subvectors far outside it
    Rv = so.fp16_bits_to_f64(mat.radius)
    g = rng.standard_normal((n, k // 8, 8))
    g /= np.linalg.norm(g, axis=2, keepdims=True)
    norms = rng.uniform(0.8 * Rv[0], 1.2 * Rv[-1], size=(n, k // 8, 1))
    norms[0, 0, 0], norms[1, 1, 0] = 1e-3 * Rv[0], 1e3 * Rv[-1]
    wp = (g * norms).reshape(n, k)
    w = np.empty((n, k), dtype=np.float32)
    w[:, perm] = wp
    s, d, r = se.encode_fields(w, perm, bd, mat.codebook, mat.radius)
    D = [_exact(row) for row in so.fp16_bits_to_f64(np.asarray(mat.codebook).reshape(-1, 8))]
    R = _exact(so.fp16_bits_to_f64(mat.radius))
    for i in range(n):
        for c in range(k // 8):
            v = [Fraction(float(w[i, perm[8 * c + l]])) for l in range(8)]
            a = [abs(x) for x in v]
            # signs
            assert int(s[i, c]) == sum(1 << l for l in range(8) if np.signbit(w[i, perm[8 * c + l]]))
            # direction: no row scores higher, no earlier row scores as high
            score = [sum(ai * dj for ai, dj in zip(a, row)) for row in D]
            dc = int(d[i, c])
            assert all(score[dc] >= sc for sc in score)
            assert all(score[j] < score[dc] for j in range(dc))
            # radius: |norm - R[t]| <= |norm - R[u]| <=> norm^2 vs midpoint^2
            nsq = sum(ai * ai for ai in a)
            rc = int(r[i, c])
            for t in range(len(R)):
                mid = (R[min(t, rc)] + R[max(t, rc)]) / 2
                if t < rc:
                    assert nsq > mid * mid  # strictly nearer than every lower radius
                elif t > rc:
                    assert nsq <= mid * mid  # at least as near as every higher radius


def test_scaling_by_a_power_of_two_keeps_signs_and_directions():
    rng = np.random.default_rng(42)
    mat = synth.random_matrix(8, 64, 7, seed=(42, 7, 0))
    w = rng.standard_normal((8, 64)).astype(np.float32)
    s0, d0, _ = se.encode_fields(w, mat.perm, 7, mat.codebook, mat.radius)
    s1, d1, _ = se.encode_fields(w * np.float32(8.0), mat.perm, 7, mat.codebook, mat.radius)
    assert np.array_equal(s0, s1) and np.array_equal(d0, d1)


def test_rejects_unsorted_radius_table_and_bad_perm():
    mat = synth.random_matrix(2, 16, 8, seed=(43, 8, 0))
    w = np.ones((2, 16), dtype=np.float32)
    bad = np.asarray(mat.radius).copy()[::-1]
    with pytest.raises(ValueError):
        se.encode_matrix(w, mat.perm, 8, mat.codebook, bad)
    with pytest.raises(ValueError):
        se.encode_matrix(w, np.zeros(16, dtype=np.int32), 8, mat.codebook, mat.radius)


# ---- planted mistakes (CPU only): every one must be caught by the pins above

def _fields_with(w, perm, bd, cb, radius, *, sign_by_value=False, last_max=False,
                 signed_dot=False, log_radius=False, radius_of_square=False):
    v = se.gather_subvectors(w, perm)
    a = np.abs(v)
    neg = (v < 0) if sign_by_value else np.signbit(v)
    s = np.zeros(v.shape[:2], dtype=np.uint32)
    for l in range(8):
        s |= neg[:, :, l].astype(np.uint32) << np.uint32(l)
    D = so.fp16_bits_to_f64(np.asarray(cb).reshape(1 << bd, 8))
    score = np.einsum("icl,jl->icj", v if signed_dot else a, D)
    d = (score.shape[2] - 1 - np.argmax(score[:, :, ::-1], axis=2)) if last_max else np.argmax(score, axis=2)
    nrm = np.sqrt((a * a).sum(axis=2))
    if radius_of_square:
        nrm = nrm * nrm
    R = so.fp16_bits_to_f64(radius)
    dist = np.abs(np.log(nrm[:, :, None]) - np.log(R)) if log_radius else np.abs(nrm[:, :, None] - R)
    r = np.argmin(dist, axis=2)
    return s, d.astype(np.uint32), r.astype(np.uint32)


ENCODER_MUTATIONS = ["sign_by_value", "last_max", "signed_dot", "log_radius", "radius_of_square"]


@pytest.mark.parametrize("mutation", ENCODER_MUTATIONS)
def test_pins_catch_encoder_mutation(monkeypatch, mutation):
    def mutant(w, perm, bd, cb, radius):
        return _fields_with(w, perm, bd, cb, radius, **{mutation: True})
    monkeypatch.setattr(se, "encode_fields", mutant)
    pins = [test_golden_hand_worked_encoding,
            lambda: test_round_trip_through_the_decode(7),
            lambda: test_fields_are_optimal_in_exact_arithmetic(6),
            lambda: test_fields_are_optimal_in_exact_arithmetic(8)]
    caught = False
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught = True
    assert caught, f"mutation '{mutation}' slipped through the encoder pins"


def test_unmutated_reference_form_agrees():
    """The plain (einsum / sqrt / argmin) form of the same rules gives the
    oracle's codes on random data, so the mutants above differ only in the
    planted mistake."""
    rng = np.random.default_rng(44)
    mat = synth.random_matrix(16, 128, 7, seed=(44, 7, 0))
    w = rng.standard_normal((16, 128)).astype(np.float32)
    a = se.encode_fields(w, mat.perm, 7, mat.codebook, mat.radius)
    b = _fields_with(w, mat.perm, 7, mat.codebook, mat.radius)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
