"""Plant plausible mistakes in the oracle (CPU only) and check that the
hand-worked fixtures catch every one of them."""
import numpy as np
import pytest

from oracle import svq_oracle as so
from tests.test_oracle import _golden_bounds_ok, _golden_case


def _golden_ok(name):
    n, k, bd, stream, cb, radius, perm, x, codes, y, w = _golden_case(name)
    W = so.decode_matrix(stream, n, k, bd, cb, radius, perm)
    return np.array_equal(so.linear(x, W).reshape(-1), y)


def _mut_no_radius(codes, bd, cb, radius):
    ones = np.full_like(np.asarray(radius), 0x3C00)
    return ORIG_DECODE(codes, bd, cb, ones)


def _mut_sign_polarity(codes, bd, cb, radius):
    return -ORIG_DECODE(codes, bd, cb, radius)


def _mut_sign_lane_order(codes, bd, cb, radius):
    c = np.asarray(codes, dtype=np.uint32)
    s = c & np.uint32(0xFF)
    rev = np.zeros_like(s)
    for l in range(8):
        rev |= ((s >> np.uint32(l)) & np.uint32(1)) << np.uint32(7 - l)
    return ORIG_DECODE((c & ~np.uint32(0xFF)) | rev, bd, cb, radius)


def _mut_field_order(codes, bd):
    c = np.asarray(codes, dtype=np.uint32)
    br = 10 - bd
    s = c & np.uint32(0xFF)
    r = (c >> np.uint32(8)) & np.uint32((1 << br) - 1)  # radius read first
    d = c >> np.uint32(8 + br)
    return s, d, r


def _mut_scatter_perm(wp, perm):
    perm = np.asarray(perm)
    return wp[:, perm]


def _mut_msb_first(stream, n, k):
    s = np.asarray(stream, dtype=np.uint8)
    rev = np.zeros_like(s)
    for b in range(8):
        rev |= ((s >> b) & 1) << (7 - b)
    return ORIG_UNPACK(rev, n, k)


ORIG_DECODE = so.decode_permuted
ORIG_UNPACK = so.unpack_codes

MUTATIONS = {
    "dropped radius": ("decode_permuted", _mut_no_radius),
    "sign polarity": ("decode_permuted", _mut_sign_polarity),
    "sign lane order": ("decode_permuted", _mut_sign_lane_order),
    "field order": ("split_fields", _mut_field_order),
    "permutation direction": ("unpermute", _mut_scatter_perm),
    "bit order": ("unpack_codes", _mut_msb_first),
}


def test_fixtures_pass_unmutated():
    assert _golden_ok("single_subvector.txt")
    assert _golden_ok("two_rows_bd6.txt")


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_fixture_catches_mutation(monkeypatch, mutation):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(so, attr, fn)
    caught = False
    for name in ("single_subvector.txt", "two_rows_bd6.txt"):
        try:
            caught |= not _golden_ok(name)
        except (AssertionError, ValueError, IndexError):
            caught = True
    assert caught, f"mutation '{mutation}' slipped through the fixtures"


# Planted mistakes in the parity bound itself: every GPU parity test passes
# or fails on so.tolerance, so a slip that loosens it must not go unnoticed.
ORIG_F64 = so.bf16_bits_to_f64


def _mut_bound_signed_x(x_bits, w):
    x = ORIG_F64(x_bits).reshape(-1, w.shape[1])  # |x| forgotten
    return x @ np.abs(w).T


def _mut_bound_signed_w(x_bits, w):
    x = np.abs(ORIG_F64(x_bits).reshape(-1, w.shape[1]))
    return x @ w.T  # |W| forgotten


def _mut_tolerance_rel(x_bits, w, rel=8e-2, atol=1e-6):
    return rel * so.abs_bound(x_bits, w) + atol


def _mut_tolerance_atol(x_bits, w, rel=8e-3, atol=1e-3):
    return rel * so.abs_bound(x_bits, w) + atol


BOUND_MUTATIONS = {
    "bound without |x|": ("abs_bound", _mut_bound_signed_x),
    "bound without |W|": ("abs_bound", _mut_bound_signed_w),
    "tolerance rel 8e-2": ("tolerance", _mut_tolerance_rel),
    "tolerance atol 1e-3": ("tolerance", _mut_tolerance_atol),
}


def test_bound_fixtures_pass_unmutated():
    assert _golden_bounds_ok("single_subvector.txt")
    assert _golden_bounds_ok("two_rows_bd6.txt")


@pytest.mark.parametrize("mutation", sorted(BOUND_MUTATIONS))
def test_bound_fixture_catches_mutation(monkeypatch, mutation):
    attr, fn = BOUND_MUTATIONS[mutation]
    monkeypatch.setattr(so, attr, fn)
    caught = not (_golden_bounds_ok("single_subvector.txt") and _golden_bounds_ok("two_rows_bd6.txt"))
    assert caught, f"mutation '{mutation}' slipped through the bound fixtures"
