"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: hand-worked fixtures
in tests/golden/, a pure-Python brute force that reads the bitstream one bit
at a time, closed forms, invariants of the code structure in the SAGE
paper's Fig. 2 caption (signs + direction + radius: the decoded subvector's
norm is the radius, signs only flip), and torch's CPU casts for the scalar
rounding helpers.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import bruteforce as bf
from oracle import svq_oracle as so
from tests.conftest import load_golden


def _hex(vals):
    return [int(v, 16) for v in vals]


def _golden_case(name):
    g = load_golden(name)
    n = int(g["n"][0][0])
    k = int(g["k"][0][0])
    bd = int(g["bd"][0][0])
    stream = np.array(_hex(g["stream"][0]), dtype=np.uint8)
    cb = np.zeros((1 << bd, 8), dtype=np.uint16)
    for row in g["codebook_row"]:
        cb[int(row[0])] = _hex(row[1:])
    radius = np.array(_hex(g["radius"][0]), dtype=np.uint16)
    perm = np.array([int(v) for v in g["perm"][0]], dtype=np.int32)
    x = np.array(_hex(g["x"][0]), dtype=np.uint16).reshape(1, k)
    codes = np.array(_hex(g["codes"][0]), dtype=np.uint32).reshape(n, k // 8)
    y = np.array([float(v) for v in g["y"][0]])
    w = np.array([float(v) for v in g["w"][0]]) if "w" in g else None
    return n, k, bd, stream, cb, radius, perm, x, codes, y, w


@pytest.mark.parametrize("name", ["single_subvector.txt", "two_rows_bd6.txt"])
def test_golden_worked_examples(name):
    n, k, bd, stream, cb, radius, perm, x, codes, y, w = _golden_case(name)
    assert so.stream_bytes(n, k) == stream.size
    assert np.array_equal(so.unpack_codes(stream, n, k), codes)
    assert np.array_equal(so.pack_codes(codes), stream)
    W = so.decode_matrix(stream, n, k, bd, cb, radius, perm)
    if w is not None:
        assert np.array_equal(W.reshape(-1), w)
    y64 = so.linear(x, W)
    assert np.array_equal(y64.reshape(-1), y)
    # the brute force reaches the same exact values
    yb = bf.linear(list(stream), n, k, bd, cb.tolist(), radius.tolist(), perm.tolist(),
                   x.tolist())
    assert [float(v) for v in yb[0]] == list(y)


def _golden_bounds_ok(name):
    """The parity bound of a hand-worked fixture: abs_bound equals the
    fixture's hand sum of |W_ij||x_j| exactly (small dyadic values, so the
    fp64 product is exact), and tolerance is 8e-3 times it plus 1e-6."""
    g = load_golden(name)
    n, k, bd, stream, cb, radius, perm, x, codes, y, w = _golden_case(name)
    W = so.decode_matrix(stream, n, k, bd, cb, radius, perm)
    cases = [(x, np.array([float(v) for v in g["bound"][0]]))]
    if "x_signed" in g:
        xs = np.array(_hex(g["x_signed"][0]), dtype=np.uint16).reshape(1, k)
        ys = np.array([float(v) for v in g["y_signed"][0]])
        if not np.array_equal(so.linear(xs, W).reshape(-1), ys):
            return False
        cases.append((xs, np.array([float(v) for v in g["bound_signed"][0]])))
    for xb, bound in cases:
        if not np.array_equal(so.abs_bound(xb, W).reshape(-1), bound):
            return False
        if not np.array_equal(so.tolerance(xb, W).reshape(-1), 8e-3 * bound + 1e-6):
            return False
    return True


@pytest.mark.parametrize("name", ["single_subvector.txt", "two_rows_bd6.txt"])
def test_golden_parity_bound(name):
    assert _golden_bounds_ok(name)


def test_golden_two_codes_stream():
    g = load_golden("two_codes_stream.txt")
    codes = np.array(_hex(g["codes"][0]), dtype=np.uint32)
    stream = np.array(_hex(g["stream"][0]), dtype=np.uint8)
    assert np.array_equal(so.pack_codes(codes), stream)
    assert np.array_equal(so.unpack_codes(stream, 1, 16).reshape(-1), codes)
    assert so.stream_bytes(1, 16) == 5


def test_fields_hand_example():
    # signs 0x17, d 3, r 2 with bd 8 (single_subvector.txt)
    s, d, r = so.split_fields(np.array([0x20317], dtype=np.uint32), 8)
    assert (int(s[0]), int(d[0]), int(r[0])) == (0x17, 3, 2)
    # bd 6: the radius starts at bit 14
    s, d, r = so.split_fields(np.array([0x3FEFF], dtype=np.uint32), 6)
    assert (int(s[0]), int(d[0]), int(r[0])) == (0xFF, 62, 15)
    assert int(so.join_fields(0xFF, 62, 15, 6)) == 0x3FEFF


@pytest.mark.parametrize("n,k", [(1, 8), (3, 8), (1, 24), (5, 40), (7, 1024), (4, 768)])
def test_pack_unpack_roundtrip(n, k):
    rng = np.random.default_rng(n * 1000 + k)
    codes = rng.integers(0, 1 << 18, size=(n, k // 8), dtype=np.uint32)
    stream = so.pack_codes(codes)
    assert stream.size == so.stream_bytes(n, k) == (n * k * 9 + 31) // 32
    assert np.array_equal(so.unpack_codes(stream, n, k), codes)
    # and the other way round, from random bytes (unused tail bits zeroed)
    raw = rng.integers(0, 256, size=stream.size, dtype=np.uint8)
    tail = (n * (k // 8) * 18) % 8
    if tail:
        raw[-1] &= (1 << tail) - 1
    assert np.array_equal(so.pack_codes(so.unpack_codes(raw, n, k)), raw)


def test_unpack_matches_bitwise_reader():
    rng = np.random.default_rng(7)
    n, k = 3, 64
    raw = rng.integers(0, 256, size=so.stream_bytes(n, k), dtype=np.uint8)
    codes = so.unpack_codes(raw, n, k).reshape(-1)
    for g in range(codes.size):
        assert int(codes[g]) == bf.read_field(list(raw), 18 * g, 18)


def test_stream_size_matches_bits_per_weight():
    # 18 bits per 8 weights = 2.25 bits per weight (Table 1, SPHQuant row)
    for n, k in [(512, 1024), (4096, 2560), (2560, 9728), (768, 2048), (2048, 768)]:
        assert so.stream_bytes(n, k) * 8 == n * k * 9 // 4
    assert so.stream_bytes(512, 1024) == 147456
    assert so.stream_bytes(9728, 2560) == 7004160
    assert so.stream_bytes(768, 2048) == 442368


@pytest.mark.parametrize("bd", [6, 7, 8])
def test_synthetic_codebook_unit_norm_positive_orthant(bd):
    for seed in range(4):
        cb = synth.make_codebook(np.random.default_rng(seed), bd)
        assert cb.shape == (1 << bd, 8)
        assert np.all((cb & 0x8000) == 0)  # sign bit clear: positive orthant
        v = so.fp16_bits_to_f64(cb)
        assert np.all(np.abs(np.linalg.norm(v, axis=1) - 1.0) <= 1e-3)


def test_synthetic_radius_table():
    r2 = so.fp16_bits_to_f64(synth.make_radius_table(2))
    expect = 0.02 * np.sqrt(8) * np.array([0.5, 1.0, 2.0, 4.0])
    assert np.allclose(r2, expect, rtol=2 ** -11)
    for br in (2, 3, 4):
        r = so.fp16_bits_to_f64(synth.make_radius_table(br))
        assert r.size == 1 << br and np.all(np.diff(r) > 0)
        assert np.isclose(r[0], 0.02 * np.sqrt(8) * 0.5, rtol=2 ** -11)
        assert np.isclose(r[-1], 0.02 * np.sqrt(8) * 4.0, rtol=2 ** -11)


@pytest.mark.parametrize("bd", [6, 7, 8])
def test_norm_invariant(bd):
    # the decoded subvector's norm is radius * |D row| (= radius up to the
    # fp16 rounding of the unit-norm row)
    w = synth.random_matrix(8, 256, bd, seed=(1, bd, 0))
    codes = so.unpack_codes(w.codes, w.n, w.k)
    wp = so.decode_permuted(codes, bd, w.codebook, w.radius).reshape(w.n, w.k // 8, 8)
    _, d, r = so.split_fields(codes, bd)
    R = so.fp16_bits_to_f64(w.radius)[r]
    Dn = np.linalg.norm(so.fp16_bits_to_f64(w.codebook)[d], axis=-1)
    nrm = np.linalg.norm(wp, axis=-1)
    assert np.allclose(nrm, R * Dn, rtol=1e-14, atol=0)
    assert np.all(np.abs(nrm - R) <= R * 1e-3)


def test_sign_invariants():
    w = synth.random_matrix(6, 64, 7, seed=(2, 0, 0))
    codes = so.unpack_codes(w.codes, w.n, w.k)
    wp = so.decode_permuted(codes, 7, w.codebook, w.radius)
    flipped = codes ^ np.uint32(0xFF)
    wp_f = so.decode_permuted(flipped, 7, w.codebook, w.radius)
    assert np.array_equal(wp_f, -wp)
    cleared = codes & ~np.uint32(0xFF)
    assert np.array_equal(np.abs(so.decode_permuted(cleared, 7, w.codebook, w.radius)), np.abs(wp))
    # flipping every sign of row 3 negates y[:, 3] exactly
    x = synth.random_activations(3, 64)
    W = so.unpermute(wp, w.perm)
    codes2 = codes.copy()
    codes2[3] ^= np.uint32(0xFF)
    W2 = so.unpermute(so.decode_permuted(codes2, 7, w.codebook, w.radius), w.perm)
    y1, y2 = so.linear(x, W), so.linear(x, W2)
    assert np.array_equal(y2[:, 3], -y1[:, 3])
    assert np.array_equal(np.delete(y2, 3, axis=1), np.delete(y1, 3, axis=1))


def test_closed_form_zero_radius():
    w = synth.random_matrix(4, 32, 8, seed=(3, 0, 0))
    zero_r = np.zeros_like(w.radius)
    W = so.decode_matrix(w.codes, w.n, w.k, 8, w.codebook, zero_r, w.perm)
    x = synth.random_activations(2, 32)
    assert np.all(so.linear(x, W) == 0)


def test_closed_form_unit_directions():
    # every codebook row = e_0, perm = identity: W[i, 8c] = +-R[r_ic], rest 0
    n, k, bd = 3, 24, 6
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 1 << 18, size=(n, k // 8), dtype=np.uint32)
    cb = np.zeros((1 << bd, 8), dtype=np.uint16)
    cb[:, 0] = 0x3C00
    radius = np.arange(1, 17).astype(np.float16).view(np.uint16)
    W = so.decode_matrix(so.pack_codes(codes), n, k, bd, cb, radius, np.arange(k))
    expect = np.zeros((n, k))
    for i in range(n):
        for c in range(k // 8):
            code = int(codes[i, c])
            r = code >> (8 + bd)
            sgn = -1.0 if code & 1 else 1.0
            expect[i, 8 * c] = sgn * (r + 1)
    assert np.array_equal(W, expect)


def test_closed_form_constant_rows():
    # D rows all = fp16(1/sqrt 8): y[m,i] = sum_c R[r_ic] D0 sum_l +-x[m, perm[8c+l]]
    n, k, bd = 4, 32, 7
    w = synth.random_matrix(n, k, bd, seed=(4, 0, 0))
    d0 = np.float16(1 / np.sqrt(8))
    cb = np.full((1 << bd, 8), d0, dtype=np.float16).view(np.uint16)
    x = synth.random_activations(2, k)
    W = so.decode_matrix(w.codes, n, k, bd, cb, w.radius, w.perm)
    y = so.linear(x, W)
    codes = so.unpack_codes(w.codes, n, k)
    xv = so.bf16_bits_to_f64(x)
    R = so.fp16_bits_to_f64(w.radius)
    expect = np.zeros((2, n))
    for m in range(2):
        for i in range(n):
            for c in range(k // 8):
                s, d, r = (int(v) for v in so.split_fields(codes[i, c], bd))
                acc = sum((-1 if (s >> l) & 1 else 1) * xv[m, w.perm[8 * c + l]] for l in range(8))
                expect[m, i] += R[r] * float(d0) * acc
    assert np.allclose(y, expect, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("bd", [2, 5, 6, 7, 8, 9])
def test_bruteforce_agrees_tiny(bd):
    rng = np.random.default_rng(100 + bd)
    for trial in range(3):
        n = int(rng.integers(1, 5))
        k = 8 * int(rng.integers(1, 5))
        w = synth.random_matrix(n, k, bd, seed=(5, bd, trial))
        x = synth.random_activations(2, k, seed=(5, bd, trial + 10))
        W = so.decode_matrix(w.codes, n, k, bd, w.codebook, w.radius, w.perm)
        Wb = bf.decode_dense(list(w.codes), n, k, bd, w.codebook.tolist(), w.radius.tolist(),
                             w.perm.tolist())
        assert np.array_equal(W, np.array([[float(v) for v in row] for row in Wb]))
        y = so.linear(x, W)
        yb = bf.linear(list(w.codes), n, k, bd, w.codebook.tolist(), w.radius.tolist(),
                       w.perm.tolist(), x.tolist())
        exact = np.array([[float(v) for v in row] for row in yb])
        scale = so.abs_bound(x, W)
        assert np.all(np.abs(y - exact) <= 1e-15 * scale + 1e-300)


def test_all_codes_one_subvector():
    # every one of the 2**18 codes of one subvector, bd = 8, checked against a
    # per-code pure-Python decode of the fields
    bd = 8
    w = synth.random_matrix(1, 8, bd, seed=(6, 0, 0))
    codes = np.arange(1 << 18, dtype=np.uint32).reshape(1, -1)
    wp = so.decode_permuted(codes, bd, w.codebook, w.radius).reshape(-1, 8)
    D = [[float(bf.fp16_value(int(b))) for b in row] for row in w.codebook]
    R = [float(bf.fp16_value(int(b))) for b in w.radius]
    expect = np.empty((1 << 18, 8))
    for code in range(1 << 18):
        s, d, r = code & 0xFF, (code >> 8) & 0xFF, code >> 16
        rad, row = R[r], D[d]
        expect[code] = [(-rad if (s >> l) & 1 else rad) * row[l] for l in range(8)]
    assert np.array_equal(wp, expect)
    # and a fixed x: y for each code equals the per-code dot product
    xb = synth.random_activations(1, 8, seed=(6, 1, 0))
    xv = so.bf16_bits_to_f64(xb)[0]
    assert np.allclose(wp @ xv, expect @ xv, rtol=0, atol=0)


def test_permutation_equivariance():
    n, k = 5, 96
    w = synth.random_matrix(n, k, 7, seed=(7, 0, 0))
    x = synth.random_activations(3, k, seed=(7, 1, 0))
    W = so.decode_matrix(w.codes, n, k, 7, w.codebook, w.radius, w.perm)
    Wid = so.decode_matrix(w.codes, n, k, 7, w.codebook, w.radius, np.arange(k))
    assert np.array_equal(W[:, w.perm], Wid)
    y1 = so.linear(x, W)
    y2 = so.linear(x[:, w.perm], Wid)
    assert np.allclose(y1, y2, rtol=1e-13, atol=1e-14)


def test_linearity():
    n, k = 4, 64
    w = synth.random_matrix(n, k, 8, seed=(8, 0, 0))
    W = so.decode_matrix(w.codes, n, k, 8, w.codebook, w.radius, w.perm)
    x = synth.random_activations(2, k, seed=(8, 1, 0))
    x2 = so.bf16_bits_from_f64(2.0 * so.bf16_bits_to_f64(x))
    assert np.array_equal(so.linear(x2, W), 2.0 * so.linear(x, W))
    xa = synth.random_activations(2, k, seed=(8, 2, 0))
    xb = synth.random_activations(2, k, seed=(8, 3, 0))
    ya, yb = so.linear(xa, W), so.linear(xb, W)
    xs = so.bf16_bits_to_f64(xa) + so.bf16_bits_to_f64(xb)
    ys = xs @ W.T
    assert np.allclose(ys, ya + yb, rtol=1e-12, atol=1e-13)


def test_dense_matches_per_subvector_sum():
    n, k, bd = 6, 128, 6
    w = synth.random_matrix(n, k, bd, seed=(9, 0, 0))
    x = synth.random_activations(2, k, seed=(9, 1, 0))
    W = so.decode_matrix(w.codes, n, k, bd, w.codebook, w.radius, w.perm)
    y = so.linear(x, W)
    codes = so.unpack_codes(w.codes, n, k)
    s, d, r = so.split_fields(codes, bd)
    D = so.fp16_bits_to_f64(w.codebook)
    R = so.fp16_bits_to_f64(w.radius)
    xv = so.bf16_bits_to_f64(x)
    fused = np.zeros((2, n))
    for m in range(2):
        for i in range(n):
            for c in range(k // 8):
                t = 0.0
                for l in range(8):
                    sg = -1.0 if (int(s[i, c]) >> l) & 1 else 1.0
                    t += sg * D[d[i, c], l] * xv[m, w.perm[8 * c + l]]
                fused[m, i] += R[r[i, c]] * t
    assert np.allclose(y, fused, rtol=1e-12, atol=1e-14)


def test_scalar_formats_match_torch():
    rng = np.random.default_rng(12)
    f = rng.standard_normal(1 << 20).astype(np.float32) * np.float32(3.0)
    f[:1000] = np.ldexp(rng.standard_normal(1000), rng.integers(-140, -120, 1000)).astype(np.float32)
    # exact ties between two bf16 values
    base = rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16
    f[1000:3000] = (base | np.uint32(0x8000)).view(np.float32)
    f[3000:3010] = [0.0, -0.0, 1.0, -1.0, 3.3895314e38, 1e-45, -1e-45, 65504.0, 2 ** -126, 2 ** -133]
    f = f[np.isfinite(f)]
    ours = so.bf16_bits_from_f64(f.astype(np.float64))
    theirs = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # +0 / -0 compare by value
    same = (ours == theirs) | ((ours & 0x7FFF) == 0) & ((theirs & 0x7FFF) == 0)
    assert np.all(same)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    fin = np.isfinite(h)
    ref16 = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    assert np.array_equal(so.fp16_bits_to_f64(bits)[fin], ref16[fin])
    refb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    finb = np.isfinite(refb)
    assert np.array_equal(so.bf16_bits_to_f64(bits)[finb], refb[finb])


def test_moe_oracle_matches_per_slot_products():
    k, n, topk, E = 32, 16, 3, 5
    mats = [synth.random_matrix(n, k, 6 + (e % 3), seed=(10, e, 0)) for e in range(E)]
    Ws = [so.decode_matrix(w.codes, n, k, w.bd, w.codebook, w.radius, w.perm) for w in mats]
    ids = np.array([0, 2, 4, 1, 2, 3], dtype=np.int32)  # 2 tokens x top-3
    x_tok = synth.random_activations(2, k, seed=(10, 9, 0))
    y = so.moe_linear(x_tok, ids, topk, False, Ws)
    for q, e in enumerate(ids):
        assert np.array_equal(y[q], so.linear(x_tok[q // topk:q // topk + 1], Ws[e])[0])
    x_slot = synth.random_activations(6, k, seed=(10, 8, 0))
    y = so.moe_linear(x_slot, ids, topk, True, Ws)
    for q, e in enumerate(ids):
        assert np.array_equal(y[q], so.linear(x_slot[q:q + 1], Ws[e])[0])


def test_round_to_bf16_hand_values():
    # 1 + 2**-8 is halfway between 1 and 1 + 2**-7: ties to even -> 1
    assert so.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    # 1 + 3*2**-8 is halfway between 1+2**-7 and 1+2**-6: ties to even -> 1+2**-6
    assert so.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert so.round_to_bf16(np.array([1 + 2 ** -8 + 2 ** -30]))[0] == 1 + 2 ** -7
    assert so.round_to_bf16(np.array([-(1 + 2 ** -8 + 2 ** -30)]))[0] == -(1 + 2 ** -7)
