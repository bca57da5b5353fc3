"""CPU oracle for the SVQ encoder (float weights -> 18-bit codes).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP
library never calls it and it imports nothing from the library.

What it computes.  "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward
Real-World Usability", Fig. 2 caption: spherical vector quantization codes
each 8-weight subvector (taken along the channel permutation) by its signs,
a direction index into a codebook of unit directions and a quantized radius,
18 bits per subvector.  The pages do not spell out how a subvector is mapped
to its code; the readings taken here (each is the library's contract too):

* Subvector c of row i is ``v[l] = W[i, perm[8c + l]]`` (the same gather as
  the decode side).
* Sign bit l = the IEEE sign bit of ``v[l]`` (1 for negative numbers and for
  -0.0), so that signs round-trip exactly through the decode.
* Direction index d = the codebook row with the largest inner product with
  ``|v|`` (the codebook directions lie in the positive orthant and have unit
  norm, so this is the direction of largest cosine); ties go to the smaller
  index.
* Radius index r = the radius-table entry nearest to the Euclidean norm of
  ``v``; ties go to the smaller index.  The table must be strictly
  increasing, so "nearest" is "number of midpoints (R[t] + R[t+1]) / 2 that
  lie strictly below the norm".

Arithmetic (fixed so that a GPU implementation can take the same integer
decisions bit for bit): float64 throughout.  The products ``|v_l| * D[j][l]``
(float32 x fp16) and the squares ``v_l**2`` are exact in float64; the eight
terms of each score and of the squared norm are added one at a time in lane
order 0..7, with no fused multiply-add.  The radius decision compares the
squared norm with the squared midpoints (both sides of each comparison are
exact float64 values except for the rounding of the sequential sum), which
avoids a square root.
"""
from __future__ import annotations

import numpy as np

from oracle.svq_oracle import INDEX_BITS, SIGN_BITS, fp16_bits_to_f64, join_fields, pack_codes


def gather_subvectors(w: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Permuted weights, float64 [n, k/8, 8]: ``[i, c, l] = W[i, perm[8c + l]]``."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    perm = np.asarray(perm, dtype=np.int64)
    if k % 8 or perm.shape != (k,) or not np.array_equal(np.sort(perm), np.arange(k)):
        raise ValueError("perm must be a permutation of range(k), k a multiple of 8")
    return w[:, perm].astype(np.float64).reshape(n, k // 8, 8)


def radius_midpoints_sq(radius_bits: np.ndarray) -> np.ndarray:
    """Squared midpoints between consecutive radii (exact in float64)."""
    R = fp16_bits_to_f64(radius_bits)
    if R.size < 2 or not np.all(np.isfinite(R)) or not np.all(np.diff(R) > 0) or R[0] < 0:
        raise ValueError("radius table must be finite, non-negative and strictly increasing")
    mid = (R[:-1] + R[1:]) / 2.0  # 12 significant bits at most: exact
    return mid * mid              # 24 significant bits: exact


def encode_fields(w: np.ndarray, perm: np.ndarray, bd: int, codebook_bits: np.ndarray,
                  radius_bits: np.ndarray):
    """(signs, direction index, radius index), each uint32 [n, k/8]."""
    v = gather_subvectors(w, perm)
    a = np.abs(v)
    # signs: bit l set when v[l] carries a negative sign bit
    neg = np.signbit(v).astype(np.uint32)
    s = np.zeros(v.shape[:2], dtype=np.uint32)
    for l in range(8):
        s |= neg[:, :, l] << np.uint32(l)
    # direction: sequential float64 sums of exact products, first maximum
    D = fp16_bits_to_f64(np.asarray(codebook_bits).reshape(1 << bd, 8))
    if not np.all(np.isfinite(D)):
        raise ValueError("codebook entries must be finite")
    score = a[:, :, 0, None] * D[None, None, :, 0]
    for l in range(1, 8):
        score = score + a[:, :, l, None] * D[None, None, :, l]
    d = np.argmax(score, axis=2).astype(np.uint32)  # first index of the maximum
    # radius: squared norm against squared midpoints
    nsq = a[:, :, 0] * a[:, :, 0]
    for l in range(1, 8):
        nsq = nsq + a[:, :, l] * a[:, :, l]
    msq = radius_midpoints_sq(np.asarray(radius_bits).reshape(1 << (INDEX_BITS - bd)))
    r = np.zeros(nsq.shape, dtype=np.uint32)
    for t in range(msq.size):
        r += (nsq > msq[t]).astype(np.uint32)
    return s, d, r


def encode_matrix(w: np.ndarray, perm: np.ndarray, bd: int, codebook_bits: np.ndarray,
                  radius_bits: np.ndarray) -> np.ndarray:
    """uint32 codes [n, k/8] (bits 0-7 signs, then bd direction bits, then
    the radius bits)."""
    s, d, r = encode_fields(w, perm, bd, codebook_bits, radius_bits)
    return join_fields(s, d, r, bd)


def encode_stream(w: np.ndarray, perm: np.ndarray, bd: int, codebook_bits: np.ndarray,
                  radius_bits: np.ndarray) -> np.ndarray:
    """Canonical LSB-first bitstream of :func:`encode_matrix`."""
    return pack_codes(encode_matrix(w, perm, bd, codebook_bits, radius_bits))


def _fit_weights(h: np.ndarray, perm: np.ndarray, C: int) -> np.ndarray:
    """Per-slot fitting weights, float64 [C, 8]: ``[c, l] = h[perm[8c + l]]``
    (the weight of the input channel that lane l of subvector c reads)."""
    h = np.asarray(h, dtype=np.float64)
    if h.shape != (8 * C,) or not np.all(np.isfinite(h)) or np.any(h < 0):
        raise ValueError("h must hold k finite, non-negative channel weights")
    return h[np.asarray(perm, dtype=np.int64)].reshape(C, 8)


def _weighted_magnitudes(hp: np.ndarray, a: np.ndarray) -> np.ndarray:
    """h_l |v_l|, float64 [n, C, 8], one rounding each."""
    return hp[None, :, :] * a


def _direction_sums(hw: np.ndarray, hp: np.ndarray, Dd: np.ndarray):
    """A_d = sum_l (h_l |v_l|) D_dl [n, C] and B_d = sum_l (h_l D_dl) D_dl
    [C] for one direction row Dd, lanes added in order 0..7."""
    A = hw[:, :, 0] * Dd[0]
    B = (hp[:, 0] * Dd[0]) * Dd[0]
    for l in range(1, 8):
        A = A + hw[:, :, l] * Dd[l]
        B = B + (hp[:, l] * Dd[l]) * Dd[l]
    return A, B


def _reduced_error(Rr: float, A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The code-dependent part of the weighted error of (d, r):
    (R_r R_r) B_d - (R_r + R_r) A_d."""
    return (Rr * Rr) * B[None, :] - (Rr + Rr) * A


def _improves(E: np.ndarray, best: np.ndarray) -> np.ndarray:
    """A later pair replaces the best one only when strictly smaller, so the
    first minimum in (d, r) order wins."""
    return E < best


def encode_fields_weighted(w: np.ndarray, perm: np.ndarray, h: np.ndarray, bd: int,
                           codebook_bits: np.ndarray, radius_bits: np.ndarray):
    """(signs, direction index, radius index), each uint32 [n, k/8], by
    activation-weighted fitting.

    What it follows: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward
    Real-World Usability", Abstract and Fig. 2 caption: ESG protects
    sensitive channels through fitting weighted by calibration activations.
    The pages give no formula; the reading taken here: with the weight
    h_l = h[perm[8c + l]] of each lane (h[j] e.g. the ESG energy of input
    channel j raised to an exponent), the code of subvector v is the one
    whose decoded weights w_hat minimise the weighted squared error
    sum_l h_l (v_l - w_hat_l)^2.

    * Signs: the IEEE sign bits of v, as in :func:`encode_fields`.  The
      directions and radii are non-negative, so a decoded weight with the
      sign of v_l is never farther from it than one with the other sign.
    * Direction d and radius r, searched jointly over every pair: with
      a_l = |v_l|, the error of (d, r) is
      sum_l h_l a_l^2 - 2 R_r A_d + R_r^2 B_d, where
      A_d = sum_l (h_l a_l) D_dl and B_d = sum_l (h_l D_dl) D_dl.  The first
      term does not depend on the code, so the pair minimising the reduced
      error E = (R_r R_r) B_d - (R_r + R_r) A_d is chosen; pairs are taken
      in order (d ascending, then r ascending) and the first minimum wins.

    Arithmetic (fixed so that the GPU takes the same decisions): float64;
    h_l a_l, A_d and B_d with one rounding per product and per addition,
    lanes added in order 0..7; E as written, no fused multiply-adds."""
    v = gather_subvectors(w, perm)                       # [n, C, 8]
    n, C, _ = v.shape
    a = np.abs(v)
    neg = np.signbit(v).astype(np.uint32)
    s = np.zeros((n, C), dtype=np.uint32)
    for l in range(8):
        s |= neg[:, :, l] << np.uint32(l)
    hp = _fit_weights(h, perm, C)                        # [C, 8]
    D = fp16_bits_to_f64(np.asarray(codebook_bits).reshape(1 << bd, 8))
    if not np.all(np.isfinite(D)):
        raise ValueError("codebook entries must be finite")
    rad = np.asarray(radius_bits).reshape(1 << (INDEX_BITS - bd))
    radius_midpoints_sq(rad)                             # same table checks as the plain rule
    R = fp16_bits_to_f64(rad)
    hw = _weighted_magnitudes(hp, a)
    best = None
    d_best = np.zeros((n, C), dtype=np.uint32)
    r_best = np.zeros((n, C), dtype=np.uint32)
    for d in range(1 << bd):
        A, B = _direction_sums(hw, hp, D[d])
        for r in range(R.size):
            E = _reduced_error(float(R[r]), A, B)
            if best is None:
                best = E
                continue
            better = _improves(E, best)
            best = np.where(better, E, best)
            d_best = np.where(better, np.uint32(d), d_best)
            r_best = np.where(better, np.uint32(r), r_best)
    return s, d_best, r_best


def encode_matrix_weighted(w: np.ndarray, perm: np.ndarray, h: np.ndarray, bd: int,
                           codebook_bits: np.ndarray, radius_bits: np.ndarray) -> np.ndarray:
    """uint32 codes [n, k/8] of :func:`encode_fields_weighted`."""
    s, d, r = encode_fields_weighted(w, perm, h, bd, codebook_bits, radius_bits)
    return join_fields(s, d, r, bd)


def encode_stream_weighted(w: np.ndarray, perm: np.ndarray, h: np.ndarray, bd: int,
                           codebook_bits: np.ndarray, radius_bits: np.ndarray) -> np.ndarray:
    """Canonical LSB-first bitstream of :func:`encode_matrix_weighted`."""
    return pack_codes(encode_matrix_weighted(w, perm, h, bd, codebook_bits, radius_bits))


__all__ = ["gather_subvectors", "radius_midpoints_sq", "encode_fields", "encode_matrix",
           "encode_stream", "encode_fields_weighted", "encode_matrix_weighted",
           "encode_stream_weighted", "SIGN_BITS"]
