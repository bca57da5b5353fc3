"""CPU oracle for the SVQ decode-and-multiply path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP
library never calls it and it imports nothing from the library; the only
code the two sides share is the seeded input generator in ``synth/``.

What it computes.  The page cited throughout is the SAGE paper, "SAGE:
Pushing 2-Bit Vector-Quantized LLMs toward Real-World Usability":

* Fig. 2 caption: each subvector of 8 weights is coded by sign bits, a
  direction index into a codebook and a quantized radius; a per-matrix split
  of the index bits, 18 bits per 8 weights in total.
* Table 1 (SPHQuant row, 2.25 bits per weight): 18 bits / 8 weights.
* Fig. 1 and Fig. 5 captions: weights are rebuilt on demand, i.e. the
  product uses the decoded weights directly.
* Fig. 6 caption: the kernel's subvector input is eight reordered (permuted)
  activations.

Readings where the pages are silent (each is the library's contract too):

* Field order inside a code, LSB first: bits 0-7 signs, then ``bd`` direction
  bits, then ``br = 10 - bd`` radius bits.
* Sign bit ``l`` of a code applies to lane ``l`` of its subvector; 1 means
  negative.
* Code ``g = i*(k/8) + c`` (row i, subvector c) sits at stream bits
  ``[18g, 18g+18)``; stream bit ``t`` is bit ``t % 8`` of byte ``t // 8``.
* Gather permutation: permuted slot ``p`` holds input channel ``perm[p]``, so
  ``W[i, perm[p]] = Wp[i, p]``.
* One codebook and one radius table per matrix; no per-row scales.

Decoded weight: ``Wp[i, 8c+l] = R[r] * (-1)**s_l * D[d][l]``.  R and D are
fp16, so the product has at most 22 significant bits and is exact in float32
and float64; the oracle forms it in float64 and checks that a float32 cast
is lossless.  The product ``y = x W^T`` is evaluated in float64 (BLAS dgemm)
on the exact bf16 values of x.

Every function here is pinned by ``tests/test_oracle.py`` against hand-worked
values (``tests/golden/``), closed forms, invariants and a pure-Python brute
force (``oracle/bruteforce.py``).
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

FIELD_BITS = 18
SIGN_BITS = 8
INDEX_BITS = 10


# --------------------------------------------------------------------------
# Scalar formats (plain definitions; pinned against torch's CPU casts)
# --------------------------------------------------------------------------

def fp16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): the top half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range.  For a
    value v = m * 2**e with m in [0.5, 1) the spacing of bf16 numbers is
    2**(e-8); below the normal range (e <= -126) it stays 2**-133.  Dividing by
    a power of two and ``np.rint`` (ties to even) are exact in float64, so the
    result is the correctly rounded bf16 value, returned as float64.
    Overflow gives +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    finite = np.isfinite(v) & (v != 0)
    _, e = np.frexp(v[finite])
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(v[finite] / q) * q
    big = np.abs(r) > 3.3895313892515355e38  # largest finite bfloat16
    r[big] = np.copysign(np.inf, r[big])
    out[finite] = r
    return out


def bf16_bits_from_f64(v) -> np.ndarray:
    """Round float64 to bfloat16 and return the bit patterns (uint16)."""
    r = round_to_bf16(v).astype(np.float32)  # exact: r is a bf16 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# Canonical bitstream
# --------------------------------------------------------------------------

def stream_bytes(n: int, k: int) -> int:
    return (n * (k // 8) * FIELD_BITS + 7) // 8


def unpack_codes(stream: np.ndarray, n: int, k: int) -> np.ndarray:
    """Canonical bitstream -> uint32 codes [n, k/8].

    Code g occupies stream bits [18g, 18g+18), stream bit t being bit t % 8
    of byte t // 8 (LSB first).  Bit offsets 18g mod 8 are 0, 2, 4 or 6, so a
    field lies within 3 consecutive bytes.
    """
    c = k // 8
    count = n * c
    need = stream_bytes(n, k)
    buf = np.zeros(need + 3, dtype=np.uint32)
    buf[:need] = np.asarray(stream, dtype=np.uint8)[:need]
    start = np.arange(count, dtype=np.int64) * FIELD_BITS
    byte = start // 8
    shift = (start % 8).astype(np.uint32)
    word = buf[byte] | (buf[byte + 1] << np.uint32(8)) | (buf[byte + 2] << np.uint32(16))
    codes = (word >> shift) & np.uint32((1 << FIELD_BITS) - 1)
    return codes.reshape(n, c)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """uint32 codes [n, c] (each < 2**18) -> canonical bitstream (uint8)."""
    codes = np.asarray(codes, dtype=np.uint64).reshape(-1)
    if codes.size and int(codes.max()) >= (1 << FIELD_BITS):
        raise ValueError("code does not fit in 18 bits")
    count = codes.size
    nbytes = (count * FIELD_BITS + 7) // 8
    out = np.zeros(nbytes + 3, dtype=np.uint64)
    start = np.arange(count, dtype=np.int64) * FIELD_BITS
    byte = start // 8
    shifted = codes << (start % 8).astype(np.uint64)  # < 2**24
    for b in range(3):
        np.add.at(out, byte + b, (shifted >> np.uint64(8 * b)) & np.uint64(0xFF))
    if out.max(initial=0) > 0xFF:
        raise AssertionError("fields overlapped while packing")
    return out[:nbytes].astype(np.uint8)


def split_fields(codes: np.ndarray, bd: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """18-bit codes -> (signs, direction index, radius index).

    Bits 0-7 are the sign byte, bits 8..8+bd-1 the direction index and bits
    8+bd..17 the radius index, in the order the Fig. 2 caption lists them.
    """
    _check_split(bd)
    codes = np.asarray(codes, dtype=np.uint32)
    s = codes & np.uint32(0xFF)
    d = (codes >> np.uint32(SIGN_BITS)) & np.uint32((1 << bd) - 1)
    r = codes >> np.uint32(SIGN_BITS + bd)
    return s, d, r


def join_fields(s, d, r, bd: int) -> np.ndarray:
    """Inverse of :func:`split_fields`."""
    _check_split(bd)
    s = np.asarray(s, dtype=np.uint32)
    d = np.asarray(d, dtype=np.uint32)
    r = np.asarray(r, dtype=np.uint32)
    if np.any(s > 0xFF) or np.any(d >= (1 << bd)) or np.any(r >= (1 << (INDEX_BITS - bd))):
        raise ValueError("field out of range")
    return s | (d << np.uint32(SIGN_BITS)) | (r << np.uint32(SIGN_BITS + bd))


def _check_split(bd: int) -> None:
    if not (1 <= bd <= 9):
        raise ValueError("bd must leave at least one radius bit")


# --------------------------------------------------------------------------
# Decode (reconstruction) and the product
# --------------------------------------------------------------------------

def decode_permuted(codes: np.ndarray, bd: int, codebook_bits: np.ndarray,
                    radius_bits: np.ndarray) -> np.ndarray:
    """Decoded weights in permuted order, float64 [n, k].

    Wp[i, 8c+l] = R[r_ic] * (-1)**(bit l of s_ic) * D[d_ic][l].
    """
    codes = np.asarray(codes)
    n, c = codes.shape
    s, d, r = split_fields(codes, bd)
    D = fp16_bits_to_f64(np.asarray(codebook_bits).reshape(1 << bd, 8))
    R = fp16_bits_to_f64(np.asarray(radius_bits).reshape(1 << (INDEX_BITS - bd)))
    lanes = np.arange(8, dtype=np.uint32)
    neg = (s[:, :, None] >> lanes) & np.uint32(1)  # [n, c, 8]
    sign = 1.0 - 2.0 * neg.astype(np.float64)
    wp = R[r][:, :, None] * sign * D[d]  # [n, c, 8]
    wp = wp.reshape(n, c * 8)
    if not np.array_equal(wp.astype(np.float32).astype(np.float64), wp):
        raise AssertionError("decoded weight is not exact in float32")
    return wp


def unpermute(wp: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Permuted columns -> input-channel order: W[:, perm[p]] = Wp[:, p]."""
    perm = np.asarray(perm, dtype=np.int64)
    k = wp.shape[1]
    if perm.shape != (k,) or not np.array_equal(np.sort(perm), np.arange(k)):
        raise ValueError("perm is not a permutation of range(k)")
    w = np.empty_like(wp)
    w[:, perm] = wp
    return w


def decode_matrix(stream, n: int, k: int, bd: int, codebook_bits, radius_bits,
                  perm) -> np.ndarray:
    """Dense decoded matrix W (float64 [n, k], input-channel order)."""
    codes = unpack_codes(stream, n, k)
    return unpermute(decode_permuted(codes, bd, codebook_bits, radius_bits), perm)


def linear(x_bits: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T in float64; x given as bf16 bit patterns [m, k]."""
    x = bf16_bits_to_f64(x_bits).reshape(-1, w.shape[1])
    return x @ w.T


def linear_from_inputs(mat, x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(y64, W) for a ``synth.MatrixInputs``-like object."""
    w = decode_matrix(mat.codes, mat.n, mat.k, mat.bd, mat.codebook, mat.radius, mat.perm)
    return linear(x_bits, w), w


def abs_bound(x_bits: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum_j |W_ij| |x_mj| for every output element (float64 [m, n])."""
    x = np.abs(bf16_bits_to_f64(x_bits).reshape(-1, w.shape[1]))
    return x @ np.abs(w).T


def tolerance(x_bits: np.ndarray, w: np.ndarray, rel: float = 8e-3,
              atol: float = 1e-6) -> np.ndarray:
    """Per-element bound |y - y_ref| <= rel * sum_j |W_ij||x_j| + atol."""
    return rel * abs_bound(x_bits, w) + atol


def moe_linear(x_bits: np.ndarray, expert_ids: np.ndarray, topk: int,
               x_per_slot: bool, weights: Sequence[Optional[np.ndarray]]) -> np.ndarray:
    """Grouped expert product, one output row per routed slot.

    Slot ``q = t*topk + j`` uses expert ``expert_ids[q]``; its input row is
    ``x[t]`` (``x_per_slot`` False: gate/up share the token's row) or ``x[q]``
    (``x_per_slot`` True: down reads the slot's own row).  ``weights[e]`` is
    the dense decoded matrix of expert e (only the routed ones are needed).
    Returns float64 [m*topk, n].
    """
    ids = np.asarray(expert_ids, dtype=np.int64).reshape(-1)
    x = bf16_bits_to_f64(x_bits)
    k = x.shape[1]
    n = next(w.shape[0] for w in weights if w is not None)
    y = np.zeros((ids.size, n), dtype=np.float64)
    for e in np.unique(ids):
        slots = np.nonzero(ids == e)[0]
        rows = slots if x_per_slot else slots // topk
        y[slots] = x[rows].reshape(-1, k) @ weights[e].T
    return y
