"""CPU oracle for the calibration steps before encoding: Energy-Stratified
Grouping (ESG) and Adaptive Bit Split (ABS).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP
library never calls it and it imports nothing from the library.

What the pages fix ("SAGE: Pushing 2-Bit Vector-Quantized LLMs toward
Real-World Usability"):

* Abstract and Fig. 2 caption: ESG measures channel energy on calibration
  activations and builds every 8-channel subvector from channels of
  different energy tiers; ABS encodes a matrix under each direction/radius
  split of the 10 index bits and keeps the split whose activation-weighted
  reconstruction error is lowest.
* Fig. 3 and Fig. 4 captions: the energy is per input channel and enters the
  weighting through an exponent (gamma).

What they leave open, and the readings taken here (the library's contract):

* Energy of channel j: the mean of x[t, j]**2 over the T calibration tokens,
  summed in float64 in token order 0..T-1 (each square of a bf16 value is
  exact) and divided by T once at the end.
* Tiers: the channels sorted by energy, largest first, equal energies in
  ascending channel order; with C = k/8, tier l holds ranks
  [l*C, (l+1)*C).  Subvector c takes lane l from tier l: permuted slot
  8c + l holds the channel of rank l*C + c.  So every subvector has one
  channel of each tier, and the lane of a channel is its tier.
* Fitting weights: h[j] = energy[j] ** gamma; the caller forms them (gamma
  is the caller's hyper-parameter).
* Activation-weighted reconstruction error of row i:
  sum over subvectors c (in order) of sum over lanes l (in order) of
  (v[l] - w_hat[l])**2 * h[perm[8c + l]], where v is the float32 weight and
  w_hat the decoded weight (exact in float64), all in float64 without fused
  multiply-adds; the matrix error is the sum of the row errors in row order.
* ABS: the candidate (in the caller's order) with the smallest matrix
  error, the first one on ties.  Every candidate is coded by the plain
  encoder rule of ``oracle/svq_encoder.py`` or, on request, by its
  activation-weighted fitting rule with the same h.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from oracle.svq_encoder import encode_matrix, encode_matrix_weighted, gather_subvectors
from oracle.svq_oracle import bf16_bits_to_f64, decode_permuted


def esg_energy(x_bits: np.ndarray) -> np.ndarray:
    """Per-channel mean square of bf16 calibration activations [T, k]
    (float64 [k]), token-order float64 sum, one division."""
    x = bf16_bits_to_f64(np.asarray(x_bits))
    if x.ndim != 2 or x.shape[0] < 1:
        raise ValueError("need at least one calibration token")
    acc = x[0] * x[0]
    for t in range(1, x.shape[0]):
        acc = acc + x[t] * x[t]
    return acc / float(x.shape[0])


def esg_rank_order(energy: np.ndarray) -> np.ndarray:
    """Channels by decreasing energy, equal energies by increasing index."""
    e = np.asarray(energy, dtype=np.float64)
    if not np.all(np.isfinite(e)):
        raise ValueError("energies must be finite")
    return np.array(sorted(range(e.size), key=lambda j: (-e[j], j)), dtype=np.int64)


def esg_perm(energy: np.ndarray) -> np.ndarray:
    """The ESG permutation (int32 [k]): slot 8c + l <- rank l*C + c."""
    k = int(np.asarray(energy).size)
    if k % 8 or k == 0:
        raise ValueError("k must be a positive multiple of 8")
    order = esg_rank_order(energy)
    C = k // 8
    perm = np.empty(k, dtype=np.int32)
    for c in range(C):
        for lane in range(8):
            perm[8 * c + lane] = order[lane * C + c]
    return perm


def weighted_error_rows(w: np.ndarray, perm: np.ndarray, h: np.ndarray, codes: np.ndarray,
                        bd: int, codebook_bits: np.ndarray, radius_bits: np.ndarray) -> np.ndarray:
    """Activation-weighted reconstruction error of every row (float64 [n]);
    ``codes`` are the unpacked uint32 codes [n, k/8]."""
    v = gather_subvectors(w, perm)                              # [n, C, 8] float64
    n, C, _ = v.shape
    wh = decode_permuted(codes, bd, codebook_bits, radius_bits).reshape(n, C, 8)
    hp = np.asarray(h, dtype=np.float64)[np.asarray(perm, dtype=np.int64)].reshape(C, 8)
    d = v - wh
    e = (d[:, :, 0] * d[:, :, 0]) * hp[None, :, 0]              # [n, C], lane order
    for lane in range(1, 8):
        e = e + (d[:, :, lane] * d[:, :, lane]) * hp[None, :, lane]
    row = e[:, 0].copy()
    for c in range(1, C):
        row = row + e[:, c]
    return row


def total_in_order(values: np.ndarray) -> float:
    """Sequential float64 sum in index order."""
    tot = 0.0
    for v in np.asarray(values, dtype=np.float64):
        tot = tot + float(v)
    return tot


def abs_select(w: np.ndarray, perm: np.ndarray, h: np.ndarray,
               candidates: Sequence[Tuple[int, np.ndarray, np.ndarray]], weighted_fit: bool = False):
    """(chosen index, errors [len(candidates)], codes of every candidate):
    each candidate (bd, codebook bits, radius bits) is encoded -- by the
    plain rule, or by activation-weighted fitting with the same h when
    ``weighted_fit`` -- and scored by its activation-weighted reconstruction
    error."""
    errs, all_codes = [], []
    for bd, cb, rad in candidates:
        if weighted_fit:
            codes = encode_matrix_weighted(w, perm, h, bd, cb, rad)
        else:
            codes = encode_matrix(w, perm, bd, cb, rad)
        errs.append(total_in_order(weighted_error_rows(w, perm, h, codes, bd, cb, rad)))
        all_codes.append(codes)
    errs = np.array(errs, dtype=np.float64)
    return int(np.argmin(errs)), errs, all_codes


__all__ = ["esg_energy", "esg_rank_order", "esg_perm", "weighted_error_rows", "total_in_order",
           "abs_select"]
