"""Seeded generators for the synthetic SVQ workloads.

Every input is synthetic; no trained weights or datasets are used.  The
shapes follow a 4B-class dense decoder layer (hidden 2560, q 4096, k/v 1024,
FFN 9728) and a 30B-A3B-class MoE FFN (128 experts, hidden 2048, expert FFN
768, top-8 routing), as the SAGE paper's efficiency and accuracy studies use
those model shapes ("SAGE: Pushing 2-Bit Vector-Quantized LLMs toward
Real-World Usability", Fig. 1, Fig. 5, Table 3).

Recipe (stated once, used everywhere):

* One ``numpy.random.Generator`` per matrix, seeded with
  ``SeedSequence([workload_id, matrix_id, seed])``.  Draw order inside it:
  codes, then codebook, then permutation, then hot channels, then x.
* Codes: the canonical bitstream is ``n*k*9/32`` uniform random bytes.  Every
  bit of an 18-bit field is then an independent fair coin, so each field is
  uniform over ``[0, 2**18)``; no packing arithmetic is needed here.
* Direction codebook: ``2**bd`` rows of 8 ``|N(0,1)|`` draws, each row
  divided by its L2 norm in float64, then rounded to fp16 (round to nearest
  even, subnormals kept).  Signs are stored apart from the direction (SAGE
  paper, Fig. 2 caption), so the rows live in the positive orthant.
* Radius table: ``2**br`` values ``0.02*sqrt(8)*g`` with ``g`` geometrically
  spaced over ``[0.5, 4.0]`` (both ends included, ascending), rounded to fp16.
* Permutation: ``rng.permutation(k)`` (int32); slot ``p`` takes channel
  ``perm[p]``.
* Activations: N(0,1) in float32, ``round(0.01*k)`` channels (chosen without
  replacement, shared by all rows) scaled by 10 in float32, then rounded to
  bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# Workload ids used in the seed recipe.
WL_SINGLE = 0
WL_LAYER = 1
WL_LAYER_SMALL_BATCH = 2
WL_PREFILL = 3
WL_MOE = 4
WL_DECODE = 5

DENSE_LAYER_SHAPES: List[Tuple[str, int, int]] = [
    ("q", 4096, 2560),
    ("k", 1024, 2560),
    ("v", 1024, 2560),
    ("o", 2560, 4096),
    ("gate", 9728, 2560),
    ("up", 9728, 2560),
    ("down", 2560, 9728),
]
PREFILL_SHAPES: List[Tuple[str, int, int]] = [
    ("gate", 9728, 2560),
    ("up", 9728, 2560),
    ("down", 2560, 9728),
]
MOE_SHAPES: List[Tuple[str, int, int]] = [
    ("gate", 768, 2048),
    ("up", 768, 2048),
    ("down", 2048, 768),
]
MOE_EXPERTS = 128
MOE_TOPK = 8

# Named workloads (sizes only; the generators below build them).
WORKLOADS: Dict[str, dict] = {
    "single_512x1024_m1": dict(kind="dense", shapes=[("w", 512, 1024)], m=1, bd=8),
    "layer4b_m1": dict(kind="dense", shapes=DENSE_LAYER_SHAPES, m=1, bd=None),
    "layer4b_m4": dict(kind="dense", shapes=DENSE_LAYER_SHAPES, m=4, bd=None),
    "layer4b_m16": dict(kind="dense", shapes=DENSE_LAYER_SHAPES, m=16, bd=None),
    "prefill_m2048": dict(kind="dense", shapes=PREFILL_SHAPES, m=2048, bd=7),
    "moe128_m1": dict(kind="moe", shapes=MOE_SHAPES, m=1),
    "moe128_m512": dict(kind="moe", shapes=MOE_SHAPES, m=512),
    # the encoder (the step before the packed path): one gate-shaped matrix
    "encode_gate_bd7": dict(kind="encode", shapes=[("gate", 9728, 2560)], m=0, bd=7),
    # the same with activation-weighted fitting, h = ESG energies of 2048
    # calibration tokens of the layer input
    "encode_weighted_gate_bd7": dict(kind="encode", shapes=[("gate", 9728, 2560)], m=0, bd=7,
                                     weighted=True),
    # calibration before encoding: ESG over 2048 tokens of the 2560-wide
    # layer input; ABS over the three splits of one gate-shaped matrix
    "esg_calib_t2048_k2560": dict(kind="esg", shapes=[("x", 2048, 2560)], m=2048),
    "abs_gate_3splits": dict(kind="abs", shapes=[("gate", 9728, 2560)], m=0, bds=(6, 7, 8)),
    # one decode step's linears: 36 layers of the seven 4B-class matrices at
    # batch 1, four dependent calls per layer, each layer its own matrices;
    # beside it the first-token pass: the same calls over a 128-token prompt
    "decode4b_36l": dict(kind="decode", shapes=DENSE_LAYER_SHAPES, m=1, layers=36,
                         prefill_tokens=128),
}


@dataclasses.dataclass
class MatrixInputs:
    """Canonical inputs for one SVQ-coded matrix (host arrays)."""

    name: str
    n: int  # output rows
    k: int  # input channels
    bd: int  # direction-index bits
    br: int  # radius-index bits (bd + br == 10)
    codes: np.ndarray  # uint8, n*k*9//32 bytes, canonical LSB-first bitstream
    codebook: np.ndarray  # uint16 [2**bd, 8] fp16 bit patterns
    radius: np.ndarray  # uint16 [2**br] fp16 bit patterns
    perm: np.ndarray  # int32 [k]; slot p takes channel perm[p]

    @property
    def nbytes_codes(self) -> int:
        return int(self.codes.size)


def code_bytes(n: int, k: int) -> int:
    """Bytes of the canonical bitstream: n*(k/8) fields of 18 bits."""
    bits = n * (k // 8) * 18
    return (bits + 7) // 8


def n_hot_channels(k: int) -> int:
    return int(round(0.01 * k))


def _rng(workload_id: int, matrix_id: int, seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload_id, matrix_id, seed]))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even, via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def make_codebook(rng: np.random.Generator, bd: int) -> np.ndarray:
    rows = np.abs(rng.standard_normal((1 << bd, 8)))
    rows = rows / np.sqrt(np.sum(rows * rows, axis=1, keepdims=True))
    return rows.astype(np.float16).view(np.uint16)


def make_radius_table(br: int) -> np.ndarray:
    g = np.geomspace(0.5, 4.0, 1 << br)
    return (0.02 * math.sqrt(8.0) * g).astype(np.float16).view(np.uint16)


def make_activations(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """bf16 bit patterns [m, k]: N(0,1), 1% of channels x10."""
    hot = rng.choice(k, n_hot_channels(k), replace=False)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, hot] *= np.float32(10.0)
    return bf16_bits_from_f32(x)


def _draw_matrix(rng: np.random.Generator, name: str, n: int, k: int, bd: int) -> MatrixInputs:
    if k % 8 != 0:
        raise ValueError("k must be a multiple of 8")
    nbytes = code_bytes(n, k)
    codes = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    codebook = make_codebook(rng, bd)
    perm = rng.permutation(k).astype(np.int32)
    return MatrixInputs(name=name, n=n, k=k, bd=bd, br=10 - bd, codes=codes,
                        codebook=codebook, radius=make_radius_table(10 - bd), perm=perm)


def make_matrix(workload_id: int, matrix_id: int, name: str, n: int, k: int,
                bd: Optional[int] = None, seed: int = 0,
                bd_choices: Sequence[int] = (6, 7, 8)) -> Tuple[MatrixInputs, np.random.Generator]:
    """One matrix.  If ``bd`` is None it is drawn first from ``bd_choices``.

    Returns the matrix and its generator (positioned after the permutation),
    so that callers can go on to draw hot channels and activations from it.
    """
    rng = _rng(workload_id, matrix_id, seed)
    if bd is None:
        bd = int(rng.choice(np.asarray(bd_choices)))
    return _draw_matrix(rng, name, n, k, bd), rng


def random_matrix(n: int, k: int, bd: int, seed: Sequence[int] = (9, 0, 0)) -> MatrixInputs:
    """A matrix of any shape for tests (same recipe, caller-chosen seed)."""
    rng = np.random.default_rng(np.random.SeedSequence(list(seed)))
    return _draw_matrix(rng, "w", n, k, bd)


def random_activations(m: int, k: int, seed: Sequence[int] = (9, 1, 0)) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(list(seed)))
    return make_activations(rng, m, k)


def single_matrix(seed: int = 0, m: int = 1) -> Tuple[MatrixInputs, np.ndarray]:
    """512 x 1024, bd=8, with its M x 1024 activations."""
    w, rng = make_matrix(WL_SINGLE, 0, "w", 512, 1024, bd=8, seed=seed)
    return w, make_activations(rng, m, 1024)


def dense_layer(seed: int = 0) -> Tuple[List[MatrixInputs], List[np.ndarray]]:
    """The seven 4B-class decoder-layer matrices (bd drawn per matrix) and
    their batch-1 activations."""
    mats, xs = [], []
    for j, (name, n, k) in enumerate(DENSE_LAYER_SHAPES):
        w, rng = make_matrix(WL_LAYER, j, name, n, k, bd=None, seed=seed)
        mats.append(w)
        xs.append(make_activations(rng, 1, k))
    return mats, xs


# The linear calls of one decoder layer in their data-dependence order:
# indices into DENSE_LAYER_SHAPES of the matrices that share one input
# (q/k/v read the attention input, o the attention output, gate/up the MLP
# input, down the gated product).
DECODE_CALLS: Tuple[Tuple[int, ...], ...] = ((0, 1, 2), (3,), (4, 5), (6,))
DECODE_LAYERS = 36


def decode_stack(layers: int = DECODE_LAYERS, seed: int = 0
                 ) -> List[Tuple[List[MatrixInputs], List[np.ndarray]]]:
    """Per layer: its seven matrices (bd drawn per matrix, distinct codes,
    codebooks and permutations in every layer) and one batch-1 input per
    call of DECODE_CALLS."""
    stack = []
    for layer in range(layers):
        mats = [make_matrix(WL_DECODE, 7 * layer + j, f"l{layer}.{name}", n, k, bd=None,
                            seed=seed)[0]
                for j, (name, n, k) in enumerate(DENSE_LAYER_SHAPES)]
        xs = [make_activations(_rng(WL_DECODE, 1000 + 4 * layer + c, seed), 1, mats[call[0]].k)
              for c, call in enumerate(DECODE_CALLS)]
        stack.append((mats, xs))
    return stack


PREFILL_TOKENS = 128


def prompt_activations(layer: int, ks: Sequence[int], tokens: int = PREFILL_TOKENS,
                       seed: int = 0) -> List[np.ndarray]:
    """The first-token (prompt) pass of the decode stack: one [tokens, k]
    input per call of DECODE_CALLS of ``layer``, ``ks[c]`` the input width of
    call c (same distribution as every other activation here)."""
    return [make_activations(_rng(WL_DECODE, 5000 + 4 * layer + c, seed * 65536 + tokens), tokens, ks[c])
            for c in range(len(DECODE_CALLS))]


def call_input_widths(mats: Sequence["MatrixInputs"]) -> List[int]:
    """Input width k of each call of DECODE_CALLS for one layer's matrices."""
    return [mats[call[0]].k for call in DECODE_CALLS]


def dense_layer_activations(m: int) -> List[np.ndarray]:
    """Small-batch activations for the seven layer matrices (same matrices as
    :func:`dense_layer`)."""
    out = []
    for j, (_, _, k) in enumerate(DENSE_LAYER_SHAPES):
        rng = _rng(WL_LAYER_SMALL_BATCH, j, m)
        out.append(make_activations(rng, m, k))
    return out


def prefill_set(m: int = 2048, seed: int = 0,
                shapes: Sequence[Tuple[str, int, int]] = PREFILL_SHAPES
                ) -> Tuple[List[MatrixInputs], List[np.ndarray]]:
    mats, xs = [], []
    for j, (name, n, k) in enumerate(shapes):
        w, rng = make_matrix(WL_PREFILL, j, name, n, k, bd=7, seed=seed)
        mats.append(w)
        xs.append(make_activations(rng, m, k))
    return mats, xs


def moe_expert_bd(seed: int = 0) -> np.ndarray:
    """Per-expert direction bits, uniform over {6,7,8}; shared by the
    expert's gate, up and down matrices."""
    rng = _rng(WL_MOE, 998, seed)
    return rng.integers(6, 9, size=MOE_EXPERTS).astype(np.int32)


def moe_expert(expert: int, proj: int, bd: int, seed: int = 0,
               shapes: Sequence[Tuple[str, int, int]] = MOE_SHAPES) -> MatrixInputs:
    name, n, k = shapes[proj]
    rng = _rng(WL_MOE, expert * 3 + proj, seed)
    return _draw_matrix(rng, f"e{expert}.{name}", n, k, bd)


def moe_routing(m: int, n_experts: int = MOE_EXPERTS, topk: int = MOE_TOPK) -> np.ndarray:
    """int32 [m*topk]: for each token, topk distinct experts drawn uniformly."""
    rng = _rng(WL_MOE, 999, m)
    ids = np.empty((m, topk), dtype=np.int32)
    for t in range(m):
        ids[t] = rng.choice(n_experts, topk, replace=False)
    return ids.reshape(-1)


def moe_activations(m: int, proj: int, topk: int = MOE_TOPK,
                    shapes: Sequence[Tuple[str, int, int]] = MOE_SHAPES) -> np.ndarray:
    """gate/up read one row per token ([m, k]); down reads one row per routed
    slot ([m*topk, k])."""
    _, _, k = shapes[proj]
    rows = m * topk if proj == 2 else m
    rng = _rng(WL_MOE, 997 - proj, m)
    return make_activations(rng, rows, k)
