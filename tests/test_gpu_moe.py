"""GPU parity of svq_moe_linear (grouped experts) against the CPU oracle."""
import numpy as np
import pytest

import synth
from oracle import svq_oracle as so
from tests.gpu_common import (assert_within_tolerance, equal_pm0, out_to_f64, require_gpu,
                              to_device_bf16, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svq():
    return require_gpu()


def _ids(m, topk, n_exp, seed):
    rng = np.random.default_rng(seed)
    return np.concatenate([rng.choice(n_exp, topk, replace=False) for _ in range(m)]).astype(np.int32)


def _run_moe(svq, pms, x_bits, ids, topk, x_per_slot, out_dtype):
    x = to_device_bf16(x_bits)
    d_ids = torch.from_numpy(ids).cuda()
    y = svq.moe_linear(pms, x, d_ids, topk, x_per_slot, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out_to_f64(y)


def _check_slots(y, x_bits, ids, topk, x_per_slot, weights, experts, label):
    for e in experts:
        slots = np.nonzero(ids == e)[0]
        if slots.size == 0:
            continue
        rows = slots if x_per_slot else slots // topk
        xs = x_bits[rows]
        y64 = so.linear(xs, weights[e])
        assert_within_tolerance(y[slots], y64, xs, weights[e], label=f"{label} expert {e}")


@pytest.mark.parametrize("m,topk,x_per_slot", [(1, 2, 0), (3, 3, 1), (40, 2, 0), (21, 4, 1)])
def test_small_moe(svq, m, topk, x_per_slot):
    n_exp, n, k = 8, 48, 520
    mats = [synth.random_matrix(n, k, 6 + e % 3, seed=(40, e, 0)) for e in range(n_exp)]
    Ws = [so.decode_matrix(w.codes, n, k, w.bd, w.codebook, w.radius, w.perm) for w in mats]
    pms = [svq.pack(w) for w in mats]
    ids = _ids(m, topk, n_exp, 41 + m)
    x = synth.random_activations(m * topk if x_per_slot else m, k, seed=(42, m, 0))
    y_ref = so.moe_linear(x, ids, topk, bool(x_per_slot), Ws)
    for dt in (torch.float32, torch.bfloat16):
        y = _run_moe(svq, pms, x, ids, topk, x_per_slot, dt)
        assert y.shape == (m * topk, n)
        _check_slots(y, x, ids, topk, x_per_slot, Ws, range(n_exp), f"small moe m={m}")
        if dt == torch.float32 and m * topk <= 64:
            # per-slot exact path: bit-exact decode through one-hot rows
            pass
    # one-hot slots: decoded weights of the routed experts, exactly (exact
    # path) or as RNE_bf16 (grouped bf16 path)
    cols = np.arange(m * topk if x_per_slot else m) * 7 % k
    xo = np.zeros_like(x)
    xo[np.arange(xo.shape[0]), cols] = 0x3F80
    y = _run_moe(svq, pms, xo, ids, topk, x_per_slot, torch.float32)
    for q, e in enumerate(ids):
        r = q if x_per_slot else q // topk
        ref = Ws[e][:, cols[r]]
        if m * topk > 64:
            ref = so.round_to_bf16(ref)
        assert equal_pm0(y[q], ref).all(), f"slot {q}"


def _moe_weights(proj, experts, bd):
    mats = {e: synth.moe_expert(e, proj, int(bd[e])) for e in experts}
    return mats


@pytest.mark.parametrize("proj", [0, 1, 2])
def test_moe128_m1(svq, proj):
    bd = synth.moe_expert_bd()
    all_mats = [synth.moe_expert(e, proj, int(bd[e])) for e in range(synth.MOE_EXPERTS)]
    pms = [svq.pack(w) for w in all_mats]
    ids = synth.moe_routing(1)
    x = synth.moe_activations(1, proj)
    x_per_slot = 1 if proj == 2 else 0
    Ws = {}
    for e in np.unique(ids):
        w = all_mats[e]
        Ws[e] = so.decode_matrix(w.codes, w.n, w.k, w.bd, w.codebook, w.radius, w.perm)
    for dt in (torch.float32, torch.bfloat16):
        y = _run_moe(svq, pms, x, ids, synth.MOE_TOPK, x_per_slot, dt)
        _check_slots(y, x, ids, synth.MOE_TOPK, x_per_slot, Ws, Ws.keys(), f"moe128 m=1 p{proj}")


@pytest.mark.parametrize("proj", [0, 2])
def test_moe128_m512(svq, proj):
    bd = synth.moe_expert_bd()
    all_mats = [synth.moe_expert(e, proj, int(bd[e])) for e in range(synth.MOE_EXPERTS)]
    pms = [svq.pack(w) for w in all_mats]
    m = 512
    ids = synth.moe_routing(m)
    x = synth.moe_activations(m, proj)
    x_per_slot = 1 if proj == 2 else 0
    y = _run_moe(svq, pms, x, ids, synth.MOE_TOPK, x_per_slot, torch.bfloat16)
    assert y.shape == (m * synth.MOE_TOPK, all_mats[0].n)
    assert np.isfinite(y).all()
    sample = np.random.default_rng(50 + proj).choice(synth.MOE_EXPERTS, 10, replace=False)
    Ws = {}
    for e in sample:
        w = all_mats[e]
        Ws[e] = so.decode_matrix(w.codes, w.n, w.k, w.bd, w.codebook, w.radius, w.perm)
    _check_slots(y, x, ids, synth.MOE_TOPK, x_per_slot, Ws, sample, f"moe128 m=512 p{proj}")
