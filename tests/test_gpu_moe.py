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


@pytest.mark.parametrize("proj", [0, 1, 2])
def test_moe128_m512(svq, proj):
    """Every routed slot of all 128 experts, both output types, against the
    oracle (each expert decoded once, then dropped)."""
    bd = synth.moe_expert_bd()
    all_mats = [synth.moe_expert(e, proj, int(bd[e])) for e in range(synth.MOE_EXPERTS)]
    pms = [svq.pack(w) for w in all_mats]
    m = 512
    ids = synth.moe_routing(m)
    x = synth.moe_activations(m, proj)
    x_per_slot = 1 if proj == 2 else 0
    ys = {dt: _run_moe(svq, pms, x, ids, synth.MOE_TOPK, x_per_slot, dt)
          for dt in (torch.bfloat16, torch.float32)}
    for y in ys.values():
        assert y.shape == (m * synth.MOE_TOPK, all_mats[0].n)
        assert np.isfinite(y).all()
    assert set(np.unique(ids)) == set(range(synth.MOE_EXPERTS))
    for e in range(synth.MOE_EXPERTS):
        w = all_mats[e]
        We = so.decode_matrix(w.codes, w.n, w.k, w.bd, w.codebook, w.radius, w.perm)
        for dt, y in ys.items():
            _check_slots(y, x, ids, synth.MOE_TOPK, x_per_slot, {e: We}, [e],
                         f"moe128 m=512 p{proj} {dt}")


@pytest.mark.parametrize("m,topk", [(3, 4), (40, 4)])
def test_moe_out_of_range_ids_are_skipped(svq, m, topk):
    """Slots whose expert id is outside [0, E) get zero rows (per-slot path
    for 12 slots, grouped path for 160); every other slot is unaffected."""
    n_exp, n, k = 6, 40, 520
    mats = [synth.random_matrix(n, k, 6 + e % 3, seed=(43, e, 0)) for e in range(n_exp)]
    Ws = [so.decode_matrix(w.codes, n, k, w.bd, w.codebook, w.radius, w.perm) for w in mats]
    pms = [svq.pack(w) for w in mats]
    ids = _ids(m, topk, n_exp, 44 + m)
    bad = np.arange(1, ids.size, 5)
    ids[bad] = np.where(bad % 2 == 0, -1, n_exp + 3)
    x = synth.random_activations(m, k, seed=(45, m, 0))
    for dt in (torch.float32, torch.bfloat16):
        y = _run_moe(svq, pms, x, ids, topk, 0, dt)
        assert np.all(y[bad] == 0)
        good = np.setdiff1d(np.arange(ids.size), bad)
        for e in range(n_exp):
            slots = good[ids[good] == e]
            if slots.size:
                assert_within_tolerance(y[slots], so.linear(x[slots // topk], Ws[e]), x[slots // topk],
                                        Ws[e], label=f"valid slots of expert {e}")


@pytest.mark.parametrize("k", [8, 200, 256])
def test_moe_grouped_single_half_unit(svq, k):
    """Grouped path (120 slots) for matrices of one 512-slot unit whose real
    slots end within its first half: every slice of the product is a half
    slice and the full-unit loop runs zero times.  Against the oracle, both
    output types, and one-hot columns against RNE_bf16 of the decoded
    weights."""
    n_exp, n, m, topk = 5, 40, 40, 3
    mats = [synth.random_matrix(n, k, 6 + e % 3, seed=(49, e, k)) for e in range(n_exp)]
    Ws = [so.decode_matrix(w.codes, n, k, w.bd, w.codebook, w.radius, w.perm) for w in mats]
    pms = [svq.pack(w) for w in mats]
    ids = _ids(m, topk, n_exp, 50 + k)
    x = synth.random_activations(m, k, seed=(51, k, 0))
    for dt in (torch.float32, torch.bfloat16):
        y = _run_moe(svq, pms, x, ids, topk, 0, dt)
        _check_slots(y, x, ids, topk, 0, Ws, range(n_exp), f"half-unit moe k={k} {dt}")
    cols = np.arange(m) * 5 % k
    xo = np.zeros_like(x)
    xo[np.arange(m), cols] = 0x3F80
    y = _run_moe(svq, pms, xo, ids, topk, 0, torch.float32)
    for q, e in enumerate(ids):
        assert equal_pm0(y[q], so.round_to_bf16(Ws[e][:, cols[q // topk]])).all(), f"slot {q}"


@pytest.mark.parametrize("x_per_slot", [0, 1])
def test_moe_grouped_strided_unaligned(svq, x_per_slot):
    """Grouped path (160 slots) with odd row strides for x and y (rows only
    2-byte aligned, so the element-wise load and store forms run), n not a
    multiple of 8 and k not a multiple of the unit width; the padding
    columns of y are left untouched."""
    n_exp, n, k, m, topk = 6, 44, 520, 40, 4
    mats = [synth.random_matrix(n, k, 6 + e % 3, seed=(46, e, 0)) for e in range(n_exp)]
    Ws = [so.decode_matrix(w.codes, n, k, w.bd, w.codebook, w.radius, w.perm) for w in mats]
    pms = [svq.pack(w) for w in mats]
    ids = _ids(m, topk, n_exp, 47)
    rows = m * topk if x_per_slot else m
    x = synth.random_activations(rows, k, seed=(48, x_per_slot, 0))
    xb = torch.zeros((rows, k + 3), dtype=torch.int16)
    xb[:, :k] = torch.from_numpy(x.view(np.int16))
    xd = xb.cuda().view(torch.bfloat16)[:, :k]
    d_ids = torch.from_numpy(ids).cuda()
    for dt in (torch.float32, torch.bfloat16):
        yb = torch.full((m * topk, n + 5), 7.0, dtype=dt, device="cuda")
        y = yb[:, :n]
        svq.moe_linear(pms, xd, d_ids, topk, bool(x_per_slot), out=y)
        torch.cuda.synchronize()
        assert torch.all(yb[:, n:] == 7.0)
        y64 = out_to_f64(y)
        _check_slots(y64, x, ids, topk, x_per_slot, Ws, range(n_exp), f"strided moe {dt}")


@pytest.mark.parametrize("m,topk", [(2048, 4), (2100, 4)])
def test_moe_routing_paths(svq, m, topk):
    """8192 slots (the routing done inside the prep launch, its largest case)
    and 8400 slots (the separate routing launch), some ids out of range:
    every valid slot matches the oracle, every invalid slot gets a zero row."""
    n_exp, n, k = 6, 40, 520
    mats = [synth.random_matrix(n, k, 6 + e % 3, seed=(49, e, 0)) for e in range(n_exp)]
    Ws = [so.decode_matrix(w.codes, n, k, w.bd, w.codebook, w.radius, w.perm) for w in mats]
    pms = [svq.pack(w) for w in mats]
    rng = np.random.default_rng(50 + m)
    ids = rng.integers(0, n_exp, size=m * topk).astype(np.int32)
    bad = np.arange(3, ids.size, 97)
    ids[bad] = np.where(bad % 2 == 0, -2, n_exp)
    x = synth.random_activations(m, k, seed=(51, m, 0))
    for dt in (torch.float32, torch.bfloat16):
        y = _run_moe(svq, pms, x, ids, topk, 0, dt)
        assert np.all(y[bad] == 0)
        good = np.setdiff1d(np.arange(ids.size), bad)
        for e in range(n_exp):
            slots = good[ids[good] == e]
            assert_within_tolerance(y[slots], so.linear(x[slots // topk], Ws[e]), x[slots // topk], Ws[e],
                                    label=f"{m * topk} slots, expert {e}, {dt}")


def _separate(svq, sets, xs, ids, topk, x_per_slot, dt):
    d_ids = torch.from_numpy(ids).cuda()
    return [out_to_f64(svq.moe_linear(p, to_device_bf16(x), d_ids, topk, x_per_slot, out_dtype=dt))
            for p, x in zip(sets, xs)]


@pytest.mark.parametrize("m,topk,x_per_slot", [(1, 3, 0), (4, 4, 1), (16, 4, 0), (40, 4, 0), (37, 5, 1),
                                                (2100, 4, 0)])
def test_moe_batched_equals_separate_calls(svq, m, topk, x_per_slot):
    """Three projections of different shapes (the first two reading one
    input) in one svq_moe_linear_batched call give the outputs of three
    svq_moe_linear calls bit for bit: one launch up to 64 slots (m = 1, 4,
    16), one staging and one product launch for all three up to 8192 slots
    (160 and 185 slots), the projections in turn beyond (8400 slots); some
    ids out of range."""
    n_exp = 6
    shapes = [(48, 520), (40, 520), (56, 264)]
    sets_in, sets, Ws = [], [], []
    for c, (n, k) in enumerate(shapes):
        mats = [synth.random_matrix(n, k, 6 + (e + c) % 3, seed=(52, c, e)) for e in range(n_exp)]
        sets_in.append(mats)
        sets.append([svq.pack(w) for w in mats])
        Ws.append([so.decode_matrix(w.codes, n, k, w.bd, w.codebook, w.radius, w.perm) for w in mats])
    ids = _ids(m, topk, n_exp, 53 + m)
    bad = np.arange(2, ids.size, 7)
    ids[bad] = np.where(bad % 2 == 0, -1, n_exp)
    rows = m * topk if x_per_slot else m
    xa = synth.random_activations(rows, 520, seed=(54, m, 0))
    xb = synth.random_activations(rows, 264, seed=(54, m, 1))
    xs = [xa, xa, xb]
    d_ids = torch.from_numpy(ids).cuda()
    xd = [to_device_bf16(x) for x in (xa, xb)]
    for dt in (torch.float32, torch.bfloat16):
        outs = svq.moe_linear_batched(sets, [xd[0], xd[0], xd[1]], d_ids, topk, bool(x_per_slot), out_dtype=dt)
        torch.cuda.synchronize()
        got = [out_to_f64(o) for o in outs]
        want = _separate(svq, sets, xs, ids, topk, bool(x_per_slot), dt)
        for c in range(3):
            assert np.array_equal(got[c], want[c]), f"projection {c}, {dt}"
            assert np.all(got[c][bad] == 0)
            # slots with an id outside [0, E) match no expert and are skipped here
            _check_slots(got[c], xs[c], ids, topk, x_per_slot, Ws[c], range(n_exp),
                         f"batched projection {c} m={m}")


def test_moe128_m1_gate_up_batched(svq):
    """The 128-expert gate and up projections of one token in one launch,
    bit for bit against two separate calls."""
    bd = synth.moe_expert_bd()
    sets = [[svq.pack(synth.moe_expert(e, p, int(bd[e]))) for e in range(synth.MOE_EXPERTS)]
            for p in (0, 1)]
    ids = synth.moe_routing(1)
    x = synth.moe_activations(1, 0)
    got = svq.moe_linear_batched(sets, [to_device_bf16(x)] * 2, torch.from_numpy(ids).cuda(),
                                 synth.MOE_TOPK, False, out_dtype=torch.float32)
    want = _separate(svq, sets, [x, x], ids, synth.MOE_TOPK, False, torch.float32)
    for c in range(2):
        assert np.array_equal(out_to_f64(got[c]), want[c])


@pytest.mark.parametrize("m,topk", [(3, 4), (40, 4)])
def test_moe_batched_mixed_alignment(svq, m, topk):
    """A batched call whose first projection has 16-byte aligned rows and
    whose second has odd row strides (x and y), on the per-slot path (12
    slots) and the grouped path (160 slots): every projection equals its
    separate call bit for bit, and the padding columns of y are untouched."""
    n_exp, n, k = 6, 44, 520
    sets = [[svq.pack(synth.random_matrix(n, k, 6 + (e + c) % 3, seed=(55, c, e))) for e in range(n_exp)]
            for c in range(2)]
    ids = _ids(m, topk, n_exp, 56 + m)
    x = synth.random_activations(m, k, seed=(57, m, 0))
    d_ids = torch.from_numpy(ids).cuda()
    xa = to_device_bf16(x)
    xb_pad = torch.zeros((m, k + 3), dtype=torch.int16)
    xb_pad[:, :k] = torch.from_numpy(x.view(np.int16))
    xb = xb_pad.cuda().view(torch.bfloat16)[:, :k]
    for dt in (torch.float32, torch.bfloat16):
        ya = torch.empty((m * topk, n), dtype=dt, device="cuda")
        yb_pad = torch.full((m * topk, n + 5), 7.0, dtype=dt, device="cuda")
        yb = yb_pad[:, :n]
        svq.MoeBatchedCall(sets, [xa, xb], d_ids, topk, False, [ya, yb])()
        torch.cuda.synchronize()
        assert torch.all(yb_pad[:, n:] == 7.0)
        want = [svq.moe_linear(sets[c], xa, d_ids, topk, False, out_dtype=dt) for c in range(2)]
        torch.cuda.synchronize()
        assert torch.equal(ya, want[0]) and torch.equal(yb, want[1]), f"{dt}"


@pytest.mark.parametrize("m", [8, 100])
def test_moe_batched_full_expert_table(svq, m):
    """Four projections of 64 experts each fill the 256-entry expert table of
    the batched launches (per-slot path at 32 slots, grouped path at 400):
    every projection equals its separate call bit for bit."""
    n_exp, topk, shapes = 64, 4, [(40, 264), (24, 264), (40, 520), (16, 8)]
    sets = [[svq.pack(synth.random_matrix(n, k, 6 + (e + c) % 3, seed=(58, c, e))) for e in range(n_exp)]
            for c, (n, k) in enumerate(shapes)]
    ids = _ids(m, topk, n_exp, 59 + m)
    d_ids = torch.from_numpy(ids).cuda()
    xs = [to_device_bf16(synth.random_activations(m, k, seed=(60, m, c))) for c, (_, k) in enumerate(shapes)]
    got = svq.moe_linear_batched(sets, xs, d_ids, topk, False, out_dtype=torch.float32)
    want = [svq.moe_linear(sets[c], xs[c], d_ids, topk, False, out_dtype=torch.float32) for c in range(4)]
    torch.cuda.synchronize()
    for c in range(4):
        assert torch.equal(got[c], want[c]), f"projection {c}"
