"""libsvq C ABI on a host without a GPU: the library loads, exports every
function include/svq.h declares, answers size queries and rejects bad
arguments before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from tests.conftest import ROOT

svq = pytest.importorskip("bit_spherical_vector_amd.svq")


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "svq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == {"svq_pack", "svq_linear", "svq_linear_batched", "svq_linear_noalloc",
                             "svq_moe_linear", "svq_moe_linear_batched", "svq_encode", "svq_encode_weighted", "svq_esg_perm",
                             "svq_abs_select", "svq_status_string"}
    for name in declared:
        assert hasattr(svq.LIB, name), name
    assert set(declared) == set(svq.EXPORTED)


def test_status_strings():
    assert svq.status_string(0) == "ok"
    assert svq.status_string(-3) == "buffer too small"
    assert svq.status_string(-99) == "unknown status"


def _desc(mat, **over):
    fields = dict(n=mat.n, k=mat.k, bd=mat.bd, br=mat.br, codes=mat.codes,
                  codebook=mat.codebook, radius=mat.radius, perm=mat.perm)
    fields.update(over)
    return svq.make_desc(**fields)


def _expected_bytes(n, k):
    a = lambda v: (v + 255) // 256 * 256
    tiles, units = (n + 15) // 16, (k + 511) // 512
    return a(4096) + a(2048) + a(16384) + a(32768) + a(2 * units * 512) + a(tiles * units * 2304)


@pytest.mark.parametrize("n,k,bd", [(512, 1024, 8), (37, 104, 6), (1, 8, 7), (2048, 768, 7)])
def test_pack_size_query(n, k, bd):
    mat = synth.random_matrix(n, k, bd, seed=(20, n, k))
    desc, keep = _desc(mat)
    st, nbytes = svq.svq_pack(desc, None, 0, None, 0)
    assert st == svq.SVQ_OK
    assert nbytes == _expected_bytes(n, k)


def test_pack_rejects_bad_arguments():
    mat = synth.random_matrix(32, 64, 7, seed=(21, 0, 0))
    cases = [
        (dict(k=60), svq.SVQ_ERR_INVALID_ARG),          # k % 8 != 0
        (dict(n=0), svq.SVQ_ERR_INVALID_ARG),
        (dict(k=0), svq.SVQ_ERR_INVALID_ARG),
        (dict(br=4), svq.SVQ_ERR_INVALID_ARG),          # bd + br != 10
        (dict(bd=5, br=5), svq.SVQ_ERR_UNSUPPORTED),     # codebook split outside {6,7,8}
        (dict(bd=9, br=1), svq.SVQ_ERR_UNSUPPORTED),
        (dict(k=65544), svq.SVQ_ERR_UNSUPPORTED),        # beyond the uint16 permutation
    ]
    for over, expect in cases:
        if "k" in over and over["k"] not in (0, 60):
            continue  # perm length would not match; covered separately
        desc, keep = _desc(mat, **over)
        st, _ = svq.svq_pack(desc, None, 0, None, 0)
        assert st == expect, over
    # non-permutations
    bad = mat.perm.copy()
    bad[3] = bad[4]
    desc, keep = _desc(mat, perm=bad)
    assert svq.svq_pack(desc, None, 0, None, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    bad = mat.perm.copy()
    bad[0] = 64
    desc, keep = _desc(mat, perm=bad)
    assert svq.svq_pack(desc, None, 0, None, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    bad = mat.perm.copy()
    bad[0] = -1
    desc, keep = _desc(mat, perm=bad)
    assert svq.svq_pack(desc, None, 0, None, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    # null pointers
    desc, keep = _desc(mat)
    desc.codes = None
    assert svq.svq_pack(desc, None, 0, None, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    # null desc / null size
    assert svq.LIB.svq_pack(None, None, ctypes.byref(ctypes.c_size_t(0)), None, None) == \
        svq.SVQ_ERR_INVALID_ARG
    desc, keep = _desc(mat)
    assert svq.LIB.svq_pack(ctypes.byref(desc), None, None, None, None) == svq.SVQ_ERR_INVALID_ARG


def test_pack_k_limit():
    k = 65536 + 8
    mat = synth.random_matrix(1, 8, 7, seed=(22, 0, 0))
    desc, keep = svq.make_desc(1, k, 7, 3, np.zeros(k * 9 // 32 + 1, np.uint8), mat.codebook,
                               mat.radius, np.arange(k, dtype=np.int32))
    assert svq.svq_pack(desc, None, 0, None, 0)[0] == svq.SVQ_ERR_UNSUPPORTED


def test_pack_undersized_destination_before_device_work():
    mat = synth.random_matrix(16, 64, 8, seed=(23, 0, 0))
    desc, keep = _desc(mat)
    st, need = svq.svq_pack(desc, None, 0, None, 0)
    h = svq.Handle()
    # a fake non-null device pointer: the size check fails before any copy
    st, reported = svq.svq_pack(desc, 0x1000, need - 1, h, 0)
    assert st == svq.SVQ_ERR_BUFFER_TOO_SMALL
    assert reported == need


def _fake_handle(n, k, bd):
    a = lambda v: (v + 255) // 256 * 256
    h = svq.Handle()
    h.dev = 0x1000
    h.n, h.k, h.bd, h.br = n, k, bd, 10 - bd
    h.n_tiles, h.units = (n + 15) // 16, (k + 511) // 512
    h.off_dtab = 0
    h.off_rtab = a(4096)
    h.off_btab = h.off_rtab + a(2048)
    h.off_xtab = h.off_btab + a(16384)
    h.off_perm = h.off_xtab + a(32768)
    h.xscale_log2 = 17
    h.off_codes = h.off_perm + a(2 * h.units * 512)
    h.padded_code_bytes = h.n_tiles * h.units * 2304
    h.bytes = h.off_codes + a(h.padded_code_bytes)
    h.code_bytes = (n * k * 9 + 31) // 32
    return h


def _dequant_gemm_need(shapes, m, cus=256):
    """Workspace of the m > 4 path: permuted activations padded to the block
    height (64 rows below m = 256, else 256), plus fp32 partial tiles of the
    K splits taken when the output tiles give fewer than 2 blocks per compute
    unit (no device here: 256 compute units assumed)."""
    a = lambda v: (v + 255) // 256 * 256
    cdiv = lambda p, q: -(-p // q)
    bm = 256 if m >= 256 else 64
    m_pad = cdiv(m, bm) * bm
    tiles = [cdiv(cdiv(n, 16), 16) for n, _ in shapes]
    units = [cdiv(k, 512) for _, k in shapes]
    need = sum(a(m_pad * u * 512 * 2) for u in units)
    blocks = sum(t * (m_pad // bm) for t in tiles)
    if blocks < 2 * cus:
        per = cdiv(sum(t * (m_pad // bm) * u for t, u in zip(tiles, units)), 2 * cus)
        for t, u in zip(tiles, units):
            sp = max(1, cdiv(u, per))
            ups = cdiv(u, sp)
            sp = cdiv(u, ups)
            if sp > 1:
                need += a(sp * m_pad * t * 256 * 4)
    return need


def _small_items(shapes, cus=256):
    """Items (row tile x unit) per block on the 4 < m <= 16 path: every block
    resident at once at two blocks per compute unit, between 16 and 32."""
    cdiv = lambda p, q: -(-p // q)
    total = sum(cdiv(n, 16) * cdiv(k, 512) for n, k in shapes)
    return max(16, min(32, cdiv(total, 2 * cus)))


def _small_plan(n_tiles, units, items):
    """Block shape of the 4 < m <= 16 path: up to 8 units in one K range,
    else ranges of about 5 units; then as many row tiles per block (1..6) as
    give about `items` items, at most 32."""
    splits = 1 if units <= 8 else (units + 4) // 5
    upr = -(-units // splits)
    splits = -(-units // upr)
    tiles = max(1, min(6, (items + upr // 2) // upr))
    while tiles > 1 and tiles * upr > 32:
        tiles -= 1
    return tiles, upr, splits, -(-n_tiles // tiles)


def _small_need(shapes):
    """Workspace of the 4 < m <= 16 path, per matrix: the fragment-ordered
    activations (16 rows x 512 slots fp16 = 16 KB per unit) and their
    inverse scales (16 fp32 per unit); with K ranges, fp32 partial tiles for
    every (tile of the groups, range) and one arrival counter per group."""
    a = lambda v: (v + 255) // 256 * 256
    cdiv = lambda p, q: -(-p // q)
    items = _small_items(shapes)
    need = 0
    for n, k in shapes:
        units = cdiv(k, 512)
        tiles, _, splits, groups = _small_plan(cdiv(n, 16), units, items)
        need += a(units * 16384) + a(units * 64)
        if splits > 1:
            need += a(groups * tiles * splits * 1024) + a(groups * 4)
    return need


def _exact_need(shapes, m):
    """Workspace of the m <= 4 path: none for the fused m = 1 launch (256
    bytes reported); for m = 2..4, per matrix, the gathered fp16 activations
    (1 KB per unit and row) and the units' scales (16 bytes per unit)."""
    if m == 1:
        return 256
    a = lambda v: (v + 255) // 256 * 256
    units = [-(-k // 512) for _, k in shapes]
    return sum(a(m * u * 1024) + a(u * 16) for u in units)


def test_linear_workspace_query_and_validation():
    h = _fake_handle(512, 1024, 8)
    dq = lambda m: _dequant_gemm_need([(512, 1024)], m)
    assert dq(17) == 64 * 2048 + 2 * 64 * 512 * 4  # two K splits of one unit each
    assert _exact_need([(512, 1024)], 2) == 4096 + 256
    assert _small_need([(512, 1024)]) == 2 * 16384 + 256
    assert _small_need([(100, 2560)]) == 5 * 16384 + 512
    assert _small_plan(160, 19, 16) == (3, 5, 4, 54)
    assert _small_need([(2560, 9728)]) == 19 * 16384 + 1280 + 54 * 3 * 4 * 1024 + 256
    layer = [(4096, 2560), (1024, 2560), (1024, 2560), (2560, 4096), (9728, 2560), (9728, 2560),
             (2560, 9728)]
    assert _small_items(layer) == 25
    big = _fake_handle(2560, 9728, 7)  # 19 units: K ranges
    for m in (5, 16):
        st, need = svq.svq_linear(big, None, m, 9728, None, 2560, svq.SVQ_BF16, None, 0, 0)
        assert st == svq.SVQ_OK and need == _small_need([(2560, 9728)]), (m, need)
    for m, expect in [(1, _exact_need([(512, 1024)], 1)), (4, _exact_need([(512, 1024)], 4)),
                      (5, _small_need([(512, 1024)])), (16, _small_need([(512, 1024)])),
                      (17, dq(17)), (64, dq(64)), (65, dq(65)), (300, dq(300))]:
        st, need = svq.svq_linear(h, None, m, 1024, None, 512, svq.SVQ_BF16, None, 0, 0)
        assert st == svq.SVQ_OK and need == expect, (m, need)
    # bad arguments
    assert svq.svq_linear(h, None, 0, 1024, None, 512, 0, None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    assert svq.svq_linear(h, None, 1, 1000, None, 512, 0, None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    assert svq.svq_linear(h, None, 1, 1024, None, 500, 0, None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    assert svq.svq_linear(h, None, 1, 1024, None, 512, 7, None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    # undersized workspace: rejected before launching
    st, _ = svq.svq_linear(h, 0x2000, 1, 1024, 0x3000, 512, 0, 0x4000, 100, 0)
    assert st == svq.SVQ_ERR_BUFFER_TOO_SMALL
    # null x / y with a workspace
    st, _ = svq.svq_linear(h, None, 1, 1024, 0x3000, 512, 0, 0x4000, 1 << 20, 0)
    assert st == svq.SVQ_ERR_INVALID_ARG
    # a handle that does not describe a packed buffer
    bad = _fake_handle(512, 1024, 8)
    bad.off_codes += 256
    assert svq.svq_linear(bad, None, 1, 1024, None, 512, 0, None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    bad = _fake_handle(512, 1024, 8)
    bad.dev = None
    assert svq.svq_linear(bad, None, 1, 1024, None, 512, 0, None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG


def test_moe_workspace_query_and_validation():
    hs = (svq.Handle * 4)()
    for e in range(4):
        hs[e] = _fake_handle(768, 2048, 6 + e % 3)
    st, need_small = svq.svq_moe_linear(hs, 4, None, 2048, 0, None, 1, 2, None, 768, 0, None, 0, 0)
    assert st == svq.SVQ_OK and need_small > 0
    st, need_big = svq.svq_moe_linear(hs, 4, None, 2048, 0, None, 512, 2, None, 768, 0, None, 0, 0)
    assert st == svq.SVQ_OK and need_big > need_small
    # topk > experts, bad x_per_slot, mismatched shapes
    assert svq.svq_moe_linear(hs, 4, None, 2048, 0, None, 1, 5, None, 768, 0, None, 0, 0)[0] == \
        svq.SVQ_ERR_INVALID_ARG
    assert svq.svq_moe_linear(hs, 4, None, 2048, 2, None, 1, 2, None, 768, 0, None, 0, 0)[0] == \
        svq.SVQ_ERR_INVALID_ARG
    hs[2] = _fake_handle(768, 1024, 7)
    assert svq.svq_moe_linear(hs, 4, None, 2048, 0, None, 1, 2, None, 768, 0, None, 0, 0)[0] == \
        svq.SVQ_ERR_INVALID_ARG
    assert svq.svq_moe_linear(hs, 0, None, 2048, 0, None, 1, 1, None, 768, 0, None, 0, 0)[0] == \
        svq.SVQ_ERR_UNSUPPORTED


def test_moe_batched_query_and_validation():
    gate = (svq.Handle * 4)(*[_fake_handle(768, 2048, 6 + e % 3) for e in range(4)])
    down = (svq.Handle * 4)(*[_fake_handle(2048, 768, 6 + e % 3) for e in range(4)])
    for m in (1, 512):
        singles = [svq.svq_moe_linear(h, 4, None, h[0].k, 0, None, m, 2, None, h[0].n, 0, None, 0, 0)
                   for h in (gate, down)]
        assert all(st == svq.SVQ_OK for st, _ in singles)
        st, need = svq.svq_moe_linear_batched([gate, down], 2, 4, None, None, 0, None, m, 2, None, None,
                                              0, None, 0, 0)
        assert st == svq.SVQ_OK
        if m == 1:  # one per-slot launch: no staging
            assert need == max(n for _, n in singles)
        else:  # the routing once, the staged activations of both projections
            assert max(n for _, n in singles) < need < sum(n for _, n in singles)
    # projection count outside 1..4; count * num_experts beyond 256
    for count in (0, 5):
        assert svq.svq_moe_linear_batched([gate] * max(count, 1), count, 4, None, None, 0, None, 1, 2,
                                          None, None, 0, None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    wide = (svq.Handle * 128)(*[_fake_handle(64, 512, 6) for _ in range(128)])
    assert svq.svq_moe_linear_batched([wide] * 2, 2, 128, None, None, 0, None, 1, 2, None, None, 0,
                                      None, 0, 0)[0] == svq.SVQ_OK
    assert svq.svq_moe_linear_batched([wide] * 3, 3, 128, None, None, 0, None, 1, 2, None, None, 0,
                                      None, 0, 0)[0] == svq.SVQ_ERR_UNSUPPORTED
    # a stride below a projection's k or n; one projection with mixed shapes
    assert svq.svq_moe_linear_batched([gate, down], 2, 4, None, [2048, 700], 0, None, 1, 2, None,
                                      [768, 2048], 0, None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG
    mixed = (svq.Handle * 4)(*[_fake_handle(768, 2048, 7) for _ in range(3)] + [_fake_handle(768, 1024, 7)])
    assert svq.svq_moe_linear_batched([gate, mixed], 2, 4, None, None, 0, None, 1, 2, None, None, 0,
                                      None, 0, 0)[0] == svq.SVQ_ERR_INVALID_ARG


def test_linear_batched_query_and_validation():
    hs = (svq.Handle * 3)(_fake_handle(512, 1024, 8), _fake_handle(64, 2560, 6),
                          _fake_handle(300, 768, 7))
    st, need = svq.svq_linear_batched(hs, 3, None, None, 1, None, None, 0, None, 0, 0)
    assert st == svq.SVQ_OK and need == _exact_need([(512, 1024), (64, 2560), (300, 768)], 1)
    st, need = svq.svq_linear_batched(hs, 3, None, None, 16, None, None, 0, None, 0, 0)
    assert st == svq.SVQ_OK and need == _small_need([(512, 1024), (64, 2560), (300, 768)])
    # the whole 4B-class layer: the long-k matrix is cut into K ranges
    layer = [(4096, 2560), (1024, 2560), (1024, 2560), (2560, 4096), (9728, 2560), (9728, 2560),
             (2560, 9728)]
    hl = (svq.Handle * 7)(*[_fake_handle(n, k, 7) for n, k in layer])
    st, need = svq.svq_linear_batched(hl, 7, None, None, 16, None, None, 0, None, 0, 0)
    assert st == svq.SVQ_OK and need == _small_need(layer)
    st, need = svq.svq_linear_batched(hs, 3, None, None, 40, None, None, 0, None, 0, 0)
    assert st == svq.SVQ_OK and need == _dequant_gemm_need([(512, 1024), (64, 2560), (300, 768)], 40)
    assert svq.svq_linear_batched(hs, 0, None, None, 1, None, None, 0, None, 0, 0)[0] == \
        svq.SVQ_ERR_INVALID_ARG
    assert svq.svq_linear_batched(hs, 9, None, None, 1, None, None, 0, None, 0, 0)[0] == \
        svq.SVQ_ERR_INVALID_ARG
    ldx = (ctypes.c_int64 * 3)(1024, 2000, 768)  # 2000 < k of the second matrix
    ldy = (ctypes.c_int64 * 3)(512, 64, 300)
    assert svq.svq_linear_batched(hs, 3, None, ldx, 1, None, ldy, 0, None, 0, 0)[0] == \
        svq.SVQ_ERR_INVALID_ARG
    ldx[1] = 2560
    assert svq.svq_linear_batched(hs, 3, None, ldx, 1, None, ldy, 0, None, 0, 0)[0] == svq.SVQ_OK
    # missing pointer arrays with a workspace
    assert svq.svq_linear_batched(hs, 3, None, ldx, 1, None, ldy, 0, 0x1000, 4096, 0)[0] == \
        svq.SVQ_ERR_INVALID_ARG


def test_encode_workspace_query_and_validation():
    """svq_encode: size query without a GPU, and every host-side check
    before any device work (the pointers below are never dereferenced)."""
    import synth
    mat = synth.random_matrix(16, 64, 7, seed=(45, 7, 0))
    cb, rad, perm = mat.codebook, mat.radius, mat.perm
    a = lambda v: (v + 255) // 256 * 256
    st, need = svq.svq_encode(None, 64, 16, 64, 7, cb, rad, perm, None, None, 0, 0)
    # every table slot is sized for bd = 8 (codebook 256 x 8, 16 radii, 15 midpoints)
    assert st == svq.SVQ_OK and need == a(256 * 8 * 8 + 2 * 16 * 8) + a(64 * 4)
    q = lambda **kw: svq.svq_encode(kw.get("w"), kw.get("ldw", 64), kw.get("n", 16), kw.get("k", 64),
                                    kw.get("bd", 7), kw.get("cb", cb), kw.get("rad", rad),
                                    kw.get("perm", perm), kw.get("codes"), kw.get("ws"),
                                    kw.get("wsb", 0), 0)[0]
    assert q(k=60) == svq.SVQ_ERR_INVALID_ARG          # k not a multiple of 8
    assert q(n=0) == svq.SVQ_ERR_INVALID_ARG
    assert q(ldw=32) == svq.SVQ_ERR_INVALID_ARG        # ldw < k
    assert q(bd=5) == svq.SVQ_ERR_UNSUPPORTED
    bad_perm = perm.copy()
    bad_perm[1] = bad_perm[0]
    assert q(perm=bad_perm) == svq.SVQ_ERR_INVALID_ARG
    assert q(rad=rad[::-1].copy()) == svq.SVQ_ERR_INVALID_ARG   # not increasing
    inf_cb = np.asarray(cb).copy()
    inf_cb[3, 2] = 0x7C00
    assert q(cb=inf_cb) == svq.SVQ_ERR_INVALID_ARG      # infinite codebook entry
    neg = np.asarray(rad).copy()
    neg[0] = 0xBC00                                     # -1.0
    assert q(rad=neg) == svq.SVQ_ERR_INVALID_ARG
    # a workspace without the weight or code pointers, then too small a one
    assert q(ws=0x1000, wsb=1 << 20) == svq.SVQ_ERR_INVALID_ARG
    assert q(w=0x2000, codes=0x3000, ws=0x1000, wsb=100) == svq.SVQ_ERR_BUFFER_TOO_SMALL



def test_encode_weighted_workspace_query_and_validation():
    """svq_encode_weighted: the size query and host checks of svq_encode, and
    a workspace call without the channel weights is refused before any
    device work (the pointers below are never dereferenced)."""
    import synth
    mat = synth.random_matrix(16, 64, 7, seed=(45, 7, 0))
    cb, rad, perm = mat.codebook, mat.radius, mat.perm
    st_plain, need_plain = svq.svq_encode(None, 64, 16, 64, 7, cb, rad, perm, None, None, 0, 0)
    q = lambda **kw: svq.svq_encode_weighted(kw.get("w"), kw.get("ldw", 64), kw.get("n", 16),
                                             kw.get("k", 64), kw.get("bd", 7), kw.get("cb", cb),
                                             kw.get("rad", rad), kw.get("perm", perm), kw.get("h"),
                                             kw.get("codes"), kw.get("ws"), kw.get("wsb", 0), 0)
    st, need = q()
    assert st == svq.SVQ_OK == st_plain and need == need_plain
    assert q(k=60)[0] == svq.SVQ_ERR_INVALID_ARG
    assert q(bd=9)[0] == svq.SVQ_ERR_UNSUPPORTED
    assert q(rad=np.asarray(rad)[::-1].copy())[0] == svq.SVQ_ERR_INVALID_ARG
    bad_perm = np.asarray(perm).copy()
    bad_perm[2] = bad_perm[3]
    assert q(perm=bad_perm)[0] == svq.SVQ_ERR_INVALID_ARG
    # weights, codes and workspace present but no h: refused
    assert q(w=0x2000, codes=0x3000, ws=0x1000, wsb=need)[0] == svq.SVQ_ERR_INVALID_ARG
    assert q(w=0x2000, h=0x4000, codes=0x3000, ws=0x1000, wsb=100)[0] == svq.SVQ_ERR_BUFFER_TOO_SMALL


def test_esg_workspace_query_and_validation():
    a = lambda v: (v + 255) // 256 * 256
    q = lambda **kw: svq.svq_esg_perm(kw.get("x"), kw.get("t", 100), kw.get("ldx", 64),
                                      kw.get("k", 64), kw.get("e"), kw.get("p"), kw.get("ws"),
                                      kw.get("wsb", 0), 0)
    st, need = q()
    assert st == svq.SVQ_OK and need == a(64 * 4)
    assert q(k=60)[0] == svq.SVQ_ERR_INVALID_ARG        # k not a multiple of 8
    assert q(t=0)[0] == svq.SVQ_ERR_INVALID_ARG         # no calibration token
    assert q(ldx=32)[0] == svq.SVQ_ERR_INVALID_ARG      # ldx < k
    assert q(ldx=68)[0] == svq.SVQ_ERR_INVALID_ARG      # rows not 16-byte aligned
    assert q(ws=0x1000, wsb=1 << 20)[0] == svq.SVQ_ERR_INVALID_ARG        # no x / outputs
    assert q(x=0x2008, e=0x3000, p=0x4000, ws=0x1000, wsb=1 << 20)[0] == svq.SVQ_ERR_INVALID_ARG
    assert q(x=0x2000, e=0x3000, p=0x4000, ws=0x1000, wsb=8)[0] == svq.SVQ_ERR_BUFFER_TOO_SMALL


def test_abs_workspace_query_and_validation():
    import synth
    cands = [(bd, m.codebook, m.radius) for bd, m in
             ((bd, synth.random_matrix(16, 64, bd, seed=(46, bd, 0))) for bd in (6, 7, 8))]
    perm = synth.random_matrix(16, 64, 7, seed=(46, 7, 0)).perm
    a = lambda v: (v + 255) // 256 * 256
    q = lambda **kw: svq.svq_abs_select(kw.get("w"), kw.get("ldw", 64), kw.get("n", 16),
                                        kw.get("k", 64), kw.get("h"), kw.get("perm", perm),
                                        kw.get("cands", cands), kw.get("codes"), kw.get("ws"),
                                        kw.get("wsb", 0), 0)
    st, need, _, _ = q()
    count = 16 * 8
    tab = a(256 * 8 * 8 + 2 * 16 * 8)
    assert st == svq.SVQ_OK
    assert need == 3 * tab + a(64 * 4) + 3 * a(count * 18 // 8) + a(count * 8) + a(3 * 16 * 8) + a(64)
    assert q(cands=[])[0] == svq.SVQ_ERR_INVALID_ARG
    assert q(cands=cands * 3)[0] == svq.SVQ_ERR_INVALID_ARG          # more than 8
    assert q(cands=[(5,) + cands[0][1:]])[0] == svq.SVQ_ERR_UNSUPPORTED
    bad = np.asarray(cands[1][2]).copy()[::-1]
    assert q(cands=[cands[0], (7, cands[1][1], bad)])[0] == svq.SVQ_ERR_INVALID_ARG
    bad_perm = np.asarray(perm).copy()
    bad_perm[0] = bad_perm[1]
    assert q(perm=bad_perm)[0] == svq.SVQ_ERR_INVALID_ARG
    assert q(ldw=8)[0] == svq.SVQ_ERR_INVALID_ARG
    assert q(ws=0x1000, wsb=1 << 20)[0] == svq.SVQ_ERR_INVALID_ARG    # no w, h, codes
    assert q(w=0x2000, h=0x3000, codes=0x4000, ws=0x1000, wsb=64)[0] == svq.SVQ_ERR_BUFFER_TOO_SMALL
    # the fit selector is 0 or 1
    fit = lambda v: svq.svq_abs_select(None, 64, 16, 64, None, perm, cands, None, None, 0, 0,
                                       weighted_fit=v)[0]
    assert fit(1) == svq.SVQ_OK
    assert fit(2) == svq.SVQ_ERR_INVALID_ARG


def test_calibration_wrappers_reject_bad_tensors_before_any_device_work():
    """The binding checks dtypes and layouts on the host (CPU tensors here:
    nothing reaches the library or the device)."""
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        svq.esg_perm(torch.zeros((4, 8), dtype=torch.float32))          # not bf16
    with pytest.raises(ValueError):
        svq.esg_perm(torch.zeros((8, 4), dtype=torch.bfloat16).t())     # column stride != 1
    w = torch.zeros((4, 8), dtype=torch.float32)
    h = torch.zeros(8, dtype=torch.float64)
    perm = np.arange(8, dtype=np.int32)
    with pytest.raises(ValueError):
        svq.abs_select(w.double(), perm, h, [])                          # weights not fp32
    with pytest.raises(ValueError):
        svq.abs_select(w, perm, h.float(), [])                           # h not fp64
    with pytest.raises(ValueError):
        svq.abs_select(w, perm, torch.zeros(16, dtype=torch.float64)[::2], [])  # h strided


def test_linear_noalloc_rejects_before_device_work():
    """svq_linear_noalloc checks its arguments and the scratch size before it
    looks up the device array, so a host without a GPU sees the errors."""
    big = _fake_handle(2560, 9728, 7)
    need = _dequant_gemm_need([(2560, 9728)], 4096)
    assert need > svq.SVQ_SCRATCH_BYTES
    assert svq.svq_linear_noalloc(big, 0x2000, 4096, 9728, 0x3000, 2560, 0, 0) == \
        svq.SVQ_ERR_UNSUPPORTED
    h = _fake_handle(512, 1024, 8)
    assert svq.svq_linear_noalloc(h, 0x2000, 0, 1024, 0x3000, 512, 0, 0) == svq.SVQ_ERR_INVALID_ARG
    assert svq.svq_linear_noalloc(h, 0x2000, 1, 1000, 0x3000, 512, 0, 0) == svq.SVQ_ERR_INVALID_ARG
    assert svq.svq_linear_noalloc(h, 0x2000, 1, 1024, 0x3000, 512, 9, 0) == svq.SVQ_ERR_INVALID_ARG
    bad = _fake_handle(512, 1024, 8)
    bad.off_codes += 256
    assert svq.svq_linear_noalloc(bad, 0x2000, 1, 1024, 0x3000, 512, 0, 0) == svq.SVQ_ERR_INVALID_ARG
