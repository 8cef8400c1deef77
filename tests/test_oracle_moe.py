"""Pins for the oracle's expert sort and grouped GEMM: invariants, brute force,
and the one-expert top-1 case that reduces to the dense GEMM."""
import numpy as np

from oracle import gemm, moe, quant
from synthetic import router_topk


def test_sort_invariants_and_brute_force():
    ids, _ = router_topk(4, 64, 256, 8)
    counts, offsets, sp = moe.moe_sort_ref(ids, 256)
    flat = ids.ravel()
    assert counts.sum() == flat.size
    assert (np.diff(offsets) >= 0).all() and offsets[0] == 0 and offsets[-1] == flat.size
    assert np.array_equal(np.sort(sp), np.arange(flat.size))
    for e in range(256):
        seg = sp[offsets[e]:offsets[e + 1]]
        brute = [p for p in range(flat.size) if flat[p] == e]
        assert list(seg) == brute                     # stable: ascending pair ids


def test_router_shape_distinct_descending():
    ids, w = router_topk(4, 200, 256, 8)
    assert ids.shape == (200, 8)
    for row in ids:
        assert len(set(row.tolist())) == 8
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert (np.diff(w, axis=1) <= 1e-7).all()        # descending logits -> descending weights


def test_moe_single_expert_top1_is_dense():
    r = np.random.default_rng(7)
    t, k, n = 9, 256, 48
    x = r.normal(size=(t, k))
    w = r.normal(0, 0.02, (n, k)).astype(np.float32)
    st = quant.quantize(quant.FMT_INT4_SYM, w)
    wq = quant.dequant(quant.FMT_INT4_SYM, st["codes"], st["scales"]).astype(np.float64)
    ids = np.zeros((t, 1), dtype=np.int32)
    y, b, _ = moe.moe_gemm_ref(x, False, 1, ids, lambda e: wq, n)
    yd, bd = gemm.gemm_ref(x, wq)
    assert np.array_equal(y, yd) and np.array_equal(b, bd)


def test_moe_rows_follow_pairs():
    r = np.random.default_rng(8)
    t, topk, E, k, n = 6, 2, 3, 128, 16
    ids = np.array([[0, 1], [2, 0], [1, 2], [0, 2], [1, 0], [2, 1]], dtype=np.int32)
    x = r.normal(size=(t, k))
    ws = [r.normal(size=(n, k)) for _ in range(E)]
    y, _, _ = moe.moe_gemm_ref(x, False, topk, ids, lambda e: ws[e], n)
    for p in range(t * topk):
        assert np.allclose(y[p], ws[ids.ravel()[p]] @ x[p // topk], atol=1e-12)
    a = r.normal(size=(t * topk, k))               # down projection: one row per pair
    y2, _, _ = moe.moe_gemm_ref(a, True, topk, ids, lambda e: ws[e], n)
    for p in range(t * topk):
        assert np.allclose(y2[p], ws[ids.ravel()[p]] @ a[p], atol=1e-12)


def test_silu_mul_closed_forms():
    """silu(x) = x * sigmoid(x): silu(0) = 0; sigmoid(1) = 1 / (1 + 1/e), the
    logistic function's value at 1, 0.7310585786300049, and sigmoid(2) =
    0.8807970779778823 (a sign error in the exponent gives sigmoid(-1)
    instead); silu(x) - silu(-x) = x for every x (sigmoid(x) + sigmoid(-x) =
    1), which a dropped factor x breaks; gate and up are not interchangeable
    (gate 2, up 3 gives 3 silu(2), not 2 silu(3))."""
    gu = np.array([[0.0, 1.0, 2.0, 5.0, 1.0, 3.0]])
    h = moe.silu_mul_ref(gu, 3)
    assert h[0, 0] == 0.0
    assert abs(h[0, 1] - 0.7310585786300049) < 1e-15                   # silu(1) * 1
    assert abs(h[0, 2] - 3.0 * 2.0 * 0.8807970779778823) < 1e-14     # sigmoid(2)
    r = np.random.default_rng(3)
    x = r.normal(0, 4, 1000)
    ones = np.ones_like(x)
    hp = moe.silu_mul_ref(np.stack([x, ones], 1), 1)[:, 0]
    hm_ = moe.silu_mul_ref(np.stack([-x, ones], 1), 1)[:, 0]
    assert np.allclose(hp - hm_, x, rtol=0, atol=1e-12)
    big = moe.silu_mul_ref(np.array([[60.0, -800.0, 1.0, 1.0]]), 2)
    assert abs(big[0, 0] - 60.0) < 1e-12 and big[0, 1] == 0.0          # limits, exp overflow handled


def test_silu_mul_brute_force():
    r = np.random.default_rng(4)
    gu = r.normal(size=(5, 6))
    h = moe.silu_mul_ref(gu, 3)
    for i in range(5):
        for j in range(3):
            g, u = gu[i, j], gu[i, 3 + j]
            assert abs(h[i, j] - g / (1.0 + np.exp(-g)) * u) < 1e-14


def test_combine_one_hot_and_brute_force():
    """A one-hot weight row gathers that pair's row exactly; otherwise the
    result equals the explicit loop over pairs t*topk + j."""
    r = np.random.default_rng(5)
    t, topk, n = 4, 3, 7
    y = r.normal(size=(t * topk, n))
    w = np.zeros((t, topk))
    w[np.arange(t), [2, 0, 1, 2]] = 1.0
    out, b = moe.combine_ref(y, w, topk)
    for i, j in enumerate([2, 0, 1, 2]):
        assert np.array_equal(out[i], y[i * topk + j])
        assert np.array_equal(b[i], np.abs(y[i * topk + j]))
    w = r.random((t, topk))
    out, b = moe.combine_ref(y, w, topk)
    for i in range(t):
        ref = np.zeros(n)
        ab = np.zeros(n)
        for j in range(topk):
            ref += w[i, j] * y[i * topk + j]
            ab += abs(w[i, j]) * np.abs(y[i * topk + j])
        assert np.allclose(out[i], ref, rtol=0, atol=1e-13)
        assert np.allclose(b[i], ab, rtol=0, atol=1e-13)


def test_check_elementwise_rejects_two_ulps():
    from oracle import codecs
    ref = np.array([1.0, 3.0, -0.5])
    bits = codecs.bf16_rne_bits(ref.astype(np.float32))
    assert gemm.check_elementwise(bits, ref)["ok"]
    off = bits.copy()
    off[1] += 2                                    # two bf16 ulps away
    assert not gemm.check_elementwise(off, ref)["ok"]


def test_moe_pairs_subset_brute_force():
    """The pairs= path (used by every workload-size parity test) returns the
    rows of exactly the listed pairs, in the listed order, for both
    projections: each row equals W_{ids[p]} @ a[row(p)] computed by an
    explicit loop, and the subset equals the full result indexed by it
    (unsorted pairs, a repeated pair, pairs of one expert and of several).
    Rows taken by the subset index instead of the pair id fail."""
    r = np.random.default_rng(9)
    t, topk, E, k, n = 11, 3, 4, 128, 12
    ids = np.stack([r.choice(E, topk, replace=False) for _ in range(t)]).astype(np.int32)
    ws = [r.normal(size=(n, k)) for _ in range(E)]
    flat = ids.ravel()
    for rows_are_pairs in (False, True):
        a = r.normal(size=(t * topk if rows_are_pairs else t, k))
        pairs = np.array([31, 2, 17, 2, 0, 25, 9, 32])
        y, b, pp = moe.moe_gemm_ref(a, rows_are_pairs, topk, ids, lambda e: ws[e], n, pairs=pairs)
        assert np.array_equal(pp, pairs)
        for i, p in enumerate(pairs):
            row = a[p] if rows_are_pairs else a[p // topk]
            w = ws[flat[p]]
            ref = np.array([sum(w[c, kk] * row[kk] for kk in range(k)) for c in range(n)])
            bnd = np.array([sum(abs(w[c, kk] * row[kk]) for kk in range(k)) for c in range(n)])
            assert np.allclose(y[i], ref, rtol=0, atol=1e-12)
            assert np.allclose(b[i], bnd, rtol=0, atol=1e-12)
        yf, bf, _ = moe.moe_gemm_ref(a, rows_are_pairs, topk, ids, lambda e: ws[e], n)
        # (BLAS may block a subset differently: equal up to fp64 rounding)
        assert np.allclose(y, yf[pairs], rtol=1e-13, atol=1e-13)
        assert np.allclose(b, bf[pairs], rtol=1e-13, atol=1e-13)


def test_gated_rows_written_out():
    """The gated layout's row order, written out for n = 64 and n = 96 from
    the rule (device block 2i = gate rows 16i.., block 2i+1 = up rows
    d + 16i..): a swapped gate/up or a wrong block stride fails it."""
    from oracle import layout
    r = lambda a, b: list(range(a, b))
    assert list(layout.gated_rows(64)) == r(0, 16) + r(32, 48) + r(16, 32) + r(48, 64)
    assert list(layout.gated_rows(96)) == (r(0, 16) + r(48, 64) + r(16, 32) + r(64, 80) + r(32, 48)
                                           + r(80, 96))
    p = layout.gated_rows(4096)
    assert sorted(p) == list(range(4096))


def test_silu_mul_bound_slope_and_corners():
    """The slope constant bounds |silu'| (finite differences on a fine grid:
    the maximum, about 1.0998, is within 1% of it), and the bound holds at
    the worst corners of random error boxes (g +- eg, u +- eu), including
    boxes around the slope maximum and wide ones; dropping either term of
    the bound fails the corners."""
    x = np.linspace(-30, 30, 600001)
    f = x / (1 + np.exp(-x))
    slope = np.abs(np.diff(f) / np.diff(x)).max()
    assert 1.089 < slope <= moe.SILU_SLOPE
    r = np.random.default_rng(11)
    g = np.concatenate([r.normal(0, 4, 4000), np.full(200, 2.4)])
    u = r.normal(0, 3, g.size)
    eg = np.abs(r.normal(0, 0.5, g.size))
    eu = np.abs(r.normal(0, 0.5, g.size))
    b = moe.silu_mul_bound(g, u, eg, eu)
    h0 = g / (1 + np.exp(-g)) * u
    worst = np.zeros_like(g)
    for sg in (-1, 0, 1):
        for su in (-1, 1):
            gp, up = g + sg * eg, u + su * eu
            worst = np.maximum(worst, np.abs(gp / (1 + np.exp(-gp)) * up - h0))
    assert np.all(worst <= b * (1 + 1e-12))
    sgv = np.abs(g / (1 + np.exp(-g)))
    assert np.any(worst > moe.SILU_SLOPE * eg * (np.abs(u) + eu))          # the eu term is needed
    assert np.any(worst > sgv * eu)                                         # and the eg term
