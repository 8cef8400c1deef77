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
