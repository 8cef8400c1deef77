"""GPU parity for the MoE path: the expert sort is exact (counts, offsets and
the stable pair order), and the grouped GEMM matches the oracle's per-expert
fp64 GEMM for every pair, on small shapes that mix streaming units (small
experts, cut into 16- or 32-row units), 128-row and 256-row tile units, and
at the workload sizes on sampled pairs."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, moe, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev, to_dev, xhat_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("t,topk,E", [(1, 1, 1), (64, 8, 256), (1024, 8, 256), (333, 3, 17),
                                      (5000, 6, 512), (16384, 8, 256), (4096, 1, 7), (4097, 1, 7),
                                      (140000, 8, 256)])
def test_sort_exact(t, topk, E):
    """One workgroup up to 4096 pairs, chunks of ~2048 pairs above (4097
    pairs: three ragged chunks; 1.12 M pairs: the 512-chunk cap)."""
    import quantized_gemm_int4_amd as hm
    if E == 256 and topk == 8:
        ids, _ = synthetic.router_topk(4, t, E, topk)
    else:
        ids = np.random.default_rng(t).integers(0, E, size=(t, topk)).astype(np.int32)
    c, o, sp = hm.hm_moe_sort(to_dev(ids), E)
    torch.cuda.synchronize()
    rc, ro, rsp = moe.moe_sort_ref(ids, E)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert np.array_equal(o.cpu().numpy(), ro)
    assert np.array_equal(sp.cpu().numpy(), rsp)


def test_sort_chunks_drop_out_of_range_ids_and_reuse_workspace():
    """Chunked sort with ids outside [0, E) in every chunk, into one caller
    workspace used twice (the second call with fewer pairs)."""
    import quantized_gemm_int4_amd as hm
    E = 40
    ws = torch.empty(hm.hm_moe_sort_workspace_size(9000, 4, E), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    for t in (9000, 3000):
        ids = np.random.default_rng(t).integers(-3, E + 3, size=(t, 4)).astype(np.int32)
        c, o, sp = hm.hm_moe_sort(to_dev(ids), E, ws=ws)
        torch.cuda.synchronize()
        flat = ids.ravel()
        keep = np.nonzero((flat >= 0) & (flat < E))[0]          # the pairs that are placed
        rc, ro, rsub = moe.moe_sort_ref(flat[keep], E)
        n = int(ro[-1])
        assert n == keep.size < flat.size
        assert np.array_equal(c.cpu().numpy(), rc)
        assert np.array_equal(o.cpu().numpy(), ro)
        assert np.array_equal(sp.cpu().numpy()[:n], keep[rsub])


def test_sort_drops_out_of_range_ids():
    import quantized_gemm_int4_amd as hm
    ids = np.array([[0, 3], [-1, 2], [4, 0], [2, 99]], dtype=np.int32)
    c, o, sp = hm.hm_moe_sort(to_dev(ids), 4)
    c, o, sp = c.cpu().numpy(), o.cpu().numpy(), sp.cpu().numpy()
    assert list(c) == [2, 0, 2, 1]
    assert list(o) == [0, 2, 2, 4, 5]
    assert list(sp[:5]) == [0, 5, 3, 6, 1]


def _skewed_ids(t, topk, E, seed):
    """Distinct experts per token with a skew: expert 0 and 1 get most tokens
    (tile units), the rest few (streaming units)."""
    r = np.random.default_rng(seed)
    p = np.array([40.0, 20.0] + [1.0] * (E - 2))
    p /= p.sum()
    return np.stack([r.choice(E, topk, replace=False, p=p) for _ in range(t)]).astype(np.int32)


def _run_moe(fmt, E, n, k, t, topk, ids, rows_are_pairs, seed, tuning=None):
    import quantized_gemm_int4_amd as hm
    ws = [synthetic.weights(12, n, k, index=seed * 100 + e) for e in range(E)]
    codes, scales, zeros, what = quantize_experts(fmt, ws)
    d = hm.wdesc(fmt, n, k, E)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros))
    P = t * topk
    rows = P if rows_are_pairs else t
    xb = synthetic.activations(12, rows, k, index=seed, outliers=0.01 if fmt == quant.FMT_MXFP4 else 0)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    x = bf16_to_dev(xb)
    if fmt == quant.FMT_MXFP4:
        x8, s = hm.hm_quant_fp8_rows(x)
        y = hm.hm_moe_gemm(d, w, x8, off, sp, t, topk, rows_are_pairs, a_scales=s, tuning=tuning)
    else:
        y = hm.hm_moe_gemm(d, w, x, off, sp, t, topk, rows_are_pairs, tuning=tuning)
    torch.cuda.synchronize()
    xh = xhat_of(fmt, xb)
    yref, b, _ = moe.moe_gemm_ref(xh, bool(rows_are_pairs), topk, ids,
                                  lambda e: what[e].astype(np.float64), n)
    res = gemm.check(bits_of(y), yref, b)
    assert res["ok"], res


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("rows_are_pairs", [0, 1])
@pytest.mark.parametrize("mid", [1, 0])
def test_moe_mixed_units(fmt, rows_are_pairs, mid):
    """Streaming, 128-row and 256-row units in one call; W4A16 128-row units
    on the 128 x 64 tile kernel (mid=1, the default) or the 128 x 128 one."""
    t, topk, E, n, k = 150, 2, 8, 208, 384
    ids = _skewed_ids(t, topk, E, 1)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() > 128 and (counts[counts > 0] <= 32).any()   # both kernels used, multi-unit
    _run_moe(fmt, E, n, k, t, topk, ids, rows_are_pairs, 1, tuning=dict(moe_tile=1 if mid else 2))


@pytest.mark.parametrize("fmt", [quant.FMT_INT4_SYM, quant.FMT_MXFP4])
def test_moe_single_expert_top1(fmt):
    t, topk, E, n, k = 77, 1, 1, 160, 256
    ids = np.zeros((t, 1), dtype=np.int32)
    _run_moe(fmt, E, n, k, t, topk, ids, 0, 2)


def test_moe_router_small():
    t, topk, E, n, k = 64, 8, 32, 128, 256
    ids, _ = synthetic.router_topk(5, t, E, topk)
    _run_moe(quant.FMT_INT4_SYM, E, n, k, t, topk, ids, 0, 3)


def _random_codes_dev(fmt, E, n, k, seed):
    """Random standard-format weights generated on the device (values do not
    matter for these shape tests); returns device tensors."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    codes = torch.randint(0, 256, (E, n, k // 2), dtype=torch.uint8, device="cuda", generator=g)
    if fmt == quant.FMT_MXFP4:
        scales = torch.randint(118, 122, (E, n, k // 32), dtype=torch.uint8, device="cuda", generator=g)
        zeros = None
    else:
        scales = (0x3B00 + torch.randint(0, 0x100, (E, n, k // 128), device="cuda", generator=g)).to(torch.int16)
        zeros = (torch.randint(0, 16, (E, n, k // 128), dtype=torch.uint8, device="cuda", generator=g)
                 if fmt == quant.FMT_UINT4_ZP else None)
    return codes, scales, zeros


@pytest.mark.parametrize("fmt,t,proj", [(quant.FMT_INT4_SYM, 64, "gate_up"), (quant.FMT_INT4_SYM, 1024, "down"),
                                        (quant.FMT_MXFP4, 1024, "gate_up"), (quant.FMT_MXFP4, 512, "down")])
def test_moe_workload_size_sampled(fmt, t, proj):
    """256 experts, top-8 Zipf routing, gate_up N=4096 K=7168 / down N=7168 K=2048,
    checked on pairs sampled from the largest and a few small experts."""
    import quantized_gemm_int4_amd as hm
    E, topk = 256, 8
    n, k = (4096, 7168) if proj == "gate_up" else (7168, 2048)
    rows_are_pairs = 0 if proj == "gate_up" else 1
    codes, scales, zeros = _random_codes_dev(fmt, E, n, k, 7)
    d = hm.wdesc(fmt, n, k, E)
    w = hm.hm_transform(d, codes, scales, zeros)
    ids, _ = synthetic.router_topk(4 if fmt == quant.FMT_INT4_SYM else 5, t, E, topk)
    P = t * topk
    xb = synthetic.activations(13, P if rows_are_pairs else t, k, outliers=0.01 if fmt == quant.FMT_MXFP4 else 0)
    _, off, sp = hm.hm_moe_sort(to_dev(ids), E)
    x = bf16_to_dev(xb)
    if fmt == quant.FMT_MXFP4:
        x8, s = hm.hm_quant_fp8_rows(x)
        y = hm.hm_moe_gemm(d, w, x8, off, sp, t, topk, rows_are_pairs, a_scales=s)
    else:
        y = hm.hm_moe_gemm(d, w, x, off, sp, t, topk, rows_are_pairs)
    torch.cuda.synchronize()
    counts = np.bincount(ids.ravel(), minlength=E)
    flat = ids.ravel()
    big = int(np.argmax(counts))
    small = [e for e in np.argsort(counts) if counts[e] > 0][:3]
    r = np.random.default_rng(0)
    pairs = np.concatenate([r.choice(np.nonzero(flat == big)[0], 24, replace=False)] +
                           [np.nonzero(flat == e)[0][:4] for e in small])
    xh = xhat_of(fmt, xb)
    cache = {}

    def what(e):
        if e not in cache:
            st_c = codes[e].cpu().numpy()
            st_s = scales[e].cpu().numpy().view(np.uint16) if fmt != quant.FMT_MXFP4 else scales[e].cpu().numpy()
            st_z = zeros[e].cpu().numpy() if zeros is not None else None
            cache[e] = quant.dequant(fmt, st_c, st_s, st_z).astype(np.float64)
        return cache[e]

    yref, b, _ = moe.moe_gemm_ref(xh, bool(rows_are_pairs), topk, ids, what, n, pairs=pairs)
    res = gemm.check(bits_of(y)[pairs], yref, b)
    assert res["ok"], res


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("ks", [2, 4])
def test_moe_stream_wave_splits(fmt, ks):
    """Streaming units with K split over 2 or 4 waves of a block (K = 5 groups:
    uneven slices, and with 4 waves one wave holds a single group)."""
    t, topk, E, n, k = 150, 2, 8, 208, 640
    ids = _skewed_ids(t, topk, E, 3)
    _run_moe(fmt, E, n, k, t, topk, ids, 0, 3, tuning=dict(moe_stream_ks=ks))


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("rows_are_pairs", [0, 1])
@pytest.mark.parametrize("big", [1, 0])
def test_moe_big_units(fmt, rows_are_pairs, big):
    """Experts large enough for 256-row units: 600 rows (two units of 256 and
    an 88-row tile unit), 450 rows (256 + a 194-row remainder, which takes a
    second 256-row unit), 100 rows (tile unit) and a few rows (streaming), on
    K = 5 groups and ragged N; with HM_MOE_BIG=0 the same call uses tile
    units only."""
    t, topk, E, n, k = 600, 2, 6, 288, 640
    r = np.random.default_rng(7)
    ids = np.zeros((t, topk), dtype=np.int32)
    ids[:, 0] = 0                                   # expert 0: 600 rows
    second = np.concatenate([np.full(450, 1), np.full(100, 2), np.full(30, 3), np.full(12, 4),
                             np.full(8, 5)])
    ids[:, 1] = r.permutation(second)
    _run_moe(fmt, E, n, k, t, topk, ids, rows_are_pairs, 9, tuning=None if big else dict(moe_big_min=-1))


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("s_max,nbw,s_rows", [(64, 2, 16), (128, 1, 16), (128, 2, 32), (16, 2, 16)])
def test_moe_stream_multi_unit(fmt, s_max, nbw, s_rows):
    """Experts of 120, 64, 33, 17, 16 and 5 rows: those with at most s_max
    rows stream as several consecutive units of s_rows rows (the others take
    tile units), with one or two 16-column blocks per wave on a ragged N (13
    column blocks) and K = 5 groups."""
    t, topk, E, n, k = 255, 1, 6, 208, 640
    r = np.random.default_rng(11)
    ids = r.permutation(np.concatenate([np.full(c, e) for e, c in enumerate([120, 64, 33, 17, 16, 5])]))
    ids = ids.reshape(t, topk).astype(np.int32)
    _run_moe(fmt, E, n, k, t, topk, ids, 0, 13,
             tuning=dict(moe_stream_max=s_max, moe_stream_nbw=nbw, moe_stream_rows=s_rows))
