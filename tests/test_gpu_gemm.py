"""GPU parity for the dense GEMM against the oracle (fp64 GEMM of the exact
dequantized weights): the five acceptance shapes of the workloads at full
size (large M on sampled rows), ragged shapes on both kernel paths, closed
forms, degenerate inputs and run-to-run determinism."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import codecs, gemm, quant
from gpu_util import bf16_to_dev, bits_of, quantize_experts, std_to_dev, xhat_of

pytestmark = pytest.mark.gpu


class Layer:
    """One dense layer prepared on both sides from the same fp32 weights."""

    def __init__(self, fmt, n, k, cfg=2, wseed=0):
        import quantized_gemm_int4_amd as hm
        self.fmt, self.n, self.k = fmt, n, k
        wf = synthetic.weights(cfg, n, k, index=wseed)
        codes, scales, zeros, what = quantize_experts(fmt, [wf])
        self.what = what[0].astype(np.float64)
        self.desc = hm.wdesc(fmt, n, k)
        self.w = hm.hm_transform(self.desc, *std_to_dev(fmt, codes, scales, zeros))

    def run(self, x_bits, tuning=None):
        import quantized_gemm_int4_amd as hm
        x = bf16_to_dev(x_bits)
        if self.fmt == quant.FMT_MXFP4:
            x8, s = hm.hm_quant_fp8_rows(x)
            y = hm.hm_gemm(self.desc, self.w, x8, s, tuning=tuning)
        else:
            y = hm.hm_gemm(self.desc, self.w, x, tuning=tuning)
        torch.cuda.synchronize()
        return bits_of(y)

    def check(self, x_bits, rows=None, tuning=None):
        yb = self.run(x_bits, tuning)
        xh = xhat_of(self.fmt, x_bits)
        if rows is not None:
            xh, yb = xh[rows], yb[rows]
        yref, b = gemm.gemm_ref(xh, self.what, bound_dtype=np.float32 if xh.shape[0] > 512 else np.float64)
        res = gemm.check(yb, yref, b)
        assert res["ok"], res
        return res


def test_config1_symmetric_decode():
    L = Layer(quant.FMT_INT4_SYM, 256, 512, cfg=1)
    L.check(synthetic.activations(1, 1, 512))


@pytest.fixture(scope="module")
def config2():
    return Layer(quant.FMT_UINT4_ZP, 14336, 4096, cfg=2)


@pytest.mark.parametrize("m", [1, 16, 128, 1024])
def test_config2_asym_full(config2, m):
    config2.check(synthetic.activations(2, m, 4096, index=m))


def test_config2_m4096_sampled_rows(config2):
    rows = np.random.default_rng(0).choice(4096, 96, replace=False)
    rows = np.concatenate([rows, [0, 127, 128, 4095]])
    config2.check(synthetic.activations(2, 4096, 4096, index=4096), rows=rows)


@pytest.fixture(scope="module")
def config3():
    return Layer(quant.FMT_MXFP4, 7168, 2048, cfg=3)


@pytest.mark.parametrize("m", [16, 64, 100, 128, 256])
def test_config3_mxfp4_full(config3, m):
    """W4A8 at the full layer shape: M = 64..128 stream 32-row chunks in
    eight-wave blocks (100: a ragged last chunk), 256 runs 64 x 128 tiles."""
    config3.check(synthetic.activations(3, m, 2048, index=m, outliers=0.01))


@pytest.mark.parametrize("m", [33, 100, 128])
def test_w4a8_chunked_streaming_ragged(m):
    """W4A8 rows streamed in 32-row chunks on eight-wave blocks (the default
    for 33..128 rows when the grid holds enough blocks) with N ragged against
    the block's column sets and K not a multiple of the K slices."""
    import quantized_gemm_int4_amd as hm
    L = Layer(quant.FMT_MXFP4, 7000, 2304, cfg=3, wseed=17)
    assert "stream" in hm.hm_gemm_plan(L.desc, hm.HM_A_FP8_ROWSCALE, m)
    L.check(synthetic.activations(3, m, 2304, index=m + 1, outliers=0.01))


def test_config3_m4096_sampled_rows(config3):
    rows = np.random.default_rng(1).choice(4096, 96, replace=False)
    config3.check(synthetic.activations(3, 4096, 2048, index=4096, outliers=0.01), rows=rows)


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("n,k", [(200, 384), (37, 128), (1000, 1152)])
@pytest.mark.parametrize("m", [1, 7, 16, 17, 32, 33, 100, 129, 257])
def test_ragged_default_path(fmt, n, k, m):
    L = Layer(fmt, n, k, cfg=7, wseed=n + k)
    L.check(synthetic.activations(7, m, k, index=m))


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("m", [1, 17, 32])
@pytest.mark.parametrize("path", [1, 2, 4])
def test_forced_paths_agree_with_oracle(fmt, m, path):
    L = Layer(fmt, 328, 640, cfg=8)
    L.check(synthetic.activations(8, m, 640, index=m), tuning=dict(path=path))


@pytest.mark.parametrize("splits", [1, 2, 3, 5])
def test_stream_split_counts(splits):
    L = Layer(quant.FMT_UINT4_ZP, 512, 640, cfg=9)
    L.check(synthetic.activations(9, 5, 640), tuning=dict(stream_splits=splits))


def test_one_hot_weights_exact():
    """Closed form: one nonzero code per row with a power-of-two scale makes Y a
    scaled column gather of X.  Every path multiplies exact weights (the
    streaming path feeds u - z, or q / 16, to the MFMA, the tile paths s * q),
    and every other product is an exact zero, so both reproduce it bit for
    bit, also with K split over the waves of a block or over blocks."""
    import quantized_gemm_int4_amd as hm
    n, k = 96, 512
    ks = np.random.default_rng(3).integers(0, k, size=n)
    q = np.zeros((n, k), dtype=np.int64)
    q[np.arange(n), ks] = 3
    codes = quant.pack_nibbles(q)[None]
    scales = np.full((1, n, k // 128), 0x3E00, dtype=np.uint16)     # bf16 0.125
    d = hm.wdesc("int4_sym", n, k)
    w = hm.hm_transform(d, *std_to_dev(quant.FMT_INT4_SYM, codes, scales, None))
    for m, path, extra in [(3, 1, {}), (40, 2, {}), (1, 1, {"stream_ks": 4}),
                           (16, 1, {"stream_splits": 3}), (32, 1, {})]:
        xb = synthetic.activations(10, m, k, index=m)
        y = bits_of(hm.hm_gemm(d, w, bf16_to_dev(xb), tuning=dict(extra, path=path)))
        x = codecs.bf16_value(xb).astype(np.float64)
        want = codecs.bf16_rne_bits((x[:, ks] * 0.375).astype(np.float32))
        assert np.array_equal(y, want), (m, path, extra)


@pytest.mark.parametrize("fmt", [quant.FMT_UINT4_ZP, quant.FMT_INT4_SYM])
@pytest.mark.parametrize("m", [1, 16, 32])
def test_mostly_zero_point_codes(fmt, m):
    """Groups in which 120 or more of the 128 codes equal the zero point
    (pruned or outlier-dominated groups): sum |x w| is small against sum |x|,
    and the decode path must still meet the acceptance rule element by
    element with the plain bound."""
    import quantized_gemm_int4_amd as hm
    n, k = 2048, 4096
    r = np.random.default_rng(40 + m)
    kg = k // 128
    if fmt == quant.FMT_UINT4_ZP:
        zeros = r.integers(0, 16, size=(n, kg)).astype(np.uint8)
    else:
        zeros = np.full((n, kg), 8, dtype=np.uint8)             # q = u - 8 = 0
    u = np.repeat(zeros, 128, axis=1).astype(np.int64).reshape(n, kg, 128)
    pos = np.argsort(r.random((n, kg, 128)), axis=2)[:, :, :6]   # 6 codes per group may differ
    np.put_along_axis(u, pos, r.integers(0, 16, size=pos.shape), axis=2)
    per_group = (u == zeros[:, :, None]).sum(axis=2)
    assert per_group.min() >= 122
    u = u.reshape(n, k)
    scales = (0x3B00 + r.integers(0, 0x100, size=(n, kg))).astype(np.uint16)
    if fmt == quant.FMT_INT4_SYM:
        codes = quant.pack_nibbles(u - 8)                       # two's complement q
        zz = None
    else:
        codes = quant.pack_nibbles(u)
        zz = zeros
    what = quant.dequant(fmt, codes, scales, zz).astype(np.float64)
    d = hm.wdesc(fmt, n, k)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes[None], scales[None], zz[None] if zz is not None else None))
    assert " stream " in hm.hm_gemm_plan(d, hm.HM_A_BF16, m)
    xb = synthetic.activations(19, m, k, index=m)
    y = bits_of(hm.hm_gemm(d, w, bf16_to_dev(xb)))
    yref, b = gemm.gemm_ref(codecs.bf16_value(xb).astype(np.float64), what)
    res = gemm.check(y, yref, b)
    assert res["ok"], res


@pytest.mark.parametrize("fmt", quant.FORMATS)
def test_zero_weights_give_exact_zeros(fmt):
    import quantized_gemm_int4_amd as hm
    n, k = 64, 256
    zcode = {quant.FMT_INT4_SYM: 0, quant.FMT_UINT4_ZP: 5, quant.FMT_MXFP4: 0}[fmt]
    codes = quant.pack_nibbles(np.full((n, k), zcode))[None]
    if fmt == quant.FMT_MXFP4:
        scales = np.full((1, n, k // 32), 130, dtype=np.uint8)
        zeros = None
    else:
        scales = np.full((1, n, k // 128), 0x3F80, dtype=np.uint16)
        zeros = np.full((1, n, k // 128), 5, dtype=np.uint8) if fmt == quant.FMT_UINT4_ZP else None
    d = hm.wdesc(fmt, n, k)
    w = hm.hm_transform(d, *std_to_dev(fmt, codes, scales, zeros))
    for m in (2, 50):
        xb = synthetic.activations(11, m, k, index=m)
        x = bf16_to_dev(xb)
        if fmt == quant.FMT_MXFP4:
            x8, s = hm.hm_quant_fp8_rows(x)
            y = hm.hm_gemm(d, w, x8, s)
        else:
            y = hm.hm_gemm(d, w, x)
        assert (bits_of(y) & 0x7FFF == 0).all()


def test_deterministic_repeat(config2):
    xb = synthetic.activations(2, 16, 4096, index=99)
    a = config2.run(xb)
    b = config2.run(xb)
    assert np.array_equal(a, b)


def test_m_zero_is_noop(config2):
    import quantized_gemm_int4_amd as hm
    x = torch.empty(0, 4096, dtype=torch.bfloat16, device="cuda")
    y = hm.hm_gemm(config2.desc, config2.w, x)
    assert y.shape == (0, 14336)


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("ks", [1, 2, 4])
@pytest.mark.parametrize("nbw", [1, 2])
@pytest.mark.parametrize("m", [1, 13, 32])
def test_stream_wave_splits(fmt, ks, nbw, m):
    """Every streaming launch shape: K split over 1, 2 or 4 waves of a block
    (7 groups: uneven slices, one wave with a single group), one or two column
    blocks per wave, N ragged against the block's column sets."""
    L = Layer(fmt, 200, 896, cfg=10, wseed=ks + 3 * nbw)
    x = synthetic.activations(10, m, 896, index=m)
    L.check(x, tuning=dict(path=1, stream_ks=ks, stream_nbw=nbw))


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("ks", [1, 4])
@pytest.mark.parametrize("m", [17, 32])
@pytest.mark.parametrize("splits", [1, 3])
def test_stream_multi_piece(fmt, ks, m, splits):
    """Activation rows larger than LDS: K is walked in several staged pieces
    (32 rows x 3072 bf16 or 6144 fp8 bytes exceed the 159 KiB budget)."""
    k = 6144 if fmt == quant.FMT_MXFP4 else 3072
    L = Layer(fmt, 96, k, cfg=11, wseed=ks)
    x = synthetic.activations(11, m, k, index=m + splits)
    L.check(x, tuning=dict(path=1, stream_ks=ks, stream_splits=splits))


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("m,n,k", [(1, 200, 384), (300, 1000, 1152), (513, 528, 640), (256, 256, 128),
                                   (700, 96, 256)])
def test_big_tiles_ragged(fmt, m, n, k):
    """The 256 x 256 tile kernel on ragged shapes: M and N not multiples of
    256, one or an odd number of K groups, a single row, a single tile."""
    L = Layer(fmt, n, k, cfg=13, wseed=m)
    x = synthetic.activations(13, m, k, index=m, outliers=0.01 if fmt == quant.FMT_MXFP4 else 0)
    L.check(x, tuning=dict(path=3))


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("m,n,k", [(1, 200, 384), (300, 1000, 1152), (128, 72, 128), (129, 64, 256),
                                   (77, 520, 640), (256, 136, 768), (200, 48, 896), (40, 2000, 1024)])
def test_mid_tiles_ragged(fmt, m, n, k):
    """The 128-row tile path (W4A16: 128 x 64 tiles with the K groups split
    over the waves) on ragged shapes: M and N not multiples of the tile, one
    to eight K groups (fewer than, equal to and more than the copy-ahead
    depths), a single row."""
    L = Layer(fmt, n, k, cfg=14, wseed=m + n)
    x = synthetic.activations(14, m, k, index=m, outliers=0.01 if fmt == quant.FMT_MXFP4 else 0)
    L.check(x, tuning=dict(path=2))


@pytest.mark.parametrize("fmt", [quant.FMT_UINT4_ZP, quant.FMT_INT4_SYM])
@pytest.mark.parametrize("m,halves", [(4352, 32), (4288, 32), (4160, 0)])
def test_big_half_tiles(fmt, m, halves):
    """Dense W4A16 with more 256 x 256 tiles than the persistent grid and at
    most half a round left over (N = 4096: 16 column tiles, 17 tile rows =
    272 tiles on 256 blocks): the last 16 tiles run as 32 halves of 128
    rows, the last of them holding 64 rows when M = 4288; with 64 rows in
    the last tile row (M = 4160) nothing is split.  Every output is checked."""
    import quantized_gemm_int4_amd as hm
    n, k = 4096, 256
    L = Layer(fmt, n, k, cfg=15, wseed=m)
    plan = hm.hm_gemm_plan(L.desc, hm.HM_A_BF16, m)
    assert "256x256" in plan and f"half_tiles={halves}" in plan, plan
    L.check(synthetic.activations(15, m, k, index=m))


@pytest.mark.parametrize("n,k", [(1792, 4096), (14336, 512)])
@pytest.mark.parametrize("m", [16, 128, 256, 300, 600])
def test_tp8_shard_shapes(n, k, m):
    """One rank's GEMM of the dense uint4 layer under 8-way tensor
    parallelism: the column shard (N=1792, K=4096: M = 128 and 256 stream in
    32-row chunks) and the row shard (N=14336, K=512), on the streaming,
    128-row and 256-row paths."""
    L = Layer(quant.FMT_UINT4_ZP, n, k, cfg=18, wseed=n + m)
    L.check(synthetic.activations(18, m, k, index=m))


@pytest.mark.parametrize("fmt", quant.FORMATS)
@pytest.mark.parametrize("ks", [2, 4, 8])
@pytest.mark.parametrize("nbw", [1, 2])
@pytest.mark.parametrize("m,splits", [(1, 1), (16, 2), (32, 1)])
def test_stream_eight_wave_blocks(fmt, ks, nbw, m, splits):
    """Dense streaming with eight waves per block: K split over 2, 4 or 8 of
    them (9 groups: uneven slices, waves with one group or none), one or two
    column blocks per wave, N ragged against the block's column sets, with
    and without a K split over blocks."""
    L = Layer(fmt, 216, 1152, cfg=21, wseed=ks + 5 * nbw)
    x = synthetic.activations(21, m, 1152, index=m)
    L.check(x, tuning=dict(path=1, stream_waves=8, stream_ks=ks, stream_nbw=nbw, stream_splits=splits))
