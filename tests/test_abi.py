"""The C library loads, exports every entry point include/hm.h declares, and
rejects bad arguments before any launch (no GPU needed: these calls return
before touching HIP)."""
import ctypes
import os
import re

import pytest

import quantized_gemm_int4_amd as hm
from oracle import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hm_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(hm.lib, n), n
    out = os.popen(f"nm -D --defined-only {hm.LIB_PATH}").read()
    exported = set(re.findall(r" T (hm_[a-z0-9_]+)", out))
    assert set(names) <= exported
    # nothing else leaks out of the library's namespace
    assert all(s.startswith("hm_") for s in exported)


def test_status_strings():
    for code in range(9):
        s = hm.lib.hm_status_string(code)
        assert s and s.decode() != "unknown status"
    assert hm.lib.hm_status_string(99).decode() == "unknown status"


@pytest.mark.parametrize("fmt", ["int4_sym", "uint4_zp", "mxfp4", "mxint4", "uint3_zp", "uint2_zp", "int8_sym"])
@pytest.mark.parametrize("E,N,K", [(1, 256, 512), (1, 14336, 4096), (3, 37, 640), (256, 4096, 7168)])
def test_transform_size_matches_layout_spec(fmt, E, N, K):
    d = hm.wdesc(fmt, N, K, E)
    assert hm.hm_transform_size(d) == layout.sizes(fmt, E, N, K)[2]


def _err(fn, *args):
    return getattr(hm.lib, fn)(*args)


def test_descriptor_checks():
    sz = ctypes.c_size_t()
    d = hm.wdesc("int4_sym", 256, 512)
    assert _err("hm_transform_size", None, ctypes.byref(sz)) == 1
    bad = hm.wdesc("int4_sym", 256, 512); bad.abi = 99
    assert _err("hm_transform_size", ctypes.byref(bad), ctypes.byref(sz)) == 7
    bad = hm.wdesc("int4_sym", 256, 500)                       # K not a multiple of 128
    assert _err("hm_transform_size", ctypes.byref(bad), ctypes.byref(sz)) == 2
    bad = hm.wdesc("int4_sym", 256, 512); bad.group = 64
    assert _err("hm_transform_size", ctypes.byref(bad), ctypes.byref(sz)) == 2
    bad = hm.wdesc("int4_sym", 0, 512)
    assert _err("hm_transform_size", ctypes.byref(bad), ctypes.byref(sz)) == 2
    bad = hm.wdesc("int4_sym", 256, 512); bad.wfmt = 9
    assert _err("hm_transform_size", ctypes.byref(bad), ctypes.byref(sz)) == 4
    assert _err("hm_transform_size", ctypes.byref(d), None) == 1


def test_gemm_argument_checks():
    d = hm.wdesc("uint4_zp", 256, 512)
    P = ctypes.c_void_p
    good = P(0x100000)          # aligned fake addresses: never dereferenced, calls return first
    odd = P(0x100008)
    # wrong activation format for the weight format
    assert _err("hm_gemm", ctypes.byref(d), good, 1, good, good, 4, good, None, 0, None, None) == 4
    # m = 0 is a no-op even with null pointers
    assert _err("hm_gemm", ctypes.byref(d), None, 0, None, None, 0, None, None, 0, None, None) == 0
    assert _err("hm_gemm", ctypes.byref(d), None, 0, good, None, 4, good, None, 0, None, None) == 1
    assert _err("hm_gemm", ctypes.byref(d), good, 0, good, None, -1, good, None, 0, None, None) == 2
    assert _err("hm_gemm", ctypes.byref(d), odd, 0, good, None, 4, good, None, 0, None, None) == 3
    # the streaming path at M=1 needs a split-K workspace
    need = hm.hm_gemm_workspace_size(d, 0, 1)
    assert need > 0
    assert _err("hm_gemm", ctypes.byref(d), good, 0, good, None, 1, good, None, 0, None, None) == 1
    assert _err("hm_gemm", ctypes.byref(d), good, 0, good, None, 1, good, good, need - 1, None, None) == 5
    mx = hm.wdesc("mxfp4", 256, 512)
    assert _err("hm_gemm", ctypes.byref(mx), good, 1, good, None, 4, good, None, 0, None, None) == 1
    moe = hm.wdesc("int4_sym", 256, 512, 4)
    assert _err("hm_gemm", ctypes.byref(moe), good, 0, good, None, 4, good, None, 0, None, None) == 2


def test_plan_strings():
    d = hm.wdesc("uint4_zp", 14336, 4096)
    assert "stream" in hm.hm_gemm_plan(d, 0, 1)
    assert "stream" in hm.hm_gemm_plan(d, 0, 16)
    assert "tile" in hm.hm_gemm_plan(d, 0, 4096)
    assert hm.hm_gemm_workspace_size(d, 0, 4096) == 0


def test_mxfp4_bf16_rows_plans():
    """MXFP4 weights take bf16 rows too: the streaming kernel for few rows,
    the 128 x 64 kernel above, 256 x 256 tiles from 512 rows (128 x 128 when
    forced; bf16 MFMA); MXINT4 has no 256 x 256 kernel; FP8 rows keep the
    W4A8 kernels; INT4 weights reject FP8 rows."""
    mx = hm.wdesc("mxfp4", 7168, 2048)
    for m in (1, 16, 32):
        p = hm.hm_gemm_plan(mx, hm.HM_A_BF16, m)
        assert p.startswith("w4a16-mxfp4 stream") and p.endswith("mfma=16x16x32_bf16"), p
    for m in (33, 256):
        p = hm.hm_gemm_plan(mx, hm.HM_A_BF16, m)
        assert p.startswith("w4a16-mxfp4 tile 128x64") and p.endswith("32x32x16_bf16"), p
    # estimated time in rounds of each kernel's tiles (measured round costs)
    p = hm.hm_gemm_plan(mx, hm.HM_A_BF16, 1024)
    assert p.startswith("w4a16-mxfp4 tile 128x128") and p.endswith("16x16x32_bf16"), p
    p = hm.hm_gemm_plan(mx, hm.HM_A_BF16, 4096)
    assert p.startswith("w4a16-mxfp4 tile 256x256 waves=1x4 mfma=32x32x16_bf16"), p
    assert "128x64" in hm.hm_gemm_plan(mx, hm.HM_A_BF16, 512)
    big = hm.wdesc("mxfp4", 14336, 4096)
    assert "128x128" in hm.hm_gemm_plan(big, hm.HM_A_BF16, 512)
    assert "256x256" in hm.hm_gemm_plan(big, hm.HM_A_BF16, 1024)
    assert "256x256" in hm.hm_gemm_plan(big, hm.HM_A_BF16, 4096)
    p = hm.hm_gemm_plan(mx, hm.HM_A_BF16, 256, dict(path=4))
    assert p.startswith("w4a16-mxfp4 tile 128x128") and p.endswith("16x16x32_bf16"), p
    assert "128x64" in hm.hm_gemm_plan(mx, hm.HM_A_BF16, 4096, dict(path=2))
    assert "256x256" in hm.hm_gemm_plan(mx, hm.HM_A_BF16, 256, dict(path=3))
    assert "256x256" in hm.hm_gemm_plan(hm.wdesc("mxint4", 7168, 2048), hm.HM_A_BF16, 4096, dict(path=3))
    i8 = hm.wdesc("int8_sym", 7168, 2048)
    assert "256x256" in hm.hm_gemm_plan(i8, hm.HM_A_BF16, 4096)
    assert "128x128" in hm.hm_gemm_plan(i8, hm.HM_A_BF16, 1024)
    with pytest.raises(hm.HmError) as e:             # no 128-row tile kernel for INT8
        hm.hm_gemm_plan(i8, hm.HM_A_BF16, 4096, dict(path=2))
    assert e.value.code == 8
    assert hm.hm_gemm_plan(mx, hm.HM_A_FP8_ROWSCALE, 4096).startswith("w4a8-mxfp4 tile 256x256")
    assert hm.hm_gemm_plan(mx, hm.HM_A_FP8_ROWSCALE, 1).startswith("w4a8-mxfp4 stream")
    # W4A8 streams up to four 32-row chunks in eight-wave blocks without a K split
    for m, nbw in ((33, 1), (64, 1), (96, 2), (128, 2)):
        p = hm.hm_gemm_plan(mx, hm.HM_A_FP8_ROWSCALE, m)
        assert p.startswith(f"w4a8-mxfp4 stream mb=2 nbw={nbw} ks=2 waves=8 splits=1"), (m, p)
    for m in (129, 256):
        assert hm.hm_gemm_plan(mx, hm.HM_A_FP8_ROWSCALE, m).startswith("w4a8-mxfp4 tile 64x128")
    # a narrow N whose chunk grid would be under 128 blocks stays on tiles
    narrow = hm.wdesc("mxfp4", 2048, 7168)
    assert hm.hm_gemm_plan(narrow, hm.HM_A_FP8_ROWSCALE, 64).startswith("w4a8-mxfp4 tile 64x128")
    sz = ctypes.c_size_t()
    i4 = hm.wdesc("int4_sym", 256, 512)
    assert _err("hm_gemm_workspace_size", ctypes.byref(i4), 1, 4, None, ctypes.byref(sz)) == 4
    moe = hm.wdesc("mxfp4", 4096, 7168, 256)
    assert _err("hm_moe_gemm_workspace_size", ctypes.byref(moe), 0, 64, 8, None, ctypes.byref(sz)) == 0
    assert sz.value > 0


def test_mxint4_pairs_and_plans():
    """MXINT4 (group 32) takes bf16 rows only, on the same kernels as MXFP4 with bf16 rows."""
    sz = ctypes.c_size_t()
    d = hm.wdesc("mxint4", 7168, 2048)
    bad = hm.wdesc("mxint4", 7168, 2048); bad.group = 128
    assert _err("hm_transform_size", ctypes.byref(bad), ctypes.byref(sz)) == 2
    assert _err("hm_gemm_workspace_size", ctypes.byref(d), 1, 16, None, ctypes.byref(sz)) == 4
    assert hm.hm_gemm_plan(d, hm.HM_A_BF16, 16).startswith("w4a16-mxint4 stream")
    assert hm.hm_gemm_plan(d, hm.HM_A_BF16, 256).startswith("w4a16-mxint4 tile 128x64")
    assert hm.hm_gemm_plan(d, hm.HM_A_BF16, 4096).startswith("w4a16-mxint4 tile 256x256")
    assert "128x64" in hm.hm_gemm_plan(d, hm.HM_A_BF16, 4096, dict(path=2))


def test_moe_argument_checks():
    P = ctypes.c_void_p
    good = P(0x100000)
    assert _err("hm_moe_sort", good, 4, 9, 8, good, good, good, None, 0, None) == 2      # topk > E
    assert _err("hm_moe_sort", good, 4, 2, 600, good, good, good, None, 0, None) == 2    # E > 512
    assert _err("hm_moe_sort", None, 0, 2, 8, None, None, None, None, 0, None) == 0      # t = 0
    assert _err("hm_moe_sort", None, 4, 2, 8, good, good, good, None, 0, None) == 1
    assert _err("hm_moe_sort", P(0x100002), 4, 2, 8, good, good, good, None, 0, None) == 3
    # one workgroup up to 4096 pairs (no workspace), then ~2048-pair chunks
    # of E counts each, at most 512 chunks
    assert hm.hm_moe_sort_workspace_size(512, 8, 256) == 0
    assert hm.hm_moe_sort_workspace_size(4096, 1, 7) == 0
    assert hm.hm_moe_sort_workspace_size(4097, 1, 7) == 3 * 7 * 4
    assert hm.hm_moe_sort_workspace_size(16384, 8, 256) == 64 * 256 * 4
    assert hm.hm_moe_sort_workspace_size(2 ** 28 - 1, 8, 512) == 512 * 512 * 4
    assert _err("hm_moe_sort", good, 1024, 8, 256, good, good, good, None, 0, None) == 1     # ws needed
    assert _err("hm_moe_sort", good, 1024, 8, 256, good, good, good, good, 4095, None) == 5
    assert _err("hm_moe_sort", good, 1024, 8, 256, good, good, good, P(0x100002), 4096, None) == 3
    d = hm.wdesc("int4_sym", 4096, 7168, 256)
    need = hm.hm_moe_gemm_workspace_size(d, 0, 64, 8)
    assert need > 0
    args = (ctypes.byref(d), good, 0, good, None, 0, 64, 8, good, good, good, good)
    assert _err("hm_moe_gemm", *args, need - 1, None, None) == 5
    assert _err("hm_moe_gemm", ctypes.byref(d), good, 0, good, None, 2, 64, 8, good, good, good,
                good, need, None, None) == 2
    assert _err("hm_moe_gemm", ctypes.byref(d), good, 0, good, None, 0, 64, 8, None, good, good,
                good, need, None, None) == 1


def test_moe_block_argument_checks():
    """Validation of the MoE block steps happens before any launch."""
    P = ctypes.c_void_p
    good = P(0x100000)
    assert _err("hm_silu_mul", good, 4, 0, good, None) == 2                 # d <= 0
    assert _err("hm_silu_mul", good, -1, 8, good, None) == 2                # rows < 0
    assert _err("hm_silu_mul", None, 0, 8, None, None) == 0                 # rows = 0: no-op
    assert _err("hm_silu_mul", None, 4, 8, good, None) == 1
    assert _err("hm_silu_mul", good, 4, 8, P(0x100008), None) == 3          # h not 16-byte aligned
    assert _err("hm_moe_combine", good, good, 4, 0, 8, good, None) == 2     # topk < 1
    assert _err("hm_moe_combine", good, good, 4, 2, 0, good, None) == 2     # n <= 0
    assert _err("hm_moe_combine", None, None, 0, 2, 8, None, None) == 0     # t = 0: no-op
    assert _err("hm_moe_combine", good, None, 4, 2, 8, good, None) == 1
    assert _err("hm_moe_combine", good, P(0x100002), 4, 2, 8, good, None) == 3   # w not 4-byte aligned


def test_tile_kernel_choice_by_rounds():
    """The dense planner takes 256 x 256 tiles unless 128 x 64 tiles need
    fewer rounds of the chip (a round of large tiles costs ~3.8 small ones):
    the TP8 column shard (N = 1792) runs its M = 512..2048 on the 128-row
    kernel, the full layer and the row shard keep 256 x 256 from M = 512."""
    col = hm.wdesc("uint4_zp", 1792, 4096)
    full = hm.wdesc("uint4_zp", 14336, 4096)
    row = hm.wdesc("uint4_zp", 14336, 512)
    for m in (512, 1024, 2048):
        assert "128x64" in hm.hm_gemm_plan(col, 0, m)
    # narrow N streams up to 256 rows while 32-row chunks x N <= 16384
    for m in (48, 128, 256):
        assert " stream " in hm.hm_gemm_plan(col, 0, m)
    assert "128x64" in hm.hm_gemm_plan(col, 0, 257)
    for m in (33, 64, 128):
        assert "128x64" in hm.hm_gemm_plan(full, 0, m)
    assert "256x256" in hm.hm_gemm_plan(col, 0, 4096)
    for d in (full, row):
        for m in (512, 1024, 4096):
            assert "256x256" in hm.hm_gemm_plan(d, 0, m)
    assert "128x64" in hm.hm_gemm_plan(full, 0, 511)
    assert "half_tiles=256" in hm.hm_gemm_plan(full, 0, 4096)


def test_tuning_validation():
    """Explicit tuning: out-of-range fields and forced kernels that cannot run
    the call give HM_ERR_TUNING (8) before any launch; a wrong abi gives
    HM_ERR_ABI; the plan reports what a tuning selects."""
    d = hm.wdesc("uint4_zp", 14336, 4096)
    sz = ctypes.c_size_t()
    for bad in (dict(path=5), dict(stream_ks=3), dict(stream_nbw=4), dict(stream_splits=-1),
                dict(moe_stream_rows=8), dict(moe_stream_max=5000), dict(moe_stream_lds_kb=10),
                dict(moe_big_min=300), dict(moe_tile=3)):
        t = hm.make_tuning(**bad)
        assert _err("hm_gemm_workspace_size", ctypes.byref(d), 0, 16, ctypes.byref(t), ctypes.byref(sz)) == 8, bad
    t = hm.make_tuning()
    t.abi = 1
    assert _err("hm_gemm_workspace_size", ctypes.byref(d), 0, 16, ctypes.byref(t), ctypes.byref(sz)) == 7
    # streaming is for at most 256 rows; K splits at most K / 128
    assert _err("hm_gemm_workspace_size", ctypes.byref(d), 0, 257, ctypes.byref(hm.make_tuning(path=1)),
                ctypes.byref(sz)) == 8
    assert _err("hm_gemm_workspace_size", ctypes.byref(d), 0, 16, ctypes.byref(hm.make_tuning(stream_splits=33)),
                ctypes.byref(sz)) == 8
    p = hm.hm_gemm_plan(d, 0, 16, dict(stream_ks=4, stream_nbw=1, stream_splits=4))
    assert "ks=4" in p and "nbw=1" in p and "splits=4" in p, p
    assert hm.hm_gemm_workspace_size(d, 0, 16, dict(stream_splits=4)) == 4 * 16 * 14336 * 4
    assert hm.hm_gemm_workspace_size(d, 0, 16, dict(stream_splits=1)) == 0
    for path, tag in ((1, " stream "), (2, "128x64"), (3, "256x256"), (4, "128x128")):
        assert tag in hm.hm_gemm_plan(d, 0, 200, dict(path=path))
    # an all-zero tuning is the default choice
    for m in (1, 16, 128, 1024, 4096):
        assert hm.hm_gemm_plan(d, 0, m, hm.make_tuning()) == hm.hm_gemm_plan(d, 0, m)


def test_moe_big_unit_threshold_by_k():
    """Expert remainders take 256-row units from 49 rows when K <= 2048 (short
    K loops: the down projection) and from 97 rows otherwise; an explicit
    moe_big_min overrides both."""
    for k, rows in ((2048, 49), (1024, 49), (2176, 97), (7168, 97)):
        for fmt in ("int4_sym", "uint4_zp", "mxfp4"):
            d = hm.wdesc(fmt, 4096, k, 64)
            p = hm.hm_moe_gemm_plan(d, 0, 1024, 8, 1)
            assert f"k_gemm_big from {rows} rows" in p, (fmt, k, p)
    d = hm.wdesc("int4_sym", 4096, 2048, 64)
    assert "k_gemm_big from 97 rows" in hm.hm_moe_gemm_plan(d, 0, 1024, 8, 1, dict(moe_big_min=97))
    assert "k_gemm_big from 129 rows" in hm.hm_moe_gemm_plan(d, 0, 1024, 8, 1, dict(moe_big_min=129))


def test_moe_plan_and_large_activation_guard():
    """The grouped GEMM's unit kinds, and the guard for activations of 4 GiB
    or more: the 128-row tile kernels and the 256-row kernel address
    activation rows with 32-bit offsets, so such calls schedule their
    up-to-128-row units on the 128 x 128 kernel (64-bit row addressing) and
    take no 256-row units; forcing either gives HM_ERR_TUNING."""
    gu = hm.wdesc("int4_sym", 4096, 7168, 256)
    dn = hm.wdesc("int4_sym", 7168, 2048, 256)
    p = hm.hm_moe_gemm_plan(gu, 0, 8192, 8, 0)
    assert "stream(rows=16 max=64 nbw=2" in p and "k_gemm_mid 128x64" in p and "k_gemm_big from 97 rows" in p, p
    assert "activations>=4GiB" not in p
    # down projection, bf16 rows: P = t * 8 pairs of 2048 * 2 bytes; 4 GiB at P = 2^20
    small = hm.hm_moe_gemm_plan(dn, 0, (1 << 17) - 1, 8, 1)
    assert "k_gemm_mid 128x64" in small and "k_gemm_big" in small and ">=4GiB" not in small, small
    big = hm.hm_moe_gemm_plan(dn, 0, 1 << 17, 8, 1)
    assert "k_gemm_tile 128x128" in big and "big(256 rows)=none" in big and "activations>=4GiB" in big, big
    # the same token count with token-indexed rows (gate_up) stays below 4 GiB
    assert ">=4GiB" not in hm.hm_moe_gemm_plan(hm.wdesc("int4_sym", 4096, 2048, 256), 0, 1 << 17, 8, 0)
    for bad in (dict(moe_tile=1), dict(moe_big_min=97)):
        with pytest.raises(hm.HmError) as e:
            hm.hm_moe_gemm_plan(dn, 0, 1 << 17, 8, 1, bad)
        assert e.value.code == 8
    # FP8 rows take one byte per value: 4 GiB at P = 2^21 for K = 2048
    mx = hm.wdesc("mxfp4", 7168, 2048, 256)
    assert ">=4GiB" not in hm.hm_moe_gemm_plan(mx, 1, (1 << 18) - 1, 8, 1)
    assert "k_gemm_tile 128x128" in hm.hm_moe_gemm_plan(mx, 1, 1 << 18, 8, 1)
    # MX weights with bf16 rows take 256-row units, INT8 ones never
    mxa = hm.hm_moe_gemm_plan(mx, 0, 8192, 8, 1)
    assert "k_gemm_big from 49 rows" in mxa, mxa
    mxi = hm.hm_moe_gemm_plan(hm.wdesc("mxint4", 7168, 2048, 256), 0, 8192, 8, 1)
    assert "k_gemm_big from 49 rows" in mxi, mxi
    i8p = hm.hm_moe_gemm_plan(hm.wdesc("int8_sym", 7168, 2048, 256), 0, 8192, 8, 1)
    assert "k_gemm_big from 49 rows" in i8p and "k_gemm_tile" in i8p, i8p
    # explicit tuning shows up in the plan and in the workspace size
    t = dict(moe_stream_rows=32, moe_stream_max=128, moe_stream_nbw=1, moe_big_min=-1, moe_tile=2)
    p2 = hm.hm_moe_gemm_plan(gu, 0, 1024, 8, 0, t)
    assert "stream(rows=32 max=128 nbw=1" in p2 and "k_gemm_tile" in p2 and "big(256 rows)=none" in p2, p2
    assert hm.hm_moe_gemm_workspace_size(gu, 0, 1024, 8, t) > 0


def test_read_probe_argument_checks():
    P = ctypes.c_void_p
    good = P(0x100000)
    assert _err("hm_read_probe", good, 0, 64, 4, good, None) == 2          # no bytes
    assert _err("hm_read_probe", good, 24, 64, 4, good, None) == 2         # not a multiple of 16
    assert _err("hm_read_probe", good, 1024, 0, 4, good, None) == 2        # no blocks
    assert _err("hm_read_probe", good, 1024, 64, 3, good, None) == 2       # unroll
    assert _err("hm_read_probe", None, 1024, 64, 4, good, None) == 1
    assert _err("hm_read_probe", P(0x100008), 1024, 64, 4, good, None) == 3


def test_tuner_candidates_are_valid_and_distinct():
    """The autotuner's search space: every candidate is accepted by the
    planner, selects a distinct kernel configuration, and the default choice
    comes first; grouped candidates likewise (no GPU needed: plans only)."""
    from quantized_gemm_int4_amd import tune
    d = hm.wdesc("uint4_zp", 14336, 4096)
    for m in (1, 16, 128, 300, 4096):
        cands = tune.dense_candidates(d, 0, m)
        assert cands[0] == {}
        plans = [hm.hm_gemm_plan(d, 0, m, c or None) for c in cands]
        assert len(set(plans)) == len(plans)
        assert any(" stream " in p for p in plans) == (m <= 256)
        assert any("256x256" in p for p in plans) and any("128x128" in p for p in plans)
    i8 = hm.wdesc("int8_sym", 7168, 2048)
    assert not any("128x64" in hm.hm_gemm_plan(i8, 0, 64, c or None) for c in tune.dense_candidates(i8, 0, 64))
    mx = hm.wdesc("mxfp4", 7168, 2048)
    assert any("256x256" in hm.hm_gemm_plan(mx, 0, 64, c or None) for c in tune.dense_candidates(mx, 0, 64))
    moe = hm.wdesc("int4_sym", 4096, 7168, 256)
    mc = tune.moe_candidates(moe, 0, 1024, 8, 0)
    mplans = [hm.hm_moe_gemm_plan(moe, 0, 1024, 8, 0, c or None) for c in mc]
    assert mc[0] == {} and len(set(mplans)) == len(mplans) > 10


def test_tuning_table_lookup(tmp_path):
    from quantized_gemm_int4_amd import tune
    d = hm.wdesc("uint4_zp", 512, 1024)
    t = tune.Table(meta=dict(device="test"))
    t.put(tune._key(d, 0), 16, dict(path=1, stream_ks=2), 5.0, 6.0, "p16")
    t.put(tune._key(d, 0), 128, {}, 9.0, 9.0, "p128")
    f = tmp_path / "t.json"
    t.save(str(f))
    t2 = tune.Table.load(str(f))
    assert t2.lookup(d, 0, 1) == dict(path=1, stream_ks=2)        # next tuned row count up
    assert t2.lookup(d, 0, 16) == dict(path=1, stream_ks=2)
    assert t2.lookup(d, 0, 17) is None                             # tuned default
    assert t2.lookup(d, 0, 5000) is None                           # beyond: the largest
    assert t2.lookup(hm.wdesc("uint4_zp", 512, 2048), 0, 16) is None
    assert t2.meta["device"] == "test"


def test_static_moe_gemm_limits():
    """The allocation-free grouped GEMM rejects calls whose work lists exceed
    its static array (HM_ERR_WORKSPACE) and bad arguments before any launch."""
    P = ctypes.c_void_p
    good = P(0x100000)
    cap = hm.hm_moe_gemm_static_max_workspace()
    assert cap == 4 << 20
    d = hm.wdesc("int4_sym", 4096, 7168, 256)
    t_big = 500000                                              # 4 million pairs
    assert hm.hm_moe_gemm_workspace_size(d, 0, t_big, 8) > cap
    assert hm.hm_moe_gemm_workspace_size(d, 0, 200000, 8) <= cap
    args = (ctypes.byref(d), good, 0, good, None, 0)
    assert _err("hm_moe_gemm_static", *args, t_big, 8, good, good, good, None, None) == 5
    assert _err("hm_moe_gemm_static", *args, 0, 8, None, None, None, None, None) == 0      # t = 0
    assert _err("hm_moe_gemm_static", *args, 64, 8, None, good, good, None, None) == 1     # no offsets
    assert _err("hm_moe_gemm_static", *args, 64, 8, good, good, P(0x100008), None, None) == 3
    assert _err("hm_moe_gemm_static", ctypes.byref(d), good, 0, good, None, 2, 64, 8, good, good, good,
                None, None) == 2
