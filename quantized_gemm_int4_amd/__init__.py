"""Python binding of the MI355X low-bit GEMM library (libhm.so).

Thin argument marshalling only: every function takes torch tensors (device
memory), passes their data pointers, sizes and the current HIP stream to the C
entry point of the same name, and raises HmError on a non-zero status.  All
work runs in the library's HIP kernels.  Importing this package fails loudly if
libhm.so has not been built (python quantized_gemm_int4_amd/build.py).

The C functions are declared and documented in include/hm.h.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhm.so")

HM_ABI_VERSION = 2
HM_W_INT4_SYM, HM_W_UINT4_ZP, HM_W_MXFP4, HM_W_MXINT4, HM_W_UINT3_ZP, HM_W_UINT2_ZP, HM_W_INT8_SYM = range(7)
HM_A_BF16, HM_A_FP8_ROWSCALE, HM_A_MXFP4 = 0, 1, 2
WFMT = {"int4_sym": HM_W_INT4_SYM, "uint4_zp": HM_W_UINT4_ZP, "mxfp4": HM_W_MXFP4, "mxint4": HM_W_MXINT4,
        "uint3_zp": HM_W_UINT3_ZP, "uint2_zp": HM_W_UINT2_ZP, "int8_sym": HM_W_INT8_SYM}
CODE_BITS = {HM_W_UINT3_ZP: 3, HM_W_UINT2_ZP: 2, HM_W_INT8_SYM: 8}     # other formats: 4
STATUS = {0: "HM_OK", 1: "HM_ERR_NULL", 2: "HM_ERR_SHAPE", 3: "HM_ERR_ALIGN",
          4: "HM_ERR_UNSUPPORTED", 5: "HM_ERR_WORKSPACE", 6: "HM_ERR_HIP", 7: "HM_ERR_ABI", 8: "HM_ERR_TUNING"}
HM_PATH_STREAM, HM_PATH_MID, HM_PATH_BIG, HM_PATH_TILE = 1, 2, 3, 4


class HmError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({lib.hm_status_string(code).decode()})")


class hm_wdesc(ctypes.Structure):
    _fields_ = [("abi", ctypes.c_int32), ("wfmt", ctypes.c_int32), ("group", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64)]


class hm_tuning(ctypes.Structure):
    _fields_ = [("abi", ctypes.c_int32), ("path", ctypes.c_int32), ("stream_ks", ctypes.c_int32),
                ("stream_nbw", ctypes.c_int32), ("stream_splits", ctypes.c_int32), ("stream_waves", ctypes.c_int32),
                ("moe_stream_rows", ctypes.c_int32), ("moe_stream_max", ctypes.c_int32),
                ("moe_stream_nbw", ctypes.c_int32), ("moe_stream_ks", ctypes.c_int32),
                ("moe_stream_lds_kb", ctypes.c_int32), ("moe_big_min", ctypes.c_int32),
                ("moe_tile", ctypes.c_int32)]


TUNING_FIELDS = tuple(f for f, _ in hm_tuning._fields_ if f != "abi")


def make_tuning(**fields):
    """Explicit choices of one call (hm_tuning); unnamed fields keep the default."""
    t = hm_tuning(HM_ABI_VERSION)
    for k, v in fields.items():
        if k not in TUNING_FIELDS:
            raise ValueError(f"unknown tuning field {k}")
        setattr(t, k, int(v))
    return t


def _tune(t):
    if t is None:
        return None
    if isinstance(t, dict):
        t = make_tuning(**t)
    return ctypes.byref(t)


def wdesc(wfmt, n, k, num_experts=1):
    """Layer description; wfmt is an HM_W_* value or 'int4_sym' / 'uint4_zp' / 'mxfp4'."""
    f = WFMT.get(wfmt, wfmt)
    return hm_wdesc(HM_ABI_VERSION, int(f), 32 if f in (HM_W_MXFP4, HM_W_MXINT4) else 128, int(num_experts),
                    int(n), int(k))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python quantized_gemm_int4_amd/build.py` (needs hipcc)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(hm_wdesc)
    T = ctypes.POINTER(hm_tuning)
    sig = {
        "hm_transform_size": [D, ctypes.POINTER(SZ)],
        "hm_transform": [D, P, P, P, P, SZ, P],
        "hm_transform_gated": [D, P, P, P, P, SZ, P],
        "hm_dequant": [D, P, SZ, I32, P, P],
        "hm_quant_fp8_rows": [P, I64, I64, P, P, P],
        "hm_quant_mxfp4_rows": [P, I64, I64, P, P, P],
        "hm_gemm_workspace_size": [D, I32, I64, T, ctypes.POINTER(SZ)],
        "hm_gemm": [D, P, I32, P, P, I64, P, P, SZ, T, P],
        "hm_gemm_plan": [D, I32, I64, T, ctypes.c_char_p, SZ],
        "hm_moe_sort_workspace_size": [I64, I32, I32, ctypes.POINTER(SZ)],
        "hm_moe_sort": [P, I64, I32, I32, P, P, P, P, SZ, P],
        "hm_moe_gemm_workspace_size": [D, I32, I64, I32, T, ctypes.POINTER(SZ)],
        "hm_moe_gemm": [D, P, I32, P, P, I32, I64, I32, P, P, P, P, SZ, T, P],
        "hm_moe_gemm_gated": [D, P, I32, P, P, I32, I64, I32, P, P, P, P, SZ, T, P],
        "hm_moe_gemm_plan": [D, I32, I64, I32, I32, T, ctypes.c_char_p, SZ],
        "hm_moe_gemm_gated_plan": [D, I32, I64, I32, I32, T, ctypes.c_char_p, SZ],
        "hm_silu_mul": [P, I64, I64, P, P],
        "hm_silu_mul_fp8": [P, I64, I64, P, P, P],
        "hm_moe_combine": [P, P, I64, I32, I64, P, P],
        "hm_read_probe": [P, I64, I32, I32, P, P],
        "hm_moe_gemm_static": [D, P, I32, P, P, I32, I64, I32, P, P, P, T, P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.hm_moe_gemm_static_max_workspace.argtypes = []
    L.hm_moe_gemm_static_max_workspace.restype = ctypes.c_size_t
    L.hm_status_string.argtypes = [ctypes.c_int]
    L.hm_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ok(fn, code):
    if code != 0:
        raise HmError(fn, code)


def _need(t, dtype, numel, name):
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype or t.numel() < numel:
        raise ValueError(f"{name}: need a contiguous CUDA {dtype} tensor with >= {numel} elements")


# --------------------------------------------------------------------- weights

def hm_transform_size(desc):
    out = ctypes.c_size_t()
    _ok("hm_transform_size", lib.hm_transform_size(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def hm_transform(desc, codes, scales, zeros=None, w_dev=None, stream=None, gated=False):
    """codes uint8 [E,N,K/2]; scales int16/uint16 bits [E,N,K/128] (INT4) or uint8
    [E,N,K/32] (MXFP4); zeros uint8 [E,N,K/128] (UINT4_ZP).  Returns w_dev (uint8).
    gated: a gate_up weight (gate rows, then up rows) into the gated layout
    of hm_moe_gemm_gated (hm_transform_gated)."""
    nbytes = hm_transform_size(desc)
    if w_dev is None:
        w_dev = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    E, n, k = desc.num_experts, desc.n, desc.k
    _need(codes, torch.uint8, E * n * k * CODE_BITS.get(desc.wfmt, 4) // 8, "codes")
    _need(w_dev, torch.uint8, nbytes, "w_dev")
    fn = "hm_transform_gated" if gated else "hm_transform"
    _ok(fn, getattr(lib, fn)(ctypes.byref(desc), _ptr(codes), _ptr(scales), _ptr(zeros),
                             _ptr(w_dev), w_dev.numel(), _stream(stream)))
    return w_dev


def hm_dequant(desc, w_dev, expert=0, out=None, stream=None):
    if out is None:
        out = torch.empty(desc.n, desc.k, dtype=torch.float32, device=w_dev.device)
    _need(out, torch.float32, desc.n * desc.k, "out")
    _ok("hm_dequant", lib.hm_dequant(ctypes.byref(desc), _ptr(w_dev), w_dev.numel(), int(expert),
                                     _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------------------------ activations

def hm_quant_fp8_rows(x, x8=None, row_scale=None, stream=None):
    """x bf16 [m,k] -> (E4M3 bytes uint8 [m,k], fp32 row scales [m])."""
    m, k = x.shape
    _need(x, torch.bfloat16, m * k, "x")
    if x8 is None:
        x8 = torch.empty(m, k, dtype=torch.uint8, device=x.device)
    if row_scale is None:
        row_scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _ok("hm_quant_fp8_rows", lib.hm_quant_fp8_rows(_ptr(x), m, k, _ptr(x8), _ptr(row_scale),
                                                   _stream(stream)))
    return x8, row_scale


def hm_quant_mxfp4_rows(x, codes=None, scales=None, stream=None):
    """x bf16 [m,k] -> (E2M1 codes uint8 [m,k/2], E8M0 scales uint8 [m,k/32])."""
    m, k = x.shape
    _need(x, torch.bfloat16, m * k, "x")
    if codes is None:
        codes = torch.empty(m, k // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(m, k // 32, dtype=torch.uint8, device=x.device)
    _ok("hm_quant_mxfp4_rows", lib.hm_quant_mxfp4_rows(_ptr(x), m, k, _ptr(codes), _ptr(scales),
                                                       _stream(stream)))
    return codes, scales


# -------------------------------------------------------------------- dense GEMM

def _afmt(x, x_scales=None):
    """Activation format from the tensors: bf16 rows, E4M3 bytes with fp32
    row scales, or E2M1 codes with E8M0 scale bytes (uint8 x_scales)."""
    if x.dtype != torch.uint8:
        return HM_A_BF16
    return HM_A_MXFP4 if x_scales is not None and x_scales.dtype == torch.uint8 else HM_A_FP8_ROWSCALE


def hm_gemm_workspace_size(desc, afmt, m, tuning=None):
    out = ctypes.c_size_t()
    _ok("hm_gemm_workspace_size", lib.hm_gemm_workspace_size(ctypes.byref(desc), int(afmt), int(m),
                                                             _tune(tuning), ctypes.byref(out)))
    return out.value


def hm_gemm_plan(desc, afmt, m, tuning=None):
    buf = ctypes.create_string_buffer(256)
    _ok("hm_gemm_plan", lib.hm_gemm_plan(ctypes.byref(desc), int(afmt), int(m), _tune(tuning), buf, 256))
    return buf.value.decode()


def hm_gemm(desc, w_dev, x, x_scales=None, y=None, ws=None, afmt=None, tuning=None, stream=None):
    """y[m,n] = x_hat . w_hat^T in bf16.  x: bf16 [m,k] (W4A16, any weight
    format) or uint8 E4M3 [m,k] with fp32 x_scales [m] (W4A8-MXFP4).
    tuning: None (default choice), an hm_tuning, or a dict of its fields."""
    afmt = _afmt(x, x_scales) if afmt is None else afmt
    m = x.shape[0]
    if y is None:
        y = torch.empty(m, desc.n, dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, m * desc.n, "y")
    if isinstance(tuning, dict):
        tuning = make_tuning(**tuning)
    if ws is None:
        # a caller-provided workspace is passed through as is (the library checks its size)
        need = hm_gemm_workspace_size(desc, afmt, m, tuning)
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    _ok("hm_gemm", lib.hm_gemm(ctypes.byref(desc), _ptr(w_dev), int(afmt), _ptr(x), _ptr(x_scales),
                               m, _ptr(y), _ptr(ws), ws.numel() if ws is not None else 0,
                               _tune(tuning), _stream(stream)))
    return y


# -------------------------------------------------------------------------- MoE

def hm_moe_sort_workspace_size(t, topk, num_experts):
    out = ctypes.c_size_t()
    _ok("hm_moe_sort_workspace_size", lib.hm_moe_sort_workspace_size(int(t), int(topk),
                                                                     int(num_experts), ctypes.byref(out)))
    return out.value


def hm_moe_sort(topk_ids, num_experts, counts=None, offsets=None, sorted_pairs=None, ws=None, stream=None):
    """topk_ids int32 [t, topk] -> (counts [E], offsets [E+1], sorted_pairs [t*topk]).
    ws: a uint8 buffer of hm_moe_sort_workspace_size bytes (allocated here
    when None and needed)."""
    t, topk = topk_ids.shape
    dev = topk_ids.device
    _need(topk_ids, torch.int32, t * topk, "topk_ids")
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    sorted_pairs = (torch.empty(t * topk, dtype=torch.int32, device=dev)
                    if sorted_pairs is None else sorted_pairs)
    need = hm_moe_sort_workspace_size(t, topk, num_experts)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    wsp, wsb = (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())
    _ok("hm_moe_sort", lib.hm_moe_sort(_ptr(topk_ids), t, topk, int(num_experts), _ptr(counts),
                                       _ptr(offsets), _ptr(sorted_pairs), wsp, wsb, _stream(stream)))
    return counts, offsets, sorted_pairs


def hm_moe_gemm_workspace_size(desc, afmt, t, topk, tuning=None):
    out = ctypes.c_size_t()
    _ok("hm_moe_gemm_workspace_size", lib.hm_moe_gemm_workspace_size(ctypes.byref(desc), int(afmt), int(t),
                                                                     int(topk), _tune(tuning), ctypes.byref(out)))
    return out.value


def hm_moe_gemm_plan(desc, afmt, t, topk, a_rows_are_pairs, tuning=None, gated=False):
    buf = ctypes.create_string_buffer(512)
    fn = "hm_moe_gemm_gated_plan" if gated else "hm_moe_gemm_plan"
    _ok(fn, getattr(lib, fn)(ctypes.byref(desc), int(afmt), int(t), int(topk),
                             int(a_rows_are_pairs), _tune(tuning), buf, 512))
    return buf.value.decode()


def hm_moe_gemm(desc, w_dev, a, offsets, sorted_pairs, t, topk, a_rows_are_pairs, a_scales=None,
                y=None, ws=None, afmt=None, tuning=None, stream=None, gated=False):
    """Grouped GEMM; returns y bf16 [t*topk, n] in pair order.  a: bf16 rows,
    or E4M3 bytes with fp32 a_scales (MXFP4 weights only).  tuning: None, an
    hm_tuning, or a dict of its fields.  gated: hm_moe_gemm_gated on weights
    from hm_transform(..., gated=True); returns h bf16 [t*topk, n/2]."""
    afmt = _afmt(a, a_scales) if afmt is None else afmt
    P = t * topk
    ncols = desc.n // 2 if gated else desc.n
    if y is None:
        y = torch.empty(P, ncols, dtype=torch.bfloat16, device=a.device)
    _need(y, torch.bfloat16, P * ncols, "y")
    if isinstance(tuning, dict):
        tuning = make_tuning(**tuning)
    if ws is None:
        need = hm_moe_gemm_workspace_size(desc, afmt, t, topk, tuning)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=a.device)
    fn = "hm_moe_gemm_gated" if gated else "hm_moe_gemm"
    _ok(fn, getattr(lib, fn)(ctypes.byref(desc), _ptr(w_dev), int(afmt), _ptr(a),
                             _ptr(a_scales), int(a_rows_are_pairs), int(t), int(topk),
                             _ptr(offsets), _ptr(sorted_pairs), _ptr(y), _ptr(ws),
                             ws.numel(), _tune(tuning), _stream(stream)))
    return y


def hm_moe_gemm_static(desc, w_dev, a, offsets, sorted_pairs, t, topk, a_rows_are_pairs, a_scales=None,
                       y=None, afmt=None, tuning=None, stream=None):
    """hm_moe_gemm with the library's static work-list array instead of a
    workspace (no device allocation in the call; calls on one GPU must not
    overlap).  y may be passed in so that nothing is allocated here either."""
    afmt = _afmt(a, a_scales) if afmt is None else afmt
    P = t * topk
    if y is None:
        y = torch.empty(P, desc.n, dtype=torch.bfloat16, device=a.device)
    _need(y, torch.bfloat16, P * desc.n, "y")
    _ok("hm_moe_gemm_static", lib.hm_moe_gemm_static(ctypes.byref(desc), _ptr(w_dev), int(afmt), _ptr(a),
                                                     _ptr(a_scales), int(a_rows_are_pairs), int(t), int(topk),
                                                     _ptr(offsets), _ptr(sorted_pairs), _ptr(y), _tune(tuning),
                                                     _stream(stream)))
    return y


def hm_moe_gemm_static_max_workspace():
    return lib.hm_moe_gemm_static_max_workspace()


# --------------------------------------------------------------- MoE block steps

def hm_silu_mul(gu, h=None, stream=None):
    """gu bf16 [rows, 2d] (gate | up) -> h bf16 [rows, d] = silu(gate) * up."""
    rows, two_d = gu.shape
    if two_d % 2:
        raise ValueError("gu: the last dimension must be even (gate | up)")
    d = two_d // 2
    _need(gu, torch.bfloat16, rows * two_d, "gu")
    if h is None:
        h = torch.empty(rows, d, dtype=torch.bfloat16, device=gu.device)
    _need(h, torch.bfloat16, rows * d, "h")
    _ok("hm_silu_mul", lib.hm_silu_mul(_ptr(gu), rows, d, _ptr(h), _stream(stream)))
    return h


def hm_silu_mul_fp8(gu, h8=None, h_scales=None, stream=None):
    """gu bf16 [rows, 2d] -> (E4M3 bytes [rows, d], fp32 row scales [rows]) of
    silu(gate) * up, in one pass."""
    rows, two_d = gu.shape
    d = two_d // 2
    _need(gu, torch.bfloat16, rows * two_d, "gu")
    if h8 is None:
        h8 = torch.empty(rows, d, dtype=torch.uint8, device=gu.device)
    if h_scales is None:
        h_scales = torch.empty(rows, dtype=torch.float32, device=gu.device)
    _ok("hm_silu_mul_fp8", lib.hm_silu_mul_fp8(_ptr(gu), rows, d, _ptr(h8), _ptr(h_scales), _stream(stream)))
    return h8, h_scales


def hm_moe_combine(y, weights, topk, out=None, stream=None):
    """y bf16 [t*topk, n] (pair order), weights fp32 [t, topk] -> out bf16 [t, n]."""
    t = weights.shape[0]
    n = y.shape[1]
    _need(y, torch.bfloat16, t * topk * n, "y")
    _need(weights, torch.float32, t * topk, "weights")
    if out is None:
        out = torch.empty(t, n, dtype=torch.bfloat16, device=y.device)
    _need(out, torch.bfloat16, t * n, "out")
    _ok("hm_moe_combine", lib.hm_moe_combine(_ptr(y), _ptr(weights), t, int(topk), n, _ptr(out),
                                             _stream(stream)))
    return out


# ----------------------------------------------------------------- measurement

def hm_read_probe(buf, blocks=2048, unroll=4, out=None, stream=None):
    """Plain-read reference over a device buffer (any dtype, byte size a
    multiple of 16); returns the per-block words."""
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(blocks, dtype=torch.int32, device=buf.device)
    _ok("hm_read_probe", lib.hm_read_probe(_ptr(buf), nbytes, int(blocks), int(unroll), _ptr(out),
                                           _stream(stream)))
    return out
