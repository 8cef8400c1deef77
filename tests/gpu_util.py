"""Helpers shared by the GPU parity tests: numpy <-> device tensors and the
oracle-side preparation of standard-format weights."""
import numpy as np
import torch

from oracle import codecs, quant


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_to_dev(bits):
    """uint16 bf16 patterns -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def bits_of(y):
    """device bfloat16 tensor -> uint16 numpy patterns."""
    return y.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def std_to_dev(fmt, codes, scales, zeros):
    """Standard-format numpy arrays ([E,...]) -> device tensors for hm_transform."""
    c = to_dev(codes.astype(np.uint8))
    if fmt in quant.MX_FORMATS:
        s = to_dev(scales.astype(np.uint8))
    else:
        s = to_dev(scales.astype(np.uint16).view(np.int16))
    z = to_dev(zeros.astype(np.uint8)) if zeros is not None else None
    return c, s, z


def quantize_experts(fmt, ws):
    """Oracle-quantize a list of fp32 [N,K] weights; returns stacked standard
    format (codes [E,N,K/2], scales, zeros or None) and exact fp32 dequant [E,N,K]."""
    sts = [quant.quantize(fmt, w) for w in ws]
    codes = np.stack([s["codes"] for s in sts])
    scales = np.stack([s["scales"] for s in sts])
    zeros = np.stack([s["zeros"] for s in sts]) if sts[0]["zeros"] is not None else None
    what = np.stack([quant.dequant(fmt, s["codes"], s["scales"], s["zeros"]) for s in sts])
    return codes, scales, zeros, what


def xhat_of(fmt, x_bits):
    """The activation values the kernel multiplies: bf16 values (W4A16) or the
    dequantized per-token FP8 values (W4A8), float64."""
    if fmt == quant.FMT_MXFP4:
        c, s = quant.quant_fp8_rows(x_bits)
        return quant.fp8_rows_dequant(c, s)
    return codecs.bf16_value(x_bits).astype(np.float64)

