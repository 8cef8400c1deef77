"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This module holds no arithmetic of the quantized-GEMM method: it only draws
random numbers with the shapes and distributions of the workloads (weights
~ N(0, 0.02), activations ~ N(0, 1) rounded to bf16, optional sparse outliers,
a Zipf-skewed top-k router) and random standard-format codes for runs whose
values do not matter (throughput).  The quantizers live in the oracle.

Seeds are lists [config, role, index, repeat] fed to numpy's default_rng, so
every array can be regenerated independently and reproducibly.
Roles: 0 = weights, 1 = activations, 2 = router, 3 = outlier mask,
4 = down-projection input, 5 = random codes.
"""
import numpy as np

ROLE_W, ROLE_X, ROLE_ROUTER, ROLE_OUTLIER, ROLE_DOWN, ROLE_CODES = range(6)


def rng(cfg, role, index=0, rep=0):
    return np.random.default_rng([int(cfg), int(role), int(index), int(rep)])


def weights(cfg, n, k, index=0, rep=0, std=0.02):
    """fp32 [n, k] ~ N(0, std)."""
    return rng(cfg, ROLE_W, index, rep).normal(0.0, std, size=(n, k)).astype(np.float32)


def to_bf16_bits(x32):
    """fp32 -> bf16 bit patterns using torch's own conversion (round to
    nearest even), returned as uint16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def activations(cfg, m, k, index=0, rep=0, outliers=0.0, outlier_scale=20.0, role=ROLE_X):
    """bf16 bits [m, k]: N(0,1), optionally with an element-wise Bernoulli
    outlier mask (probability `outliers`) multiplying by `outlier_scale`
    before the rounding to bf16."""
    x = rng(cfg, role, index, rep).normal(0.0, 1.0, size=(m, k)).astype(np.float32)
    if outliers > 0:
        mask = rng(cfg, ROLE_OUTLIER, index, rep).random(size=(m, k)) < outliers
        x = np.where(mask, x * np.float32(outlier_scale), x).astype(np.float32)
    return to_bf16_bits(x)


def router_topk(cfg, t, num_experts=256, topk=8, rep=0, zipf=1.1):
    """Top-k expert ids [t, topk] (int32) from Gaussian logits plus a
    Zipf(zipf) log-popularity: p_e ~ (rank_e + 1)^-zipf with rank a random
    permutation (popular experts are not the low ids); logits = N(0,1) + ln p_e;
    ids = the topk largest logits in descending order, ties to the lower id.
    Also returns the softmax routing weights over the chosen logits."""
    r = rng(cfg, ROLE_ROUTER, 0, rep)
    rank = r.permutation(num_experts)
    logp = -zipf * np.log(rank + 1.0)
    logp = logp - np.log(np.exp(logp).sum())
    logits = r.normal(0.0, 1.0, size=(t, num_experts)) + logp[None, :]
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    chosen = np.take_along_axis(logits, order, axis=1)
    wts = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    wts = wts / wts.sum(axis=1, keepdims=True)
    return order.astype(np.int32), wts.astype(np.float32)


def random_std_format(fmt, num_experts, n, k, seed=0):
    """Random standard-format arrays (codes, scales, zeros) for throughput runs.
    Codes are uniform nibbles; int4 scales are bf16 patterns drawn from the
    exponent range of N(0,0.02)/7 (about 2^-9..2^-8); E8M0 bytes in 118..121;
    zero points uniform 0..15.  fmt is 'int4_sym', 'uint4_zp' or 'mxfp4'."""
    r = rng(0, ROLE_CODES, seed, 0)
    codes = r.integers(0, 256, size=(num_experts, n, k // 2), dtype=np.uint8)
    if fmt == "mxfp4":
        scales = r.integers(118, 122, size=(num_experts, n, k // 32), dtype=np.uint8)
        zeros = None
    else:
        scales = (0x3B00 + r.integers(0, 0x100, size=(num_experts, n, k // 128))).astype(np.uint16)
        zeros = r.integers(0, 16, size=(num_experts, n, k // 128), dtype=np.uint8) \
            if fmt == "uint4_zp" else None
    return codes, scales, zeros


def activations_dev(seed, m, k, device="cuda", outliers=0.0, outlier_scale=20.0):
    """Device-side draw of bf16 [m, k] activations for large runs: N(0,1) from
    torch's seeded generator on the device, optionally times `outlier_scale`
    where a Bernoulli(`outliers`) mask fires, rounded to bf16 by torch.
    Returns the device tensor; any row can be copied back to the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn((m, k), generator=g, device=device, dtype=torch.float32)
    if outliers > 0:
        mask = torch.rand((m, k), generator=g, device=device) < outliers
        x = torch.where(mask, x * outlier_scale, x)
    return x.to(torch.bfloat16)


def random_std_format_dev(fmt, num_experts, n, k, seed, device="cuda"):
    """Device-side random standard-format weights (codes, scales, zeros) with
    the value ranges of random_std_format; MX formats take E8M0 bytes in
    118..121.  Returns device tensors (scales of the INT4 formats as int16
    bf16 patterns)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    codes = torch.randint(0, 256, (num_experts, n, k // 2), dtype=torch.uint8, device=device, generator=g)
    if fmt in ("mxfp4", "mxint4"):
        scales = torch.randint(118, 122, (num_experts, n, k // 32), dtype=torch.uint8, device=device, generator=g)
        zeros = None
    else:
        scales = (0x3B00 + torch.randint(0, 0x100, (num_experts, n, k // 128), device=device,
                                         generator=g)).to(torch.int16)
        zeros = (torch.randint(0, 16, (num_experts, n, k // 128), dtype=torch.uint8, device=device, generator=g)
                 if fmt == "uint4_zp" else None)
    return codes, scales, zeros
