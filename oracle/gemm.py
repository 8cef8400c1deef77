"""Dense GEMM reference and the acceptance check (oracle side).

A linear layer is Y[M,N] = X[M,K] . W[N,K]^T (ywsung.com note "How vLLM Humming
computes 4 bits", section on one token vs many tokens); the contraction costs
about 2*M*N*K flops there.  Here X_hat is the activation the kernel actually
multiplies (bf16 values, or the dequantized per-token FP8 values) and W_hat is
the exact dequantized weight, so the reference is the plain definition:

    Y_ref = X_hat @ W_hat^T          in float64
    B     = |X_hat| @ |W_hat|^T      (the sum_k |x_k w_k| bound)

Acceptance of a bf16 result Y (both must hold):
    ||Y - Y_ref||_F / ||Y_ref||_F <= 5e-3
    |Y - Y_ref| <= 4e-3 * B + ulp_bf16(Y_ref)      element by element
"""
import numpy as np

from . import codecs

NORM_TOL = 5e-3
ELEM_TOL = 4e-3


def gemm_ref(xhat, what, bound=True, bound_dtype=np.float64):
    """Y_ref = xhat @ what^T in fp64, and optionally B = |xhat| @ |what|^T."""
    x = np.asarray(xhat, dtype=np.float64)
    w = np.asarray(what, dtype=np.float64)
    y = x @ w.T
    if not bound:
        return y, None
    b = np.abs(x).astype(bound_dtype) @ np.abs(w).astype(bound_dtype).T
    return y, b.astype(np.float64)


def flops(m, n, k):
    return 2.0 * m * n * k


def check(y_bf16_bits, y_ref, b, norm_tol=NORM_TOL, elem_tol=ELEM_TOL):
    """Apply the acceptance rule to a bf16 result given as uint16 bits.
    Returns a dict with 'ok', the normwise error and the worst element ratio."""
    y = codecs.bf16_value(np.asarray(y_bf16_bits, dtype=np.uint16)).astype(np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = np.abs(y - y_ref)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    if den > 0:
        norm_err = num / den
    else:
        norm_err = 0.0 if num == 0 else np.inf
    lim = elem_tol * b + codecs.ulp_bf16(y_ref)
    ratio = d / lim
    finite = bool(np.all(np.isfinite(y)))
    worst = float(ratio.max()) if ratio.size else 0.0
    ok = finite and norm_err <= norm_tol and worst <= 1.0
    bad = int((ratio > 1.0).sum())
    return dict(ok=ok, norm_err=float(norm_err), worst_ratio=worst, n_bad=bad,
                finite=finite)


def check_elementwise(y_bf16_bits, y_ref, extra=0.0):
    """Element-wise acceptance of a bf16 result of an elementwise step (SiLU
    product, weighted combine): |Y - Y_ref| <= ulp_bf16(Y_ref) + extra, where
    extra covers the fp32 accumulation of a sum (0 for a single product)."""
    y = codecs.bf16_value(np.asarray(y_bf16_bits, dtype=np.uint16)).astype(np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    lim = codecs.ulp_bf16(y_ref) + np.asarray(extra, dtype=np.float64)
    ratio = np.abs(y - y_ref) / lim
    finite = bool(np.all(np.isfinite(y)))
    worst = float(ratio.max()) if ratio.size else 0.0
    return dict(ok=finite and worst <= 1.0, worst_ratio=worst, n_bad=int((ratio > 1.0).sum()),
                finite=finite)
