"""MoE expert sort and grouped GEMM reference (oracle side).

Tokens are split by expert, so each expert's GEMM has its own M that depends on
the routing load (ywsung.com note "How vLLM Humming computes 4 bits", section on
one token vs many tokens; aihaber.org article, "what problem does it solve"),
and a grouped path runs all experts' GEMMs (aihaber.org, Performance).

Pairs: with T tokens and top-k routing, pair p = t*topk + j is token t's j-th
expert choice ids[t, j].  Rows of the grouped GEMM are in pair order.

Around the two grouped GEMMs of an MoE feed-forward block (tokens split per
expert, each token activating only some experts: aihaber.org article, "what
problem does it solve"; ywsung.com note, section on one token vs many
tokens) sit a gated activation between gate_up and down and the weighted
combine of each token's expert outputs.  The pages name neither formula; the
readings here are the plainest ones:
  h[p, i]   = silu(gu[p, i]) * gu[p, d + i],  silu(x) = x / (1 + exp(-x))
              (gate in columns 0..d-1 of the gate_up output, up in d..2d-1);
  out[t, n] = sum_j w[t, j] * y[t*topk + j, n]   (w: the routing weights).
"""
import numpy as np

from .gemm import gemm_ref


def moe_sort_ref(ids, num_experts):
    """counts[e] = number of pairs routed to e; offsets = [0, cumsum(counts)];
    sorted_pairs = pair ids grouped by expert, ascending within each expert."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    return counts, offsets, sorted_pairs


def moe_gemm_ref(a_hat, a_rows_are_pairs, topk, ids, w_hat_of, n, bound=True,
                 bound_dtype=np.float64, pairs=None):
    """Y_ref[p] = A_row(p) . W_hat_{ids[p]}^T for every pair p (or only for the
    pairs listed in `pairs`).

    a_hat: float64 [T,K] (gate_up: row of pair p is t = p // topk) or [P,K]
           (down: row of pair p is p).
    w_hat_of(e) -> float64 [N,K] exact dequantized weights of expert e.
    Returns (Y_ref [len(pairs), N], B or None, pairs)."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    P = flat.size
    if pairs is None:
        pairs = np.arange(P)
    pairs = np.asarray(pairs, dtype=np.int64)
    y = np.zeros((pairs.size, n), dtype=np.float64)
    b = np.zeros((pairs.size, n), dtype=np.float64) if bound else None
    experts = flat[pairs]
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        p = pairs[sel]
        rows = p if a_rows_are_pairs else p // topk
        ye, be = gemm_ref(a_hat[rows], w_hat_of(int(e)), bound=bound, bound_dtype=bound_dtype)
        y[sel] = ye
        if bound:
            b[sel] = be
    return y, b, pairs


def silu_mul_ref(gu_hat, d):
    """h = silu(gate) * up in float64 from the [rows, 2d] gate_up output
    (gate = columns 0..d-1, up = columns d..2d-1)."""
    x = np.asarray(gu_hat, dtype=np.float64)
    g, u = x[:, :d], x[:, d:2 * d]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))          # exp overflow -> sigmoid 0
    return g * sig * u


# |d silu(x) / dx| = |s (1 + x (1 - s))| with s the logistic function: at
# most 1.0998 (near x = 2.40), so 1.1 bounds it everywhere
SILU_SLOPE = 1.1


def silu_mul_bound(g, u, eg, eu):
    """Bound on |silu(g') u' - silu(g) u| over |g' - g| <= eg, |u' - u| <= eu
    (the gated product of a gate_up output known to within eg, eu element by
    element): |silu(g') - silu(g)| <= 1.1 eg and |silu(g')| <= |silu(g)| + 1.1 eg,
    so the difference is at most 1.1 eg (|u| + eu) + |silu(g)| eu."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        sg = g / (1.0 + np.exp(-g))
    return SILU_SLOPE * eg * (np.abs(u) + eu) + np.abs(sg) * eu


def combine_ref(y_hat, weights, topk):
    """out[t] = sum_j w[t, j] * y[t*topk + j] in float64 over pair-order rows
    y_hat [T*topk, N], and the bound sum_j |w[t, j] * y[t*topk + j]|."""
    w = np.asarray(weights, dtype=np.float64)
    t = w.shape[0]
    y = np.asarray(y_hat, dtype=np.float64).reshape(t, topk, -1)
    out = np.einsum("tj,tjn->tn", w, y)
    bnd = np.einsum("tj,tjn->tn", np.abs(w), np.abs(y))
    return out, bnd
