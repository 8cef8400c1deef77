"""Tile-configuration autotuner for hm_gemm and hm_moe_gemm on one GPU.

The library's default choices come from fixed heuristics; the pages say
such device-specific heuristic defaults are not globally optimal and that
auto-tuning was unfinished (cocoloop.cn news item, stated weaknesses), and
name the tuning knobs: tile shapes, pipeline stages, wave roles, matrix
instructions (aihaber.org article, Architecture).  This module searches the
explicit choices of hm_tuning for given call shapes:

  * candidates: every valid combination of the kernel path and the streaming
    launch shape (waves splitting K, column blocks per wave, K split over
    blocks) for a dense call; of the grouped unit sizes and kernels for a
    grouped call.  A candidate the library rejects (HM_ERR_TUNING) is
    skipped, so the search never runs an unsupported configuration.
  * timing: a HIP graph of `reps` back-to-back calls on the current stream,
    rotating over weight copies that together exceed the last-level cache,
    replayed once to warm up and once under HIP events; the per-call time is
    the event time / reps.  The default choice is timed once before the
    search and discarded (the first timed graph of a process runs slow), and
    the fastest candidate is re-timed against the default, alternating, at
    the end: it replaces the default only if it is faster there too.
  * check: each candidate's output is compared with the default choice's
    (normwise relative difference at most 1e-2 and finite), which catches a
    misconfigured launch; the parity tests cover every path against the
    oracle.
  * result: a Table of the fastest tuning per (format pair, N, K, experts,
    rows), saved as JSON and looked up per call (nearest tuned row count of
    the same layer, rounding up).

Everything runs through the C entry points; nothing here computes the GEMM.
"""
import itertools
import json
import math

import torch

from . import (HM_A_BF16, HM_A_FP8_ROWSCALE, HM_W_INT8_SYM, HmError, hm_gemm, hm_gemm_plan,
               hm_gemm_workspace_size, hm_moe_gemm, hm_moe_gemm_plan, hm_moe_gemm_workspace_size)

LLC_BYTES = 256 * 2 ** 20


def _key(desc, afmt):
    return f"w{int(desc.wfmt)}a{int(afmt)}_n{int(desc.n)}_k{int(desc.k)}_e{int(desc.num_experts)}"


def dense_candidates(desc, afmt, m):
    """Valid explicit tunings of hm_gemm for m rows (the default first)."""
    out = [dict()]
    seen = {hm_gemm_plan(desc, afmt, m)}
    kg = int(desc.k) // 128
    paths = [2, 3, 4] + ([1] if m <= 256 else [])
    for path in paths:
        if path == 1:
            combos = [dict(path=1, stream_ks=ks, stream_nbw=nbw, stream_splits=sp)
                      for ks, nbw, sp in itertools.product((1, 2, 4), (1, 2), (1, 2, 4, 8)) if sp <= kg]
            combos += [dict(path=1, stream_waves=8, stream_ks=ks, stream_nbw=nbw, stream_splits=sp)
                       for ks, nbw, sp in itertools.product((2, 4, 8), (1, 2), (1, 2, 4)) if sp <= kg]
        else:
            combos = [dict(path=path)]
        for c in combos:
            try:
                plan = hm_gemm_plan(desc, afmt, m, c)
            except HmError:
                continue
            if plan in seen:
                continue
            seen.add(plan)
            out.append(c)
    return out


def moe_candidates(desc, afmt, t, topk, rows_are_pairs):
    """Valid explicit tunings of hm_moe_gemm (the default first)."""
    out = [dict()]
    seen = {hm_moe_gemm_plan(desc, afmt, t, topk, rows_are_pairs)}
    no_big = int(desc.wfmt) == HM_W_INT8_SYM                         # no 256-row units
    for rows, smax, nbw, big, tile in itertools.product((16, 32), (16, 32, 64, 128), (1, 2),
                                                        (0, -1, 65, 129), (1, 2)):
        if smax < rows or (no_big and big > 0):
            continue
        c = dict(moe_stream_rows=rows, moe_stream_max=smax, moe_stream_nbw=nbw, moe_big_min=big, moe_tile=tile)
        try:
            plan = hm_moe_gemm_plan(desc, afmt, t, topk, rows_are_pairs, c)
        except HmError:
            continue
        if plan in seen:
            continue
        seen.add(plan)
        out.append(c)
    return out


def _graph_us(fn, reps):
    """Per-call microseconds of `fn(i)` over a graph of reps calls."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    b.synchronize()
    del g
    return a.elapsed_time(b) * 1e3 / reps


def _confirm(fn_default, fn_best, reps, rounds=2):
    """Alternating re-timing of the default and the best candidate; returns
    (default us, best us) as the minimum over the rounds."""
    d, b = [], []
    for _ in range(rounds):
        d.append(_graph_us(fn_default, reps))
        b.append(_graph_us(fn_best, reps))
    return min(d), min(b)


def _close(y, y0):
    d = (y.float() - y0.float()).norm().item()
    n = y0.float().norm().item()
    return math.isfinite(d) and d <= 1e-2 * max(n, 1e-30)


class Table:
    """Fastest tuning per layer shape and row count."""

    def __init__(self, entries=None, meta=None):
        self.entries = dict(entries or {})
        self.meta = dict(meta or {})

    def put(self, key, rows, tuning, us, default_us, plan):
        self.entries.setdefault(key, {})[str(int(rows))] = dict(tuning=tuning, us=round(us, 3),
                                                                default_us=round(default_us, 3), plan=plan)

    def lookup(self, desc, afmt, rows):
        """The tuning of the smallest tuned row count >= rows (else the largest)
        for this layer, or None (the library's default choice)."""
        e = self.entries.get(_key(desc, afmt))
        if not e:
            return None
        tuned = sorted(int(r) for r in e)
        pick = next((r for r in tuned if r >= rows), tuned[-1])
        t = e[str(pick)]["tuning"]
        return dict(t) if t else None

    def save(self, path):
        with open(path, "w") as f:
            json.dump(dict(meta=self.meta, entries=self.entries), f, indent=1, sort_keys=True)

    @classmethod
    def load(cls, path):
        with open(path) as f:
            d = json.load(f)
        return cls(d.get("entries"), d.get("meta"))


def tune_dense(desc, w_copies, x, ms, x_scales=None, reps=30, table=None, log=None):
    """Search hm_gemm tunings for each row count in ms.
    w_copies: list of transformed weight buffers of one layer (rotated so the
    weights come from HBM); x: activations [max(ms), k] (bf16, or E4M3 bytes
    with fp32 x_scales).  Returns the Table (new, or the one given)."""
    table = table or Table()
    afmt = HM_A_FP8_ROWSCALE if x.dtype == torch.uint8 else HM_A_BF16
    dev = x.device
    for m in ms:
        xm = x[:m]
        xs = x_scales[:m] if x_scales is not None else None
        y0 = torch.empty(m, desc.n, dtype=torch.bfloat16, device=dev)
        y = torch.empty_like(y0)
        best = None
        default_us = None
        warm_ws = torch.empty(max(hm_gemm_workspace_size(desc, afmt, m, None), 256), dtype=torch.uint8, device=dev)
        _graph_us(lambda i: hm_gemm(desc, w_copies[i % len(w_copies)], xm, xs, y=y0, ws=warm_ws), reps)
        for c in dense_candidates(desc, afmt, m):
            need = hm_gemm_workspace_size(desc, afmt, m, c or None)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
            out = y0 if not c else y
            hm_gemm(desc, w_copies[0], xm, xs, y=out, ws=ws, tuning=c or None)
            torch.cuda.synchronize()
            if c and not _close(y, y0):
                if log:
                    log(f"m={m} {c}: output differs from the default choice, skipped")
                continue
            us = _graph_us(lambda i: hm_gemm(desc, w_copies[i % len(w_copies)], xm, xs, y=out, ws=ws,
                                             tuning=c or None), reps)
            if not c:
                default_us = us
            if log:
                log(f"m={m} {hm_gemm_plan(desc, afmt, m, c or None)}: {us:.2f} us")
            if best is None or us < best[1]:
                best = (c, us)
        if best[0]:
            bws = torch.empty(max(hm_gemm_workspace_size(desc, afmt, m, best[0]), 256), dtype=torch.uint8, device=dev)
            d_us, b_us = _confirm(
                lambda i: hm_gemm(desc, w_copies[i % len(w_copies)], xm, xs, y=y0, ws=warm_ws),
                lambda i: hm_gemm(desc, w_copies[i % len(w_copies)], xm, xs, y=y, ws=bws, tuning=best[0]), reps)
            default_us = d_us
            best = (best[0], b_us) if b_us < d_us else ({}, d_us)
            if log:
                log(f"m={m} confirm: default {d_us:.2f} us, best {b_us:.2f} us")
        table.put(_key(desc, afmt), m, best[0], best[1], default_us, hm_gemm_plan(desc, afmt, m, best[0] or None))
    return table


def tune_moe(desc, w, a, offsets, sorted_pairs, t, topk, rows_are_pairs, a_scales=None, reps=5,
             table=None, log=None):
    """Search hm_moe_gemm tunings for one routed call (t tokens, top-k)."""
    table = table or Table()
    afmt = HM_A_FP8_ROWSCALE if a.dtype == torch.uint8 else HM_A_BF16
    dev = a.device
    P = t * topk
    y0 = torch.empty(P, desc.n, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(y0)
    best, default_us = None, None
    warm_ws = torch.empty(max(hm_moe_gemm_workspace_size(desc, afmt, t, topk, None), 256), dtype=torch.uint8,
                          device=dev)
    _graph_us(lambda i: hm_moe_gemm(desc, w, a, offsets, sorted_pairs, t, topk, rows_are_pairs, a_scales, y=y0,
                                    ws=warm_ws), reps)
    for c in moe_candidates(desc, afmt, t, topk, rows_are_pairs):
        need = hm_moe_gemm_workspace_size(desc, afmt, t, topk, c or None)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        out = y0 if not c else y
        hm_moe_gemm(desc, w, a, offsets, sorted_pairs, t, topk, rows_are_pairs, a_scales, y=out, ws=ws,
                    tuning=c or None)
        torch.cuda.synchronize()
        if c and not _close(y, y0):
            if log:
                log(f"t={t} {c}: output differs from the default choice, skipped")
            continue
        us = _graph_us(lambda i: hm_moe_gemm(desc, w, a, offsets, sorted_pairs, t, topk, rows_are_pairs,
                                             a_scales, y=out, ws=ws, tuning=c or None), reps)
        if not c:
            default_us = us
        if log:
            log(f"t={t} {c}: {us:.1f} us")
        if best is None or us < best[1]:
            best = (c, us)
    if best[0]:
        bws = torch.empty(max(hm_moe_gemm_workspace_size(desc, afmt, t, topk, best[0]), 256), dtype=torch.uint8,
                          device=dev)
        d_us, b_us = _confirm(
            lambda i: hm_moe_gemm(desc, w, a, offsets, sorted_pairs, t, topk, rows_are_pairs, a_scales, y=y0,
                                  ws=warm_ws),
            lambda i: hm_moe_gemm(desc, w, a, offsets, sorted_pairs, t, topk, rows_are_pairs, a_scales, y=y,
                                  ws=bws, tuning=best[0]), reps)
        default_us = d_us
        best = (best[0], b_us) if b_us < d_us else ({}, d_us)
        if log:
            log(f"t={t} confirm: default {d_us:.1f} us, best {b_us:.1f} us")
    key = _key(desc, afmt) + f"_moe_topk{topk}_rp{rows_are_pairs}"
    table.put(key, t, best[0], best[1], default_us,
              hm_moe_gemm_plan(desc, afmt, t, topk, rows_are_pairs, best[0] or None))
    return table
