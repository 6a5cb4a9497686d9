"""CQS partials and their recomposition in float64 (oracle; test infrastructure only).

These follow the method's own steps, in the order the pages give them:
"Stream-CQSA: Breaking the Billion-Token Barrier on a Single GPU" (wispaper
explainer), section "Implementation: From High-Level Logic to GPU Kernels":
divide into subsequences, move each task's Q, K, V, form each task's softmax
numerator and denominator sums, aggregate them.  The abstract of
"Stream-CQSA: Exact Out-of-Memory Recovery for Attention" (arXiv 2604.20819)
says the local statistics are recomposed into the full output; the merge rule
for (max, denominator, numerator) triples is the one of "Online normalizer
calculation for softmax" (cited by title on the same page).

Statistics of one task for one query row (natural-log units):
    m = max_j s_ij,  l = sum_j exp(s_ij - m),  n = sum_j exp(s_ij - m) v_j
over the keys the task admits (readings R4/R5 of ``oracle.plan``; R16 for causal
plans, where a row also drops the keys after it).  A row with
no admitted key has m = -inf, l = 0, n = 0 and is the identity of the merge.

Merge of two triples (a, b):  m = max(m_a, m_b),
    l = l_a exp(m_a - m) + l_b exp(m_b - m),  n = n_a exp(m_a - m) + n_b exp(m_b - m).
Finalize:  O = n / l,  LSE = m + ln l.
"""
from __future__ import annotations

import numpy as np

from .attention import default_scale, to_f64
from .plan import Plan

__all__ = ["task_partials_fp64", "merge_fp64", "finalize_fp64", "recompose_fp64"]


def _key_tokens(plan: Plan, task, a: int) -> np.ndarray:
    """Global token indices of the keys task admits for its local query unit a
    (padding positions >= N excluded, reading R12 of oracle.plan)."""
    u = plan.unit_tokens
    parts = []
    for b0, cnt in task.key_runs(a, plan.causal):
        for b in range(b0, b0 + cnt):
            g = task.units[b]
            parts.append(np.arange(g * u, min((g + 1) * u, plan.n), dtype=np.int64))
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts)


def task_partials_fp64(q, k, v, plan: Plan, task, dtype="f32", scale=None,
                       rows_of_unit=None):
    """Local (m, l, n) of every query row of one task, two passes, float64.

    Returns a dict: global unit p -> (rows [r], m [r, H], l [r, H], n [r, H, d]).
    ``rows_of_unit`` optionally restricts each unit to a subset of its rows
    (global token indices); by default all rows of each unit are computed.
    """
    n_tok, h_count, d = q.shape
    if scale is None:
        scale = default_scale(d)
    u = plan.unit_tokens
    out = {}
    for a, p in enumerate(task.units):
        if rows_of_unit is None:
            rows = np.arange(p * u, min((p + 1) * u, plan.n), dtype=np.int64)
        else:
            rows = np.asarray(rows_of_unit.get(p, []), dtype=np.int64)
        keys = _key_tokens(plan, task, a)
        m = np.full((rows.size, h_count), -np.inf)
        lsum = np.zeros((rows.size, h_count))
        num = np.zeros((rows.size, h_count, d))
        if rows.size and keys.size:
            for h in range(h_count):
                qh = to_f64(q[rows, h, :], dtype)
                kh = to_f64(k[keys, h, :], dtype)
                vh = to_f64(v[keys, h, :], dtype)
                s = (qh @ kh.T) * scale
                if plan.causal:  # the diagonal block: key j is seen by row i only if j <= i
                    s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
                mh = s.max(axis=1)
                pexp = np.exp(s - np.where(np.isfinite(mh), mh, 0.0)[:, None])
                m[:, h] = mh
                lsum[:, h] = pexp.sum(axis=1)
                num[:, h, :] = pexp @ vh
        out[p] = (rows, m, lsum, num)
    return out


def merge_fp64(a, b):
    """Merge two (m, l, n) triples; the empty triple (m=-inf, l=0) is the identity."""
    ma, la, na = a
    mb, lb, nb = b
    m = np.maximum(ma, mb)
    finite = np.isfinite(m)
    safe = np.where(finite, m, 0.0)
    wa = np.where(finite, np.exp(np.where(np.isfinite(ma), ma, -np.inf) - safe), 0.0)
    wb = np.where(finite, np.exp(np.where(np.isfinite(mb), mb, -np.inf) - safe), 0.0)
    l = la * wa + lb * wb
    n = na * wa[..., None] + nb * wb[..., None]
    return m, l, n


def finalize_fp64(m, l, n):
    """O = n / l and LSE = m + ln l."""
    return n / l[..., None], m + np.log(l)


def recompose_fp64(q, k, v, plan: Plan, dtype="f32", scale=None, rows=None):
    """Run every task in ascending id and merge its statistics per row.

    Returns (O [R, H, d], LSE [H, R]) for ``rows`` (default: all N rows), which
    by the pages' claim equals ``attention_fp64`` up to float64 rounding.
    """
    n_tok, h_count, d = q.shape
    if rows is None:
        rows = np.arange(n_tok, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    u = plan.unit_tokens
    by_unit = {}
    for r in rows:
        by_unit.setdefault(int(r) // u, []).append(int(r))
    index = {int(r): i for i, r in enumerate(rows)}
    acc_m = np.full((rows.size, h_count), -np.inf)
    acc_l = np.zeros((rows.size, h_count))
    acc_n = np.zeros((rows.size, h_count, d))
    for task in plan.tasks:
        parts = task_partials_fp64(q, k, v, plan, task, dtype=dtype, scale=scale,
                                   rows_of_unit={p: by_unit.get(p, []) for p in task.units})
        for p, (prow, m, lsum, num) in parts.items():
            if prow.size == 0:
                continue
            idx = np.asarray([index[int(r)] for r in prow])
            acc_m[idx], acc_l[idx], acc_n[idx] = merge_fp64(
                (acc_m[idx], acc_l[idx], acc_n[idx]), (m, lsum, num))
    o, lse = finalize_fp64(acc_m, acc_l, acc_n)
    return o, lse.T.copy()
