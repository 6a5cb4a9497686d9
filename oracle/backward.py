"""Gradients of exact softmax attention, and their CQS decomposition, in float64
(oracle; test infrastructure only).

"Stream-CQSA: Exact Out-of-Memory Recovery for Attention" (arXiv 2604.20819),
abstract: the decomposition is exact for the backward pass as well as the
forward, with gradient error on par with FlashAttention-2.  The pages give no
formulas for it, so the oracle is the definition -- the derivative of

    O[i] = sum_j P_ij V[j],   P_ij = exp(s_ij - LSE_i),   s_ij = scale <Q[i], K[j]>

for an upstream gradient dO, per head:

    dV[j]  = sum_i P_ij dO[i]
    dP_ij  = <dO[i], V[j]>
    Delta_i = sum_j P_ij dP_ij  (= <dO[i], O[i]>)
    dS_ij  = P_ij (dP_ij - Delta_i)
    dQ[i]  = scale sum_j dS_ij K[j]
    dK[j]  = scale sum_i dS_ij Q[i]

(the chain rule through the softmax: d softmax = P (dP - <P, dP>)).

Causal variant (reading R16 of ``oracle.plan``): the same with P_ij = 0 for j > i.

CQS decomposition (reading R15): every (query, key) pair is admitted by exactly
one task (readings R4/R5 of ``oracle.plan``), and with the final LSE each pair's
terms above no longer depend on any other pair, so each gradient is the sum over
tasks of the terms of the pairs the task admits; tasks are summed in ascending
id.  Nothing is rescaled across tasks (the forward's merge is not needed).
"""
from __future__ import annotations

import numpy as np

from .attention import default_scale, to_f64
from .plan import Plan

__all__ = ["attention_backward_fp64", "attention_backward_given_fp64", "task_backward_fp64",
           "recompose_backward_fp64", "dq_rows_fp64"]


def _dense_head(q, k, v, do, scale, causal=False):
    """All of the definition for one head: (dq, dk, dv, lse) in float64, N x N at once."""
    s = (q @ k.T) * scale
    if causal:
        s = np.where(np.triu(np.ones(s.shape, dtype=bool), 1), -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    lse = m[:, 0] + np.log(e.sum(axis=1))
    p = np.exp(s - lse[:, None])
    dv = p.T @ do
    dp = do @ v.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv, lse


def attention_backward_fp64(q, k, v, do, dtype="f32", scale=None, causal=False):
    """(dQ, dK, dV) [N, H, d] float64 of exact attention for upstream gradient dO.

    q, k, v, do: [N, H, d] float32 arrays or bf16 bit patterns (uint16), widened
    exactly.  Dense per head (N x N scores), for the sizes the parity tests check
    element by element.
    """
    n, h_count, d = q.shape
    if scale is None:
        scale = default_scale(d)
    out = [np.zeros((n, h_count, d)) for _ in range(3)]
    for h in range(h_count):
        qh, kh, vh, doh = (to_f64(x[:, h, :], dtype) for x in (q, k, v, do))
        dq, dk, dv, _ = _dense_head(qh, kh, vh, doh, scale, causal)
        out[0][:, h], out[1][:, h], out[2][:, h] = dq, dk, dv
    return tuple(out)


def attention_backward_given_fp64(q, k, v, o, lse, do, dtype="f32", scale=None, causal=False):
    """(dQ, dK, dV) of the backward as an operation on its inputs, in float64.

    A backward pass receives the forward's saved O and LSE (rounded to their storage
    precision) and uses them as given: P_ij = exp(s_ij - LSE_i), Delta_i = <dO_i, O_i>,
    then the formulas above.  With the exact O and LSE this is attention_backward_fp64;
    with rounded ones it is what an exact implementation of the operation returns for
    those inputs.  o: [N, H, d] in dtype (float32 or bf16 bits) or float64; lse: [H, N].
    """
    n, h_count, d = q.shape
    if scale is None:
        scale = default_scale(d)
    o64 = np.asarray(o, dtype=np.float64) if np.asarray(o).dtype == np.float64 else to_f64(o, dtype)
    lse64 = np.asarray(lse, dtype=np.float64)
    out = [np.zeros((n, h_count, d)) for _ in range(3)]
    for h in range(h_count):
        qh, kh, vh, doh = (to_f64(x[:, h, :], dtype) for x in (q, k, v, do))
        s = (qh @ kh.T) * scale
        p = np.exp(s - lse64[h][:, None])
        if causal:
            p = np.where(np.triu(np.ones(p.shape, dtype=bool), 1), 0.0, p)
        delta = (doh * o64[:, h, :]).sum(axis=1)
        ds = p * (doh @ vh.T - delta[:, None])
        out[0][:, h], out[1][:, h], out[2][:, h] = scale * (ds @ kh), scale * (ds.T @ qh), p.T @ doh
    return tuple(out)


def _unit_rows(plan: Plan, p: int) -> np.ndarray:
    u = plan.unit_tokens
    return np.arange(p * u, min((p + 1) * u, plan.n), dtype=np.int64)


def task_backward_fp64(q, k, v, do, lse, delta, plan: Plan, task, dtype="f32", scale=None):
    """Gradient terms of the pairs one task admits.

    lse [H, N] and delta [H, N] are the final (natural-log) LSE and Delta rows.
    Returns three dicts keyed by global unit p: dQ terms of p's rows as queries,
    dK and dV terms of p's rows as keys, each [rows, H, d].
    """
    n, h_count, d = q.shape
    if scale is None:
        scale = default_scale(d)
    dq_t, dk_t, dv_t = {}, {}, {}
    for p in task.units:
        r = _unit_rows(plan, p).size
        for acc in (dq_t, dk_t, dv_t):
            acc[p] = np.zeros((r, h_count, d))
    for a, pa in enumerate(task.units):
        qi = _unit_rows(plan, pa)
        if qi.size == 0:
            continue
        for b, pb in enumerate(task.units):
            if not task.admitted(a, b) or (plan.causal and b > a):
                continue
            kj = _unit_rows(plan, pb)
            if kj.size == 0:
                continue
            for h in range(h_count):
                qh, doh = to_f64(q[qi, h], dtype), to_f64(do[qi, h], dtype)
                kh, vh = to_f64(k[kj, h], dtype), to_f64(v[kj, h], dtype)
                p_ = np.exp((qh @ kh.T) * scale - lse[h, qi][:, None])
                if plan.causal:
                    p_ = np.where(kj[None, :] > qi[:, None], 0.0, p_)
                dp = doh @ vh.T
                ds = p_ * (dp - delta[h, qi][:, None])
                dq_t[pa][:, h] += scale * (ds @ kh)
                dk_t[pb][:, h] += scale * (ds.T @ qh)
                dv_t[pb][:, h] += p_.T @ doh
    return dq_t, dk_t, dv_t


def recompose_backward_fp64(q, k, v, do, plan: Plan, dtype="f32", scale=None):  # noqa: C901
    """Sum every task's gradient terms in ascending task id: (dQ, dK, dV) [N, H, d].

    The final LSE and Delta come from the dense definition (they are inputs of a
    backward pass: the forward's saved statistics).
    """
    n, h_count, d = q.shape
    if scale is None:
        scale = default_scale(d)
    lse = np.zeros((h_count, n))
    delta = np.zeros((h_count, n))
    for h in range(h_count):
        qh, kh, vh, doh = (to_f64(x[:, h, :], dtype) for x in (q, k, v, do))
        s = (qh @ kh.T) * scale
        if plan.causal:
            s = np.where(np.triu(np.ones(s.shape, dtype=bool), 1), -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        lse[h] = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        o = np.exp(s - lse[h][:, None]) @ vh
        delta[h] = (doh * o).sum(axis=1)
    grads = [np.zeros((n, h_count, d)) for _ in range(3)]
    for task in plan.tasks:
        parts = task_backward_fp64(q, k, v, do, lse, delta, plan, task, dtype=dtype, scale=scale)
        for g, part in zip(grads, parts):
            for p, val in part.items():
                rows = _unit_rows(plan, p)
                g[rows] += val
    return tuple(grads)


def dq_rows_fp64(q, k, v, do, rows, dtype="f32", scale=None, key_block=16384):
    """dQ of selected query rows only (the definition restricted to those rows).

    Needs each row's own LSE and Delta, which depend on that row alone, so the cost is
    O(rows x N x d) per head: usable at sizes where the dense gradients are not.
    Two passes over key blocks: (max, sum) for LSE and O, then the dQ sum.
    Returns dQ [R, H, d] float64.
    """
    n, h_count, d = q.shape
    if scale is None:
        scale = default_scale(d)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, h_count, d))
    for h in range(h_count):
        qh = to_f64(q[rows, h, :], dtype)
        doh = to_f64(do[rows, h, :], dtype)
        m = np.full(rows.size, -np.inf)
        for j0 in range(0, n, key_block):
            kb = to_f64(k[j0:j0 + key_block, h, :], dtype)
            m = np.maximum(m, ((qh @ kb.T) * scale).max(axis=1))
        l = np.zeros(rows.size)
        o = np.zeros((rows.size, d))
        for j0 in range(0, n, key_block):
            kb = to_f64(k[j0:j0 + key_block, h, :], dtype)
            vb = to_f64(v[j0:j0 + key_block, h, :], dtype)
            e = np.exp((qh @ kb.T) * scale - m[:, None])
            l += e.sum(axis=1)
            o += e @ vb
        o /= l[:, None]
        lse = m + np.log(l)
        delta = (doh * o).sum(axis=1)
        acc = np.zeros((rows.size, d))
        for j0 in range(0, n, key_block):
            kb = to_f64(k[j0:j0 + key_block, h, :], dtype)
            vb = to_f64(v[j0:j0 + key_block, h, :], dtype)
            p = np.exp((qh @ kb.T) * scale - lse[:, None])
            ds = p * (doh @ vb.T - delta[:, None])
            acc += ds @ kb
        out[:, h, :] = scale * acc
    return out
