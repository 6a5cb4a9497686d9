"""Dense exact softmax attention in float64 (oracle; test infrastructure only).

Follows the definition the method reproduces exactly: "Stream-CQSA: Exact
Out-of-Memory Recovery for Attention" (arXiv 2604.20819), abstract, measures its
error against dense attention computed in float64; the Lattice summary of
arXiv:2604.20819 states that the recomposed output equals that of undivided
attention.  So the oracle for outputs is the definition itself, not the
method's algorithm:

    s_ij   = scale * <Q[i,h,:], K[j,h,:]>
    M_i    = max_j s_ij
    O[i,h] = sum_j exp(s_ij - M_i) V[j,h,:] / sum_j exp(s_ij - M_i)
    LSE    = M_i + ln sum_j exp(s_ij - M_i)

Batch 1.  Non-causal (every one of the N keys) by default; with causal=True row i
attends the keys j <= i only (the causal variant, reading R16 of ``oracle.plan``).
Computed in two passes over key
blocks (pass 1: the row maximum; pass 2: the exponential sums), i.e. the
textbook stable softmax with no running rescale.  Inputs are taken at their
exact values: float32 arrays, or bfloat16 given as uint16 bit patterns, are
widened to float64 without rounding.
"""
from __future__ import annotations

import numpy as np

__all__ = ["to_f64", "attention_fp64", "default_scale"]


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen an input tensor to float64 exactly.

    ``dtype`` is ``"f32"`` (x is float32) or ``"bf16"`` (x holds the 16-bit
    patterns as uint16: a bfloat16 is the upper half of a float32).
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def default_scale(d: int) -> float:
    """Softmax scale 1/sqrt(d) (stated for the tiny fp32 case; taken for all)."""
    return 1.0 / np.sqrt(float(d))


def attention_fp64(q, k, v, rows=None, dtype="f32", scale=None,
                   key_block=16384, row_block=1024, causal=False):
    """Exact attention outputs for the selected query rows.

    Parameters
    ----------
    q, k, v : arrays [N, H, d] (token-major), float32 or bf16 bits (uint16).
    rows    : 1-D int array of query rows to evaluate (default: all N).
    dtype   : "f32" or "bf16", how q/k/v are stored.
    scale   : softmax scale (default 1/sqrt(d)).
    causal  : mask keys j > i (row i sees tokens 0..i).

    Returns
    -------
    O   : float64 [R, H, d]
    LSE : float64 [H, R] natural-log log-sum-exp of the scaled scores.
    """
    n, h_count, d = q.shape
    if k.shape != (n, h_count, d) or v.shape != (n, h_count, d):
        raise ValueError("q, k, v must share one [N, H, d] shape")
    if rows is None:
        rows = np.arange(n, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    r_count = rows.shape[0]
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((r_count, h_count, d), dtype=np.float64)
    lse = np.zeros((h_count, r_count), dtype=np.float64)
    if r_count == 0:
        return out, lse
    if n == 0:
        raise ValueError("attention over zero keys is undefined")

    for h in range(h_count):
        for r0 in range(0, r_count, row_block):
            sel = rows[r0:r0 + row_block]
            qh = to_f64(q[sel, h, :], dtype)                       # [r, d]
            kend = int(sel.max()) + 1 if causal else n

            def scores(k0):
                kh = to_f64(k[k0:k0 + key_block, h, :], dtype)     # [b, d]
                s = (qh @ kh.T) * scale                            # [r, b]
                if causal:
                    keys = np.arange(k0, k0 + kh.shape[0])
                    s = np.where(keys[None, :] > sel[:, None], -np.inf, s)
                return s

            # pass 1: M_i = max_j s_ij over all (admitted) keys
            row_max = np.full(sel.shape[0], -np.inf)
            for k0 in range(0, kend, key_block):
                np.maximum(row_max, scores(k0).max(axis=1), out=row_max)
            # pass 2: sums of exp(s - M_i) and of exp(s - M_i) * v_j
            denom = np.zeros(sel.shape[0])
            numer = np.zeros((sel.shape[0], d))
            for k0 in range(0, kend, key_block):
                vh = to_f64(v[k0:k0 + key_block, h, :], dtype)
                p = np.exp(scores(k0) - row_max[:, None])
                denom += p.sum(axis=1)
                numer += p @ vh
            out[r0:r0 + sel.shape[0], h, :] = numer / denom[:, None]
            lse[h, r0:r0 + sel.shape[0]] = row_max + np.log(denom)
    return out, lse
