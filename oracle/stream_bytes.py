"""Bytes the streamed CQS forward moves, counted by walking the plan (oracle; test
infrastructure only).

"Stream-CQSA: Breaking the Billion-Token Barrier on a Single GPU" (wispaper
explainer), section "Implementation: From High-Level Logic to GPU Kernels": each task
moves its Q, K and V to the GPU, the kernel forms local statistics, and the results
are aggregated (in host memory when the device cannot hold them -- reading R10).
Counted per task in ascending id, per the oracle planner's segments (cut at N,
reading R12):

* H2D: K and V of every segment; Q of every (task, unit) block; with a host
  accumulator, the accumulator block of every visit but a row's first.
* D2H: with a host accumulator, the accumulator block of every visit but the last;
  O (input dtype) and LSE (fp32) of every row once, at its last visit.
* merge (HBM bytes): a row's only visit reads its partial and writes O and LSE; a
  later visit reads the accumulator and the partial and writes the accumulator, or
  O and LSE at the last visit.  A first visit of several writes its partial straight
  into the accumulator (no merge).
* chunk reuse (two K/V staging buffers): a task that follows a task of the same outer
  task copies the K/V rows both hold from the previous staging buffer instead of the
  host (device to device).
"""
from __future__ import annotations

from .plan import Plan

__all__ = ["stream_traffic"]


def stream_traffic(plan: Plan, heads: int, d: int, elem_bytes: int, host_acc: bool, kv_buffers: int = 1) -> dict:
    row = heads * d * elem_bytes          # one token of Q, K, V or O
    part = heads * (d + 2) * 4            # one token's (n, m, l) statistics, fp32
    fin = heads * (d * elem_bytes + 4)    # one token's O and LSE
    visits = 1
    for l in plan.ls:
        visits *= l
    h2d = d2h = merge = d2d = 0
    seen: dict[int, int] = {}
    u = plan.unit_tokens
    prev = None
    for task in plan.tasks:
        tokens = set()
        for g, length, _ in task.segments(u, plan.n):
            tokens.update(range(g, g + length))
        shared = 0
        if kv_buffers == 2 and prev is not None and prev[0] == task.ids[:-1]:
            shared = len(tokens & prev[1])
        d2d += 2 * shared * row
        h2d += 2 * (len(tokens) - shared) * row
        prev = (task.ids[:-1], tokens)
        for p in task.units:
            r = max(0, min(u, plan.n - p * u))
            if r == 0:
                continue
            v = seen.get(p, 0)
            seen[p] = v + 1
            first, last = v == 0, v == visits - 1
            h2d += r * row
            if host_acc and not first:
                h2d += r * part
            if host_acc and not last:
                d2h += r * part
            if last:
                d2h += r * fin
            if visits == 1:
                merge += r * (part + fin)
            elif not first:
                merge += r * (2 * part + (fin if last else part))
    return {"bytes_h2d": h2d, "bytes_d2h": d2h, "merge_bytes": merge, "bytes_d2d": d2d}
