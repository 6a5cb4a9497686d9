"""Reference CQS planner (oracle; test infrastructure only).

What the pages fix
------------------
"Stream-CQSA: Breaking the Billion-Token Barrier on a Single GPU" (wispaper
explainer):
  * section "The 'CQS Divide': Attention as a Steiner System": N tokens are cut
    into c chunks; when c = l(l-1)+1 there are c subsequences of l chunks each
    in which any two chunks appear together in one subsequence and no other
    (a Steiner system S(2,l,c));
  * section "The Recursive Benefit": a subsequence that is still too large is
    divided again with CQS Divide;
  * section "Implementation: From High-Level Logic to GPU Kernels": a CQS Mask
    prevents redundant computation in overlapping chunk regions.
"Stream-CQSA: Exact Out-of-Memory Recovery for Attention" (arXiv 2604.20819),
abstract: the construction comes from cyclic quorum sets.

Readings (the pages leave these steps open; each is the plainest one the rest
supports)
---------------------------------------------------------------------------
R1  Difference set: for l >= 2, the lexicographically smallest sorted set
    D of l residues mod c with {0, 1} in D whose l(l-1) differences (a-b) mod c,
    a != b, are exactly 1..c-1 (a perfect difference set; cyclic quorum).  For
    l = 1, D = {0} and c = 1 (no division).  l = 7 (c = 43) has none.
R2  Chunks: a level's token list of length T is cut into c equal contiguous
    chunks.  The whole plan requires N to be a multiple of prod(c_k) (the "unit"
    grid); otherwise the division is rejected.
R3  Subsequence t = sorted{(t + d) mod c : d in D}; its token list is its chunks
    concatenated in ascending chunk order (order preserving).
R4  CQS Mask: inside task t, query i and key j are admitted iff they lie in
    different chunks, or in the same chunk x with x == t (the chunk that enters
    task t through d = 0 owns its diagonal block).
R5  Recursion: R2-R4 are applied to each task's token list with the next
    level's l; admission is the AND of all levels' masks; the task id is
    mixed-radix, outer level most significant; tasks run in ascending id.
R6  Unit = N / prod(c_k) tokens; every ownership boundary is unit aligned.
R16 Causal variant (optional): row i attends keys j <= i.  The division and the
    owners are unchanged; inside a task (whose token list is in ascending global
    order, R3) an admitted unit pair (a, b) is kept only if b <= a: b < a is fully
    visible, b == a is the diagonal block, masked element by element (j <= i).
R12 Padding (optional): an N >= prod(c_k) that is not a multiple of prod(c_k) is
    divided as N_pad = ceil(N / prod(c_k)) * prod(c_k) tokens; positions >= N are padding.
    They belong to no segment, no key run and no query block, so every real
    query still meets every real key exactly once and the result is attention
    over the N real tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["NoDifferenceSet", "DivideError", "difference_set", "Plan", "make_plan"]

MAX_L = 10


class NoDifferenceSet(ValueError):
    """No perfect difference set exists for this l (e.g. l = 7)."""


class DivideError(ValueError):
    """N does not divide into the unit grid of the requested levels."""


def difference_set(l: int) -> list[int]:
    """Reading R1: lexicographically smallest perfect difference set with {0,1}.

    Depth-first search over increasing residues; a candidate x is kept only if
    both differences x-a and a-x (mod c) against every chosen a are new.
    """
    if l < 1 or l > MAX_L:
        raise ValueError(f"l must be in 1..{MAX_L}")
    if l == 1:
        return [0]
    c = l * (l - 1) + 1
    chosen = [0, 1]
    used = {1, c - 1}

    def extend(start: int) -> bool:
        if len(chosen) == l:
            return True
        for x in range(start, c):
            new = []
            ok = True
            for a in chosen:
                for diff in ((x - a) % c, (a - x) % c):
                    if diff in used or diff in new:
                        ok = False
                        break
                    new.append(diff)
                if not ok:
                    break
            if not ok:
                continue
            chosen.append(x)
            used.update(new)
            if extend(x + 1):
                return True
            chosen.pop()
            used.difference_update(new)
        return False

    if not extend(2):
        raise NoDifferenceSet(f"no perfect difference set for l={l} (c={c})")
    return chosen


@dataclass
class Task:
    """One innermost subsequence task.

    ``units``    global unit index of each local unit, in local order.
    ``chunk``    chunk[k][a] = chunk index of local unit a at level k, counted in
                 the parent token list of level k.
    ``ids``      the per-level subsequence index t_k (the mixed-radix digits).
    """
    tid: int
    ids: tuple
    units: list
    chunk: list = field(default_factory=list)

    def admitted(self, a: int, b: int) -> bool:
        """Reading R4/R5: query unit a may attend key unit b inside this task."""
        for k, t_k in enumerate(self.ids):
            ca, cb = self.chunk[k][a], self.chunk[k][b]
            if ca == cb and ca != t_k:
                return False
        return True

    def key_runs(self, a: int, causal: bool = False) -> list:
        """Admitted key units of local query unit a as (local start, count) runs
        (with causal, only units b <= a: reading R16)."""
        runs = []
        for b in range(len(self.units)):
            if not self.admitted(a, b) or (causal and b > a):
                continue
            if runs and runs[-1][0] + runs[-1][1] == b:
                runs[-1][1] += 1
            else:
                runs.append([b, 1])
        return [tuple(r) for r in runs]

    def segments(self, unit_tokens: int, n_real: int | None = None) -> list:
        """Maximal globally contiguous pieces: (global_start, length, local_offset) in tokens.

        With ``n_real`` (reading R12) the pieces are cut at the first padding token.
        """
        segs = []
        for a, g in enumerate(self.units):
            if segs and segs[-1][0] + segs[-1][1] == g:
                segs[-1][1] += 1
            else:
                segs.append([g, 1, a])
        out = [(g * unit_tokens, n * unit_tokens, a * unit_tokens) for g, n, a in segs]
        if n_real is not None:
            out = [(g, min(ln, n_real - g), a) for g, ln, a in out if g < n_real]
        return out


@dataclass
class Plan:
    n: int
    ls: list
    cs: list
    sets: list
    unit_tokens: int
    n_units: int
    tasks: list
    n_pad: int = 0   # tokens the division covers (n_pad >= n; == n unless padded)
    causal: bool = False

    def coverage(self) -> np.ndarray:
        """[U, U] int32: entry [p][q] is the id of the task owning (query unit p, key unit q).

        -1 marks a pair no task admits; -2 marks a pair admitted twice.  A valid
        plan has neither (the S(2,l,c) property of the CQS Divide section).
        """
        u = self.n_units
        cov = np.full((u, u), -1, dtype=np.int32)
        for task in self.tasks:
            for a, p in enumerate(task.units):
                for b, q in enumerate(task.units):
                    if task.admitted(a, b) and not (self.causal and q > p):
                        cov[p, q] = task.tid if cov[p, q] == -1 else -2
        return cov

    def serialize(self) -> np.ndarray:
        """Canonical int64 schedule record.

        header: n_levels, (c_k, l_k) per level, n_tasks, unit_tokens, n_units
        per task in ascending id:
            tid, t_1..t_L, n_segments, (global_start, length, local_offset) per
            segment [tokens], n_query_units, then per local query unit:
            global_unit, n_runs, (key_local_unit_start, key_unit_count) per run
        """
        out = [len(self.cs)]
        for c, l in zip(self.cs, self.ls):
            out += [c, l]
        out += [len(self.tasks), self.unit_tokens, self.n_units]
        for task in self.tasks:
            out.append(task.tid)
            out += list(task.ids)
            segs = task.segments(self.unit_tokens, self.n)
            out.append(len(segs))
            for s in segs:
                out += list(s)
            out.append(len(task.units))
            for a, g in enumerate(task.units):
                runs = task.key_runs(a, self.causal)
                out += [g, len(runs)]
                for r in runs:
                    out += list(r)
        return np.asarray(out, dtype=np.int64)


def make_plan(n: int, ls: list, pad: bool = False, causal: bool = False) -> Plan:
    """Build the plan for N tokens and per-level l values (readings R1-R6; R12 if pad,
    R16 if causal)."""
    if n <= 0 or not ls:
        raise ValueError("need n > 0 and at least one level")
    sets = [difference_set(l) for l in ls]
    cs = [l * (l - 1) + 1 for l in ls]
    prod_c = int(np.prod(cs))
    if n % prod_c and not pad:
        raise DivideError(f"N={n} is not a multiple of prod(c)={prod_c}")
    if prod_c > n:
        raise DivideError(f"N={n} is smaller than prod(c)={prod_c}")
    n_pad = -(-n // prod_c) * prod_c
    unit = n_pad // prod_c

    # (global units, per-level chunk indices, per-level ids) of partially divided tasks
    frontier = [(list(range(prod_c)), [], ())]
    for c, l, dset in zip(cs, ls, sets):
        nxt = []
        for units, chunks, ids in frontier:
            per_chunk = len(units) // c
            for t in range(c):
                members = sorted((t + d) % c for d in dset)
                pos = [x * per_chunk + i for x in members for i in range(per_chunk)]
                sub_units = [units[p] for p in pos]
                sub_chunks = [[ch[p] for p in pos] for ch in chunks]
                sub_chunks.append([p // per_chunk for p in pos])
                nxt.append((sub_units, sub_chunks, ids + (t,)))
        frontier = nxt

    tasks = []
    for units, chunks, ids in frontier:
        tid = 0
        for c, t in zip(cs, ids):
            tid = tid * c + t
        tasks.append(Task(tid=tid, ids=ids, units=units, chunk=chunks))
    tasks.sort(key=lambda t: t.tid)
    return Plan(n=n, ls=list(ls), cs=cs, sets=sets, unit_tokens=unit,
                n_units=prod_c, tasks=tasks, n_pad=n_pad, causal=causal)
