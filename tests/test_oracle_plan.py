"""Pins for the oracle's CQS planner (CPU only).

Each check ties the planner to something other than itself: the closed
difference-set invariant, brute-force enumeration, the Steiner property
S(2,l,c) stated in "Stream-CQSA: Breaking the Billion-Token Barrier on a Single
GPU" (section "The 'CQS Divide': Attention as a Steiner System"), and a coverage
table derived by hand (tests/golden/l3_coverage.txt).
"""
import itertools
import os

import numpy as np
import pytest

from oracle.plan import DivideError, NoDifferenceSet, difference_set, make_plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# The five workload plans: (levels, N)
CONFIG_PLANS = {
    "n3584_l3": ([3], 3584),
    "n57344_l3": ([3], 57344),
    "n212992_l4": ([4], 212992),
    "n1376256_l5": ([5], 1376256),
    "n12845056_l3x3": ([3, 3], 12845056),
}


def _is_perfect(dset, c):
    diffs = sorted((a - b) % c for a in dset for b in dset if a != b)
    return diffs == list(range(1, c))


@pytest.mark.parametrize("l", [2, 3, 4, 5, 6, 8, 9, 10])
def test_difference_set_closed_invariant(l):
    c = l * (l - 1) + 1
    dset = difference_set(l)
    assert len(dset) == l and dset[:2] == [0, 1] and dset == sorted(dset)
    assert _is_perfect(dset, c)


def test_difference_sets_of_the_workloads():
    # the sets the five workload definitions name
    assert difference_set(3) == [0, 1, 3]
    assert difference_set(4) == [0, 1, 3, 9]
    assert difference_set(5) == [0, 1, 4, 14, 16]
    assert difference_set(1) == [0]


@pytest.mark.parametrize("l", [2, 3, 4, 5])
def test_difference_set_is_lexicographic_minimum_brute_force(l):
    c = l * (l - 1) + 1
    best = None
    for rest in itertools.combinations(range(2, c), l - 2):
        cand = [0, 1] + list(rest)
        if _is_perfect(cand, c):
            best = cand
            break  # combinations() enumerates in lexicographic order
    assert best == difference_set(l)


def test_no_difference_set_for_l7_brute_force():
    # order 6: no projective plane (Bruck-Ryser); confirm by exhausting all
    # 5-subsets of {2..42} next to {0, 1} with a vectorised difference count.
    c = 43
    combos = np.array(list(itertools.combinations(range(2, c), 5)), dtype=np.int64)
    sets = np.concatenate([np.zeros((len(combos), 1), np.int64),
                           np.ones((len(combos), 1), np.int64), combos], axis=1)
    diff = (sets[:, :, None] - sets[:, None, :]) % c
    counts = np.zeros((len(sets), c), dtype=np.int64)
    np.add.at(counts, (np.repeat(np.arange(len(sets)), 49), diff.reshape(len(sets), -1).ravel()), 1)
    perfect = np.all(counts[:, 1:] == 1, axis=1)
    assert not perfect.any()
    with pytest.raises(NoDifferenceSet):
        difference_set(7)


def test_l3_coverage_matches_hand_derived_table():
    want = np.loadtxt(os.path.join(GOLDEN, "l3_coverage.txt"), dtype=np.int32, comments="#")
    plan = make_plan(3584, [3])
    assert plan.unit_tokens == 512
    np.testing.assert_array_equal(plan.coverage(), want)
    assert [t.units for t in plan.tasks] == [[0, 1, 3], [1, 2, 4], [2, 3, 5], [3, 4, 6],
                                             [0, 4, 5], [1, 5, 6], [0, 2, 6]]


@pytest.mark.parametrize("name", list(CONFIG_PLANS))
def test_every_unit_pair_exactly_once(name):
    ls, n = CONFIG_PLANS[name]
    plan = make_plan(n, ls)
    u = plan.n_units
    hits = np.zeros((u, u), dtype=np.int64)
    for task in plan.tasks:
        for a, p in enumerate(task.units):
            for b, q in enumerate(task.units):
                if task.admitted(a, b):
                    hits[p, q] += 1
    assert (hits == 1).all()
    cov = plan.coverage()
    assert (cov >= 0).all()
    assert (cov == cov.T).all()  # a chunk pair meets once, in both directions
    visits = np.zeros(u, dtype=np.int64)
    for task in plan.tasks:
        assert len(task.units) == int(np.prod(ls))
        assert task.units == sorted(task.units)
        for a in range(len(task.units)):
            assert task.key_runs(a), "every (task, query unit) has some key"
        for p in task.units:
            visits[p] += 1
    assert (visits == int(np.prod(ls))).all()


@pytest.mark.parametrize("l", [2, 3, 4, 5])
def test_single_level_load_balance(l):
    # every task owns exactly one diagonal block, so it computes c of its l*l blocks
    c = l * (l - 1) + 1
    plan = make_plan(c, [l])
    for task in plan.tasks:
        work = sum(task.admitted(a, b) for a in range(l) for b in range(l))
        assert work == c
        diag = [task.units[a] for a in range(l) if task.admitted(a, a)]
        assert diag == [task.tid]


def test_two_level_12m_token_plan_shape():
    plan = make_plan(12845056, [3, 3])
    assert plan.unit_tokens == 262144 and plan.n_units == 49 and len(plan.tasks) == 49
    work = [sum(t.admitted(a, b) for a in range(9) for b in range(9)) for t in plan.tasks]
    assert min(work) == 36 and max(work) == 63 and sum(work) == 49 * 49
    # task ids are mixed radix, outer level first
    assert [t.ids for t in plan.tasks[:3]] == [(0, 0), (0, 1), (0, 2)]
    # inner chunks of 3 units straddle the outer chunks of 7 units
    # (outer task 0 = units 0..13 and 21..27, re-cut into 7 chunks of 3 units)
    assert plan.tasks[0].units == [0, 1, 2, 3, 4, 5, 9, 10, 11]
    t4 = plan.tasks[4]  # inner chunks {0, 4, 5}; inner chunk 4 = units {12, 13, 21}
    assert t4.units == [0, 1, 2, 12, 13, 21, 22, 23, 24]
    segs = t4.segments(plan.unit_tokens)
    assert [(s[0] // 262144, s[1] // 262144, s[2] // 262144) for s in segs] == [(0, 3, 0), (12, 2, 3), (21, 4, 5)]


def test_divide_errors():
    with pytest.raises(DivideError):
        make_plan(100, [3])
    with pytest.raises(DivideError):
        make_plan(7 * 7 * 7 * 5, [3, 3, 3, 3])
    with pytest.raises(NoDifferenceSet):
        make_plan(43, [7])


@pytest.mark.parametrize("ls", [[1], [2], [3], [2, 2], [3, 2], [2, 3], [3, 3, 2]])
def test_serialization_round_trip(ls):
    u = int(np.prod([l * (l - 1) + 1 for l in ls]))
    plan = make_plan(u * 5, ls)
    rec = plan.serialize()
    pos = 0
    nl = rec[pos]; pos += 1
    assert nl == len(ls)
    for c, l in zip(plan.cs, plan.ls):
        assert list(rec[pos:pos + 2]) == [c, l]; pos += 2
    n_tasks, unit, n_units = rec[pos:pos + 3]; pos += 3
    assert (n_tasks, unit, n_units) == (len(plan.tasks), 5, u)
    for task in plan.tasks:
        assert rec[pos] == task.tid; pos += 1
        assert tuple(rec[pos:pos + nl]) == task.ids; pos += nl
        nseg = rec[pos]; pos += 1
        covered = 0
        for _ in range(nseg):
            g, ln, off = rec[pos:pos + 3]; pos += 3
            assert off == covered and ln > 0
            covered += ln
        assert covered == len(task.units) * 5
        nq = rec[pos]; pos += 1
        assert nq == len(task.units)
        for a in range(nq):
            assert rec[pos] == task.units[a]; pos += 1
            nr = rec[pos]; pos += 1
            pos += 2 * nr
    assert pos == len(rec)


@pytest.mark.parametrize("ls,unit", [([3], 2), ([4], 1), ([2, 2], 1), ([3, 2], 1), ([1], 5)])
def test_causal_coverage_is_the_lower_triangle_once(ls, unit):
    from oracle.plan import make_plan as mk
    n = int(np.prod([l * (l - 1) + 1 for l in ls])) * unit
    plan = mk(n, ls, causal=True)
    full = mk(n, ls).coverage()
    cov = plan.coverage()
    u = plan.n_units
    lower = np.tril(np.ones((u, u), dtype=bool))
    assert (cov[lower] >= 0).all() and (cov[~lower] == -1).all()
    np.testing.assert_array_equal(cov[lower], full[lower])  # same owners as the non-causal plan
    for task in plan.tasks:
        for a in range(len(task.units)):
            assert all(b0 + c - 1 <= a for b0, c in task.key_runs(a, True))
