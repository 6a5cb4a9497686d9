"""Pins for the oracle's CQS recomposition (CPU only).

"Stream-CQSA: Exact Out-of-Memory Recovery for Attention" (abstract) and the
Lattice summary of arXiv:2604.20819 state that recomposing the tasks' local
statistics gives exactly full-sequence attention.  The recomposition therefore
has to match the dense definition up to float64 rounding on every plan shape;
a dropped or doubled block, a wrong merge weight or a wrong owner fails here.
"""
import itertools

import numpy as np
import pytest

from memory_bounded_streaming_amd.inputs import gen_qkv
from oracle.attention import attention_fp64
from oracle.plan import make_plan
from oracle.recompose import finalize_fp64, merge_fp64, recompose_fp64, task_partials_fp64

PLANS = [[1], [2], [3], [4], [2, 2], [3, 2], [2, 3], [3, 3], [4, 2]]


@pytest.mark.parametrize("ls,unit", [(ls, u) for ls in PLANS for u in (1, 3)] + [([3], 64), ([2, 2], 16)])
def test_recompose_equals_dense_attention(ls, unit):
    n = int(np.prod([l * (l - 1) + 1 for l in ls])) * unit
    plan = make_plan(n, ls)
    seed = 100 + n + len(ls)
    q, k, v = gen_qkv(seed, n, 2, 8, dtype="f32")
    o_ref, lse_ref = attention_fp64(q, k, v, dtype="f32")
    o, lse = recompose_fp64(q, k, v, plan, dtype="f32")
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)


def test_recompose_on_n3584_shape_bf16():
    plan = make_plan(3584, [3])
    q, k, v = gen_qkv(0, 3584, 1, 64, dtype="bf16")
    rows = np.array([0, 1, 511, 512, 2047, 3583])
    o_ref, lse_ref = attention_fp64(q, k, v, rows=rows, dtype="bf16")
    o, lse = recompose_fp64(q, k, v, plan, dtype="bf16", rows=rows)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13)


def test_merge_identity_and_commutativity():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(5), rng.random(5) + 0.5, rng.standard_normal((5, 3)))
    empty = (np.full(5, -np.inf), np.zeros(5), np.zeros((5, 3)))
    m, l, n = merge_fp64(a, empty)
    np.testing.assert_array_equal(m, a[0])
    np.testing.assert_array_equal(l, a[1])
    np.testing.assert_array_equal(n, a[2])
    m2, l2, n2 = merge_fp64(empty, empty)
    assert np.isneginf(m2).all() and (l2 == 0).all() and np.isfinite(n2).all()
    b = (rng.standard_normal(5), rng.random(5) + 0.5, rng.standard_normal((5, 3)))
    for x, y in zip(merge_fp64(a, b), merge_fp64(b, a)):
        np.testing.assert_array_equal(x, y)


def test_merge_of_any_key_split_is_exact():
    # split the keys of one row set into random disjoint groups: merge == dense
    rng = np.random.default_rng(2)
    n, d = 90, 6
    q, k, v = (rng.standard_normal((n, 1, d)) for _ in range(3))
    s = (q[:, 0] @ k[:, 0].T) / np.sqrt(d)
    groups = np.array_split(rng.permutation(n), 4)
    acc = (np.full(n, -np.inf), np.zeros(n), np.zeros((n, d)))
    for g in groups:
        sg = s[:, g]
        m = sg.max(axis=1)
        p = np.exp(sg - m[:, None])
        acc = merge_fp64(acc, (m, p.sum(axis=1), p @ v[g, 0]))
    o, lse = finalize_fp64(*acc)
    o_ref, lse_ref = attention_fp64(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                                    dtype="f32")
    # q/k/v were float64 draws; compare against the same arithmetic in float64
    p = np.exp(s - s.max(axis=1, keepdims=True))
    np.testing.assert_allclose(o, (p @ v[:, 0]) / p.sum(axis=1, keepdims=True), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, s.max(axis=1) + np.log(p.sum(axis=1)), rtol=1e-13)
    assert o_ref.shape == (n, 1, d) and lse_ref.shape == (1, n)


def test_single_task_partial_is_the_dense_statistic():
    plan = make_plan(40, [1])
    q, k, v = gen_qkv(9, 40, 2, 5, dtype="f32")
    parts = task_partials_fp64(q, k, v, plan, plan.tasks[0], dtype="f32")
    rows, m, l, n = parts[0]
    _, lse_ref = attention_fp64(q, k, v, dtype="f32")
    np.testing.assert_allclose(m + np.log(l), lse_ref.T, rtol=1e-14)


def test_partials_cover_each_pair_once_by_key_count():
    # count admitted keys per (row, task): summed over tasks it is N for every row
    plan = make_plan(13 * 2, [4])
    total = np.zeros(plan.n_units, dtype=np.int64)
    for task in plan.tasks:
        for a, p in enumerate(task.units):
            total[p] += sum(c for _, c in task.key_runs(a)) * plan.unit_tokens
    assert (total == plan.n).all()
    for ls in itertools.product([2, 3], repeat=2):
        plan = make_plan(int(np.prod([l * (l - 1) + 1 for l in ls])), list(ls))
        total = np.zeros(plan.n_units, dtype=np.int64)
        for task in plan.tasks:
            for a, p in enumerate(task.units):
                total[p] += sum(c for _, c in task.key_runs(a))
        assert (total == plan.n_units).all()


@pytest.mark.parametrize("ls,n", [([3], 50), ([3], 8), ([4], 100), ([2, 2], 20), ([3, 2], 100), ([2], 4), ([1], 5)])
def test_padded_recompose_equals_dense_attention(ls, n):
    # reading R12: positions past N are padding and are never attended
    plan = make_plan(n, ls, pad=True)
    assert plan.n == n and plan.n_pad >= n and plan.n_pad % plan.n_units == 0
    assert plan.n_pad - n < plan.n_units
    q, k, v = gen_qkv(300 + n, n, 2, 8, dtype="f32")
    o_ref, lse_ref = attention_fp64(q, k, v, dtype="f32")
    o, lse = recompose_fp64(q, k, v, plan, dtype="f32")
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)


def test_padded_segments_stop_at_n():
    plan = make_plan(50, [3], pad=True)  # 7 units of 8 tokens: 56 padded positions
    assert plan.unit_tokens == 8
    for task in plan.tasks:
        for g, ln, off in task.segments(plan.unit_tokens, plan.n):
            assert 0 < ln and g + ln <= 50
    with pytest.raises(Exception):
        make_plan(50, [3])
    with pytest.raises(Exception):  # fewer tokens than units
        make_plan(5, [3], pad=True)


@pytest.mark.parametrize("ls,n", [([3], 21), ([4], 13 * 3), ([2, 2], 18), ([3, 2], 42), ([1], 9), ([3], 50)])
def test_causal_recompose_equals_dense_causal_attention(ls, n):
    prod_c = int(np.prod([l * (l - 1) + 1 for l in ls]))
    plan = make_plan(n, ls, pad=n % prod_c != 0, causal=True)
    q, k, v = gen_qkv(500 + n, n, 2, 8, dtype="f32")
    o_ref, lse_ref = attention_fp64(q, k, v, dtype="f32", causal=True)
    o, lse = recompose_fp64(q, k, v, plan, dtype="f32")
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)
