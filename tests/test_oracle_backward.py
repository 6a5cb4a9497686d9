"""Pins for the fp64 attention gradients and their CQS decomposition (CPU only).

The gradient formulas are checked against things other than themselves: central
finite differences of the loss <dO, O> written here with scipy's softmax, torch's
float64 autograd of the same forward, closed forms (one token, zero keys,
constant values) and the identities sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.
The per-task decomposition must equal the dense gradients on every plan shape.
"""
import numpy as np
import pytest
from scipy.special import softmax

from memory_bounded_streaming_amd.inputs import gen_qkv, gen_tensor
from oracle.backward import (attention_backward_fp64, attention_backward_given_fp64, dq_rows_fp64,
                             recompose_backward_fp64)
from oracle.plan import make_plan


def _loss(q, k, v, do, scale):
    # L = sum_i <dO_i, O_i>, one head, everything float64
    p = softmax((q @ k.T) * scale, axis=1)
    return float(np.sum(do * (p @ v)))


def _inputs(seed, n, h, d):
    q, k, v = gen_qkv(seed, n, h, d, "f32")
    do = gen_tensor(seed, 3, n, h, d, "f32")
    return q, k, v, do


@pytest.mark.parametrize("n,d", [(1, 3), (5, 4), (9, 2)])
def test_gradients_match_central_differences(n, d):
    q, k, v, do = _inputs(11 + n, n, 2, d)
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = attention_backward_fp64(q, k, v, do, dtype="f32")
    eps = 1e-6
    for h in range(2):
        base = [x[:, h].astype(np.float64) for x in (q, k, v)]
        dof = do[:, h].astype(np.float64)
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            num = np.zeros((n, d))
            for i in range(n):
                for t in range(d):
                    plus = [b.copy() for b in base]
                    minus = [b.copy() for b in base]
                    plus[which][i, t] += eps
                    minus[which][i, t] -= eps
                    num[i, t] = (_loss(*plus, dof, scale) - _loss(*minus, dof, scale)) / (2 * eps)
            np.testing.assert_allclose(grad[:, h], num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("n,h,d", [(7, 1, 8), (33, 2, 16), (64, 3, 5)])
def test_gradients_match_torch_autograd(n, h, d):
    torch = pytest.importorskip("torch")
    q, k, v, do = _inputs(3 * n + d, n, h, d)
    dq, dk, dv = attention_backward_fp64(q, k, v, do, dtype="f32")
    tq, tk, tv = (torch.tensor(x.astype(np.float64).transpose(1, 0, 2), requires_grad=True) for x in (q, k, v))
    p = torch.softmax(tq @ tk.transpose(1, 2) / np.sqrt(d), dim=-1)
    o = p @ tv
    o.backward(torch.tensor(do.astype(np.float64).transpose(1, 0, 2)))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-13)


def test_closed_forms():
    # one token: O = V, so dV = dO and no gradient reaches Q or K
    q, k, v, do = _inputs(1, 1, 2, 6)
    dq, dk, dv = attention_backward_fp64(q, k, v, do, dtype="f32")
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    np.testing.assert_array_equal(dv, do.astype(np.float64))
    # K = 0: uniform weights; dV_j = mean_i dO_i for every j, dQ = 0,
    # dK_j = scale/N sum_i <dO_i, V_j - mean V> Q_i
    n, d = 12, 4
    q, k, v, do = _inputs(2, n, 1, d)
    k[:] = 0
    dq, dk, dv = attention_backward_fp64(q, k, v, do, dtype="f32")
    q64, v64, do64 = (x[:, 0].astype(np.float64) for x in (q, v, do))
    np.testing.assert_allclose(dv[:, 0], np.broadcast_to(do64.mean(axis=0), (n, d)), rtol=1e-13, atol=1e-15)
    assert np.abs(dq).max() < 1e-15
    want = (do64 @ (v64 - v64.mean(axis=0)).T).T @ q64 / (n * np.sqrt(d))
    np.testing.assert_allclose(dk[:, 0], want, rtol=1e-12, atol=1e-14)
    # every key has the same value vector: O is that vector whatever the weights, so
    # Q and K get no gradient
    q, k, v, do = _inputs(3, n, 1, d)
    v[:] = v[0]
    dq, dk, dv = attention_backward_fp64(q, k, v, do, dtype="f32")
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gradient_identities(dtype):
    n, h, d = 50, 2, 8
    q, k, v = gen_qkv(4, n, h, d, dtype)
    do = gen_tensor(4, 3, n, h, d, dtype)
    dq, dk, dv = attention_backward_fp64(q, k, v, do, dtype=dtype)
    from oracle.attention import to_f64
    # sum_j dS_ij = 0 for every row, hence sum_j dK_j = 0; sum_j P_ij = 1, hence
    # sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), to_f64(do, dtype).sum(axis=0), rtol=1e-12, atol=1e-12)


PLANS = [([1], 9), ([2], 3 * 4), ([3], 7 * 3), ([4], 13), ([2, 2], 9 * 2), ([3, 2], 21), ([2, 3], 21 * 2)]


@pytest.mark.parametrize("ls,n", PLANS + [([3], 50), ([2, 2], 20), ([4], 100)])
def test_task_decomposition_equals_dense_gradients(ls, n):
    prod_c = int(np.prod([l * (l - 1) + 1 for l in ls]))
    plan = make_plan(n, ls, pad=n % prod_c != 0)
    q, k, v, do = _inputs(40 + n, n, 2, 6)
    dense = attention_backward_fp64(q, k, v, do, dtype="f32")
    split = recompose_backward_fp64(q, k, v, do, plan, dtype="f32")
    for a, b in zip(split, dense):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_decomposition_misses_a_pair_if_a_task_is_dropped():
    # planting a mistake: drop one task and the sum no longer matches
    plan = make_plan(21, [3])
    q, k, v, do = _inputs(5, 21, 1, 4)
    dense = attention_backward_fp64(q, k, v, do, dtype="f32")
    plan.tasks = plan.tasks[1:]
    split = recompose_backward_fp64(q, k, v, do, plan, dtype="f32")
    assert max(np.abs(a - b).max() for a, b in zip(split, dense)) > 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dq_rows_equal_dense_rows(dtype):
    # the row-restricted dQ (blocked keys, two passes) against the dense gradients
    n, h, d = 70, 2, 8
    q, k, v = gen_qkv(8, n, h, d, dtype)
    do = gen_tensor(8, 3, n, h, d, dtype)
    dq, _, _ = attention_backward_fp64(q, k, v, do, dtype=dtype)
    rows = np.array([0, 3, 31, 69])
    np.testing.assert_allclose(dq_rows_fp64(q, k, v, do, rows, dtype=dtype, key_block=16), dq[rows],
                               rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("n,h,d", [(9, 1, 4), (40, 2, 8)])
def test_causal_gradients_match_torch_autograd(n, h, d):
    torch = pytest.importorskip("torch")
    q, k, v, do = _inputs(7 * n, n, h, d)
    dq, dk, dv = attention_backward_fp64(q, k, v, do, dtype="f32", causal=True)
    tq, tk, tv = (torch.tensor(x.astype(np.float64).transpose(1, 0, 2), requires_grad=True) for x in (q, k, v))
    s = tq @ tk.transpose(1, 2) / np.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    (torch.softmax(s, dim=-1) @ tv).backward(torch.tensor(do.astype(np.float64).transpose(1, 0, 2)))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("ls,n", [([3], 21), ([2, 2], 18), ([3], 50), ([4], 13)])
def test_causal_task_decomposition_equals_dense(ls, n):
    prod_c = int(np.prod([l * (l - 1) + 1 for l in ls]))
    plan = make_plan(n, ls, pad=n % prod_c != 0, causal=True)
    q, k, v, do = _inputs(60 + n, n, 2, 6)
    dense = attention_backward_fp64(q, k, v, do, dtype="f32", causal=True)
    split = recompose_backward_fp64(q, k, v, do, plan, dtype="f32")
    for a, b in zip(split, dense):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_grad_metric_floors_rows_that_vanish():
    from oracle.tolerance import GRAD_ROW_FLOOR, grad_rel_err, rowwise_rel_err
    ref = np.array([[[0.0, 0.0]], [[1.0, -2.0]]])
    got = ref + np.array([[[1e-4, 0.0]], [[0.0, 1e-3]]])
    assert rowwise_rel_err(got, ref) > 1e100          # the zero row breaks a pure row-wise ratio
    assert grad_rel_err(got, ref) == pytest.approx(max(1e-4 / (GRAD_ROW_FLOOR * 2.0), 1e-3 / 2.0))
    # causal dQ: the first query attends only itself, so its gradient row is exactly zero
    q, k, v, do = _inputs(3, 6, 1, 4)
    dq, _, _ = attention_backward_fp64(q, k, v, do, dtype="f32", causal=True)
    assert np.abs(dq[0]).max() < 1e-15 and np.abs(dq[1:]).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_backward_given_exact_statistics_is_the_gradient(causal):
    from oracle.attention import attention_fp64
    n, h, d = 30, 2, 8
    q, k, v, do = _inputs(21, n, h, d)
    o, lse = attention_fp64(q, k, v, dtype="f32", causal=causal)
    want = attention_backward_fp64(q, k, v, do, dtype="f32", causal=causal)
    got = attention_backward_given_fp64(q, k, v, o, lse, do, dtype="f32", causal=causal)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)
    # a rounded O moves Delta and so dQ, dK (not dV, which does not involve O)
    o_r = o.astype(np.float32)
    got_r = attention_backward_given_fp64(q, k, v, o_r, lse, do, dtype="f32", causal=causal)
    np.testing.assert_allclose(got_r[2], want[2], rtol=1e-11, atol=1e-13)
    assert np.abs(got_r[0] - want[0]).max() > 0
