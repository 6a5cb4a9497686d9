"""GPU parity of padded plans (CQSA_FLAG_PAD): any N, divided over the unit grid rounded
up, with positions past N never loaded, attended or written (needs an MI355X).

The oracle takes the same reading (R12 of oracle.plan); every comparison is against
dense fp64 attention over the N real tokens, or against the oracle's per-task
statistics.  Streamed runs must equal the device-resident run bit for bit.
"""
import math

import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import gen_qkv, sample_rows
from oracle.attention import attention_fp64
from oracle.plan import make_plan
from oracle.recompose import task_partials_fp64
from oracle.tolerance import (BF16_LSE_TOL, BF16_REL_TOL, F32_ABS_TOL, F32_LSE_TOL, max_abs_err,
                              rowwise_rel_err)

from gpu_util import DT, as_f64, empty_device, log, pinned, to_device, to_numpy

pytestmark = pytest.mark.gpu

LN2 = math.log(2.0)
PAD = cqsa.CQSA_FLAG_PAD

CASES = [  # levels, N, heads, head_dim, dtype
    ([3], 7 * 192 + 5, 2, 128, "bf16"),    # last unit 191 of 193 rows
    ([3], 8, 1, 64, "f32"),                # units of 2 tokens; units 4..6 are all padding
    ([4], 13 * 97 - 50, 1, 64, "bf16"),
    ([2, 2], 9 * 30 + 1, 2, 64, "bf16"),   # two levels, last unit 23 of 31 rows
    ([3, 2], 21 * 20 + 3, 1, 128, "f32"),
    ([1], 333, 2, 128, "bf16"),            # undivided: nothing to pad
]


def _ids(c):
    return f"l{'x'.join(map(str, c[0]))}-n{c[1]}-h{c[2]}-d{c[3]}-{c[4]}"


def _check(out, ref, dtype):
    if dtype == "f32":
        err = max_abs_err(out, ref)
        assert err <= F32_ABS_TOL, err
    else:
        err = rowwise_rel_err(out, ref)
        assert err <= BF16_REL_TOL, err
    return err


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_padded_partials_match_oracle(case):
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype = case
    log(f"padded partials {_ids(case)}")
    plan = make_plan(n, levels, pad=True)
    q, k, v = gen_qkv(61 + n, n, h, d, dtype)
    V = int(np.prod(levels))
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=PAD) as p:
        assert p.info["padded_tokens"] == plan.n_pad
        nsl = torch.full((V, n, h, d), float("nan"), device="cuda")
        mls = torch.full((V, n, h, 2), float("nan"), device="cuda")
        p.partials(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), nsl, mls)
        torch.cuda.synchronize()
        nsl, mls = nsl.cpu().numpy().astype(np.float64), mls.cpu().numpy().astype(np.float64)
    assert not np.isnan(nsl).any() and not np.isnan(mls).any(), "every real row has every visit slot"
    seen = {}
    for task in plan.tasks:
        for pu, (rows, m_ref, l_ref, n_ref) in task_partials_fp64(q, k, v, plan, task, dtype=dtype).items():
            s = seen.get(pu, 0)
            seen[pu] = s + 1
            if rows.size == 0:
                continue
            m_k, l_k, n_k = mls[s, rows, :, 0], mls[s, rows, :, 1], nsl[s, rows]
            if (l_ref == 0).all():  # every admitted key is padding: the empty triple
                assert np.isneginf(m_k).all() and (l_k == 0).all() and (n_k == 0).all()
                continue
            lse_tol = F32_LSE_TOL if dtype == "f32" else BF16_LSE_TOL
            assert np.abs(m_k * LN2 + np.log(l_k) - (m_ref + np.log(l_ref))).max() <= lse_tol
            _check(n_k / l_k[..., None], n_ref / l_ref[..., None], dtype)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_padded_forward_matches_dense_attention(case):
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype = case
    log(f"padded forward {_ids(case)}")
    q, k, v = gen_qkv(71 + n, n, h, d, dtype)
    o_ref, lse_ref = attention_fp64(q, k, v, dtype=dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=PAD) as p:
        o = empty_device((n, h, d), dtype)
        lse = torch.empty((h, n), device="cuda")
        p.forward(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), o, lse)
        torch.cuda.synchronize()
        err = _check(as_f64(to_numpy(o, dtype), dtype), o_ref, dtype)
        lse_err = np.abs(lse.cpu().numpy() - lse_ref).max()
    log(f"  err {err:.3e} lse {lse_err:.3e}")
    assert lse_err <= (F32_LSE_TOL if dtype == "f32" else BF16_LSE_TOL)


STREAM = [CASES[0], CASES[2], CASES[3], CASES[4]]
MODES = [0, cqsa.CQSA_FLAG_HOST_ACC, cqsa.CQSA_FLAG_KV_SINGLE, cqsa.CQSA_FLAG_HOST_ACC | cqsa.CQSA_FLAG_KV_SINGLE]


def _stream(p, q, k, v, n, h, d, dtype):
    import torch
    tq, qa = pinned((n, h, d), dtype)
    tk, ka = pinned((n, h, d), dtype)
    tv, va = pinned((n, h, d), dtype)
    qa[...], ka[...], va[...] = q, k, v
    to, oa = pinned((n, h, d), dtype)
    tl = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
    st = p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED, stats=True)
    return oa.copy(), tl.numpy().copy(), st


@pytest.mark.parametrize("case", STREAM, ids=_ids)
@pytest.mark.parametrize("flags", MODES, ids=["devacc-kv2", "hostacc-kv2", "devacc-kv1", "hostacc-kv1"])
def test_padded_stream_equals_device_path(case, flags):
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype = case
    log(f"padded stream {_ids(case)} flags={flags}")
    q, k, v = gen_qkv(83 + n, n, h, d, dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=flags | PAD) as p:
        o = empty_device((n, h, d), dtype)
        lse = torch.empty((h, n), device="cuda")
        p.forward(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), o, lse)
        torch.cuda.synchronize()
        o_dev, lse_dev = to_numpy(o, dtype), lse.cpu().numpy()
        oa, la, st = _stream(p, q, k, v, n, h, d, dtype)
    e = 2 if dtype == "bf16" else 4
    # only real rows move: K and V of every visit, Q of every visit (plus accumulators)
    assert st["bytes_h2d"] + st["bytes_d2d"] >= 3 * int(np.prod(levels)) * n * h * d * e
    est = cqsa.cqsa_plan_estimate(n, h, d, DT[dtype], levels, flags=flags | PAD,
                                  rates={"attn_tflops": 1.0, "merge_gbs": 1.0, "h2d_gbs": 1.0, "d2h_gbs": 1.0})
    assert est["bytes_d2h"] == st["bytes_d2h"], "dry run bytes exact"
    assert est["bytes_h2d"] + est["bytes_d2d"] == st["bytes_h2d"] + st["bytes_d2d"]  # padding rows are never copied
    assert np.array_equal(oa, o_dev) and np.array_equal(la, lse_dev), "bit-identical to the device path"


def test_padded_auto_levels_recover_under_budget():
    """An off-grid N whose undivided footprint exceeds the budget: auto levels with padding
    divide until the streamed path fits, and the result is still exact attention."""
    torch = pytest.importorskip("torch")
    n, h, d, dtype = 13 * 13 * 96 + 37, 2, 128, "bf16"
    budget = 10 << 20
    log(f"padded auto levels N={n} budget={budget}")
    q, k, v = gen_qkv(97, n, h, d, dtype)
    with cqsa.Plan(n, h, d, DT[dtype], [4], n_levels=0, budget_bytes=budget, flags=PAD) as p:
        info = p.info
        log(f"  levels {info['l']} unit {info['unit_tokens']} ws {info['stream_workspace_bytes']}")
        assert info["l"] == [4, 4] and info["stream_workspace_bytes"] <= budget
        oa, la, st = _stream(p, q, k, v, n, h, d, dtype)
        assert st["peak_device_bytes"] <= budget
    rows = sample_rows(n, 512, 3, unit_tokens=info["unit_tokens"])
    rows = np.unique(np.concatenate([rows, np.arange(n - 40, n)]))
    o_ref, lse_ref = attention_fp64(q, k, v, rows=rows, dtype=dtype)
    err = rowwise_rel_err(as_f64(oa[rows], dtype), o_ref)
    log(f"  err {err:.3e} on {rows.size} rows")
    assert err <= BF16_REL_TOL
    assert np.abs(la[:, rows] - lse_ref).max() <= BF16_LSE_TOL


def test_padded_full_size_device_sampled_rows():
    """N = 57344 + 333 (off the 7-unit grid), H=8, d=128, bf16, l=3, device-resident:
    2048 sampled rows plus the unit edges and the last rows before N."""
    torch = pytest.importorskip("torch")
    n, h, d = 57344 + 333, 8, 128
    log(f"padded full size N={n}")
    q, k, v = gen_qkv(5, n, h, d, "bf16")
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3], flags=PAD) as p:
        u = p.info["unit_tokens"]
        assert p.info["padded_tokens"] == 7 * u == n + 3
        o = empty_device((n, h, d), "bf16")
        lse = torch.empty((h, n), device="cuda")
        p.forward(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), o, lse)
        torch.cuda.synchronize()
        out, lse = to_numpy(o, "bf16"), lse.cpu().numpy()
    rows = np.unique(np.concatenate([sample_rows(n, 2048, 1, unit_tokens=u), np.arange(n - 64, n)]))
    o_ref, lse_ref = attention_fp64(q, k, v, rows=rows, dtype="bf16")
    err = rowwise_rel_err(as_f64(out[rows], "bf16"), o_ref)
    log(f"  err {err:.3e} on {rows.size} rows")
    assert err <= BF16_REL_TOL
    assert np.abs(lse[:, rows] - lse_ref).max() <= BF16_LSE_TOL
