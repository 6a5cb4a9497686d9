"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every call goes through the C ABI (ctypes binding).  Small plans are compared element
by element on every row (they span several tiles and ragged tails); full-size
workloads are compared on seeded sampled rows.  Tolerances: float32 inputs 1e-5 max
abs; bfloat16 inputs 2e-2 max row-wise relative error (oracle.tolerance).
"""
import math

import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import bf16_bits_to_f32, gen_qkv, round_to_bf16_bits
from oracle.attention import attention_fp64
from oracle.plan import make_plan
from oracle.recompose import finalize_fp64, merge_fp64, task_partials_fp64
from oracle.tolerance import (BF16_LSE_TOL, BF16_REL_TOL, F32_ABS_TOL, F32_LSE_TOL, error_report, max_abs_err,
                              rowwise_rel_err)

from gpu_util import DT, as_f64, empty_device, log, oracle_rows, to_device, to_numpy

pytestmark = pytest.mark.gpu

LN2 = math.log(2.0)

# (levels, unit tokens, heads, head_dim, dtype): tiles of 128 query rows / 64 keys, ragged tails
SMALL = [
    ([3], 40, 2, 128, "bf16"),
    ([3], 200, 1, 64, "bf16"),
    ([4], 130, 3, 128, "bf16"),
    ([2, 2], 24, 2, 64, "bf16"),      # has a (task, query unit) with no admitted key
    ([1], 300, 2, 128, "bf16"),       # undivided: one task
    ([3], 64, 1, 64, "f32"),
    ([4], 97, 2, 128, "f32"),
    ([2, 3], 8, 1, 64, "f32"),
    ([1], 1, 1, 64, "f32"),           # a single token: O = V
    ([3], 1, 1, 128, "bf16"),         # units of one token
    ([5], 70, 2, 64, "f32"),          # l = 5 .. 10: 21 .. 91 tasks of 5 .. 10 units
    ([6], 50, 1, 128, "bf16"),
    ([8], 33, 1, 64, "bf16"),
    ([9], 24, 1, 64, "f32"),
    ([10], 20, 2, 128, "bf16"),
    ([3], 40, 32, 128, "bf16"),       # many heads: row stride 4096 elements
    ([4], 20, 40, 64, "bf16"),        # a head count that is not a power of two
]


def _ids(case):
    levels, u, h, d, dt = case
    return f"l{'x'.join(map(str, levels))}-u{u}-h{h}-d{d}-{dt}"


def _check(out, ref, dtype, what):
    if dtype == "f32":
        err = max_abs_err(out, ref)
        log(f"  {what}: max abs err {err:.3e}")
        assert err <= F32_ABS_TOL, what
    else:
        err = rowwise_rel_err(out, ref)
        log(f"  {what}: row-wise rel err {err:.3e}")
        assert err <= BF16_REL_TOL, what


def _visit_slots(plan):
    seen, slots = {}, {}
    for t in plan.tasks:
        for p in t.units:
            slots[(t.tid, p)] = seen.get(p, 0)
            seen[p] = seen.get(p, 0) + 1
    return slots


@pytest.mark.parametrize("case", SMALL, ids=_ids)
def test_partials_match_oracle_task_statistics(case):
    levels, u, h, d, dtype = case
    n = int(np.prod([l * (l - 1) + 1 for l in levels])) * u
    log(f"partials {_ids(case)} N={n}")
    torch = pytest.importorskip("torch")
    plan = make_plan(n, levels)
    q, k, v = gen_qkv(17 + n, n, h, d, dtype)
    V = int(np.prod(levels))
    with cqsa.Plan(n, h, d, DT[dtype], levels) as p:
        nsl = torch.full((V, n, h, d), float("nan"), device="cuda")
        mls = torch.full((V, n, h, 2), float("nan"), device="cuda")
        p.partials(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), nsl, mls)
        torch.cuda.synchronize()
        nsl, mls = nsl.cpu().numpy().astype(np.float64), mls.cpu().numpy().astype(np.float64)
    slots = _visit_slots(plan)
    assert not np.isnan(nsl).any() and not np.isnan(mls).any(), "every slot row is written"
    tol_o = F32_ABS_TOL if dtype == "f32" else BF16_REL_TOL
    for task in plan.tasks:
        parts = task_partials_fp64(q, k, v, plan, task, dtype=dtype)
        for a, pu in enumerate(task.units):
            rows, m_ref, l_ref, n_ref = parts[pu]
            s = slots[(task.tid, pu)]
            m_k = mls[s, rows, :, 0]
            l_k = mls[s, rows, :, 1]
            n_k = nsl[s, rows]
            if not task.key_runs(a):
                assert np.isneginf(m_k).all() and (l_k == 0).all() and (n_k == 0).all()
                continue
            lse_k = m_k * LN2 + np.log(l_k)
            lse_ref = m_ref + np.log(l_ref)
            assert np.abs(lse_k - lse_ref).max() <= (F32_LSE_TOL if dtype == "f32" else BF16_LSE_TOL)
            o_k = n_k / l_k[..., None]
            o_ref = n_ref / l_ref[..., None]
            err = max_abs_err(o_k, o_ref) if dtype == "f32" else rowwise_rel_err(o_k, o_ref)
            assert err <= tol_o, (task.tid, pu, err)


@pytest.mark.parametrize("case", SMALL, ids=_ids)
def test_forward_device_matches_dense_attention(case):
    levels, u, h, d, dtype = case
    n = int(np.prod([l * (l - 1) + 1 for l in levels])) * u
    log(f"forward {_ids(case)} N={n}")
    torch = pytest.importorskip("torch")
    q, k, v = gen_qkv(29 + n, n, h, d, dtype)
    o_ref, lse_ref = attention_fp64(q, k, v, dtype=dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels) as p:
        o = empty_device((n, h, d), dtype)
        lse = torch.empty((h, n), device="cuda")
        ws = torch.empty(p.workspace_size(cqsa.CQSA_RES_DEVICE), dtype=torch.uint8, device="cuda")
        p.forward(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), o, lse,
                  residency=cqsa.CQSA_RES_DEVICE, workspace=ws)
        torch.cuda.synchronize()
        out = as_f64(to_numpy(o, dtype), dtype)
        _check(out, o_ref, dtype, "O")
        assert np.abs(lse.cpu().numpy() - lse_ref).max() <= (F32_LSE_TOL if dtype == "f32" else BF16_LSE_TOL)


@pytest.mark.parametrize("profile", ["ramp", "spikes"])
def test_forward_reference_max_moves(profile):
    """Scores that keep growing along the keys, so the running reference max of the bf16
    kernel must move on many tiles ("ramp"), and isolated keys whose logits pass it by far
    more than 2^7 in log2 units, so the weights formed against the old reference overflow
    to inf before it moves ("spikes").  Device path and per-task partials against the
    fp64 oracle."""
    torch = pytest.importorskip("torch")
    levels, u, h, d = [3], 300, 2, 128
    n = 7 * u
    log(f"reference max {profile} N={n}")
    q, k, v = gen_qkv(71, n, h, d, "bf16")
    kf = bf16_bits_to_f32(k)
    if profile == "ramp":
        factor = 1.0 + 6.0 * np.arange(n) / n
    else:
        factor = np.ones(n)
        factor[37::211] = 40.0
    k = round_to_bf16_bits((kf * factor[:, None, None]).astype(np.float32))
    o_ref, lse_ref = attention_fp64(q, k, v, dtype="bf16")
    plan = make_plan(n, levels)
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels) as p:
        qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
        o = empty_device((n, h, d), "bf16")
        lse = torch.empty((h, n), device="cuda")
        p.forward(qd, kd, vd, o, lse)
        nsl = torch.full((3, n, h, d), float("nan"), device="cuda")
        mls = torch.full((3, n, h, 2), float("nan"), device="cuda")
        p.partials(qd, kd, vd, nsl, mls)
        torch.cuda.synchronize()
        out = as_f64(to_numpy(o, "bf16"), "bf16")
        nsl, mls = nsl.cpu().numpy().astype(np.float64), mls.cpu().numpy().astype(np.float64)
        lse_k = lse.cpu().numpy()
    _check(out, o_ref, "bf16", "O")
    lse_err = np.abs(lse_k - lse_ref).max()
    log(f"  LSE abs err {lse_err:.3e} (|LSE| up to {np.abs(lse_ref).max():.1f})")
    assert lse_err <= BF16_LSE_TOL
    slots = _visit_slots(plan)
    for task in plan.tasks:
        parts = task_partials_fp64(q, k, v, plan, task, dtype="bf16")
        for a, pu in enumerate(task.units):
            rows, m_ref, l_ref, n_ref = parts[pu]
            if not task.key_runs(a):
                continue
            sl = slots[(task.tid, pu)]
            m_k, l_k, n_k = mls[sl, rows, :, 0], mls[sl, rows, :, 1], nsl[sl, rows]
            assert np.isfinite(m_k).all() and (l_k >= 1.0).all() and (l_k <= 2.0 ** 8 * 2 * n).all()
            assert np.abs(m_k * LN2 + np.log(l_k) - (m_ref + np.log(l_ref))).max() <= BF16_LSE_TOL
            assert rowwise_rel_err(n_k / l_k[..., None], n_ref / l_ref[..., None]) <= BF16_REL_TOL


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_merge_kernel_matches_fp64_merge(dtype, d):
    torch = pytest.importorskip("torch")
    levels, u, h = [3], 50, 2
    n = 7 * u
    log(f"merge {dtype} d={d}")
    plan = make_plan(n, levels)
    q, k, v = gen_qkv(5, n, h, d, dtype)
    slots = _visit_slots(plan)
    V = 3
    n_in = np.zeros((V, n, h, d), np.float32)
    ml_in = np.zeros((V, n, h, 2), np.float32)
    acc = {}
    for task in plan.tasks:
        for pu, (rows, m, l, nn) in task_partials_fp64(q, k, v, plan, task, dtype=dtype).items():
            s = slots[(task.tid, pu)]
            # the same float32 values feed both merges
            m32, l32, n32 = (m / LN2).astype(np.float32), l.astype(np.float32), nn.astype(np.float32)
            ml_in[s, rows, :, 0], ml_in[s, rows, :, 1], n_in[s, rows] = m32, l32, n32
            trip = (m32.astype(np.float64) * LN2, l32.astype(np.float64), n32.astype(np.float64))
            acc[pu] = merge_fp64(acc[pu], trip) if pu in acc else trip
    o_ref = np.zeros((n, h, d))
    lse_ref = np.zeros((h, n))
    for pu, trip in acc.items():
        o_u, lse_u = finalize_fp64(*trip)
        o_ref[pu * u:(pu + 1) * u] = o_u
        lse_ref[:, pu * u:(pu + 1) * u] = lse_u.T
    with cqsa.Plan(n, h, d, DT[dtype], levels) as p:
        o = empty_device((n, h, d), dtype)
        lse = torch.empty((h, n), device="cuda")
        p.merge(torch.from_numpy(n_in).cuda(), torch.from_numpy(ml_in).cuda(), o, lse)
        torch.cuda.synchronize()
        out = as_f64(to_numpy(o, dtype), dtype)
    if dtype == "f32":
        assert max_abs_err(out, o_ref) <= 2e-6
    else:
        assert rowwise_rel_err(out, o_ref) <= 4.0 * 2.0 ** -9
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= 1e-5


def test_n3584_fp32_every_row():
    """N=3584, H=1, d=64, fp32, l=3 ({0,1,3} mod 7, chunks of 512): every row."""
    torch = pytest.importorskip("torch")
    n, h, d = 3584, 1, 64
    log("N=3584 fp32, every row")
    q, k, v = gen_qkv(0, n, h, d, "f32")
    o_ref, lse_ref = attention_fp64(q, k, v, dtype="f32")
    with cqsa.Plan(n, h, d, cqsa.CQSA_F32, [3]) as p:
        assert p.info["unit_tokens"] == 512
        o = torch.empty((n, h, d), device="cuda")
        lse = torch.empty((h, n), device="cuda")
        p.forward(to_device(q, "f32"), to_device(k, "f32"), to_device(v, "f32"), o, lse)
        torch.cuda.synchronize()
        rep = error_report(o.cpu().numpy(), o_ref)
        log(f"  N=3584 {rep}")
        assert rep["max_abs"] <= F32_ABS_TOL
        assert np.abs(lse.cpu().numpy() - lse_ref).max() <= 1e-5


def test_n57344_bf16_every_row_and_determinism():
    """N=57344, H=8, d=128, bf16, l=3, device-resident: every row against the oracle
    (1.35e13 fp64 FLOP, spread over the host's cores), and two calls bit-identical."""
    torch = pytest.importorskip("torch")
    n, h, d = 57344, 8, 128
    log("N=57344 H=8 bf16 device-resident")
    q, k, v = gen_qkv(0, n, h, d, "bf16")
    rows = np.arange(n)
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
        ws = torch.empty(p.workspace_size(cqsa.CQSA_RES_DEVICE), dtype=torch.uint8, device="cuda")
        outs = []
        for _ in range(2):
            o = empty_device((n, h, d), "bf16")
            lse = torch.empty((h, n), device="cuda")
            p.forward(qd, kd, vd, o, lse, workspace=ws)
            torch.cuda.synchronize()
            outs.append((to_numpy(o, "bf16"), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1]), "deterministic"
    log(f"  oracle on all {rows.size} rows")
    o_ref, lse_ref = oracle_rows(q, k, v, rows, "bf16")
    out = as_f64(outs[0][0][rows], "bf16")
    rep = error_report(out, o_ref)
    log(f"  N=57344 {rep}")
    assert rep["rowwise_rel"] <= BF16_REL_TOL
    assert np.abs(outs[0][1][:, rows] - lse_ref).max() <= BF16_LSE_TOL


def test_workspace_errors_and_library_allocation():
    torch = pytest.importorskip("torch")
    n, h, d = 7 * 32, 1, 64
    q, k, v = gen_qkv(3, n, h, d, "bf16")
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
        o1 = empty_device((n, h, d), "bf16")
        o2 = empty_device((n, h, d), "bf16")
        small = torch.empty(16, dtype=torch.uint8, device="cuda")
        with pytest.raises(cqsa.CqsaError) as e:
            p.forward(qd, kd, vd, o1, workspace=small)
        assert e.value.status == -7
        st = p.forward(qd, kd, vd, o1, stats=True)  # library allocates its own workspace
        assert st["n_attn_launches"] == 1 and st["peak_device_bytes"] >= p.info["device_workspace_bytes"]
        ws = torch.empty(p.workspace_size(cqsa.CQSA_RES_DEVICE), dtype=torch.uint8, device="cuda")
        p.forward(qd, kd, vd, o2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
