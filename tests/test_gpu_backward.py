"""GPU parity of the CQS backward pass against the fp64 oracle (needs an MI355X).

Inputs: seeded Q, K, V, dO; O and LSE either from the fp64 oracle (rounded to the
input dtype / float32) or from this library's own forward.  Gradients are compared
with the dense fp64 definition (oracle.backward) element by element on small plans
(ragged units, several tiles, one to three levels, empty (task, unit) pairs, padded
N), and on the full-size bench workload via sampled dQ rows and the identities
sum_j dK_j = 0, sum_j dV_j = sum_i dO_i.  Tolerances as for the forward output:
float32 1e-5 max abs, bfloat16 2e-2 max row-wise relative.
"""
import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import gen_qkv, gen_tensor, round_to_bf16_bits, sample_rows
from oracle.attention import attention_fp64, to_f64
from oracle.backward import attention_backward_fp64, attention_backward_given_fp64, dq_rows_fp64
from oracle.tolerance import BF16_REL_TOL, F32_ABS_TOL, grad_rel_err, max_abs_err

from gpu_util import DT, as_f64, empty_device, log, to_device, to_numpy

pytestmark = pytest.mark.gpu

CASES = [  # levels, N, heads, head_dim, dtype, pad
    ([3], 7 * 40, 2, 128, "bf16", False),
    ([3], 7 * 200, 1, 64, "bf16", False),
    ([4], 13 * 130, 2, 128, "bf16", False),
    ([2, 2], 9 * 24, 2, 64, "bf16", False),     # a (task, unit) with no admitted partner
    ([1], 300, 2, 128, "bf16", False),
    ([3, 2], 21 * 20 + 3, 1, 128, "bf16", True),  # padded N
    ([3], 7 * 64, 1, 64, "f32", False),
    ([4], 13 * 30, 2, 128, "f32", False),
    ([2, 3], 21 * 8, 1, 64, "f32", False),
    ([3], 7 * 33 - 5, 1, 64, "f32", True),
    ([2, 3], 21 * 9 + 2, 1, 128, "f32", True),  # fp32 d=128 dQ (once wrong while its kernel spilled)
    ([8], 57 * 24, 1, 128, "bf16", False),      # 57 tasks of 8 units
    ([10], 91 * 12 + 5, 1, 64, "f32", True),    # 91 tasks of 10 units, padded N
]


def _ids(c):
    return f"l{'x'.join(map(str, c[0]))}-n{c[1]}-h{c[2]}-d{c[3]}-{c[4]}{'-pad' if c[5] else ''}"


def _round(x64, dtype):
    x32 = np.asarray(x64, dtype=np.float32)
    return round_to_bf16_bits(x32) if dtype == "bf16" else x32


def _check(got, ref, dtype, what):
    if dtype == "f32":
        err = max_abs_err(got, ref)
        tol = F32_ABS_TOL
    else:
        err = grad_rel_err(got, ref)
        tol = BF16_REL_TOL
    log(f"  {what}: {err:.3e}")
    assert err <= tol, (what, err)


def _run_backward(p, dev, dtype, n, h, d, workspace=None):
    torch = pytest.importorskip("torch")
    dq, dk, dv = (empty_device((n, h, d), dtype) for _ in range(3))
    p.backward(*dev, dq, dk, dv, workspace=workspace)
    torch.cuda.synchronize()
    return [as_f64(to_numpy(t, dtype), dtype) for t in (dq, dk, dv)]


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_backward_matches_dense_gradients(case):
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype, pad = case
    log(f"backward {_ids(case)}")
    q, k, v = gen_qkv(101 + n, n, h, d, dtype)
    do = gen_tensor(101 + n, 3, n, h, d, dtype)
    o_ref, lse_ref = attention_fp64(q, k, v, dtype=dtype)
    # the operation's inputs: the forward's O and LSE in their storage precision
    o_in, lse_in = _round(o_ref, dtype), lse_ref.astype(np.float32)
    grads_ref = attention_backward_given_fp64(q, k, v, o_in, lse_in, do, dtype=dtype)
    flags = cqsa.CQSA_FLAG_PAD if pad else 0
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=flags) as p:
        dev = [to_device(x, dtype) for x in (q, k, v, o_in)]
        dev.append(torch.from_numpy(lse_in).cuda())
        dev.append(to_device(do, dtype))
        got = _run_backward(p, dev, dtype, n, h, d)
    for name, g, r in zip(("dQ", "dK", "dV"), got, grads_ref):
        _check(g, r, dtype, name)


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[6]], ids=_ids)
def test_forward_then_backward_end_to_end(case):
    """O and LSE from this library's forward feed its backward; compared with the oracle."""
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype, pad = case
    log(f"forward+backward {_ids(case)}")
    q, k, v = gen_qkv(7 + n, n, h, d, dtype)
    do = gen_tensor(7 + n, 3, n, h, d, dtype)
    grads_ref = attention_backward_fp64(q, k, v, do, dtype=dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels) as p:
        qd, kd, vd, dod = (to_device(x, dtype) for x in (q, k, v, do))
        o = empty_device((n, h, d), dtype)
        lse = torch.empty((h, n), device="cuda")
        p.forward(qd, kd, vd, o, lse)
        outs = []
        for _ in range(2):
            outs.append(_run_backward(p, [qd, kd, vd, o, lse, dod], dtype, n, h, d))
    for a, b in zip(*outs):
        assert np.array_equal(a, b), "deterministic"
    for name, g, r in zip(("dQ", "dK", "dV"), outs[0], grads_ref):
        _check(g, r, dtype, name)


def test_backward_full_size_sampled_rows_and_identities():
    """N=57344, H=8, d=128, bf16, l=3: dQ on sampled rows against the oracle, and the
    identities sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i over all rows."""
    torch = pytest.importorskip("torch")
    n, h, d = 57344, 8, 128
    log("backward full size")
    q, k, v = gen_qkv(0, n, h, d, "bf16")
    do = gen_tensor(0, 3, n, h, d, "bf16")
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
        o = empty_device((n, h, d), "bf16")
        lse = torch.empty((h, n), device="cuda")
        p.forward(qd, kd, vd, o, lse)
        ws = torch.empty(p.backward_workspace_size(), dtype=torch.uint8, device="cuda")
        dq, dk, dv = _run_backward(p, [qd, kd, vd, o, lse, dod], "bf16", n, h, d, workspace=ws)
    rows = sample_rows(n, 256, 2, unit_tokens=8192)
    log(f"  oracle dQ on {rows.size} rows")
    dq_ref = dq_rows_fp64(q, k, v, do, rows, dtype="bf16")
    _check(dq[rows], dq_ref, "bf16", "dQ sampled")
    # identities over all rows, per head: tolerance from the bf16 rounding of every term
    do64 = to_f64(do, "bf16")
    sv, sdo = dv.sum(axis=0), do64.sum(axis=0)
    err_v = np.abs(sv - sdo).max() / np.abs(sdo).max()
    err_k = np.abs(dk.sum(axis=0)).max() / np.abs(dk).sum(axis=0).max()
    log(f"  sum dV vs sum dO rel {err_v:.3e}; |sum dK| / sum |dK| {err_k:.3e}")
    assert err_v <= BF16_REL_TOL and err_k <= BF16_REL_TOL


def test_backward_errors():
    torch = pytest.importorskip("torch")
    n, h, d = 7 * 32, 1, 64
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        t = [torch.zeros((n, h, d), dtype=torch.bfloat16, device="cuda") for _ in range(8)]
        lse = torch.zeros((h, n), device="cuda")
        small = torch.empty(16, dtype=torch.uint8, device="cuda")
        with pytest.raises(cqsa.CqsaError) as e:
            p.backward(t[0], t[1], t[2], t[3], lse, t[4], t[5], t[6], t[7], workspace=small)
        assert e.value.status == -7
        with pytest.raises(cqsa.CqsaError) as e:
            p.backward(t[0], t[1], t[2], t[3], lse, t[4], t[5], t[6], t[7], residency=7)
        assert e.value.status == -1


STREAM_CASES = [  # levels, N, heads, head_dim, dtype, flags
    ([3], 7 * 300, 2, 128, "bf16", 0),
    ([3], 7 * 300, 2, 128, "bf16", cqsa.CQSA_FLAG_HOST_ACC),
    ([4], 13 * 100 + 9, 1, 64, "bf16", cqsa.CQSA_FLAG_PAD),
    ([2, 2], 9 * 40, 2, 128, "bf16", cqsa.CQSA_FLAG_HOST_ACC),
    ([3, 2], 21 * 16, 1, 64, "bf16", 0),
    ([3], 7 * 64, 1, 64, "f32", cqsa.CQSA_FLAG_HOST_ACC),
    ([2, 3], 21 * 9 + 2, 1, 128, "f32", cqsa.CQSA_FLAG_PAD),
    ([3], 7 * 300, 2, 128, "bf16", cqsa.CQSA_FLAG_KV_SINGLE),  # one task staging set
    ([4], 13 * 64, 2, 64, "bf16", cqsa.CQSA_FLAG_KV_SINGLE | cqsa.CQSA_FLAG_HOST_ACC),
    ([3], 7 * 300, 2, 128, "bf16", cqsa.CQSA_FLAG_CAUSAL),
    ([2, 2], 9 * 40 + 5, 1, 64, "bf16", cqsa.CQSA_FLAG_CAUSAL | cqsa.CQSA_FLAG_PAD | cqsa.CQSA_FLAG_HOST_ACC),
    ([3], 7 * 33, 1, 128, "f32", cqsa.CQSA_FLAG_CAUSAL | cqsa.CQSA_FLAG_KV_SINGLE),
]


@pytest.mark.parametrize("case", STREAM_CASES,
                         ids=lambda c: f"l{'x'.join(map(str, c[0]))}-n{c[1]}-h{c[2]}-d{c[3]}-{c[4]}-f{c[5]}")
def test_streamed_backward_equals_device_backward(case):
    """Host-pinned backward (tasks staged through the device under the plan's layout) gives
    the device-resident backward's gradients bit for bit."""
    from gpu_util import pinned
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype, flags = case
    log(f"streamed backward {case}")
    q, k, v = gen_qkv(151 + n, n, h, d, dtype)
    do = gen_tensor(151 + n, 3, n, h, d, dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=flags) as p:
        qd, kd, vd, dod = (to_device(x, dtype) for x in (q, k, v, do))
        o = empty_device((n, h, d), dtype)
        lse = torch.empty((h, n), device="cuda")
        p.forward(qd, kd, vd, o, lse)
        want = _run_backward(p, [qd, kd, vd, o, lse, dod], dtype, n, h, d)
        hosts = []
        for x in (q, k, v, to_numpy(o, dtype), do):
            t, a = pinned((n, h, d), dtype)
            a[...] = x
            hosts.append(t)
        lse_h = lse.cpu().pin_memory()
        outs = [pinned((n, h, d), dtype) for _ in range(3)]
        st = p.backward(*hosts[:4], lse_h, hosts[4], *(t for t, _ in outs), residency=cqsa.CQSA_RES_HOST_PINNED,
                        stats=True)
        assert st["peak_device_bytes"] >= p.backward_workspace_size(cqsa.CQSA_RES_HOST_PINNED)
        got = [as_f64(a, dtype) for _, a in outs]
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        assert np.array_equal(g, w), f"{name} differs from the device path"


def test_streamed_backward_respects_budget():
    torch = pytest.importorskip("torch")
    n, h, d = 13 * 512, 4, 128
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [4]) as probe:
        need_dev = probe.backward_workspace_size(cqsa.CQSA_RES_HOST_PINNED)
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [4], budget_bytes=need_dev // 2) as p:
        ws = p.backward_workspace_size(cqsa.CQSA_RES_HOST_PINNED)
        assert ws <= need_dev // 2  # the accumulators moved to pinned host memory


def _smallest_budget_with_backward(n, h, d, dtype, levels, flags):
    """The smallest budget at which the plan builds and has a streamed backward layout
    (bisection over plan creation; host-side only)."""
    def ok(b):
        try:
            with cqsa.Plan(n, h, d, DT[dtype], levels, budget_bytes=b, flags=flags) as p:
                return p.info["bwd_stream_mode"] != 0
        except cqsa.CqsaError:
            return False
    lo, hi = 1, 1 << 20
    while not ok(hi):
        lo, hi = hi, hi * 2
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (lo, mid) if ok(mid) else (mid, hi)
    return hi


HOST_STATS_CASES = [  # levels, N, heads, head_dim, dtype, flags
    ([3], 7 * 2048, 4, 128, "bf16", 0),
    ([4], 13 * 100 + 9, 2, 64, "bf16", cqsa.CQSA_FLAG_PAD),
    ([2, 2], 9 * 40, 2, 128, "bf16", cqsa.CQSA_FLAG_CAUSAL),
    ([3], 7 * 64, 1, 64, "f32", cqsa.CQSA_FLAG_KV_SINGLE),
]


@pytest.mark.parametrize("case", HOST_STATS_CASES,
                         ids=lambda c: f"l{'x'.join(map(str, c[0]))}-n{c[1]}-h{c[2]}-d{c[3]}-{c[4]}-f{c[5]}")
def test_streamed_backward_with_host_statistics_equals_device_backward(case):
    """Under the smallest budget that admits a streamed backward, L and Delta of every row
    stay in pinned host memory (no layout with them on the device fits) and each task's
    rows are gathered with its staging; the gradients equal the device-resident
    backward's bit for bit, and the device memory stays within the budget."""
    from gpu_util import init_device_runtime, pinned
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype, flags = case
    budget = _smallest_budget_with_backward(n, h, d, dtype, levels, flags)
    log(f"streamed backward with host statistics {case}: budget {budget}")
    init_device_runtime()
    q, k, v = gen_qkv(171 + n, n, h, d, dtype)
    do = gen_tensor(171 + n, 3, n, h, d, dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=flags) as p:
        qd, kd, vd, dod = (to_device(x, dtype) for x in (q, k, v, do))
        o = empty_device((n, h, d), dtype)
        lse = torch.empty((h, n), device="cuda")
        p.forward(qd, kd, vd, o, lse)
        want = _run_backward(p, [qd, kd, vd, o, lse, dod], dtype, n, h, d)
    hosts = []
    for x in (q, k, v, to_numpy(o, dtype), do):
        t, a = pinned((n, h, d), dtype)
        a[...] = x
        hosts.append(t)
    lse_h = lse.cpu().pin_memory()
    outs = [pinned((n, h, d), dtype) for _ in range(3)]
    with cqsa.Plan(n, h, d, DT[dtype], levels, budget_bytes=budget, flags=flags) as p:
        info = p.info
        assert info["bwd_host_stats"] == 1, info
        assert 0 < info["bwd_stream_workspace_bytes"] <= budget
        st = p.backward(*hosts[:4], lse_h, hosts[4], *(t for t, _ in outs), residency=cqsa.CQSA_RES_HOST_PINNED,
                        stats=True)
        log(f"  modelled {st['peak_device_bytes']} observed {st['observed_peak_bytes']} of {budget}")
        assert st["peak_device_bytes"] <= budget
        got = [as_f64(a, dtype) for _, a in outs]
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        assert np.array_equal(g, w), f"{name} differs from the device path"
