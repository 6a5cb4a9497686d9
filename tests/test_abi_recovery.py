"""CPU tests of the out-of-memory recovery's host side: the fallback plan (one CQS
Divide level deeper, "The Recursive Benefit" section of the wispaper explainer; a
capacity failure made recoverable, abstract of arXiv 2604.20819), the budget taken from
free device memory, and the fault-injection hook's argument checks.  No call here
touches a GPU.
"""
import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from oracle.plan import make_plan

GiB = 1 << 30


def _same_schedule(plan, n, levels, pad):
    ref = make_plan(n, levels, pad=pad)
    assert plan.schedule().tobytes() == ref.serialize().tobytes()
    assert plan.coverage().tobytes() == ref.coverage().tobytes()


@pytest.mark.parametrize("n,levels,h,budget,want_levels", [
    # the 16 GiB workload (l=4) re-planned under 3 GiB: (4,4), 169 units, padded
    (212992, [4], 16, 3 * GiB, [4, 4]),
    # the 2 GiB two-level workload re-planned under 1 GiB: (3,3,3), 343 units, padded
    (12845056, [3, 3], 1, 1 * GiB, [3, 3, 3]),
    # an undivided plan divides with l = 3
    (3584, [1], 1, 64 << 20, [3]),
    # a budget the first deeper level cannot meet: divided again
    (57344, [3], 8, 40 << 20, [3, 3, 3]),
])
def test_fallback_goes_one_level_deeper(n, levels, h, budget, want_levels):
    with cqsa.Plan(n, h, 128, cqsa.CQSA_BF16, levels) as p:
        with p.fallback(budget) as f:
            info = f.info
            assert info["l"] == want_levels
            assert info["budget_bytes"] == budget
            assert info["stream_workspace_bytes"] <= budget
            c = int(np.prod([l * (l - 1) + 1 for l in want_levels]))
            assert info["padded_tokens"] == -(-n // c) * c
            if n <= 100000:  # the oracle planner walks small plans quickly
                _same_schedule(f, n, want_levels, pad=n % c != 0)


def test_fallback_keeps_causality_and_dtype():
    with cqsa.Plan(4096 * 7, 2, 64, cqsa.CQSA_F32, [3], flags=cqsa.CQSA_FLAG_CAUSAL) as p:
        with p.fallback(1 * GiB) as f:
            assert f.info["l"] == [3, 3]
            assert f.info["dtype"] == cqsa.CQSA_F32 and f.info["head_dim"] == 64
            assert f.info["useful_flop"] == p.info["useful_flop"]  # causal: 2 N (N+1) d H
            ref = make_plan(4096 * 7, [3, 3], pad=True, causal=True)
            assert f.schedule().tobytes() == ref.serialize().tobytes()


def test_fallback_errors():
    with cqsa.Plan(49, 1, 64, cqsa.CQSA_BF16, [3, 3]) as p:
        # 343 units would exceed 49 tokens
        with pytest.raises(cqsa.CqsaError) as e:
            p.fallback(1 * GiB)
        assert e.value.status == -3
    with cqsa.Plan(57344, 8, 128, cqsa.CQSA_BF16, [3]) as p:
        with pytest.raises(cqsa.CqsaError) as e:
            p.fallback(0)
        assert e.value.status == -1
        # a budget no depth can meet
        with pytest.raises(cqsa.CqsaError) as e:
            p.fallback(4096)
        assert e.value.status in (-3, -4)
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.cqsa_plan_fallback(None, GiB)
    assert e.value.status == -1


def test_free_budget_needs_a_device():
    # without a GPU the free memory cannot be read: EHIP, and no plan
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.Plan(57344, 8, 128, cqsa.CQSA_BF16, [3], budget_bytes=1 << 28, flags=cqsa.CQSA_FLAG_FREE_BUDGET)
    assert e.value.status == -5
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.Plan(57344, 8, 128, cqsa.CQSA_BF16, [3], budget_bytes=-1, flags=cqsa.CQSA_FLAG_FREE_BUDGET)
    assert e.value.status == -1


def test_fault_injection_arguments():
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.cqsa_debug_fail_allocations(-1)
    assert e.value.status == -1
    cqsa.cqsa_debug_fail_allocations(0)


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                    reason="passes placeholder device pointers; the budget test must reject the call before any "
                           "HIP call, which only a host without a GPU shows safely")
def test_device_paths_count_descriptor_tables_against_the_budget():
    """A budget that holds a device-resident call's workspace exactly, but not the plan's
    descriptor tables beside it, is rejected with EBUDGET before any HIP call, by the
    forward and the backward alike (the tables are uploaded to the device with the
    workspace, so both count against the budget the plan was made for)."""
    placeholder = 1 << 20  # 16-byte aligned, never dereferenced: the call ends at the budget test
    with cqsa.Plan(57344, 8, 128, cqsa.CQSA_BF16, [3]) as free:
        fwd_ws = free.workspace_size(cqsa.CQSA_RES_DEVICE)
        bwd_ws = free.backward_workspace_size(cqsa.CQSA_RES_DEVICE)
    for budget, call in ((fwd_ws, "forward"), (bwd_ws, "backward")):
        with cqsa.Plan(57344, 8, 128, cqsa.CQSA_BF16, [3], budget_bytes=budget) as p:
            with pytest.raises(cqsa.CqsaError) as exc:
                if call == "forward":
                    p.forward(placeholder, placeholder, placeholder, placeholder, placeholder)
                else:
                    p.backward(*([placeholder] * 9))  # q, k, v, o, lse, dO, dQ, dK, dV
            assert exc.value.status == cqsa.CQSA_EBUDGET, (call, exc.value)
            assert "descriptor bytes" in str(exc.value), (call, str(exc.value))
