"""CPU tests of the C ABI: exported symbols, the host planner against the oracle
planner (bit-exact schedule and coverage), the footprint model and error paths.
No call here touches a GPU.
"""
import os
import re

import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from oracle.plan import difference_set, make_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GiB = 1 << 30

CONFIGS = {  # name: (N, H, d, dtype, levels, budget)
    "n3584_f32_l3": (3584, 1, 64, cqsa.CQSA_F32, [3], 0),
    "n57344_h8_l3": (57344, 8, 128, cqsa.CQSA_BF16, [3], 0),
    "n212992_h16_l4_16GiB": (212992, 16, 128, cqsa.CQSA_BF16, [4], 16 * GiB),
    "n1376256_h8_l5_8GiB": (1376256, 8, 128, cqsa.CQSA_BF16, [5], 8 * GiB),
    "n12845056_h1_l3x3_2GiB": (12845056, 1, 128, cqsa.CQSA_BF16, [3, 3], 2 * GiB),
}


def _header_symbols():
    text = open(os.path.join(ROOT, "include", "cqsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cqsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = _header_symbols()
    assert len(names) == 19
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(cqsa.EXPORTS)


def test_difference_sets_match_oracle(lib):
    for l in range(1, 11):
        if l == 7:
            with pytest.raises(cqsa.CqsaError) as e:
                cqsa.cqsa_difference_set(7)
            assert e.value.status == -2
            continue
        assert cqsa.cqsa_difference_set(l) == difference_set(l)
    for bad in (0, 11, -3):
        with pytest.raises(cqsa.CqsaError) as e:
            cqsa.cqsa_difference_set(bad)
        assert e.value.status == -1


SMALL_PLANS = [([1], 1), ([1], 37), ([2], 3), ([3], 7), ([3], 21), ([4], 13), ([5], 42), ([6], 31),
               ([2, 2], 9), ([3, 2], 21), ([2, 3], 42), ([3, 3], 49), ([4, 2], 39), ([2, 2, 2], 27),
               ([8], 57), ([8], 114), ([9], 73), ([10], 91), ([6, 2], 93),
               ([3, 3, 3, 3], 2401)]  # 2,401 tasks of 81 units: built on several host threads


@pytest.mark.parametrize("levels,n", SMALL_PLANS + [(v[4], v[0]) for v in CONFIGS.values()])
def test_schedule_and_coverage_bit_exact(levels, n):
    ref = make_plan(n, levels)
    with cqsa.Plan(n, 2, 64, cqsa.CQSA_BF16, levels) as p:
        sched = p.schedule()
        want = ref.serialize()
        assert sched.dtype == np.int64 and sched.shape == want.shape
        assert sched.tobytes() == want.tobytes()
        cov = p.coverage()
        assert cov.tobytes() == ref.coverage().tobytes()
        assert (cov >= 0).all()
        info = p.info
        assert info["levels"] == len(levels) and info["l"] == levels
        assert info["c"] == ref.cs
        assert info["n_tasks"] == len(ref.tasks)
        assert info["unit_tokens"] == ref.unit_tokens and info["visits"] == int(np.prod(levels))


@pytest.mark.parametrize("name", list(CONFIGS))
def test_footprint_fits_budget(name):
    n, h, d, dt, levels, budget = CONFIGS[name]
    with cqsa.Plan(n, h, d, dt, levels, budget_bytes=budget) as p:
        info = p.info
        e = 2 if dt == cqsa.CQSA_BF16 else 4
        if budget:
            assert info["stream_workspace_bytes"] <= budget
        assert p.workspace_size(cqsa.CQSA_RES_HOST_PINNED) == info["stream_workspace_bytes"]
        # device-resident slots: V partial triples per (row, head)
        assert info["device_workspace_bytes"] >= info["visits"] * n * h * (d + 2) * 4
        assert info["useful_flop"] == pytest.approx(4.0 * n * n * d * h)
        # the K/V staging alone: kv_buffers x (K + V) x task tokens
        assert info["stream_workspace_bytes"] >= info["kv_buffers"] * 2 * info["task_tokens"] * h * d * e
    modes = {"n3584_f32_l3": 1, "n57344_h8_l3": 1, "n212992_h16_l4_16GiB": 1, "n1376256_h8_l5_8GiB": 2, "n12845056_h1_l3x3_2GiB": 4}
    assert info["stream_mode"] == modes[name]


def test_n1376256_device_accumulator_does_not_fit_8gib():
    # a device accumulator for all N rows (5.33 GiB) + the K/V double buffer (2.5 GiB) + the
    # two-slot query ring exceeds 8 GiB, so the accumulator moves to pinned host memory
    n, h, d = 1376256, 8, 128
    acc = n * h * (d + 2) * 4
    kv2 = 2 * 2 * 5 * 65536 * h * d * 2
    ring = 2 * 65536 * h * (d * 2 + (d + 2) * 4 + d * 2 + 4)
    assert acc + kv2 + ring > 8 * GiB
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [5]) as p:
        assert p.info["stream_mode"] == 1 and p.info["stream_workspace_bytes"] > 8 * GiB
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [5], budget_bytes=8 * GiB) as p:
        assert p.info["host_acc_bytes"] == n * h * (d + 2) * 4


def test_auto_levels_follow_the_budget():
    with cqsa.Plan(12845056, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=2 * GiB) as p:
        assert p.info["levels"] == 2 and p.info["l"] == [3, 3]
    with cqsa.Plan(12845056, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=16 * GiB) as p:
        assert p.info["levels"] == 1 and p.info["l"] == [3]
    # the undivided plan when it fits (nothing to recover from)
    with cqsa.Plan(12845056, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=64 * GiB) as p:
        assert p.info["levels"] == 1 and p.info["l"] == [1] and p.info["stream_workspace_bytes"] <= 64 * GiB
    with pytest.raises(cqsa.CqsaError) as e:  # a third level would not divide
        cqsa.Plan(12845056, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=256 << 20)
    assert e.value.status == -4


def test_forced_modes():
    n = 13 * 64
    for flags, mode in ((0, 1), (cqsa.CQSA_FLAG_HOST_ACC, 2), (cqsa.CQSA_FLAG_KV_SINGLE, 3),
                        (cqsa.CQSA_FLAG_HOST_ACC | cqsa.CQSA_FLAG_KV_SINGLE, 4)):
        with cqsa.Plan(n, 2, 64, cqsa.CQSA_BF16, [4], flags=flags) as p:
            assert p.info["stream_mode"] == mode
            assert p.info["kv_buffers"] == (1 if mode in (3, 4) else 2)
            assert (p.info["host_acc_bytes"] > 0) == (mode in (2, 4))


def test_budget_selects_modes_in_order():
    n, h, d = 13 * 256, 2, 64
    sizes = {}
    for flags in (0, 1, 2, 3):
        with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [4], flags=flags) as p:
            sizes[p.info["stream_mode"]] = p.info["stream_workspace_bytes"]
    for mode, size in sizes.items():
        with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [4], budget_bytes=size + 65536) as p:
            chosen = p.info["stream_mode"]
            assert sizes[chosen] <= size + 65536
            assert chosen <= mode or sizes[chosen] <= sizes[mode]
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [4], budget_bytes=min(sizes.values()) // 2)
    assert e.value.status == -4


@pytest.mark.parametrize("args,status", [
    ((100, 1, 64, cqsa.CQSA_BF16, [3]), -3),        # 100 is not a multiple of 7
    ((43, 1, 64, cqsa.CQSA_BF16, [7]), -2),         # no difference set
    ((49, 1, 96, cqsa.CQSA_BF16, [3]), -1),         # unsupported head_dim
    ((49, 0, 64, cqsa.CQSA_BF16, [3]), -1),         # no heads
    ((0, 1, 64, cqsa.CQSA_BF16, [3]), -1),          # no tokens
    ((49, 1, 64, 7, [3]), -1),                      # unknown dtype
    ((49, 1, 64, cqsa.CQSA_BF16, [11]), -1),        # l out of range
    ((7 ** 4, 1, 64, cqsa.CQSA_BF16, [3] * 13), -1),  # more than 12 levels
])
def test_plan_errors(args, status):
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.cqsa_plan_create(*args)
    assert e.value.status == status
    assert cqsa.cqsa_last_error()


def test_bad_flags_and_null_arguments(lib):
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.cqsa_plan_create(49, 1, 64, cqsa.CQSA_BF16, [3], flags=0x40)
    assert e.value.status == -1
    import ctypes
    assert lib.cqsa_plan_create(49, 1, 64, 0, None, 1, 0, 0, ctypes.byref(ctypes.c_void_p())) == -1
    assert lib.cqsa_plan_info_get(None, None) == -1
    assert lib.cqsa_forward(None, None, None, None, None, None, 0, None, 0, None, None) == -1
    with cqsa.Plan(49, 1, 64, cqsa.CQSA_BF16, [3]) as p:
        needed = ctypes.c_int64()
        small = np.zeros(3, np.int64)
        assert lib.cqsa_plan_schedule(p.handle, small.ctypes.data, 3, ctypes.byref(needed)) == -7
        assert needed.value > 3
        assert lib.cqsa_forward(p.handle, 1, 1, 1, 1, None, 5, None, 0, None, None) == -1
    lib.cqsa_plan_destroy(None)


def test_misaligned_device_pointers_are_rejected(lib):
    """Device tensors and workspaces must start on 16 bytes (lse on 4); the check runs
    before any HIP call, so fake addresses are never dereferenced."""
    import ctypes
    good, bad = 1 << 20, (1 << 20) + 2
    with cqsa.Plan(49, 1, 64, cqsa.CQSA_BF16, [3]) as p:
        h = p.handle
        assert lib.cqsa_partials(h, good, good, bad, good, good, None) == -1
        assert "16-byte" in cqsa.cqsa_last_error()
        assert lib.cqsa_merge(h, good, good, good, good + 2, None) == -1
        assert lib.cqsa_forward(h, bad, good, good, good, None, cqsa.CQSA_RES_DEVICE, None, 0, None, None) == -1
        assert lib.cqsa_forward(h, good, good, good, good, None, cqsa.CQSA_RES_HOST_PINNED, bad, 64, None, None) == -1
        assert lib.cqsa_backward(h, good, good, good, good, good, good, good, bad, good, cqsa.CQSA_RES_DEVICE, None, 0,
                                 None, None) == -1
        assert "16-byte" in cqsa.cqsa_last_error()


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert cqsa.cqsa_status_string(s)
    assert "unknown" in cqsa.cqsa_status_string(42)


PADDED_PLANS = [([3], 50), ([3], 8), ([3], 7 * 192 + 5), ([4], 100), ([2, 2], 20), ([3, 2], 100), ([2], 4),
                ([2, 2, 2], 28), ([5], 21 * 64 - 1), ([3, 3], 12845055)]


@pytest.mark.parametrize("levels,n", PADDED_PLANS)
def test_padded_schedule_bit_exact(levels, n):
    # reading R12 of the oracle planner: N is rounded up to the unit grid, segments stop at N
    ref = make_plan(n, levels, pad=True)
    with cqsa.Plan(n, 2, 64, cqsa.CQSA_BF16, levels, flags=cqsa.CQSA_FLAG_PAD) as p:
        assert p.schedule().tobytes() == ref.serialize().tobytes()
        assert p.coverage().tobytes() == ref.coverage().tobytes()
        info = p.info
        assert info["n_tokens"] == n and info["padded_tokens"] == ref.n_pad
        assert info["unit_tokens"] == ref.unit_tokens and info["unit_tokens"] * info["n_units"] == ref.n_pad
        assert info["useful_flop"] == pytest.approx(4.0 * n * n * 64 * 2)
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.Plan(n, 2, 64, cqsa.CQSA_BF16, levels)
    assert e.value.status == -3


def test_pad_flag_is_a_no_op_on_the_grid():
    with cqsa.Plan(49, 1, 64, cqsa.CQSA_BF16, [3]) as a, \
            cqsa.Plan(49, 1, 64, cqsa.CQSA_BF16, [3], flags=cqsa.CQSA_FLAG_PAD) as b:
        assert a.schedule().tobytes() == b.schedule().tobytes()
        assert a.info["padded_tokens"] == b.info["padded_tokens"] == 49
    with pytest.raises(cqsa.CqsaError) as e:  # fewer tokens than units: no division at all
        cqsa.Plan(5, 1, 64, cqsa.CQSA_BF16, [3], flags=cqsa.CQSA_FLAG_PAD)
    assert e.value.status == -3


def test_auto_levels_with_padding():
    # an N off every grid still recovers once padding is allowed
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.Plan(12845057, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=2 * GiB)
    assert e.value.status == -3
    with cqsa.Plan(12845057, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=2 * GiB,
                   flags=cqsa.CQSA_FLAG_PAD) as p:
        assert p.info["l"] == [3, 3] and p.info["stream_workspace_bytes"] <= 2 * GiB
        assert p.info["padded_tokens"] == 12845057 + 48


def test_backward_workspace_size_and_argument_errors(lib):
    n, h, d = 7 * 100, 3, 128
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        np_ = -(-n // 64) * 64
        al = lambda x: -(-x // 256) * 256  # noqa: E731
        want = al(h * n * 4) + 3 * al(h * d * np_ * 2) + 3 * al(3 * n * h * d * 4)
        assert p.backward_workspace_size() == want
        # streamed: L, Delta; Q, K, V, dO staging of a task; three transposed copies; the
        # task's L and Delta rows; a two-slot ring of terms and output blocks; device accumulators
        t = 3 * 100
        tnp = -(-t // 64) * 64
        ring = 2 * 3 * (al(100 * h * d * 4) + al(100 * h * d * 2))
        want_s = 2 * al(h * n * 4) + 2 * (4 * al(t * h * d * 2) + 3 * al(h * d * tnp * 2) + 2 * al(h * t * 4)) + ring \
            + 3 * al(n * h * d * 4)
        assert p.backward_workspace_size(cqsa.CQSA_RES_HOST_PINNED) == want_s
    with cqsa.Plan(n, h, d, cqsa.CQSA_F32, [3]) as p:
        assert p.backward_workspace_size() == al(h * n * 4) + 3 * al(3 * n * h * d * 4)
    assert lib.cqsa_backward(None, None, None, None, None, None, None, None, None, None, 0, None, 0, None,
                             None) == -1


RATES = {"attn_tflops": 800.0, "merge_gbs": 5000.0, "h2d_gbs": 50.0, "d2h_gbs": 40.0}


@pytest.mark.parametrize("n,h,d,dt,levels,budget,flags", [
    (3584, 1, 64, cqsa.CQSA_F32, [3], 0, 0),
    (212992, 16, 128, cqsa.CQSA_BF16, [4], 16 * GiB, 0),
    (1376256, 8, 128, cqsa.CQSA_BF16, [5], 8 * GiB, 0),
    (12845056, 1, 128, cqsa.CQSA_BF16, [3, 3], 2 * GiB, 0),
    (7 * 192 + 5, 2, 128, cqsa.CQSA_BF16, [3], 0, cqsa.CQSA_FLAG_PAD | cqsa.CQSA_FLAG_HOST_ACC),
    (21 * 20 + 3, 1, 64, cqsa.CQSA_BF16, [3, 2], 0, cqsa.CQSA_FLAG_PAD | cqsa.CQSA_FLAG_KV_SINGLE),
    (500, 2, 64, cqsa.CQSA_BF16, [1], 0, cqsa.CQSA_FLAG_HOST_ACC),
])
def test_estimate_matches_built_plan_and_walked_traffic(n, h, d, dt, levels, budget, flags):
    from oracle.stream_bytes import stream_traffic
    est = cqsa.cqsa_plan_estimate(n, h, d, dt, levels, budget_bytes=budget, flags=flags, rates=RATES)
    with cqsa.Plan(n, h, d, dt, levels, budget_bytes=budget, flags=flags) as p:
        info = p.info
    for key in ("levels", "c", "l", "n_tasks", "unit_tokens", "visits", "task_tokens", "stream_mode", "kv_buffers",
                "stream_workspace_bytes", "padded_tokens"):
        assert est[key] == info[key], key
    assert est["materializable"] == 1
    e = 2 if dt == cqsa.CQSA_BF16 else 4
    padded = n % int(np.prod([l * (l - 1) + 1 for l in levels])) != 0
    ref = stream_traffic(make_plan(n, levels, pad=padded), h, d, e, host_acc=est["stream_mode"] in (2, 4),
                         kv_buffers=est["kv_buffers"])
    for key in ("bytes_d2h", "merge_bytes"):
        assert est[key] == ref[key], key
    assert est["bytes_h2d"] + est["bytes_d2d"] == ref["bytes_h2d"] + ref["bytes_d2d"]
    if not padded:  # with padding a shared chunk may hold padding rows: the estimate bounds it
        assert (est["bytes_h2d"], est["bytes_d2d"]) == (ref["bytes_h2d"], ref["bytes_d2d"])
    else:
        assert est["bytes_h2d"] <= ref["bytes_h2d"]
    if est["kv_buffers"] == 2 and max(levels) > 1:
        assert est["bytes_d2d"] > 0
    assert est["useful_flop"] == pytest.approx(4.0 * n * n * d * h)
    assert est["t_attn_s"] == pytest.approx(est["useful_flop"] / 800e12)
    assert est["t_est_s"] >= max(est["t_h2d_s"], est["t_d2h_s"], est["t_attn_s"])


def test_estimate_of_a_billion_tokens_needs_no_plan():
    # 2^30 tokens, one head, d=128, bf16, l=3: nine levels would be 7^9 tasks; padding
    # makes every depth divide, and the budget decides the depth
    n = 1 << 30
    est = cqsa.cqsa_plan_estimate(n, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=16 * GiB,
                                  flags=cqsa.CQSA_FLAG_PAD, rates=RATES)
    assert est["stream_workspace_bytes"] <= 16 * GiB and est["levels"] >= 2 and set(est["l"]) == {3}
    assert est["padded_tokens"] % est["n_tasks"] == 0 and est["padded_tokens"] - n < est["n_tasks"]
    assert est["bytes_h2d"] + est["bytes_d2d"] >= 3 * est["visits"] * n * 256
    nine = cqsa.cqsa_plan_estimate(n, 1, 128, cqsa.CQSA_BF16, [3] * 9, flags=cqsa.CQSA_FLAG_PAD, rates=RATES)
    assert nine["n_tasks"] == 7 ** 9 and nine["visits"] == 3 ** 9 and nine["materializable"] == 0
    assert nine["task_tokens"] == -(-n // 7 ** 9) * 3 ** 9
    with pytest.raises(cqsa.CqsaError) as e:  # the engine does not build such a plan
        cqsa.Plan(n, 1, 128, cqsa.CQSA_BF16, [3] * 9, flags=cqsa.CQSA_FLAG_PAD)
    assert e.value.status == -6
    with pytest.raises(cqsa.CqsaError) as e:
        cqsa.cqsa_plan_estimate(n, 1, 128, cqsa.CQSA_BF16, [3], rates={**RATES, "h2d_gbs": 0.0})
    assert e.value.status == -1


CAUSAL_PLANS = [([3], 21), ([3], 7 * 100), ([4], 13 * 3), ([2, 2], 18), ([3, 2], 42), ([1], 9), ([2, 3], 42),
                ([3], 50), ([5], 21 * 4 + 3), ([3, 3], 12845056)]


@pytest.mark.parametrize("levels,n", CAUSAL_PLANS)
def test_causal_schedule_and_coverage_bit_exact(levels, n):
    prod_c = int(np.prod([l * (l - 1) + 1 for l in levels]))
    pad = n % prod_c != 0
    ref = make_plan(n, levels, pad=pad, causal=True)
    flags = cqsa.CQSA_FLAG_CAUSAL | (cqsa.CQSA_FLAG_PAD if pad else 0)
    with cqsa.Plan(n, 2, 64, cqsa.CQSA_BF16, levels, flags=flags) as p:
        assert p.schedule().tobytes() == ref.serialize().tobytes()
        cov = p.coverage()
        assert cov.tobytes() == ref.coverage().tobytes()
        u = p.info["n_units"]
        lower = np.tril(np.ones((u, u), dtype=bool))
        assert (cov[lower] >= 0).all() and (cov[~lower] == -1).all()
        assert p.info["useful_flop"] == pytest.approx(2.0 * n * (n + 1) * 64 * 2)


def test_last_error_is_per_thread(lib):
    """Each thread reads back the message of its own last failure."""
    import threading
    results = {}

    def worker(tag, l):
        try:
            cqsa.cqsa_difference_set(l)
        except cqsa.CqsaError:
            pass
        results[tag] = cqsa.cqsa_last_error()

    threads = [threading.Thread(target=worker, args=(i, l)) for i, l in enumerate((7, 0, 7, 11))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert "l=7" in results[0] and results[2] == results[0]
    assert "1..10" in results[1] and results[3] == results[1]


def _create_or_none(n, h, d, levels, budget, n_levels=None):
    try:
        with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, levels, n_levels=n_levels, budget_bytes=budget,
                       flags=cqsa.CQSA_FLAG_PAD) as p:
            return p.info["levels"], p.info["stream_mode"], p.info["stream_workspace_bytes"]
    except cqsa.CqsaError as e:
        assert e.status in (-4, -6)  # over the budget, or too deep a plan to build
        return None if e.status == -4 else "unbuildable"


def _estimate_or_none(n, h, d, levels, budget, n_levels=None):
    try:
        e = cqsa.cqsa_plan_estimate(n, h, d, cqsa.CQSA_BF16, levels, n_levels=n_levels, budget_bytes=budget,
                                    flags=cqsa.CQSA_FLAG_PAD, rates=RATES)
        return e["levels"], e["stream_mode"], e["stream_workspace_bytes"]
    except cqsa.CqsaError as e:
        assert e.status == -4
        return None


def _built(made, field):
    """A field of a built plan's (levels, mode, workspace); 99 when there is none."""
    return made[field] if isinstance(made, tuple) else 99


def _first_budget(pred, lo=1, hi=64 * GiB):
    """Smallest budget in (lo, hi] for which pred holds (pred monotonic in the budget)."""
    assert pred(hi)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid
    return hi


@pytest.mark.parametrize("n,h,d,levels,n_levels", [
    (57344, 8, 128, [3], None), (212992, 16, 128, [4], None), (7 * 13 * 40 + 5, 2, 64, [3, 4], None),
    (1376256, 8, 128, [5], None), (7 * 7 * 64 * 4, 2, 64, [3], 0), (7 * 7 * 7 * 30, 1, 128, [3], 0)])
def test_estimate_and_plan_agree_at_budget_edges(n, h, d, levels, n_levels):
    """cqsa_plan_estimate applies cqsa_plan_create's budget test (workspace + descriptor
    tables), so at every budget where the plan's choice changes -- the smallest budget it
    fits, each staging mode's threshold, each depth of the automatic recursion -- both
    give the same depth, mode and workspace one byte below and at the edge."""
    edges = set()
    for mode in (1, 2, 3, 4):
        pred = lambda b, m=mode: _built(_create_or_none(n, h, d, levels, b, n_levels), 1) <= m  # noqa: E731
        if pred(64 * GiB):
            edges.add(_first_budget(pred))
    if n_levels == 0:
        for depth in (1, 2, 3):
            pred = lambda b, k=depth: _built(_create_or_none(n, h, d, levels, b, n_levels), 0) <= k  # noqa: E731
            if pred(64 * GiB):
                edges.add(_first_budget(pred))
    assert edges
    for b in sorted(edges):
        for budget in (b - 1, b):
            made = _create_or_none(n, h, d, levels, budget, n_levels)
            if made != "unbuildable":
                assert _estimate_or_none(n, h, d, levels, budget, n_levels) == made, budget


@pytest.mark.parametrize("n,h,d,dt,levels,flags", [
    (7 * 2048, 4, 128, cqsa.CQSA_BF16, [3], 0),
    (13 * 100 + 9, 2, 64, cqsa.CQSA_BF16, [4], cqsa.CQSA_FLAG_PAD),
    (9 * 40, 2, 128, cqsa.CQSA_BF16, [2, 2], cqsa.CQSA_FLAG_CAUSAL),
    (7 * 64, 1, 64, cqsa.CQSA_F32, [3], cqsa.CQSA_FLAG_KV_SINGLE),
])
def test_estimate_backward_matches_built_plan(n, h, d, dt, levels, flags):
    """The dry run's backward figures (mode, L and Delta placement, workspace) equal those of
    the plan cqsa_plan_create builds, at budgets around the backward's layouts: none
    fitting, host statistics only, statistics on the device, unlimited."""
    rates = {"attn_tflops": 1.0, "merge_gbs": 1.0, "h2d_gbs": 1.0, "d2h_gbs": 1.0}
    with cqsa.Plan(n, h, d, dt, levels, flags=flags) as free:
        big = free.info["bwd_stream_workspace_bytes"]
    budgets = [0, big + (16 << 20)]
    # the smallest budget with a backward layout, and the bytes just below it
    lo, hi = 1, big + (16 << 20)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        try:
            with cqsa.Plan(n, h, d, dt, levels, budget_bytes=mid, flags=flags) as p:
                fits = p.info["bwd_stream_mode"] != 0
        except cqsa.CqsaError:
            fits = False
        lo, hi = (lo, mid) if fits else (mid, hi)
    budgets += [hi, hi - 1, hi + 4 * h * n]
    seen_host_stats = set()
    for b in budgets:
        try:
            p = cqsa.Plan(n, h, d, dt, levels, budget_bytes=b, flags=flags)
        except cqsa.CqsaError:
            continue  # the forward itself does not fit
        with p:
            info = p.info
        e = cqsa.cqsa_plan_estimate(n, h, d, dt, levels, budget_bytes=b, flags=flags, rates=rates)
        if info["bwd_stream_mode"] == 0:
            assert e["bwd_levels"] == 0 and e["bwd_stream_workspace_bytes"] == -1, b
            continue
        assert e["bwd_levels"] == len(levels), b
        assert e["bwd_stream_mode"] == info["bwd_stream_mode"], b
        assert e["bwd_host_stats"] == info["bwd_host_stats"], b
        assert e["bwd_stream_workspace_bytes"] == info["bwd_stream_workspace_bytes"], b
        assert e["bwd_task_tokens"] == info["task_tokens"], b
        seen_host_stats.add(info["bwd_host_stats"])
    assert seen_host_stats == {0, 1}


def test_estimate_backward_of_a_billion_tokens_divides_further():
    """A billion tokens under 2 GiB: the forward fits at 7 levels of l = 3, the backward (four
    staged tensors and three transposed copies per task) only at 9, with L and Delta (8 GiB
    at this N) in pinned host memory; with the 7 levels fixed it has no layout."""
    rates = {"attn_tflops": 1.0, "merge_gbs": 1.0, "h2d_gbs": 1.0, "d2h_gbs": 1.0}
    GiB = 1 << 30
    e = cqsa.cqsa_plan_estimate(1 << 30, 1, 128, cqsa.CQSA_BF16, [3], n_levels=0, budget_bytes=2 * GiB,
                                flags=cqsa.CQSA_FLAG_PAD, rates=rates)
    assert e["levels"] == 7 and e["bwd_levels"] == 9
    assert e["bwd_host_stats"] == 1 and 0 < e["bwd_stream_workspace_bytes"] <= 2 * GiB
    unit = -(-(1 << 30) // 7 ** 9)  # tokens per unit of the padded 9-level grid
    assert e["bwd_task_tokens"] == unit * 3 ** 9
    fixed = cqsa.cqsa_plan_estimate(1 << 30, 1, 128, cqsa.CQSA_BF16, [3] * 7, budget_bytes=2 * GiB,
                                    flags=cqsa.CQSA_FLAG_PAD, rates=rates)
    assert fixed["bwd_levels"] == 0 and fixed["bwd_stream_workspace_bytes"] == -1
