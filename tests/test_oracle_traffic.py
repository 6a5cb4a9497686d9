"""Pins of the oracle's traffic walk (``oracle.stream_bytes.stream_traffic``) against
values fixed by the mathematics of the plan, not by any implementation.

What the streamed method moves ("Stream-CQSA: Breaking the Billion-Token Barrier on a
Single GPU", section "Implementation: From High-Level Logic to GPU Kernels": stream
Q_i/K_i/V_i of each task to the GPU, aggregate the local statistics, in host memory
when the device cannot hold them):

* every query row is visited by prod(l_k) tasks and each task holds its rows' K and V,
  so with one K/V staging buffer the host-to-device bytes of Q, K and V are exactly
  prod(l) * 3 * N * H * d * e;
* with a host accumulator every visit but a row's first brings its accumulator block
  back (H2D) and every visit but its last sends it out (D2H): (prod(l) - 1) * N * H *
  (d + 2) * 4 bytes each way; O and LSE leave once per row;
* a perfect difference set D meets its shift D + 1 in exactly one residue (the
  difference 1 occurs once), so consecutive tasks S_t, S_{t+1} of one parent share
  exactly one chunk; with two staging buffers that chunk's K/V rows are copied on the
  device: c - 1 transitions per parent of one chunk each.

The five workloads' byte counts are written out as numbers (10.47, 42.28, 88.79 GB of
Q/K/V for the 16 GiB, 8 GiB and 2 GiB workloads), and one 3-task plan is walked by hand.
"""
import pytest

from oracle.plan import make_plan
from oracle.stream_bytes import stream_traffic

GB = 1e9


def closed_form(n, h, d, e, ls, host_acc, kv_buffers):
    """The byte counts of an unpadded plan from the formulas in the module docstring."""
    visits = 1
    for l in ls:
        visits *= l
    row, part, fin = h * d * e, h * (d + 2) * 4, h * (d * e + 4)
    h2d = visits * 3 * n * row + (visits - 1) * n * part * host_acc
    d2h = n * fin + (visits - 1) * n * part * host_acc
    d2d = 0
    if kv_buffers == 2:
        c_in, l_in = ls[-1] * (ls[-1] - 1) + 1, ls[-1]
        parents = 1
        for l in ls[:-1]:
            parents *= l * (l - 1) + 1
        task_tokens = n * visits
        for l in ls:
            task_tokens //= l * (l - 1) + 1
        if c_in > 1:
            d2d = parents * (c_in - 1) * (task_tokens // l_in) * row * 2
    # merge: a row's first visit lands in the accumulator, middle visits read the
    # accumulator and the partial and write the accumulator, the last writes O and LSE
    merge = n * (part + fin) if visits == 1 else n * ((visits - 2) * 3 * part + 2 * part + fin)
    return {"bytes_h2d": h2d - d2d, "bytes_d2h": d2h, "merge_bytes": merge, "bytes_d2d": d2d}


WORKLOADS = [
    # n, h, d, levels, expected Q/K/V H2D bytes with one staging buffer
    (3584, 1, 64, [3], 3 * 3 * 3584 * 64 * 4, 4),
    (57344, 8, 128, [3], 3 * 3 * 57344 * 8 * 128 * 2, 2),
    (212992, 16, 128, [4], 10_468_982_784, 2),
    (1376256, 8, 128, [5], 42_278_584_320, 2),
    (12845056, 1, 128, [3, 3], 88_785_027_072, 2),
]


@pytest.mark.parametrize("n,h,d,ls,qkv_bytes,e", WORKLOADS)
def test_qkv_bytes_of_the_workloads(n, h, d, ls, qkv_bytes, e):
    # the written-out totals are prod(l) * 3 * N * H * d * e
    visits = 1
    for l in ls:
        visits *= l
    assert qkv_bytes == visits * 3 * n * h * d * e
    got = stream_traffic(make_plan(n, ls), h, d, e, host_acc=False, kv_buffers=1)
    assert got["bytes_h2d"] == qkv_bytes
    assert got["bytes_d2d"] == 0
    assert got["bytes_d2h"] == n * h * (d * e + 4)  # O and LSE once


def test_workload_totals_in_gigabytes():
    assert 10_468_982_784 / GB == pytest.approx(10.47, abs=0.005)
    assert 42_278_584_320 / GB == pytest.approx(42.28, abs=0.005)
    assert 88_785_027_072 / GB == pytest.approx(88.79, abs=0.005)


@pytest.mark.parametrize("n,h,d,ls,qkv_bytes,e", WORKLOADS[:4])
@pytest.mark.parametrize("host_acc", [False, True])
@pytest.mark.parametrize("kv_buffers", [1, 2])
def test_walk_equals_closed_form(n, h, d, ls, qkv_bytes, e, host_acc, kv_buffers):
    got = stream_traffic(make_plan(n, ls), h, d, e, host_acc=host_acc, kv_buffers=kv_buffers)
    assert got == closed_form(n, h, d, e, ls, host_acc, kv_buffers)


@pytest.mark.parametrize("host_acc,kv_buffers", [(True, 1), (True, 2)])
def test_two_level_workload_equals_closed_form(host_acc, kv_buffers):
    # the 2 GiB workload runs with its accumulator on the host; one staging buffer
    # (its footprint) and two (chunk reuse inside each outer task)
    n, h, d, ls = 12845056, 1, 128, [3, 3]
    got = stream_traffic(make_plan(n, ls), h, d, 2, host_acc=host_acc, kv_buffers=kv_buffers)
    want = closed_form(n, h, d, 2, ls, host_acc, kv_buffers)
    assert got == want
    if host_acc:
        # (prod(l) - 1) * N * H * (d + 2) * 4 each way on top of Q/K/V and O/LSE
        assert want["bytes_d2h"] - n * h * (d * 2 + 4) == 8 * n * 130 * 4


def test_sixteen_gib_workload_chunk_reuse_bytes():
    # 13 tasks, 12 transitions, one 16,384-token chunk of K and V each, 4,096-byte rows
    got = stream_traffic(make_plan(212992, [4]), 16, 128, 2, host_acc=False, kv_buffers=2)
    assert got["bytes_d2d"] == 12 * 16384 * 4096 * 2 == 1_610_612_736
    assert got["bytes_h2d"] + got["bytes_d2d"] == 10_468_982_784


def test_consecutive_tasks_share_one_chunk():
    # |D ∩ (D + 1)| = 1 for a perfect difference set, so S_t and S_{t+1} share one chunk
    for n, ls in ((7, [3]), (13, [4]), (21, [5]), (31, [6])):
        plan = make_plan(n, ls)
        for a, b in zip(plan.tasks, plan.tasks[1:]):
            ta = {g for g, length, _ in a.segments(1, n) for g in range(g, g + length)}
            tb = {g for g, length, _ in b.segments(1, n) for g in range(g, g + length)}
            assert len(ta & tb) == 1


def test_three_task_plan_walked_by_hand():
    # l = 2: c = 3, D = {0, 1}, tasks S_0 = {0,1}, S_1 = {1,2}, S_2 = {0,2}; N = 6 tokens,
    # 2 per chunk; H = 1, d = 4, bf16.  A token of Q/K/V/O is 8 bytes, a token's
    # statistics (n, m, l) 24 bytes, a token's O and LSE 12 bytes.  Two visits per row.
    #   task 0 (tokens 0-3): K,V 4*2*8 = 64 H2D; unit 0 and unit 1 first visits:
    #          Q 16 H2D each, accumulator 48 D2H each
    #   task 1 (tokens 2-5): tokens 2,3 shared with task 0 -> 32 D2D, 32 H2D of K,V;
    #          unit 1 last visit: Q 16 + accumulator 48 H2D, O/LSE 24 D2H, merge
    #          2*(2*24 + 12) = 120; unit 2 first visit: Q 16 H2D, accumulator 48 D2H
    #   task 2 (tokens 0,1,4,5): tokens 4,5 shared with task 1 -> 32 D2D, 32 H2D;
    #          units 0 and 2 last visits: 16 + 48 H2D, 24 D2H, merge 120 each
    plan = make_plan(6, [2])
    got = stream_traffic(plan, 1, 4, 2, host_acc=True, kv_buffers=2)
    assert got == {"bytes_h2d": (64 + 16 + 16) + (32 + 64 + 16) + (32 + 64 + 64),
                   "bytes_d2h": (48 + 48) + (24 + 48) + (24 + 24),
                   "merge_bytes": 3 * 120,
                   "bytes_d2d": 32 + 32}
    # one staging buffer: no reuse, and the device accumulator: no round trips
    got = stream_traffic(plan, 1, 4, 2, host_acc=False, kv_buffers=1)
    assert got == {"bytes_h2d": 3 * 64 + 6 * 16, "bytes_d2h": 6 * 12, "merge_bytes": 3 * 120, "bytes_d2d": 0}
