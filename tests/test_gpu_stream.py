"""GPU tests of the host-pinned stream engine (needs an MI355X).

Inputs live in pinned host memory; tasks stream through device staging under the
plan's budget.  Each staging mode is forced in turn; the streamed output must equal
the device-resident output bit for bit (same key tiles, same merge order) and match
the fp64 oracle within tolerance.
"""
import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import gen_qkv
from oracle.attention import attention_fp64
from oracle.tolerance import BF16_REL_TOL, F32_ABS_TOL, max_abs_err, rowwise_rel_err

from gpu_util import DT, as_f64, empty_device, log, pinned, to_device, to_numpy

pytestmark = pytest.mark.gpu

MODES = [0, cqsa.CQSA_FLAG_HOST_ACC, cqsa.CQSA_FLAG_KV_SINGLE, cqsa.CQSA_FLAG_HOST_ACC | cqsa.CQSA_FLAG_KV_SINGLE]

CASES = [  # levels, unit, heads, d, dtype
    ([4], 256, 2, 128, "bf16"),
    ([3, 2], 40, 2, 64, "bf16"),
    ([2, 2], 100, 1, 128, "bf16"),
    ([3], 96, 2, 64, "f32"),
    ([1], 500, 1, 128, "bf16"),
    ([8], 24, 1, 128, "bf16"),       # 57 tasks of 8 units: consecutive tasks share one chunk
    ([10], 16, 2, 64, "f32"),        # 91 tasks of 10 units
]


def _device_forward(p, q, k, v, n, h, d, dtype):
    import torch
    o = empty_device((n, h, d), dtype)
    lse = torch.empty((h, n), device="cuda")
    p.forward(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), o, lse)
    torch.cuda.synchronize()
    return to_numpy(o, dtype), lse.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"l{'x'.join(map(str, c[0]))}-u{c[1]}-h{c[2]}-d{c[3]}-{c[4]}")
@pytest.mark.parametrize("flags", MODES, ids=["devacc-kv2", "hostacc-kv2", "devacc-kv1", "hostacc-kv1"])
def test_stream_modes_equal_device_path(case, flags):
    torch = pytest.importorskip("torch")
    levels, u, h, d, dtype = case
    n = int(np.prod([l * (l - 1) + 1 for l in levels])) * u
    log(f"stream {levels} u={u} h={h} d={d} {dtype} flags={flags}")
    q, k, v = gen_qkv(41 + n, n, h, d, dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=flags) as p:
        o_dev, lse_dev = _device_forward(p, q, k, v, n, h, d, dtype)
        tq, qa = pinned((n, h, d), dtype)
        tk, ka = pinned((n, h, d), dtype)
        tv, va = pinned((n, h, d), dtype)
        qa[...], ka[...], va[...] = q, k, v
        to, oa = pinned((n, h, d), dtype)
        tl = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
        st = p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED, stats=True)
        assert st["peak_device_bytes"] >= p.info["stream_workspace_bytes"]
        e = 2 if dtype == "bf16" else 4
        visits = int(np.prod(levels))
        assert st["bytes_h2d"] + st["bytes_d2d"] >= 3 * visits * n * h * d * e
        est = cqsa.cqsa_plan_estimate(n, h, d, DT[dtype], levels, flags=flags,
                                      rates={"attn_tflops": 1.0, "merge_gbs": 1.0, "h2d_gbs": 1.0, "d2h_gbs": 1.0})
        assert (est["bytes_h2d"], est["bytes_d2h"], est["bytes_d2d"]) == (st["bytes_h2d"], st["bytes_d2h"], st["bytes_d2d"]), \
            "dry run bytes exact"
        assert np.array_equal(oa, o_dev), "streamed output equals the device-resident output bit for bit"
        assert np.array_equal(tl.numpy(), lse_dev)
    o_ref, _ = attention_fp64(q, k, v, dtype=dtype)
    out = as_f64(oa, dtype)
    if dtype == "f32":
        assert max_abs_err(out, o_ref) <= F32_ABS_TOL
    else:
        assert rowwise_rel_err(out, o_ref) <= BF16_REL_TOL


def test_stream_respects_budget_and_reports_phases():
    torch = pytest.importorskip("torch")
    n, h, d = 13 * 512, 4, 128
    q, k, v = gen_qkv(7, n, h, d, "bf16")
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [4]) as probe:
        need = probe.workspace_size(cqsa.CQSA_RES_HOST_PINNED)
    budget = need // 2 + (64 << 20)
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [4], budget_bytes=budget) as p:
        assert p.info["stream_workspace_bytes"] <= budget
        tq, qa = pinned((n, h, d), "bf16")
        tk, ka = pinned((n, h, d), "bf16")
        tv, va = pinned((n, h, d), "bf16")
        qa[...], ka[...], va[...] = q, k, v
        to, oa = pinned((n, h, d), "bf16")
        free0, _ = torch.cuda.mem_get_info()
        st = p.forward(tq, tk, tv, to, None, residency=cqsa.CQSA_RES_HOST_PINNED, stats=True)
        assert st["peak_device_bytes"] <= budget
        assert st["n_attn_launches"] == 13 * 4
        for key in ("t_h2d_ms", "t_attn_ms", "t_merge_ms", "t_d2h_ms"):
            assert st[key] > 0.0, key
        free1, _ = torch.cuda.mem_get_info()
        assert abs(free1 - free0) < (64 << 20), "the call frees its workspace"
    rows = np.arange(0, n, 37)
    o_ref, _ = attention_fp64(q, k, v, rows=rows, dtype="bf16")
    assert rowwise_rel_err(as_f64(oa[rows], "bf16"), o_ref) <= BF16_REL_TOL


def test_host_pinned_residency_rejects_device_and_pageable_buffers():
    """The streamed paths copy with explicit host/device directions: a device tensor or
    pageable host memory given as a host-pinned buffer is EINVAL before any copy, and a
    correct call on the same plan still works afterwards."""
    torch = pytest.importorskip("torch")
    n, h, d = 7 * 64, 1, 64
    q, k, v = gen_qkv(3, n, h, d, "bf16")
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        pins = []
        for x in (q, k, v):
            t, a = pinned((n, h, d), "bf16")
            a[...] = x
            pins.append(t)
        to, oa = pinned((n, h, d), "bf16")
        dev = to_device(q, "bf16")
        pageable = np.zeros((n, h, d), np.uint16)
        for bad in ((dev, pins[1], pins[2], to), (pins[0], pins[1], pins[2], pageable)):
            with pytest.raises(cqsa.CqsaError) as e:
                p.forward(*bad, None, residency=cqsa.CQSA_RES_HOST_PINNED)
            assert e.value.status == -1 and "pinned" in str(e.value)
        lse = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
        g = [pinned((n, h, d), "bf16")[0] for _ in range(3)]
        with pytest.raises(cqsa.CqsaError) as e:
            p.backward(pins[0], pins[1], pins[2], to, lse, dev, *g, residency=cqsa.CQSA_RES_HOST_PINNED)
        assert e.value.status == -1 and "d_o" in str(e.value)
        p.forward(*pins, to, lse, residency=cqsa.CQSA_RES_HOST_PINNED)
        o_dev, _ = _device_forward(p, q, k, v, n, h, d, "bf16")
        assert np.array_equal(oa, o_dev)


def test_concurrent_first_calls_on_one_plan():
    """Two threads make the first forward calls on one plan at once, each on its own stream
    (both race to upload the plan's descriptor tables); both outputs equal a later
    sequential call bit for bit."""
    import threading
    torch = pytest.importorskip("torch")
    n, h, d = 7 * 96, 2, 128
    q, k, v = gen_qkv(11, n, h, d, "bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3]) as p:
        outs = [empty_device((n, h, d), "bf16") for _ in range(2)]
        streams = [torch.cuda.Stream() for _ in range(2)]
        errors = []

        def worker(i):
            try:
                with torch.cuda.stream(streams[i]):
                    p.forward(qd, kd, vd, outs[i], None, stream=streams[i])
                streams[i].synchronize()
            except Exception as e:  # reported below
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        assert not errors, errors
        o_seq, _ = _device_forward(p, q, k, v, n, h, d, "bf16")
    for o in outs:
        assert np.array_equal(to_numpy(o, "bf16"), o_seq)


@pytest.mark.parametrize("flags", [cqsa.CQSA_FLAG_HOST_ACC, cqsa.CQSA_FLAG_HOST_ACC | cqsa.CQSA_FLAG_KV_SINGLE],
                         ids=["hostacc-kv2", "hostacc-kv1"])
def test_repeated_calls_reuse_the_host_accumulator(flags):
    """A plan keeps its pinned host accumulator between streamed calls: a second call with
    other inputs must not see what the first left in it (every block is written before it
    is read back), and each call equals the device path bit for bit."""
    torch = pytest.importorskip("torch")
    levels, u, h, d, dtype = [3, 2], 64, 2, 128, "bf16"
    n = 7 * 3 * u
    log(f"repeated streamed calls {levels} u={u} flags={flags}")
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=flags) as p:
        tq, qa = pinned((n, h, d), dtype)
        tk, ka = pinned((n, h, d), dtype)
        tv, va = pinned((n, h, d), dtype)
        to, oa = pinned((n, h, d), dtype)
        tl = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
        for seed in (301, 302, 301):
            q, k, v = gen_qkv(seed, n, h, d, dtype)
            o_dev, lse_dev = _device_forward(p, q, k, v, n, h, d, dtype)
            qa[...], ka[...], va[...] = q, k, v
            oa[...] = 0
            p.forward(tq, tk, tv, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED)
            assert np.array_equal(oa, o_dev), f"seed {seed}: streamed output equals the device path"
            assert np.array_equal(tl.numpy(), lse_dev), f"seed {seed}: LSE equals the device path"
