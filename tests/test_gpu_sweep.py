"""Seeded sweep over small random plans (needs an MI355X).

Each case draws a plan shape -- levels, unit or token count, heads, head dim, dtype,
padding, causality and a forced staging mode -- and checks, through the C ABI:
  * the host-pinned streamed forward equals the device-resident forward bit for bit;
  * the device-resident forward matches the fp64 oracle on every row;
  * the host-pinned streamed backward equals the device-resident backward bit for bit;
  * the device-resident backward matches the oracle evaluated at the forward's own O
    and LSE (dQ, dK, dV, every row).
"""
import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import gen_qkv, gen_tensor
from oracle.attention import attention_fp64
from oracle.backward import attention_backward_given_fp64
from oracle.tolerance import (BF16_LSE_TOL, BF16_REL_TOL, F32_ABS_TOL, F32_LSE_TOL, grad_rel_err, max_abs_err,
                              rowwise_rel_err)

from gpu_util import DT, as_f64, empty_device, log, pinned, to_device, to_numpy

pytestmark = pytest.mark.gpu

LEVELS = [[2], [3], [4], [2, 2], [3, 2], [2, 3]]
STAGING = [0, cqsa.CQSA_FLAG_HOST_ACC, cqsa.CQSA_FLAG_KV_SINGLE, cqsa.CQSA_FLAG_HOST_ACC | cqsa.CQSA_FLAG_KV_SINGLE]


def _cases(count=48, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        levels = LEVELS[rng.integers(len(LEVELS))]
        prod_c = int(np.prod([l * (l - 1) + 1 for l in levels]))
        pad = bool(rng.integers(2))
        causal = bool(rng.integers(2))
        if pad:
            n = int(rng.integers(prod_c, min(1500, prod_c * 120) + 1))
        else:
            n = prod_c * int(rng.integers(1, max(2, 1500 // prod_c) + 1))
        heads = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        flags = STAGING[rng.integers(len(STAGING))] | (cqsa.CQSA_FLAG_PAD if pad else 0) | \
            (cqsa.CQSA_FLAG_CAUSAL if causal else 0)
        out.append((i, levels, n, heads, d, dtype, flags))
    return out


def _id(case):
    i, levels, n, h, d, dtype, flags = case
    return f"{i}-l{'x'.join(map(str, levels))}-n{n}-h{h}-d{d}-{dtype}-f{flags}"


@pytest.mark.parametrize("case", _cases(), ids=_id)
def test_random_plan_forward_and_backward(case):
    torch = pytest.importorskip("torch")
    i, levels, n, h, d, dtype, flags = case
    causal = bool(flags & cqsa.CQSA_FLAG_CAUSAL)
    log(f"sweep {_id(case)}")
    q, k, v = gen_qkv(900 + i, n, h, d, dtype)
    do = gen_tensor(900 + i, 3, n, h, d, dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=flags) as p:
        qd, kd, vd, dod = (to_device(x, dtype) for x in (q, k, v, do))
        o = empty_device((n, h, d), dtype)
        lse = torch.empty((h, n), device="cuda")
        p.forward(qd, kd, vd, o, lse)
        grads = [empty_device((n, h, d), dtype) for _ in range(3)]
        ws = torch.empty(max(p.backward_workspace_size(), 1), dtype=torch.uint8, device="cuda")
        p.backward(qd, kd, vd, o, lse, dod, *grads, workspace=ws)
        torch.cuda.synchronize()
        o_dev, lse_dev = to_numpy(o, dtype), lse.cpu().numpy()
        g_dev = [to_numpy(g, dtype) for g in grads]

        # the same plan streamed from pinned host memory
        hosts = []
        for x in (q, k, v):
            t, a = pinned((n, h, d), dtype)
            a[...] = x
            hosts.append(t)
        to_h, oa = pinned((n, h, d), dtype)
        lse_h = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
        p.forward(*hosts, to_h, lse_h, residency=cqsa.CQSA_RES_HOST_PINNED)
        assert np.array_equal(oa, o_dev), "streamed O equals the device-resident O bit for bit"
        assert np.array_equal(lse_h.numpy(), lse_dev)
        t_o, a_o = pinned((n, h, d), dtype)
        a_o[...] = o_dev
        t_do, a_do = pinned((n, h, d), dtype)
        a_do[...] = do
        outs = [pinned((n, h, d), dtype) for _ in range(3)]
        p.backward(*hosts, t_o, lse_h, t_do, *(t for t, _ in outs), residency=cqsa.CQSA_RES_HOST_PINNED)
        for name, (_, a), g in zip(("dQ", "dK", "dV"), outs, g_dev):
            assert np.array_equal(a, g), f"streamed {name} equals the device-resident {name} bit for bit"

    o_ref, lse_ref = attention_fp64(q, k, v, dtype=dtype, causal=causal)
    out = as_f64(o_dev, dtype)
    if dtype == "f32":
        assert max_abs_err(out, o_ref) <= F32_ABS_TOL
        assert np.abs(lse_dev - lse_ref).max() <= F32_LSE_TOL
    else:
        assert rowwise_rel_err(out, o_ref) <= BF16_REL_TOL
        assert np.abs(lse_dev - lse_ref).max() <= BF16_LSE_TOL
    g_ref = attention_backward_given_fp64(q, k, v, o_dev, lse_dev, do, dtype=dtype, causal=causal)
    for name, g, r in zip(("dQ", "dK", "dV"), g_dev, g_ref):
        got = as_f64(g, dtype)
        if dtype == "f32":
            assert max_abs_err(got, r) <= F32_ABS_TOL, name
        else:
            assert grad_rel_err(got, r) <= BF16_REL_TOL, name
