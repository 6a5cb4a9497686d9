"""GPU parity of the causal variant (CQSA_FLAG_CAUSAL: row i attends keys j <= i)
against the fp64 oracle (needs an MI355X).

Forward on device and streamed through all four staging modes (which must equal the
device path bit for bit), the backward on device, and the full-size bench shape on
sampled rows.  The oracle takes the same reading (R16 of oracle.plan): the division
and owners are unchanged, a task keeps the unit pairs whose key unit does not come
after the query unit, and the diagonal block is masked element by element.
"""
import numpy as np
import pytest

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import gen_qkv, gen_tensor, round_to_bf16_bits, sample_rows
from oracle.attention import attention_fp64
from oracle.backward import attention_backward_given_fp64
from oracle.tolerance import (BF16_LSE_TOL, BF16_REL_TOL, F32_ABS_TOL, F32_LSE_TOL, grad_rel_err, max_abs_err,
                              rowwise_rel_err)

from gpu_util import DT, as_f64, empty_device, log, pinned, to_device, to_numpy

pytestmark = pytest.mark.gpu
CAUSAL, PAD = cqsa.CQSA_FLAG_CAUSAL, cqsa.CQSA_FLAG_PAD

CASES = [  # levels, N, heads, head_dim, dtype
    ([3], 7 * 300, 2, 128, "bf16"),       # units longer than a 256-row query tile
    ([3], 7 * 40, 1, 64, "bf16"),
    ([4], 13 * 130 + 7, 2, 128, "bf16"),  # padded
    ([2, 2], 9 * 24, 2, 64, "bf16"),
    ([3, 2], 21 * 20, 1, 128, "bf16"),
    ([1], 333, 2, 128, "bf16"),           # undivided: one task, one diagonal run
    ([3], 7 * 64, 1, 64, "f32"),
    ([2, 3], 21 * 9 + 2, 1, 128, "f32"),  # padded
    ([8], 57 * 24, 1, 128, "bf16"),       # 57 tasks of 8 units
    ([6], 31 * 30 + 3, 2, 64, "f32"),     # 31 tasks of 6 units, padded
]


def _ids(c):
    return f"l{'x'.join(map(str, c[0]))}-n{c[1]}-h{c[2]}-d{c[3]}-{c[4]}"


def _flags(levels, n):
    prod_c = int(np.prod([l * (l - 1) + 1 for l in levels]))
    return CAUSAL | (PAD if n % prod_c else 0)


def _check(got, ref, dtype, what, grad=False):
    err = max_abs_err(got, ref) if dtype == "f32" else (grad_rel_err if grad else rowwise_rel_err)(got, ref)
    log(f"  {what}: {err:.3e}")
    assert err <= (F32_ABS_TOL if dtype == "f32" else BF16_REL_TOL), (what, err)


def _device_forward(p, q, k, v, n, h, d, dtype):
    import torch
    o = empty_device((n, h, d), dtype)
    lse = torch.empty((h, n), device="cuda")
    p.forward(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), o, lse)
    torch.cuda.synchronize()
    return to_numpy(o, dtype), lse.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_causal_forward_matches_oracle(case):
    pytest.importorskip("torch")
    levels, n, h, d, dtype = case
    log(f"causal forward {_ids(case)}")
    q, k, v = gen_qkv(211 + n, n, h, d, dtype)
    o_ref, lse_ref = attention_fp64(q, k, v, dtype=dtype, causal=True)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=_flags(levels, n)) as p:
        o, lse = _device_forward(p, q, k, v, n, h, d, dtype)
    _check(as_f64(o, dtype), o_ref, dtype, "O")
    assert np.abs(lse - lse_ref).max() <= (F32_LSE_TOL if dtype == "f32" else BF16_LSE_TOL)


MODES = [0, cqsa.CQSA_FLAG_HOST_ACC, cqsa.CQSA_FLAG_KV_SINGLE, cqsa.CQSA_FLAG_HOST_ACC | cqsa.CQSA_FLAG_KV_SINGLE]


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[4], CASES[7]], ids=_ids)
@pytest.mark.parametrize("mode", MODES, ids=["devacc-kv2", "hostacc-kv2", "devacc-kv1", "hostacc-kv1"])
def test_causal_stream_equals_device_path(case, mode):
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype = case
    log(f"causal stream {_ids(case)} mode={mode}")
    q, k, v = gen_qkv(223 + n, n, h, d, dtype)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=_flags(levels, n) | mode) as p:
        o_dev, lse_dev = _device_forward(p, q, k, v, n, h, d, dtype)
        ins = []
        for x in (q, k, v):
            t, a = pinned((n, h, d), dtype)
            a[...] = x
            ins.append(t)
        to, oa = pinned((n, h, d), dtype)
        tl = torch.empty((h, n), dtype=torch.float32, pin_memory=True)
        st = p.forward(*ins, to, tl, residency=cqsa.CQSA_RES_HOST_PINNED, stats=True)
        assert st["useful_flop"] == pytest.approx(2.0 * n * (n + 1) * d * h)
    assert np.array_equal(oa, o_dev) and np.array_equal(tl.numpy(), lse_dev), "bit-identical to the device path"


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[3], CASES[5], CASES[6], CASES[7]], ids=_ids)
def test_causal_backward_matches_oracle(case):
    torch = pytest.importorskip("torch")
    levels, n, h, d, dtype = case
    log(f"causal backward {_ids(case)}")
    q, k, v = gen_qkv(227 + n, n, h, d, dtype)
    do = gen_tensor(227 + n, 3, n, h, d, dtype)
    o_ref, lse_ref = attention_fp64(q, k, v, dtype=dtype, causal=True)
    o32 = o_ref.astype(np.float32)
    o_in, lse_in = (round_to_bf16_bits(o32) if dtype == "bf16" else o32), lse_ref.astype(np.float32)
    grads = attention_backward_given_fp64(q, k, v, o_in, lse_in, do, dtype=dtype, causal=True)
    with cqsa.Plan(n, h, d, DT[dtype], levels, flags=_flags(levels, n)) as p:
        dev = [to_device(x, dtype) for x in (q, k, v, o_in)]
        dev.append(torch.from_numpy(lse_in).cuda())
        dev.append(to_device(do, dtype))
        outs = [empty_device((n, h, d), dtype) for _ in range(3)]
        p.backward(*dev, *outs)
        torch.cuda.synchronize()
        got = [as_f64(to_numpy(t, dtype), dtype) for t in outs]
    for name, g, r in zip(("dQ", "dK", "dV"), got, grads):
        _check(g, r, dtype, name, grad=True)


def test_causal_full_size_sampled_rows():
    """N=57344, H=8, d=128, bf16, l=3, causal, device-resident: 2048 sampled rows."""
    torch = pytest.importorskip("torch")
    n, h, d = 57344, 8, 128
    log("causal full size")
    q, k, v = gen_qkv(0, n, h, d, "bf16")
    with cqsa.Plan(n, h, d, cqsa.CQSA_BF16, [3], flags=CAUSAL) as p:
        o = empty_device((n, h, d), "bf16")
        lse = torch.empty((h, n), device="cuda")
        p.forward(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), o, lse)
        torch.cuda.synchronize()
        out, lse = to_numpy(o, "bf16"), lse.cpu().numpy()
    rows = sample_rows(n, 2048, 5, unit_tokens=8192)
    rows = np.unique(np.concatenate([rows, [0, 1, 2, 255, 256, 8191, 8192]]))
    o_ref, lse_ref = attention_fp64(q, k, v, rows=rows, dtype="bf16", causal=True)
    _check(as_f64(out[rows], "bf16"), o_ref, "bf16", "O sampled")
    assert np.abs(lse[:, rows] - lse_ref).max() <= BF16_LSE_TOL
