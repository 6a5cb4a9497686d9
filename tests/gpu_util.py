"""Helpers for the GPU tests: moving seeded inputs into device or pinned host memory
and reading results back (torch is used for memory only)."""
import numpy as np

from memory_bounded_streaming_amd import cqsa
from memory_bounded_streaming_amd.inputs import bf16_bits_to_f32, gen_tensor

DT = {"bf16": cqsa.CQSA_BF16, "f32": cqsa.CQSA_F32}


def torch_mod():
    import torch
    return torch


def to_device(arr, dtype):
    torch = torch_mod()
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(arr).cuda()


def empty_device(shape, dtype):
    torch = torch_mod()
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")


def to_numpy(t, dtype):
    torch = torch_mod()
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(arr, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def pinned(shape, dtype):
    """A pinned host tensor and a numpy view of it (uint16 bits for bf16)."""
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.empty(shape, dtype=torch.int16, pin_memory=True)
        return t, t.numpy().view(np.uint16)
    t = torch.empty(shape, dtype=torch.float32, pin_memory=True)
    return t, t.numpy()


def pinned_qkv(seed, n, h, d, dtype):
    """Q, K, V drawn straight into pinned host memory: ((tq, tk, tv), (q, k, v) numpy views)."""
    ts, views = [], []
    for i in range(3):
        t, a = pinned((n, h, d), dtype)
        gen_tensor(seed, i, n, h, d, dtype, out=a)
        ts.append(t)
        views.append(a)
    return tuple(ts), tuple(views)


def log(msg):
    print(msg, flush=True)


def oracle_rows(q, k, v, rows, dtype, workers=None):
    """attention_fp64 over disjoint chunks of the sampled rows in parallel threads.

    Each thread runs the unchanged oracle on its rows with BLAS limited to one thread,
    so the host's cores are used once each; results are reassembled in row order.
    """
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle.attention import attention_fp64

    rows = np.asarray(rows, dtype=np.int64)
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = [c for c in np.array_split(rows, workers) if c.size]
    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=len(chunks)) as pool:
            parts = list(pool.map(lambda c: attention_fp64(q, k, v, rows=c, dtype=dtype, key_block=8192), chunks))
    return np.concatenate([p[0] for p in parts], axis=0), np.concatenate([p[1] for p in parts], axis=1)


def init_device_runtime():
    """Make the HIP runtime's one-time device set-up of this process happen now: it takes
    device memory (about 150 MiB on this image) at the process's first device allocation,
    copy and kernel, whoever makes them, and would otherwise be counted in the observed
    memory of whichever library call came first.  Returns the free device memory it took
    (0 when the set-up had already happened)."""
    torch = torch_mod()
    free0, _ = torch.cuda.mem_get_info()
    x = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    x.copy_(torch.ones(1 << 20, dtype=torch.uint8).pin_memory())
    x.copy_(torch.ones(1 << 20, dtype=torch.uint8))
    x.fill_(2)
    assert int(x.cpu()[0]) == 2
    del x
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    return max(0, free0 - free1)
