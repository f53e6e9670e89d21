"""sol_attn_fwd_noalloc (the entry point that allocates nothing) against
sol_attn_fwd_ex (caller workspace) on the same inputs, through the C ABI.

Both run the same kernels on the same inputs, so outputs and row statistics
must agree bit for bit. Two calls in a row on one device, the second with a
smaller problem, so the second runs on the scratch the first one left behind.
"""
import math

import pytest
import torch

from free_block_sparse_mean_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = [
    # first call (larger), second call (smaller), beta, flags name
    (wl.small("noalloc_big", 2, 3, 64 * 70, 128, grid=(2, 35, 64)),
     wl.small("noalloc_small", 1, 2, 64 * 33, 128, grid=(3, 11, 64), seed=5), 1.0, "corr"),
    (wl.small("noalloc_d64", 1, 3, 64 * 40, 64, grid=(4, 10, 64)),
     wl.small("noalloc_d64_small", 1, 1, 64 * 9, 64, grid=(1, 9, 64), seed=3), 1.5, "none"),
    (wl.small("noalloc_f32", 1, 2, 64 * 33, 64, dtype="f32", grid=(3, 11, 64)),
     wl.small("noalloc_f32_small", 1, 1, 64 * 12, 64, dtype="f32", grid=(1, 12, 64), seed=7), 1.0, "row"),
]


def _flags(lib, name):
    return {"corr": lib.SOL_CORRECTION, "none": 0, "row": lib.SOL_CORRECTION_ROW}[name]


def _run(lib, fn, q, k, v, beta, flags):
    B, H, N, _ = q.shape
    nb = N // 64
    out = torch.full_like(q, float("nan"))
    kept = torch.full((B, H, nb), -1, dtype=torch.int32, device=q.device)
    mask = torch.zeros((B, H, nb, (nb + 63) // 64), dtype=torch.int64, device=q.device)
    tau = torch.empty((B, H, nb), dtype=torch.float32, device=q.device)
    fn(q, k, v, out, beta, flags, kept_per_row=kept, mask_bits=mask, tau=tau)
    return out, kept, mask, tau


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_noalloc_equals_workspace_entry(case, gpu_lib):
    big, small, beta, fname = case
    flags = _flags(gpu_lib, fname)
    for w in (big, small):
        print(f"[noalloc] {w.name} B{w.B} H{w.H} N{w.N} d{w.d} {w.dtype} beta {beta} {fname}", flush=True)
        q, k, v = (x.cuda() for x in wl.make_qkv(w))
        got = _run(gpu_lib, gpu_lib.sol_attn_fwd_noalloc, q, k, v, beta, flags)
        ref = _run(gpu_lib, lambda *a, **kw: gpu_lib.sol_attn_fwd_ex(*a[:6], **kw), q, k, v, beta, flags)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "kept_per_row", "mask_bits", "tau"), got, ref):
            assert torch.equal(a, b), f"{w.name}: {name} differs from sol_attn_fwd_ex"
        assert not torch.isnan(got[0].float()).any()


def test_noalloc_on_side_stream_and_dense(gpu_lib):
    """On a side stream, dense limit (every block kept): equals sol_attn_fwd_ex there too."""
    w = wl.small("noalloc_stream", 1, 2, 64 * 20, 128, grid=(1, 20, 64), seed=11)
    q, k, v = (x.cuda() for x in wl.make_qkv(w))
    s = torch.cuda.Stream()
    flags = gpu_lib.SOL_DENSE | gpu_lib.SOL_CORRECTION
    with torch.cuda.stream(s):
        a = torch.empty_like(q)
        b = torch.empty_like(q)
        gpu_lib.sol_attn_fwd_noalloc(q, k, v, a, -math.inf, flags, stream=s)
        gpu_lib.sol_attn_fwd_ex(q, k, v, b, -math.inf, flags, stream=s)
    s.synchronize()
    assert torch.equal(a, b)
