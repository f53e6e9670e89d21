"""GPU parity of the low-memory mode (SOL_LOW_MEMORY): no V^T copy in the workspace,
value tiles read from V itself with transposing LDS reads.

The mode computes the same products in the same order as the default mode, so
outputs, selections and row statistics are compared bit for bit with the
default mode on the same inputs; one case per head dim and correction form is
also checked against the oracle. Every call gets a workspace of exactly
sol_attn_workspace_bytes_flags(..., SOL_LOW_MEMORY) bytes, so a read or write
past it would show as a device fault or as a difference.
"""
import math

import numpy as np
import pytest
import torch

from free_block_sparse_mean_amd import workloads as wl
from tests import parity_utils as pu

pytestmark = pytest.mark.gpu

CASES = [
    wl.small("lm_ragged_d128", 2, 3, 64 * 100, 128, grid=(4, 25, 64)),
    wl.small("lm_ragged_d64", 1, 2, 64 * 70, 64, grid=(2, 35, 64)),
    wl.small("lm_skewed_d128", 1, 2, 64 * 130, 128, grid=(2, 65, 64), skewed=True),
]


def _run(gpu_lib, q, k, v, beta, flags):
    """Pre-pass and fused pass with stats, on an exactly sized workspace."""
    B, H, N, d = q.shape
    nb = N // 64
    W = (nb + 63) // 64
    ws = gpu_lib.new_workspace(B, H, N, d, q.device, flags)
    assert ws.numel() == gpu_lib.sol_attn_workspace_bytes(B, H, N, d, flags)
    out = torch.empty_like(q)
    kept = torch.full((B, H, nb), -1, dtype=torch.int32, device=q.device)
    mask = torch.zeros((B, H, nb, W), dtype=torch.int64, device=q.device)
    tau = torch.empty((B, H, nb), dtype=torch.float32, device=q.device)
    gpu_lib.sol_block_summaries(k, v, ws, flags)
    gpu_lib.sol_attn_fused(q, k, v, out, beta, flags, ws, kept_per_row=kept, mask_bits=mask, tau=tau)
    torch.cuda.synchronize()
    return out, kept, mask, tau


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("form", ["none", "block", "row"])
@pytest.mark.parametrize("beta", [0.5, 2.0, -math.inf])
def test_low_memory_bit_equal(w, form, beta, gpu_lib):
    print(f"case low-memory {w.name} {form} beta={beta}", flush=True)
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    base = {"none": 0, "block": gpu_lib.SOL_CORRECTION, "row": gpu_lib.SOL_CORRECTION_ROW}[form]
    ref = _run(gpu_lib, q, k, v, beta, base)
    low = _run(gpu_lib, q, k, v, beta, base | gpu_lib.SOL_LOW_MEMORY)
    small = gpu_lib.sol_attn_workspace_bytes(w.B, w.H, w.N, w.d, gpu_lib.SOL_LOW_MEMORY)
    assert small < gpu_lib.sol_attn_workspace_bytes(w.B, w.H, w.N, w.d)
    for a, b, name in zip(ref, low, ("out", "kept", "mask", "tau")):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("w", [CASES[0], CASES[1]], ids=lambda w: w.name)
@pytest.mark.parametrize("form", ["block", "row"])
def test_low_memory_against_oracle(w, form, gpu_lib):
    q, k, v = wl.make_qkv(w)
    flags = gpu_lib.SOL_LOW_MEMORY | (gpu_lib.SOL_CORRECTION if form == "block" else gpu_lib.SOL_CORRECTION_ROW)
    out, kept, mask, tau = _run(gpu_lib, q.cuda(), k.cuda(), v.cuda(), 1.0, flags)
    m = gpu_lib.decode_mask(mask, w.n_blocks)
    for b in range(w.B):
        for h in range(w.H):
            pu.check_head(q[b, h], k[b, h], v[b, h], out[b, h].float().cpu().numpy(), m[b, h].numpy(),
                          tau[b, h].cpu().numpy(), 1.0, True, w.dtype,
                          label=f"low-memory {w.name} {form} b{b} h{h}", correction_form=form)


def test_low_memory_given_mask_and_joint(gpu_lib):
    """The given-mask pass and the joint text segment in the low-memory mode."""
    w = CASES[0]
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    nb = w.n_blocks
    _, _, mask, _ = _run(gpu_lib, q, k, v, 1.0, gpu_lib.SOL_CORRECTION)
    outs = []
    for flags in (0, gpu_lib.SOL_LOW_MEMORY):
        ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d, q.device, flags)
        gpu_lib.sol_block_summaries(k, v, ws, flags)
        o1 = torch.empty_like(q)
        gpu_lib.sol_attn_masked(q, k, v, o1, mask, flags, ws)
        o2 = torch.empty_like(q)
        gpu_lib.sol_attn_fused(q, k, v, o2, 1.0, flags | gpu_lib.SOL_CORRECTION, ws, text_blocks=7)
        torch.cuda.synchronize()
        outs.append((o1, o2))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("form", ["none", "block", "row"])
def test_low_memory_strided(form, gpu_lib):
    """[B, N, H, d] tensors in the low-memory mode: the value tiles come straight from the
    strided V; bit for bit the contiguous default-mode result, for every correction form."""
    w = CASES[0]
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    base = {"none": 0, "block": gpu_lib.SOL_CORRECTION, "row": gpu_lib.SOL_CORRECTION_ROW}[form]
    ref = torch.empty_like(q)
    gpu_lib.sol_attn_fwd_ex(q, k, v, ref, 1.0, base)
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    out = torch.empty_like(qs)
    gpu_lib.sol_attn_fwd_strided(qs, ks, vs, out, 1.0, base | gpu_lib.SOL_LOW_MEMORY)
    torch.cuda.synchronize()
    assert torch.equal(out.contiguous(), ref)


def test_low_memory_noalloc_larger_shape(gpu_lib):
    """Without the V^T copy a 16K-token, 24-head problem fits the 64 MiB scratch of the
    no-allocation entry point (with the copy it does not); equal to sol_attn_fwd_ex."""
    w = wl.small("lm_noalloc_16k", 1, 24, 16384, 128, grid=(16, 32, 32))
    flags = gpu_lib.SOL_CORRECTION | gpu_lib.SOL_LOW_MEMORY
    assert gpu_lib.sol_attn_workspace_bytes(w.B, w.H, w.N, w.d, flags) <= 64 << 20
    assert gpu_lib.sol_attn_workspace_bytes(w.B, w.H, w.N, w.d) > 64 << 20
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    ref = torch.empty_like(q)
    gpu_lib.sol_attn_fwd_ex(q, k, v, ref, 1.5, gpu_lib.SOL_CORRECTION)
    out = torch.empty_like(q)
    gpu_lib.sol_attn_fwd_noalloc(q, k, v, out, 1.5, flags)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("form", ["none", "block", "row"])
def test_low_memory_f32_inputs(form, gpu_lib):
    """float32 inputs have no V^T copy in either mode: the flag only shrinks the
    workspace, and the results are bit for bit those of the default mode."""
    w = wl.small("lm_f32_d128", 1, 2, 64 * 70, 128, dtype="f32", grid=(2, 35, 64))
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    base = gpu_lib.SOL_F32 | {"none": 0, "block": gpu_lib.SOL_CORRECTION, "row": gpu_lib.SOL_CORRECTION_ROW}[form]
    ref = _run(gpu_lib, q, k, v, 1.0, base)
    low = _run(gpu_lib, q, k, v, 1.0, base | gpu_lib.SOL_LOW_MEMORY)
    for a, b, name in zip(ref, low, ("out", "kept", "mask", "tau")):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("form", ["block", "row"])
def test_low_memory_max_sequence_length(form, gpu_lib):
    """N = 262144 (n_b = 4096, the largest), two heads: one taken by the statically mapped
    workgroups, one dealt from the work-item queue. The value tiles then lie up to 64 MiB
    into each head's V; outputs, selections and row statistics bit for bit the default mode's."""
    print(f"case low-memory max N {form}", flush=True)
    w = wl.small("lm_max_n", 1, 2, 262144, 128, grid=(64, 64, 64))
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    base = gpu_lib.SOL_CORRECTION if form == "block" else gpu_lib.SOL_CORRECTION_ROW
    ref = _run(gpu_lib, q, k, v, 1.5, base)
    low = _run(gpu_lib, q, k, v, 1.5, base | gpu_lib.SOL_LOW_MEMORY)
    for a, b, name in zip(ref, low, ("out", "kept", "mask", "tau")):
        assert torch.equal(a, b), name


def test_low_memory_routing_baselines_and_masked(gpu_lib):
    """The map-based routing baselines and the given-mask pass on a workspace of the
    low-memory size (with the flag): the same proxy map, masks and outputs as on a full
    workspace."""
    w = CASES[0]
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    nb = w.n_blocks
    W = (nb + 63) // 64
    res = []
    for flags in (0, gpu_lib.SOL_LOW_MEMORY):
        ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d, q.device, flags)
        assert ws.numel() == gpu_lib.sol_attn_workspace_bytes(w.B, w.H, w.N, w.d, flags)
        gpu_lib.sol_block_summaries(k, v, ws, flags)
        pm = torch.empty((w.B, w.H, nb, nb), dtype=torch.float32, device=q.device)
        got = []
        for mode, kw in ((gpu_lib.SOL_ROUTE_THRESHOLD, {"beta": 1.0}), (gpu_lib.SOL_ROUTE_TOPK, {"top_k": 9}),
                         (gpu_lib.SOL_ROUTE_TOPP, {"top_p": 0.5})):
            words = torch.zeros((w.B, w.H, nb, W), dtype=torch.int64, device=q.device)
            gpu_lib.sol_route(q, mode, ws, pm, words, flags=flags, **kw)
            out = torch.empty_like(q)
            gpu_lib.sol_attn_masked(q, k, v, out, words, flags, ws)
            torch.cuda.synchronize()
            got += [pm.clone(), words, out]
        res.append(got)
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.parametrize("N", [64, 128, 192, 64 * 65])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("form", ["block", "row"])
def test_low_memory_tiny_and_word_edges(N, d, form, gpu_lib):
    """One to 65 key blocks (a single partial tile, a tile plus one block): the low-memory
    mode bit for bit the default mode, keep-all, threshold and keep-none."""
    w = wl.small(f"lm_edge_{N}_{d}", 1, 2, N, d, grid=(1, N // 64, 64))
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    base = gpu_lib.SOL_CORRECTION if form == "block" else gpu_lib.SOL_CORRECTION_ROW
    for beta in (-math.inf, 0.5, math.inf):
        print(f"case low-memory edge N={N} d={d} {form} beta={beta}", flush=True)
        ref = _run(gpu_lib, q, k, v, beta, base)
        low = _run(gpu_lib, q, k, v, beta, base | gpu_lib.SOL_LOW_MEMORY)
        for a, b, name in zip(ref, low, ("out", "kept", "mask", "tau")):
            assert torch.equal(a, b), name
