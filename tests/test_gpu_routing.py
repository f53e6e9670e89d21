"""GPU parity of the routing baselines (sol_route): the materialized proxy map
against the oracle's proxy scores, and each selection rule against the oracle's
rule applied to the same map.

Bar: map within fp32 rounding of the oracle's block-mean products; threshold
masks bit-exact except ties within 1e-4 of tau; top-k masks and index lists
bit-exact (equal scores go to the lower j on both sides); top-p masks equal to
the oracle's except where the oracle's cumulative probability at the cut lies
within 1e-5 of p (fp32 against float64 sums), where the cut may move by one.
"""
import numpy as np
import pytest
import torch

from free_block_sparse_mean_amd import workloads as wl
from oracle import sol_oracle as orc
from tests import parity_utils as pu

pytestmark = pytest.mark.gpu

CASES = [
    wl.Workload("c1_small_f32", 1, 1, 4096, 64, "f32", "centroid"),
    wl.small("ragged_d128", 2, 3, 64 * 100, 128, grid=(4, 25, 64)),
    wl.small("ragged_d64", 1, 2, 64 * 70, 64, grid=(2, 35, 64)),
    wl.small("wide_d128", 1, 1, 64 * 1000, 128, grid=(10, 100, 64)),
]


def _route(w, gpu_lib, mode, **kw):
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    nb = w.n_blocks
    W = (nb + 63) // 64
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    gpu_lib.sol_block_summaries(kd, vd, ws)
    pm = torch.empty((w.B, w.H, nb, nb), dtype=torch.float32, device=qd.device)
    words = torch.zeros((w.B, w.H, nb, W), dtype=torch.int64, device=qd.device)
    kept = torch.full((w.B, w.H, nb), -1, dtype=torch.int32, device=qd.device)
    idx = None
    if mode == gpu_lib.SOL_ROUTE_TOPK:
        idx = torch.full((w.B, w.H, nb, max(1, kw["top_k"])), -1, dtype=torch.int32, device=qd.device)
    gpu_lib.sol_route(qd, mode, ws, pm, words, kept_per_row=kept, topk_idx=idx, **kw)
    torch.cuda.synchronize()
    mask = gpu_lib.decode_mask(words, nb).numpy()
    assert np.array_equal(kept.cpu().numpy(), mask.sum(-1))
    return q, k, pm.cpu().numpy().astype(np.float64), mask, None if idx is None else idx.cpu().numpy()


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_proxy_map(w, gpu_lib):
    q, k, pm, _, _ = _route(w, gpu_lib, gpu_lib.SOL_ROUTE_THRESHOLD, beta=1.0)
    for b in range(w.B):
        for h in range(w.H):
            qb = orc.block_means(q[b, h].float().numpy())
            kb = orc.block_means(k[b, h].float().numpy())
            ref = orc.proxy_scores(qb, kb)            # float64
            scale = np.abs(qb).max() * np.abs(kb).max() * w.d ** 0.5
            np.testing.assert_allclose(pm[b, h], ref, rtol=0, atol=1e-5 * scale)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("beta", [-0.5, 1.0, 2.0])
def test_threshold_from_map(w, beta, gpu_lib):
    _, _, pm, mask, _ = _route(w, gpu_lib, gpu_lib.SOL_ROUTE_THRESHOLD, beta=beta)
    for b in range(w.B):
        for h in range(w.H):
            mu, sd = orc.row_mean_std(pm[b, h])
            tau = orc.thresholds(mu, sd, beta)
            ref = orc.select_blocks(pm[b, h], tau)
            diff = ref != mask[b, h]
            if diff.any():
                gap = np.abs(pm[b, h] - tau[:, None])[diff]
                assert gap.max() <= pu.TIE_BAND


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("frac", [0.0, 0.15, 0.5, 1.2])
def test_topk_from_map(w, frac, gpu_lib):
    nb = w.n_blocks
    k = int(round(frac * nb))
    _, _, pm, mask, idx = _route(w, gpu_lib, gpu_lib.SOL_ROUTE_TOPK, top_k=k)
    kk = min(k, nb)
    for b in range(w.B):
        for h in range(w.H):
            ref = orc.select_topk(pm[b, h], k)
            assert np.array_equal(ref, mask[b, h])
            if kk:
                order = np.lexsort((np.arange(nb)[None, :].repeat(nb, 0), -pm[b, h]), axis=1)[:, :kk]
                assert np.array_equal(idx[b, h][:, :kk], order)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("p", [0.05, 0.5, 0.66, 0.95, 1.0])
def test_topp_from_map(w, p, gpu_lib):
    _, _, pm, mask, _ = _route(w, gpu_lib, gpu_lib.SOL_ROUTE_TOPP, top_p=p)
    nb = w.n_blocks
    for b in range(w.B):
        for h in range(w.H):
            ref = orc.select_topp(pm[b, h], p)
            for i in np.flatnonzero((ref != mask[b, h]).any(1)):
                row = pm[b, h, i]
                order = sorted(range(nb), key=lambda j: (-row[j], j))
                prob = np.exp(row - row.max())
                prob /= prob.sum()
                cum = np.cumsum(prob[order])
                m_ref, m_gpu = int(ref[i].sum()), int(mask[b, h, i].sum())
                assert abs(m_ref - m_gpu) == 1, (i, m_ref, m_gpu)
                edge = min(m_ref, m_gpu) - 1           # last position kept by both
                assert abs(cum[edge] - p) <= 1e-5
                kept = np.zeros(nb, dtype=bool)
                kept[order[:m_gpu]] = True
                assert np.array_equal(kept, mask[b, h, i])


def test_topk_masks_drive_block_sparse_attention(gpu_lib):
    """Top-k selection fed to the given-mask kernel: the oracle with the same mask agrees."""
    w = CASES[1]
    nb = w.n_blocks
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    gpu_lib.sol_block_summaries(kd, vd, ws)
    pm = torch.empty((w.B, w.H, nb, nb), dtype=torch.float32, device=qd.device)
    words = torch.zeros((w.B, w.H, nb, (nb + 63) // 64), dtype=torch.int64, device=qd.device)
    gpu_lib.sol_route(qd, gpu_lib.SOL_ROUTE_TOPK, ws, pm, words, top_k=15)
    out = torch.empty_like(qd)
    gpu_lib.sol_attn_masked(qd, kd, vd, out, words, 0, ws)
    torch.cuda.synchronize()
    mask = gpu_lib.decode_mask(words, nb).numpy()
    got = out.float().cpu().numpy()
    for b in range(w.B):
        for h in range(w.H):
            ref = orc.sol_attention_head(q[b, h].float().numpy(), k[b, h].float().numpy(),
                                         v[b, h].float().numpy(), 0.0, False,
                                         mask_override=mask[b, h])["out"]
            assert pu.rel_l2(got[b, h], ref) <= pu.BF16_REL_L2
            assert float(np.abs(got[b, h] - ref).max()) <= pu.BF16_MAX_ABS


@pytest.mark.parametrize("w", [CASES[1], CASES[3]], ids=lambda w: w.name)
def test_proxy_map_unaligned_output(w, gpu_lib):
    """A proxy map that starts 4 bytes past a 16-byte boundary takes the map kernel's
    element-wise stores instead of its 16-byte ones: the same map and masks, bit for bit."""
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    nb = w.n_blocks
    W = (nb + 63) // 64
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    gpu_lib.sol_block_summaries(kd, vd, ws)
    outs = []
    for shift in (0, 1):
        flat = torch.empty(w.B * w.H * nb * nb + 4, dtype=torch.float32, device=qd.device)
        pm = flat[shift:shift + w.B * w.H * nb * nb].view(w.B, w.H, nb, nb)
        assert (pm.data_ptr() % 16 == 0) == (shift == 0)
        words = torch.zeros((w.B, w.H, nb, W), dtype=torch.int64, device=qd.device)
        gpu_lib.sol_route(qd, gpu_lib.SOL_ROUTE_THRESHOLD, ws, pm, words, beta=1.0)
        torch.cuda.synchronize()
        outs.append((pm.clone(), words.clone()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
