"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle, compare.

The oracle (oracle/sol_oracle.py) and the HIP library share no code; only the
seeded inputs of free_block_sparse_mean_amd.workloads feed both.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Sequence

import numpy as np
import torch

from oracle import sol_oracle as orc

BLK = 64
TIE_BAND = 1e-4            # |s_hat - tau| within which either side of the test is accepted
BF16_REL_L2 = 1e-2         # bf16 inputs: tolerance fixed for the method's outputs
BF16_MAX_ABS = 2e-2
# float32 inputs: the kernel keeps every step in fp32; rounding of sums of up to
# N = 4096 terms and of exp2 gives errors around 1e-6 relative; the bound leaves
# a 10x margin (derivation in the design notes).
F32_REL_L2 = 1e-5
F32_MAX_ABS = 1e-4


def run_gpu(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: float, flags: int,
            binding, stream=None) -> Dict[str, torch.Tensor]:
    """One sol_attn_fwd_ex call with stats; returns host tensors."""
    B, H, N, d = q.shape
    nb = N // BLK
    W = (nb + 63) // 64
    dev = q.device
    out = torch.empty_like(q)
    kept = torch.full((B, H, nb), -1, dtype=torch.int32, device=dev)
    mask = torch.zeros((B, H, nb, W), dtype=torch.int64, device=dev)
    tau = torch.empty((B, H, nb), dtype=torch.float32, device=dev)
    binding.sol_attn_fwd_ex(q, k, v, out, beta, flags, stream=stream,
                            kept_per_row=kept, mask_bits=mask, tau=tau)
    torch.cuda.synchronize()
    return {"out": out.float().cpu(), "kept": kept.cpu(), "mask": binding.decode_mask(mask, nb),
            "tau": tau.cpu()}


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (den if den > 0 else 1.0)


def check_head(qh, kh, vh, gpu_out_h: np.ndarray, gpu_mask_h: np.ndarray, gpu_tau_h: np.ndarray,
               beta: float, correction: bool, dtype: str,
               query_blocks: Optional[Sequence[int]] = None, label: str = "",
               correction_form: str = "block") -> Dict[str, float]:
    """Compare one head of the HIP result with the oracle.

    qh, kh, vh: host tensors [N, d] (bf16 or f32) - the exact values the GPU read.
    gpu_out_h: [N, d] float; gpu_mask_h: [n_b, n_b] bool; gpu_tau_h: [n_b].
    Checks (1) the mask is bit-exact except for ties |s_hat - tau| <= TIE_BAND,
    (2) arithmetic: output vs the oracle run with the GPU's own mask,
    (3) end to end: output vs the oracle with its own mask (when no tie flipped).
    """
    q = qh.float().numpy()
    k = kh.float().numpy()
    v = vh.float().numpy()
    nb = q.shape[0] // BLK
    qb = np.arange(nb) if query_blocks is None else np.asarray(query_blocks)
    ref = orc.sol_attention_head(q, k, v, beta, correction, query_blocks=qb,
                                 correction_form=correction_form)
    gmask = gpu_mask_h[qb]
    diff = ref["mask"] != gmask
    n_flip = int(diff.sum())
    if n_flip:
        gap = np.abs(ref["s_hat"] - ref["tau"][:, None])[diff]
        assert gap.max() <= TIE_BAND, (
            f"{label}: {n_flip} mask differences, largest |s_hat - tau| = {gap.max():.3e} > {TIE_BAND}")
    # tau itself agrees with the brute-force tau (finite rows)
    fin = np.isfinite(ref["tau"])
    if fin.any():
        assert np.allclose(gpu_tau_h[qb][fin], ref["tau"][fin], rtol=0, atol=TIE_BAND), label
    rows = (qb[:, None] * BLK + np.arange(BLK)[None, :]).ravel()
    got = gpu_out_h[rows]
    rel_tol, abs_tol = (BF16_REL_L2, BF16_MAX_ABS) if dtype == "bf16" else (F32_REL_L2, F32_MAX_ABS)
    arith = orc.sol_attention_head(q, k, v, beta, correction, query_blocks=qb, mask_override=gmask,
                                   correction_form=correction_form)
    r1, a1 = rel_l2(got, arith["out"]), float(np.abs(got - arith["out"]).max())
    assert r1 <= rel_tol and a1 <= abs_tol, f"{label}: arithmetic rel-L2 {r1:.3e}, max-abs {a1:.3e}"
    res = {"rel_l2_arith": r1, "max_abs_arith": a1, "flips": n_flip,
           "density": float(gmask.mean())}
    if n_flip == 0:
        r2, a2 = rel_l2(got, ref["out"]), float(np.abs(got - ref["out"]).max())
        assert r2 <= rel_tol and a2 <= abs_tol, f"{label}: end-to-end rel-L2 {r2:.3e}, max-abs {a2:.3e}"
        res.update(rel_l2=r2, max_abs=a2)
    return res


def check_routing_head(qh, kh, gpu_mask_h: np.ndarray, gpu_tau_h: np.ndarray, beta: float,
                       label: str = "") -> Dict[str, float]:
    """Selection of every query block of one head against the oracle's routing steps."""
    q = qh.float().numpy()
    k = kh.float().numpy()
    kbar = orc.block_means(k).astype(np.float32)
    qbar = orc.block_means(q).astype(np.float32)
    s_hat = orc.proxy_scores(qbar, kbar)
    mu, sd = orc.row_mean_std(s_hat)
    tau = orc.thresholds(mu, sd, beta)
    mask = orc.select_blocks(s_hat, tau)
    diff = mask != gpu_mask_h
    n_flip = int(diff.sum())
    if n_flip:
        gap = np.abs(s_hat - tau[:, None])[diff]
        assert gap.max() <= TIE_BAND, (
            f"{label}: {n_flip} mask differences, largest |s_hat - tau| = {gap.max():.3e}")
    fin = np.isfinite(tau)
    if fin.any():
        err = np.abs(gpu_tau_h[fin] - tau[fin]).max()
        assert err <= TIE_BAND, f"{label}: tau differs by {err:.3e}"
    return {"flips": n_flip, "density": float(gpu_mask_h.mean())}
