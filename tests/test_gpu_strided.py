"""GPU checks of sol_attn_fwd_strided (tensors in other layouts than contiguous
[B][H][N][d]).

On [B, N, H, d] tensors and on slices of a packed [B, N, 3, H, d] projection,
the strided entry must give, bit for bit, the output and the row statistics
of sol_attn_fwd_ex on contiguous copies of the same logical tensors (whose
parity against the oracle the other GPU tests establish), and write nothing
outside its output rows. One case is also compared with the oracle directly.
"""
import numpy as np
import pytest
import torch

from free_block_sparse_mean_amd import workloads as wl
from tests import parity_utils as pu

pytestmark = pytest.mark.gpu

CASES = [
    wl.small("strided_d128", 2, 3, 64 * 70, 128, grid=(2, 35, 64)),
    wl.small("strided_d64", 1, 2, 64 * 40, 64, grid=(4, 10, 64)),
    wl.small("strided_f32", 1, 2, 64 * 33, 64, dtype="f32", grid=(3, 11, 64)),
]


def _flags(gpu_lib, kind):
    return {"corr": gpu_lib.SOL_CORRECTION, "none": 0, "dense": gpu_lib.SOL_DENSE | gpu_lib.SOL_CORRECTION,
            "row": gpu_lib.SOL_CORRECTION_ROW}[kind]


def _reference(gpu_lib, q, k, v, beta, flags):
    """sol_attn_fwd_ex on contiguous copies: output and kept blocks per row."""
    qc, kc, vc = q.contiguous(), k.contiguous(), v.contiguous()
    out = torch.empty_like(qc)
    B, H, N, _ = qc.shape
    kept = torch.full((B, H, N // 64), -1, dtype=torch.int32, device=qc.device)
    gpu_lib.sol_attn_fwd_ex(qc, kc, vc, out, beta, flags, kept_per_row=kept)
    return out, kept


def _views_bnhd(q, k, v):
    """[B, H, N, d] views of [B, N, H, d] storage holding the same values."""
    to = lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)
    return to(q), to(k), to(v)


def _views_packed(q, k, v):
    """[B, H, N, d] views of one packed [B, N, 3, H, d] projection."""
    B, H, N, d = q.shape
    qkv = torch.empty((B, N, 3, H, d), dtype=q.dtype, device=q.device)
    for i, x in enumerate((q, k, v)):
        qkv[:, :, i] = x.transpose(1, 2)
    return qkv[:, :, 0].transpose(1, 2), qkv[:, :, 1].transpose(1, 2), qkv[:, :, 2].transpose(1, 2)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("layout", ["bnhd", "packed"])
@pytest.mark.parametrize("kind", ["corr", "none", "dense", "row"])
def test_strided_equals_contiguous(w, layout, kind, gpu_lib):
    q, k, v = (x.cuda() for x in wl.make_qkv(w))
    B, H, N, d = q.shape
    beta = 1.0
    flags = _flags(gpu_lib, kind)
    qs, ks, vs = _views_bnhd(q, k, v) if layout == "bnhd" else _views_packed(q, k, v)
    # output rows inside a wider [B, N, H, d + 16] buffer: the pad must stay untouched
    buf = torch.full((B, N, H, d + 16), float("nan"), dtype=q.dtype, device=q.device)
    out = buf[..., :d].transpose(1, 2)
    kept = torch.full((B, H, N // 64), -1, dtype=torch.int32, device=q.device)
    gpu_lib.sol_attn_fwd_strided(qs, ks, vs, out, beta, flags, kept_per_row=kept)
    ref, kept_ref = _reference(gpu_lib, q, k, v, beta, flags)
    torch.cuda.synchronize()
    print(f"[strided] {w.name} {layout} {kind}", flush=True)
    assert torch.equal(out.contiguous(), ref), "strided output differs from the contiguous call"
    assert torch.equal(kept, kept_ref)
    assert torch.isnan(buf[..., d:].float()).all(), "wrote outside the output rows"


def test_strided_against_oracle(gpu_lib):
    """[B, N, H, d] inputs straight against the oracle (mask, tau and output)."""
    w = CASES[0]
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = _views_bnhd(q.cuda(), k.cuda(), v.cuda())
    B, H, N, d = q.shape
    nb = N // 64
    beta = 1.0
    out = torch.empty((B, N, H, d), dtype=q.dtype, device=qd.device).transpose(1, 2)
    mask = torch.zeros((B, H, nb, (nb + 63) // 64), dtype=torch.int64, device=qd.device)
    tau = torch.empty((B, H, nb), dtype=torch.float32, device=qd.device)
    gpu_lib.sol_attn_fwd_strided(qd, kd, vd, out, beta, gpu_lib.SOL_CORRECTION, mask_bits=mask, tau=tau)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    m = gpu_lib.decode_mask(mask, nb).numpy()
    t = tau.cpu().numpy()
    for b in range(B):
        for h in range(H):
            pu.check_head(q[b, h], k[b, h], v[b, h], got[b, h], m[b, h], t[b, h], beta, True, w.dtype,
                          label=f"strided b{b} h{h}")
