"""Host-side checks of the Python binding (no GPU): every wrapper rejects
tensors whose shape, dtype or device does not match q before it reaches the
library, so a wrong-sized buffer becomes a ValueError, never an out-of-bounds
device access."""
import pytest
import torch

from free_block_sparse_mean_amd import binding as sb

B, H, N, d = 1, 2, 64 * 4, 64
NB = N // 64


def _qkv(dtype=torch.bfloat16):
    return [torch.zeros((B, H, N, d), dtype=dtype) for _ in range(4)]


def _ws():
    return torch.zeros(1 << 20, dtype=torch.uint8)


@pytest.mark.parametrize("bad", ["k", "v", "out"])
def test_io_shape_mismatch(bad):
    q, k, v, out = _qkv()
    t = {"k": k, "v": v, "out": out}
    t[bad] = torch.zeros((B, H, N - 64, d), dtype=torch.bfloat16)
    for call in (lambda: sb.sol_attn_fused(q, t["k"], t["v"], t["out"], 1.0, 0, _ws()),
                 lambda: sb.sol_attn_fwd_ex(q, t["k"], t["v"], t["out"], 1.0, 0, workspace=_ws()),
                 lambda: sb.sol_attn_fwd(q, t["k"], t["v"], t["out"], 1.0, 0),
                 lambda: sb.sol_attn_masked(q, t["k"], t["v"], t["out"],
                                            torch.zeros((B, H, NB, 1), dtype=torch.int64), 0, _ws()),
                 lambda: sb.sol_attn_fwd_strided(q, t["k"], t["v"], t["out"], 1.0, 0, workspace=_ws())):
        with pytest.raises(ValueError, match=bad):
            call()


def test_io_dtype_mismatch():
    q, k, v, out = _qkv()
    with pytest.raises(ValueError, match="v is"):
        sb.sol_attn_fused(q, k, v.float(), out, 1.0, 0, _ws())
    with pytest.raises(ValueError, match="v"):
        sb.sol_block_summaries(k, v.float(), _ws())
    with pytest.raises(ValueError, match="shape"):
        sb.sol_block_summaries(k, v[:, :1], _ws())


@pytest.mark.parametrize("name,bad", [
    ("kept_per_row", torch.zeros(B * H * NB - 1, dtype=torch.int32)),
    ("kept_per_row", torch.zeros(B * H * NB, dtype=torch.int64)),
    ("mask_bits", torch.zeros(B * H * NB, dtype=torch.int32)),
    ("mask_bits", torch.zeros(B * H * NB + 1, dtype=torch.int64)),
    ("tau", torch.zeros(B * H * NB, dtype=torch.float64)),
    ("tau", torch.zeros(B * H * NB * 2, dtype=torch.float32)),
    ("item_clock", torch.zeros(B * H * NB, dtype=torch.int64)),
])
def test_debug_outputs_checked(name, bad):
    q, k, v, out = _qkv()
    for call in (lambda: sb.sol_attn_fused(q, k, v, out, 1.0, 0, _ws(), **{name: bad}),
                 lambda: sb.sol_attn_fwd_ex(q, k, v, out, 1.0, 0, workspace=_ws(), **{name: bad}),
                 lambda: sb.sol_attn_fwd_strided(q, k, v, out, 1.0, 0, workspace=_ws(), **{name: bad})):
        with pytest.raises(ValueError, match=name):
            call()


def test_masked_outputs_checked():
    q, k, v, out = _qkv()
    words = torch.zeros((B, H, NB, 1), dtype=torch.int64)
    with pytest.raises(ValueError, match="mask_bits"):
        sb.sol_attn_masked(q, k, v, out, words[:, :, :-1], 0, _ws())
    with pytest.raises(ValueError, match="kept_per_row"):
        sb.sol_attn_masked(q, k, v, out, words, 0, _ws(), kept_per_row=torch.zeros(3, dtype=torch.int32))


def test_route_outputs_checked():
    q = _qkv()[0]
    pm = torch.zeros((B, H, NB, NB), dtype=torch.float32)
    words = torch.zeros((B, H, NB, 1), dtype=torch.int64)
    with pytest.raises(ValueError, match="kept_per_row"):
        sb.sol_route(q, sb.SOL_ROUTE_THRESHOLD, _ws(), pm, words, beta=1.0,
                     kept_per_row=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="topk_idx"):
        sb.sol_route(q, sb.SOL_ROUTE_TOPK, _ws(), pm, words, top_k=3,
                     topk_idx=torch.zeros(B * H * NB * 2, dtype=torch.int32))


def test_host_tensors_rejected():
    """Well-shaped tensors that are not on a GPU are refused before any library call."""
    q, k, v, out = _qkv()
    with pytest.raises(ValueError, match="device"):
        sb.sol_attn_fused(q, k, v, out, 1.0, 0, _ws())
    with pytest.raises(ValueError, match="device"):
        sb.sol_block_summaries(k, v, _ws())
