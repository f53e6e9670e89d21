"""ctypes binding of libsolattn.so (the C ABI declared in include/sol_attn.h).

Argument marshalling only: every step of the attention runs in the HIP
kernels of the library. Tensors are torch tensors on a ROCm device, used for
device memory and streams. There is no fallback: if the library is missing
or fails, these functions raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsolattn.so")

SOL_OK = 0
SOL_ERR_INVALID_ARG = 1
SOL_ERR_UNSUPPORTED = 2
SOL_ERR_DEVICE = 3
SOL_ERR_NOMEM = 4
SOL_ERR_WORKSPACE = 5

SOL_BF16 = 0x0
SOL_F32 = 0x1
SOL_CORRECTION = 0x2
SOL_DENSE = 0x4
SOL_SYNC = 0x8
SOL_CORRECTION_ROW = 0x10
SOL_LOW_MEMORY = 0x20

SOL_ROUTE_THRESHOLD = 0
SOL_ROUTE_TOPK = 1
SOL_ROUTE_TOPP = 2

BLOCK = 64


class SolError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sol_attn status {status}: {message}")
        self.status = status


class sol_debug(ctypes.Structure):
    _fields_ = [("kept_per_row", ctypes.c_void_p),
                ("mask_bits", ctypes.c_void_p),
                ("tau", ctypes.c_void_p),
                ("item_clock", ctypes.c_void_p)]


class sol_strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class sol_workspace_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("total_bytes", "kbar_t", "kbar", "vsum", "kmean", "kcov", "vt", "qbar", "kbar_bf",
                  "vbar_t", "scratch", "vbar_bf")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsolattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m free_block_sparse_mean_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, u, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint, ctypes.c_size_t
    lib.sol_abi_version.argtypes = []
    lib.sol_abi_version.restype = i
    lib.sol_last_error.argtypes = []
    lib.sol_last_error.restype = ctypes.c_char_p
    lib.sol_attn_workspace_bytes.argtypes = [i, i, i, i]
    lib.sol_attn_workspace_bytes.restype = sz
    lib.sol_attn_workspace_bytes_flags.argtypes = [i, i, i, i, ctypes.c_uint]
    lib.sol_attn_workspace_bytes_flags.restype = sz
    lib.sol_attn_workspace_layout.argtypes = [i, i, i, i, ctypes.POINTER(sol_workspace_layout)]
    lib.sol_attn_workspace_layout.restype = i
    lib.sol_block_summaries.argtypes = [vp, vp, i, i, i, i, u, vp, sz, vp]
    lib.sol_block_summaries.restype = i
    lib.sol_attn_fused.argtypes = [vp, vp, vp, vp, i, i, i, i, f, u, vp, sz,
                                   ctypes.POINTER(sol_debug), vp]
    lib.sol_attn_fused.restype = i
    lib.sol_attn_fused_joint.argtypes = [vp, vp, vp, vp, i, i, i, i, f, u, i, vp, sz,
                                         ctypes.POINTER(sol_debug), vp]
    lib.sol_attn_fused_joint.restype = i
    lib.sol_route.argtypes = [vp, i, i, i, i, u, i, f, i, f, vp, sz, vp, vp, vp, vp, vp]
    lib.sol_route.restype = i
    lib.sol_attn_masked.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, u, vp, sz, vp, vp]
    lib.sol_attn_masked.restype = i
    lib.sol_attn_fwd_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, f, u, vp, vp, sz,
                                    ctypes.POINTER(sol_debug)]
    lib.sol_attn_fwd_ex.restype = i
    lib.sol_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, f, u]
    lib.sol_attn_fwd.restype = i
    lib.sol_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, f, u, vp, ctypes.POINTER(sol_debug)]
    lib.sol_attn_fwd_noalloc.restype = i
    sp = ctypes.POINTER(sol_strides)
    lib.sol_attn_fwd_strided.argtypes = [vp, vp, vp, vp, i, i, i, i, sp, sp, sp, sp, f, u, vp, vp, sz,
                                         ctypes.POINTER(sol_debug)]
    lib.sol_attn_fwd_strided.restype = i
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != SOL_OK:
        raise SolError(status, sol_last_error())


def sol_abi_version() -> int:
    return load_library().sol_abi_version()


def sol_last_error() -> str:
    return load_library().sol_last_error().decode()


def sol_attn_workspace_bytes(B: int, H: int, N: int, d: int, flags: int = 0) -> int:
    """Workspace bytes for the shape and the calls' flags (SOL_LOW_MEMORY: no V^T copy)."""
    return load_library().sol_attn_workspace_bytes_flags(B, H, N, d, flags)


def sol_attn_workspace_layout(B: int, H: int, N: int, d: int) -> sol_workspace_layout:
    lay = sol_workspace_layout()
    _check(load_library().sol_attn_workspace_layout(B, H, N, d, ctypes.byref(lay)))
    return lay


def _shape(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    return tuple(int(x) for x in q.shape)


def _same_as(q: torch.Tensor, **others: torch.Tensor) -> None:
    """Every named tensor has q's [B, H, N, d] shape, dtype and device."""
    for name, t in others.items():
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, q has {tuple(q.shape)}")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} is {t.dtype}, q is {q.dtype}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q is on {q.device}")


def _check_out(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, numel: int,
               device: torch.device) -> None:
    """An optional per-call output: dtype, element count, device and contiguity."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements (got {t.numel()})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_dbg(q: torch.Tensor, kept_per_row=None, mask_bits=None, tau=None, item_clock=None) -> None:
    B, H, N, _ = _shape(q)
    nb = N // BLOCK
    rows = B * H * nb
    _check_out(kept_per_row, "kept_per_row", torch.int32, rows, q.device)
    _check_out(mask_bits, "mask_bits", torch.int64, rows * ((nb + 63) // 64), q.device)
    _check_out(tau, "tau", torch.float32, rows, q.device)
    _check_out(item_clock, "item_clock", torch.int64, rows * 2, q.device)


def _dtype_flag(*ts: torch.Tensor) -> int:
    dts = {t.dtype for t in ts}
    if dts == {torch.bfloat16}:
        return SOL_BF16
    if dts == {torch.float32}:
        return SOL_F32
    raise ValueError(f"all tensors must be bfloat16 or all float32, got {dts}")


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")


def _ws_bytes(workspace: torch.Tensor) -> int:
    return workspace.numel() * workspace.element_size()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dbg(kept_per_row=None, mask_bits=None, tau=None, item_clock=None):
    if kept_per_row is None and mask_bits is None and tau is None and item_clock is None:
        return None
    ptr = lambda t: None if t is None else t.data_ptr()
    return ctypes.byref(sol_debug(ptr(kept_per_row), ptr(mask_bits), ptr(tau), ptr(item_clock)))


def new_workspace(B: int, H: int, N: int, d: int, device=None, flags: int = 0) -> torch.Tensor:
    """A uint8 device tensor of sol_attn_workspace_bytes bytes (for the calls' flags)."""
    n = sol_attn_workspace_bytes(B, H, N, d, flags)
    if n == 0:
        raise ValueError("invalid or unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def workspace_views(ws: torch.Tensor, B: int, H: int, N: int, d: int) -> Dict[str, torch.Tensor]:
    """Typed views of the pre-pass arrays inside a workspace tensor."""
    lay = sol_attn_workspace_layout(B, H, N, d)
    nb = N // BLOCK
    nbp = (nb + 3) // 4 * 4
    f32 = lambda off, shape: ws[off:off + 4 * math.prod(shape)].view(torch.float32).view(shape)
    views = {
        "kbar_t": f32(lay.kbar_t, (B, H, d, nbp))[..., :nb],
        "kbar": f32(lay.kbar, (B, H, nb, d)),
        "vsum": f32(lay.vsum, (B, H, nb, d)),
        "kmean": f32(lay.kmean, (B, H, d)),
        "kcov": f32(lay.kcov, (B, H, d, d)),
        "qbar": f32(lay.qbar, (B, H, nb, d)),
    }
    nw = (nb + 63) // 64
    bf = lambda off, shape: ws[off:off + 2 * math.prod(shape)].view(torch.bfloat16).view(shape)
    views["kbar_bf"] = bf(lay.kbar_bf, (B, H, nw, BLOCK, d))
    views["vbar_t"] = bf(lay.vbar_t, (B, H, nw, d, BLOCK))
    views["vbar_bf"] = bf(lay.vbar_bf, (B, H, nw, BLOCK, d))
    if ws.numel() >= lay.vt + 2 * B * H * N * d:   # not a low-memory workspace
        views["vt"] = ws[lay.vt:lay.vt + 2 * B * H * N * d].view(torch.bfloat16).view(B, H, nb, d, BLOCK)
    return views


def sol_block_summaries(k: torch.Tensor, v: torch.Tensor, workspace: torch.Tensor,
                        flags: int = 0, stream=None) -> None:
    B, H, N, d = _shape(k)
    _same_as(k, v=v)
    _dev(k, v, workspace)
    flags |= _dtype_flag(k, v)
    _check(load_library().sol_block_summaries(k.data_ptr(), v.data_ptr(), B, H, N, d, flags,
                                              workspace.data_ptr(), _ws_bytes(workspace),
                                              _stream(stream)))


def sol_attn_fused(q, k, v, out, beta: float, flags: int, workspace: torch.Tensor, *,
                   kept_per_row=None, mask_bits=None, tau=None, item_clock=None, stream=None,
                   text_blocks: int = 0) -> None:
    B, H, N, d = _shape(q)
    _same_as(q, k=k, v=v, out=out)
    _check_dbg(q, kept_per_row, mask_bits, tau, item_clock)
    _dev(q, k, v, out, workspace)
    flags |= _dtype_flag(q, k, v, out)
    if text_blocks:
        _check(load_library().sol_attn_fused_joint(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d, float(beta), flags,
            int(text_blocks), workspace.data_ptr(), _ws_bytes(workspace),
            _dbg(kept_per_row, mask_bits, tau, item_clock), _stream(stream)))
        return
    _check(load_library().sol_attn_fused(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         B, H, N, d, float(beta), flags, workspace.data_ptr(),
                                         _ws_bytes(workspace), _dbg(kept_per_row, mask_bits, tau, item_clock),
                                         _stream(stream)))


def sol_route(q, mode: int, workspace: torch.Tensor, proxy_map: torch.Tensor, mask_bits: torch.Tensor, *,
              beta: float = 0.0, top_k: int = 0, top_p: float = 0.0, kept_per_row=None, topk_idx=None,
              flags: int = 0, stream=None) -> None:
    """Routing baseline with a materialized proxy map (float32 [B, H, n_b, n_b]); mask words
    int64 [B, H, n_b, W] written; the workspace must hold the pre-pass of the same K."""
    B, H, N, d = _shape(q)
    nb = N // BLOCK
    if proxy_map.dtype != torch.float32 or proxy_map.numel() != B * H * nb * nb:
        raise ValueError("proxy_map must be float32 [B, H, n_b, n_b]")
    if mask_bits.dtype != torch.int64 or mask_bits.numel() != B * H * nb * ((nb + 63) // 64):
        raise ValueError("mask_bits must be int64 [B, H, n_b, ceil(n_b/64)]")
    _check_out(proxy_map, "proxy_map", torch.float32, B * H * nb * nb, q.device)
    _check_out(mask_bits, "mask_bits", torch.int64, B * H * nb * ((nb + 63) // 64), q.device)
    _check_out(kept_per_row, "kept_per_row", torch.int32, B * H * nb, q.device)
    if int(mode) == SOL_ROUTE_TOPK and topk_idx is not None:
        # rows of top_k entries (only min(top_k, n_b) of each written)
        if topk_idx.numel() < B * H * nb * max(int(top_k), 0):
            raise ValueError(f"topk_idx must hold B*H*n_b*top_k = {B * H * nb * max(int(top_k), 0)} entries")
        _check_out(topk_idx, "topk_idx", torch.int32, topk_idx.numel(), q.device)
    _dev(q, workspace, proxy_map, mask_bits)
    flags |= _dtype_flag(q)
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(load_library().sol_route(q.data_ptr(), B, H, N, d, flags, int(mode), float(beta), int(top_k),
                                    float(top_p), workspace.data_ptr(), _ws_bytes(workspace),
                                    proxy_map.data_ptr(), mask_bits.data_ptr(), ptr(kept_per_row),
                                    ptr(topk_idx), _stream(stream)))


def sol_attn_masked(q, k, v, out, mask_bits: torch.Tensor, flags: int, workspace: torch.Tensor, *,
                    kept_per_row=None, stream=None) -> None:
    """Block-sparse attention on a given selection (mask_bits: int64 [B, H, n_b, W] words)."""
    B, H, N, d = _shape(q)
    _same_as(q, k=k, v=v, out=out)
    if mask_bits.dtype != torch.int64 or mask_bits.numel() != B * H * (N // BLOCK) * ((N // BLOCK + 63) // 64):
        raise ValueError("mask_bits must be int64 [B, H, n_b, ceil(n_b/64)]")
    _check_dbg(q, kept_per_row=kept_per_row, mask_bits=mask_bits)
    _dev(q, k, v, out, mask_bits, workspace)
    flags |= _dtype_flag(q, k, v, out)
    _check(load_library().sol_attn_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                          B, H, N, d, mask_bits.data_ptr(), flags, workspace.data_ptr(),
                                          _ws_bytes(workspace),
                                          None if kept_per_row is None else kept_per_row.data_ptr(),
                                          _stream(stream)))


def sol_attn_fwd_ex(q, k, v, out, beta: float, flags: int, stream=None,
                    workspace: Optional[torch.Tensor] = None, *, kept_per_row=None,
                    mask_bits=None, tau=None, item_clock=None) -> None:
    B, H, N, d = _shape(q)
    _same_as(q, k=k, v=v, out=out)
    _check_dbg(q, kept_per_row, mask_bits, tau, item_clock)
    _dev(q, k, v, out)
    flags |= _dtype_flag(q, k, v, out)
    if workspace is None:
        workspace = new_workspace(B, H, N, d, q.device, flags)
    _dev(workspace)
    _check(load_library().sol_attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                          B, H, N, d, float(beta), flags, _stream(stream),
                                          workspace.data_ptr(), _ws_bytes(workspace),
                                          _dbg(kept_per_row, mask_bits, tau, item_clock)))


def sol_attn_fwd_noalloc(q, k, v, out, beta: float, flags: int, stream=None, *, kept_per_row=None,
                         mask_bits=None, tau=None, item_clock=None) -> None:
    """sol_attn_fwd_ex without a workspace: the library's static per-GPU scratch (64 MiB)
    holds the pre-pass arrays and nothing is allocated. Calls that may overlap on one GPU
    race on that scratch."""
    B, H, N, d = _shape(q)
    _same_as(q, k=k, v=v, out=out)
    _check_dbg(q, kept_per_row, mask_bits, tau, item_clock)
    _dev(q, k, v, out)
    flags |= _dtype_flag(q, k, v, out)
    _check(load_library().sol_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                               B, H, N, d, float(beta), flags, _stream(stream),
                                               _dbg(kept_per_row, mask_bits, tau, item_clock)))


def _strides(t: torch.Tensor):
    """sol_strides of a logical [B, H, N, d] view whose last dimension is contiguous."""
    if not t.is_cuda or t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("tensors must be [B, H, N, d] device views with contiguous rows of d")
    return ctypes.byref(sol_strides(t.stride(0), t.stride(1), t.stride(2)))


def sol_attn_fwd_strided(q, k, v, out, beta: float, flags: int, stream=None,
                         workspace: Optional[torch.Tensor] = None, *, kept_per_row=None,
                         mask_bits=None, tau=None, item_clock=None) -> None:
    """sol_attn_fwd_ex on [B, H, N, d] views of any strides (rows of d contiguous), e.g.
    x.transpose(1, 2) of a [B, N, H, d] tensor or slices of a packed QKV projection."""
    B, H, N, d = _shape(q)
    _same_as(q, k=k, v=v, out=out)
    _check_dbg(q, kept_per_row, mask_bits, tau, item_clock)
    sq, sk, sv, so = _strides(q), _strides(k), _strides(v), _strides(out)
    flags |= _dtype_flag(q, k, v, out)
    if workspace is None:
        workspace = new_workspace(B, H, N, d, q.device, flags)
    _check(load_library().sol_attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                               B, H, N, d, sq, sk, sv, so, float(beta), flags,
                                               _stream(stream), workspace.data_ptr(), _ws_bytes(workspace),
                                               _dbg(kept_per_row, mask_bits, tau, item_clock)))


def sol_attn_fwd(q, k, v, out, beta: float, flags: int) -> None:
    """The whole forward on the null stream with the library's own workspace. The null
    stream is made to wait for torch's current stream before the call, and the current
    stream to wait for the null stream after it, so the call is ordered like any other
    operation on the current stream (torch's side streams do not synchronise with the
    null stream by themselves)."""
    B, H, N, d = _shape(q)
    _same_as(q, k=k, v=v, out=out)
    _dev(q, k, v, out)
    flags |= _dtype_flag(q, k, v, out)
    cur = torch.cuda.current_stream(q.device)
    null = torch.cuda.default_stream(q.device)
    side = cur.cuda_stream != null.cuda_stream
    if side:
        null.wait_stream(cur)
    _check(load_library().sol_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       B, H, N, d, float(beta), flags))
    if side:
        cur.wait_stream(null)


def decode_mask(mask_bits: torch.Tensor, n_b: int) -> torch.Tensor:
    """[..., W] int64 words -> [..., n_b] bool (bit j%64 of word j//64)."""
    words = mask_bits.cpu()
    bits = torch.arange(64, dtype=torch.int64)
    m = ((words.unsqueeze(-1) >> bits) & 1).bool()
    return m.reshape(*words.shape[:-1], -1)[..., :n_b]
