"""Seeded synthetic Q/K/V generators for the Sol-Attn workloads.

This module only draws inputs. It holds none of the attention method's
arithmetic, so both the CPU oracle (tests) and the HIP path (tests, bench)
can take their inputs from here without sharing any of the computation.

The pages measure the kernel on activations of video diffusion transformers
(Wan 2.1, HunyuanVideo 1.5, LTX 2.3) at up to 128K tokens and around 90%
sparsity (page "Sol-Attn: l'attenzione sparsa che sceglie al volo" on
paithon.it, sections "Perché l'attenzione pesa tanto nei video" and
"I numeri"). Those activations are not available, so the fields below stand
in for them: a smooth 3-D sinusoidal positional field over a T x H x W latent
grid (raster order, t major, then y, then x), a per-64-token-block centroid
shared by Q and K, and Gaussian noise.

Every tensor is returned on the host as a torch tensor of shape
[B, H, N, d] (bfloat16, rounded to nearest even from float32, or float32).
Heads are drawn from independent streams keyed by (seed, b, h), so one head
can be regenerated alone, bit for bit, without drawing the others.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator, Optional, Tuple

import numpy as np
import torch

BLOCK = 64  # tokens per block, fixed by the method


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic problem: shape, dtype, generator recipe and beta list."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                      # "bf16" or "f32"
    kind: str                       # "centroid" (config-1 recipe) or "field"
    grid: Optional[Tuple[int, int, int]] = None   # (T, Y, X) for "field"
    rotate: bool = False            # per-head Haar rotation applied to q and k
    skewed: bool = False            # half the query blocks concentrated, half diffuse
    betas: Tuple[float, ...] = (1.0,)
    seed: int = 0

    @property
    def n_blocks(self) -> int:
        return self.N // BLOCK


# The five synthetic configurations of the build plan (shapes and recipes).
CONFIGS = {
    "c1_small_f32": Workload("c1_small_f32", 1, 1, 4096, 64, "f32", "centroid",
                             betas=(1.0, -math.inf)),
    "c2_video_16k": Workload("c2_video_16k", 1, 24, 16384, 128, "bf16", "field",
                             grid=(16, 32, 32), betas=(0.5, 1.0, 1.5)),
    "c3_dit14b_77k": Workload("c3_dit14b_77k", 1, 40, 76800, 128, "bf16", "field",
                              grid=(20, 48, 80), rotate=True, betas=(1.0,)),
    "c4_stress_128k": Workload("c4_stress_128k", 1, 24, 131072, 128, "bf16", "field",
                               grid=(32, 64, 64), betas=(1.5, 2.0)),
    "c5_batched_skewed_64k": Workload("c5_batched_skewed_64k", 2, 24, 65536, 128, "bf16",
                                      "field", grid=(16, 64, 64), skewed=True,
                                      betas=(-0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 2.5)),
}


def _head_rng(seed: int, tag: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tag, b, h]))


def _field(grid: Tuple[int, int, int], d: int, seed: int) -> np.ndarray:
    """Smooth positional field F[n, c] = sin(2*pi*nu_c*p_a/L_a + phi_c), a = c mod 3.

    nu_c ~ U[0.5, 4) cycles over the axis extent, phi_c ~ U[0, 2*pi). Drawn once
    and shared by Q, K and every head.
    """
    T, Y, X = grid
    rng = _head_rng(seed, 1, 0, 0)
    nu = rng.uniform(0.5, 4.0, size=d)
    phi = rng.uniform(0.0, 2.0 * math.pi, size=d)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    coords = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)  # [N, 3]
    extent = np.array([T, Y, X], dtype=np.float64)
    axis = np.arange(d) % 3
    arg = 2.0 * math.pi * nu[None, :] * coords[:, axis] / extent[axis][None, :] + phi[None, :]
    return np.sin(arg).astype(np.float32)


def _haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-random orthogonal matrix: QR of a Gaussian with the signs of R's diagonal fixed."""
    a = rng.standard_normal((d, d))
    qm, r = np.linalg.qr(a)
    qm = qm * np.sign(np.diag(r))[None, :]
    return qm.astype(np.float32)


def head_qkv(w: Workload, b: int, h: int, field: Optional[np.ndarray] = None
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Draw one head's (q, k, v) as float32 arrays [N, d], before any dtype rounding."""
    N, d, nb = w.N, w.d, w.n_blocks
    rng = _head_rng(w.seed, 2, b, h)
    if w.kind == "centroid":
        c = rng.standard_normal((nb, d), dtype=np.float32)
        c2 = c + 0.3 * rng.standard_normal((nb, d), dtype=np.float32)
        cq = np.repeat(c, BLOCK, axis=0)
        ck = np.repeat(c2, BLOCK, axis=0)
        q = 0.8 * cq + 0.6 * rng.standard_normal((N, d), dtype=np.float32)
        k = 0.8 * ck + 0.6 * rng.standard_normal((N, d), dtype=np.float32)
        v = rng.standard_normal((N, d), dtype=np.float32)
        return q, k, v
    if w.kind != "field":
        raise ValueError(f"unknown workload kind {w.kind!r}")
    if field is None:
        field = _field(w.grid, d, w.seed)
    cent = rng.standard_normal((nb, d), dtype=np.float32)
    if w.skewed:
        # a seeded half of the query blocks is concentrated (scale 2.0), the rest diffuse (0.2)
        qscale = np.where(rng.permutation(nb) < nb // 2, 2.0, 0.2).astype(np.float32)
    else:
        qscale = np.full(nb, 0.5, dtype=np.float32)
    cq = np.repeat(cent * qscale[:, None], BLOCK, axis=0)
    ck = np.repeat(cent * 0.5, BLOCK, axis=0)
    q = field + cq + 0.5 * rng.standard_normal((N, d), dtype=np.float32)
    k = field + ck + 0.5 * rng.standard_normal((N, d), dtype=np.float32)
    v = rng.standard_normal((N, d), dtype=np.float32)
    if w.rotate:
        rot = _haar_orthogonal(rng, d)
        q = q @ rot
        k = k @ rot
    return q, k, v


def _to_torch(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def iter_heads(w: Workload) -> Iterator[Tuple[int, int, torch.Tensor, torch.Tensor, torch.Tensor]]:
    """Yield (b, h, q, k, v) per head as host tensors [N, d] in the workload dtype."""
    field = _field(w.grid, w.d, w.seed) if w.kind == "field" else None
    for b in range(w.B):
        for h in range(w.H):
            q, k, v = head_qkv(w, b, h, field)
            yield b, h, _to_torch(q, w.dtype), _to_torch(k, w.dtype), _to_torch(v, w.dtype)


def make_qkv(w: Workload, threads: int = 8) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """All heads as host tensors [B, H, N, d] in the workload dtype.

    Heads are drawn in parallel threads; each head has its own seeded stream,
    so the result does not depend on the thread count.
    """
    from concurrent.futures import ThreadPoolExecutor
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = torch.empty((w.B, w.H, w.N, w.d), dtype=tdt)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    field = _field(w.grid, w.d, w.seed) if w.kind == "field" else None

    def one(bh):
        b, h = divmod(bh, w.H)
        qh, kh, vh = head_qkv(w, b, h, field)
        q[b, h].copy_(_to_torch(qh, w.dtype))
        k[b, h].copy_(_to_torch(kh, w.dtype))
        v[b, h].copy_(_to_torch(vh, w.dtype))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(w.B * w.H)))
    return q, k, v


def make_head(w: Workload, b: int, h: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """One head as host tensors [N, d] in the workload dtype (same values as make_qkv)."""
    q, k, v = head_qkv(w, b, h)
    return _to_torch(q, w.dtype), _to_torch(k, w.dtype), _to_torch(v, w.dtype)


def small(name: str, B: int, H: int, N: int, d: int, dtype: str = "bf16",
          kind: str = "field", grid: Optional[Tuple[int, int, int]] = None,
          rotate: bool = False, skewed: bool = False, seed: int = 0) -> Workload:
    """A reduced workload with the same recipe, for parity tests the oracle finishes quickly."""
    if kind == "field" and grid is None:
        grid = (1, N // BLOCK, BLOCK)
    return Workload(name, B, H, N, d, dtype, kind, grid=grid, rotate=rotate,
                    skewed=skewed, seed=seed)
