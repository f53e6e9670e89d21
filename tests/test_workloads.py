"""The seeded input generators (free_block_sparse_mean_amd/workloads.py), which feed
both the oracle and the HIP path: reproducible, independent of threading, one
stream per head, and with the structure each recipe states."""
import numpy as np
import torch

from free_block_sparse_mean_amd import workloads as wl


def _small(**kw):
    base = dict(name="t", B=2, H=3, N=64 * 12, d=64, grid=(2, 6, 64))
    base.update(kw)
    return wl.small(base.pop("name"), base.pop("B"), base.pop("H"), base.pop("N"), base.pop("d"), **base)


def test_make_qkv_independent_of_thread_count():
    w = _small()
    a = wl.make_qkv(w, threads=1)
    b = wl.make_qkv(w, threads=6)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_entry_points_agree():
    w = _small(dtype="f32")
    q, k, v = wl.make_qkv(w)
    for b, h, qh, kh, vh in wl.iter_heads(w):
        assert torch.equal(qh, q[b, h]) and torch.equal(kh, k[b, h]) and torch.equal(vh, v[b, h])
        mq, mk, mv = wl.make_head(w, b, h)
        assert torch.equal(mq, qh) and torch.equal(mk, kh) and torch.equal(mv, vh)


def test_heads_and_seeds_differ():
    w = _small(dtype="f32")
    q, _, v = wl.make_qkv(w)
    assert not torch.equal(q[0, 0], q[0, 1]) and not torch.equal(q[0, 0], q[1, 0])
    assert not torch.equal(v[0, 0], v[1, 2])
    w2 = _small(dtype="f32", seed=1)
    q2, _, _ = wl.make_qkv(w2)
    assert not torch.equal(q, q2)


def test_bf16_is_the_rounded_f32_draw():
    qf, kf, vf = wl.make_qkv(_small(dtype="f32"))
    qb, kb, vb = wl.make_qkv(_small(dtype="bf16"))
    assert torch.equal(qf.to(torch.bfloat16), qb) and torch.equal(vf.to(torch.bfloat16), vb)


def test_rotation_preserves_query_key_products():
    """rotate=True applies one orthogonal matrix to q and k of a head (drawn after them),
    so every q . k product, and the values, match the unrotated draw."""
    plain = _small(dtype="f32", B=1, H=2)
    rot = _small(dtype="f32", B=1, H=2, rotate=True)
    for h in range(2):
        q0, k0, v0 = (x.numpy().astype(np.float64) for x in wl.make_head(plain, 0, h))
        q1, k1, v1 = (x.numpy().astype(np.float64) for x in wl.make_head(rot, 0, h))
        assert np.array_equal(v0, v1)
        assert not np.allclose(q0, q1)
        s0, s1 = q0 @ k0.T, q1 @ k1.T
        assert np.abs(s0 - s1).max() <= 1e-4 * np.abs(s0).max()


def test_skewed_query_scales():
    """skewed: half of the query blocks carry their block centre at scale 2.0, the rest at
    0.2, so the block-mean query norms split into two well separated groups."""
    w = wl.small("sk", 1, 1, 64 * 64, 64, dtype="f32", kind="field",
                 grid=(4, 16, 64), skewed=True)
    q, _, _ = wl.make_head(w, 0, 0)
    qbar = q.numpy().reshape(64, 64, 64).mean(axis=1)
    field = wl._field(w.grid, w.d, w.seed).reshape(64, 64, 64).mean(axis=1)
    norms = np.linalg.norm(qbar - field, axis=1)
    lo, hi = np.sort(norms)[:32], np.sort(norms)[32:]
    assert hi.min() > 3 * lo.max()
