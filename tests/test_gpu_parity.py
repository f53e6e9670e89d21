"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: selection masks bit-exact except ties within 1e-4 of tau_i; outputs
within rel-L2 1e-2 and max-abs 2e-2 for bf16 inputs (1e-5 / 1e-4 for float32).
Small problems are compared on every row; they span several 64-block ballot
words, ragged tails (n_b not a multiple of 64 or 4) and both head dims.
"""
import math

import numpy as np
import pytest
import torch

from free_block_sparse_mean_amd import workloads as wl
from tests import parity_utils as pu

pytestmark = pytest.mark.gpu

BF, F32 = "bf16", "f32"


def _case(w, beta, correction, gpu_lib, flags_extra=0, label=""):
    q, k, v = wl.make_qkv(w)
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    flags = (gpu_lib.SOL_CORRECTION if correction else 0) | flags_extra
    r = pu.run_gpu(qd, kd, vd, beta, flags, gpu_lib)
    eff_beta = -math.inf if flags_extra & gpu_lib.SOL_DENSE else beta
    nb = w.n_blocks
    # stats are consistent with the mask
    assert torch.equal(r["kept"], r["mask"].sum(-1).to(torch.int32))
    assert torch.isfinite(r["out"]).all()
    stats = []
    for b in range(w.B):
        for h in range(w.H):
            stats.append(pu.check_head(q[b, h], k[b, h], v[b, h], r["out"][b, h].numpy(),
                                       r["mask"][b, h].numpy(), r["tau"][b, h].numpy(),
                                       eff_beta, correction, w.dtype,
                                       label=f"{label or w.name} b{b} h{h} beta={beta}"))
    return r, stats


SMALL = [
    wl.Workload("c1_small_f32", 1, 1, 4096, 64, F32, "centroid"),
    wl.small("ragged_d128", 2, 3, 64 * 100, 128, grid=(4, 25, 64)),
    wl.small("ragged_d64", 1, 2, 64 * 70, 64, grid=(2, 35, 64)),
    wl.Workload("centroid_bf16", 1, 2, 64 * 90, 128, BF, "centroid"),
    wl.small("rotated", 1, 2, 64 * 80, 128, grid=(2, 40, 64), rotate=True),
    wl.small("skewed", 1, 2, 64 * 130, 128, grid=(2, 65, 64), skewed=True),
    wl.small("f32_d128", 1, 2, 64 * 40, 128, dtype=F32, grid=(2, 20, 64)),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("beta", [-0.5, 0.5, 1.0, 2.0])
@pytest.mark.parametrize("correction", [True, False], ids=["corr", "nocorr"])
def test_small_parity(w, beta, correction, gpu_lib):
    print(f"case {w.name} beta={beta} corr={correction}", flush=True)
    _case(w, beta, correction, gpu_lib)


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[2]], ids=lambda w: w.name)
@pytest.mark.parametrize("correction", [True, False], ids=["corr", "nocorr"])
def test_dense_limit(w, correction, gpu_lib):
    """beta = -inf and the SOL_DENSE flag both keep every block: dense attention."""
    print(f"case dense {w.name} corr={correction}", flush=True)
    r1, _ = _case(w, -math.inf, correction, gpu_lib)
    assert r1["mask"].all()
    r2, _ = _case(w, 1.0, correction, gpu_lib, flags_extra=gpu_lib.SOL_DENSE)
    assert torch.equal(r1["out"], r2["out"])
    # and against the textbook dense routine directly
    q, k, v = wl.make_qkv(w)
    from oracle import sol_oracle as orc
    for b in range(w.B):
        ref = orc.dense_attention(q[b, 0].float().numpy(), k[b, 0].float().numpy(), v[b, 0].float().numpy())
        got = r1["out"][b, 0].numpy()
        tol = (pu.BF16_REL_L2, pu.BF16_MAX_ABS) if w.dtype == BF else (pu.F32_REL_L2, pu.F32_MAX_ABS)
        assert pu.rel_l2(got, ref) <= tol[0] and np.abs(got - ref).max() <= tol[1]


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1]], ids=lambda w: w.name)
@pytest.mark.parametrize("correction", [True, False], ids=["corr", "nocorr"])
def test_keep_none(w, correction, gpu_lib):
    """beta = +inf keeps no block: pooled attention with the correction, zeros without."""
    print(f"case keep-none {w.name} corr={correction}", flush=True)
    r, _ = _case(w, math.inf, correction, gpu_lib)
    assert not r["mask"].any()
    assert (r["kept"] == 0).all()
    if not correction:
        assert not r["out"].any()


@pytest.mark.parametrize("N", [64, 128, 192, 64 * 65])
@pytest.mark.parametrize("d", [64, 128])
def test_tiny_and_word_edges(N, d, gpu_lib):
    """n_b = 1, 2, 3 and 65 (one block past a full 64-block mask word)."""
    w = wl.small(f"edge_{N}_{d}", 1, 2, N, d, grid=(1, N // 64, 64))
    for beta in (0.0, 1.0):
        for corr in (True, False):
            print(f"case edge N={N} d={d} beta={beta} corr={corr}", flush=True)
            _case(w, beta, corr, gpu_lib)


def test_identical_keys_sigma_zero(gpu_lib):
    """All key blocks equal: sigma_i = 0, every score ties with tau; the GPU may take
    either side, and its output must match the oracle run on its own mask."""
    torch.manual_seed(0)
    B, H, N, d = 1, 1, 64 * 20, 128
    q = torch.randn(B, H, N, d).to(torch.bfloat16)
    k = torch.randn(1, 1, 64, d).repeat(1, 1, N // 64, 1).to(torch.bfloat16)
    v = torch.randn(B, H, N, d).to(torch.bfloat16)
    dev = torch.device("cuda")
    for corr in (True, False):
        r = pu.run_gpu(q.to(dev), k.to(dev), v.to(dev), 0.5, gpu_lib.SOL_CORRECTION if corr else 0, gpu_lib)
        pu.check_head(q[0, 0], k[0, 0], v[0, 0], r["out"][0, 0].numpy(), r["mask"][0, 0].numpy(),
                      r["tau"][0, 0].numpy(), 0.5, corr, BF, label=f"identical keys corr={corr}")


def test_deterministic_and_stream(gpu_lib):
    """Two calls give bit-identical results, on a side stream and through sol_attn_fwd."""
    w = SMALL[1]
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    flags = gpu_lib.SOL_CORRECTION
    a = pu.run_gpu(q, k, v, 1.0, flags, gpu_lib)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = pu.run_gpu(q, k, v, 1.0, flags, gpu_lib, stream=s)
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["mask"], b["mask"])
    out = torch.empty_like(q)
    gpu_lib.sol_attn_fwd(q, k, v, out, 1.0, flags)
    torch.cuda.synchronize()
    assert torch.equal(out.float().cpu(), a["out"])


def test_concurrent_fused_shared_workspace(gpu_lib):
    """Fused calls on several streams at once, of two head dims (two kernel instantiations),
    each group sharing one pre-pass workspace (which the fused pass only reads), give bit for
    bit the result of the same call alone: every launch deals its queued work items from a
    counter of its own."""
    cases = []
    for d in (128, 64):
        w = wl.small(f"concurrent_d{d}", 1, 8, 64 * 256, d, grid=(4, 64, 64))
        q, k, v = (t.cuda() for t in wl.make_qkv(w))
        ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
        gpu_lib.sol_block_summaries(k, v, ws)
        for i in range(3):   # other queries, same keys and workspace
            cases.append((torch.roll(q, shifts=64 * i, dims=2).contiguous(), k, v, ws))
    flags = gpu_lib.SOL_CORRECTION
    ref = []
    for qi, k, v, ws in cases:
        o = torch.empty_like(qi)
        gpu_lib.sol_attn_fused(qi, k, v, o, 1.0, flags, ws)
        ref.append(o)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [[torch.empty_like(c[0]) for c in cases] for _ in range(3)]
    torch.cuda.synchronize()
    for rep in range(3):
        for i, ((qi, k, v, ws), st) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(st):
                gpu_lib.sol_attn_fused(qi, k, v, outs[rep][i], 1.0, flags, ws, stream=st)
    torch.cuda.synchronize()
    print(f"[concurrent] {len(cases)} streams x 3 launches", flush=True)
    for rep in range(3):
        for i in range(len(cases)):
            assert torch.equal(outs[rep][i], ref[i]), f"stream {i}, launch {rep}"


def test_graph_capture_replays(gpu_lib):
    """The pre-pass and the fused pass captured in a HIP graph (its work-item queue counter
    is cleared by a kernel, not a memset) replay bit for bit the eager result, several times,
    with eager work and synchronisations between the replays."""
    w = SMALL[1]
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    flags = gpu_lib.SOL_CORRECTION
    ref = torch.empty_like(q)
    gpu_lib.sol_block_summaries(k, v, ws)
    gpu_lib.sol_attn_fused(q, k, v, ref, 1.0, flags, ws)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            gpu_lib.sol_block_summaries(k, v, ws, stream=side)
            gpu_lib.sol_attn_fused(q, k, v, out, 1.0, flags, ws, stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        scratch = torch.empty_like(q)
        gpu_lib.sol_attn_fused(q, k, v, scratch, 0.5, flags, ws)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        assert torch.equal(out, ref), f"replay {rep}"


# The moment kernels sum key-block chunks of 128, 64 or 32 blocks (smaller when B*H*n_b is
# small): the small cases take chunks of 32 (several per head), this one chunks of 64.
CHUNK64 = wl.small("chunk64_d64", 1, 16, 65536, 64, grid=(16, 64, 64))


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[2], CHUNK64], ids=lambda w: w.name)
def test_prepass_summaries(w, gpu_lib):
    """k_bar, v sums, m and C of the pre-pass against the oracle's float64 block means."""
    from oracle import sol_oracle as orc
    q, k, v = wl.make_qkv(w)
    kd, vd = k.cuda(), v.cuda()
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    gpu_lib.sol_block_summaries(kd, vd, ws)
    torch.cuda.synchronize()
    raw = gpu_lib.workspace_views(ws, w.B, w.H, w.N, w.d)
    if w.dtype == BF:
        # each 64 x d block of V transposed, bit for bit, keys in the documented order
        c = torch.arange(64)
        g, sl = (c % 32) // 8, c % 8
        key = 32 * (c // 32) + torch.where(sl < 4, 4 * g + sl, 16 + 4 * g + sl - 4)
        assert sorted(key.tolist()) == list(range(64))
        vt_ref = v.view(w.B, w.H, w.n_blocks, 64, w.d).transpose(-1, -2)[..., key]
        assert torch.equal(raw["vt"].cpu(), vt_ref)
    views = {n: t.cpu().double().numpy() for n, t in raw.items() if n != "vt"}
    for b in range(w.B):
        for h in range(w.H):
            kbar = orc.block_means(k[b, h].float().numpy())
            vbar = orc.block_means(v[b, h].float().numpy())
            m, C = orc.key_summary_moments(kbar)
            sc = np.abs(kbar).max()
            np.testing.assert_allclose(views["kbar"][b, h], kbar, rtol=0, atol=1e-6 * sc)
            np.testing.assert_allclose(views["kbar_t"][b, h], kbar.T, rtol=0, atol=1e-6 * sc)
            np.testing.assert_allclose(views["vsum"][b, h], 64 * vbar, rtol=0, atol=64e-6 * np.abs(vbar).max())
            np.testing.assert_allclose(views["kmean"][b, h], m, rtol=0, atol=1e-6 * sc)
            np.testing.assert_allclose(views["kcov"][b, h], C, rtol=0, atol=1e-5 * np.abs(C).max())


TILE_CASES = [SMALL[1], SMALL[2], SMALL[5], CHUNK64,
              wl.small("tiles_d128_65", 1, 3, 64 * 65, 128, grid=(1, 65, 64))]


@pytest.mark.parametrize("lm", [False, True], ids=["default", "low_memory"])
@pytest.mark.parametrize("w", TILE_CASES, ids=lambda w: w.name)
def test_prepass_summary_tiles(w, lm, gpu_lib):
    """The bf16 summary tiles (block correction, per-row correction) bit for bit: k_bar and
    v_bar = vsum / 64 of the workspace's own fp32 summaries rounded to bf16, 64 key blocks per
    tile, v_bar^T columns in the V^T key order, rows and columns past n_b zero; the row-major
    v_bar tiles in the low-memory mode. The workspace is filled with a sentinel first, so any
    entry the pre-pass leaves unwritten shows."""
    flags = gpu_lib.SOL_LOW_MEMORY if lm else 0
    q, k, v = wl.make_qkv(w)
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d, flags=flags)
    ws.fill_(0x7F)
    gpu_lib.sol_block_summaries(k.cuda(), v.cuda(), ws, flags)
    torch.cuda.synchronize()
    raw = {n: t.cpu() for n, t in gpu_lib.workspace_views(ws, w.B, w.H, w.N, w.d).items()}
    nb = w.n_blocks
    nw = (nb + 63) // 64
    pad = lambda x: torch.nn.functional.pad(x, (0, 0, 0, 64 * nw - nb))
    kb = pad(raw["kbar"]).to(torch.bfloat16).view(w.B, w.H, nw, 64, w.d)
    vb = pad(raw["vsum"] / 64).to(torch.bfloat16).view(w.B, w.H, nw, 64, w.d)
    c = torch.arange(64)
    g, sl = (c % 32) // 8, c % 8
    key = 32 * (c // 32) + torch.where(sl < 4, 4 * g + sl, 16 + 4 * g + sl - 4)
    assert torch.equal(raw["kbar_bf"], kb)
    assert torch.equal(raw["vbar_t"], vb.transpose(-1, -2)[..., key])
    if lm:
        assert torch.equal(raw["vbar_bf"], vb)


def test_item_clock_export(gpu_lib):
    """The optional work-item clock: one (start, end) pair per workgroup, at the entry of its
    first query block; workgroups take G consecutive blocks; other entries untouched."""
    w = SMALL[1]
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    nb = w.n_blocks
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    out = torch.empty_like(q)
    clk = torch.zeros((w.B * w.H * nb, 2), dtype=torch.int64, device=q.device)
    gpu_lib.sol_block_summaries(k, v, ws)
    gpu_lib.sol_attn_fused(q, k, v, out, 1.0, gpu_lib.SOL_CORRECTION, ws, item_clock=clk)
    torch.cuda.synchronize()
    c = clk.cpu().view(w.B * w.H, nb, 2)
    set_ = c[..., 0] != 0
    starts = torch.nonzero(set_[0]).flatten().tolist()
    G = starts[1] - starts[0] if len(starts) > 1 else nb
    assert 1 <= G <= 4 and starts == list(range(0, nb, G))
    assert bool((set_ == set_[0]).all())                      # the same pattern in every head
    assert bool((c[..., 1][set_] >= c[..., 0][set_]).all())
    assert bool((c[..., 1][~set_] == 0).all())


def _encode_mask(mask: np.ndarray, pad_bits: bool) -> torch.Tensor:
    """bool [..., n_b] -> int64 words [..., W]; bits past n_b set when pad_bits (to be ignored)."""
    nb = mask.shape[-1]
    W = (nb + 63) // 64
    full = np.zeros(mask.shape[:-1] + (W * 64,), dtype=bool)
    full[..., :nb] = mask
    if pad_bits:
        full[..., nb:] = True
    words = np.packbits(full.reshape(-1, W, 64), axis=-1, bitorder="little").view(np.int64)
    return torch.from_numpy(words.reshape(mask.shape[:-1] + (W,)).copy())


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[2], SMALL[6]], ids=lambda w: w.name)
def test_masked_parity(w, gpu_lib):
    """Given-mask block-sparse mode against the oracle run with the same mask (no correction);
    rows with no kept block give zeros; bits past n_b are ignored."""
    print(f"case masked {w.name}", flush=True)
    q, k, v = wl.make_qkv(w)
    nb = w.n_blocks
    rng = np.random.default_rng(7)
    mask = rng.random((w.B, w.H, nb, nb)) < 0.2
    mask[:, :, 1, :] = False                                   # an empty row
    mask[:, :, 2, :] = True                                    # a dense row
    words = _encode_mask(mask, pad_bits=True).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    gpu_lib.sol_block_summaries(kd, vd, ws)
    out = torch.empty_like(qd)
    kept = torch.full((w.B, w.H, nb), -1, dtype=torch.int32, device=qd.device)
    gpu_lib.sol_attn_masked(qd, kd, vd, out, words, 0, ws, kept_per_row=kept)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), torch.from_numpy(mask.sum(-1).astype(np.int32)))
    got = out.float().cpu().numpy()
    rel_tol, abs_tol = (pu.BF16_REL_L2, pu.BF16_MAX_ABS) if w.dtype == BF else (pu.F32_REL_L2, pu.F32_MAX_ABS)
    from oracle import sol_oracle as orc
    for b in range(w.B):
        for h in range(w.H):
            ref = orc.sol_attention_head(q[b, h].float().numpy(), k[b, h].float().numpy(),
                                         v[b, h].float().numpy(), 0.0, False,
                                         mask_override=mask[b, h])["out"]
            g = got[b, h]
            assert np.all(g[64:128] == 0.0)
            r, a = pu.rel_l2(g, ref), float(np.abs(g - ref).max())
            assert r <= rel_tol and a <= abs_tol, f"{w.name} b{b} h{h}: rel-L2 {r:.3e} max-abs {a:.3e}"


def test_masked_equals_fused_without_correction(gpu_lib):
    """On the routing's own selection the given-mask mode is the fused pass without the
    correction, bit for bit."""
    w = SMALL[1]
    q, k, v = (t.cuda() for t in wl.make_qkv(w))
    nb = w.n_blocks
    W = (nb + 63) // 64
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    gpu_lib.sol_block_summaries(k, v, ws)
    a = torch.empty_like(q)
    words = torch.zeros((w.B, w.H, nb, W), dtype=torch.int64, device=q.device)
    gpu_lib.sol_attn_fused(q, k, v, a, 1.0, 0, ws, mask_bits=words)
    b = torch.empty_like(q)
    gpu_lib.sol_attn_masked(q, k, v, b, words, 0, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("beta", [0.5, 2.0, math.inf])
def test_row_correction_parity(w, beta, gpu_lib):
    """SOL_CORRECTION_ROW against the oracle's per-row correction form (same mask)."""
    print(f"case row-correction {w.name} beta={beta}", flush=True)
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    r = pu.run_gpu(qd, kd, vd, beta, gpu_lib.SOL_CORRECTION_ROW, gpu_lib)
    assert torch.isfinite(r["out"]).all()
    for b in range(w.B):
        for h in range(w.H):
            pu.check_head(q[b, h], k[b, h], v[b, h], r["out"][b, h].numpy(), r["mask"][b, h].numpy(),
                          r["tau"][b, h].numpy(), beta, True, w.dtype,
                          label=f"{w.name} b{b} h{h} beta={beta} row", correction_form="row")


@pytest.mark.parametrize("dtype", [BF, F32])
def test_row_correction_exact_for_constant_key_blocks(dtype, gpu_lib):
    """Constant key blocks: the per-row correction reproduces dense attention at any beta."""
    rng = np.random.default_rng(11)
    nb, d = 70, 64
    q = rng.standard_normal((1, 1, nb * 64, d)).astype(np.float32)
    k = np.repeat(rng.standard_normal((1, 1, nb, d)).astype(np.float32), 64, axis=2)
    v = rng.standard_normal((1, 1, nb * 64, d)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == BF else torch.float32
    qt, kt, vt = (torch.from_numpy(x).to(tdt) for x in (q, k, v))
    from oracle import sol_oracle as orc
    dense = orc.dense_attention(qt[0, 0].float().numpy(), kt[0, 0].float().numpy(), vt[0, 0].float().numpy())
    for beta in (0.0, 1.5):
        r = pu.run_gpu(qt.cuda(), kt.cuda(), vt.cuda(), beta, gpu_lib.SOL_CORRECTION_ROW, gpu_lib)
        got = r["out"][0, 0].numpy()
        rel, mab = (pu.BF16_REL_L2, pu.BF16_MAX_ABS) if dtype == BF else (pu.F32_REL_L2, pu.F32_MAX_ABS)
        m = r["mask"][0, 0].numpy()
        assert 0 < m.sum() < nb * nb
        # rows that keep key block 31 and leave some of blocks 32..63 to the
        # correction: the two 32-bit halves of a 64-bit exclusion word both matter
        assert (m[:, 31] & ~m[:, 32:64].all(1)).any()
        assert pu.rel_l2(got, dense) <= rel and float(np.abs(got - dense).max()) <= mab


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[5]], ids=lambda w: w.name)
@pytest.mark.parametrize("flags_name", ["SOL_CORRECTION", "SOL_CORRECTION_ROW", None])
def test_joint_text_segment(w, flags_name, gpu_lib):
    """Joint attention: the last T blocks are text, always exact (kept columns, dense rows)."""
    print(f"case joint {w.name} {flags_name}", flush=True)
    T = 3
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    nb = w.n_blocks
    W = (nb + 63) // 64
    flags = getattr(gpu_lib, flags_name) if flags_name else 0
    ws = gpu_lib.new_workspace(w.B, w.H, w.N, w.d)
    out = torch.empty_like(qd)
    mask = torch.zeros((w.B, w.H, nb, W), dtype=torch.int64, device=qd.device)
    tau = torch.empty((w.B, w.H, nb), dtype=torch.float32, device=qd.device)
    gpu_lib.sol_block_summaries(kd, vd, ws)
    gpu_lib.sol_attn_fused(qd, kd, vd, out, 1.5, flags, ws, mask_bits=mask, tau=tau, text_blocks=T)
    torch.cuda.synchronize()
    m = gpu_lib.decode_mask(mask, nb).numpy()
    assert m[..., nb - T:].all() and m[:, :, nb - T:, :].all()
    got = out.float().cpu().numpy()
    rel, mab = (pu.BF16_REL_L2, pu.BF16_MAX_ABS) if w.dtype == BF else (pu.F32_REL_L2, pu.F32_MAX_ABS)
    from oracle import sol_oracle as orc
    form = "row" if flags_name == "SOL_CORRECTION_ROW" else "block"
    for b in range(w.B):
        for h in range(w.H):
            r = orc.sol_attention_head(q[b, h].float().numpy(), k[b, h].float().numpy(),
                                       v[b, h].float().numpy(), 1.5, flags != 0, mask_override=m[b, h],
                                       correction_form=form, text_blocks=T)
            assert pu.rel_l2(got[b, h], r["out"]) <= rel
            assert float(np.abs(got[b, h] - r["out"]).max()) <= mab
            diff = r["mask"] != m[b, h]
            if diff.any():
                assert np.abs(r["s_hat"] - r["tau"][:, None])[diff].max() <= pu.TIE_BAND
