#!/usr/bin/env python3
"""Benchmark of the Sol-Attn forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the block-summary pre-pass (sol_block_summaries) followed by the fused
route + exact sparse attention + correction pass (sol_attn_fused), the same
work as one sol_attn_fwd_ex call. Inputs are resident in HBM before the timed
region starts.

Workload (default): B=1, H=24, N=131072 (2048 blocks of 64), d=128, bf16,
synthetic video-latent field on a 32x64x64 grid; headline beta=1.5 with the
correction; beta=2.0 and the dense path (every block kept) are timed too.

Prints ONE JSON line. `value` is dense-equivalent TFLOP/s of the headline
step (4*B*H*N^2*d / step time); per-beta ms and TFLOP/s are in `per_beta`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "sparse-attn fwd ms + dense-equiv TFLOP/s at seq 128K, H24 d128 bf16, per β"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fused_c4_pmc.json")
FUSED_SRC = os.path.join(ROOT, "free_block_sparse_mean_amd", "csrc", "fused.hip")


def dense_equiv_flop(w) -> float:
    return 4.0 * w.B * w.H * float(w.N) ** 2 * w.d


def kept_flop(w, kept_blocks: int) -> float:
    """MFMA work the method must do: 4 * 64 * 64 * d per kept (query block, key block) tile."""
    return 4.0 * 64 * 64 * w.d * kept_blocks


def source_hash(path: str) -> str:
    """Hash of a source file's code: comments and whitespace do not count, so a
    counter summary stays valid across edits that leave the compiled kernel as it was."""
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
    text = re.sub(r"//[^\n]*", " ", text)                 # line comments
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per fused launch from the committed rocprofv3 counter summary, or None
    if there is none or the fused kernel source changed since it was taken."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    s = json.load(open(PMC_SUMMARY))
    if s.get("fused_src_sha256_16") != source_hash(FUSED_SRC):
        return None
    return s.get("hbm_bytes_per_launch")


def time_steps(fn_pre, fn_fused, steps: int):
    """Time `steps` steps on the current stream; returns (ms/step, mean fused ms, prepass ms,
    wall s, fused ms of each step)."""
    import torch
    st = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1 = ev(), ev()
    pa, pb, fa, fb = ([ev() for _ in range(steps)] for _ in range(4))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(st)
    for i in range(steps):
        pa[i].record(st)
        fn_pre()
        pb[i].record(st)
        fa[i].record(st)
        fn_fused()
        fb[i].record(st)
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    fused_each = [fa[i].elapsed_time(fb[i]) for i in range(steps)]
    pre = sum(pa[i].elapsed_time(pb[i]) for i in range(steps)) / steps
    return ms, sum(fused_each) / steps, pre, wall, fused_each


def time_flushed(fn_pre, fn_fused, reps: int, flush=None):
    """Time `reps` steps one at a time, each after `flush` (if given) has evicted the
    inputs from the Infinity Cache; returns (median step ms, median fused ms, median
    pre-pass ms, fused ms of each step)."""
    import torch
    st = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    steps, fused, pre = [], [], []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b, c = ev(), ev(), ev()
        a.record(st)
        fn_pre()
        b.record(st)
        fn_fused()
        c.record(st)
        torch.cuda.synchronize()
        steps.append(a.elapsed_time(c))
        pre.append(a.elapsed_time(b))
        fused.append(b.elapsed_time(c))
    return statistics.median(steps), statistics.median(fused), statistics.median(pre), fused


SWEEP_BETAS = {"c4_stress_128k": (1.2816, 1.5, 1.645, 2.0)}


def dense_rows(qs, k, v):
    """Textbook softmax attention of the query rows qs [r, d] over every key of one head,
    float64 on the host (the reference of the error report)."""
    import torch
    qs, k, v = (torch.as_tensor(x, dtype=torch.float64) for x in (qs, k, v))
    z = (qs @ k.T) / math.sqrt(qs.shape[1])
    z = z - z.max(dim=1, keepdim=True).values
    e = torch.exp(z)
    return ((e @ v) / e.sum(dim=1, keepdim=True)).numpy()


def config_sweep(name: str, reps: int, error_report: bool = False) -> dict:
    """Timing of every beta a configuration lists (with the correction, and without it for
    the batched skewed config) and of the dense path; inputs smaller than twice the
    Infinity Cache are flushed before each step by writing a 512 MiB buffer. With
    error_report: rel-L2 and max-abs of the output against dense attention on sampled rows
    (two heads, four seeded query blocks each), for every beta with the per-row
    correction, the block correction and none."""
    import numpy as np
    import torch
    from free_block_sparse_mean_amd import binding as sb, workloads as wl
    dev = torch.device("cuda:0")
    w = wl.CONFIGS[name]
    t_gen = time.perf_counter()
    q, k, v = wl.make_qkv(w)
    t_gen = time.perf_counter() - t_gen
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    ws = sb.new_workspace(w.B, w.H, w.N, w.d, dev)
    nb = w.n_blocks
    kept = torch.zeros((w.B, w.H, nb), dtype=torch.int32, device=dev)
    in_bytes = 3 * qd.numel() * qd.element_size()
    flush = None
    if in_bytes < 2 * 256 * 2 ** 20:
        junk = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        flush = lambda: junk.fill_(1)
    pre = lambda: sb.sol_block_summaries(kd, vd, ws)

    def one(beta, flags):
        sb.sol_block_summaries(kd, vd, ws)
        sb.sol_attn_fused(qd, kd, vd, out, beta, flags, ws, kept_per_row=kept)
        torch.cuda.synchronize()
        n_kept = int(kept.sum().item())
        fused = lambda: sb.sol_attn_fused(qd, kd, vd, out, beta, flags, ws)
        pre(); fused()
        ms, fms, pms, each = time_flushed(pre, fused, reps, flush)
        kf = kept_flop(w, n_kept)
        return {"beta": beta if math.isfinite(beta) else str(beta),
                "correction": bool(flags & (sb.SOL_CORRECTION | sb.SOL_CORRECTION_ROW)),
                "ms": ms, "fused_ms": fms,
                "prepass_ms": pms, "fused_ms_min": min(each),
                "density": n_kept / (w.B * w.H * nb * nb),
                "dense_equiv_tflops": dense_equiv_flop(w) / (ms * 1e-3) / 1e12,
                "kept_tflops_fused": kf / (fms * 1e-3) / 1e12,
                "mfma_frac_fused": kf / (fms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}

    rows = []
    betas = SWEEP_BETAS.get(name, w.betas)
    corr_opts = (sb.SOL_CORRECTION, 0) if w.skewed else (sb.SOL_CORRECTION,)
    for beta in betas:
        for c in corr_opts:
            rows.append(one(beta, c))
    dense = one(-math.inf, sb.SOL_CORRECTION | sb.SOL_DENSE)
    for r in rows:
        r["speedup_vs_dense"] = dense["ms"] / r["ms"]
    res = {"config": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "input_gen_s": t_gen,
           "flushed": flush is not None, "reps": reps, "settings": rows, "dense": dense}
    if error_report:
        heads = [(0, 0), (w.B - 1, w.H - 1)]
        rng = np.random.default_rng(5)
        picks = {bh: np.sort(rng.choice(nb, size=4, replace=False)) for bh in heads}
        idx = {bh: np.concatenate([np.arange(i * 64, (i + 1) * 64) for i in picks[bh]]) for bh in heads}
        ref = np.concatenate([dense_rows(q[b, h][idx[(b, h)]].float().numpy(), k[b, h].float().numpy(),
                                         v[b, h].float().numpy()) for (b, h) in heads])
        table = []
        for beta in w.betas:
            row = {"beta": beta}
            for tag, flags in (("row_correction", sb.SOL_CORRECTION_ROW), ("correction", sb.SOL_CORRECTION),
                               ("none", 0)):
                sb.sol_attn_fwd_ex(qd, kd, vd, out, beta, flags, workspace=ws, kept_per_row=kept)
                torch.cuda.synchronize()
                got = np.concatenate([out[b, h][torch.as_tensor(idx[(b, h)], device=dev)].float().cpu().numpy()
                                      for (b, h) in heads])
                row["density"] = int(kept.sum().item()) / (w.B * w.H * nb * nb)
                row[tag] = {"rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                            "max_abs": float(np.abs(got - ref).max())}
            table.append(row)
        res["error_vs_dense"] = {"rows": f"query blocks {', '.join(f'b{b}h{h}:{list(map(int, picks[(b, h)]))}' for (b, h) in heads)}",
                                 "reference": "float64 softmax attention over every key (host)", "table": table}
    del qd, kd, vd, out, ws, kept
    torch.cuda.empty_cache()
    return res


def progress(msg: str) -> None:
    """A progress line on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sweep(names, reps: int) -> int:
    """One JSON line per configuration (config_sweep)."""
    for name in names:
        print(json.dumps(config_sweep(name, reps)), flush=True)
    return 0


def calibrate_density(sb, qd, kd, vd, out, ws, w, kept, target: float, flags: int) -> float:
    """beta at which the kernel's realised density is closest to `target`: bisection on the
    kept counts of the fused pass (monotone in beta)."""
    import torch
    nb = w.n_blocks
    lo, hi = 0.0, 4.0

    def density(beta):
        sb.sol_attn_fused(qd, kd, vd, out, beta, flags, ws, kept_per_row=kept)
        torch.cuda.synchronize()
        return int(kept.sum().item()) / (w.B * w.H * nb * nb)

    sb.sol_block_summaries(kd, vd, ws)
    for _ in range(14):
        mid = 0.5 * (lo + hi)
        if density(mid) > target:
            lo = mid
        else:
            hi = mid
    return lo if abs(density(lo) - target) <= abs(density(hi) - target) else hi


def prepass_report(w, pre_ms: float) -> dict:
    """Bandwidth of the block-summary pre-pass (all its kernels). Algorithmic bytes:
    one read of K and V. Moved bytes add what it writes for the fused pass: the bf16
    V^T copy (bf16 inputs) and the fp32 k_bar (row-major and transposed) and v sums."""
    el = 2 if w.dtype == "bf16" else 4
    n_b = w.N // 64
    algo = 2.0 * w.B * w.H * w.N * w.d * el
    moved = algo + (w.B * w.H * w.N * w.d * 2 if w.dtype == "bf16" else 0) + 3.0 * w.B * w.H * n_b * w.d * 4
    sec = pre_ms * 1e-3
    return {"ms": pre_ms, "algorithmic_bytes": algo, "moved_bytes": moved,
            "hbm_gbs": algo / sec / 1e9, "frac": algo / sec / 1e9 / PEAK_HBM_GBS,
            "moved_gbs": moved / sec / 1e9, "frac_moved": moved / sec / 1e9 / PEAK_HBM_GBS}


def cpu_baseline(w, q, k, v, beta: float, blocks_per_head: int, heads):
    """The oracle, untuned, on a bounded sample: `blocks_per_head` seeded query blocks of
    each listed head, on one host thread (numpy's BLAS limited to one thread, so `cores`
    is exactly what it used; the oracle itself is a single Python loop over query
    blocks). Returns the dense-equivalent TFLOP/s of the sampled rows."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import sol_oracle as orc
    rng = np.random.default_rng(1234)
    nb = w.N // 64
    per_block = 4.0 * 64 * w.N * w.d
    arrays = [(q[0, h].float().numpy(), k[0, h].float().numpy(), v[0, h].float().numpy()) for h in heads]
    picks = [np.sort(rng.choice(nb, size=blocks_per_head, replace=False)) for _ in heads]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for (qh, kh, vh), qb in zip(arrays, picks):
            orc.sol_attention_head(qh, kh, vh, beta, True, query_blocks=qb)
        el = time.perf_counter() - t0
    n_blocks = blocks_per_head * len(heads)
    tflops = n_blocks * per_block / el / 1e12
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count() or 1
    return {
        "value": tflops, "unit": "TFLOP/s (dense-equivalent)", "cores": 1, "kind": "oracle",
        "threads_used": 1, "host_cores_nproc": nproc, "host_cpu_count": os.cpu_count(),
        "cpu_model": cpu_model(),
        "sample": (f"{blocks_per_head} seeded query blocks x {len(heads)} heads of the "
                   f"{w.name} workload (B={w.B}, H={w.H}, N={w.N}, d={w.d}), beta={beta}, "
                   f"correction on: {n_blocks} of {w.B * w.H * nb} query blocks, one host thread"),
        "seconds": el,
        "extrapolated_full_s": el * (w.B * w.H * nb) / n_blocks,
    }


def row_stats(kept) -> dict:
    """Kept key blocks per query block (row of blocks) of the last stats call: histogram in
    bins of 8, max/mean, p99/mean and coefficient of variation."""
    import numpy as np
    x = kept.flatten().cpu().numpy().astype(np.float64)
    mean = float(x.mean())
    hist, edges = np.histogram(x, bins=np.arange(0, x.max() + 9, 8))
    return {"mean": mean, "max_over_mean": float(x.max() / mean) if mean else None,
            "p99_over_mean": float(np.percentile(x, 99) / mean) if mean else None,
            "cv": float(x.std() / mean) if mean else None, "min": int(x.min()), "max": int(x.max()),
            "hist_bin": 8, "hist": hist.tolist()}


def load_balance(sb, qd, kd, vd, out, ws, beta, flags, w) -> dict:
    """One untimed fused call that records each workgroup's start and end on the device's
    100 MHz clock: spread (max - min) / mean of the per-work-item busy times."""
    import numpy as np
    import torch
    nb = w.n_blocks
    clk = torch.zeros((w.B * w.H * nb, 2), dtype=torch.int64, device=qd.device)
    sb.sol_block_summaries(kd, vd, ws)
    sb.sol_attn_fused(qd, kd, vd, out, beta, flags, ws, item_clock=clk)
    torch.cuda.synchronize()
    c = clk.cpu().numpy()
    c = c[c[:, 0] != 0].astype(np.float64)
    busy = (c[:, 1] - c[:, 0]) * 0.01   # microseconds
    span = (c[:, 1].max() - c[:, 0].min()) * 0.01
    m = float(busy.mean())
    return {"work_items": int(len(busy)), "busy_us_mean": m, "busy_us_min": float(busy.min()),
            "busy_us_max": float(busy.max()), "spread": float((busy.max() - busy.min()) / m),
            "p99_over_mean": float(np.percentile(busy, 99) / m), "launch_span_us": float(span)}


def routing_overhead(sb, qd, kd, vd, out, ws, beta, w, steps) -> dict:
    """Kernel-time ablation at one beta: the fused pass with and without the correction
    against plain block-sparse attention on the routing's own mask (sol_attn_masked: no
    routing, no correction), and the separate path the fused pass replaces: threshold
    routing from a materialized proxy map (sol_route) followed by block-sparse attention
    on that map's mask. Pre-pass done beforehand, untimed."""
    import torch
    nb = w.n_blocks
    W = (nb + 63) // 64
    words = torch.zeros((w.B, w.H, nb, W), dtype=torch.int64, device=qd.device)
    sb.sol_block_summaries(kd, vd, ws)
    sb.sol_attn_fused(qd, kd, vd, out, beta, 0, ws, mask_bits=words)
    torch.cuda.synchronize()

    def timed(fn):
        fn()
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev)

    masked = timed(lambda: sb.sol_attn_masked(qd, kd, vd, out, words, 0, ws))
    nocorr = timed(lambda: sb.sol_attn_fused(qd, kd, vd, out, beta, 0, ws))
    withcorr = timed(lambda: sb.sol_attn_fused(qd, kd, vd, out, beta, sb.SOL_CORRECTION, ws))
    pm = torch.empty((w.B, w.H, nb, nb), dtype=torch.float32, device=qd.device)
    map_words = torch.zeros_like(words)
    route = timed(lambda: sb.sol_route(qd, sb.SOL_ROUTE_THRESHOLD, ws, pm, map_words, beta=beta))
    masked_map = timed(lambda: sb.sol_attn_masked(qd, kd, vd, out, map_words, 0, ws))
    same = int((map_words != words).sum().item())
    del pm
    return {"beta": beta, "reps": steps, "given_mask_ms": masked, "fused_no_correction_ms": nocorr,
            "fused_ms": withcorr, "routing_overhead": nocorr / masked - 1.0,
            "routing_and_correction_overhead": withcorr / masked - 1.0,
            "separate_path": {"map_routing_ms": route, "block_sparse_on_map_mask_ms": masked_map,
                              "total_ms": route + masked_map, "mask_words_differing_from_fused": same},
            "fused_vs_separate": withcorr / (route + masked_map),
            "fused_no_correction_vs_separate": nocorr / (route + masked_map)}


def routing_study(sb, qd, kd, vd, out, ws, w, steps) -> dict:
    """Routing cost and per-row budget at about 15% mean density (the pages' ablation
    point): the fused pass's in-pass threshold routing (beta = +inf, no correction: the
    proxy scan and test with no exact tile) against the baselines that materialize the
    proxy map (sol_route: threshold from the map, top-k, top-p). beta, k and p are
    chosen for 15% mean density on this workload (calibrated offline with the oracle's
    selection rules on three heads)."""
    import numpy as np
    import torch
    nb = w.n_blocks
    W = (nb + 63) // 64
    dev = qd.device
    pm = torch.empty((w.B, w.H, nb, nb), dtype=torch.float32, device=dev)
    words = torch.zeros((w.B, w.H, nb, W), dtype=torch.int64, device=dev)
    kept = torch.zeros((w.B, w.H, nb), dtype=torch.int32, device=dev)
    sb.sol_block_summaries(kd, vd, ws)
    torch.cuda.synchronize()

    def timed(fn):
        fn()
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev)

    def spread():
        x = kept.flatten().cpu().numpy().astype(np.float64) / nb
        m = float(x.mean())
        return {"mean_density": m, "row_cv": float(x.std() / m) if m else None,
                "row_min_over_mean": float(x.min() / m) if m else None,
                "row_max_over_mean": float(x.max() / m) if m else None,
                "row_p99_over_mean": float(np.percentile(x, 99) / m) if m else None}

    res = {"proxy_map_bytes": 4 * w.B * w.H * nb * nb, "reps": steps}
    fused_route = timed(lambda: sb.sol_attn_fused(qd, kd, vd, out, math.inf, 0, ws))
    res["fused_threshold_routing_ms"] = fused_route
    sb.sol_attn_fused(qd, kd, vd, out, 1.1, 0, ws, kept_per_row=kept)
    torch.cuda.synchronize()
    res["fused_threshold"] = dict(beta=1.1, **spread())
    k = int(round(0.15 * nb))
    for name, kw in (("threshold_map", dict(beta=1.1)), ("top_k", dict(top_k=k)), ("top_p", dict(top_p=0.66))):
        mode = {"threshold_map": sb.SOL_ROUTE_THRESHOLD, "top_k": sb.SOL_ROUTE_TOPK, "top_p": sb.SOL_ROUTE_TOPP}[name]
        ms = timed(lambda: sb.sol_route(qd, mode, ws, pm, words, **kw))
        sb.sol_route(qd, mode, ws, pm, words, kept_per_row=kept, **kw)
        torch.cuda.synchronize()
        res[name] = dict(routing_ms=ms, **kw, **spread())
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def dense_reference(q, k, v, w, reps: int):
    """Dense softmax attention over the same tensors by PyTorch's own
    scaled_dot_product_attention, restricted to its flash backend (it raises instead of
    falling back to the N^2 math path): context for the dense-path ratios, not part of the
    library. Returns the error text when the backend is unavailable."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    kernel = "torch.nn.functional.scaled_dot_product_attention, flash backend"
    st = torch.cuda.current_stream()
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v)   # untimed
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                o = torch.nn.functional.scaled_dot_product_attention(q, k, v)
                b.record(st)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
        del o
    except Exception as e:   # context only: never let it end the benchmark
        return {"kernel": kernel, "torch": torch.__version__, "error": f"{type(e).__name__}: {str(e)[:300]}"}
    flop = 4.0 * w.B * w.H * w.N * w.N * w.d
    return {"kernel": kernel, "torch": torch.__version__, "reps": reps, "ms": statistics.median(ts),
            "ms_min": min(ts), "tflops": flop / (min(ts) * 1e-3) / 1e12,
            "frac_of_peak": flop / (min(ts) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def tile_mix(iters: int) -> int:
    """The tile loop's instruction mix alone (csrc/tile_mix.hip): per step of 16 bf16 MFMAs
    (v_mfma_f32_16x16x32_bf16, 16384 flop each), 0 to 16 LDS operand reads, 24 FMAs and 8
    exponentials, with 1 or 2 waves per SIMD on every CU, each launch timed with HIP events.
    Reports the MFMA rate, its fraction of the 2.5 PFLOP/s bf16 peak and of the pure-MFMA
    mix's rate at two waves per SIMD."""
    import ctypes
    from free_block_sparse_mean_amd import build as _b
    if not os.path.exists(_b.MIX_LIB):
        print(f"{_b.MIX_LIB} is not built (python -m free_block_sparse_mean_amd.build)", file=sys.stderr)
        return 2
    lib = ctypes.CDLL(_b.MIX_LIB)
    lib.sol_tile_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_int)]
    lib.sol_tile_mix_shape.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int)] * 3
    rows = []
    for wps in (2, 1):
        for mix in range(6):
            shape = [ctypes.c_int() for _ in range(3)]
            if lib.sol_tile_mix_shape(mix, *[ctypes.byref(x) for x in shape]) != 0:
                break
            ms, cus = ctypes.c_double(), ctypes.c_int()
            rc = lib.sol_tile_mix(mix, wps, iters, ctypes.byref(ms), ctypes.byref(cus))
            if rc != 0:
                print(f"sol_tile_mix(mix {mix}, {wps} waves per SIMD) failed: {rc}", file=sys.stderr)
                return 1
            mfmas = cus.value * 4 * wps * iters * 16
            tflops = mfmas * 16384.0 / (ms.value * 1e-3) / 1e12
            rows.append({"mix": mix, "waves_per_simd": wps, "lds_reads": shape[0].value,
                         "fmas": shape[1].value, "exps": shape[2].value, "mfmas_per_step": 16,
                         "ms": ms.value, "tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS})
    pure = next(r["tflops"] for r in rows if r["mix"] == 0 and r["waves_per_simd"] == 2)
    for r in rows:
        r["of_pure_mfma_rate"] = r["tflops"] / pure
    print(json.dumps({"tile_mix": rows, "steps_per_wave": iters, "cus": cus.value}))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4_stress_128k")
    ap.add_argument("--beta", type=float, default=1.5, help="headline beta")
    ap.add_argument("--extra-betas", default="1.645,2.0", help="comma list, '' for none")
    ap.add_argument("--no-dense", action="store_true", help="skip timing the dense path")
    ap.add_argument("--no-correction", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-routing-study", action="store_true")
    ap.add_argument("--no-dense-reference", action="store_true",
                    help="skip timing PyTorch's flash-backend dense attention on the same tensors")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the beta calibrated to 5%% density (it runs the fused pass at many betas)")
    ap.add_argument("--cpu-blocks-per-head", type=int, default=96)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy 5 times (for counter scaling)")
    ap.add_argument("--configs", default="c2_video_16k,c3_dit14b_77k,c5_batched_skewed_64k",
                    help="other configurations timed in the default run ('' for none)")
    ap.add_argument("--config-reps", type=int, default=5)
    ap.add_argument("--tile-mix", action="store_true",
                    help="only run the issue-rate microbenchmark of the tile loop's instruction mix "
                         "(libsoltilemix.so) and print one JSON line")
    ap.add_argument("--sweep", default="",
                    help="comma list of bf16 configs to time at every beta they list (one JSON "
                         "line each) instead of the headline benchmark")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2

    if args.sweep:
        return sweep([x for x in args.sweep.split(",") if x], max(3, args.steps))

    if args.tile_mix:
        return tile_mix(20000)

    if args.copy_calibration:
        n = 512 * 2 ** 20
        x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return 0

    from free_block_sparse_mean_amd import binding as sb, workloads as wl

    w = wl.CONFIGS[args.workload]
    t_gen = time.perf_counter()
    q, k, v = wl.make_qkv(w)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    ws = sb.new_workspace(w.B, w.H, w.N, w.d, dev)
    nb = w.n_blocks
    kept = torch.zeros((w.B, w.H, nb), dtype=torch.int32, device=dev)
    corr = 0 if args.no_correction else sb.SOL_CORRECTION
    torch.cuda.synchronize()

    def stepper(beta, flags):
        pre = lambda: sb.sol_block_summaries(kd, vd, ws, flags)
        fused = lambda: sb.sol_attn_fused(qd, kd, vd, out, beta, flags, ws)
        return pre, fused

    def measure(beta, flags, steps, warmup):
        # untimed call with stats: kept blocks (the algorithmic work) of this setting
        sb.sol_block_summaries(kd, vd, ws, flags)
        sb.sol_attn_fused(qd, kd, vd, out, beta, flags, ws, kept_per_row=kept)
        torch.cuda.synchronize()
        n_kept = int(kept.sum().item())
        pre, fused = stepper(beta, flags)
        for _ in range(warmup):
            pre(); fused()
        ms, fused_ms, pre_ms, wall, each = time_steps(pre, fused, steps)
        kf = kept_flop(w, n_kept)
        return {
            "beta": beta if math.isfinite(beta) else str(beta),
            "ms": ms, "fused_ms": fused_ms, "prepass_ms": pre_ms, "wall_s": wall,
            "fused_ms_median": statistics.median(each), "fused_ms_min": min(each), "reps": steps,
            "dense_equiv_tflops": dense_equiv_flop(w) / (ms * 1e-3) / 1e12,
            "density": n_kept / (w.B * w.H * nb * nb),
            "kept_blocks": n_kept,
            "kept_tflops_fused": kf / (fused_ms * 1e-3) / 1e12,
            "mfma_frac_fused": kf / (fused_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "prepass_hbm_gbs": 2.0 * w.B * w.H * w.N * w.d * 2 / (pre_ms * 1e-3) / 1e9,
        }

    head = measure(args.beta, corr, args.steps, args.warmup)
    progress(f"headline beta {args.beta}: {head['ms']:.3f} ms per step")
    # the two-call step equals one sol_attn_fwd_ex call (bit for bit)
    ref = out.clone()
    sb.sol_attn_fwd_ex(qd, kd, vd, out, args.beta, corr, workspace=ws)
    torch.cuda.synchronize()
    same_as_fwd_ex = bool(torch.equal(ref, out))
    rows = row_stats(kept)
    balance = load_balance(sb, qd, kd, vd, out, ws, args.beta, corr, w)
    ablation = routing_overhead(sb, qd, kd, vd, out, ws, args.beta, w, max(3, args.steps // 2))
    rowc = None if args.no_correction else measure(args.beta, sb.SOL_CORRECTION_ROW, max(3, args.steps // 2), 3)
    # the low-memory mode (no V^T copy; value tiles from V with transposing LDS reads)
    lowmem = measure(args.beta, corr | sb.SOL_LOW_MEMORY, max(3, args.steps // 2), 3)
    lowmem["workspace_bytes"] = sb.sol_attn_workspace_bytes(w.B, w.H, w.N, w.d, sb.SOL_LOW_MEMORY)
    lowmem["default_workspace_bytes"] = sb.sol_attn_workspace_bytes(w.B, w.H, w.N, w.d)
    lowmem["bit_equal_to_default"] = bool(torch.equal(out, ref))   # same beta and correction
    study = None if args.no_routing_study else routing_study(sb, qd, kd, vd, out, ws, w, 5)
    dense_ref = None
    if not args.no_dense_reference and w.dtype == "bf16":
        dense_ref = dense_reference(qd, kd, vd, w, 3)
        if "ms" in dense_ref:
            dense_ref["fused_speedup_at_headline_beta"] = dense_ref["ms_min"] / head["fused_ms"]
    if study is not None:
        # like for like: the in-pass routing's cost inside the fused pass (fused pass without
        # the correction minus plain block-sparse attention on the same selection) against
        # routing from a materialized map; and the whole paths
        study["in_pass_routing_in_context_ms"] = ablation["fused_no_correction_ms"] - ablation["given_mask_ms"]
        study["map_routing_at_headline_beta_ms"] = ablation["separate_path"]["map_routing_ms"]
    progress("ablation, per-row correction and routing study done")

    per_beta = {str(args.beta): head}
    small_steps = max(3, args.steps // 2)
    for b in [float(x) for x in args.extra_betas.split(",") if x.strip()]:
        per_beta[str(b)] = measure(b, corr, small_steps, 3)
    if not args.no_calibration:
        calib = calibrate_density(sb, qd, kd, vd, out, ws, w, kept, 0.05, corr)
        per_beta["5pct"] = measure(calib, corr, small_steps, 3)
        per_beta["5pct"]["calibrated_for_density"] = 0.05
    if not args.no_dense:
        dense = measure(-math.inf, corr | sb.SOL_DENSE, small_steps, 3)
        per_beta["dense"] = dense
        for key, r in per_beta.items():
            if key != "dense":
                r["speedup_vs_dense"] = dense["ms"] / r["ms"]

    kf = kept_flop(w, head["kept_blocks"])
    achieved = kf / (head["fused_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": traffic_from_profile(),
                "kernel": "fused_kernel<bf16,128,correction>",
                "algorithmic_flop_per_launch": kf}

    # the other configurations (each generated, timed and freed in turn)
    del qd, kd, vd, out, ws
    torch.cuda.empty_cache()
    configs = {}
    for name in [x for x in args.configs.split(",") if x]:
        configs[name] = config_sweep(name, args.config_reps, error_report=wl.CONFIGS[name].skewed)
        progress(f"config {name} done")

    cpu = None
    if not args.no_cpu_baseline:
        heads = list(range(w.H))
        cpu = cpu_baseline(w, q, k, v, args.beta, args.cpu_blocks_per_head, heads)

    line = {
        "metric": METRIC,
        "value": head["dense_equiv_tflops"],
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "beta": args.beta, "correction": not args.no_correction,
                   "grid": list(w.grid) if w.grid else None},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_beta": per_beta,
        "kept_per_row": rows,
        "load_balance": balance,
        "routing_ablation": ablation,
        "row_correction": rowc,
        "low_memory": lowmem,
        "dense_reference": dense_ref,
        "routing_study": study,
        "prepass": prepass_report(w, head["prepass_ms"]),
        "configs": configs,
        "checks": {"two_call_step_equals_fwd_ex": same_as_fwd_ex},
        "input_gen_s": t_gen,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
