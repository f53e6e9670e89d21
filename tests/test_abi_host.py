"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/sol_attn.h declares, and rejects invalid arguments before any
device call."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sol_attn.h")
LIB = os.path.join(ROOT, "free_block_sparse_mean_amd", "libsolattn.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sol_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libsolattn.so is not built (run __graft_entry__.build())")
    from free_block_sparse_mean_amd import binding
    return binding.load_library(LIB)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert "sol_attn_fwd" in names and "sol_attn_fused" in names and len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sol_attn.h but not exported"


def test_abi_version(lib):
    text = open(HEADER).read()
    want = int(re.search(r"#define SOL_ATTN_ABI_VERSION (\d+)", text).group(1))
    assert lib.sol_abi_version() == want


def test_workspace_bytes(lib):
    n = lib.sol_attn_workspace_bytes(1, 24, 131072, 128)
    nb = 2048
    assert n >= 24 * (3 * nb * 128 * 4 + 128 * 4 + 128 * 128 * 4)
    assert n < 1024 * 2 ** 20
    assert lib.sol_attn_workspace_bytes(1, 1, 100, 64) == 0      # not a multiple of 64
    assert lib.sol_attn_workspace_bytes(1, 1, 4096, 96) == 0     # unsupported d
    assert lib.sol_attn_workspace_bytes(0, 1, 4096, 64) == 0


@pytest.mark.parametrize("args,code", [
    ((1, 1, 4096, 64, 1.0, 0), 1),              # null pointers
    ((1, 1, 100, 64, 1.0, 0), 1),               # N % 64
    ((1, 1, 4096, 96, 1.0, 0), 2),              # d unsupported
    ((0, 1, 4096, 64, 1.0, 0), 1),              # B <= 0
    ((1, 1, 64 * 5000, 64, 1.0, 0), 2),         # N beyond the maximum
])
def test_invalid_arguments_fwd(lib, args, code):
    B, H, N, d, beta, flags = args
    st = lib.sol_attn_fwd(None, None, None, None, B, H, N, d, beta, flags)
    assert st == code
    assert lib.sol_last_error().decode()


def test_invalid_beta_and_flags(lib):
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    assert lib.sol_attn_fwd(p, p, p, p, 1, 1, 4096, 64, math.nan, 0) == 1
    assert "NaN" in lib.sol_last_error().decode()
    assert lib.sol_attn_fwd(p, p, p, p, 1, 1, 4096, 64, 1.0, 0x100) == 1
    assert "flag" in lib.sol_last_error().decode()


def test_workspace_too_small(lib):
    p = ctypes.c_void_p(16)
    st = lib.sol_attn_fwd_ex(p, p, p, p, 1, 1, 4096, 64, 1.0, 0, None, p, 10, None)
    assert st == 5
    assert "workspace" in lib.sol_last_error().decode()
    st = lib.sol_block_summaries(p, p, 1, 1, 4096, 64, 0, None, 0, None)
    assert st == 5


def test_layout_offsets(lib):
    from free_block_sparse_mean_amd import binding
    lay = binding.sol_workspace_layout()
    assert lib.sol_attn_workspace_layout(2, 3, 64 * 100, 128, ctypes.byref(lay)) == 0
    offs = [lay.kbar_t, lay.kbar, lay.vsum, lay.kmean, lay.kcov, lay.qbar, lay.kbar_bf,
            lay.vbar_t, lay.vbar_bf, lay.scratch, lay.vt]
    assert offs == sorted(offs) and offs[0] == 0 and lay.total_bytes > lay.vt
    assert all(o % 256 == 0 for o in offs)
    assert lay.kbar - lay.kbar_t >= 6 * 128 * 100 * 4
    # the V^T copy is the last array: the low-memory workspace is everything before it
    assert lay.total_bytes - lay.vt >= 6 * 100 * 128 * 64 * 2
    assert lib.sol_attn_workspace_bytes(2, 3, 64 * 100, 128) == lay.total_bytes
    assert lib.sol_attn_workspace_bytes_flags(2, 3, 64 * 100, 128, 0x20) == lay.vt
    assert lib.sol_attn_workspace_bytes_flags(2, 3, 64 * 100, 128, 0x2) == lay.total_bytes


def test_low_memory_workspace_validation(lib):
    """A SOL_LOW_MEMORY call accepts a workspace of the smaller size; the same call
    without the flag refuses it before any device call."""
    p = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    small = lib.sol_attn_workspace_bytes_flags(1, 2, 4096, 128, 0x20)
    full = lib.sol_attn_workspace_bytes(1, 2, 4096, 128)
    assert 0 < small < full
    assert lib.sol_block_summaries(p, p, 1, 2, 4096, 128, 0, p, small, None) == 5
    assert "workspace" in lib.sol_last_error().decode()
    assert lib.sol_attn_fused(p, p, p, p, 1, 2, 4096, 128, ctypes.c_float(1.0), 0x2, p, small, None, None) == 5
    assert lib.sol_attn_fused(p, p, p, p, 1, 2, 4096, 128, ctypes.c_float(1.0), 0x40, p, small, None, None) == 1
    assert "flag" in lib.sol_last_error().decode()


def test_masked_validation(lib):
    """The given-mask entry point checks its arguments before any device call."""
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    assert lib.sol_attn_masked(p, p, p, p, 1, 1, 4096, 64, None, 0, p, 1 << 30, None, None) == 1
    assert "mask_bits" in lib.sol_last_error().decode()
    assert lib.sol_attn_masked(p, p, p, p, 1, 1, 4096, 64, p, 0x2, p, 1 << 30, None, None) == 1
    assert "SOL_CORRECTION" in lib.sol_last_error().decode()
    assert lib.sol_attn_masked(p, p, p, p, 1, 1, 4096, 64, p, 0x4, p, 1 << 30, None, None) == 1
    assert lib.sol_attn_masked(p, p, p, p, 1, 1, 4096, 64, p, 0, p, 10, None, None) == 5
    assert lib.sol_attn_masked(p, p, p, p, 1, 1, 4096, 96, p, 0, p, 1 << 30, None, None) == 2


def test_route_validation(lib):
    """The routing entry point checks its arguments before any device call."""
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    big = 1 << 30
    assert lib.sol_route(p, 1, 1, 4096, 64, 0, 0, 1.0, 0, 0.0, p, big, None, p, None, None, None) == 1
    assert "proxy_map" in lib.sol_last_error().decode()
    assert lib.sol_route(p, 1, 1, 4096, 64, 0, 7, 1.0, 0, 0.0, p, big, p, p, None, None, None) == 1
    assert "mode" in lib.sol_last_error().decode()
    assert lib.sol_route(p, 1, 1, 4096, 64, 0, 0, math.nan, 0, 0.0, p, big, p, p, None, None, None) == 1
    assert lib.sol_route(p, 1, 1, 4096, 64, 0, 1, 0.0, -1, 0.0, p, big, p, p, None, None, None) == 1
    assert lib.sol_route(p, 1, 1, 4096, 64, 0, 2, 0.0, 0, math.nan, p, big, p, p, None, None, None) == 1
    assert lib.sol_route(p, 1, 1, 4096, 64, 0x2, 0, 1.0, 0, 0.0, p, big, p, p, None, None, None) == 1
    assert lib.sol_route(p, 1, 1, 4096, 64, 0, 0, 1.0, 0, 0.0, p, 10, p, p, None, None, None) == 5


def test_joint_validation(lib):
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    big = 1 << 30
    assert lib.sol_attn_fused_joint(p, p, p, p, 1, 1, 4096, 64, 1.0, 0, -1, p, big, None, None) == 1
    assert lib.sol_attn_fused_joint(p, p, p, p, 1, 1, 4096, 64, 1.0, 0, 65, p, big, None, None) == 1
    assert "text_blocks" in lib.sol_last_error().decode()
    assert lib.sol_attn_fused_joint(p, p, p, p, 1, 1, 4096, 64, 1.0, 0, 3, p, 10, None, None) == 5


def test_strided_validation(lib):
    from free_block_sparse_mean_amd.binding import sol_strides
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    big = 1 << 30
    B, H, N, d = 1, 2, 4096, 64
    bnhd = sol_strides(N * H * d, d, H * d)
    call = lambda q=p, sq=None, sk=None, sv=None, so=None, flags=0, ws=big: lib.sol_attn_fwd_strided(
        q, p, p, p, B, H, N, d, sq, sk, sv, so, 1.0, flags, None, p, ws, None)
    ref = lambda s: ctypes.byref(s)
    # valid strides reach the workspace check (error 5), invalid ones stop before it (error 1)
    assert call(sq=ref(bnhd), sk=ref(bnhd), sv=ref(bnhd), so=ref(bnhd), ws=10) == 5
    assert call(sq=ref(sol_strides(0, d, H * d)), ws=10) == 5          # b stride unused when B = 1
    assert call(q=ctypes.c_void_p(24)) == 1
    assert "aligned" in lib.sol_last_error().decode()
    assert call(sq=ref(sol_strides(N * H * d, d, H * d + 4))) == 1     # not 16-byte rows (bf16)
    assert "multiple of 8" in lib.sol_last_error().decode()
    assert call(sq=ref(sol_strides(N * H * d, d, H * d + 4)), flags=1, ws=10) == 5   # fp32: 4 suffice
    assert call(sk=ref(sol_strides(N * H * d, 0, H * d))) == 1        # h stride 0 with H = 2
    assert call(sv=ref(sol_strides(N * H * d, d, -H * d))) == 1
    assert call(sq=ref(sol_strides(N * H * d, d, 1 << 24))) == 1
    assert call(so=ref(sol_strides(N * H * d, d, 8))) == 1              # out rows would overlap
    assert "at least d" in lib.sol_last_error().decode()


def test_misaligned_pointers_rejected(lib):
    """Every entry point refuses q, k, v, out not 16-byte aligned, a workspace not
    256-byte aligned and debug outputs not aligned to their elements, before any device
    call (the pointers are never dereferenced)."""
    p = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4096 + 8)
    big = 1 << 30
    B, H, N, d = 1, 1, 4096, 64

    def expect(st, what):
        assert st == 1, (what, st)
        assert "aligned" in lib.sol_last_error().decode(), what

    expect(lib.sol_attn_fwd(odd, p, p, p, B, H, N, d, 1.0, 0), "fwd q")
    expect(lib.sol_attn_fwd(p, p, p, odd, B, H, N, d, 1.0, 0), "fwd out")
    expect(lib.sol_attn_fwd_ex(p, odd, p, p, B, H, N, d, 1.0, 0, None, p, big, None), "fwd_ex k")
    expect(lib.sol_attn_fwd_ex(p, p, p, p, B, H, N, d, 1.0, 0, None, ctypes.c_void_p(4096 + 16), big, None),
           "fwd_ex workspace")
    expect(lib.sol_block_summaries(p, odd, B, H, N, d, 0, p, big, None), "summaries v")
    expect(lib.sol_block_summaries(p, p, B, H, N, d, 0, ctypes.c_void_p(4096 + 128), big, None),
           "summaries workspace")
    expect(lib.sol_attn_fused(p, p, odd, p, B, H, N, d, 1.0, 0, p, big, None, None), "fused v")
    expect(lib.sol_attn_fused_joint(odd, p, p, p, B, H, N, d, 1.0, 0, 1, p, big, None, None), "joint q")
    expect(lib.sol_attn_masked(p, p, p, odd, B, H, N, d, p, 0, p, big, None, None), "masked out")
    expect(lib.sol_attn_masked(p, p, p, p, B, H, N, d, ctypes.c_void_p(4096 + 4), 0, p, big, None, None),
           "masked mask_bits")
    expect(lib.sol_route(odd, B, H, N, d, 0, 0, 1.0, 0, 0.0, p, big, p, p, None, None, None), "route q")
    expect(lib.sol_route(p, B, H, N, d, 0, 0, 1.0, 0, 0.0, p, big, p, ctypes.c_void_p(4096 + 4), None, None,
                         None), "route mask_bits")
    from free_block_sparse_mean_amd.binding import sol_debug
    dbg = sol_debug(None, ctypes.c_void_p(4096 + 4).value, None, None)
    expect(lib.sol_attn_fused(p, p, p, p, B, H, N, d, 1.0, 0, p, big, ctypes.byref(dbg), None), "dbg mask_bits")
    dbg = sol_debug(ctypes.c_void_p(4096 + 2).value, None, None, None)
    expect(lib.sol_attn_fwd_ex(p, p, p, p, B, H, N, d, 1.0, 0, None, p, big, ctypes.byref(dbg)), "dbg kept")


def test_queue_slot_pool(tmp_path):
    """The pool of work-item queue counters (host C++, built here with g++): eager
    launches never take a slot of the range kept for launches recorded into graphs,
    and each range is dealt round-robin."""
    src = tmp_path / "slots.cpp"
    src.write_text(r'''
#include <cstdio>
#include "queue_slots.hpp"
int main() {
  sol::QueueSlots pool;
  for (int i = 0; i < 3 * sol::kQueueSlots; ++i) {
    const int e = pool.take(false);
    if (e != i % sol::kEagerSlots) { std::printf("eager %d -> %d\n", i, e); return 1; }
    if (i % 3 == 0) {
      const int c = pool.take(true);
      if (c < sol::kEagerSlots || c >= sol::kQueueSlots || c != sol::kEagerSlots + (i / 3) % sol::kCapturedSlots) {
        std::printf("captured %d -> %d\n", i, c); return 1;
      }
    }
  }
  std::printf("ok\n");
  return 0;
}
''')
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.fail("g++ is needed for this host test")
    exe = tmp_path / "slots"
    inc = os.path.join(ROOT, "free_block_sparse_mean_amd", "csrc")
    subprocess.run([gxx, "-std=c++17", "-O1", "-I", inc, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_noalloc_rejects_beyond_its_scratch(lib):
    """sol_attn_fwd_noalloc refuses, before any device call, a shape whose workspace
    exceeds its 64 MiB scratch, and validates like sol_attn_fwd_ex."""
    p = ctypes.c_void_p(4096)
    B, H, N, d = 1, 24, 16384, 128
    assert lib.sol_attn_workspace_bytes(B, H, N, d) > 64 * 2 ** 20
    assert lib.sol_attn_fwd_noalloc(p, p, p, p, B, H, N, d, 1.0, 0, None, None) == 2
    assert "64" in lib.sol_last_error().decode() and "sol_attn_fwd_ex" in lib.sol_last_error().decode()
    assert lib.sol_attn_fwd_noalloc(None, p, p, p, 1, 1, 4096, 64, 1.0, 0, None, None) == 1
    assert lib.sol_attn_fwd_noalloc(p, p, p, p, 1, 1, 4096, 64, math.nan, 0, None, None) == 1
    assert lib.sol_attn_fwd_noalloc(p, p, p, p, 1, 1, 4096, 96, 1.0, 0, None, None) == 2
    assert lib.sol_attn_fwd_noalloc(ctypes.c_void_p(4104), p, p, p, 1, 1, 4096, 64, 1.0, 0, None, None) == 1
