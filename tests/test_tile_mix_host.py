"""The tile-loop microbenchmark library (libsoltilemix.so, bench.py --tile-mix) on the host:
it loads, exports its two entry points, describes its mixes, and rejects bad arguments
before any device call (no GPU needed)."""
import ctypes
import os

import pytest

from free_block_sparse_mean_amd import build as _b


@pytest.fixture(scope="module")
def mixlib():
    if not os.path.exists(_b.MIX_LIB):
        pytest.fail(f"{_b.MIX_LIB} is not built (python -m free_block_sparse_mean_amd.build)")
    lib = ctypes.CDLL(_b.MIX_LIB)
    lib.sol_tile_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_int)]
    lib.sol_tile_mix_shape.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int)] * 3
    return lib


def test_mix_shapes(mixlib):
    got = []
    for mix in range(8):
        x = [ctypes.c_int(-7) for _ in range(3)]
        rc = mixlib.sol_tile_mix_shape(mix, *[ctypes.byref(v) for v in x])
        if rc != 0:
            assert [v.value for v in x] == [-7, -7, -7]   # untouched on error
            break
        got.append(tuple(v.value for v in x))
    # pure MFMA; operand reads only; VALU only; one read per MFMA; half; a quarter
    assert got == [(0, 0, 0), (16, 0, 0), (0, 24, 8), (16, 24, 8), (8, 24, 8), (4, 24, 8)]
    assert mixlib.sol_tile_mix_shape(-1, *[ctypes.byref(ctypes.c_int()) for _ in range(3)]) == -1


@pytest.mark.parametrize("mix,wps,iters", [(6, 2, 10), (-1, 2, 10), (0, 3, 10), (0, 0, 10), (0, 2, 0),
                                           (0, 2, (1 << 24) + 1)])
def test_bad_arguments_rejected_on_host(mixlib, mix, wps, iters):
    ms, cus = ctypes.c_double(-1.0), ctypes.c_int(-1)
    assert mixlib.sol_tile_mix(mix, wps, iters, ctypes.byref(ms), ctypes.byref(cus)) == -1
    assert ms.value == -1.0 and cus.value == -1
    assert mixlib.sol_tile_mix(0, 2, 10, None, ctypes.byref(cus)) == -1
    assert mixlib.sol_tile_mix(0, 2, 10, ctypes.byref(ms), None) == -1
