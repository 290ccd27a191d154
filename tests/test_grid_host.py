"""Launch-grid arithmetic of the HIP library, checked on the CPU.

HIP limits one grid dimension to 2^32 - 1 work-items; the library caps its
grids there and its kernels walk the remaining work in grid-stride loops.
The header is compiled for the host with g++ (it has no HIP dependency).
"""
import ctypes
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
MAX_ITEMS = (1 << 32) - 1


@pytest.fixture(scope="module")
def grid_blocks(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("grid") / "grid_check.so")
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-o", so,
                           os.path.join(HERE, "grid_check.cpp")])
    lib = ctypes.CDLL(so)
    lib.lowbit_test_grid_blocks.restype = ctypes.c_longlong
    lib.lowbit_test_grid_blocks.argtypes = [ctypes.c_longlong, ctypes.c_int]
    return lib.lowbit_test_grid_blocks


@pytest.mark.parametrize("threads", [64, 128, 256])
def test_grid_within_hip_limit(grid_blocks, threads):
    wpb = threads // 64
    cap = MAX_ITEMS // threads
    for ntrips in [0, 1, 2, 3, 4, 5, 1 << 20, (1 << 20) + 1, cap * wpb - 1, cap * wpb,
                   cap * wpb + 1, 1 << 33, 1 << 40, 1 << 42]:
        b = grid_blocks(ntrips, threads)
        assert 1 <= b and b * threads <= MAX_ITEMS
        want = max(1, -(-ntrips // wpb))
        assert b == min(want, cap)


# (elements per wave trip, threads per workgroup) of each kernel family
TRIPS = {
    "row-layout EF compress / stage-2 reduce (256 elements)": (256, 256),
    "1-bit compress (2048 elements)": (2048, 256),
    "4-bit general tile, 2 tiles (1024 elements)": (1024, 256),
    "decompress, 2 rows of 256": (512, 128),
    "apply, 2 rows of 512": (1024, 128),
    "Hadamard decompress B4096, a workgroup of 4 waves per block": (1024, 256),
}


@pytest.mark.parametrize("name", sorted(TRIPS))
def test_grid_at_2_35_elements(grid_blocks, name):
    """At n = 2^35 the uncapped grid would exceed 2^32 work-items for the
    smallest trips; the capped grid stays valid and the grid-stride loop
    makes up the rest (trips per wave = ceil(trips / waves in the grid))."""
    per_trip, threads = TRIPS[name]
    n = 1 << 35
    ntrips = n // per_trip
    b = grid_blocks(ntrips, threads)
    assert b * threads <= MAX_ITEMS
    waves = b * (threads // 64)
    loops = -(-ntrips // waves)
    assert loops >= 1 and (loops - 1) * waves < ntrips <= loops * waves
    if ntrips * 64 > MAX_ITEMS:
        assert b == MAX_ITEMS // threads
