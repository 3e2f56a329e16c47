"""The decode kernel's work split checked on the CPU (no GPU).

tests/partition_check.cpp compiles the kernel's own partition header
(quantization_error_compensation_amd/csrc/partition.hpp) for the host and
checks it by brute force over a grid of layer shapes and workgroup counts:
every rank and row unit has one owner and the owner functions the kernel
uses find it, runs are non-empty and ordered, row runs start on an even
block, each band's segment count (what the last-arriver count relies on)
equals the number of workgroups that really meet it, and the partial-sum
slots of shared bands are distinct and inside the workspace.
"""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "partition_check.cpp")
CSRC = os.path.join(ROOT, "quantization_error_compensation_amd", "csrc")
OUT = os.path.join(ROOT, "tests", "_build", "libpartition_check.so")
MAX_SLOTS = 256   # kMaxSlots of the library (one workgroup per compute unit)


@pytest.fixture(scope="module")
def lib():
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    extra = os.environ.get("SPEAR_SANITIZE_CXXFLAGS", "").split()   # set by the sanitizer test
    out = OUT.replace(".so", "_san.so") if extra else OUT
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                           *extra, "-I/opt/rocm/include", "-I", CSRC, SRC, "-o", out])
    L = ctypes.CDLL(out)
    L.check_split.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(ctypes.c_longlong)]
    L.check_split.restype = ctypes.c_int
    L.check_message.restype = ctypes.c_char_p
    L.check_fastdiv.argtypes = [ctypes.c_uint32]
    L.check_fastdiv.restype = ctypes.c_int
    return L


def test_fast_division_matches_the_divider(lib):
    # the split divides by fixed values with a multiply and a shift
    assert lib.check_fastdiv(1100) == 0, lib.check_message().decode()


def run(lib, K, N, r, slots, shared=True):
    KB, NB, RB = K // 128, (N + 127) // 128, (r + 63) // 64
    st = (ctypes.c_longlong * 8)()
    rc = lib.check_split(KB, RB, NB, slots, MAX_SLOTS, int(shared), st)
    assert rc == 0, (K, N, r, slots, shared, lib.check_message().decode())
    return dict(zip(("P", "Rw", "S", "D", "seg_row", "seg_rank", "ws_slots", "maxrun"), list(st)))


LAYERS = [(128, 16), (128, 128), (256, 16), (512, 512), (1024, 48), (4096, 4096), (8192, 8192),
          (4096, 11008), (28672, 8192), (2048, 1008), (131072, 128), (1152, 6400)]


@pytest.mark.parametrize("K,N", LAYERS)
@pytest.mark.parametrize("r", [0, 16, 64, 128])
def test_split_holds_for_every_slot_count(lib, K, N, r):
    for slots in (1, 2, 3, 7, 32, 100, 255, 256):
        run(lib, K, N, r, slots)
        run(lib, K, N, r, slots, shared=False)


def test_separate_mode_when_asked(lib):
    # the 70B layer at rank 128 (two rank bands) would share its rank
    # workgroups with rows; asked for separate mode it keeps them apart
    assert run(lib, 28672, 8192, 128, 256)["S"] == 1
    st = run(lib, 28672, 8192, 128, 256, shared=False)
    assert st["S"] == st["Rw"] > 1, st


def test_large_layers(lib):
    for K, N, r in ((131072, 131072, 128), (131072, 4096, 64), (16384, 131072, 16)):
        run(lib, K, N, r, 256)


@pytest.mark.parametrize("K,N,r", [(28672, 8192, 64), (8192, 8192, 128), (8192, 8192, 16),
                                   (8192, 8192, 64)])
def test_benchmark_layers_fill_the_device(lib, K, N, r):
    # at full size at least three quarters of the compute units get a row
    # workgroup (all of them under the stream-K split) and a rank band is
    # shared by a bounded number of rank workgroups
    st = run(lib, K, N, r, 256)
    assert 4 * (st["P"] - st["S"]) >= 3 * (256 - st["S"]), st
    assert 8 <= st["Rw"] <= 32 and st["seg_rank"] <= 32, st


def test_the_70b_layer_shares_rank_workgroups_with_rows(lib):
    # 28672 -> 8192: a rank workgroup's eight rank units are a small part of
    # its share, so all but the reducing workgroup 0 go on to stream rows
    st = run(lib, 28672, 8192, 64, 256)
    assert st["S"] == 1 and st["D"] > 0, st


def test_small_layers_keep_rank_workgroups_apart(lib):
    # a 4096 x 4096 layer is too small for a rank workgroup to also take two
    # row units: its rank workgroups take no rows and the rows go to the rest
    st = run(lib, 4096, 4096, 32, 256)
    assert st["S"] == st["Rw"] >= 1, st


@pytest.mark.parametrize("K,N,r", [(4096, 4096, 32), (4096, 4096, 0), (2048, 1008, 16),
                                   (8192, 8192, 128), (8192, 8192, 0)])
def test_short_runs_keep_to_one_band(lib, K, N, r):
    # runs of a few units: each band goes to a fixed number of row
    # workgroups of its own, so no run crosses a band (the row workgroups
    # then meet NB x that number of bands in all, one each)
    NB = (N + 127) // 128
    st = run(lib, K, N, r, 256)
    assert st["P"] - st["S"] == NB * st["seg_row"], st


@pytest.mark.parametrize("K,N,r", [(16384, 8192, 0), (4096, 11008, 32)])
def test_other_layers_stay_stream_k(lib, K, N, r):
    # runs of 32 units or more, or bands that would leave more than a
    # quarter of the row workgroups idle: the stream-K split over all of them
    st = run(lib, K, N, r, 256)
    assert st["P"] == 256, st
