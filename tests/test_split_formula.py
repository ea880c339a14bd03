"""Decode split-K sizing (csrc/qk4v8_split.h) on the host, with stub CU counts
and occupancies: the formula is plain C++, compiled here with g++ and called
through a tiny extern "C" shim, so no GPU is needed."""
import ctypes
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_attention_online_amd", "csrc")

SHIM = r'''
#include "qk4v8_split.h"
extern "C" int split_count(long long units, int span, long long capacity, int requested) {
  return qk4v8::decode_split_count(units, span, capacity, requested);
}
extern "C" int key_span(int kv_len, int q_len, int window) { return qk4v8::decode_key_span(kv_len, q_len, window); }
extern "C" int row_blocks(int rows) { return qk4v8::decode_row_blocks(rows); }
'''


@pytest.fixture(scope="module")
def shim():
    d = tempfile.mkdtemp(prefix="qk4v8_split_")
    src, lib = os.path.join(d, "shim.cpp"), os.path.join(d, "shim.so")
    with open(src, "w") as f:
        f.write(SHIM)
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, src, "-o", lib], check=True)
    L = ctypes.CDLL(lib)
    L.split_count.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_longlong, ctypes.c_int]
    return L


def test_mi355x_workloads(shim):
    # 256 CUs; resident workgroups per CU as the runtime reports them for the
    # compiled kernels: 4 one-wave workgroups (decode, 8 rows) and 3 four-wave
    # workgroups (block verify, 64 rows)
    assert shim.split_count(64 * 8, 32768, 256 * 4, 0) == 2        # decode: 512 units -> 1024 slots
    assert shim.split_count(32 * 8, 16392, 256 * 3, 0) == 3        # block verify: 256 units -> 768 slots


def test_partitioned_device_and_occupancy_follow_the_query(shim):
    # a device partition with 32 CUs, or a kernel holding fewer workgroups,
    # shrinks the split count with it instead of keeping a fixed machine
    assert shim.split_count(64 * 8, 32768, 32 * 4, 0) == 1
    assert shim.split_count(4 * 8, 32768, 32 * 4, 0) == 4
    assert shim.split_count(32 * 8, 16392, 256 * 2, 0) == 2
    assert shim.split_count(1, 1 << 20, 256 * 4, 0) == 1024


def test_tiles_per_split_floor_and_requests(shim):
    assert shim.split_count(1, 128 * 20, 1 << 20, 0) == 2          # at least 8 tiles of 128 keys per split
    assert shim.split_count(1, 100, 1 << 20, 0) == 1
    assert shim.split_count(1, 1000, 0, 3) == 3                     # requested count, no device needed
    assert shim.split_count(1, 300, 0, 9) == 3                      # at most one split per 128-key tile
    assert shim.split_count(1, 1000, 0, 0) == 0                     # no capacity, nothing requested: unknown


def test_window_bounds_the_span(shim):
    # with a window the splits cover at most window + q_len + 126 keys, so the
    # split count (and workspace) stops growing with the cache length
    assert shim.key_span(1 << 20, 1, 1024) == 1024 + 1 + 126
    assert shim.key_span(1 << 19, 8, 1024) == 1024 + 8 + 126
    assert shim.key_span(1000, 1, 1000) == 1000
    assert shim.key_span(1000, 1, 0) == 1000
    full = shim.split_count(1, shim.key_span(1 << 20, 1, 0), 1024, 0)
    win = shim.split_count(1, shim.key_span(1 << 20, 1, 1024), 1024, 0)
    assert win < full and win == 1


def test_row_blocks(shim):
    assert [shim.row_blocks(r) for r in (1, 8, 16, 17, 32, 40, 48, 49, 64)] == [1, 1, 1, 2, 2, 3, 3, 4, 4]
