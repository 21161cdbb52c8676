"""Pins of the gfx950 instruction semantics the matrix-core kernels rely on.

* ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives, as its
  element e (e = 0..3), 16-bit word (j mod 4) of the 8 bytes addressed by lane
  4e + j div 4 of the same group.  Read with lanes addressing a 4-row x 16-column
  block of a row-major tile (lane l: row l div 4, columns 4 (l mod 4) ..), lane j
  gets column j of the 4 rows: the transpose the B operand needs.
* ds_read_b64_tr_b8: within each group of 16 lanes, lane j receives, as its
  byte e (e = 0..7), byte (j mod 8) of the 8 bytes addressed by lane 2e + j div 8
  of the same group.  Read with lanes addressing an 8-row x 16-byte block (lane
  l: row l div 2, bytes 8 (l mod 2) ..), lane j gets column j of the 8 rows: the
  transpose an 8-bit B operand needs.
* global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16 l, whatever
  global address the lane supplied; nothing else in LDS changes.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "probes", "libprobes.so")


def _lib():
    L = ctypes.CDLL(LIB)
    L.probe_tr16.argtypes = [ctypes.c_void_p] * 3
    L.probe_lds_load.argtypes = [ctypes.c_void_p] * 4
    L.probe_tr8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return L


def _tr16(addr):
    a = torch.tensor(addr, dtype=torch.int32, device="cuda")
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    assert _lib().probe_tr16(a.data_ptr(), out.data_ptr(),
                             torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16).reshape(64, 4).astype(np.int64)


def _model(addr):
    addr = np.asarray(addr)
    want = np.zeros((64, 4), dtype=np.int64)
    for lane in range(64):
        g0, j = lane - lane % 16, lane % 16
        for e in range(4):
            src = g0 + 4 * e + j // 4
            want[lane, e] = addr[src] // 2 + (j % 4)
    return want


def _tr8(addr):
    a = torch.tensor(addr, dtype=torch.int32, device="cuda")
    got = np.zeros((64, 8), dtype=np.int64)
    for mode, shift in ((0, 0), (1, 8)):
        out = torch.zeros(512, dtype=torch.uint8, device="cuda")
        assert _lib().probe_tr8(a.data_ptr(), out.data_ptr(), mode,
                                torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        got += out.cpu().numpy().reshape(64, 8).astype(np.int64) << shift
    return got


def _model8(addr):
    addr = np.asarray(addr)
    want = np.zeros((64, 8), dtype=np.int64)
    for lane in range(64):
        g0, j = lane - lane % 16, lane % 16
        for e in range(8):
            want[lane, e] = (addr[g0 + 2 * e + j // 8] & 8184) + (j % 8)
    return want


@pytest.mark.parametrize("pattern", ["contiguous", "tile", "random"])
def test_ds_read_b64_tr_b8_lane_map(pattern):
    if pattern == "contiguous":
        addr = [8 * l for l in range(64)]
    elif pattern == "tile":
        # row-major byte tile with a 128-byte row pitch: group g reads rows 16g..16g+7
        addr = []
        for l in range(64):
            g, li = l // 16, l % 16
            addr.append((16 * g + li // 2) * 128 + 8 * (li % 2))
    else:
        addr = list(8 * np.random.default_rng(1).permutation(1024)[:64])
    got = _tr8(addr)
    assert np.array_equal(got, _model8(addr))
    if pattern == "tile":
        # lane j of group g holds column j of rows 16g .. 16g+7
        for l in range(64):
            g, j = l // 16, l % 16
            assert list(got[l]) == [(16 * g + e) * 128 + j for e in range(8)]


@pytest.mark.parametrize("pattern", ["contiguous", "tile", "random"])
def test_ds_read_b64_tr_b16_lane_map(pattern):
    if pattern == "contiguous":
        addr = [8 * l for l in range(64)]
    elif pattern == "tile":
        # row-major tile with a 64-element row pitch: group g reads rows 8g..8g+3
        addr = []
        for l in range(64):
            g, li = l // 16, l % 16
            row, col = 8 * g + li // 4, 4 * (li % 4)
            addr.append(2 * (row * 64 + col))
    else:
        addr = list(8 * np.random.default_rng(0).permutation(1024)[:64])
    got = _tr16(addr)
    assert np.array_equal(got, _model(addr))
    if pattern == "tile":
        # lane j of group g holds column j of rows 8g .. 8g+3
        for l in range(64):
            g, j = l // 16, l % 16
            assert list(got[l]) == [(8 * g + e) * 64 + j for e in range(4)]


def test_global_load_lds_lane_placement():
    src = torch.arange(256, dtype=torch.int32, device="cuda")
    perm = np.random.default_rng(1).permutation(64)
    off = torch.tensor(perm, dtype=torch.int32, device="cuda")
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")
    assert _lib().probe_lds_load(src.data_ptr(), off.data_ptr(), out.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    want = np.full(1024, 0xffffffff, dtype=np.uint32)
    for lane in range(64):
        want[64 + 4 * lane: 64 + 4 * lane + 4] = np.arange(4 * perm[lane], 4 * perm[lane] + 4)
    assert np.array_equal(got, want)
