"""The library's per-lane row selection (select_lane.hpp, the selection of the
per-token prune kernel) built for the host and run on the CPU against the
oracle's rule (a stable sort by magnitude key, ties to the lower channel) on
random, tie-heavy and special rows at every keep 0..128, and the channel-wise
selection of a lane's channel pair (lane_select_columns) against the oracle's
channel-wise rule on full 64-row tiles.  No GPU needed."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows(rng, n):
    out = [rng.standard_normal((n, 128)).astype(np.float16).view(np.uint16),
           (rng.integers(-3, 4, (n, 128)).astype(np.float16)).view(np.uint16),
           rng.choice(np.array([0, 0x8000, 1, 0x8001, 0x7BFF, 0xFBFF, 0x3C00, 0xBC00], np.uint16), (n, 128)),
           rng.integers(0, 0x7C00, (n, 128)).astype(np.uint16) | (rng.integers(0, 2, (n, 128)) << 15).astype(np.uint16)]
    x = np.concatenate(out)
    x[0] = 0                      # all zero
    x[1] = 0x3C00                 # all equal
    x[2] = np.arange(128, dtype=np.uint16)[::-1]  # strictly decreasing keys
    x[3, ::2] = 0x7BFF            # half of the channels at the largest finite magnitude
    return x


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_lane_selection_matches_oracle(tmp_path):
    exe = tmp_path / "select_rows"
    subprocess.run(["g++", "-O2", "-std=c++17", os.path.join(ROOT, "tests", "cpu_select", "select_rows.cpp"),
                    "-o", str(exe)], check=True)
    rng = np.random.default_rng(2024)
    rows = _rows(rng, 300)
    keeps = np.arange(rows.shape[0], dtype=np.int32) % 129
    blob = b"".join(np.int32(k).tobytes() + r.tobytes() for k, r in zip(keeps, rows))
    r = subprocess.run([str(exe)], input=blob, capture_output=True, check=True)
    got = np.frombuffer(r.stdout, dtype=np.uint32).reshape(-1, 4)
    assert got.shape[0] == rows.shape[0]
    for i, (k, row) in enumerate(zip(keeps, rows)):
        mask = oracle.prune_rows(row[None], int(k))[0]
        words = np.zeros(4, np.uint32)
        for ch in np.nonzero(mask)[0]:
            words[ch // 32] |= np.uint32(1 << int(ch % 32))
        assert np.array_equal(got[i], words), (i, int(k))


def _tiles(rng, n):
    out = []
    for i in range(n):
        kind = i % 4
        if kind == 0:
            t = rng.standard_normal((64, 128)).astype(np.float16).view(np.uint16)
        elif kind == 1:
            t = rng.integers(-3, 4, (64, 128)).astype(np.float16).view(np.uint16)
        elif kind == 2:
            t = rng.choice(np.array([0, 0x8000, 1, 0x8001, 0x7BFF, 0xFBFF, 0x3C00, 0xBC00], np.uint16), (64, 128))
        else:
            t = (rng.integers(0, 0x7C00, (64, 128)).astype(np.uint16)
                 | (rng.integers(0, 2, (64, 128)) << 15).astype(np.uint16))
        out.append(t)
    out[0][:, 0] = 0                                   # an all-zero channel
    out[1][:, 1] = 0x3C00                              # an all-equal channel
    out[2][:, 2] = np.arange(64, dtype=np.uint16)      # strictly increasing keys down a channel
    return out


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_lane_channel_selection_matches_oracle(tmp_path):
    """lane_select_columns (the channel-wise prune's selection, one channel
    pair per lane) on full 64-row tiles against the oracle's channel-wise rule
    (each channel keeps keep/2 rows, ties to the earlier row)."""
    exe = tmp_path / "select_cols"
    subprocess.run(["g++", "-O2", "-std=c++17", os.path.join(ROOT, "tests", "cpu_select", "select_cols.cpp"),
                    "-o", str(exe)], check=True)
    rng = np.random.default_rng(77)
    tiles = _tiles(rng, 40)
    keeps = [2 * ((5 * i) % 65) for i in range(len(tiles))]   # even keeps 0..128
    keeps[3], keeps[4] = 0, 128
    blob = b"".join(np.int32(k).tobytes() + t.tobytes() for k, t in zip(keeps, tiles))
    r = subprocess.run([str(exe)], input=blob, capture_output=True, check=True)
    got = np.frombuffer(r.stdout, dtype=np.uint32).reshape(len(tiles), 64, 4)
    for i, (k, t) in enumerate(zip(keeps, tiles)):
        c = oracle.compress_channel(t[None, None], np.array([64], np.int32), int(k))
        want = c.bitmaps.reshape(64, 2).view(np.uint32).reshape(64, 4)
        assert np.array_equal(got[i], want), (i, k)
