"""CPU oracle for the MUSTAFAR hot path (ctypes binding of mustafar_oracle.cpp).

TEST INFRASTRUCTURE ONLY: the plain fp64 / exact-integer definition that the
HIP library is checked against.  Only tests/, the smoke check in
__graft_entry__ and the CPU-baseline leg of bench.py may import this package.
It shares no code with the HIP library (unstructured_sparse_kv_amd).

Every function is pinned by CPU tests against things other than itself: see
tests/test_oracle_*.py.  The pages print no worked example, so nothing here is
pinned to a value printed on the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mustafar_oracle.cpp")
_LIB = os.path.join(_HERE, "libmustafar_oracle.so")

_lib = None

P = ctypes.c_void_p
I32, I64, F64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double


def build(extra_flags: tuple = ()) -> str:
    """Compile the oracle with the host C++ compiler (no HIP)."""
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", *extra_flags, _SRC,
           "-o", _LIB + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        # MUSTAFAR_ORACLE_LIB names another build of the same source (the CPU
        # sanitizer test loads an ASan/UBSan build this way)
        path = os.environ.get("MUSTAFAR_ORACLE_LIB")
        if path is None:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        L.orc_half_to_double.restype = F64
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_half_to_double_array.argtypes = [P, I64, P]
        L.orc_hardware_threads.restype = ctypes.c_int
        L.orc_keep_from_sparsity.restype = ctypes.c_int
        L.orc_keep_from_sparsity.argtypes = [F64, ctypes.c_int]
        L.orc_prune_rows.argtypes = [P, I64, ctypes.c_int, ctypes.c_int, P]
        L.orc_compress.restype = ctypes.c_int
        L.orc_compress.argtypes = [P, ctypes.c_int, ctypes.c_int, I64, ctypes.c_int, P, ctypes.c_int,
                                   I64, P, P, P, ctypes.c_int]
        L.orc_decompress.restype = ctypes.c_int
        L.orc_decompress.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, I64, ctypes.c_int,
                                     ctypes.c_int, P, P]
        L.orc_used_bytes.restype = I64
        L.orc_used_bytes.argtypes = [ctypes.c_int, ctypes.c_int, P, I64, ctypes.c_int, ctypes.c_int]
        L.orc_attention_dense.restype = ctypes.c_int
        L.orc_attention_dense.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          P, P, I64, P, F64, P, ctypes.c_int]
        L.orc_attention_compressed.restype = ctypes.c_int
        L.orc_attention_compressed.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, P, P, P, ctypes.c_int, P, P, P,
                                               ctypes.c_int, I64, P, F64, P, I64, P, ctypes.c_int]
        Ci = ctypes.c_int
        L.orc_prune_rows_24.restype = Ci
        L.orc_prune_rows_24.argtypes = [P, I64, Ci, P]
        L.orc_compress_channel.restype = Ci
        L.orc_compress_channel.argtypes = [P, Ci, Ci, I64, Ci, P, Ci, I64, P, P, P, Ci]
        L.orc_compress_24.restype = Ci
        L.orc_compress_24.argtypes = [P, Ci, Ci, I64, Ci, P, I64, P, P, P, Ci]
        L.orc_compress_hk.restype = Ci
        L.orc_compress_hk.argtypes = [P, Ci, Ci, I64, Ci, P, Ci, P, I64, P, P, P, Ci]
        L.orc_decompress_hk.restype = Ci
        L.orc_decompress_hk.argtypes = [P, P, P, Ci, Ci, I64, Ci, Ci, P, P, P]
        L.orc_used_bytes_hk.restype = I64
        L.orc_used_bytes_hk.argtypes = [Ci, Ci, P, I64, Ci, Ci, P]
        L.orc_append_rows.restype = Ci
        L.orc_append_rows.argtypes = [P, P, P, Ci, Ci, I64, Ci, Ci, P, P, P, P]
        L.orc_attention_compressed_hk.restype = Ci
        L.orc_attention_compressed_hk.argtypes = [P, Ci, Ci, Ci, Ci, P, P, P, Ci, P, P, P, P, Ci, P,
                                                  I64, P, F64, P, I64, P, Ci]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    """fp16 data (numpy float16/uint16 or a CPU torch tensor) as contiguous uint16 bits."""
    if hasattr(a, "detach"):
        import torch
        a = a.detach().cpu().contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(a)
    return a.view(np.uint16)


def hardware_threads() -> int:
    return lib().orc_hardware_threads()


def half_to_double(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().orc_half_to_double_array(_p(b), b.size, _p(out))
    return out


def keep_from_sparsity(s: float, d: int = 128) -> int:
    return lib().orc_keep_from_sparsity(float(s), int(d))


def prune_rows(x, k: int) -> np.ndarray:
    """x: [..., d] fp16 -> uint8 keep mask of the same shape."""
    x = _u16(x)
    d = x.shape[-1]
    keep = np.zeros(x.shape, dtype=np.uint8)
    lib().orc_prune_rows(_p(x), x.size // d, d, int(k), _p(keep))
    return keep


def prune_rows_24(x) -> np.ndarray:
    """x: [..., d] fp16, d % 4 == 0 -> uint8 keep mask (2:4 rule, R23)."""
    x = _u16(x)
    d = x.shape[-1]
    keep = np.zeros(x.shape, dtype=np.uint8)
    if lib().orc_prune_rows_24(_p(x), x.size // d, d, _p(keep)) != 0:
        raise ValueError("orc_prune_rows_24: bad arguments")
    return keep


def compress_24(dense, seq_lens, cap: int | None = None, nthreads: int = 0) -> "Compressed":
    """2:4 compression (R23) into the bitmap format with keep = d / 2."""
    x = _u16(dense)
    B, H, T, d = x.shape
    cap = T if cap is None else cap
    cap = (cap + 63) // 64 * 64
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    c = Compressed(B, H, cap, d, d // 2)
    rc = lib().orc_compress_24(_p(x), B, H, T, d, _p(seq), cap, _p(c.bitmaps), _p(c.values),
                               _p(c.tile_off), int(nthreads))
    if rc != 0:
        raise ValueError("orc_compress_24: bad arguments")
    return c


def compress_channel(dense, seq_lens, keep: int, cap: int | None = None,
                     nthreads: int = 0) -> "Compressed":
    """Channel-wise pruning (R24) into the bitmap format: per full 64-row tile each channel
    keeps keep/2 entries; a final partial tile is pruned per token to keep."""
    x = _u16(dense)
    B, H, T, d = x.shape
    cap = T if cap is None else cap
    cap = (cap + 63) // 64 * 64
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    c = Compressed(B, H, cap, d, keep)
    rc = lib().orc_compress_channel(_p(x), B, H, T, d, _p(seq), int(keep), cap, _p(c.bitmaps),
                                    _p(c.values), _p(c.tile_off), int(nthreads))
    if rc != 0:
        raise ValueError("orc_compress_channel: bad arguments")
    return c


class Compressed:
    """One compressed tensor: bitmaps [B][H][cap][d/64] u64, tile_off [B][H][cap/64+1] u32 and
    values: [B][H][cap*k] u16 when every head keeps k; with head_keep (R22: head h keeps
    head_keep[h] per row) values is [B][cap * sum(head_keep)] u16 and the region of (b, h)
    starts at cap * sum(head_keep[:h]) within row b."""

    def __init__(self, B, H, cap, d, k, head_keep=None):
        self.B, self.H, self.cap, self.d, self.k = B, H, cap, d, k
        self.head_keep = None
        self.bitmaps = np.zeros((B, H, cap, d // 64), dtype=np.uint64)
        if head_keep is None:
            self.values = np.zeros((B, H, cap * k), dtype=np.uint16)
        else:
            hk = np.ascontiguousarray(np.asarray(head_keep, dtype=np.int32))
            assert hk.shape == (H,)
            self.head_keep = hk
            self.values = np.zeros((B, cap * int(hk.sum())), dtype=np.uint16)
        self.tile_off = np.zeros((B, H, cap // 64 + 1), dtype=np.uint32)

    def _hk(self):
        return None if self.head_keep is None else _p(self.head_keep)


def compress(dense, seq_lens, k: int, cap: int | None = None, nthreads: int = 0,
             head_keep=None) -> Compressed:
    """dense: [B][H][T][d] fp16 -> Compressed (rows >= seq_lens[b] left zero).  With
    head_keep, head h keeps head_keep[h] channels per row (k is then ignored by the rule)."""
    x = _u16(dense)
    B, H, T, d = x.shape
    cap = T if cap is None else cap
    cap = (cap + 63) // 64 * 64
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    c = Compressed(B, H, cap, d, k, head_keep)
    rc = lib().orc_compress_hk(_p(x), B, H, T, d, _p(seq), int(k), c._hk(), cap, _p(c.bitmaps),
                               _p(c.values), _p(c.tile_off), int(nthreads))
    if rc != 0:
        raise ValueError("orc_compress: bad arguments")
    return c


def append_rows(c: Compressed, rows, seq_lens) -> int:
    """Appends one new row per (b, h) (rows: [B][H][d] fp16) to `c` in place at row
    seq_lens[b], pruned per token (the oracle's append rule).  seq_lens is not changed.
    Returns the status bits (1: some sequence was already at capacity)."""
    x = _u16(rows)
    assert x.shape == (c.B, c.H, c.d), x.shape
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    st = np.zeros(1, dtype=np.uint32)
    rc = lib().orc_append_rows(_p(c.bitmaps), _p(c.values), _p(c.tile_off), c.B, c.H, c.cap, c.d,
                               c.k, c._hk(), _p(x), _p(seq), _p(st))
    if rc != 0:
        raise ValueError("orc_append_rows: bad arguments")
    return int(st[0])


def append_step(kc: Compressed, vc: Compressed, k_new, v_new, seq_lens) -> tuple:
    """One decode-time append to both caches: the new key and value rows are appended
    at seq_lens[b]; returns (new seq_lens, status).  A sequence at capacity keeps its
    length and sets status bit 0."""
    seq = np.asarray(seq_lens, dtype=np.int32)
    st = append_rows(kc, k_new, seq) | append_rows(vc, v_new, seq)
    grown = np.where(np.clip(seq, 0, kc.cap) < kc.cap, np.clip(seq, 0, kc.cap) + 1, np.clip(seq, 0, kc.cap))
    return grown.astype(np.int32), st


def decompress(c: Compressed, seq_lens) -> np.ndarray:
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    out = np.empty((c.B, c.H, c.cap, c.d), dtype=np.uint16)
    rc = lib().orc_decompress_hk(_p(c.bitmaps), _p(c.values), _p(c.tile_off), c.B, c.H, c.cap,
                                 c.d, c.k, c._hk(), _p(seq), _p(out))
    if rc != 0:
        raise ValueError("orc_decompress: bad arguments")
    return out


def used_bytes(B, H, seq_lens, cap, d, k, head_keep=None) -> int:
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if head_keep is None:
        return int(lib().orc_used_bytes(B, H, _p(seq), cap, d, k))
    hk = np.ascontiguousarray(np.asarray(head_keep, dtype=np.int32))
    return int(lib().orc_used_bytes_hk(B, H, _p(seq), cap, d, k, _p(hk)))


def attention_dense(q, K, V, seq_lens, scale: float, nthreads: int = 0) -> np.ndarray:
    """q [B][Hq][d], K/V [B][Hkv][T][d] fp16 -> out [B][Hq][d] float64."""
    qb, Kb, Vb = _u16(q), _u16(K), _u16(V)
    B, Hq, d = qb.shape
    Hkv, T = Kb.shape[1], Kb.shape[2]
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    out = np.zeros((B, Hq, d), dtype=np.float64)
    rc = lib().orc_attention_dense(_p(qb), B, Hq, Hkv, d, _p(Kb), _p(Vb), T, _p(seq), float(scale),
                                   _p(out), int(nthreads))
    if rc != 0:
        raise ValueError("orc_attention_dense: bad arguments")
    return out


def attention_compressed(q, kc: Compressed, vc: Compressed, seq_lens, scale: float,
                         units=None, nthreads: int = 0) -> np.ndarray:
    """Attention over compressed caches; `units` = list of b*Hq+hq to compute (others stay 0)."""
    qb = _u16(q)
    B, Hq, d = qb.shape
    seq = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    out = np.zeros((B, Hq, d), dtype=np.float64)
    if units is None:
        up, n = None, 0
    else:
        u = np.ascontiguousarray(np.asarray(units, dtype=np.int64))
        up, n = _p(u), u.size
    rc = lib().orc_attention_compressed_hk(_p(qb), B, Hq, kc.H, d, _p(kc.bitmaps),
                                           _p(kc.values), _p(kc.tile_off), kc.k, kc._hk(),
                                           _p(vc.bitmaps), _p(vc.values), _p(vc.tile_off), vc.k,
                                           vc._hk(), kc.cap, _p(seq), float(scale), up, n, _p(out),
                                           int(nthreads))
    if rc != 0:
        raise ValueError("orc_attention_compressed: bad arguments")
    return out
