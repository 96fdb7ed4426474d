"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol the header declares, and rejects bad arguments with the documented status
codes before touching a device."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import unstructured_sparse_kv_amd as usk
from tests.conftest import gpu_available

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mustafar.h")

L = usk.lib()
KV = usk.KVStruct
A16 = 0x10000  # aligned, non-null stand-ins: only used where the call must fail before any launch


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mustafar_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    decl = header_symbols()
    assert len(decl) == 18, decl
    assert sorted(usk.EXPORTS) == decl
    nm = subprocess.run(["nm", "-D", "--defined-only", usk.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r" T (mustafar_[a-z0-9_]+)", nm))
    for name in decl:
        assert name in exported, name
        assert hasattr(L, name)


def test_library_carries_gfx950_code_object():
    blob = open(usk.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


@pytest.mark.parametrize("s,k", [(0.0, 128), (0.5, 64), (0.7, 38), (1.0, 0), (0.9, 13)])
def test_keep_from_sparsity_matches_closed_form_and_oracle(s, k):
    assert usk.keep_from_sparsity(s) == k == oracle.keep_from_sparsity(s)


def test_keep_from_sparsity_rejects():
    assert L.mustafar_keep_from_sparsity(1.5, 128) == usk.MUSTAFAR_EINVAL
    assert L.mustafar_keep_from_sparsity(-0.01, 128) == usk.MUSTAFAR_EINVAL
    assert L.mustafar_keep_from_sparsity(float("nan"), 128) == usk.MUSTAFAR_EINVAL
    assert L.mustafar_keep_from_sparsity(0.5, 0) == usk.MUSTAFAR_EINVAL


def _alloc(batch, heads, keep, cap, hd=128):
    s = KV(batch, heads, hd, keep, cap, None, None, None)
    b, v, o = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    rc = L.mustafar_kv_alloc_bytes(ctypes.byref(s), ctypes.byref(b), ctypes.byref(v), ctypes.byref(o))
    return rc, b.value, v.value, o.value


def test_alloc_bytes_closed_form():
    rc, b, v, o = _alloc(8, 8, 38, 32768)
    assert rc == 0
    assert b == 64 * 32768 * 16
    assert v == 64 * 32768 * 38 * 2 + 64
    assert o == 64 * (512 + 1) * 4
    assert _alloc(1, 1, 38, 100)[0] == usk.MUSTAFAR_EINVAL      # capacity not a multiple of 64
    assert _alloc(1, 1, 129, 64)[0] == usk.MUSTAFAR_EINVAL      # keep > head_dim
    assert _alloc(1, 1, -1, 64)[0] == usk.MUSTAFAR_EINVAL
    assert _alloc(1, 1, 38, 64, hd=64)[0] == usk.MUSTAFAR_EUNSUPPORTED
    assert _alloc(0, 1, 38, 64)[0] == usk.MUSTAFAR_EINVAL


def test_used_bytes_matches_oracle_accounting():
    rng = np.random.default_rng(3)
    seq = rng.integers(0, 5000, size=16).astype(np.int32)
    seq[0], seq[1] = 0, 4160
    for keep in (0, 38, 64, 128):
        s = KV(16, 8, 128, keep, 4160, None, None, None)
        out = ctypes.c_int64()
        assert L.mustafar_kv_used_bytes(ctypes.byref(s), seq.ctypes.data_as(ctypes.c_void_p),
                                        ctypes.byref(out)) == 0
        assert out.value == oracle.used_bytes(16, 8, seq, 4160, 128, keep)
    # dense comparison for the Llama-3-8B-shaped layer at 70% sparsity: 35.96% of dense
    s = KV(8, 8, 128, 38, 32768, None, None, None)
    seq = np.full(8, 32768, np.int32)
    out = ctypes.c_int64()
    L.mustafar_kv_used_bytes(ctypes.byref(s), seq.ctypes.data_as(ctypes.c_void_p), ctypes.byref(out))
    assert abs(out.value / (8 * 8 * 32768 * 256) - 0.3596) < 1e-4


def _kv(keep=38, cap=128, bm=A16, vals=A16, toff=A16, batch=1, heads=2, hd=128):
    return KV(batch, heads, hd, keep, cap, bm, vals, toff)


def test_prune_compress_argument_errors():
    f = L.mustafar_prune_compress
    ok = _kv()
    assert f(None, A16, 128, A16, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(_kv(bm=None)), A16, 128, A16, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(_kv(vals=A16 + 2)), A16, 128, A16, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(_kv(hd=64)), A16, 128, A16, None) == usk.MUSTAFAR_EUNSUPPORTED
    assert f(ctypes.byref(_kv(keep=200)), A16, 128, A16, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(_kv(cap=100)), A16, 128, A16, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(ok), A16 + 8, 128, A16, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(ok), A16, 0, A16, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(ok), A16, 128, None, None) == usk.MUSTAFAR_EINVAL


def test_append_argument_errors():
    f = L.mustafar_append_token
    k, v = _kv(), _kv(keep=64)
    assert f(ctypes.byref(k), ctypes.byref(_kv(cap=192)), A16, A16, A16, None, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(k), ctypes.byref(_kv(heads=3)), A16, A16, A16, None, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(k), ctypes.byref(v), None, A16, A16, None, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(k), ctypes.byref(v), A16, A16 + 4, A16, None, None) == usk.MUSTAFAR_EINVAL
    assert f(ctypes.byref(k), ctypes.byref(v), A16, A16, A16, A16 + 2, None) == usk.MUSTAFAR_EINVAL


def _ws_bytes(B, Hq, Hkv, T, splits=0, hd=128):
    out = ctypes.c_uint64()
    rc = L.mustafar_decode_workspace_bytes(B, Hq, Hkv, hd, T, splits, ctypes.byref(out))
    return rc, out.value


def test_workspace_sizing_and_auto_splits():
    rc, n = _ws_bytes(8, 32, 8, 32768)
    sp = L.mustafar_decode_auto_splits(8, 8, 32768)
    assert rc == 0 and 1 <= sp <= 1024
    assert n == 8 * 32 * sp * 132 * 4  # one (m, l, acc[128], pad) partial per (b, q head, split)
    assert _ws_bytes(8, 32, 8, 32768, splits=4)[1] == 8 * 32 * 4 * 132 * 4
    assert _ws_bytes(8, 30, 8, 100)[0] == usk.MUSTAFAR_EINVAL
    assert _ws_bytes(8, 32, 8, 100, hd=96)[0] == usk.MUSTAFAR_EUNSUPPORTED
    assert _ws_bytes(8, 32, 8, 100, splits=5000)[0] == usk.MUSTAFAR_EINVAL
    # small sequences get one split; long single-sequence shapes get many
    assert L.mustafar_decode_auto_splits(1, 2, 256) == 1
    assert L.mustafar_decode_auto_splits(1, 32, 4096) >= 4
    # the documented rule: floor(512 / units), at least 1, at most ceil(tiles / 4)
    assert L.mustafar_decode_auto_splits(8, 8, 32768) == 8
    assert L.mustafar_decode_auto_splits(6, 8, 32768) == 10
    assert L.mustafar_decode_auto_splits(1, 8, 65536) == 64
    assert L.mustafar_decode_auto_splits(64, 8, 16384) == 1
    assert L.mustafar_decode_auto_splits(128, 8, 16384) == 1
    assert L.mustafar_decode_auto_splits(1, 8, 1024) == 4  # 16 tiles: one per wave
    assert L.mustafar_decode_auto_splits(1, 8, 4096) == 16


def test_decode_argument_errors():
    f = L.mustafar_decode_attn
    k, v = _kv(heads=8), _kv(heads=8)
    rc, need = _ws_bytes(1, 32, 8, 128)
    args = lambda **o: dict(dict(q=A16, hq=32, k=ctypes.byref(k), v=ctypes.byref(v), seq=A16, T=128,
                                 scale=0.088, splits=0, out=A16, ws=A16, wsb=need), **o)
    call = lambda a: f(a["q"], a["hq"], a["k"], a["v"], a["seq"], a["T"], a["scale"], a["splits"],
                       a["out"], a["ws"], a["wsb"], None)
    assert call(args(q=None)) == usk.MUSTAFAR_EINVAL
    assert call(args(out=A16 + 8)) == usk.MUSTAFAR_EINVAL
    assert call(args(hq=30)) == usk.MUSTAFAR_EINVAL                  # Hq % Hkv != 0
    assert call(args(hq=24)) == usk.MUSTAFAR_EUNSUPPORTED            # G = 3
    assert call(args(wsb=need - 4)) == usk.MUSTAFAR_ENOSPACE
    assert call(args(scale=float("inf"))) == usk.MUSTAFAR_EINVAL
    assert call(args(splits=-1)) == usk.MUSTAFAR_EINVAL
    assert call(args(v=ctypes.byref(_kv(heads=8, cap=192)))) == usk.MUSTAFAR_EINVAL
    g = L.mustafar_dense_decode_attn
    assert g(A16, 32, A16, A16, 1, 8, 96, 128, A16, 128, 0.1, 0, A16, A16, need, None) == \
        usk.MUSTAFAR_EUNSUPPORTED
    assert g(A16, 32, None, A16, 1, 8, 128, 128, A16, 128, 0.1, 0, A16, A16, need, None) == \
        usk.MUSTAFAR_EINVAL
    assert L.mustafar_probe_stream_read(A16, 1000, A16, None) == usk.MUSTAFAR_EINVAL


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path")
def test_valid_calls_report_no_device():
    k, v = _kv(heads=8), _kv(heads=8)
    rc, need = _ws_bytes(1, 32, 8, 128)
    assert L.mustafar_prune_compress(ctypes.byref(k), A16, 128, A16, None) == usk.MUSTAFAR_ENODEV
    assert L.mustafar_append_token(ctypes.byref(k), ctypes.byref(v), A16, A16, A16, None, None) == \
        usk.MUSTAFAR_ENODEV
    assert L.mustafar_decode_attn(A16, 32, ctypes.byref(k), ctypes.byref(v), A16, 128, 0.088, 0,
                                  A16, A16, need, None) == usk.MUSTAFAR_ENODEV
    assert L.mustafar_decode_workspace_init(A16, 1024, None) == usk.MUSTAFAR_ENODEV
    with pytest.raises(usk.MustafarError):
        usk._check("x", usk.MUSTAFAR_ENODEV)


def test_status_strings():
    for code in range(-5, 1):
        assert usk.status_str(code) not in ("", "unknown status")
    assert usk.status_str(-99) == "unknown status"


def _kv_heads(head_keep, keep=None, batch=2, cap=128, ptrs=A16):
    hk = np.ascontiguousarray(np.asarray(head_keep, dtype=np.int32))
    k = int(hk.max()) if keep is None else keep
    s = KV(batch, hk.size, 128, k, cap, ptrs, ptrs, ptrs, hk.ctypes.data)
    s._hk = hk  # keep the host array alive with the struct
    return s


def test_head_keep_accounting_matches_oracle():
    hk = [26, 50, 0, 128, 38, 37]
    s = _kv_heads(hk, batch=3, cap=192, ptrs=None)
    b, v, o = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    assert L.mustafar_kv_alloc_bytes(ctypes.byref(s), ctypes.byref(b), ctypes.byref(v),
                                     ctypes.byref(o)) == 0
    assert v.value == 3 * 192 * sum(hk) * 2 + 64
    assert b.value == 3 * 6 * 192 * 16 and o.value == 3 * 6 * 4 * 4
    seq = np.array([192, 0, 77], np.int32)
    out = ctypes.c_int64()
    assert L.mustafar_kv_used_bytes(ctypes.byref(s), seq.ctypes.data_as(ctypes.c_void_p),
                                    ctypes.byref(out)) == 0
    assert out.value == oracle.used_bytes(3, 6, seq, 192, 128, 128, head_keep=hk)
    # every head at 38 takes the bytes of the uniform tensor
    su = _kv_heads([38] * 6, batch=3, cap=192, ptrs=None)
    assert L.mustafar_kv_alloc_bytes(ctypes.byref(su), ctypes.byref(b), ctypes.byref(v),
                                     ctypes.byref(o)) == 0
    assert (b.value, v.value, o.value) == _alloc(3, 6, 38, 192)[1:]


def test_head_keep_argument_errors():
    f = L.mustafar_prune_compress
    bad = [
        _kv_heads([38, 40], keep=38),          # keep is not the largest entry
        _kv_heads([38, 129], keep=129),        # entry above head_dim
        _kv_heads([38, -1], keep=38),          # negative entry
        _kv_heads([1] * 129, keep=1),          # more kv heads than a per-head keep may describe
    ]
    for s in bad:
        assert f(ctypes.byref(s), A16, 128, A16, None) == usk.MUSTAFAR_EINVAL
        b = ctypes.c_uint64()
        assert L.mustafar_kv_alloc_bytes(ctypes.byref(s), ctypes.byref(b), ctypes.byref(b),
                                         ctypes.byref(b)) == usk.MUSTAFAR_EINVAL
    k = _kv_heads([38, 40])
    v = _kv_heads([38, 40], keep=38)
    assert L.mustafar_append_token(ctypes.byref(k), ctypes.byref(v), A16, A16, A16, None, None) == \
        usk.MUSTAFAR_EINVAL
