"""Shared plumbing for the GPU parity tests: build device caches through the C ABI,
copy results back, compare with the CPU oracle on the same bits."""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle
import unstructured_sparse_kv_amd as usk

MAX_ABS = 1e-2
MAX_REL_L2 = 1e-3
SCALE = 1.0 / math.sqrt(128)
# oracle threads: the CPU share a GPU test may use (16 per GPU), whatever the host shows
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def compress_on_gpu(dense_dev: torch.Tensor, seq_dev: torch.Tensor, keep: int, cap: int):
    B, H = dense_dev.shape[0], dense_dev.shape[1]
    c = usk.CompressedKV(B, H, keep, cap, dense_dev.device)
    usk.prune_compress(c, dense_dev, seq_dev)
    return c


def assert_compressed_equal(c: usk.CompressedKV, ref: oracle.Compressed, seq, units=None, ref_units=None):
    """Bit-exact bitmaps / values / tile offsets over the rows < seq[b] of the listed
    (b, h) units; ref may hold only those units (ref_units gives their index in ref)."""
    bm, vals, toff = c.views()
    bm = bm.cpu().numpy().view(np.uint64)
    vals = vals.cpu().numpy().view(np.uint16)
    toff = toff.cpu().numpy().view(np.uint32)
    B, H = c.batch, c.num_kv_heads
    units = [(b, h) for b in range(B) for h in range(H)] if units is None else units
    ref_units = units if ref_units is None else ref_units
    for (b, h), (rb, rh) in zip(units, ref_units):
        T = max(0, min(int(seq[b]), c.capacity))
        nt = (T + 63) // 64 + 1
        assert np.array_equal(bm[b, h, :T], ref.bitmaps[rb, rh, :T]), f"bitmaps differ at unit {(b, h)}"
        assert np.array_equal(vals[b, h, :T * c.keep], ref.values[rb, rh, :T * c.keep]), \
            f"values differ at unit {(b, h)}"
        assert np.array_equal(toff[b, h, :nt], ref.tile_off[rb, rh, :nt]), \
            f"tile offsets differ at unit {(b, h)}: {toff[b, h, :nt][:8]} vs {ref.tile_off[rb, rh, :nt][:8]}"


def attn_errors(got: np.ndarray, ref: np.ndarray):
    got = got.astype(np.float64)
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    return err, rel


def assert_attn_close(got: np.ndarray, ref: np.ndarray, what: str):
    err, rel = attn_errors(got, ref)
    say(f"{what}: max_abs={err:.3e} rel_l2={rel:.3e}")
    assert err <= MAX_ABS and rel <= MAX_REL_L2, (what, err, rel)


def oracle_attention_units(q_cpu, K_cpu, V_cpu, seq, kk, kv, cap, pairs, G):
    """fp64 oracle output for the listed (b, hq) pairs, each computed from its own
    (b, kv head) slice of the dense caches: compress (oracle rule) then attend."""
    out = {}
    for b, hq in pairs:
        h = hq // G
        T = int(seq[b])
        Kb = K_cpu[b:b + 1, h:h + 1]
        Vb = V_cpu[b:b + 1, h:h + 1]
        s1 = np.array([T], np.int32)
        kc = oracle.compress(Kb, s1, kk, cap)
        vc = oracle.compress(Vb, s1, kv, cap)
        qb = q_cpu[b:b + 1, hq:hq + 1]
        out[(b, hq)] = oracle.attention_compressed(qb, kc, vc, s1, SCALE)[0, 0]
    return out
