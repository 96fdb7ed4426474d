#!/usr/bin/env python3
"""Benchmark of the MUSTAFAR decode step on one MI355X.

Workload: Llama-3-8B-shaped attention layers -- batch 8, 32 query heads over 8
kv heads, head_dim 128, 32768 cached tokens per sequence, key and value caches
pruned per token to 70% sparsity (38 of 128 channels kept) and bitmap-compressed.
Inputs are seeded synthetic data (keys N(0,1) with 4 outlier channels x10 per
kv head; values and queries N(0,1)), generated on the GPU.

A step is one pass of the decode hot path on one layer: the new key and value
row of every (sequence, kv head) is pruned and appended to the layer's
compressed caches and decode attention runs over them, in one fused call
(mustafar_decode_step; the same steps as separate mustafar_append_token +
mustafar_decode_attn calls are timed too).  Steps take turns over --layers layers (3 by default)
the way a model's decode loop visits its layers, so a step's caches (386 MB)
are not still in the 256 MB last-level cache from the step before.  `value` is
compressed key+value bytes read per step divided by the wall time of the timed
steps (GB/s).

Also reported: the decode call's own rate against the 8 TB/s HBM peak
(`roofline`, HIP events on the launch stream over the timed steps), the same
call on one layer repeated and after a 1 GiB read of other memory, the
vector-unit sparse kernel and the dense fp16 comparison kernel (batch 8 and 6)
after the same 1 GiB read, the prefill prune+compress rate, the measured
stream-read rate of the device, and the CPU oracle timed on one full decode
step (`cpu_baseline`).

Before the W warmup steps, read-only decode calls run for --ramp-s seconds (0.3 by
default) so that the timed steps see the clocks of sustained work, not of a GPU
that was idle.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--ramp-s S]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "sparse decode-attn GB/s (% HBM peak) + speedup vs dense fp16, Llama-3-8B shape 70%"
PROFILES = os.path.join(ROOT, "profiles")
# sources of the timed decode call (split kernel, its helpers, the merge kernel, the launcher)
DECODE_SOURCES = ["decode_sparse_mfma.hpp", "decode_sparse_mfma_g4.hip", "decode_walk.hpp", "merge.hpp", "tile_softmax.hpp", "device_common.hpp",
                  "kernels.hpp", "select_row.hpp", "util.hip", "api.hip"]
DECODE_KERNELS = "decode_sparse_mfma_kernel<4,40,38> + decode_reduce_kernel"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "unstructured_sparse_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "decode_sparse_llama3_8b_layer_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def stack_sweep(args) -> int:
    """The 32-layer Llama-3-8B-shaped stack: for B in {1,4,8,16,32,64} x T in
    {16384, 65536, 131072}, the KV bytes of the whole stack against 288e9 B
    (compressed and dense fp16) and, where the stack fits, the decode-attention
    tokens/s = B / (32 x the per-layer decode-attention time).  The per-layer
    time is measured over 3 layer caches of the point's shape taken in turn
    (so each is read cold, as in a 32-layer decode step).  One sequence per T
    is generated and pruned; the batch is filled with copies of its caches
    (timing depends on the shapes and the per-row keep, not on the values)."""
    import numpy as np
    import torch

    import synth
    import unstructured_sparse_kv_amd as usk

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfg = synth.CONFIGS["llama3_8b_stack"]
    Hq, Hkv, d, L = cfg.Hq, cfg.Hkv, cfg.d, cfg.layers
    keep = usk.keep_from_sparsity(cfg.sparsity)
    budget = 288e9
    NL = 3
    scale = 1.0 / math.sqrt(d)

    def per_layer_time(call, n_layers):
        for i in range(n_layers):
            call(i)
        torch.cuda.synchronize()
        ts = []
        for j in range(2 * n_layers):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(j % n_layers)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return median(ts)

    points = []
    max_batch = {}
    for T in (16384, 65536, 131072):
        K1, V1, _, _ = synth.make_inputs(cfg, device=dev, layer=0, B=1, T=T)
        seq1 = torch.full((1,), T, dtype=torch.int32, device=dev)
        kc1, vc1 = usk.CompressedKV(1, Hkv, keep, T, dev), usk.CompressedKV(1, Hkv, keep, T, dev)
        usk.prune_compress(kc1, K1, seq1)
        usk.prune_compress(vc1, V1, seq1)
        torch.cuda.synchronize()
        comp_seq = (kc1.used_bytes([T]) + vc1.used_bytes([T])) * L
        dense_seq = 2 * Hkv * T * d * 2 * L
        max_batch[T] = {"compressed": int(budget // comp_seq), "dense": int(budget // dense_seq)}
        for B in (1, 4, 8, 16, 32, 64):
            pt = {"batch": B, "seq_len": T, "stack_kv_bytes_compressed": B * comp_seq,
                  "stack_kv_bytes_dense": B * dense_seq, "fits_compressed": B * comp_seq <= budget,
                  "fits_dense": B * dense_seq <= budget}
            q = synth.normal_f16(cfg.seed, synth.S_Q, 0, (B, Hq, d), dev)
            seq = torch.full((B,), T, dtype=torch.int32, device=dev)
            out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
            if pt["fits_compressed"]:
                layers = []
                for _ in range(NL):
                    kc, vc = usk.CompressedKV(B, Hkv, keep, T, dev), usk.CompressedKV(B, Hkv, keep, T, dev)
                    for dst, src in ((kc, kc1), (vc, vc1)):
                        for a, b in zip(dst.views(), src.views()):
                            a.copy_(b.expand_as(a))
                    layers.append((kc, vc))
                ws = usk.make_workspace(B, Hq, Hkv, T)
                t = per_layer_time(lambda i: usk.decode_attn(q, layers[i][0], layers[i][1], seq, T, scale,
                                                             out, ws), NL)
                pt["sparse_layer_us"] = round(t * 1e6, 2)
                pt["sparse_tokens_per_s"] = round(B / (L * t), 1)
                pt["sparse_gbs"] = round(B * comp_seq / L / t / 1e9, 1)
                del layers, ws
            if pt["fits_dense"]:
                layers = []
                for _ in range(NL):
                    Kd = K1.expand(B, Hkv, T, d).contiguous()
                    Vd = V1.expand(B, Hkv, T, d).contiguous()
                    layers.append((Kd, Vd))
                ws = usk.make_workspace(B, Hq, Hkv, T)
                t = per_layer_time(lambda i: usk.dense_decode_attn(q, layers[i][0], layers[i][1], seq, T,
                                                                   scale, out, ws), NL)
                pt["dense_layer_us"] = round(t * 1e6, 2)
                pt["dense_tokens_per_s"] = round(B / (L * t), 1)
                del layers, ws
            torch.cuda.empty_cache()
            log(f"stack B={B} T={T}: " + ", ".join(f"{k}={v}" for k, v in pt.items()
                                                   if k.endswith(("_us", "_per_s")) or k.startswith("fits")))
            points.append(pt)
        del K1, V1, kc1, vc1
        torch.cuda.empty_cache()
    res = {"metric": "32-layer stack: max batch in 288 GB (KV bytes) and decode-attention tokens/s",
           "unit": "tokens/s", "n_gpus": 1, "dtype": "f16 in, f32 accumulate", "data": "synthetic",
           "config": {"workload": "llama3_8b_stack: 32 layers, GQA 32/8, head_dim 128, keep 38 of 128",
                      "layers_timed_in_turn": NL},
           "max_batch_288GB": {str(k): v for k, v in max_batch.items()}, "points": points}
    print(json.dumps(res), flush=True)
    return 0


def _timed(stream, fn, n, before=None):
    """n calls of fn, each bracketed by its own pair of HIP events on `stream`
    (after `before`, which is not timed); returns the seconds of each."""
    import torch
    ts = []
    for _ in range(n):
        if before is not None:
            before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    return ts


def _oracle_threads():
    import oracle
    hw = oracle.hardware_threads()
    nproc = len(os.sched_getaffinity(0))
    # the GPU machine grants each GPU a 16-core share of the host, whatever the host shows
    return hw, nproc, max(1, min(16, nproc))


def _caches_equal(c, o, seq, keep):
    import numpy as np
    bm, vals, toff = (t.cpu().numpy() for t in c.views())
    bm, vals, toff = bm.view(np.uint64), vals.view(np.uint16), toff.view(np.uint32)
    for b in range(c.batch):
        T = int(seq[b])
        nt = (T + 63) // 64 + 1
        if not (np.array_equal(bm[b, :, :T], o.bitmaps[b, :, :T])
                and np.array_equal(vals[b, :, :T * keep], o.values[b, :, :T * keep])
                and np.array_equal(toff[b, :, :nt], o.tile_off[b, :, :nt])):
            return False
    return True


def bench_llama2_layer(args) -> int:
    """The Llama-2-7B-shaped layer at batch 1 (32/32 heads, T=4096, keep 38): its
    compressed caches (24 MB) fit in the 256 MB last-level cache, so every timed
    step follows a 1 GiB read of other memory.  A step is one fused
    mustafar_decode_step (append one row per kv head, attend)."""
    import numpy as np
    import torch

    import oracle
    import synth
    import unstructured_sparse_kv_amd as usk

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfg = synth.CONFIGS["llama2_7b_layer"]
    B, Hq, Hkv, T0, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d
    keep = usk.keep_from_sparsity(cfg.sparsity)
    scale = 1.0 / math.sqrt(d)
    total = args.warmup + args.steps
    cap = (T0 + total + 63) // 64 * 64
    K, V, _, _ = synth.make_inputs(cfg, device=dev, T=cap)
    seq_d = torch.full((B,), T0, dtype=torch.int32, device=dev)
    kc, vc = usk.CompressedKV(B, Hkv, keep, cap, dev), usk.CompressedKV(B, Hkv, keep, cap, dev)
    pre = _timed(stream, lambda: (usk.prune_compress(kc, K, seq_d), usk.prune_compress(vc, V, seq_d)), 3)
    steps_in = [synth.step_inputs(cfg, i, device=dev) for i in range(total)]
    ws = usk.make_workspace(B, Hq, Hkv, cap)
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    before = lambda: usk.probe_stream_read(flush, sink)  # noqa: E731
    # clock ramp: read-only decode calls
    t_r = time.perf_counter()
    while time.perf_counter() - t_r < args.ramp_s:
        for _ in range(50):
            usk.decode_attn(steps_in[0][2], kc, vc, seq_d, cap, scale, out, ws)
        torch.cuda.synchronize()
    it = iter(range(total))
    step_fn = lambda: (lambda i: usk.decode_step(steps_in[i][2], kc, vc, steps_in[i][0], steps_in[i][1],  # noqa: E731
                                                 seq_d, cap, scale, out, ws, status))(next(it))
    _timed(stream, step_fn, args.warmup, before)
    ts = _timed(stream, step_fn, args.steps, before)
    assert status.item() == 0
    L = T0 + total
    seq_fin = np.full(B, L, np.int32)
    step_s = median(ts)
    nbytes = kc.used_bytes(np.full(B, L - 1, np.int32)) + vc.used_bytes(np.full(B, L - 1, np.int32))
    achieved = nbytes / step_s / 1e9
    # read-only decode and the dense kernel over the same T0 rows, after the same read (the
    # steps' final length, T0 + 55 rows, is 65 tiles: one wave of the 64 then walks two)
    seq_t0 = torch.full((B,), T0, dtype=torch.int32, device=dev)
    dec_s = median(_timed(stream, lambda: usk.decode_attn(steps_in[-1][2], kc, vc, seq_t0, T0, scale,
                                                          out, ws), 20, before))
    wsd = usk.make_workspace(B, Hq, Hkv, T0)
    outd = torch.empty_like(out)
    dense_s = median(_timed(stream, lambda: usk.dense_decode_attn(steps_in[-1][2], K, V, seq_t0, T0, scale,
                                                                  outd, wsd), 20, before))
    comp_t0 = kc.used_bytes(np.full(B, T0, np.int32)) + vc.used_bytes(np.full(B, T0, np.int32))
    dense_bytes = 2 * B * Hkv * T0 * d * 2
    log(f"llama2 layer: fused step {step_s * 1e6:.2f} us ({achieved:.0f} GB/s, "
        f"{achieved / HBM_PEAK_GBS:.1%}); decode only {dec_s * 1e6:.2f} us; dense {dense_s * 1e6:.2f} us")
    # oracle: same prefill bits, its own appends, the last step's query
    usk.decode_attn(steps_in[-1][2], kc, vc, seq_d, cap, scale, out, ws)
    torch.cuda.synchronize()
    hw, nproc, nth = _oracle_threads()
    Kc, Vc = K[:, :, :T0].cpu(), V[:, :, :T0].cpu()
    seq0 = np.full(B, T0, np.int32)
    c0 = time.perf_counter()
    ko = oracle.compress(Kc, seq0, keep, cap, nthreads=nth)
    vo = oracle.compress(Vc, seq0, keep, cap, nthreads=nth)
    cpu_pre = time.perf_counter() - c0
    seq_o = seq0
    for i in range(total):
        seq_o, st = oracle.append_step(ko, vo, steps_in[i][0].cpu(), steps_in[i][1].cpu(), seq_o)
    c0 = time.perf_counter()
    ref = oracle.attention_compressed(steps_in[-1][2].cpu(), ko, vo, seq_o, scale, nthreads=nth)
    cpu_s = time.perf_counter() - c0
    got = out.float().cpu().numpy().astype(np.float64)
    exact = _caches_equal(kc, ko, seq_fin, keep) and _caches_equal(vc, vo, seq_fin, keep)
    err = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    ok = exact and err <= 1e-2 and rel <= 1e-3
    res = {
        "metric": "sparse decode step GB/s (% HBM peak), Llama-2-7B layer at batch 1, after a 1 GiB read",
        "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16 in, f32 accumulate", "data": "synthetic (seeded)",
        "config": {"workload": "llama2_7b_layer: B=1, 32 q / 32 kv heads, head_dim 128, T=4096, keep 38; "
                               "step = mustafar_decode_step after a 1 GiB read of other memory",
                   "batch": B, "q_heads": Hq, "kv_heads": Hkv, "seq_len": T0, "keep": keep},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(nbytes), "avg_launch_us": round(step_s * 1e6, 2)},
        "cpu_baseline": {"value": round(nbytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": nth, "kind": "oracle",
                         "hardware_concurrency": hw, "nproc": nproc, "prefill_compress_s": round(cpu_pre, 4),
                         "sample": "the whole workload: prefill prune + compress of K and V and one decode "
                                   f"step over all {B * Hq} (batch, q head) pairs"},
        "extra": {"decode_only_us": round(dec_s * 1e6, 2), "dense_us": round(dense_s * 1e6, 2),
                  "decode_only_and_dense_seq_len": T0,
                  "speedup_vs_dense": round(dense_s / dec_s, 3),
                  "prefill_compress_us": round(median(pre) * 1e6, 2),
                  "compressed_kv_bytes": int(comp_t0), "dense_kv_bytes": int(dense_bytes),
                  "step_us_all": [round(t * 1e6, 2) for t in ts],
                  "parity": {"caches_bit_exact": bool(exact), "max_abs": err, "rel_l2": rel}},
    }
    print(json.dumps(res), flush=True)
    return 0 if ok else 3


def bench_ragged_append(args) -> int:
    """The Mistral-shaped ragged batch (B=16, 32 q / 8 kv heads, lengths uniform in
    [4096, 32768], keep 64): 64 fused decode steps, each appending one key and
    value row per (sequence, kv head) and attending.  Timed back to back with one
    event pair (the whole sequence), then per step in a second pass of 64 steps."""
    import numpy as np
    import torch

    import oracle
    import synth
    import unstructured_sparse_kv_amd as usk

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfg = synth.CONFIGS["mistral_ragged_append"]
    B, Hq, Hkv, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.d
    keep = usk.keep_from_sparsity(cfg.sparsity)
    scale = 1.0 / math.sqrt(d)
    nsteps = cfg.steps
    seq0 = synth.seq_lens_uniform(cfg.seed, B, *cfg.ragged).numpy().astype(np.int32)
    Tmax = cfg.ragged[1]
    cap = (Tmax + 2 * nsteps + 63) // 64 * 64
    K, V, _, _ = synth.make_inputs(cfg, device=dev, T=cap)
    seq_d = torch.from_numpy(seq0).to(dev)
    kc, vc = usk.CompressedKV(B, Hkv, keep, cap, dev), usk.CompressedKV(B, Hkv, keep, cap, dev)
    usk.prune_compress(kc, K, seq_d)
    usk.prune_compress(vc, V, seq_d)
    steps_in = [synth.step_inputs(cfg, i, device=dev) for i in range(2 * nsteps)]
    ws = usk.make_workspace(B, Hq, Hkv, cap)
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t_r = time.perf_counter()
    while time.perf_counter() - t_r < args.ramp_s:
        for _ in range(20):
            usk.decode_attn(steps_in[0][2], kc, vc, seq_d, cap, scale, out, ws)
        torch.cuda.synchronize()

    def step(i):
        kn, vn, q = steps_in[i]
        usk.decode_step(q, kc, vc, kn, vn, seq_d, cap, scale, out, ws, status)

    def step_bytes(i):  # compressed bytes the step reads (lengths after its append)
        sh = np.minimum(seq0 + i + 1, cap)
        return kc.used_bytes(sh) + vc.used_bytes(sh)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(nsteps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    seq_total = e0.elapsed_time(e1) * 1e-3
    total_bytes = sum(step_bytes(i) for i in range(nsteps))
    per = []
    for i in range(nsteps, 2 * nsteps):
        per.append(_timed(stream, lambda: step(i), 1)[0])
    assert status.item() == 0
    per_gbs = [step_bytes(nsteps + j) / t / 1e9 for j, t in enumerate(per)]
    value = total_bytes / seq_total / 1e9
    log(f"ragged append: 64 fused steps in {seq_total * 1e3:.3f} ms ({value:.0f} GB/s, "
        f"{value / HBM_PEAK_GBS:.1%}); per step {median(per) * 1e6:.1f} us median")
    # dense comparison over the final lengths (the dense caches of the prefill rows)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    seq_pre = torch.from_numpy(seq0).to(dev)
    wsd = usk.make_workspace(B, Hq, Hkv, cap)
    outd = torch.empty_like(out)
    dense_s = median(_timed(stream, lambda: usk.dense_decode_attn(steps_in[-1][2], K, V, seq_pre, Tmax, scale,
                                                                  outd, wsd), 10,
                            lambda: usk.probe_stream_read(flush, sink)))
    sparse_s = median(_timed(stream, lambda: usk.decode_attn(steps_in[-1][2], kc, vc, seq_pre, Tmax, scale,
                                                             outd, ws), 10,
                             lambda: usk.probe_stream_read(flush, sink)))
    del flush
    # oracle: prefill from the same dense bits, its own 128 appends, the last query
    usk.decode_attn(steps_in[-1][2], kc, vc, seq_d, cap, scale, out, ws)
    torch.cuda.synchronize()
    hw, nproc, nth = _oracle_threads()
    c0 = time.perf_counter()
    ko = oracle.compress(K.cpu(), seq0, keep, cap, nthreads=nth)
    vo = oracle.compress(V.cpu(), seq0, keep, cap, nthreads=nth)
    cpu_pre = time.perf_counter() - c0
    seq_o = seq0
    c0 = time.perf_counter()
    for i in range(2 * nsteps):
        seq_o, st = oracle.append_step(ko, vo, steps_in[i][0].cpu(), steps_in[i][1].cpu(), seq_o)
    cpu_app = time.perf_counter() - c0
    c0 = time.perf_counter()
    ref = oracle.attention_compressed(steps_in[-1][2].cpu(), ko, vo, seq_o, scale, nthreads=nth)
    cpu_s = time.perf_counter() - c0
    got = out.float().cpu().numpy().astype(np.float64)
    exact = _caches_equal(kc, ko, seq_o, keep) and _caches_equal(vc, vo, seq_o, keep)
    err = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    ok = exact and err <= 1e-2 and rel <= 1e-3 and np.array_equal(seq_d.cpu().numpy(), seq_o)
    last_bytes = step_bytes(2 * nsteps - 1)
    res = {
        "metric": "sparse decode step GB/s (% HBM peak), Mistral-7B-shaped ragged batch, 64 fused steps at 50%",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": nsteps, "warmup": 0,
        "ms_per_step": round(seq_total / nsteps * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16 in, f32 accumulate", "data": "synthetic (seeded)",
        "config": {"workload": "mistral_ragged_append: B=16, 32 q / 8 kv heads, head_dim 128, lengths "
                               "uniform in [4096, 32768], keep 64; 64 mustafar_decode_step calls back to back",
                   "batch": B, "q_heads": Hq, "kv_heads": Hkv, "seq_lens": seq0.tolist(), "keep": keep},
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(total_bytes / nsteps),
                     "avg_launch_us": round(seq_total / nsteps * 1e6, 2)},
        "cpu_baseline": {"value": round(last_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": nth,
                         "kind": "oracle", "hardware_concurrency": hw, "nproc": nproc,
                         "prefill_compress_s": round(cpu_pre, 3), "append_128_steps_s": round(cpu_app, 3),
                         "sample": f"prefill prune + compress of the batch's K and V, 128 appends, and one "
                                   f"decode step over all {B * Hq} (batch, q head) pairs ({cpu_s:.2f} s)"},
        "extra": {"per_step_gbs": {"min": round(min(per_gbs), 1), "median": round(median(per_gbs), 1),
                                   "max": round(max(per_gbs), 1)},
                  "per_step_us_with_events": [round(t * 1e6, 2) for t in per],
                  "decode_only_us_after_1gib_read": round(sparse_s * 1e6, 2),
                  "dense_us_after_1gib_read": round(dense_s * 1e6, 2),
                  "speedup_vs_dense": round(dense_s / sparse_s, 3),
                  "parity": {"caches_bit_exact": bool(exact), "max_abs": err, "rel_l2": rel}},
    }
    print(json.dumps(res), flush=True)
    return 0 if ok else 3


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ramp-s", type=float, default=0.3,
                    help="seconds of read-only decode calls before the warmup steps (clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the per-head keep, channel-wise and 2:4 measurements")
    ap.add_argument("--stack-sweep", action="store_true",
                    help="instead of the benchmark: the 32-layer stack batch x length sweep")
    ap.add_argument("--workload", default="llama3_8b_layer",
                    choices=["llama3_8b_layer", "llama2_7b_layer", "mistral_ragged_append"],
                    help="llama3_8b_layer (default): the headline layer; the others: their own JSON line")
    ap.add_argument("--layers", type=int, default=3,
                    help="layer caches the steps take turns over (>= 2 keeps them out of the LLC)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: every "
              "(batch, kv head) unit of the decode step is independent, so more GPUs would each "
              "run this same path on their own units", file=sys.stderr)
        return 2
    if args.stack_sweep:
        return stack_sweep(args)
    if args.workload == "llama2_7b_layer":
        return bench_llama2_layer(args)
    if args.workload == "mistral_ragged_append":
        return bench_ragged_append(args)

    import numpy as np
    import torch

    import synth
    import unstructured_sparse_kv_amd as usk

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfg = synth.CONFIGS["llama3_8b_layer"]
    B, Hq, Hkv, T0, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d
    keep = usk.keep_from_sparsity(cfg.sparsity)
    NL = args.layers
    sep_steps = min(args.steps, 20)  # steps timed again with separate append + decode calls
    total_steps = args.warmup + args.steps + sep_steps + 1
    cap = (T0 + (total_steps + NL - 1) // NL + 1 + 63) // 64 * 64
    scale = 1.0 / math.sqrt(d)

    # ---- NL layers of the workload's shape, each pruned + compressed from its own
    # synthetic dense caches (layer 0's dense caches stay for the dense comparison)
    kcs, vcs, seqs = [], [], []
    pre = []
    K0 = V0 = None
    for layer in range(NL):
        log(f"layer {layer}: synthetic caches B={B} Hkv={Hkv} T={T0} (capacity {cap}) on the GPU")
        K, V, _, _ = synth.make_inputs(cfg, device=dev, layer=layer, T=cap)  # rows >= T0: spare room
        seq_d = torch.full((B,), T0, dtype=torch.int32, device=dev)
        kc = usk.CompressedKV(B, Hkv, keep, cap, dev)
        vc = usk.CompressedKV(B, Hkv, keep, cap, dev)
        usk.prune_compress(kc, K, seq_d)
        usk.prune_compress(vc, V, seq_d)
        torch.cuda.synchronize()
        if layer == 0:
            K0, V0 = K, V  # kept for the prefill timing and the dense comparison
        else:
            del K, V
        kcs.append(kc)
        vcs.append(vc)
        seqs.append(seq_d)
    steps_in = [synth.step_inputs(cfg, i, device=dev) for i in range(total_steps)]
    torch.cuda.synchronize()
    seq_host = np.full(B, T0, np.int32)
    comp_bytes0 = kcs[0].used_bytes(seq_host) + vcs[0].used_bytes(seq_host)
    dense_bytes0 = 2 * B * Hkv * T0 * d * 2

    ws = usk.make_workspace(B, Hq, Hkv, cap)
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    lens = [T0] * NL

    # A step appends the new token's key and value rows to one layer's caches and
    # runs decode attention over them; the layers take turns, as in a model's
    # decode loop, so a step's caches were last read NL steps earlier (NL layers
    # of compressed caches exceed the 256 MB last-level cache).
    # A step is one mustafar_decode_step call: it prunes, compresses and stores
    # the new rows and attends over the caches in two launches.
    # After idle the GPU raises its clocks over a few hundred milliseconds of sustained
    # work: measured on this workload, the first ~50 decode calls take ~15% longer than
    # calls after ~0.3 s.  A decode loop runs at the sustained clocks, so before the
    # warmup steps the layers' caches are read by decode calls, which change nothing,
    # for --ramp-s seconds.
    ramp_calls = 0
    q_ramp = steps_in[0][2]
    t_r = time.perf_counter()
    while time.perf_counter() - t_r < args.ramp_s:
        for _ in range(50):
            layer = ramp_calls % NL
            usk.decode_attn(q_ramp, kcs[layer], vcs[layer], seqs[layer], cap, scale, out, ws)
            ramp_calls += 1
        torch.cuda.synchronize()
    log(f"clock ramp: {ramp_calls} read-only decode calls in {time.perf_counter() - t_r:.2f} s")

    # prefill prune + compress of layer 0's K and V, timed at the same clocks
    # and the same way as the decode steps: one event pair around 10 pairs of
    # calls issued back to back, three times, the median per pair (every call
    # rewrites layer 0's caches with the same bits: same dense input, same lengths)
    for _ in range(2):
        usk.prune_compress(kcs[0], K0, seqs[0])
        usk.prune_compress(vcs[0], V0, seqs[0])
    torch.cuda.synchronize()
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            usk.prune_compress(kcs[0], K0, seqs[0])
            usk.prune_compress(vcs[0], V0, seqs[0])
        e1.record(stream)
        torch.cuda.synchronize()
        pre.append(e0.elapsed_time(e1) * 1e-3 / 10)
    prefill_s = median(pre)
    log(f"prefill prune+compress K and V: {prefill_s * 1e6:.1f} us "
        f"({(dense_bytes0 + comp_bytes0) / prefill_s / 1e9:.0f} GB/s moved)")

    for i in range(args.warmup):
        layer = i % NL
        kn, vn, q = steps_in[i]
        usk.decode_step(q, kcs[layer], vcs[layer], kn, vn, seqs[layer], cap, scale, out, ws, status)
        lens[layer] += 1
    torch.cuda.synchronize()

    def timed_steps(first, count, fused):
        """`count` steps from steps_in[first], back to back; returns (wall seconds,
        GPU seconds between two events recorded around all of them, bytes)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for j in range(count):
            layer = (first + j) % NL
            kn, vn, q = steps_in[first + j]
            if fused:
                usk.decode_step(q, kcs[layer], vcs[layer], kn, vn, seqs[layer], cap, scale, out, ws,
                                status)
            else:
                usk.append_token(kcs[layer], vcs[layer], kn, vn, seqs[layer], status)
                usk.decode_attn(q, kcs[layer], vcs[layer], seqs[layer], cap, scale, out, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        nbytes = 0
        for j in range(count):
            layer = (first + j) % NL
            lens[layer] += 1
            sh = np.full(B, lens[layer], np.int32)
            nbytes += kcs[layer].used_bytes(sh) + vcs[layer].used_bytes(sh)
        return wall, e0.elapsed_time(e1) * 1e-3, nbytes

    # ---- timed steps (fused calls): wall clock and HIP events around all of them
    wall, gpu_s, total_bytes = timed_steps(args.warmup, args.steps, True)
    assert status.item() == 0
    for layer in range(NL):
        assert np.array_equal(seqs[layer].cpu().numpy(), np.full(B, lens[layer], np.int32))
    value = total_bytes / wall / 1e9
    ms_per_step = wall / args.steps * 1e3
    per_launch_bytes = total_bytes / args.steps
    kern_avg = gpu_s / args.steps
    achieved = per_launch_bytes / kern_avg / 1e9
    kern_s = [kern_avg]
    log(f"step: {ms_per_step * 1e3:.1f} us wall ({value:.0f} GB/s); GPU time per step "
        f"{kern_avg * 1e6:.1f} us = {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s)")

    # ---- the same steps as separate append + decode calls (three launches)
    sep_wall, sep_gpu, sep_bytes = timed_steps(args.warmup + args.steps, sep_steps, False)
    assert status.item() == 0
    log(f"separate append + decode calls: {sep_wall / sep_steps * 1e6:.1f} us per step wall, "
        f"{sep_gpu / sep_steps * 1e6:.1f} us GPU ({sep_bytes / sep_wall / 1e9:.0f} GB/s)")

    kc, vc, seq_d = kcs[0], vcs[0], seqs[0]
    kn, vn, q_last = steps_in[-1]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush.fill_(1)

    def timed(fn, n, before=None):
        ts = []
        for _ in range(n):
            if before is not None:
                before()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return ts

    # ---- one layer again and again: its caches partly stay in the last-level cache
    warm_s = median(timed(lambda: usk.decode_attn(q_last, kc, vc, seq_d, cap, scale, out, ws), 10))
    # ---- after a 1 GiB read of other memory (clean lines) before every call
    cold_s = median(timed(lambda: usk.decode_attn(q_last, kc, vc, seq_d, cap, scale, out, ws), 10,
                          before=lambda: usk.probe_stream_read(flush, sink)))
    bytes_l0 = kc.used_bytes(np.full(B, lens[0], np.int32)) + vc.used_bytes(np.full(B, lens[0], np.int32))
    log(f"layer 0 decode: repeated {warm_s * 1e6:.1f} us, after a 1 GiB read {cold_s * 1e6:.1f} us "
        f"({bytes_l0 / cold_s / 1e9:.0f} GB/s)")

    # ---- achievable read rate (stream-read probe) and write rate (workspace clear)
    reads = timed(lambda: usk.probe_stream_read(flush, sink), 5)
    stream_read_gbs = flush.numel() / min(reads) / 1e9
    log(f"stream-read probe: {stream_read_gbs:.0f} GB/s")

    # ---- the vector-unit sparse kernel on the same caches (comparison)
    valu_s = median(timed(lambda: usk.decode_attn_valu(q_last, kc, vc, seq_d, cap, scale, out, ws), 10,
                          before=lambda: usk.probe_stream_read(flush, sink)))
    log(f"vector-unit sparse decode (mustafar_decode_attn_valu), after a 1 GiB read: "
        f"{valu_s * 1e6:.1f} us")

    def variants():
        """Per-head keep, channel-wise pruning and the 2:4 comparator on layer 0's dense caches."""
        # ---- per-head keep: layer 0's dense caches pruned with a keep per kv head
        # (mean 38, so the same bytes as the uniform layer); the bucketed walk runs
        kheads = [28, 32, 34, 38, 38, 42, 44, 48]
        vheads = kheads[::-1]
        seq_h = torch.full((B,), T0, dtype=torch.int32, device=dev)
        sh0 = np.full(B, T0, np.int32)
        kch = usk.CompressedKV(B, Hkv, None, cap, dev, head_keep=kheads)
        vch = usk.CompressedKV(B, Hkv, None, cap, dev, head_keep=vheads)
        usk.prune_compress(kch, K0, seq_h)
        usk.prune_compress(vch, V0, seq_h)
        torch.cuda.synchronize()
        hk_s = median(timed(lambda: usk.decode_attn(q_last, kch, vch, seq_h, cap, scale, out, ws), 10,
                            before=lambda: usk.probe_stream_read(flush, sink)))
        hk_bytes = kch.used_bytes(sh0) + vch.used_bytes(sh0)
        log(f"per-head keep K {kheads} / V {vheads}: decode after a 1 GiB read {hk_s * 1e6:.1f} us "
            f"({hk_bytes / hk_s / 1e9:.0f} GB/s, {hk_bytes} bytes)")
        del kch, vch

        # ---- uniform keeps of the 50..80% sparsities (keep 64, 51, 45, 38, 32, 26):
        # layer 0's dense caches pruned at each, decode after a 1 GiB read; GB/s on
        # each keep's own compressed bytes, and relative to keep 38's
        keep_sweep = {}
        for kp in (26, 32, 38, 45, 51, 64):
            kck = usk.CompressedKV(B, Hkv, kp, cap, dev)
            vck = usk.CompressedKV(B, Hkv, kp, cap, dev)
            usk.prune_compress(kck, K0, seq_h)
            usk.prune_compress(vck, V0, seq_h)
            torch.cuda.synchronize()
            t_k = median(timed(lambda: usk.decode_attn(q_last, kck, vck, seq_h, cap, scale, out, ws), 10,
                               before=lambda: usk.probe_stream_read(flush, sink)))
            nb_k = kck.used_bytes(sh0) + vck.used_bytes(sh0)
            keep_sweep[kp] = (t_k, nb_k)
            del kck, vck
        gbs38 = keep_sweep[38][1] / keep_sweep[38][0] / 1e9
        for kp, (t_k, nb_k) in keep_sweep.items():
            log(f"uniform keep {kp}: decode after a 1 GiB read {t_k * 1e6:.1f} us "
                f"({nb_k / t_k / 1e9:.0f} GB/s, {nb_k / t_k / 1e9 / gbs38:.3f} of keep 38's)")

        # dense attention over layer 0's unpruned caches: the reference the pruned
        # variants below are compared with
        wsd0 = usk.make_workspace(B, Hq, Hkv, T0)
        outd0 = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
        usk.dense_decode_attn(q_last, K0, V0, seq_h, T0, scale, outd0, wsd0)
        torch.cuda.synchronize()
        ref_d = outd0.float()
        del wsd0

        def dist(o):
            return float(torch.linalg.norm(o.float() - ref_d) / torch.linalg.norm(ref_d))

        # ---- channel-wise pruning at 70%: layer 0's dense caches, each channel of a
        # 64-row tile keeps 19 rows (38 values per row on average, the same bytes)
        kcw = usk.CompressedKV(B, Hkv, keep, cap, dev)
        vcw = usk.CompressedKV(B, Hkv, keep, cap, dev)
        cw_pre = median(timed(lambda: (usk.prune_compress_channel(kcw, K0, seq_h),
                                       usk.prune_compress_channel(vcw, V0, seq_h)), 3))
        cw_s = median(timed(lambda: usk.decode_attn(q_last, kcw, vcw, seq_h, cap, scale, out, ws), 10,
                            before=lambda: usk.probe_stream_read(flush, sink)))
        cw_bytes = kcw.used_bytes(sh0) + vcw.used_bytes(sh0)
        cw_dist = dist(out)
        ktk = usk.CompressedKV(B, Hkv, keep, cap, dev)
        vtk = usk.CompressedKV(B, Hkv, keep, cap, dev)
        usk.prune_compress(ktk, K0, seq_h)
        usk.prune_compress(vtk, V0, seq_h)
        usk.decode_attn(q_last, ktk, vtk, seq_h, cap, scale, out, ws)
        tok_dist = dist(out)
        log(f"channel-wise pruning, keep {keep}: prefill K and V {cw_pre * 1e6:.0f} us; decode after a "
            f"1 GiB read {cw_s * 1e6:.1f} us ({cw_bytes / cw_s / 1e9:.0f} GB/s); relative L2 distance "
            f"to dense attention {cw_dist:.4f} (per-token pruning at the same keep: {tok_dist:.4f})")
        del kcw, vcw, ktk, vtk

        # ---- 2:4 comparator at 50%: layer 0's dense caches pruned 2:4 and pruned
        # per token to keep 64 (the same bytes); the 2:4 kernel and the unstructured
        # kernel on the 2:4 caches, the unstructured kernel on its own caches; each
        # output's distance to the dense attention over the unpruned caches
        k24 = usk.CompressedKV(B, Hkv, 64, cap, dev)
        v24 = usk.CompressedKV(B, Hkv, 64, cap, dev)
        usk.prune_compress_24(k24, K0, seq_h)
        usk.prune_compress_24(v24, V0, seq_h)
        k64 = usk.CompressedKV(B, Hkv, 64, cap, dev)
        v64 = usk.CompressedKV(B, Hkv, 64, cap, dev)
        usk.prune_compress(k64, K0, seq_h)
        usk.prune_compress(v64, V0, seq_h)
        torch.cuda.synchronize()
        b50 = k24.used_bytes(sh0) + v24.used_bytes(sh0)
        cmp50 = {}
        outs50 = {}
        for name, fn, kc_, vc_ in (("2:4 kernel, 2:4 caches", usk.decode_attn_24, k24, v24),
                                   ("unstructured kernel, 2:4 caches", usk.decode_attn, k24, v24),
                                   ("unstructured kernel, keep-64 caches", usk.decode_attn, k64, v64)):
            t_ = median(timed(lambda: fn(q_last, kc_, vc_, seq_h, cap, scale, out, ws), 10,
                              before=lambda: usk.probe_stream_read(flush, sink)))
            outs50[name] = out.float().clone()
            cmp50[name] = t_
            log(f"50% sparsity, {name}: {t_ * 1e6:.1f} us ({b50 / t_ / 1e9:.0f} GB/s)")
        err50 = {n: dist(o) for n, o in outs50.items()}
        for n, e in err50.items():
            log(f"50% sparsity, {n}: relative L2 distance to dense attention {e:.4f}")
        del k24, v24, k64, v64

        return {
            "keep_sweep_after_1gib_read": {
                str(kp): {"us": round(t_k * 1e6, 2), "bytes": int(nb_k), "gbs": round(nb_k / t_k / 1e9, 1),
                          "of_keep38_gbs": round(nb_k / t_k / 1e9 / gbs38, 3)}
                for kp, (t_k, nb_k) in keep_sweep.items()},
            "head_keep_of_keep38_gbs": round(hk_bytes / hk_s / 1e9 / gbs38, 3),
            "head_keep_k": kheads,
            "head_keep_v": vheads,
            "head_keep_decode_us_after_1gib_read": round(hk_s * 1e6, 2),
            "head_keep_decode_gbs_after_1gib_read": round(hk_bytes / hk_s / 1e9, 1),
            "channel_wise_prefill_us": round(cw_pre * 1e6, 1),
            "channel_wise_decode_us_after_1gib_read": round(cw_s * 1e6, 2),
            "channel_wise_decode_gbs_after_1gib_read": round(cw_bytes / cw_s / 1e9, 1),
            "sparsity70_rel_l2_to_dense": {"per-token": round(tok_dist, 5),
                                           "channel-wise": round(cw_dist, 5)},
            "sparsity50_bytes": int(b50),
            "sparsity50_us_after_1gib_read": {n: round(t_ * 1e6, 2) for n, t_ in cmp50.items()},
            "sparsity50_rel_l2_to_dense": {n: round(e, 5) for n, e in err50.items()},
        }

    var_extra = {} if args.no_variants else variants()

    # ---- dense fp16 comparison kernel (layer 0's caches, unpruned), batch 8 and batch 6
    dense = {}
    if not args.no_dense:
        seq_dense = torch.full((B,), T0, dtype=torch.int32, device=dev)
        for bsz in (8, 6):
            wsd = usk.make_workspace(bsz, Hq, Hkv, T0)
            outd = torch.empty((bsz, Hq, d), dtype=torch.float16, device=dev)
            qb = q_last[:bsz].contiguous()
            Kb, Vb, sb = K0[:bsz], V0[:bsz], seq_dense[:bsz]
            dense[bsz] = median(timed(
                lambda: usk.dense_decode_attn(qb, Kb, Vb, sb, T0, scale, outd, wsd), 10,
                before=lambda: usk.probe_stream_read(flush, sink)))
            log(f"dense fp16 decode B={bsz}, after a 1 GiB read: {dense[bsz] * 1e6:.1f} us "
                f"({bsz * Hkv * T0 * 512 / dense[bsz] / 1e9:.0f} GB/s)")
    del flush

    # ---- the CPU oracle on the same workload: parity of the whole layer and the baseline.
    # The oracle compresses layer 0's prefill cache from the dense bits the GPU
    # pruned (timed: the prefill prune + compress), grows it by its own append
    # with every row the steps appended to layer 0, and attends the last step's
    # query (timed: one decode step).  Its caches must equal the GPU's bit for
    # bit and its output must match the GPU's within the attention tolerance;
    # otherwise the line is printed and the run exits non-zero.
    cpu = None
    parity = None
    parity_ok = True
    if not args.no_cpu_baseline:
        import oracle
        usk.decode_attn(q_last, kc, vc, seq_d, cap, scale, out, ws)
        torch.cuda.synchronize()
        L = int(seq_d[0].item())
        hw = oracle.hardware_threads()
        nproc = len(os.sched_getaffinity(0))
        # the GPU machine grants each GPU a 16-core share of the host, whatever the host shows
        nthreads = max(1, min(16, nproc))
        log(f"CPU oracle: hardware_concurrency={hw}, nproc={nproc}, using {nthreads} threads")
        K0c, V0c = K0[:, :, :T0].cpu(), V0[:, :, :T0].cpu()
        seq0 = np.full(B, T0, np.int32)
        c0 = time.perf_counter()
        ko = oracle.compress(K0c, seq0, keep, cap, nthreads=nthreads)
        vo = oracle.compress(V0c, seq0, keep, cap, nthreads=nthreads)
        cpu_pre_s = time.perf_counter() - c0
        del K0c, V0c
        seq_o = seq0
        for i in range(0, args.warmup + args.steps + sep_steps, NL):  # the steps that visited layer 0
            seq_o, st = oracle.append_step(ko, vo, steps_in[i][0].cpu(), steps_in[i][1].cpu(), seq_o)
            assert st == 0
        assert int(seq_o[0]) == L, (seq_o, L)

        def same(c, o):
            bm, vals, toff = (t.cpu().numpy() for t in c.views())
            nt = (L + 63) // 64 + 1
            return (np.array_equal(bm.view(np.uint64)[:, :, :L], o.bitmaps[:, :, :L])
                    and np.array_equal(vals.view(np.uint16)[:, :, :L * keep], o.values[:, :, :L * keep])
                    and np.array_equal(toff.view(np.uint32)[:, :, :nt], o.tile_off[:, :, :nt]))

        caches_exact = same(kc, ko) and same(vc, vo)
        c0 = time.perf_counter()
        ref = oracle.attention_compressed(q_last.cpu(), ko, vo, seq_o, scale, nthreads=nthreads)
        cpu_s = time.perf_counter() - c0
        cpu_bytes = kc.used_bytes(seq_o) + vc.used_bytes(seq_o)
        got = out.float().cpu().numpy().astype(np.float64)
        parity = {"caches_bit_exact": bool(caches_exact),
                  "max_abs": float(np.abs(got - ref).max()),
                  "rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                  "tolerance": {"max_abs": 1e-2, "rel_l2": 1e-3},
                  "scope": f"layer 0 after its appended steps: all {B * Hkv} (batch, kv head) units' "
                           f"key and value caches, all {B * Hq} outputs of one decode call"}
        parity_ok = caches_exact and parity["max_abs"] <= 1e-2 and parity["rel_l2"] <= 1e-3
        pre_bytes = dense_bytes0 + comp_bytes0
        cpu = {"value": round(cpu_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": nthreads,
               "kind": "oracle", "hardware_concurrency": hw, "nproc": nproc,
               "prefill_compress_s": round(cpu_pre_s, 3),
               "prefill_compress_gbs_moved": round(pre_bytes / cpu_pre_s / 1e9, 3),
               "sample": f"one full decode step of the workload: attention for all {B * Hq} "
                         f"(batch, q head) pairs over the {L}-token compressed caches "
                         f"({cpu_bytes} compressed bytes), {cpu_s:.2f} s wall; and the prefill "
                         f"prune + compress of the layer's {T0}-token key and value caches "
                         f"({pre_bytes} bytes moved), {cpu_pre_s:.2f} s wall"}
        log(f"CPU oracle: prefill compress {cpu_pre_s:.2f} s, decode step {cpu_s:.2f} s "
            f"({cpu['value']} GB/s); caches bit-exact={caches_exact}; GPU vs oracle max_abs="
            f"{parity['max_abs']:.2e} rel_l2={parity['rel_l2']:.2e}")

    decode_s = median(kern_s)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in, f32 accumulate",
        "data": "synthetic (seeded; keys N(0,1) with 4 outlier channels x10 per kv head, values "
                "and queries N(0,1))",
        "config": {"workload": "llama3_8b_layer: Llama-3-8B-shaped attention layer, decode step = "
                               "append one token per (sequence, kv head) + sparse decode attention; "
                               f"steps take turns over {NL} such layers",
                   "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "seq_len": T0,
                   "sparsity": cfg.sparsity, "keep": keep, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": f"{DECODE_KERNELS} (one mustafar_decode_step call; GPU time of the "
                               "timed steps between two HIP events / steps)",
                     "bytes_per_launch": int(per_launch_bytes),
                     "avg_launch_us": round(kern_avg * 1e6, 2)},
        "cpu_baseline": cpu,
        "extra": {
            "compressed_kv_bytes": int(comp_bytes0),
            "dense_kv_bytes": int(dense_bytes0),
            "compressed_over_dense": round(comp_bytes0 / dense_bytes0, 4),
            "pages_ratio_at_70pct": 0.45,
            "decode_us_median": round(decode_s * 1e6, 2),
            "step_us_separate_calls": round(sep_wall / sep_steps * 1e6, 2),
            "step_gpu_us_separate_calls": round(sep_gpu / sep_steps * 1e6, 2),
            "gbs_separate_calls": round(sep_bytes / sep_wall / 1e9, 1),
            "decode_us_repeated_layer": round(warm_s * 1e6, 2),
            "decode_us_after_1gib_read": round(cold_s * 1e6, 2),
            "decode_gbs_after_1gib_read": round(bytes_l0 / cold_s / 1e9, 1),
            "decode_valu_us_after_1gib_read": round(valu_s * 1e6, 2),
            "stream_read_gbs": round(stream_read_gbs, 1),
            "decode_frac_of_stream_read": round(achieved / stream_read_gbs, 4),
            "prefill_compress_us": round(prefill_s * 1e6, 1),
            "prefill_gbs_moved": round((dense_bytes0 + comp_bytes0) / prefill_s / 1e9, 1),
            "parity_last_step": parity,
            "clock_ramp_decode_calls": ramp_calls,
        },
    }
    res["extra"].update(var_extra)
    if dense:
        res["extra"].update({
            "dense_us_b8_after_1gib_read": round(dense[8] * 1e6, 2),
            "dense_us_b6_after_1gib_read": round(dense[6] * 1e6, 2),
            "speedup_vs_dense_b8": round(dense[8] / cold_s, 3),
            "pv_arithmetic": "both kernels: fp32 softmax, P.V with p rounded to fp16 and fp32 "
                             "accumulation (sparse on the matrix cores, dense on the vector units)",
            "tokens_per_s_ratio_sparse_b8_vs_dense_b6": round((8 / cold_s) / (6 / dense[6]), 3),
            "pages_tokens_per_s_ratio_b8_vs_b6": 2.23,
        })
    print(json.dumps(res), flush=True)
    if not parity_ok:
        log("PARITY FAILURE: the GPU caches or output differ from the oracle's (see parity_last_step)")
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
