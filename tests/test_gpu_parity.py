"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
fp16 bits.  Compressed caches must match bit for bit; attention within max-abs
1e-2 and relative L2 1e-3 of the fp64 oracle."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import unstructured_sparse_kv_amd as usk
from tests.gpu_helpers import (ORACLE_THREADS, SCALE, assert_attn_close, assert_compressed_equal,
                               compress_on_gpu, oracle_attention_units, say, u16)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# The two sparse decode kernels (matrix-core and vector-unit) compute the same
# attention; every sparse case runs both.
SPARSE = {"mfma": usk.decode_attn, "valu": usk.decode_attn_valu}


def _decode(q, kc, vc, seq_dev, max_len, splits=0, variant="mfma"):
    B, Hq = q.shape[0], q.shape[1]
    ws = usk.make_workspace(B, Hq, kc.num_kv_heads, max_len, splits)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=q.device)
    SPARSE[variant](q, kc, vc, seq_dev, max_len, SCALE, out, ws, splits)
    torch.cuda.synchronize()
    return out


def _dense(q, K, V, seq_dev, max_len, splits=0):
    B, Hq = q.shape[0], q.shape[1]
    ws = usk.make_workspace(B, Hq, K.shape[1], max_len, splits)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=q.device)
    usk.dense_decode_attn(q, K, V, seq_dev, max_len, SCALE, out, ws, splits)
    torch.cuda.synchronize()
    return out


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_tiny_end_to_end(gpu):
    cfg = synth.CONFIGS["tiny"]
    K, V, q, seq = synth.make_inputs(cfg)
    keep = usk.keep_from_sparsity(cfg.sparsity)
    say(f"tiny: keep={keep} T={cfg.T}")
    seq_d = seq.to(gpu)
    kc = compress_on_gpu(K.to(gpu), seq_d, keep, cfg.T)
    vc = compress_on_gpu(V.to(gpu), seq_d, keep, cfg.T)
    torch.cuda.synchronize()
    ko, vo = oracle.compress(K, seq, keep, cfg.T), oracle.compress(V, seq, keep, cfg.T)
    assert_compressed_equal(kc, ko, seq)
    assert_compressed_equal(vc, vo, seq)
    ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
    for variant in SPARSE:
        out = _decode(q.to(gpu), kc, vc, seq_d, cfg.T, variant=variant)
        assert_attn_close(_f64(out), ref, f"tiny sparse {variant}")
    outd = _dense(q.to(gpu), K.to(gpu), V.to(gpu), seq_d, cfg.T)
    assert_attn_close(_f64(outd), oracle.attention_dense(q, K, V, seq, SCALE), "tiny dense")


def _row_from_case(case):
    row = np.full(128, np.float16(case["default"]), dtype=np.float16).view(np.uint16)
    for ch, v in case["set"].items():
        if isinstance(v, str) and v.startswith("0x"):
            row[int(ch)] = int(v, 16)
        elif v == "-0":
            row[int(ch)] = 0x8000
        else:
            row[int(ch)] = np.float16(v).view(np.uint16)
    return row


def test_crafted_rows_bitexact(gpu):
    cases = json.load(open(os.path.join(GOLDEN, "prune_worked_examples.json")))["cases"]
    for case in cases:
        row = _row_from_case(case)
        x = torch.from_numpy(row.view(np.int16).reshape(1, 1, 1, 128).copy())
        say(f"crafted case {case['name']} keep={case['k']}")
        c = compress_on_gpu(x.to(gpu), torch.ones(1, dtype=torch.int32, device=gpu), case["k"], 64)
        bm, vals, _ = c.views()
        assert [f"{int(w) & (2**64 - 1):016x}" for w in bm[0, 0, 0].cpu()] == case["bitmap_hex"], case["name"]
        assert [f"{int(v) & 0xFFFF:04x}" for v in vals[0, 0, :case["k"]].cpu()] == case["values_hex"]
    # tie-heavy rows: coarse integer values, +-0, subnormals, every keep
    rng = np.random.default_rng(99)
    rows = np.concatenate([
        (rng.integers(-3, 4, (96, 128)).astype(np.float16)).view(np.uint16),
        rng.choice(np.array([0, 0x8000, 1, 0x8001, 0x7BFF, 0xFBFF, 0x3C00], np.uint16), (32, 128)),
        rng.standard_normal((64, 128)).astype(np.float16).view(np.uint16),
    ])
    x = torch.from_numpy(rows.view(np.int16).reshape(1, 1, -1, 128).copy())
    seq = np.array([rows.shape[0]], np.int32)
    for keep in (0, 1, 2, 37, 38, 63, 64, 65, 100, 127, 128):
        say(f"tie rows keep={keep}")
        c = compress_on_gpu(x.to(gpu), torch.from_numpy(seq).to(gpu), keep, 192)
        torch.cuda.synchronize()
        assert_compressed_equal(c, oracle.compress(x, seq, keep, 192), seq)


def _small_inputs(B, Hq, Hkv, T, seed):
    g = torch.Generator().manual_seed(seed)
    K = torch.randn(B, Hkv, T, 128, generator=g, dtype=torch.float64)
    K[..., [3, 77]] *= 8
    V = torch.randn(B, Hkv, T, 128, generator=g, dtype=torch.float64)
    q = torch.randn(B, Hq, 128, generator=g, dtype=torch.float64)
    return K.half(), V.half(), q.half()


@pytest.mark.parametrize("kk,kv", [(0, 0), (1, 1), (3, 3), (13, 13), (37, 37), (38, 38), (47, 49),
                                   (64, 64), (65, 65), (101, 101), (127, 127), (128, 128), (38, 100),
                                   (100, 2)])
def test_keep_sweep(gpu, kk, kv):
    B, Hq, Hkv, T = 3, 8, 2, 200
    K, V, q = _small_inputs(B, Hq, Hkv, T, kk * 131 + kv)
    seq = np.array([200, 77, 1], np.int32)
    say(f"keep sweep kk={kk} kv={kv}")
    seq_d = torch.from_numpy(seq).to(gpu)
    kc = compress_on_gpu(K.to(gpu), seq_d, kk, 256)
    vc = compress_on_gpu(V.to(gpu), seq_d, kv, 256)
    torch.cuda.synchronize()
    ko, vo = oracle.compress(K, seq, kk, 256), oracle.compress(V, seq, kv, 256)
    assert_compressed_equal(kc, ko, seq)
    assert_compressed_equal(vc, vo, seq)
    ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
    for variant in SPARSE:
        for splits in (0, 1, 3):
            out = _decode(q.to(gpu), kc, vc, seq_d, 200, splits, variant)
            assert_attn_close(_f64(out), ref, f"kk={kk} kv={kv} splits={splits} {variant}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_group_sizes(gpu, G):
    B, Hkv, T = 2, 2, 333
    Hq = G * Hkv
    K, V, q = _small_inputs(B, Hq, Hkv, T, 1000 + G)
    seq = np.array([333, 130], np.int32)
    say(f"group size G={G}")
    seq_d = torch.from_numpy(seq).to(gpu)
    kc = compress_on_gpu(K.to(gpu), seq_d, 38, 384)
    vc = compress_on_gpu(V.to(gpu), seq_d, 38, 384)
    ko, vo = oracle.compress(K, seq, 38, 384), oracle.compress(V, seq, 38, 384)
    ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
    for variant in SPARSE:
        out = _decode(q.to(gpu), kc, vc, seq_d, 333, variant=variant)
        assert_attn_close(_f64(out), ref, f"sparse G={G} {variant}")
    outd = _dense(q.to(gpu), K.to(gpu), V.to(gpu), seq_d, 333)
    assert_attn_close(_f64(outd), oracle.attention_dense(q, K, V, seq, SCALE), f"dense G={G}")


def test_llama2_layer_full(gpu):
    cfg = synth.CONFIGS["llama2_7b_layer"]
    K, V, q, seq = synth.make_inputs(cfg)
    keep = usk.keep_from_sparsity(cfg.sparsity)
    say(f"llama2 layer: B=1 H=32 T=4096 keep={keep}")
    seq_d = seq.to(gpu)
    kc = compress_on_gpu(K.to(gpu), seq_d, keep, cfg.T)
    vc = compress_on_gpu(V.to(gpu), seq_d, keep, cfg.T)
    torch.cuda.synchronize()
    ko, vo = oracle.compress(K, seq, keep, cfg.T), oracle.compress(V, seq, keep, cfg.T)
    assert_compressed_equal(kc, ko, seq)
    assert_compressed_equal(vc, vo, seq)
    assert kc.used_bytes(seq.numpy()) + vc.used_bytes(seq.numpy()) == \
        2 * oracle.used_bytes(1, 32, seq.numpy(), cfg.T, 128, keep)
    ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
    for variant in SPARSE:
        out = _decode(q.to(gpu), kc, vc, seq_d, cfg.T, variant=variant)
        assert_attn_close(_f64(out), ref, f"llama2 sparse {variant}")
    outd = _dense(q.to(gpu), K.to(gpu), V.to(gpu), seq_d, cfg.T)
    assert_attn_close(_f64(outd), oracle.attention_dense(q, K, V, seq, SCALE), "llama2 dense")


def test_llama3_layer_full(gpu):
    """The Llama-3-8B-shaped layer at full size (B=8, 32/8 heads, T=32768, keep 38):
    every (batch, kv head) unit's key and value caches bit for bit against the
    oracle's compression of the same dense bits, every one of the 256 outputs of
    both sparse kernels at splits 0, 1, 7 and 64 within tolerance of the oracle's
    attention over its own caches, determinism, and the dense baseline's 256
    outputs against the oracle's dense attention."""
    cfg = synth.CONFIGS["llama3_8b_layer"]
    say("llama3 layer: generating B=8 Hkv=8 T=32768 on the GPU")
    K, V, q, seq = synth.make_inputs(cfg, device=gpu)
    keep = usk.keep_from_sparsity(cfg.sparsity)
    seq_d = seq.to(gpu)
    kc = compress_on_gpu(K, seq_d, keep, cfg.T)
    vc = compress_on_gpu(V, seq_d, keep, cfg.T)
    torch.cuda.synchronize()
    Kcpu, Vcpu, qcpu = K.cpu(), V.cpu(), q.cpu()
    say(f"llama3 layer: oracle compression of all 64 units ({ORACLE_THREADS} threads)")
    ko = oracle.compress(Kcpu, seq, keep, cfg.T, nthreads=ORACLE_THREADS)
    vo = oracle.compress(Vcpu, seq, keep, cfg.T, nthreads=ORACLE_THREADS)
    say("llama3 layer: bit-exact check of all units")
    assert_compressed_equal(kc, ko, seq.numpy())
    assert_compressed_equal(vc, vo, seq.numpy())
    assert kc.used_bytes(seq.numpy()) + vc.used_bytes(seq.numpy()) == 2 * 193069312
    say("llama3 layer: oracle attention, all 256 (batch, q head) pairs")
    ref = oracle.attention_compressed(qcpu, ko, vo, seq, SCALE, nthreads=ORACLE_THREADS)
    for variant in SPARSE:
        outs = {}
        for splits in (0, 1, 7, 64):
            say(f"llama3 layer: sparse decode ({variant}) splits={splits}")
            out = _decode(q, kc, vc, seq_d, cfg.T, splits, variant)
            outs[splits] = out.clone()
            assert_attn_close(_f64(out), ref, f"llama3 sparse {variant} splits={splits}")
        again = _decode(q, kc, vc, seq_d, cfg.T, 0, variant)
        assert torch.equal(again, outs[0]), f"decode ({variant}) is not deterministic"
    say("llama3 layer: dense baseline, all 256 pairs")
    refd = oracle.attention_dense(qcpu, Kcpu, Vcpu, seq, SCALE, nthreads=ORACLE_THREADS)
    outd = _dense(q, K, V, seq_d, cfg.T)
    assert_attn_close(_f64(outd), refd, "llama3 dense")


@pytest.mark.parametrize("B,T,Hq,layer", [(32, 131072, 32, 0), (64, 16384, 32, 31), (1, 16384, 64, 5)])
def test_llama3_stack_points(gpu, B, T, Hq, layer):
    """Points of the 32-layer stack sweep, one layer each, at their full shape
    (the largest batch x length the sweep times, the largest batch, and a 64 q /
    8 kv head group of 8): the layer is generated, pruned, compressed and
    attended on the GPU; sampled units -- the first, a middle one and the last --
    bit for bit, and sampled (batch, q head) outputs of both sparse kernels
    within tolerance of the oracle."""
    cfg = synth.CONFIGS["llama3_8b_stack"]
    keep = usk.keep_from_sparsity(cfg.sparsity)
    Hkv = cfg.Hkv
    G = Hq // Hkv
    say(f"stack point B={B} T={T} Hq={Hq} layer={layer}: generating on the GPU")
    K, V, q, _ = synth.make_inputs(cfg, device=gpu, layer=layer, B=B, T=T)
    if Hq != cfg.Hq:
        q = synth.normal_f16(cfg.seed, synth.S_Q, layer, (B, Hq, 128), gpu)
    seq_d = torch.full((B,), T, dtype=torch.int32, device=gpu)
    kc = compress_on_gpu(K, seq_d, keep, T)
    vc = compress_on_gpu(V, seq_d, keep, T)
    outs = {v: _decode(q, kc, vc, seq_d, T, 0, v) for v in SPARSE}
    seq = np.full(B, T, np.int32)
    units = sorted({(0, 0), (B // 2, 3), (B - 1, Hkv - 1)})
    pairs = [(0, 0), (B // 2, 3 * G + 1), (B - 1, Hq - 1)]
    qcpu = q.cpu()
    refs = {}
    for b, h in units:
        say(f"stack point B={B} T={T}: unit {(b, h)} against the oracle")
        s1 = np.array([T], np.int32)
        Kb, Vb = K[b:b + 1, h:h + 1].cpu(), V[b:b + 1, h:h + 1].cpu()
        ko = oracle.compress(Kb, s1, keep, T, nthreads=ORACLE_THREADS)
        vo = oracle.compress(Vb, s1, keep, T, nthreads=ORACLE_THREADS)
        assert_compressed_equal(kc, ko, seq, [(b, h)], [(0, 0)])
        assert_compressed_equal(vc, vo, seq, [(b, h)], [(0, 0)])
        for pb, hq in pairs:
            if pb == b and hq // G == h:
                refs[(pb, hq)] = oracle.attention_compressed(qcpu[b:b + 1, hq:hq + 1], ko, vo, s1,
                                                             SCALE)[0, 0]
    assert set(refs) == set(pairs)
    for v, out in outs.items():
        got = np.stack([_f64(out[b, hq]) for b, hq in pairs])
        assert_attn_close(got, np.stack([refs[p] for p in pairs]), f"stack B={B} T={T} Hq={Hq} {v}")


def test_llama3_stack_sampled(gpu):
    """32-layer stack at its smallest sweep point (B=1, T=16384): every layer is
    generated, pruned, compressed and attended on the GPU; three layers are
    checked against the oracle (sampled kv heads bit-exact, sampled q heads
    within tolerance, both sparse kernels)."""
    cfg = synth.CONFIGS["llama3_8b_stack"]
    keep = usk.keep_from_sparsity(cfg.sparsity)
    B, T, G = cfg.B, cfg.T, cfg.Hq // cfg.Hkv
    checks = {0: [(0, 0), (0, 31)], 13: [(0, 9)], cfg.layers - 1: [(0, 22), (0, 3)]}
    seq_d = torch.full((B,), T, dtype=torch.int32, device=gpu)
    for layer in range(cfg.layers):
        K, V, q, _ = synth.make_inputs(cfg, device=gpu, layer=layer)
        kc = compress_on_gpu(K, seq_d, keep, T)
        vc = compress_on_gpu(V, seq_d, keep, T)
        outs = {v: _decode(q, kc, vc, seq_d, T, 0, v) for v in SPARSE}
        assert all(torch.isfinite(o.float()).all() for o in outs.values()), f"layer {layer}"
        if layer not in checks:
            continue
        say(f"stack: layer {layer} oracle check")
        pairs = checks[layer]
        Kcpu, Vcpu, qcpu = K.cpu(), V.cpu(), q.cpu()
        seq = np.full(B, T, np.int32)
        units = sorted({(b, hq // G) for b, hq in pairs})
        for b, h in units:
            s1 = np.array([T], np.int32)
            ko = oracle.compress(Kcpu[b:b + 1, h:h + 1], s1, keep, T)
            vo = oracle.compress(Vcpu[b:b + 1, h:h + 1], s1, keep, T)
            assert_compressed_equal(kc, ko, seq, [(b, h)], [(0, 0)])
            assert_compressed_equal(vc, vo, seq, [(b, h)], [(0, 0)])
        ref = oracle_attention_units(qcpu, Kcpu, Vcpu, seq, keep, keep, T, pairs, G)
        for v, out in outs.items():
            got = np.stack([_f64(out[b, hq]) for b, hq in pairs])
            assert_attn_close(got, np.stack([ref[p] for p in pairs]), f"stack layer {layer} {v}")


@pytest.mark.parametrize("keep,G", [(38, 4), (64, 4), (37, 4), (38, 8), (64, 8), (13, 8)])
def test_decode_step_matches_separate_calls(gpu, keep, G):
    """The fused step (mustafar_decode_step) against mustafar_append_token +
    mustafar_decode_attn on copies of the same caches: out, caches, seq_lens
    and status bit for bit, over steps that start a tile, fill an empty
    sequence, and hit capacity."""
    B, Hkv, T, cap = 4, 2, 320, 320
    Hq = G * Hkv
    K, V, q = _small_inputs(B, Hq, Hkv, T, 777 + keep + G)
    seq0 = np.array([130, 64, 0, 318], np.int32)
    say(f"fused step vs separate calls: keep={keep} G={G}")
    seq_a = torch.from_numpy(seq0).to(gpu)
    seq_b = seq_a.clone()
    ka = compress_on_gpu(K.to(gpu), seq_a, keep, cap)
    va = compress_on_gpu(V.to(gpu), seq_a, keep, cap)
    kb_, vb_ = usk.CompressedKV(B, Hkv, keep, cap, gpu), usk.CompressedKV(B, Hkv, keep, cap, gpu)
    for dst, src in ((kb_, ka), (vb_, va)):
        for x, y in zip(dst.views(), src.views()):
            x.copy_(y)
    st_a = torch.zeros(1, dtype=torch.int32, device=gpu)
    st_b = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws_a = usk.make_workspace(B, Hq, Hkv, cap)
    ws_b = usk.make_workspace(B, Hq, Hkv, cap)
    g = torch.Generator().manual_seed(keep)
    for step in range(4):
        kn = torch.randn(B, Hkv, 128, generator=g).half().to(gpu)
        vn = torch.randn(B, Hkv, 128, generator=g).half().to(gpu)
        qs = torch.randn(B, Hq, 128, generator=g).half().to(gpu)
        out_a = torch.empty((B, Hq, 128), dtype=torch.float16, device=gpu)
        out_b = torch.empty_like(out_a)
        usk.append_token(ka, va, kn, vn, seq_a, st_a)
        usk.decode_attn(qs, ka, va, seq_a, cap, SCALE, out_a, ws_a)
        usk.decode_step(qs, kb_, vb_, kn, vn, seq_b, cap, SCALE, out_b, ws_b, st_b)
        torch.cuda.synchronize()
        assert torch.equal(seq_a, seq_b), f"step {step}: seq_lens {seq_a.tolist()} vs {seq_b.tolist()}"
        assert st_a.item() == st_b.item(), f"step {step}: status"
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"step {step}: out differs"
        for name, c1, c2 in (("k", ka, kb_), ("v", va, vb_)):
            for part, x, y in zip(("bitmaps", "values", "tile offsets"), c1.views(), c2.views()):
                assert torch.equal(x, y), f"step {step}: {name} {part} differ"
    assert seq_b.tolist() == [134, 68, 4, 320] and st_b.item() == usk.STATUS_APPEND_FULL


@pytest.mark.parametrize("mode", ["separate", "fused"])
def test_ragged_append_sequence(gpu, mode):
    """The Mistral-shaped ragged batch (B=16, 32/8 heads, lengths uniform in
    [4096, 32768], keep 64) through 64 decode steps, each appending one key and
    value row per (sequence, kv head) and attending: all 512 outputs at steps 1,
    2, 32 and 64 within tolerance of the oracle, whose caches grow by its own
    append; all 128 units' caches bit for bit after step 64; lengths exact."""
    cfg = synth.CONFIGS["mistral_ragged_append"]
    keep = usk.keep_from_sparsity(cfg.sparsity)
    seq0 = synth.seq_lens_uniform(cfg.seed, cfg.B, *cfg.ragged)
    Tmax = cfg.ragged[1]
    cap = Tmax + 64
    say(f"ragged append: B=16 Hkv=8 lens {seq0.min().item()}..{seq0.max().item()} keep={keep} "
        f"steps={cfg.steps} mode={mode}")
    K, V, _, _ = synth.make_inputs(cfg, device=gpu, T=cap)
    seq_d = seq0.to(gpu)
    kc = compress_on_gpu(K, seq_d, keep, cap)
    vc = compress_on_gpu(V, seq_d, keep, cap)
    torch.cuda.synchronize()
    say(f"ragged append: oracle compression of all 128 units ({ORACLE_THREADS} threads)")
    seq_o = seq0.numpy().astype(np.int32)
    ko = oracle.compress(K.cpu(), seq_o, keep, cap, nthreads=ORACLE_THREADS)
    vo = oracle.compress(V.cpu(), seq_o, keep, cap, nthreads=ORACLE_THREADS)
    del K, V
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws = usk.make_workspace(cfg.B, cfg.Hq, cfg.Hkv, cap)
    out = torch.empty((cfg.B, cfg.Hq, 128), dtype=torch.float16, device=gpu)
    outv = torch.empty_like(out)
    check_steps = {1, 2, 32, cfg.steps}
    for step in range(1, cfg.steps + 1):
        kn, vn, q = synth.step_inputs(cfg, step - 1, device=gpu)
        if mode == "fused":
            usk.decode_step(q, kc, vc, kn, vn, seq_d, cap, SCALE, out, ws, status)
        else:
            usk.append_token(kc, vc, kn, vn, seq_d, status)
            usk.decode_attn(q, kc, vc, seq_d, cap, SCALE, out, ws)
            usk.decode_attn_valu(q, kc, vc, seq_d, cap, SCALE, outv, ws)
        seq_o, st = oracle.append_step(ko, vo, kn.cpu(), vn.cpu(), seq_o)
        assert st == 0
        if step in check_steps:
            torch.cuda.synchronize()
            assert np.array_equal(seq_d.cpu().numpy(), seq_o)
            say(f"ragged append: step {step} parity, all 512 outputs")
            ref = oracle.attention_compressed(q.cpu(), ko, vo, seq_o, SCALE, nthreads=ORACLE_THREADS)
            assert_attn_close(_f64(out), ref, f"ragged append step {step} ({mode})")
            if mode == "separate":
                assert_attn_close(_f64(outv), ref, f"ragged append step {step} valu")
    say("ragged append: all 128 units bit for bit after the last step")
    assert_compressed_equal(kc, ko, seq_o)
    assert_compressed_equal(vc, vo, seq_o)
    assert status.item() == 0


def _thin_rows(c: "oracle.Compressed", seq, rng):
    """Rewrites an oracle-compressed tensor so that some rows hold fewer than
    keep values: random rows lose their highest 1..10 set bits, some rows lose
    a whole bitmap word, one row of the first tile loses one value (so later
    tiles start at odd offsets).  Values stay packed back to back and tile
    offsets are recomputed from the popcounts, as the format defines them."""
    B, H, cap, k = c.B, c.H, c.cap, c.k
    out = oracle.Compressed(B, H, cap, c.d, k)
    for b in range(B):
        T = int(seq[b])
        for h in range(H):
            src = c.values[b, h]
            pos = 0
            dst = []
            toff = []
            for r in range(T):
                if r % 64 == 0:
                    toff.append(len(dst))
                words = [int(w) for w in c.bitmaps[b, h, r]]
                bits = [64 * w + j for w in range(len(words)) for j in range(64) if (words[w] >> j) & 1]
                vals = list(src[pos:pos + len(bits)])
                pos += len(bits)
                keep_idx = list(range(len(bits)))
                u = rng.random()
                if u < 0.3:
                    keep_idx = keep_idx[:max(0, len(bits) - int(rng.integers(1, 11)))]
                elif u < 0.4:
                    lo, hi = (0, 32) if rng.random() < 0.5 else (96, 128)
                    keep_idx = [i for i in keep_idx if not lo <= bits[i] < hi]
                if r == 63 and (len(dst) + len(keep_idx)) % 2 == 0 and keep_idx:
                    keep_idx = keep_idx[:-1]  # the second tile starts at an odd offset
                nw = [0] * len(words)
                for i in keep_idx:
                    nw[bits[i] // 64] |= 1 << (bits[i] % 64)
                    dst.append(vals[i])
                out.bitmaps[b, h, r] = np.array(nw, dtype=np.uint64)
            toff.append(len(dst))
            out.values[b, h, :len(dst)] = np.array(dst, dtype=np.uint16)
            out.tile_off[b, h, :len(toff)] = np.array(toff, dtype=np.uint32)
    return out


def _upload(c: "oracle.Compressed", gpu):
    kv = usk.CompressedKV(c.B, c.H, c.k, c.cap, gpu)
    bm, vals, toff = kv.views()
    bm.copy_(torch.from_numpy(c.bitmaps.view(np.int64)))
    vals.copy_(torch.from_numpy(c.values.view(np.int16)))
    toff.copy_(torch.from_numpy(c.tile_off.view(np.int32)))
    return kv


@pytest.mark.parametrize("keep", [38, 64, 37])
def test_rows_below_keep(gpu, keep):
    """Caches whose rows hold fewer than keep values (and tiles starting at odd
    offsets) take the exact-start path of both sparse kernels."""
    B, Hq, Hkv, T, cap = 2, 4, 2, 300, 320
    K, V, q = _small_inputs(B, Hq, Hkv, T, 4242 + keep)
    seq = np.array([300, 130], np.int32)
    rng = np.random.default_rng(keep)
    ko = _thin_rows(oracle.compress(K, seq, keep, cap), seq, rng)
    vo = _thin_rows(oracle.compress(V, seq, keep, cap), seq, rng)
    assert ko.tile_off[0, 0, 1] % 2 == 1, "the second tile should start at an odd offset"
    say(f"rows below keep: keep={keep}")
    kc, vc = _upload(ko, gpu), _upload(vo, gpu)
    seq_d = torch.from_numpy(seq).to(gpu)
    ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
    for variant in SPARSE:
        for splits in (0, 2):
            out = _decode(q.to(gpu), kc, vc, seq_d, T, splits, variant)
            assert_attn_close(_f64(out), ref, f"rows below keep={keep} {variant} splits={splits}")


def test_edge_cases(gpu):
    B, Hq, Hkv, T = 4, 4, 2, 130
    K, V, q = _small_inputs(B, Hq, Hkv, T, 7)
    seq = np.array([0, 1, 130, 500], np.int32)  # empty, one row, full, beyond capacity (clamped to 192)
    cap = 192
    Kp = torch.zeros(B, Hkv, cap, 128, dtype=torch.float16)
    Vp = torch.zeros(B, Hkv, cap, 128, dtype=torch.float16)
    Kp[:, :, :T], Vp[:, :, :T] = K, V
    Kp[3], Vp[3] = torch.randn(Hkv, cap, 128).half(), torch.randn(Hkv, cap, 128).half()
    say("edge cases: lengths 0, 1, 130, 500 (capacity 192)")
    seq_d = torch.from_numpy(seq).to(gpu)
    kc = compress_on_gpu(Kp.to(gpu), seq_d, 38, cap)
    vc = compress_on_gpu(Vp.to(gpu), seq_d, 38, cap)
    torch.cuda.synchronize()
    seq_c = np.minimum(seq, cap)
    ko, vo = oracle.compress(Kp, seq_c, 38, cap), oracle.compress(Vp, seq_c, 38, cap)
    assert_compressed_equal(kc, ko, seq_c)
    assert_compressed_equal(vc, vo, seq_c)
    # canaries around the output
    ws = usk.make_workspace(B, Hq, Hkv, cap)
    ref = oracle.attention_compressed(q, ko, vo, seq_c, SCALE)
    v0 = oracle.decompress(vo, seq_c)[1, :, 0].view(np.float16).astype(np.float64)
    for variant, fn in SPARSE.items():
        buf = torch.full((B * Hq * 128 + 2 * 256,), 0x7E01, dtype=torch.int16, device=gpu)  # NaN bits
        out = buf[256:256 + B * Hq * 128].view(torch.float16).view(B, Hq, 128)
        fn(q.to(gpu), kc, vc, seq_d, cap, SCALE, out, ws)
        torch.cuda.synchronize()
        assert (buf[:256] == 0x7E01).all() and (buf[-256:] == 0x7E01).all(), "canary overwritten"
        assert not out[0].any(), "empty sequence must give zeros"
        assert_attn_close(_f64(out), ref, f"edge cases {variant}")
        # T = 1: the output is the stored first value row for every head of the group
        for hq in range(Hq):
            assert np.array_equal(_f64(out[1, hq]), v0[hq // 2].astype(np.float16).astype(np.float64))
    # append at capacity: status bit, caches and lengths unchanged
    full = torch.tensor([cap, cap, cap, cap], dtype=torch.int32, device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    before = [t.clone() for t in kc.views()]
    usk.append_token(kc, vc, K[:, :, 0].contiguous().to(gpu), V[:, :, 0].contiguous().to(gpu), full, status)
    torch.cuda.synchronize()
    assert status.item() == usk.STATUS_APPEND_FULL
    assert full.cpu().tolist() == [cap] * 4
    for a, b in zip(before, kc.views()):
        assert torch.equal(a, b)


def test_shared_workspace_across_shapes(gpu):
    """One workspace serves a run of calls of different shapes, split counts and
    kernels (sparse, vector-unit, dense, fused step): whatever earlier calls left
    in it, each output must match the same call on a fresh workspace bit for bit,
    and the oracle; the fused step advances every length exactly once."""
    ws = usk.make_workspace(8, 32, 8, 4096, splits=64, device=gpu)
    cases = [  # (B, Hq, Hkv, T, keep, splits, kernel)
        (3, 8, 2, 300, 38, 0, "mfma"), (3, 8, 2, 300, 38, 5, "mfma"), (1, 4, 4, 1000, 64, 0, "mfma"),
        (4, 32, 8, 200, 38, 3, "valu"), (2, 2, 2, 130, 13, 7, "mfma"), (3, 8, 2, 300, 38, 0, "mfma"),
        (2, 16, 2, 700, 38, 0, "dense"), (3, 8, 2, 300, 38, 5, "step"), (3, 8, 2, 300, 38, 5, "step"),
        (2, 8, 1, 257, 64, 64, "mfma"), (3, 8, 2, 300, 38, 0, "mfma")]
    for i, (B, Hq, Hkv, T, keep, splits, kern) in enumerate(cases):
        say(f"shared workspace call {i}: B={B} Hq={Hq} Hkv={Hkv} T={T} keep={keep} splits={splits} {kern}")
        K, V, q = _small_inputs(B, Hq, Hkv, T + 1, 7000 + i)
        cap = (T // 64 + 2) * 64  # room for the appended row
        seq = np.array([T - 17 * b for b in range(B)], np.int32)
        qd = q.to(gpu)
        out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float16, device=gpu)
        fresh = torch.full_like(out, float("nan"))
        if kern == "dense":
            Kd, Vd, sd = K[:, :, :T].contiguous().to(gpu), V[:, :, :T].contiguous().to(gpu), torch.from_numpy(seq).to(gpu)
            usk.dense_decode_attn(qd, Kd, Vd, sd, T, SCALE, out, ws, splits)
            usk.dense_decode_attn(qd, Kd, Vd, sd, T, SCALE, fresh,
                                  usk.make_workspace(B, Hq, Hkv, T, splits, device=gpu), splits)
            torch.cuda.synchronize()
            ref = oracle.attention_dense(q, K[:, :, :T].contiguous(), V[:, :, :T].contiguous(), seq, SCALE)
        elif kern == "step":
            outs = []
            for w in (ws, usk.make_workspace(B, Hq, Hkv, T + 1, splits, device=gpu)):
                sd = torch.from_numpy(seq).to(gpu)
                kc = compress_on_gpu(K.to(gpu), sd, keep, cap)
                vc = compress_on_gpu(V.to(gpu), sd, keep, cap)
                kn = K[:, :, T].contiguous().to(gpu)
                vn = V[:, :, T].contiguous().to(gpu)
                o = out if w is ws else fresh
                usk.decode_step(qd, kc, vc, kn, vn, sd, T + 1, SCALE, o, w, splits=splits)
                torch.cuda.synchronize()
                assert np.array_equal(sd.cpu().numpy(), seq + 1), "seq_lens not advanced exactly once"
                outs.append((kc, vc))
            # the reference: the caches after the step, attended over seq + 1 rows
            Kr = K.clone()
            Vr = V.clone()
            for b in range(B):  # the new row sits at seq[b]
                Kr[b, :, seq[b]] = K[b, :, T]
                Vr[b, :, seq[b]] = V[b, :, T]
            ko = oracle.compress(Kr, seq + 1, keep, cap)
            vo = oracle.compress(Vr, seq + 1, keep, cap)
            ref = oracle.attention_compressed(q, ko, vo, seq + 1, SCALE)
        else:
            sd = torch.from_numpy(seq).to(gpu)
            kc = compress_on_gpu(K.to(gpu), sd, keep, cap)
            vc = compress_on_gpu(V.to(gpu), sd, keep, cap)
            SPARSE[kern](qd, kc, vc, sd, T, SCALE, out, ws, splits)
            SPARSE[kern](qd, kc, vc, sd, T, SCALE, fresh,
                         usk.make_workspace(B, Hq, Hkv, T, splits, device=gpu), splits)
            torch.cuda.synchronize()
            ref = oracle.attention_compressed(q, oracle.compress(K, seq, keep, cap),
                                              oracle.compress(V, seq, keep, cap), seq, SCALE)
        assert np.array_equal(u16(out), u16(fresh)), f"call {i}: shared and fresh workspace differ"
        assert_attn_close(_f64(out), ref, f"shared workspace call {i} ({kern})")


def test_prune_exact_count_at_high_key_bits(gpu):
    """Rows whose keep-th and (keep+1)-th largest magnitudes first differ at key
    bit 14, 13, 12, 11 or 10, so that a candidate with exactly keep keys at or
    above it appears at that bit of the MSB-first search: the survivors must be
    the oracle's whatever bit the search stops at."""
    rng = np.random.default_rng(4242)
    rows = []
    for keep in (1, 38, 64, 127):
        for bit in (14, 13, 12, 11, 10):
            for _ in range(4):
                hi_key = (1 << bit) | int(rng.integers(0, 1 << bit))  # top bit `bit` set
                lo_key = int(rng.integers(0, 1 << bit))               # below 1 << bit
                keys = np.concatenate([np.full(keep, hi_key), rng.integers(0, lo_key + 1, 128 - keep)])
                keys = np.minimum(keys, 0x7BFF)  # finite fp16 magnitudes
                sign = rng.integers(0, 2, 128) << 15
                rows.append((keys | sign)[rng.permutation(128)].astype(np.uint16))
    x = np.stack(rows).view(np.int16).reshape(1, 1, -1, 128)
    seq = np.array([x.shape[2]], np.int32)
    cap = (x.shape[2] + 63) // 64 * 64
    xt = torch.from_numpy(x.copy())
    for keep in (1, 38, 64, 127):
        say(f"high-bit exact counts keep={keep}")
        c = compress_on_gpu(xt.to(gpu), torch.from_numpy(seq).to(gpu), keep, cap)
        torch.cuda.synchronize()
        assert_compressed_equal(c, oracle.compress(xt, seq, keep, cap), seq)
