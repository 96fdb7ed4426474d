"""Pins for the CPU oracle: each check ties the oracle to something other than
itself (the IEEE-754 binary16 definition via numpy, brute force over every
k-subset, hand-worked fixtures, closed forms, torch's scaled_dot_product_attention
in fp64, invariants of the selection rule).  No GPU needed."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- fp16 codec
def test_half_decode_exhaustive_against_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # -0 keeps its sign
    assert math.copysign(1.0, oracle.half_to_double(np.array([0x8000], np.uint16))[0]) == -1.0


def test_half_decode_ieee_constants():
    f = lambda b: float(oracle.half_to_double(np.array([b], np.uint16))[0])
    assert f(0x3C00) == 1.0
    assert f(0x7BFF) == 65504.0
    assert f(0x0001) == 2.0 ** -24
    assert f(0x03FF) == 1023 * 2.0 ** -24
    assert f(0x0400) == 2.0 ** -14
    assert f(0xC000) == -2.0
    assert f(0x7C00) == math.inf
    assert math.isnan(f(0x7E00))


# ---------------------------------------------------------------- keep count
@pytest.mark.parametrize("s,k", [(0.0, 128), (0.5, 64), (0.7, 38), (1.0, 0), (0.25, 96),
                                 (0.9, 13), (0.75, 32)])
def test_keep_closed_form(s, k):
    # (1 - 0.7) * 128 = 38.400000000000006 -> 38; 0.9 -> 12.8 -> 13
    assert oracle.keep_from_sparsity(s, 128) == k


def test_keep_rejects_out_of_range():
    assert oracle.keep_from_sparsity(-0.1, 128) == -1
    assert oracle.keep_from_sparsity(1.5, 128) == -1
    assert oracle.keep_from_sparsity(float("nan"), 128) == -1


# ---------------------------------------------------------------- prune rule
def _brute_force_keep(keys, k):
    """Among all k-subsets with the largest total magnitude key, the
    lexicographically smallest sorted index tuple (== lowest-index tie-break)."""
    d = len(keys)
    best, best_sum = None, None
    for comb in itertools.combinations(range(d), k):
        s = sum(int(keys[i]) for i in comb)
        if best_sum is None or s > best_sum or (s == best_sum and comb < best):
            best, best_sum = comb, s
    return set(best)


@pytest.mark.parametrize("d", [4, 8, 12, 16])
def test_prune_matches_brute_force(d):
    rng = np.random.default_rng(1234 + d)
    # a small alphabet forces many ties, including +-x pairs, +-0 and subnormals
    alphabet = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3C00, 0xBC00, 0x4000, 0xC000, 0x3800,
                         0x7BFF, 0xFBFF, 0x1234], dtype=np.uint16)
    for trial in range(6):
        rows = alphabet[rng.integers(0, alphabet.size, size=(1, d))]
        for k in range(d + 1):
            keep = oracle.prune_rows(rows, k)[0]
            got = set(np.nonzero(keep)[0].tolist())
            assert got == _brute_force_keep(rows[0] & 0x7FFF, k), (d, k, rows)


def _row_from_case(case, d=128):
    row = np.full(d, np.float16(case["default"]), dtype=np.float16).view(np.uint16)
    for ch, v in case["set"].items():
        if isinstance(v, str) and v.startswith("0x"):
            row[int(ch)] = int(v, 16)
        elif v == "-0":
            row[int(ch)] = 0x8000
        else:
            row[int(ch)] = np.float16(v).view(np.uint16)
    return row


def test_prune_and_encode_worked_examples():
    cases = json.load(open(os.path.join(GOLDEN, "prune_worked_examples.json")))["cases"]
    for case in cases:
        row = _row_from_case(case)
        keep = oracle.prune_rows(row[None], case["k"])[0]
        assert np.nonzero(keep)[0].tolist() == case["keep"], case["name"]
        c = oracle.compress(row.reshape(1, 1, 1, 128), [1], case["k"], cap=64)
        assert [f"{int(w):016x}" for w in c.bitmaps[0, 0, 0]] == case["bitmap_hex"], case["name"]
        vals = c.values[0, 0, :case["k"]]
        assert [f"{int(v):04x}" for v in vals] == case["values_hex"], case["name"]


def _invariants(x, keep, k):
    key = x & 0x7FFF
    assert keep.sum(axis=-1).tolist() == [k] * keep.shape[0]
    for r in range(x.shape[0]):
        kept, pruned = key[r][keep[r] == 1], key[r][keep[r] == 0]
        if kept.size and pruned.size:
            tau = kept.min()
            assert tau >= pruned.max()
            kept_at = np.nonzero((keep[r] == 1) & (key[r] == tau))[0]
            pruned_at = np.nonzero((keep[r] == 0) & (key[r] == tau))[0]
            if kept_at.size and pruned_at.size:
                assert kept_at.max() < pruned_at.min()


@pytest.mark.parametrize("k", [0, 1, 37, 38, 63, 64, 65, 127, 128])
def test_prune_invariants_random_and_tied(k):
    rng = np.random.default_rng(k)
    x = np.concatenate([
        rng.standard_normal((64, 128)).astype(np.float16).view(np.uint16),
        # coarse values: many ties at the threshold, in either 64-channel half
        (rng.integers(-3, 4, (64, 128)).astype(np.float16)).view(np.uint16),
        np.full((2, 128), 0x3C00, np.uint16),
    ])
    x[-1, ::2] |= 0x8000
    keep = oracle.prune_rows(x, k)
    _invariants(x, keep, k)


# ---------------------------------------------------------------- encode / decode
def test_roundtrip_and_layout():
    rng = np.random.default_rng(7)
    B, H, T, d, k = 2, 3, 200, 128, 38
    x = rng.standard_normal((B, H, T, d)).astype(np.float16).view(np.uint16)
    seq = np.array([200, 131], np.int32)
    c = oracle.compress(x, seq, k, cap=256)
    assert c.cap == 256
    dec = oracle.decompress(c, seq)
    keep = oracle.prune_rows(x, k)
    for b in range(B):
        T_b = seq[b]
        # decompress(compress(x)) == x with pruned entries set to +0.0
        expect = np.where(keep[b, :, :T_b] == 1, x[b, :, :T_b], 0).astype(np.uint16)
        assert np.array_equal(dec[b, :, :T_b], expect)
        assert not dec[b, :, T_b:].any()
        # popcount == k on every written row; closed-form tile offsets (64 * tile * k)
        pc = np.array([bin(int(w)).count("1") for w in
                       c.bitmaps[b, 0, :T_b].reshape(-1)]).reshape(T_b, 2).sum(1)
        assert (pc == k).all()
        ntiles = (T_b + 63) // 64
        for h in range(H):
            exp = [min(64 * j, T_b) * k for j in range(ntiles + 1)]
            assert c.tile_off[b, h, :ntiles + 1].tolist() == exp
            # values are the kept entries in ascending channel order, rows in order
            flat = x[b, h, :T_b][keep[b, h, :T_b] == 1]
            assert np.array_equal(c.values[b, h, :T_b * k], flat)


def test_keep_all_and_keep_none():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 1, 64, 128)).astype(np.float16).view(np.uint16)
    call = oracle.compress(x, [64], 128)
    assert (call.bitmaps == np.uint64(0xFFFFFFFFFFFFFFFF)).all()
    assert np.array_equal(call.values[0, 0], x[0, 0].reshape(-1))
    cnone = oracle.compress(x, [64], 0)
    assert not cnone.bitmaps.any()
    assert cnone.tile_off[0, 0, :2].tolist() == [0, 0]
    assert not oracle.decompress(cnone, [64]).any()


def test_used_bytes_closed_form():
    # per (b,h): 16 B bitmap + 2k B values per row, 4 B per tile entry (ceil(T/64)+1 entries)
    seq = np.array([32768] * 8, np.int32)
    per = 16 * 32768 + 2 * 38 * 32768 + 4 * (512 + 1)
    assert oracle.used_bytes(8, 8, seq, 32768, 128, 38) == 64 * per
    assert oracle.used_bytes(1, 1, np.array([0], np.int32), 64, 128, 38) == 4
    assert oracle.used_bytes(1, 2, np.array([65], np.int32), 128, 128, 64) == 2 * (65 * 144 + 4 * 3)


# ---------------------------------------------------------------- attention
def _sdpa_f64(q, K, V, seq, scale):
    """torch scaled_dot_product_attention in float64 on the CPU, per batch row,
    kv head h serving q heads h*G .. h*G+G-1."""
    qd = torch.from_numpy(q.view(np.float16).astype(np.float64))
    Kd = torch.from_numpy(K.view(np.float16).astype(np.float64))
    Vd = torch.from_numpy(V.view(np.float16).astype(np.float64))
    B, Hq, d = qd.shape
    G = Hq // Kd.shape[1]
    out = torch.zeros(B, Hq, d, dtype=torch.float64)
    for b in range(B):
        T = int(seq[b])
        if T == 0:
            continue
        Kb = Kd[b, :, :T].repeat_interleave(G, dim=0)
        Vb = Vd[b, :, :T].repeat_interleave(G, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(qd[b][:, None, :], Kb, Vb, scale=scale)
        out[b] = o[:, 0, :]
    return out.numpy()


def _rand_inputs(rng, B, Hq, Hkv, T, d=128, outliers=True):
    q = rng.standard_normal((B, Hq, d)).astype(np.float16).view(np.uint16)
    K = rng.standard_normal((B, Hkv, T, d))
    if outliers:
        K[..., [3, 77]] *= 8.0
    K = K.astype(np.float16).view(np.uint16)
    V = rng.standard_normal((B, Hkv, T, d)).astype(np.float16).view(np.uint16)
    return q, K, V


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (8, 2), (4, 1)])
def test_attention_dense_s0_matches_torch_sdpa(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    B, T = 2, 150
    q, K, V = _rand_inputs(rng, B, Hq, Hkv, T)
    seq = np.array([150, 77], np.int32)
    scale = 1.0 / math.sqrt(128)
    ref = _sdpa_f64(q, K, V, seq, scale)
    got = oracle.attention_dense(q, K, V, seq, scale)
    assert np.abs(got - ref).max() < 1e-12
    # keep-all compression (s = 0) gives the same result
    kc, vc = oracle.compress(K, seq, 128), oracle.compress(V, seq, 128)
    got2 = oracle.attention_compressed(q, kc, vc, seq, scale)
    assert np.abs(got2 - ref).max() < 1e-12


@pytest.mark.parametrize("kk,kv", [(38, 38), (64, 64), (13, 100), (0, 38), (38, 0)])
def test_attention_compressed_equals_sdpa_on_zero_masked_cache(kk, kv):
    rng = np.random.default_rng(kk * 1000 + kv)
    B, Hq, Hkv, T = 2, 8, 2, 130
    q, K, V = _rand_inputs(rng, B, Hq, Hkv, T)
    seq = np.array([130, 64], np.int32)
    scale = 1.0 / math.sqrt(128)
    kc, vc = oracle.compress(K, seq, kk), oracle.compress(V, seq, kv)
    Km, Vm = oracle.decompress(kc, seq), oracle.decompress(vc, seq)
    ref = _sdpa_f64(q, Km[:, :, :T], Vm[:, :, :T], seq, scale)
    got = oracle.attention_compressed(q, kc, vc, seq, scale)
    assert np.abs(got - ref).max() < 1e-12
    # subset evaluation writes the same numbers for the listed (b, hq) only
    units = [0 * Hq + 3, 1 * Hq + 7]
    sub = oracle.attention_compressed(q, kc, vc, seq, scale, units=units)
    assert np.array_equal(sub[0, 3], got[0, 3]) and np.array_equal(sub[1, 7], got[1, 7])
    assert not sub[0, 0].any()


def test_attention_closed_forms():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, T, d = 1, 4, 2, 70, 128
    q, K, V = _rand_inputs(rng, B, Hq, Hkv, T)
    scale = 1.0 / math.sqrt(d)
    vc = oracle.compress(V, [T], 64)
    Vm = oracle.decompress(vc, [T]).view(np.float16).astype(np.float64)
    kc = oracle.compress(K, [T], 64)
    # T = 1: the output is the (pruned) first value row exactly
    o1 = oracle.attention_compressed(q, kc, vc, [1], scale)
    for hq in range(Hq):
        assert np.array_equal(o1[0, hq], Vm[0, hq // 2, 0])
    # q = 0: uniform weights -> mean of the pruned value rows
    q0 = np.zeros_like(q)
    o0 = oracle.attention_compressed(q0, kc, vc, [T], scale)
    for hq in range(Hq):
        assert np.abs(o0[0, hq] - Vm[0, hq // 2, :T].mean(axis=0)).max() < 1e-14
    # empty sequence: zeros
    oe = oracle.attention_compressed(q, kc, vc, [0], scale)
    assert not oe.any()


def test_attention_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, T = 2, 8, 2, 96
    q, K, V = _rand_inputs(rng, B, Hq, Hkv, T)
    seq = np.array([96, 40], np.int32)
    scale = 0.1
    G = Hq // Hkv
    gqa = oracle.attention_compressed(q, oracle.compress(K, seq, 38), oracle.compress(V, seq, 50),
                                      seq, scale)
    Kr, Vr = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    mha = oracle.attention_compressed(q, oracle.compress(Kr, seq, 38), oracle.compress(Vr, seq, 50),
                                      seq, scale)
    assert np.array_equal(gqa, mha)


def _vec(spec, d=128):
    v = np.zeros(d, np.float16)
    for ch, x in spec.items():
        v[int(ch)] = x
    return v.view(np.uint16)


def test_attention_worked_examples():
    cases = json.load(open(os.path.join(GOLDEN, "attention_worked_examples.json")))["cases"]
    for case in cases:
        T = len(case["K"])
        q = _vec(case["q"]).reshape(1, 1, 128)
        K = np.stack([_vec(r) for r in case["K"]]).reshape(1, 1, T, 128)
        V = np.stack([_vec(r) for r in case["V"]]).reshape(1, 1, T, 128)
        out = oracle.attention_dense(q, K, V, [T], case["scale"])[0, 0]
        outc = oracle.attention_compressed(q, oracle.compress(K, [T], 128), oracle.compress(V, [T], 128),
                                           [T], case["scale"])[0, 0]
        for ch, val in case["expected_value"].items():
            assert abs(out[int(ch)] - val) < 1e-15, case["name"]
            assert abs(outc[int(ch)] - val) < 1e-15, case["name"]
        others = [c for c in range(128) if str(c) not in case["expected_value"]]
        assert not out[others].any()


# ---------------------------------------------------------------- per-head keep (R22)
HEAD_KEEP = [26, 50, 0, 128, 38, 37]


def test_head_keep_layout_and_rule():
    """Per-head compression against the uniform rule applied head by head: head h of the
    per-head cache holds exactly what a uniform compression of that head's slice with
    keep = head_keep[h] holds, and its values sit at cap * (b * S + sum(head_keep[:h]))."""
    rng = np.random.default_rng(21)
    B, H, T, d = 2, len(HEAD_KEEP), 140, 128
    x = rng.standard_normal((B, H, T, d)).astype(np.float16).view(np.uint16)
    x[..., 5] = x[..., 6]  # ties between channels 5 and 6
    seq = np.array([140, 65], np.int32)
    cap = 192
    c = oracle.compress(x, seq, max(HEAD_KEEP), cap=cap, head_keep=HEAD_KEEP)
    S = sum(HEAD_KEEP)
    assert c.values.shape == (B, cap * S)
    for h, kh in enumerate(HEAD_KEEP):
        u = oracle.compress(np.ascontiguousarray(x[:, h:h + 1]), seq, kh, cap=cap)
        pre = sum(HEAD_KEEP[:h])
        for b in range(B):
            T_b = int(seq[b])
            assert np.array_equal(c.bitmaps[b, h, :T_b], u.bitmaps[b, 0, :T_b])
            ntile = (T_b + 63) // 64
            assert np.array_equal(c.tile_off[b, h, :ntile + 1], u.tile_off[b, 0, :ntile + 1])
            assert c.tile_off[b, h, :ntile + 1].tolist() == [min(64 * j, T_b) * kh
                                                               for j in range(ntile + 1)]
            start = cap * pre
            assert np.array_equal(c.values[b, start:start + T_b * kh], u.values[b, 0, :T_b * kh])
    # decompress: each head zero-masked by its own keep
    dec = oracle.decompress(c, seq)
    for h, kh in enumerate(HEAD_KEEP):
        keep = oracle.prune_rows(x[:, h], kh)
        for b in range(B):
            T_b = int(seq[b])
            expect = np.where(keep[b, :T_b] == 1, x[b, h, :T_b], 0).astype(np.uint16)
            assert np.array_equal(dec[b, h, :T_b], expect)


def test_head_keep_all_equal_is_the_uniform_layout():
    rng = np.random.default_rng(22)
    B, H, T = 2, 3, 100
    x = rng.standard_normal((B, H, T, 128)).astype(np.float16).view(np.uint16)
    seq = np.array([100, 37], np.int32)
    a = oracle.compress(x, seq, 38, cap=128, head_keep=[38] * H)
    u = oracle.compress(x, seq, 38, cap=128)
    assert np.array_equal(a.values.reshape(u.values.shape), u.values)
    assert np.array_equal(a.bitmaps, u.bitmaps) and np.array_equal(a.tile_off, u.tile_off)


def test_head_keep_used_bytes_closed_form():
    seq = np.array([100, 0, 64], np.int32)
    hk = [10, 20, 30, 40]
    exp = 0
    for T in seq:
        for k in hk:
            exp += 16 * T + 2 * k * T + 4 * ((T + 63) // 64 + 1)
    assert oracle.used_bytes(3, 4, seq, 128, 128, 40, head_keep=hk) == exp


def test_head_keep_attention_equals_sdpa_on_zero_masked_cache():
    rng = np.random.default_rng(23)
    Hkv = len(HEAD_KEEP)
    B, Hq, T = 2, 2 * Hkv, 130
    q, K, V = _rand_inputs(rng, B, Hq, Hkv, T)
    seq = np.array([130, 70], np.int32)
    scale = 1.0 / math.sqrt(128)
    vk = HEAD_KEEP[::-1]
    kc = oracle.compress(K, seq, 128, head_keep=HEAD_KEEP)
    vc = oracle.compress(V, seq, 128, head_keep=vk)
    Km, Vm = oracle.decompress(kc, seq), oracle.decompress(vc, seq)
    ref = _sdpa_f64(q, Km[:, :, :T], Vm[:, :, :T], seq, scale)
    got = oracle.attention_compressed(q, kc, vc, seq, scale)
    assert np.abs(got - ref).max() < 1e-12
    # every head keeping all 128 channels is dense attention
    kall = oracle.compress(K, seq, 128, head_keep=[128] * Hkv)
    vall = oracle.compress(V, seq, 128, head_keep=[128] * Hkv)
    dense = _sdpa_f64(q, K, V, seq, scale)
    assert np.abs(oracle.attention_compressed(q, kall, vall, seq, scale) - dense).max() < 1e-12


# ---------------------------------------------------------------- 2:4 comparator rule (R23)
def test_prune_24_matches_brute_force_per_group():
    rng = np.random.default_rng(31)
    alphabet = np.array([0x0000, 0x8000, 0x0001, 0x3C00, 0xBC00, 0x4000, 0xC000, 0x3800, 0x7BFF],
                        dtype=np.uint16)
    for trial in range(40):
        row = alphabet[rng.integers(0, alphabet.size, size=(1, 128))]
        keep = oracle.prune_rows_24(row)[0]
        for g in range(32):
            keys = row[0, 4 * g:4 * g + 4] & 0x7FFF
            want = _brute_force_keep(keys, 2)
            got = set(np.nonzero(keep[4 * g:4 * g + 4])[0].tolist())
            assert got == want, (trial, g, keys)


def test_prune_24_invariants_and_special_rows():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((200, 128)).astype(np.float16).view(np.uint16)
    keep = oracle.prune_rows_24(x)
    kg = keep.reshape(200, 32, 4)
    assert (kg.sum(-1) == 2).all()
    key = (x & 0x7FFF).reshape(200, 32, 4).astype(np.int64)
    kept_min = np.where(kg == 1, key, 1 << 20).min(-1)
    pruned_max = np.where(kg == 0, key, -1).max(-1)
    assert (kept_min >= pruned_max).all()
    # two zeros and two non-zeros per group: the non-zeros survive, so nothing is lost
    y = x.copy().reshape(200, 32, 4)
    y[:, :, [0, 3]] = 0
    y = y.reshape(200, 128)
    c = oracle.compress_24(y.reshape(1, 1, 200, 128), [200], cap=256)
    assert np.array_equal(oracle.decompress(c, [200])[0, 0, :200], y)


def test_compress_24_layout_and_attention():
    rng = np.random.default_rng(33)
    B, Hq, Hkv, T = 2, 4, 2, 150
    q, K, V = _rand_inputs(rng, B, Hq, Hkv, T)
    seq = np.array([150, 70], np.int32)
    kc, vc = oracle.compress_24(K, seq, cap=192), oracle.compress_24(V, seq, cap=192)
    assert kc.k == 64 and kc.values.shape == (B, Hkv, 192 * 64)
    keep = oracle.prune_rows_24(K)
    for b in range(B):
        T_b = int(seq[b])
        for h in range(Hkv):
            words = kc.bitmaps[b, h, :T_b]
            nib = [(int(w) >> (4 * j)) & 0xF for w in words.reshape(-1) for j in range(16)]
            assert all(bin(n).count("1") == 2 for n in nib)
            flat = K[b, h, :T_b][keep[b, h, :T_b] == 1]
            assert np.array_equal(kc.values[b, h, :T_b * 64], flat)
            nt = (T_b + 63) // 64
            assert kc.tile_off[b, h, :nt + 1].tolist() == [min(64 * j, T_b) * 64 for j in range(nt + 1)]
    Km, Vm = oracle.decompress(kc, seq), oracle.decompress(vc, seq)
    ref = _sdpa_f64(q, Km[:, :, :T], Vm[:, :, :T], seq, 1.0 / math.sqrt(128))
    got = oracle.attention_compressed(q, kc, vc, seq, 1.0 / math.sqrt(128))
    assert np.abs(got - ref).max() < 1e-12


# ---------------------------------------------------------------- channel-wise pruning (R24)
def test_channel_wise_rule_invariants_and_layout():
    """Full 64-row tiles: every channel keeps exactly keep/2 rows, no pruned entry
    of a column outranks a kept one, and equal keys go to the earlier row (these
    three properties determine the kept set); rows of the final partial tile
    follow the per-token rule; values and tile offsets follow the format."""
    rng = np.random.default_rng(41)
    B, H, T, keep = 2, 2, 150, 38
    x = rng.standard_normal((B, H, T, 128)).astype(np.float16)
    x[0, 0, :64, 7] = np.float16(0.5)                    # a column of equal keys
    x[1, 1, 64:128, 90] = np.where(np.arange(64) % 2, 1.0, -1.0)  # +-1: equal magnitudes
    x = x.view(np.uint16)
    seq = np.array([150, 128], np.int32)
    c = oracle.compress_channel(x, seq, keep, cap=192)
    dec = oracle.decompress(c, seq)
    kc = keep // 2
    for b in range(B):
        T_b = int(seq[b])
        for h in range(H):
            kept = np.zeros((T_b, 128), bool)
            for r in range(T_b):
                w = c.bitmaps[b, h, r]
                kept[r] = [(int(w[ch // 64]) >> (ch % 64)) & 1 for ch in range(128)]
            for t0 in range(0, T_b - T_b % 64, 64):
                key = (x[b, h, t0:t0 + 64] & 0x7FFF).astype(np.int64)
                kt = kept[t0:t0 + 64]
                assert (kt.sum(0) == kc).all()
                for ch in range(128):
                    kk, pk = key[kt[:, ch], ch], key[~kt[:, ch], ch]
                    assert kk.min() >= pk.max()
                    tau = kk.min()
                    if (pk == tau).any():
                        assert np.nonzero(kt[:, ch] & (key[:, ch] == tau))[0].max() < \
                            np.nonzero(~kt[:, ch] & (key[:, ch] == tau))[0].min()
            tail = T_b - T_b % 64
            if tail < T_b:
                assert np.array_equal(kept[tail:], oracle.prune_rows(x[b, h, tail:T_b], keep) == 1)
            # format: kept values row by row in channel order, offsets = popcount prefix
            flat = x[b, h, :T_b][kept]
            assert np.array_equal(c.values[b, h, :flat.size], flat)
            pc = kept.sum(1)
            nt = (T_b + 63) // 64
            assert c.tile_off[b, h, :nt + 1].tolist() == [int(pc[:min(64 * j, T_b)].sum())
                                                           for j in range(nt + 1)]
            assert np.array_equal(dec[b, h, :T_b], np.where(kept, x[b, h, :T_b], 0))
    assert c.values.shape[-1] == 192 * keep


def test_channel_wise_attention_equals_sdpa_on_zero_masked_cache():
    rng = np.random.default_rng(42)
    B, Hq, Hkv, T = 2, 4, 2, 200
    q, K, V = _rand_inputs(rng, B, Hq, Hkv, T)
    seq = np.array([200, 64], np.int32)
    kc, vc = oracle.compress_channel(K, seq, 38, cap=256), oracle.compress_channel(V, seq, 64, cap=256)
    Km, Vm = oracle.decompress(kc, seq), oracle.decompress(vc, seq)
    ref = _sdpa_f64(q, Km[:, :, :T], Vm[:, :, :T], seq, 0.0883)
    assert np.abs(oracle.attention_compressed(q, kc, vc, seq, 0.0883) - ref).max() < 1e-12
