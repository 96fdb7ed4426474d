"""GPU parity for per-head keep (kv head h keeps head_keep[h] values per row):
prefill compression bit for bit against the oracle's per-head layout, both
sparse decode kernels and the fused decode step within the attention
tolerance of the fp64 oracle, and the fused step bit for bit against separate
append + decode calls."""
import numpy as np
import pytest
import torch

import oracle
import unstructured_sparse_kv_amd as usk
from tests.gpu_helpers import SCALE, assert_attn_close, say

pytestmark = pytest.mark.gpu

SPARSE = {"mfma": usk.decode_attn, "valu": usk.decode_attn_valu}


def _inputs(B, Hq, Hkv, T, seed):
    g = torch.Generator().manual_seed(seed)
    K = torch.randn(B, Hkv, T, 128, generator=g, dtype=torch.float64)
    K[..., [3, 77]] *= 8
    V = torch.randn(B, Hkv, T, 128, generator=g, dtype=torch.float64)
    q = torch.randn(B, Hq, 128, generator=g, dtype=torch.float64)
    return K.half(), V.half(), q.half()


def _compress(dense, seq_d, head_keep, cap):
    B, H = dense.shape[0], dense.shape[1]
    c = usk.CompressedKV(B, H, None, cap, dense.device, head_keep=head_keep)
    usk.prune_compress(c, dense, seq_d)
    return c


def _assert_equal(c, ref, seq):
    bm, vals, toff = (t.cpu().numpy() for t in c.views())
    bm, vals, toff = bm.view(np.uint64), vals.view(np.uint16), toff.view(np.uint32)
    hk = [int(x) for x in c.head_keep]
    for b in range(c.batch):
        T = max(0, min(int(seq[b]), c.capacity))
        nt = (T + 63) // 64 + 1
        for h, kh in enumerate(hk):
            assert np.array_equal(bm[b, h, :T], ref.bitmaps[b, h, :T]), f"bitmaps differ at {(b, h)}"
            assert np.array_equal(toff[b, h, :nt], ref.tile_off[b, h, :nt]), f"offsets differ at {(b, h)}"
            s = c.capacity * sum(hk[:h])
            assert np.array_equal(vals[b, s:s + T * kh], ref.values[b, s:s + T * kh]), \
                f"values differ at {(b, h)}"


def _decode(fn, q, kc, vc, seq_d, max_len, splits=0):
    B, Hq = q.shape[0], q.shape[1]
    ws = usk.make_workspace(B, Hq, kc.num_kv_heads, max_len, splits)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=q.device)
    fn(q, kc, vc, seq_d, max_len, SCALE, out, ws, splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kheads,vheads,G", [
    ([26, 50, 0, 128, 38, 37], [37, 38, 128, 0, 50, 26], 2),   # every bucket edge, keep 0 and 128
    ([28, 32, 34, 38, 38, 42, 44, 48], [48, 44, 42, 38, 38, 34, 32, 28], 4),  # mean 38
    ([38, 38, 64, 64], [64, 64, 38, 38], 1),
    ([28, 32, 34, 38, 38, 42, 44, 48], [48, 44, 42, 38, 38, 34, 32, 28], 8),  # 64 q / 8 kv heads
])
def test_head_keep_compress_and_decode(gpu, kheads, vheads, G):
    Hkv = len(kheads)
    B, T, cap = 3, 200, 256
    Hq = G * Hkv
    K, V, q = _inputs(B, Hq, Hkv, T, sum(kheads) + G)
    seq = np.array([200, 77, 1], np.int32)
    say(f"per-head keep: K {kheads} V {vheads} G={G}")
    seq_d = torch.from_numpy(seq).to(gpu)
    kc = _compress(K.to(gpu), seq_d, kheads, cap)
    vc = _compress(V.to(gpu), seq_d, vheads, cap)
    torch.cuda.synchronize()
    ko = oracle.compress(K, seq, max(kheads), cap, head_keep=kheads)
    vo = oracle.compress(V, seq, max(vheads), cap, head_keep=vheads)
    _assert_equal(kc, ko, seq)
    _assert_equal(vc, vo, seq)
    assert kc.used_bytes(seq) == oracle.used_bytes(B, Hkv, seq, cap, 128, max(kheads), kheads)
    ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
    for variant, fn in SPARSE.items():
        for splits in (0, 1, 3):
            got = _decode(fn, q.to(gpu), kc, vc, seq_d, T, splits)
            assert_attn_close(got, ref, f"per-head {variant} splits={splits}")


@pytest.mark.parametrize("G", [4, 8])
def test_head_keep_decode_step(gpu, G):
    """Fused steps over per-head caches: bit for bit the same as append + decode,
    and the final caches and attention match the oracle on the grown caches."""
    kheads, vheads = [28, 32, 34, 38, 38, 42, 44, 48], [48, 44, 42, 38, 38, 34, 32, 28]
    Hkv = len(kheads)
    B, T, cap = 3, 190, 256
    Hq = G * Hkv
    K, V, q = _inputs(B, Hq, Hkv, cap, 99)
    seq0 = np.array([190, 64, 0], np.int32)
    say(f"per-head keep: fused steps vs separate calls G={G}")
    seq_a = torch.from_numpy(seq0).to(gpu)
    seq_b = seq_a.clone()
    ka, va = _compress(K.to(gpu), seq_a, kheads, cap), _compress(V.to(gpu), seq_a, vheads, cap)
    kb = usk.CompressedKV(B, Hkv, None, cap, gpu, head_keep=kheads)
    vb = usk.CompressedKV(B, Hkv, None, cap, gpu, head_keep=vheads)
    for dst, src in ((kb, ka), (vb, va)):
        for x, y in zip(dst.views(), src.views()):
            x.copy_(y)
    st_a = torch.zeros(1, dtype=torch.int32, device=gpu)
    st_b = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws_a, ws_b = usk.make_workspace(B, Hq, Hkv, cap), usk.make_workspace(B, Hq, Hkv, cap)
    g = torch.Generator().manual_seed(5)
    Kd, Vd = K.clone(), V.clone()
    steps = 3
    for step in range(steps):
        kn = torch.randn(B, Hkv, 128, generator=g).half()
        vn = torch.randn(B, Hkv, 128, generator=g).half()
        qs = torch.randn(B, Hq, 128, generator=g).half().to(gpu)
        for b in range(B):
            Kd[b, :, seq0[b] + step] = kn[b]
            Vd[b, :, seq0[b] + step] = vn[b]
        out_a = torch.empty((B, Hq, 128), dtype=torch.float16, device=gpu)
        out_b = torch.empty_like(out_a)
        usk.append_token(ka, va, kn.to(gpu), vn.to(gpu), seq_a, st_a)
        usk.decode_attn(qs, ka, va, seq_a, cap, SCALE, out_a, ws_a)
        usk.decode_step(qs, kb, vb, kn.to(gpu), vn.to(gpu), seq_b, cap, SCALE, out_b, ws_b, st_b)
        torch.cuda.synchronize()
        assert torch.equal(seq_a, seq_b) and st_a.item() == st_b.item() == 0
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"step {step}: out"
        for c1, c2 in ((ka, kb), (va, vb)):
            for x, y in zip(c1.views(), c2.views()):
                assert torch.equal(x, y), f"step {step}: caches differ"
    seq = seq0 + steps
    assert seq_b.cpu().numpy().tolist() == seq.tolist()
    ko = oracle.compress(Kd, seq, max(kheads), cap, head_keep=kheads)
    vo = oracle.compress(Vd, seq, max(vheads), cap, head_keep=vheads)
    _assert_equal(kb, ko, seq)
    _assert_equal(vb, vo, seq)
    ref = oracle.attention_compressed(qs.cpu(), ko, vo, seq, SCALE)
    assert_attn_close(out_b.float().cpu().numpy().astype(np.float64), ref, "per-head fused step")
