"""GPU parity for channel-wise pruning: prefill compression bit for bit against
the oracle (full tiles channel-wise, a partial last tile per token), and both
sparse decode kernels over the resulting rows of varying length (up to 128
values, more than keep) within the attention tolerance of the fp64 oracle,
then appends and fused steps on top of such caches."""
import numpy as np
import pytest
import torch

import oracle
import synth
import unstructured_sparse_kv_amd as usk
from tests.gpu_helpers import SCALE, assert_attn_close, assert_compressed_equal, say

pytestmark = pytest.mark.gpu

SPARSE = {"mfma": usk.decode_attn, "valu": usk.decode_attn_valu}


def _inputs(B, Hq, Hkv, T, seed):
    g = torch.Generator().manual_seed(seed)
    K = torch.randn(B, Hkv, T, 128, generator=g, dtype=torch.float64)
    K[..., [3, 77]] *= 8
    V = torch.randn(B, Hkv, T, 128, generator=g, dtype=torch.float64)
    q = torch.randn(B, Hq, 128, generator=g, dtype=torch.float64)
    return K.half(), V.half(), q.half()


def _compress(dense, seq_d, keep, cap):
    c = usk.CompressedKV(dense.shape[0], dense.shape[1], keep, cap, dense.device)
    usk.prune_compress_channel(c, dense, seq_d)
    return c


def _run(fn, q, kc, vc, seq_d, max_len, splits=0):
    B, Hq = q.shape[0], q.shape[1]
    ws = usk.make_workspace(B, Hq, kc.num_kv_heads, max_len, splits)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=q.device)
    fn(q, kc, vc, seq_d, max_len, SCALE, out, ws, splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kk,kv,G", [(38, 38, 4), (64, 64, 4), (2, 126, 4), (0, 128, 4), (38, 8, 4),
                                     (38, 38, 8), (64, 64, 8)])
def test_channel_wise_compress_and_decode(gpu, kk, kv, G):
    B, Hkv, T, cap = 3, 2, 300, 320
    Hq = G * Hkv
    K, V, q = _inputs(B, Hq, Hkv, T, 500 + kk * 7 + kv)
    K[0, 0, :64, 5] = 0.25          # a column of equal keys: ties to the earlier rows
    K[1, 1, 70, :] = 60.0           # a row that wins every channel of its tile
    seq = np.array([300, 256, 37], np.int32)
    say(f"channel-wise keep K={kk} V={kv} G={G}")
    seq_d = torch.from_numpy(seq).to(gpu)
    kc, vc = _compress(K.to(gpu), seq_d, kk, cap), _compress(V.to(gpu), seq_d, kv, cap)
    torch.cuda.synchronize()
    ko = oracle.compress_channel(K, seq, kk, cap)
    vo = oracle.compress_channel(V, seq, kv, cap)
    assert_compressed_equal(kc, ko, seq)
    assert_compressed_equal(vc, vo, seq)
    most = max(int(sum(bin(int(w)).count("1") for w in ko.bitmaps[1, 1, r])) for r in range(64, 128))
    assert most == 128 or kk == 0
    ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
    for name, fn in SPARSE.items():
        for splits in (0, 1, 3):
            got = _run(fn, q.to(gpu), kc, vc, seq_d, T, splits)
            assert_attn_close(got, ref, f"channel-wise K={kk} V={kv} {name} splits={splits}")


def test_channel_wise_then_decode_steps(gpu):
    """Fused decode steps on channel-wise caches: the new rows are pruned per
    token; the result matches separate append + decode calls bit for bit and
    the oracle on the grown caches."""
    B, Hq, Hkv, cap, keep = 2, 8, 2, 256, 38
    K, V, q = _inputs(B, Hq, Hkv, cap, 77)
    seq0 = np.array([192, 130], np.int32)
    seq_a = torch.from_numpy(seq0).to(gpu)
    seq_b = seq_a.clone()
    ka, va = _compress(K.to(gpu), seq_a, keep, cap), _compress(V.to(gpu), seq_a, keep, cap)
    kb = usk.CompressedKV(B, Hkv, keep, cap, gpu)
    vb = usk.CompressedKV(B, Hkv, keep, cap, gpu)
    for dst, src in ((kb, ka), (vb, va)):
        for x, y in zip(dst.views(), src.views()):
            x.copy_(y)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws_a, ws_b = usk.make_workspace(B, Hq, Hkv, cap), usk.make_workspace(B, Hq, Hkv, cap)
    g = torch.Generator().manual_seed(3)
    news = []
    for step in range(3):
        kn = torch.randn(B, Hkv, 128, generator=g).half()
        vn = torch.randn(B, Hkv, 128, generator=g).half()
        qs = torch.randn(B, Hq, 128, generator=g).half().to(gpu)
        news.append((kn, vn))
        out_a = torch.empty((B, Hq, 128), dtype=torch.float16, device=gpu)
        out_b = torch.empty_like(out_a)
        usk.append_token(ka, va, kn.to(gpu), vn.to(gpu), seq_a, st)
        usk.decode_attn(qs, ka, va, seq_a, cap, SCALE, out_a, ws_a)
        usk.decode_step(qs, kb, vb, kn.to(gpu), vn.to(gpu), seq_b, cap, SCALE, out_b, ws_b, st)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"step {step}"
        for c1, c2 in ((ka, kb), (va, vb)):
            for x, y in zip(c1.views(), c2.views()):
                assert torch.equal(x, y), f"step {step}: caches differ"
    assert st.item() == 0
    # oracle: channel-wise prefill, then the oracle's append (new rows pruned per token)
    ko = oracle.compress_channel(K, seq0, keep, cap)
    vo = oracle.compress_channel(V, seq0, keep, cap)
    seq = seq0.copy()
    for kn, vn in news:
        seq, st_o = oracle.append_step(ko, vo, kn, vn, seq)
        assert st_o == 0
    assert np.array_equal(seq, seq0 + 3)
    assert_compressed_equal(kb, ko, seq)
    assert_compressed_equal(vb, vo, seq)
    ref = oracle.attention_compressed(qs.cpu(), ko, vo, seq, SCALE)
    assert_attn_close(out_b.float().cpu().numpy().astype(np.float64), ref, "channel-wise fused steps")


def test_channel_wise_llama3_layer_sampled(gpu):
    cfg = synth.CONFIGS["llama3_8b_layer"]
    keep = usk.keep_from_sparsity(cfg.sparsity)
    say("channel-wise: Llama-3 layer B=8 Hkv=8 T=32768 on the GPU")
    K, V, q, seq = synth.make_inputs(cfg, device=gpu)
    seq_d = seq.to(gpu)
    kc, vc = _compress(K, seq_d, keep, cfg.T), _compress(V, seq_d, keep, cfg.T)
    torch.cuda.synchronize()
    pairs = [(0, 0), (4, 17), (7, 31)]
    s1 = np.array([cfg.T], np.int32)
    Kc, Vc, qc = K.cpu(), V.cpu(), q.cpu()
    refs = {}
    for b, hq in pairs:
        h = hq // 4
        ko = oracle.compress_channel(Kc[b:b + 1, h:h + 1], s1, keep, cfg.T)
        vo = oracle.compress_channel(Vc[b:b + 1, h:h + 1], s1, keep, cfg.T)
        assert_compressed_equal(kc, ko, seq.numpy(), [(b, h)], [(0, 0)])
        assert_compressed_equal(vc, vo, seq.numpy(), [(b, h)], [(0, 0)])
        refs[(b, hq)] = oracle.attention_compressed(qc[b:b + 1, hq:hq + 1], ko, vo, s1, SCALE)[0, 0]
    for name, fn in SPARSE.items():
        got = _run(fn, q, kc, vc, seq_d, cfg.T)
        assert_attn_close(np.stack([got[b, hq] for b, hq in pairs]),
                          np.stack([refs[p] for p in pairs]), f"channel-wise llama3 {name}")
