"""GPU parity for the 2:4 semi-structured comparator: prefill compression bit
for bit against the oracle's 2:4 rule, the 2:4 decode kernel (and the
unstructured decode kernel on the same bytes) within the attention tolerance
of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import unstructured_sparse_kv_amd as usk
from tests.gpu_helpers import SCALE, assert_attn_close, assert_compressed_equal, say

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, T, seed):
    g = torch.Generator().manual_seed(seed)
    K = torch.randn(B, Hkv, T, 128, generator=g, dtype=torch.float64)
    K[..., [3, 77]] *= 8
    V = torch.randn(B, Hkv, T, 128, generator=g, dtype=torch.float64)
    q = torch.randn(B, Hq, 128, generator=g, dtype=torch.float64)
    return K.half(), V.half(), q.half()


def _compress_24(dense, seq_d, cap):
    c = usk.CompressedKV(dense.shape[0], dense.shape[1], 64, cap, dense.device)
    usk.prune_compress_24(c, dense, seq_d)
    return c


def _run(fn, q, kc, vc, seq_d, max_len, splits=0):
    B, Hq = q.shape[0], q.shape[1]
    ws = usk.make_workspace(B, Hq, kc.num_kv_heads, max_len, splits)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=q.device)
    fn(q, kc, vc, seq_d, max_len, SCALE, out, ws, splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_24_compress_and_decode(gpu, G):
    B, Hkv, T, cap = 3, 2, 300, 320
    Hq = G * Hkv
    K, V, q = _inputs(B, Hq, Hkv, T, 240 + G)
    K[0, 0, 5, :] = 0                   # an all-zero row: ties everywhere
    K[1, 1, 7, ::2] = K[1, 1, 7, 1::2]  # pairwise ties inside every group
    seq = np.array([300, 130, 1], np.int32)
    say(f"2:4 comparator G={G}")
    seq_d = torch.from_numpy(seq).to(gpu)
    kc, vc = _compress_24(K.to(gpu), seq_d, cap), _compress_24(V.to(gpu), seq_d, cap)
    torch.cuda.synchronize()
    ko, vo = oracle.compress_24(K, seq, cap), oracle.compress_24(V, seq, cap)
    assert_compressed_equal(kc, ko, seq)
    assert_compressed_equal(vc, vo, seq)
    ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
    for name, fn in (("2:4 kernel", usk.decode_attn_24), ("unstructured kernel", usk.decode_attn)):
        for splits in (0, 1, 3):
            got = _run(fn, q.to(gpu), kc, vc, seq_d, T, splits)
            assert_attn_close(got, ref, f"2:4 G={G} {name} splits={splits}")


def test_24_llama3_layer_sampled(gpu):
    cfg = synth.CONFIGS["llama3_8b_layer"]
    say("2:4 comparator: Llama-3 layer B=8 Hkv=8 T=32768 on the GPU")
    K, V, q, seq = synth.make_inputs(cfg, device=gpu)
    seq_d = seq.to(gpu)
    kc, vc = _compress_24(K, seq_d, cfg.T), _compress_24(V, seq_d, cfg.T)
    torch.cuda.synchronize()
    pairs = [(0, 0), (2, 9), (7, 31)]
    units = sorted({(b, hq // 4) for b, hq in pairs})
    s1 = np.array([cfg.T], np.int32)
    refs = {}
    Kc, Vc, qc = K.cpu(), V.cpu(), q.cpu()
    for b, h in units:
        ko = oracle.compress_24(Kc[b:b + 1, h:h + 1], s1, cfg.T)
        vo = oracle.compress_24(Vc[b:b + 1, h:h + 1], s1, cfg.T)
        assert_compressed_equal(kc, ko, seq.numpy(), [(b, h)], [(0, 0)])
        assert_compressed_equal(vc, vo, seq.numpy(), [(b, h)], [(0, 0)])
        for bb, hq in pairs:
            if (bb, hq // 4) == (b, h):
                refs[(bb, hq)] = oracle.attention_compressed(qc[b:b + 1, hq:hq + 1], ko, vo, s1,
                                                             SCALE)[0, 0]
    got = _run(usk.decode_attn_24, q, kc, vc, seq_d, cfg.T)
    assert_attn_close(np.stack([got[b, hq] for b, hq in pairs]), np.stack([refs[p] for p in pairs]),
                      "2:4 llama3 layer")
