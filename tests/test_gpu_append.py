"""GPU tests of the decode-time append's use of the tile offsets (the run-time
compression of decode tokens, [Summary] "Approach" / [Abstract]):

  * a cache that was never prefilled -- arbitrary bytes in its bitmaps, values
    and tile offsets -- grows from empty sequences exactly as the oracle's
    append says, through mustafar_append_token and through the fused
    mustafar_decode_step;
  * an end entry that would place a row outside its (batch, head) value region
    is never followed: that row writes nothing, MUSTAFAR_STATUS_BAD_OFFSETS is
    set, and every other (batch, head) still appends correctly.
"""
import numpy as np
import pytest
import torch

import oracle
import unstructured_sparse_kv_amd as usk
from tests.gpu_helpers import SCALE, assert_attn_close, assert_compressed_equal, say

pytestmark = pytest.mark.gpu


def _garbage(c: usk.CompressedKV, seed: int):
    g = torch.Generator(device="cpu").manual_seed(seed)
    for t in (c.bitmaps, c.values, c.tile_offsets):
        t.copy_(torch.randint(-2**15, 2**15, t.shape, generator=g, dtype=torch.int64).to(t.dtype))


def _to_oracle(c: usk.CompressedKV) -> "oracle.Compressed":
    bm, vals, toff = c.views()
    o = oracle.Compressed(c.batch, c.num_kv_heads, c.capacity, 128, c.keep)
    o.bitmaps[...] = bm.cpu().numpy().view(np.uint64)
    o.values[...] = vals.cpu().numpy().view(np.uint16)
    o.tile_off[...] = toff.cpu().numpy().view(np.uint32)
    return o


@pytest.mark.parametrize("mode", ["append", "step"])
@pytest.mark.parametrize("keep", [38, 64])
def test_grow_never_prefilled_cache(gpu, mode, keep):
    B, Hq, Hkv, cap, steps = 3, 8, 2, 128, 70
    say(f"never-prefilled cache: mode={mode} keep={keep} steps={steps}")
    kc, vc = usk.CompressedKV(B, Hkv, keep, cap, gpu), usk.CompressedKV(B, Hkv, keep, cap, gpu)
    _garbage(kc, 1)
    _garbage(vc, 2)
    ko, vo = _to_oracle(kc), _to_oracle(vc)      # the oracle starts from the same bytes
    seq_d = torch.zeros(B, dtype=torch.int32, device=gpu)
    seq = np.zeros(B, np.int32)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws = usk.make_workspace(B, Hq, Hkv, cap)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=gpu)
    g = torch.Generator().manual_seed(keep)
    for step in range(steps):
        kn = torch.randn(B, Hkv, 128, generator=g).half()
        vn = torch.randn(B, Hkv, 128, generator=g).half()
        q = torch.randn(B, Hq, 128, generator=g).half()
        if mode == "append":
            usk.append_token(kc, vc, kn.to(gpu), vn.to(gpu), seq_d, status)
            usk.decode_attn(q.to(gpu), kc, vc, seq_d, cap, SCALE, out, ws)
        else:
            usk.decode_step(q.to(gpu), kc, vc, kn.to(gpu), vn.to(gpu), seq_d, cap, SCALE, out, ws, status)
        seq, st = oracle.append_step(ko, vo, kn, vn, seq)
        assert st == 0
        if step in (0, 1, 63, 64, steps - 1):
            torch.cuda.synchronize()
            assert np.array_equal(seq_d.cpu().numpy(), seq)
            assert status.item() == 0
            assert_compressed_equal(kc, ko, seq)
            assert_compressed_equal(vc, vo, seq)
            ref = oracle.attention_compressed(q, ko, vo, seq, SCALE)
            assert_attn_close(out.float().cpu().numpy().astype(np.float64), ref,
                              f"never-prefilled {mode} keep={keep} step {step}")


@pytest.mark.parametrize("mode", ["append", "step"])
def test_bad_end_entry_is_flagged_and_not_followed(gpu, mode):
    B, Hq, Hkv, cap, keep, T = 2, 4, 2, 128, 38, 100
    say(f"bad end entry: mode={mode}")
    g = torch.Generator().manual_seed(9)
    K = torch.randn(B, Hkv, cap, 128, generator=g).half()
    V = torch.randn(B, Hkv, cap, 128, generator=g).half()
    seq = np.full(B, T, np.int32)
    seq_d = torch.from_numpy(seq).to(gpu)
    kc, vc = usk.CompressedKV(B, Hkv, keep, cap, gpu), usk.CompressedKV(B, Hkv, keep, cap, gpu)
    usk.prune_compress(kc, K.to(gpu), seq_d)
    usk.prune_compress(vc, V.to(gpu), seq_d)
    # (b=1, h=0) of the key cache: an end entry one value past the last row start that fits
    end = (T + 63) // 64
    kc.views()[2][1, 0, end] = cap * keep - keep + 1
    before_k = [t.clone() for t in kc.views()]
    kn = torch.randn(B, Hkv, 128, generator=g).half()
    vn = torch.randn(B, Hkv, 128, generator=g).half()
    q = torch.randn(B, Hq, 128, generator=g).half()
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    ws = usk.make_workspace(B, Hq, Hkv, cap)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=gpu)
    if mode == "append":
        usk.append_token(kc, vc, kn.to(gpu), vn.to(gpu), seq_d, status)
    else:
        usk.decode_step(q.to(gpu), kc, vc, kn.to(gpu), vn.to(gpu), seq_d, cap, SCALE, out, ws, status)
    torch.cuda.synchronize()
    assert status.item() == usk.STATUS_BAD_OFFSETS
    assert seq_d.cpu().tolist() == [T + 1] * B
    bm, vals, toff = kc.views()
    # the bad unit: nothing of the new row written (its value region is untouched)
    assert torch.equal(bm[1, 0], before_k[0][1, 0])
    assert torch.equal(vals[1, 0], before_k[1][1, 0])
    assert torch.equal(toff[1, 0], before_k[2][1, 0])
    # every other unit grew exactly as the oracle's append says
    ko = oracle.compress(K, seq, keep, cap)
    vo = oracle.compress(V, seq, keep, cap)
    seq1, st = oracle.append_step(ko, vo, kn, vn, seq)
    assert st == 0
    others = [(0, 0), (0, 1), (1, 1)]
    assert_compressed_equal(kc, ko, seq1, others)
    assert_compressed_equal(vc, vo, seq1)
