"""Pins for the oracle's decode-time append (oracle.append_rows / append_step):
the new row of every (batch, kv head) is pruned per token and stored after the
rows already compressed ([Summary] "Approach", [Abstract]: run-time pruning and
compression of the tokens produced during decode).

What ties it to something other than itself:
  * under per-token pruning (uniform or per-head keep), appending rows one
    step at a time must give, byte for byte, what compressing the grown dense
    cache in one go gives -- two separate routines of the oracle whose
    agreement is the definition of the format's append;
  * on a channel-wise cache the stored prefix is untouched, the new row's mask
    is the per-token rule (itself pinned by brute force elsewhere), its values
    sit at the old end entry in channel order, and the end entry moves on by
    keep (closed form); decompressing the grown cache gives the zero-masked
    new row;
  * a sequence at capacity is left unchanged and flagged.
No GPU needed."""
import numpy as np
import pytest

import oracle


def _rows(rng, shape):
    x = rng.standard_normal(shape).astype(np.float16)
    return x.view(np.uint16)


def _assert_prefix_equal(a: "oracle.Compressed", b: "oracle.Compressed", seq, end_entry=True):
    """Rows < seq[b] equal in both; tile offsets up to the end entry (without it when
    `a` has grown past seq)."""
    for bb in range(a.B):
        T = int(seq[bb])
        nt = (T + 63) // 64 + (1 if end_entry else 0)
        for h in range(a.H):
            assert np.array_equal(a.bitmaps[bb, h, :T], b.bitmaps[bb, h, :T]), (bb, h)
            if a.head_keep is None:
                assert np.array_equal(a.values[bb, h, :T * a.k], b.values[bb, h, :T * b.k]), (bb, h)
            assert np.array_equal(a.tile_off[bb, h, :nt], b.tile_off[bb, h, :nt]), (bb, h)
    if a.head_keep is not None:
        # per-head layout: compare each head's region over its stored values
        pre = np.concatenate([[0], np.cumsum(a.head_keep)])
        for bb in range(a.B):
            T = int(seq[bb])
            for h in range(a.H):
                lo = a.cap * int(pre[h])
                n = T * int(a.head_keep[h])
                assert np.array_equal(a.values[bb, lo:lo + n], b.values[bb, lo:lo + n]), (bb, h)


@pytest.mark.parametrize("k", [0, 1, 38, 64, 127, 128])
def test_append_equals_compress_of_grown_cache(k):
    rng = np.random.default_rng(100 + k)
    B, H, cap, steps = 4, 2, 192, 70
    seq0 = np.array([0, 1, 63, 120], np.int32)      # empty, one row, a tile's last row, mid-tile
    dense = _rows(rng, (B, H, cap, 128))
    c = oracle.compress(dense, seq0, k, cap)
    seq = seq0.copy()
    for step in range(steps):
        new_k = _rows(rng, (B, H, 128))
        new_v = _rows(rng, (B, H, 128))
        for b in range(B):
            if seq[b] < cap:
                dense[b, :, seq[b]] = new_k[b]
        vc = oracle.compress(dense, seq, k, cap)     # a second tensor sharing the lengths
        seq_next, st = oracle.append_step(c, vc, new_k, new_v, seq)
        assert st == 0
        assert np.array_equal(seq_next, np.minimum(seq + 1, cap))
        seq = seq_next
        if step in (0, 1, 2, 63, steps - 1):
            _assert_prefix_equal(c, oracle.compress(dense, seq, k, cap), seq)
    _assert_prefix_equal(c, oracle.compress(dense, seq, k, cap), seq)


def test_append_per_head_keep_equals_compress_of_grown_cache():
    rng = np.random.default_rng(7)
    B, H, cap = 3, 4, 128
    hk = [0, 37, 64, 128]
    seq = np.array([0, 64, 100], np.int32)
    dense = _rows(rng, (B, H, cap, 128))
    c = oracle.compress(dense, seq, max(hk), cap, head_keep=hk)
    for _ in range(28):
        new = _rows(rng, (B, H, 128))
        for b in range(B):
            dense[b, :, seq[b]] = new[b]
        assert oracle.append_rows(c, new, seq) == 0
        seq = seq + 1
        _assert_prefix_equal(c, oracle.compress(dense, seq, max(hk), cap, head_keep=hk), seq)


def test_append_to_channel_wise_cache():
    rng = np.random.default_rng(11)
    B, H, cap, keep = 2, 2, 256, 38
    seq0 = np.array([192, 130], np.int32)
    dense = _rows(rng, (B, H, cap, 128))
    c = oracle.compress_channel(dense, seq0, keep, cap)
    before = oracle.compress_channel(dense, seq0, keep, cap)
    seq = seq0.copy()
    news = []
    for step in range(3):
        new = _rows(rng, (B, H, 128))
        news.append(new)
        ends = [[int(c.tile_off[b, h, (seq[b] + 63) // 64]) for h in range(H)] for b in range(B)]
        assert oracle.append_rows(c, new, seq) == 0
        mask = oracle.prune_rows(new, keep)
        for b in range(B):
            r = int(seq[b])
            for h in range(H):
                words = [0, 0]
                for ch in np.nonzero(mask[b, h])[0]:
                    words[ch // 64] |= 1 << int(ch % 64)
                assert c.bitmaps[b, h, r].tolist() == words
                e = ends[b][h]
                assert np.array_equal(c.values[b, h, e:e + keep], new[b, h][mask[b, h] == 1])
                assert int(c.tile_off[b, h, (r + 1 + 63) // 64]) == e + keep
                if r % 64 == 0:                       # the new row starts a tile at the old end
                    assert int(c.tile_off[b, h, r // 64]) == e
        seq = seq + 1
    # the channel-wise prefix is untouched; the grown rows decompress to the masked rows
    _assert_prefix_equal(c, before, seq0, end_entry=False)
    dec = oracle.decompress(c, seq)
    for i, new in enumerate(news):
        mask = oracle.prune_rows(new, keep)
        for b in range(B):
            assert np.array_equal(dec[b, :, int(seq0[b]) + i], np.where(mask[b] == 1, new[b], 0))


def test_append_at_capacity_is_flagged_and_changes_nothing():
    rng = np.random.default_rng(3)
    B, H, cap, k = 2, 2, 64, 38
    dense = _rows(rng, (B, H, cap, 128))
    seq = np.array([64, 10], np.int32)
    c = oracle.compress(dense, seq, k, cap)
    snap = (c.bitmaps.copy(), c.values.copy(), c.tile_off.copy())
    new = _rows(rng, (B, H, 128))
    vc = oracle.compress(dense, seq, k, cap)
    seq2, st = oracle.append_step(c, vc, new, new, seq)
    assert st == 1
    assert seq2.tolist() == [64, 11]
    assert np.array_equal(c.bitmaps[0], snap[0][0])
    assert np.array_equal(c.values[0], snap[1][0])
    assert np.array_equal(c.tile_off[0], snap[2][0])
    # the other sequence did grow, as compress of its grown dense cache says
    dense[1, :, 10] = new[1]
    _assert_prefix_equal(c, oracle.compress(dense, seq2, k, cap), seq2)


def test_append_to_empty_sequence_ignores_stale_offsets():
    """An empty sequence's start entry is written, not read: stale offsets left in
    the arrays do not move the new row."""
    rng = np.random.default_rng(5)
    c = oracle.Compressed(1, 2, 64, 128, 38)
    c.tile_off[:] = 0xDEAD
    new = _rows(rng, (1, 2, 128))
    assert oracle.append_rows(c, new, [0]) == 0
    dense = np.zeros((1, 2, 64, 128), np.uint16)
    dense[0, :, 0] = new[0]
    _assert_prefix_equal(c, oracle.compress(dense, [1], 38, 64), [1])
