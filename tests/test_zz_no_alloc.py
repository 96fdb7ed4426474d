"""mustafar_decode_step_noalloc (the decode step for callers that cannot allocate:
its split partials live in the library's own device array) against
mustafar_decode_step with a caller workspace, through the C ABI: outputs,
caches, lengths and status bit for bit, on two calls in a row -- the second on
a smaller shape, so that it reads the array after a larger call left it full --
and a shape whose partials exceed the array is refused before any launch."""
import numpy as np
import pytest
import torch

import unstructured_sparse_kv_amd as usk
from tests.gpu_helpers import SCALE, say

pytestmark = pytest.mark.gpu


def _caches(B, Hq, Hkv, T, cap, keep, seed, gpu):
    g = torch.Generator().manual_seed(seed)
    K = torch.randn(B, Hkv, cap, 128, generator=g).half().to(gpu)
    V = torch.randn(B, Hkv, cap, 128, generator=g).half().to(gpu)
    seq = torch.tensor([T - 37 * b for b in range(B)], dtype=torch.int32)
    pair = []
    for _ in range(2):
        kc, vc = usk.CompressedKV(B, Hkv, keep, cap, gpu), usk.CompressedKV(B, Hkv, keep, cap, gpu)
        sd = seq.to(gpu)
        usk.prune_compress(kc, K, sd)
        usk.prune_compress(vc, V, sd)
        pair.append((kc, vc, sd))
    kn = torch.randn(B, Hkv, 128, generator=g).half().to(gpu)
    vn = torch.randn(B, Hkv, 128, generator=g).half().to(gpu)
    q = torch.randn(B, Hq, 128, generator=g).half().to(gpu)
    return pair, kn, vn, q


@pytest.mark.parametrize("keep", [38, 64])
def test_noalloc_step_matches_workspace_step(gpu, keep):
    shapes = [(8, 32, 8, 4000, 4096), (2, 16, 2, 700, 768)]  # the second call is smaller
    for i, (B, Hq, Hkv, T, cap) in enumerate(shapes):
        say(f"no-alloc step call {i}: B={B} Hq={Hq} Hkv={Hkv} T={T} keep={keep}")
        pair, kn, vn, q = _caches(B, Hq, Hkv, T, cap, keep, 100 * i + keep, gpu)
        (ka, va, sa), (kb, vb, sb) = pair
        ws = usk.make_workspace(B, Hq, Hkv, cap)
        out_a = torch.full((B, Hq, 128), float("nan"), dtype=torch.float16, device=gpu)
        out_b = torch.full_like(out_a, float("nan"))
        st_a = torch.zeros(1, dtype=torch.int32, device=gpu)
        st_b = torch.zeros(1, dtype=torch.int32, device=gpu)
        usk.decode_step(q, ka, va, kn, vn, sa, cap, SCALE, out_a, ws, st_a)
        usk.decode_step_noalloc(q, kb, vb, kn, vn, sb, cap, SCALE, out_b, st_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"call {i}: out differs"
        assert torch.equal(sa, sb) and st_a.item() == st_b.item() == 0, f"call {i}: lengths/status"
        for c1, c2 in ((ka, kb), (va, vb)):
            for x, y in zip(c1.views(), c2.views()):
                assert torch.equal(x, y), f"call {i}: caches differ"
        assert np.isfinite(out_b.float().cpu().numpy()).all()


def test_noalloc_rejects_partials_beyond_the_array(gpu):
    # batch 256 x 64 q heads x 1 split x 528 B = 8.65 MB > 8 MiB
    B, Hq, Hkv, cap, keep = 256, 64, 8, 64, 38
    kc, vc = usk.CompressedKV(B, Hkv, keep, cap, gpu), usk.CompressedKV(B, Hkv, keep, cap, gpu)
    seq = torch.zeros(B, dtype=torch.int32, device=gpu)
    q = torch.zeros(B, Hq, 128, dtype=torch.float16, device=gpu)
    kn = torch.zeros(B, Hkv, 128, dtype=torch.float16, device=gpu)
    out = torch.zeros_like(q)
    with pytest.raises(usk.MustafarError) as e:
        usk.decode_step_noalloc(q, kc, vc, kn, kn, seq, cap, SCALE, out)
    assert e.value.status == usk.MUSTAFAR_ENOSPACE
    torch.cuda.synchronize()
    assert seq.sum().item() == 0 and not out.any(), "a refused call must launch nothing"
