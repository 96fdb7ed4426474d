"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module only draws numbers.  It holds none of the method's arithmetic
(no pruning, no compression, no attention): it produces dense fp16 key /
value caches, queries and sequence lengths with the shapes and value
distributions of the workloads, from a counter-based generator, so that any
slice can be regenerated from (seed, stream, layer, flat index).

Generator (published definitions, restated):
  * SplitMix64 (Steele, Lea, Flood: "Fast splittable pseudorandom number
    generators", OOPSLA 2014): output i of a stream with key K is
    mix(K + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64), where mix is the
    two-round xor-shift-multiply finaliser below.
  * a 53-bit uniform u = (z >> 11) * 2^-53 in [0, 1);
  * Box-Muller in float64: n = sqrt(-2 ln(1 - u1)) * cos(2 pi u2), with u1 and
    u2 the stream outputs 2j and 2j + 1 for element j;
  * a scale (outlier channels), then round-to-nearest-even to fp16.

The same code runs on the CPU and on the GPU (torch int64 arithmetic wraps
modulo 2^64; logical right shifts are masked).  Float64 transcendental
results may differ in the last bit between devices, so a test always hands
the oracle the exact fp16 bits the GPU consumed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# stream ids
S_K, S_V, S_Q, S_OUTLIER, S_SEQLEN, S_KNEW, S_VNEW, S_QSTEP = range(8)


def _s64(x: int) -> int:
    """Two's-complement view of a 64-bit pattern as a Python int in int64 range."""
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (exact, modulo 2^64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def _lsr(x: torch.Tensor, s: int) -> torch.Tensor:
    return (x >> s) & ((1 << (64 - s)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(MIX1)
    z = (z ^ _lsr(z, 27)) * _s64(MIX2)
    return z ^ _lsr(z, 31)


def stream_key(seed: int, stream: int, layer: int = 0) -> int:
    return mix64_int(mix64_int(seed) ^ ((stream & 0xFFFF) << 48) ^ ((layer & 0xFFFFFF) << 20) ^ 0x5EED)


def splitmix64(key: int, start: int, n: int, device="cpu") -> torch.Tensor:
    """Outputs start .. start+n-1 of the stream with the given key, as int64 bit patterns."""
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix64(i * _s64(GAMMA) + _s64(key))


def uniform53(key: int, start: int, n: int, device="cpu") -> torch.Tensor:
    z = splitmix64(key, start, n, device)
    return _lsr(z, 11).to(torch.float64) * (2.0 ** -53)


def normal64(key: int, start: int, n: int, device="cpu") -> torch.Tensor:
    """Element j of the stream is Box-Muller of uniforms 2j and 2j+1 (float64)."""
    u = uniform53(key, 2 * start, 2 * n, device).view(n, 2)
    r = torch.sqrt(-2.0 * torch.log1p(-u[:, 0]))
    return r * torch.cos((2.0 * math.pi) * u[:, 1])


def normal_f16(seed: int, stream: int, layer: int, shape, device="cpu",
               chunk: int = 1 << 25) -> torch.Tensor:
    """fp16 N(0,1) tensor of `shape`; flat element e uses stream position e."""
    n = 1
    for s in shape:
        n *= int(s)
    key = stream_key(seed, stream, layer)
    out = torch.empty(n, dtype=torch.float16, device=device)
    for lo in range(0, n, chunk):
        m = min(chunk, n - lo)
        out[lo:lo + m] = normal64(key, lo, m, device).to(torch.float16)
    return out.view(*shape)


def outlier_channels(seed: int, layer: int, heads: int, count: int, d: int = 128) -> torch.Tensor:
    """`count` distinct channels per head: the first `count` of a seeded shuffle of 0..d-1."""
    key = stream_key(seed, S_OUTLIER, layer)
    z = splitmix64(key, 0, heads * d).view(heads, d)
    return torch.argsort(z, dim=1, stable=True)[:, :count].sort(dim=1).values


def dense_cache_f16(seed: int, stream: int, layer: int, B: int, H: int, T: int, d: int,
                    outliers: torch.Tensor | None = None, factor: float = 1.0,
                    device="cpu") -> torch.Tensor:
    """[B][H][T][d] fp16 cache; channels outliers[h] of head h are scaled by `factor`
    (in float64, before the single rounding to fp16)."""
    key = stream_key(seed, stream, layer)
    out = torch.empty((B, H, T, d), dtype=torch.float16, device=device)
    per = T * d
    if outliers is not None:
        scale = torch.ones((H, d), dtype=torch.float64, device=device)
        for h in range(H):
            scale[h, outliers[h].to(device)] = factor
    for b in range(B):
        for h in range(H):
            start = (b * H + h) * per
            x = normal64(key, start, per, device).view(T, d)
            if outliers is not None:
                x = x * scale[h]
            out[b, h] = x.to(torch.float16)
    return out


def seq_lens_uniform(seed: int, B: int, lo: int, hi: int) -> torch.Tensor:
    """B integers uniform over [lo, hi] inclusive (int32, CPU)."""
    u = uniform53(stream_key(seed, S_SEQLEN, 0), 0, B)
    return (lo + torch.floor(u * (hi - lo + 1))).to(torch.int32).clamp_(lo, hi)


@dataclass
class Config:
    """Shape and distribution of one workload (sizes as stated for it)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int                     # cached tokens (max for ragged)
    sparsity: float
    d: int = 128
    k_outliers: str = "random4x10"   # or "fixed_3_77_x8"
    ragged: tuple | None = None       # (lo, hi) inclusive
    steps: int = 0                    # decode steps with append
    layers: int = 1
    seed: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)


CONFIGS = {
    "tiny": Config("tiny", B=1, Hq=2, Hkv=2, T=256, sparsity=0.5, k_outliers="fixed_3_77_x8",
                   notes="B=1, Hq=Hkv=2, d=128, T=256, K channels 3 and 77 x8, 50% sparsity"),
    "llama2_7b_layer": Config("llama2_7b_layer", B=1, Hq=32, Hkv=32, T=4096, sparsity=0.7,
                              notes="Llama-2-7B-shaped MHA layer, B=1, T=4096, 70% sparsity"),
    "llama3_8b_layer": Config("llama3_8b_layer", B=8, Hq=32, Hkv=8, T=32768, sparsity=0.7,
                              notes="Llama-3-8B-shaped GQA 32/8 layer, B=8, T=32768, 70% sparsity"),
    "mistral_ragged_append": Config("mistral_ragged_append", B=16, Hq=32, Hkv=8, T=32768, sparsity=0.5,
                                    ragged=(4096, 32768), steps=64,
                                    notes="Mistral-7B-shaped GQA 32/8, B=16, T_b ~ U{4096..32768}, "
                                          "50% sparsity, 64 append+attend steps"),
    "llama3_8b_stack": Config("llama3_8b_stack", B=1, Hq=32, Hkv=8, T=16384, sparsity=0.7, layers=32,
                              notes="32-layer Llama-3-8B-shaped stack, 70% sparsity, "
                                    "B in {1,4,8,16,32,64} x T in {16384,65536,131072}"),
}


def key_outliers(cfg: Config, layer: int = 0):
    """(channels [Hkv][n], factor) for the key cache of a config."""
    if cfg.k_outliers == "fixed_3_77_x8":
        ch = torch.tensor([[3, 77]] * cfg.Hkv, dtype=torch.int64)
        return ch, 8.0
    return outlier_channels(cfg.seed, layer, cfg.Hkv, 4, cfg.d), 10.0


def make_inputs(cfg: Config, device="cpu", layer: int = 0, B: int | None = None, T: int | None = None):
    """Dense fp16 K, V [B][Hkv][T][d], q [B][Hq][d] and int32 seq_lens [B] for one layer."""
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    ch, f = key_outliers(cfg, layer)
    K = dense_cache_f16(cfg.seed, S_K, layer, B, cfg.Hkv, T, cfg.d, ch, f, device)
    V = dense_cache_f16(cfg.seed, S_V, layer, B, cfg.Hkv, T, cfg.d, None, 1.0, device)
    q = normal_f16(cfg.seed, S_Q, layer, (B, cfg.Hq, cfg.d), device)
    if cfg.ragged is not None:
        seq = seq_lens_uniform(cfg.seed, B, *cfg.ragged)
    else:
        seq = torch.full((B,), T, dtype=torch.int32)
    return K, V, q, seq


def step_inputs(cfg: Config, step: int, device="cpu", layer: int = 0, B: int | None = None):
    """New key/value rows [B][Hkv][d] and a fresh query [B][Hq][d] for decode step `step`
    (keys carry the same outlier channels as the cache)."""
    B = cfg.B if B is None else B
    lay = layer * 4096 + step
    ch, f = key_outliers(cfg, layer)
    kn = dense_cache_f16(cfg.seed, S_KNEW, lay, B, cfg.Hkv, 1, cfg.d, ch, f, device)[:, :, 0]
    vn = dense_cache_f16(cfg.seed, S_VNEW, lay, B, cfg.Hkv, 1, cfg.d, None, 1.0, device)[:, :, 0]
    q = normal_f16(cfg.seed, S_QSTEP, lay, (B, cfg.Hq, cfg.d), device)
    return kn.contiguous(), vn.contiguous(), q

