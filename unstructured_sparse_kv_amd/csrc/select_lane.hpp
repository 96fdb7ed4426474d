// Per-token magnitude selection of one 128-channel row held by one lane
// ([Summary] "Approach": per-token magnitude pruning of the key and value
// caches; [README] "Part II": the token-wise, magnitude-based variant).
//
// The survivors of a row are its `keep` channels of largest magnitude key
// (bits & 0x7FFF; for finite fp16 values this orders like |x|, and -0 == +0),
// ties to the lower channel.  Here every lane works on a row of its own, with
// integer arithmetic on the packed keys only (no cross-lane operations, no
// scalar unit), so one wave selects 64 rows at once:
//
//   1. the top 7 key bits (14..8) of four channels packed in the bytes of a
//      dword, each byte with bit 7 set (the sign bit position): subtracting a
//      candidate c (0..127) from every byte leaves bit 7 set exactly where the
//      byte's field is >= c, with no borrow between bytes, so the count of keys
//      whose top bits are >= c is a popcount of the masked difference (three
//      instructions per four keys).  An MSB-first bisection finds t1, the top
//      bits of the keep-th largest key.
//   2. the same on key bits 7..1 of the channels whose top bits equal t1;
//      channels above t1 count as the largest field, channels below as the
//      smallest, so the count is again that of all keys >= the candidate;
//      this gives key bits 14..1 of the keep-th largest key.
//   3. its bit 0: one count of the full 15-bit keys (two per dword, bit 15 of
//      each half set the same way) against the odd candidate.
//   4. the kept set: every key above tau, plus, of the keys equal to tau, the
//      ones in the lowest channels until `keep` are kept.
//
// The functions compile for the host too (the byte permute has a plain
// fallback there), so the same code is checked on the CPU against the
// oracle's definition.
#pragma once

#include <stdint.h>

#ifndef __HIPCC__
#define MUSTAFAR_HD inline
#else
#include <hip/hip_runtime.h>
#define MUSTAFAR_HD __host__ __device__ __forceinline__
#endif

namespace mustafar {

// v_perm_b32: byte i of the result is byte sel_i (0..7) of the 64-bit value hi:lo.
MUSTAFAR_HD uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(hi, lo, sel);
#else
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) r |= (uint32_t)((v >> (8 * ((sel >> (8 * i)) & 7u))) & 0xFFu) << (8 * i);
  return r;
#endif
}

MUSTAFAR_HD uint32_t popc32(uint32_t v) { return (uint32_t)__builtin_popcount(v); }

constexpr uint32_t kByteTop = 0x80808080u;
constexpr uint32_t kHalfTop = 0x80008000u;

// The n lowest set bits of v (all of v when n >= popcount(v)): the position of
// the n-th set bit by a five-step bisection over prefix popcounts.
MUSTAFAR_HD uint32_t lowest_set_bits(uint32_t v, uint32_t n) {
  if (n == 0u) return 0u;
  uint32_t p = 0u;  // the n-th set bit is at position >= p
#pragma unroll
  for (uint32_t s = 16u; s >= 1u; s >>= 1) {
    const uint32_t below = v & ((1u << (p + s)) - 1u);
    p = popc32(below) < n ? p + s : p;
  }
  // p = position of the n-th set bit (31 when v has fewer than n)
  return p >= 31u ? v : (v & ((2u << p) - 1u));
}

// Keeps the n lowest set bits of the 128-bit mask m (word 0 = channels 0..31).
MUSTAFAR_HD void keep_lowest128(uint32_t (&m)[4], uint32_t n) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t c = popc32(m[w]);
    m[w] = lowest_set_bits(m[w], n);
    n = n > c ? n - c : 0u;
  }
}

// Gathers flags (bit 7 of each byte) of 32 channels into one mask word.
// d[k] (k = 0..7) holds channels 4k..4k+3 in its bytes.  Summing shifted
// copies puts channel 4k + b at bit 8b + k; a fixed bit permutation (index
// bits b1 b0 k2 k1 k0 -> k2 k1 k0 b1 b0, as four swaps of index bits done with
// delta swaps) then puts it at bit 4k + b.
MUSTAFAR_HD uint32_t gather_byte_flags(const uint32_t (&d)[8]) {
  uint32_t w = 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) w |= (d[k] >> (7 - k)) & (0x01010101u << k);
  // index bits (4 3 2 1 0) hold (b1 b0 k2 k1 k0); the target is (k2 k1 k0 b1 b0).
  // Swapping index bits p > q exchanges the bits at positions a and
  // a + 2^p - 2^q for every a with index bit p clear and q set (mask M).
  uint32_t t = (w ^ (w >> 12)) & 0x0000F0F0u;  // bits 4, 2 -> (k2 b0 b1 k1 k0)
  w ^= t ^ (t << 12);
  t = (w ^ (w >> 6)) & 0x00CC00CCu;             // bits 3, 1 -> (k2 k1 b1 b0 k0)
  w ^= t ^ (t << 6);
  t = (w ^ (w >> 3)) & 0x0A0A0A0Au;             // bits 2, 0 -> (k2 k1 k0 b0 b1)
  w ^= t ^ (t << 3);
  t = (w ^ (w >> 1)) & 0x22222222u;             // bits 1, 0 -> (k2 k1 k0 b1 b0)
  w ^= t ^ (t << 1);
  return w;
}

// Selection of the row x (x[j] = channels 2j in the low half, 2j + 1 in the
// high half, fp16 bits) keeping `keep` channels (0..128): bm[w] bit j <=>
// channel 32w + j kept.  The 16-bit passes recompute their operands from x,
// so that the registers a lane holds stay near x plus the 32 byte fields.
MUSTAFAR_HD void lane_select_row(const uint32_t (&x)[64], uint32_t keep, uint32_t (&bm)[4]) {
  // 1. top 7 key bits of channels 4i .. 4i + 3, bit 7 set
  uint32_t f[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) f[i] = byte_perm(x[2 * i + 1], x[2 * i], 0x07050301u) | kByteTop;
  auto count_bytes = [&](uint32_t c) {
    const uint32_t cr = c * 0x01010101u;
    uint32_t n = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) n += popc32((f[i] - cr) & kByteTop);
    return n;
  };
  uint32_t t1 = 0u;
#pragma unroll
  for (int b = 6; b >= 0; --b) {
    const uint32_t cand = t1 | (1u << b);
    t1 = count_bytes(cand) >= keep ? cand : t1;
  }
  // 2. key bits 7..1 where the top bits equal t1; top bits above t1 take the
  // largest field (0x7F), below t1 the smallest (0)
  const uint32_t t1r = t1 * 0x01010101u, t1r1 = (t1 + 1u) * 0x01010101u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t ge = (f[i] - t1r) & kByteTop;
    const uint32_t gt = (f[i] - t1r1) & kByteTop;
    const uint32_t eq = ge ^ gt;
    const uint32_t gtm = gt - (gt >> 7), eqm = eq - (eq >> 7);  // 0x7F in flagged bytes
    const uint32_t low = byte_perm(x[2 * i + 1], x[2 * i], 0x06040200u);
    f[i] = ((low >> 1) & eqm) | gtm | kByteTop;
  }
  uint32_t t2 = 0u;
#pragma unroll
  for (int b = 6; b >= 0; --b) {
    const uint32_t cand = t2 | (1u << b);
    t2 = count_bytes(cand) >= keep ? cand : t2;
  }
  // 3. bit 0: the full keys as 16-bit fields with bit 15 set
  const uint32_t t14 = (t1 << 7) | t2;
  uint32_t n0 = 0u;
  {
    const uint32_t cr = (2u * t14 + 1u) * 0x00010001u;
#pragma unroll
    for (int j = 0; j < 64; ++j) n0 += popc32(((x[j] | kHalfTop) - cr) & kHalfTop);
  }
  const uint32_t tau = n0 >= keep ? 2u * t14 + 1u : 2u * t14;
  // 4. keys > tau, then keys == tau in channel order.  (x | 0x80008000) - tau
  // leaves bit 15 of a half set where key >= tau; one less in each half (no
  // borrow: a half is at least 1) where key > tau.
  uint32_t gt[4], ge[4];
  const uint32_t taur = tau * 0x00010001u;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t dge[8], dgt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t e0 = (x[16 * w + 2 * k] | kHalfTop) - taur;
      const uint32_t e1 = (x[16 * w + 2 * k + 1] | kHalfTop) - taur;
      dge[k] = byte_perm(e1, e0, 0x07050301u);
      dgt[k] = byte_perm(e1 - 0x00010001u, e0 - 0x00010001u, 0x07050301u);
    }
    ge[w] = gather_byte_flags(dge);
    gt[w] = gather_byte_flags(dgt);
  }
  const uint32_t ngt = popc32(gt[0]) + popc32(gt[1]) + popc32(gt[2]) + popc32(gt[3]);
  uint32_t eq[4] = {ge[0] & ~gt[0], ge[1] & ~gt[1], ge[2] & ~gt[2], ge[3] & ~gt[3]};
  keep_lowest128(eq, keep > ngt ? keep - ngt : 0u);
#pragma unroll
  for (int w = 0; w < 4; ++w) bm[w] = gt[w] | eq[w];
}

}  // namespace mustafar
