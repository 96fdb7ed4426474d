// Per-token magnitude selection of one 128-channel row held by one lane
// ([Summary] "Approach": per-token magnitude pruning of the key and value
// caches; [README] "Part II": the token-wise, magnitude-based variant).
//
// The survivors of a row are its `keep` channels of largest magnitude key
// (bits & 0x7FFF; for finite fp16 values this orders like |x|, and -0 == +0),
// ties to the lower channel.  Here every lane works on a row of its own, with
// integer arithmetic on the packed keys only (no cross-lane operations, no
// scalar unit), so one wave selects 64 rows at once.  The row's dwords first
// get bit 15 of both halves set (the sign is not part of the key), then:
//
//   1. key bits 14..8 of four channels packed in the bytes of a dword (bit 7
//      of every byte set).  The number of fields >= a candidate c comes from
//      two byte sums of absolute differences: for one field v,
//      |v - (c - 1)| - |v - c| is +1 when v >= c and -1 otherwise, so
//      sad(c - 1) - sad(c) + 128 is twice the count (two v_sad_u8 per four
//      keys).  An MSB-first bisection finds t1, bits 14..8 of the keep-th
//      largest key.
//   2. the same on key bits 7..0 of the channels whose bits 14..8 equal t1,
//      with 255 for the channels above t1 and 0 for those below, so the count
//      is again that of all keys >= the candidate.  The fields come from one
//      saturating 16-bit window per half, min(max(key - t1 * 256, 0), 255),
//      low bytes packed.  This gives tau, the keep-th largest key.
//   3. the sets {key >= tau} and {key > tau}: (key | 0x8000) - c keeps bit 15
//      set exactly where key >= c, with no borrow between the halves; a byte
//      permute spreads those bits of two dwords into four 0x00 / 0xFF bytes,
//      eight such dwords merge into one word by bit-field inserts, and a fixed
//      bit permutation puts every channel at its own bit.
//   4. the kept set: every key above tau, plus, of the keys equal to tau, the
//      ones in the lowest channels until `keep` are kept.
//
// The functions compile for the host too (plain fallbacks of the byte
// permute, the byte sum of absolute differences and the 16-bit saturating
// window), so the same code is checked on the CPU against the oracle's
// definition.
#pragma once

#include <stdint.h>

#ifndef __HIPCC__
#define MUSTAFAR_HD inline
#else
#include <hip/hip_runtime.h>
#define MUSTAFAR_HD __host__ __device__ __forceinline__
#endif

namespace mustafar {

// v_perm_b32 on the 64-bit value hi:lo: selector byte s gives byte s of it
// (0..7), the sign of byte 1, 3, 5 or 7 spread over the byte (8..11), 0x00
// (12) or 0xFF (13..).
MUSTAFAR_HD uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(hi, lo, sel);
#else
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = (sel >> (8 * i)) & 0xFFu;
    uint32_t byte;
    if (s < 8u) byte = (uint32_t)(v >> (8 * s)) & 0xFFu;
    else if (s < 12u) byte = ((v >> (16 * (s - 8u) + 15u)) & 1u) ? 0xFFu : 0u;
    else byte = s == 12u ? 0u : 0xFFu;
    r |= byte << (8 * i);
  }
  return r;
#endif
}

MUSTAFAR_HD uint32_t popc32(uint32_t v) { return (uint32_t)__builtin_popcount(v); }

// sum over the four bytes of |a_b - c_b|, plus acc (v_sad_u8).
MUSTAFAR_HD uint32_t sad_u8(uint32_t a, uint32_t c, uint32_t acc) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_sad_u8(a, c, acc);
#else
  for (int i = 0; i < 4; ++i) {
    const int d = (int)((a >> (8 * i)) & 0xFFu) - (int)((c >> (8 * i)) & 0xFFu);
    acc += (uint32_t)(d < 0 ? -d : d);
  }
  return acc;
#endif
}

// Twice the number of the 128 byte fields of f that are >= c (c replicated in
// every byte, c >= 1 in each): for one field, |v - (c - 1)| - |v - c| is +1
// when v >= c and -1 otherwise, so the difference of the two sums of absolute
// differences plus 128 is 2 * #{v >= c}.  Two v_sad_u8 per four fields.
MUSTAFAR_HD uint32_t sad_count2(const uint32_t (&f)[32], uint32_t c) {
  const uint32_t cm = c - 0x01010101u;
  uint32_t lo0 = 128u, lo1 = 0u, hi0 = 0u, hi1 = 0u;  // four independent chains
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    lo0 = sad_u8(f[i], cm, lo0);
    hi0 = sad_u8(f[i], c, hi0);
    lo1 = sad_u8(f[i + 1], cm, lo1);
    hi1 = sad_u8(f[i + 1], c, hi1);
  }
  return (lo0 + lo1) - (hi0 + hi1);
}

// Per 16-bit half: max(a - b, 0), capped at 255.
MUSTAFAR_HD uint32_t window_u16x2(uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 s = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(s, (u16x2){255, 255}));
#else
  uint32_t r = 0;
  for (int h = 0; h < 2; ++h) {
    const uint32_t p = (a >> (16 * h)) & 0xFFFFu, q = (b >> (16 * h)) & 0xFFFFu;
    const uint32_t s = p > q ? p - q : 0u;
    r |= (s > 255u ? 255u : s) << (16 * h);
  }
  return r;
#endif
}

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

// Merges eight words of 0x00 / 0xFF bytes into one: byte b of d[k] (the flag
// of channel 4k + b) lands at bit 8b + k, by bit-field inserts.
MUSTAFAR_HD uint32_t merge_byte_masks(const uint32_t (&d)[8]) {
  uint32_t w = d[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    const uint32_t m = 0x01010101u * ((1u << k) - 1u);  // bits 0 .. k-1 of every byte
    w = (w & m) | (d[k] & ~m);
  }
  return w;
}

// The fixed bit permutation from bit 8b + k to bit 4k + b (b = 0..3, k =
// 0..7): index bits (b1 b0 k2 k1 k0) -> (k2 k1 k0 b1 b0), as four swaps of
// index bits done with delta swaps (swapping index bits p > q exchanges the
// bits at positions a and a + 2^p - 2^q for every a with bit p clear and bit q
// set: mask M).
MUSTAFAR_HD uint32_t to_channel_order(uint32_t w) {
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

// m[w] bit j <=> key of channel 32w + j >= c (0 <= c <= 0x8000), in the merged
// bit order of merge_byte_masks (not yet in channel order).  xh: the row with
// bit 15 of both halves set, so (xh - c) keeps bit 15 of a half exactly where
// its key >= c, with no borrow between the halves.
MUSTAFAR_HD void keys_at_least(const uint32_t (&xh)[64], uint32_t c, uint32_t (&m)[4]) {
  const uint32_t cr = c * 0x00010001u;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t d[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      d[k] = byte_perm(xh[16 * w + 2 * k + 1] - cr, xh[16 * w + 2 * k] - cr, 0x0B0A0908u);
    m[w] = merge_byte_masks(d);
  }
}

// Selection of the row x (x[j] = channels 2j in the low half, 2j + 1 in the
// high half, fp16 bits) keeping `keep` channels (0..128): bm[w] bit j <=>
// channel 32w + j kept.  x is overwritten (bit 15 of every half set).
MUSTAFAR_HD void lane_select_row(uint32_t (&x)[64], uint32_t keep, uint32_t (&bm)[4]) {
#pragma unroll
  for (int j = 0; j < 64; ++j) x[j] |= kHalfTop;
  // the bisections compare sad(c - 1) - sad(c) + 128 = 2 * #{field >= c}
  // with 2 * keep
  const uint32_t keep2 = 2u * keep;
  // 1. key bits 14..8 of channels 4i .. 4i + 3 (bytes 1 and 3 of two dwords,
  // with bit 7 set: the same for every field and every candidate)
  uint32_t f[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) f[i] = byte_perm(x[2 * i + 1], x[2 * i], 0x07050301u);
  uint32_t t1r = kByteTop;  // t1 in every byte, bit 7 set
#pragma unroll
  for (int b = 6; b >= 0; --b) {
    const uint32_t cand = t1r | (0x01010101u << b);
    t1r = sad_count2(f, cand) >= keep2 ? cand : t1r;
  }
  const uint32_t t1 = t1r & 0x7Fu;
  // 2. key bits 7..0 where bits 14..8 equal t1 (255 above t1, 0 below):
  // min(max(key - t1 * 256, 0), 255) per half, the low bytes packed
  const uint32_t base = ((t1 << 8) | 0x8000u) * 0x00010001u;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    f[i] = byte_perm(window_u16x2(x[2 * i + 1], base), window_u16x2(x[2 * i], base), 0x06040200u);
  uint32_t t2r = 0u;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    const uint32_t cand = t2r | (0x01010101u << b);
    t2r = sad_count2(f, cand) >= keep2 ? cand : t2r;
  }
  // 3. the sets {key >= tau} and {key > tau}
  const uint32_t tau = (t1 << 8) | (t2r & 0xFFu);
  uint32_t ge[4], gt[4], eq[4];
  keys_at_least(x, tau, ge);
  keys_at_least(x, tau + 1u, gt);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    eq[w] = to_channel_order(ge[w] & ~gt[w]);
    gt[w] = to_channel_order(gt[w]);
  }
  // 4. keys > tau, then keys == tau in channel order
  const uint32_t ngt = popc32(gt[0]) + popc32(gt[1]) + popc32(gt[2]) + popc32(gt[3]);
  keep_lowest128(eq, keep > ngt ? keep - ngt : 0u);
#pragma unroll
  for (int w = 0; w < 4; ++w) bm[w] = gt[w] | eq[w];
}

// The bit at position i moves to position rotl5(i, 1): bit i of the low half
// to bit 2i, bit i of the high half to bit 2i + 1 (index bits (i4 i3 i2 i1
// i0) -> (i3 i2 i1 i0 i4): a byte permute for index bits 4, 3, then delta
// swaps for 3/2, 2/1 and 1/0).
MUSTAFAR_HD uint32_t shuffle32(uint32_t w) {
  w = byte_perm(w, w, 0x03010200u);
  uint32_t t = (w ^ (w >> 4)) & 0x00F000F0u;
  w ^= t ^ (t << 4);
  t = (w ^ (w >> 2)) & 0x0C0C0C0Cu;
  w ^= t ^ (t << 2);
  t = (w ^ (w >> 1)) & 0x22222222u;
  w ^= t ^ (t << 1);
  return w;
}

// Twice the number of the 64 byte fields of f that are >= c (see
// sad_count2).
MUSTAFAR_HD uint32_t sad_count2_64(const uint32_t (&f)[16], uint32_t c) {
  const uint32_t cm = c - 0x01010101u;
  uint32_t lo0 = 64u, lo1 = 0u, hi0 = 0u, hi1 = 0u;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    lo0 = sad_u8(f[i], cm, lo0);
    hi0 = sad_u8(f[i], c, hi0);
    lo1 = sad_u8(f[i + 1], cm, lo1);
    hi1 = sad_u8(f[i + 1], c, hi1);
  }
  return (lo0 + lo1) - (hi0 + hi1);
}

// Channel-wise selection of the two channels one lane holds over a 64-row
// tile ([README] "Part II": the channel-wise direction of magnitude pruning).
// y[r] = row r's fp16 bits of channel 2l (low half) and 2l + 1 (high half).
// Each channel keeps its kc (0..64) rows of largest magnitude key, ties to
// the earlier row: lo[w] / hi[w] bit j <=> row 32w + j kept for the low /
// high channel.  The steps are those of lane_select_row, on 64 keys per
// channel with the two channels side by side: byte fields of four rows of one
// channel per dword (from two permutes of two dwords each), the 16-bit window
// and the comparisons with a threshold per half.  y is overwritten.
MUSTAFAR_HD void lane_select_columns(uint32_t (&y)[64], uint32_t kc, uint32_t (&lo)[2],
                                     uint32_t (&hi)[2]) {
#pragma unroll
  for (int r = 0; r < 64; ++r) y[r] |= kHalfTop;
  const uint32_t kc2 = 2u * kc;
  uint32_t fl[16], fh[16];
  // byte bl of the low half and bh of the high half of rows 4i .. 4i + 3
  auto fields = [&](uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t sel, int i) {
    const uint32_t pa = byte_perm(a1, a0, sel), pb = byte_perm(a3, a2, sel);
    fl[i] = byte_perm(pb, pa, 0x05040100u);
    fh[i] = byte_perm(pb, pa, 0x07060302u);
  };
  // 1. key bits 14..8 (bytes 1 and 3, bit 7 set)
#pragma unroll
  for (int i = 0; i < 16; ++i) fields(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3], 0x07030501u, i);
  uint32_t t1l = kByteTop, t1h = kByteTop;
#pragma unroll
  for (int b = 6; b >= 0; --b) {
    const uint32_t cl = t1l | (0x01010101u << b), ch = t1h | (0x01010101u << b);
    t1l = sad_count2_64(fl, cl) >= kc2 ? cl : t1l;
    t1h = sad_count2_64(fh, ch) >= kc2 ? ch : t1h;
  }
  const uint32_t u1l = t1l & 0x7Fu, u1h = t1h & 0x7Fu;
  // 2. key bits 7..0 within each channel's t1 bucket (bytes 0 and 2 of the window)
  const uint32_t base = (((u1h << 8) | 0x8000u) << 16) | ((u1l << 8) | 0x8000u);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    fields(window_u16x2(y[4 * i], base), window_u16x2(y[4 * i + 1], base), window_u16x2(y[4 * i + 2], base),
           window_u16x2(y[4 * i + 3], base), 0x06020400u, i);
  uint32_t t2l = 0u, t2h = 0u;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    const uint32_t cl = t2l | (0x01010101u << b), ch = t2h | (0x01010101u << b);
    t2l = sad_count2_64(fl, cl) >= kc2 ? cl : t2l;
    t2h = sad_count2_64(fh, ch) >= kc2 ? ch : t2h;
  }
  // 3. rows >= tau and > tau per channel: bit 15 / 31 of y - tau, sixteen
  // rows per word (low half: the low channel), then 64-bit row masks
  const uint32_t taur = (((u1h << 8) | (t2h & 0xFFu)) << 16) | ((u1l << 8) | (t2l & 0xFFu));
  auto rows_at_least = [&](uint32_t cr, uint32_t (&ml)[2], uint32_t (&mh)[2]) {
    uint32_t g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t d[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        d[k] = byte_perm(y[16 * q + 2 * k + 1] - cr, y[16 * q + 2 * k] - cr, 0x0B0A0908u);
      g[q] = shuffle32(merge_byte_masks(d));  // low half: rows of the low channel
    }
    ml[0] = byte_perm(g[1], g[0], 0x05040100u);
    ml[1] = byte_perm(g[3], g[2], 0x05040100u);
    mh[0] = byte_perm(g[1], g[0], 0x07060302u);
    mh[1] = byte_perm(g[3], g[2], 0x07060302u);
  };
  uint32_t gel[2], geh[2], gtl[2], gth[2];
  rows_at_least(taur, gel, geh);
  rows_at_least(taur + 0x00010001u, gtl, gth);
  // 4. rows > tau, then rows == tau from the earliest
  auto finish = [&](const uint32_t (&ge)[2], const uint32_t (&gt)[2], uint32_t (&out)[2]) {
    const uint32_t ngt = popc32(gt[0]) + popc32(gt[1]);
    uint32_t n = kc > ngt ? kc - ngt : 0u;
    uint32_t e0 = ge[0] & ~gt[0], e1 = ge[1] & ~gt[1];
    const uint32_t c0 = popc32(e0);
    e0 = lowest_set_bits(e0, n);
    n = n > c0 ? n - c0 : 0u;
    e1 = lowest_set_bits(e1, n);
    out[0] = gt[0] | e0;
    out[1] = gt[1] | e1;
  };
  finish(gel, gtl, lo);
  finish(geh, gth, hi);
}

}  // namespace mustafar
