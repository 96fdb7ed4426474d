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
//   1. the top 7 key bits (14..8) of four channels packed in the bytes of a
//      dword, each byte with bit 7 set: subtracting a candidate c (0..127)
//      from every byte leaves bit 7 set exactly where the byte's field is
//      >= c, with no borrow between bytes, so the count of keys whose top bits
//      are >= c is a popcount of the masked difference (three instructions per
//      four keys).  An MSB-first bisection finds t1, the top bits of the
//      keep-th largest key.
//   2. the same on key bits 7..1 of the channels whose top bits equal t1;
//      channels above t1 count as the largest field, channels below as the
//      smallest, so the count is again that of all keys >= the candidate.  The
//      fields come from one saturating 16-bit window per half: max(key - t1 *
//      256, 0) capped at 255, shifted down one bit.  This gives key bits 14..1
//      of the keep-th largest key.
//   3. its bit 0 and the kept set from two 16-bit comparisons of all keys:
//      E = {key >= odd candidate}; the count of E decides bit 0, and with the
//      other comparison O ({key >= candidate + 1} when bit 0 is 1, {key >=
//      candidate - 1} when it is 0) E and O are the sets {key >= tau} and
//      {key > tau}.  A comparison leaves bit 15 of each half set where key >=
//      the candidate; a byte permute turns those bits of two dwords into four
//      0x00 / 0xFF bytes, eight such dwords merge into one word by bit-field
//      inserts, and a fixed bit permutation puts every channel at its own bit.
//   4. the kept set: every key above tau, plus, of the keys equal to tau, the
//      ones in the lowest channels until `keep` are kept.
//
// The functions compile for the host too (plain fallbacks of the byte permute
// and the 16-bit saturating window), so the same code is checked on the CPU
// against the oracle's definition.
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

// popcount(v) + acc as one v_bcnt_u32_b32 (left to itself the compiler turns a
// running count into a tree of separate popcounts and three-input adds).
MUSTAFAR_HD uint32_t popc_add(uint32_t v, uint32_t acc) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t r;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(acc));
  return r;
#else
  return popc32(v) + acc;
#endif
}

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
  uint32_t lo = 128u, hi = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    lo = sad_u8(f[i], cm, lo);
    hi = sad_u8(f[i], c, hi);
  }
  return lo - hi;
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

}  // namespace mustafar
