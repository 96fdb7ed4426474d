// Per-token magnitude selection of one 128-channel row by one wave, and the
// packing of its survivors (shared by the prune/append kernels and the fused
// decode step).  Sources: [Summary] "Approach" (per-token magnitude pruning
// into a bitmap-based format); [README] "Part II" (the token-wise,
// magnitude-based variant).
//
// Lane l holds channels l and l + 64, so "channel order" is "register 0 lanes,
// then register 1 lanes", which is the order ballot and mbcnt count in.
#pragma once

#include "device_common.hpp"

namespace mustafar {

struct RowMask {
  uint64_t w0, w1;  // kept channels 0..63 and 64..127
};

// Survivors of one row: the `keep` largest magnitude keys (bits & 0x7FFF; finite
// fp16 magnitudes order like these integers, and -0 == +0), ties to the lower
// channel.  tau is found by an MSB-first bisection over the 15 key bits: the
// largest value with #(key >= tau) >= keep, i.e. the keep-th largest key.  From
// bit 10 down the loop stops early once exactly `keep` keys are >= the
// candidate (any such candidate selects the same survivors); above it an exact
// count is too rare to be worth the test's scalar instructions.
__device__ __forceinline__ RowMask select_row(uint32_t x0, uint32_t x1, int keep) {
  const uint32_t k0 = x0 & 0x7FFFu, k1 = x1 & 0x7FFFu;
  uint32_t tau = 0;
#pragma unroll
  for (int b = 14; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    const int cnt = __popcll(__ballot(k0 >= cand)) + __popcll(__ballot(k1 >= cand));
    if (cnt >= keep) tau = cand;
    if (b <= 10 && cnt == keep) break;
  }
  const uint64_t g0 = __ballot(k0 > tau), g1 = __ballot(k1 > tau);
  const int need = keep - (__popcll(g0) + __popcll(g1));
  const uint64_t e0 = __ballot(k0 == tau), e1 = __ballot(k1 == tau);
  const int r0 = (int)mbcnt64(e0, 0u);
  const int r1 = (int)mbcnt64(e1, (uint32_t)__popcll(e0));
  const bool keep0 = (k0 > tau) || (k0 == tau && r0 < need);
  const bool keep1 = (k1 > tau) || (k1 == tau && r1 < need);
  return RowMask{__ballot(keep0), __ballot(keep1)};
}

template <int CTRL>
__device__ __forceinline__ uint32_t quad_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// The lane's channel survives the 2:4 rule: of the 4 lanes of its quad (one
// group of 4 consecutive channels) the 2 of largest key survive, ties to the
// lower channel.  A partner lane (lane ^ s) holds a lower channel exactly when
// the highest bit of s is set in the lane's position within the quad.
__device__ __forceinline__ bool keep_24(uint32_t k) {
  const uint32_t me = lane_id() & 3u;
  const uint32_t k1 = quad_mov<0xB1>(k);  // lane ^ 1
  const uint32_t k2 = quad_mov<0x4E>(k);  // lane ^ 2
  const uint32_t k3 = quad_mov<0x1B>(k);  // lane ^ 3
  const int beaten = (int)(k1 > k || (k1 == k && (me & 1u))) +
                     (int)(k2 > k || (k2 == k && (me & 2u))) +
                     (int)(k3 > k || (k3 == k && (me & 2u)));
  return beaten < 2;
}

// 2:4 semi-structured selection of one row (the structured comparator of the
// unstructured rule above): 2 survivors in every group of 4 consecutive
// channels, chosen by magnitude key with ties to the lower channel.
__device__ __forceinline__ RowMask select_row_24(uint32_t x0, uint32_t x1) {
  return RowMask{__ballot(keep_24(x0 & 0x7FFFu)), __ballot(keep_24(x1 & 0x7FFFu))};
}

// A new row of `keep` values starting at value `pos` of its (batch, head)
// value region (capacity * keep values) stays inside the region.  The start
// comes from the tile-offset end entry in device memory, so it is checked
// before any store follows it.
__device__ __forceinline__ bool append_fits(uint32_t pos, int keep, int cap) {
  return (uint64_t)pos + (uint64_t)keep <= (uint64_t)cap * (uint64_t)keep;
}

// Writes the row's bitmap words and packs its kept values (ascending channel)
// at `vals`.
__device__ __forceinline__ void store_row(const RowMask& m, uint32_t x0, uint32_t x1,
                                          uint64_t* bm_row, uint16_t* vals) {
  const uint32_t lane = lane_id();
  const uint32_t pos0 = mbcnt64(m.w0, 0u);
  const uint32_t pos1 = mbcnt64(m.w1, (uint32_t)__popcll(m.w0));
  if ((m.w0 >> lane) & 1ull) vals[pos0] = (uint16_t)x0;
  if ((m.w1 >> lane) & 1ull) vals[pos1] = (uint16_t)x1;
  if (lane == 0) {
    uint4 w;
    w.x = (uint32_t)m.w0;
    w.y = (uint32_t)(m.w0 >> 32);
    w.z = (uint32_t)m.w1;
    w.w = (uint32_t)(m.w1 >> 32);
    *reinterpret_cast<uint4*>(bm_row) = w;
  }
}

}  // namespace mustafar
