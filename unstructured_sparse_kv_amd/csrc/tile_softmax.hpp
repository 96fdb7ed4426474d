// Online softmax over one 64-row tile's scores, shared by the matrix-core
// decode kernels (the softmax of the attention the pages compute over the
// compressed caches, [Summary] "Approach"; split-K bookkeeping in merge.hpp).
//
// Input: the score MFMA's four 16x16 outputs.  Lane (l16, grp) holds in
// cs[mb][i] the score of tile row 16 mb + 4 grp + i for head (column) l16;
// only columns < G are heads.  Scores are in log2 units after scale_log2.
// State per lane: the reference maximum m and the running sum lsum of a head,
// and the P.V accumulators acc (rescaled when m moves).  Output: the tile's
// probabilities, fp16, at p_lds[head][row].
//
// With G <= 4 the scores are first compacted: three DPP moves per score
// register (row_shr 4, 8, 12, each writing one 4-lane bank) bring row block mb
// of head h to lane 4 mb + h of its 16-lane row, so that every lane holds 4
// real scores (head l16 % 4, rows 16 (l16 / 4) + 4 grp + i) instead of 16 of
// which most are padding; the scaling, exponentials and conversions then run a
// quarter as often.  A head's maximum and sum are gathered over the four banks
// with row_ror 4 and 8 and over the lane groups with xor 16 and 32 (lane swaps
// on the vector units).  With G = 8
// the same is done with one move per register (blocks 2 and 3 to the lanes of
// columns 8-15), leaving 8 scores per lane.
#pragma once

#include "device_common.hpp"

namespace mustafar {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The reference maximum moves only when a score exceeds it by more than this
// (log2 units), so p stays below 2^8, well inside the fp16 range at the same
// relative precision, and most tiles skip the rescale.
constexpr float kSoftmaxSlack = 8.f;

// v within each 16-lane row rotated by N lanes (DPP row_ror:N)
template <int N>
__device__ __forceinline__ float row_ror_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xF,
                                                            0xF, false));
}

template <int G>
__device__ __forceinline__ void tile_softmax(const f32x4 (&cs)[4], float scale_log2, bool partial,
                                             int nvalid, uint32_t l16, uint32_t grp, float& m,
                                             float& lsum, f32x4 (&acc)[8], uint16_t* p_lds) {
  const float ninf = -__builtin_inff();
  if constexpr (G <= 4) {
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // (vector elements copied out first: a bit cast applied to cs[mb][i]
      // directly compiles to element 0 for every i)
      const float e0 = cs[0][i], e1 = cs[1][i], e2 = cs[2][i], e3 = cs[3][i];
      int r = __builtin_bit_cast(int, e0);
      r = __builtin_amdgcn_update_dpp(r, __builtin_bit_cast(int, e1), 0x114, 0xF, 0x2, false);
      r = __builtin_amdgcn_update_dpp(r, __builtin_bit_cast(int, e2), 0x118, 0xF, 0x4, false);
      r = __builtin_amdgcn_update_dpp(r, __builtin_bit_cast(int, e3), 0x11C, 0xF, 0x8, false);
      sv[i] = __builtin_bit_cast(float, r) * scale_log2;
    }
    const int row0 = 16 * (int)(l16 >> 2) + 4 * (int)grp;
    if (partial) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = (row0 + i < nvalid) ? sv[i] : ninf;
    }
    float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mt = fmaxf(mt, row_ror_f<4>(mt));
    mt = fmaxf(mt, row_ror_f<8>(mt));
    mt = max_xor32(max_xor16(mt));
    // m, lsum belong to head l16 % 4: lanes l16 < G hold the heads' states
    if (__ballot(mt > m + kSoftmaxSlack) != 0ull) {
      const float mn = fmaxf(m, mt);
      const float alpha = exp2_raw(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb] *= alpha;
    }
    const float p0 = exp2_raw(sv[0] - m), p1 = exp2_raw(sv[1] - m);
    const float p2 = exp2_raw(sv[2] - m), p3 = exp2_raw(sv[3] - m);
    lsum += (p0 + p1) + (p2 + p3);
    if ((int)(l16 & 3u) < G)
      *reinterpret_cast<uint2*>(p_lds + (l16 & 3u) * 64 + row0) = make_uint2(
          (uint32_t)float_to_half_bits(p0) | ((uint32_t)float_to_half_bits(p1) << 16),
          (uint32_t)float_to_half_bits(p2) | ((uint32_t)float_to_half_bits(p3) << 16));
  } else if constexpr (G == 8) {
    // heads in columns 0-7: blocks 2 and 3 move to the lanes of columns 8-15,
    // so lane l16 holds head l16 % 8, row blocks 2 (l16 / 8) and 2 (l16 / 8) + 1
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e0 = cs[0][i], e1 = cs[1][i], e2 = cs[2][i], e3 = cs[3][i];
      sv[i] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                  __builtin_bit_cast(int, e0), __builtin_bit_cast(int, e2), 0x118, 0xF, 0xC, false)) *
              scale_log2;
      sv[4 + i] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                      __builtin_bit_cast(int, e1), __builtin_bit_cast(int, e3), 0x118, 0xF, 0xC, false)) *
                  scale_log2;
    }
    const int row0 = 32 * (int)(l16 >> 3) + 4 * (int)grp;  // rows row0 + i and row0 + 16 + i
    if (partial) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = (row0 + i < nvalid) ? sv[i] : ninf;
        sv[4 + i] = (row0 + 16 + i < nvalid) ? sv[4 + i] : ninf;
      }
    }
    float mt = ninf;
#pragma unroll
    for (int j = 0; j < 8; ++j) mt = fmaxf(mt, sv[j]);
    mt = fmaxf(mt, row_ror_f<8>(mt));
    mt = max_xor32(max_xor16(mt));
    if (__ballot(mt > m + kSoftmaxSlack) != 0ull) {
      const float mn = fmaxf(m, mt);
      const float alpha = exp2_raw(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb] *= alpha;
    }
    float ps = 0.f;
    uint32_t ph[4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float p0 = exp2_raw(sv[4 * hb + 0] - m), p1 = exp2_raw(sv[4 * hb + 1] - m);
      const float p2 = exp2_raw(sv[4 * hb + 2] - m), p3 = exp2_raw(sv[4 * hb + 3] - m);
      ps += (p0 + p1) + (p2 + p3);
      ph[2 * hb] = (uint32_t)float_to_half_bits(p0) | ((uint32_t)float_to_half_bits(p1) << 16);
      ph[2 * hb + 1] = (uint32_t)float_to_half_bits(p2) | ((uint32_t)float_to_half_bits(p3) << 16);
    }
    lsum += ps;
    uint16_t* pr = p_lds + (l16 & 7u) * 64 + row0;
    *reinterpret_cast<uint2*>(pr) = make_uint2(ph[0], ph[1]);
    *reinterpret_cast<uint2*>(pr + 16) = make_uint2(ph[2], ph[3]);
  } else {
    float sv[16];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * mb + i] = cs[mb][i] * scale_log2;
    if (partial) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sv[4 * mb + i] = (16 * mb + 4 * (int)grp + i < nvalid) ? sv[4 * mb + i] : ninf;
    }
    float mt = ninf;
#pragma unroll
    for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sv[j]);
    mt = max_xor32(max_xor16(mt));
    if (__ballot(mt > m + kSoftmaxSlack) != 0ull) {
      const float mn = fmaxf(m, mt);
      const float alpha = exp2_raw(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb] *= alpha;
    }
    float ps = 0.f;
    uint32_t ph[8];  // fp16 pairs for p_lds
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const float p0 = exp2_raw(sv[4 * mb + 0] - m), p1 = exp2_raw(sv[4 * mb + 1] - m);
      const float p2 = exp2_raw(sv[4 * mb + 2] - m), p3 = exp2_raw(sv[4 * mb + 3] - m);
      ps += (p0 + p1) + (p2 + p3);
      ph[2 * mb] = (uint32_t)float_to_half_bits(p0) | ((uint32_t)float_to_half_bits(p1) << 16);
      ph[2 * mb + 1] = (uint32_t)float_to_half_bits(p2) | ((uint32_t)float_to_half_bits(p3) << 16);
    }
    lsum += ps;
    if ((int)l16 < G) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        *reinterpret_cast<uint2*>(p_lds + l16 * 64 + 16 * mb + 4 * grp) =
            make_uint2(ph[2 * mb], ph[2 * mb + 1]);
    }
  }
}

// A head's total sum over the whole wave, in the lanes l16 < G.
template <int G>
__device__ __forceinline__ float tile_softmax_sum(float lsum) {
  if constexpr (G <= 4) {
    lsum += row_ror_f<4>(lsum);
    lsum += row_ror_f<8>(lsum);
  } else if constexpr (G == 8) {
    lsum += row_ror_f<8>(lsum);
  }
  return sum_xor32(sum_xor16(lsum));
}

}  // namespace mustafar
