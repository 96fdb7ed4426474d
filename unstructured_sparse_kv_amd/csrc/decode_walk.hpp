// Shared pieces of the sparse decode kernels: loading a tile's rows into
// registers and walking a row's bitmap set bit by set bit.
#pragma once

#include "device_common.hpp"

namespace mustafar {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <int KMAX>
struct RowCfg {
  static constexpr int kChunks = (KMAX / 2 + 1 + 3) / 4;  // 16 B chunks per row (+1 dword for realign)
  static constexpr int kW = kChunks * 4;                   // dwords of a row in registers
};

// q[c][g] for the G heads of the group, from the LDS table q[c][g] at byte
// address `addr` = table + c * 2G.
template <int G>
__device__ __forceinline__ void load_q(const char* addr, uint32_t (&qh)[G]) {
  if constexpr (G == 1) {
    qh[0] = *reinterpret_cast<const uint16_t*>(addr);
  } else if constexpr (G == 2) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(addr);
    qh[0] = x & 0xFFFFu;
    qh[1] = x >> 16;
  } else if constexpr (G == 4) {
    const uint2 x = *reinterpret_cast<const uint2*>(addr);
    qh[0] = x.x & 0xFFFFu; qh[1] = x.x >> 16; qh[2] = x.y & 0xFFFFu; qh[3] = x.y >> 16;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(addr);
    qh[0] = x.x & 0xFFFFu; qh[1] = x.x >> 16; qh[2] = x.y & 0xFFFFu; qh[3] = x.y >> 16;
    qh[4] = x.z & 0xFFFFu; qh[5] = x.z >> 16; qh[6] = x.w & 0xFFFFu; qh[7] = x.w >> 16;
  }
}

template <int KW>
__device__ __forceinline__ uint32_t value_at(const uint32_t (&row)[KW], int i) {
  const uint32_t w = row[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Walks over the set bits of a row.  For the n-th set bit (channel c) the
// callback gets f(base + c * MUL, stored value n): callers pass the address of
// channel 0 in their own table as `base` and the byte stride of a channel as
// MUL (a shift or one v_mad_u32_u24).
//
// Fast walk: every valid row holds exactly n set bits and all four bitmap
// dwords are non-zero (invalid lanes carry all-ones words and zero values), so
// the next dword is never empty and no lane runs out before the last step.
// With EXACT the count is the compile-time NMAX and the walk is straight-line
// code the compiler can software-pipeline.  Otherwise the count n (uniform
// across the wave) is taken in chunks of 8 steps: a chunk that n covers
// entirely is straight-line code too, and only the chunk holding the end of
// the row tests each step (rows of up to 64 values; longer ones test every
// step).
template <int NMAX, bool EXACT, uint32_t MUL, int KW, class F>
__device__ __forceinline__ void walk_fast(const uint32_t (&row)[KW], uint4 w, int n, uint32_t base,
                                          F&& f) {
  uint32_t cur = w.x, n1 = w.y, n2 = w.z, n3 = w.w;
  auto step = [&](int i) {
    f(base + (uint32_t)__builtin_ctz(cur) * MUL, value_at(row, i));
    cur &= cur - 1u;
    const bool z = (cur == 0u);
    cur = z ? n1 : cur;
    n1 = z ? n2 : n1;
    n2 = z ? n3 : n2;
    base += z ? 32u * MUL : 0u;
  };
  if constexpr (EXACT) {
#pragma unroll
    for (int i = 0; i < NMAX; ++i) step(i);
  } else if constexpr (NMAX > 64) {  // long rows: chunked code would spill registers
#pragma unroll
    for (int i = 0; i < NMAX; ++i)
      if (i < n) step(i);
  } else {
    constexpr int kChunk = 8;
#pragma unroll
    for (int i0 = 0; i0 < NMAX; i0 += kChunk) {
      if (i0 >= n) break;
      if (i0 + kChunk <= n) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
          if (i0 + j < NMAX) step(i0 + j);
      } else {
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
          if (i0 + j < NMAX && i0 + j < n) step(i0 + j);
      }
    }
  }
}

// General walk: empty dwords are compacted away (each kept dword carries its
// channel base) and a lane that has used all its set bits reports channel 128
// (the zero q entry / the dump row); its remaining values are zero.  The walk
// state survives between calls of run(), so a row with more set bits than the
// value registers hold is walked in rounds, the registers reloaded between
// them.
template <uint32_t MUL>
struct GeneralWalk {
  uint32_t cur, b0, n1, b1, n2, b2, n3, b3, dump;
  __device__ __forceinline__ GeneralWalk(uint4 w, uint32_t base) {
    dump = base + 128u * MUL;
    uint32_t cw[4] = {w.x, w.y, w.z, w.w};
    uint32_t cb[4] = {base, base + 32u * MUL, base + 64u * MUL, base + 96u * MUL};
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const bool sw = (cw[j] == 0u) && (cw[j + 1] != 0u);
        const uint32_t a = cw[j], ab = cb[j];
        cw[j] = sw ? cw[j + 1] : cw[j];
        cb[j] = sw ? cb[j + 1] : cb[j];
        cw[j + 1] = sw ? a : cw[j + 1];
        cb[j + 1] = sw ? ab : cb[j + 1];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) cb[j] = cw[j] ? cb[j] : dump;
    cur = cw[0]; b0 = cb[0]; n1 = cw[1]; b1 = cb[1]; n2 = cw[2]; b2 = cb[2]; n3 = cw[3]; b3 = cb[3];
  }
  // The next `iters` set bits (uniform across the wave), paired with values
  // 0 .. iters-1 of `row`.  Values past a lane's own count must be zero in
  // `row` (the callers mask them): the walk then runs in chunks of 8 steps with
  // no test per step, since a step past every lane's last set bit stores that
  // zero at the dump slot.  (Per-step tests cost 12-16% on channel-wise caches,
  // where every tile takes this walk.)
  template <int NMAX, int KW, class F>
  __device__ __forceinline__ void run(const uint32_t (&row)[KW], int iters, F&& f) {
    auto step = [&](int i) {
      f(cur ? b0 + (uint32_t)__builtin_ctz(cur) * MUL : dump, value_at(row, i));
      cur &= cur - 1u;
      const bool z = (cur == 0u);
      cur = z ? n1 : cur; b0 = z ? b1 : b0;
      n1 = z ? n2 : n1; b1 = z ? b2 : b1;
      n2 = z ? n3 : n2; b2 = z ? b3 : b2;
      n3 = z ? 0u : n3; b3 = z ? dump : b3;
    };
    constexpr int kChunk = 8;
#pragma unroll
    for (int i0 = 0; i0 < NMAX; i0 += kChunk) {
      if (i0 >= iters) break;
#pragma unroll
      for (int j = 0; j < kChunk; ++j)
        if (i0 + j < NMAX) step(i0 + j);
    }
  }
};

// Loads the dwords holding the stored values from half index `start` of the
// region on: row[0] holds values 0 and 1 of the row when start is even, the
// half before it and value 0 when it is odd (realign_row then shifts them).
template <int KW>
__device__ __forceinline__ void load_row_raw(__amdgpu_buffer_rsrc_t rs, uint32_t start, int nchunks,
                                             uint32_t (&row)[KW]) {
  const uint32_t dw0 = start >> 1;
#pragma unroll
  for (int j = 0; j < KW / 4; ++j) {
    uint4 c = make_uint4(0u, 0u, 0u, 0u);
    if (j < nchunks) c = buf_load16(rs, (dw0 + 4u * j) * 4u);
    row[4 * j + 0] = c.x; row[4 * j + 1] = c.y; row[4 * j + 2] = c.z; row[4 * j + 3] = c.w;
  }
}

// Shifts a row loaded from half index `start` so that row[i] holds values 2i
// and 2i + 1.  It reads every loaded register, so a prefetch realigns only when
// its tile is walked: realigning at issue time makes the wave wait for the loads
// there (odd keeps measured 20% slower that way).
template <int KW>
__device__ __forceinline__ void realign_row(uint32_t start, uint32_t (&row)[KW]) {
  const uint32_t sh = (start & 1u) << 4;  // 16 for an odd start, 0 (no change) otherwise
#pragma unroll
  for (int j = 0; j < KW - 1; ++j) row[j] = __builtin_amdgcn_alignbit(row[j + 1], row[j], sh);
}

// load_row_raw, then realign_row when the start may be odd.
template <int KW>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t rs, uint32_t start, int nchunks,
                                         bool odd_possible, uint32_t (&row)[KW]) {
  load_row_raw<KW>(rs, start, nchunks, row);
  if (odd_possible) realign_row<KW>(start, row);
}

// Chunks of 16 B covering n values starting at any half offset (+1 dword slack).
__host__ __device__ constexpr int row_chunks(int n) { return (((n + 1) >> 1) + 1 + 3) >> 2; }

// Zeroes stored values beyond the first `count` of the row.  The masks come
// from sign bits (all ones where the index is below count) rather than from
// compares, which would each hold a scalar register pair.
template <int KW>
__device__ __forceinline__ void mask_row(uint32_t (&row)[KW], uint32_t count) {
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    const uint32_t lo = (uint32_t)((int32_t)(2u * j - count) >> 31);
    const uint32_t hi = (uint32_t)((int32_t)(2u * j + 1u - count) >> 31);
    row[j] &= (lo & 0xFFFFu) | (hi & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint32_t pop4(uint4 w) {
  return __popc(w.x) + __popc(w.y) + __popc(w.z) + __popc(w.w);
}

// Decodes one side (keys or values) of a 64-row tile: for every stored entry of
// the lane's row, f(base + channel * MUL, value bits).
//
// The rows were prefetched into `row` from the start each would have if every
// row held exactly `keep` values (`start_ok`: that load also handled an odd
// start).  When every valid row of the wave has exactly `keep` set bits spread
// over all four bitmap dwords, the fast walk runs on the prefetched registers
// as they are: lanes past the end of the sequence walk an all-ones bitmap and
// either write to `dump` (REDIRECT: a region that absorbs keep * MUL bytes and
// is never read) or have their values zeroed.  Otherwise the rows are reloaded
// from their exact starts (prefix sum of the popcounts) into registers of
// their own and walked by the general walk; lanes past the end walk nothing.
// The prefetched registers are only read here, so the next prefetch can
// overwrite them in place.  `patch` may overwrite rows of the reloaded
// registers (a row whose stored bytes this kernel wrote itself).
struct NoPatch {
  template <int KW>
  __device__ __forceinline__ void operator()(uint32_t (&)[KW]) const {}
};

template <int NMAX, int NK, bool REDIRECT, uint32_t MUL, int KW, class F, class P = NoPatch>
__device__ __forceinline__ void decode_side(__amdgpu_buffer_rsrc_t rs, uint32_t toff, int keep,
                                            bool valid, bool partial, bool start_ok, uint4 bm,
                                            const uint32_t (&row)[KW], uint32_t base,
                                            uint32_t dump, F&& f, P&& patch = P()) {
  const uint32_t pop = pop4(bm);
  const bool lane_fast = !valid || (pop == (uint32_t)keep && bm.x && bm.y && bm.z && bm.w);
  if (start_ok && __ballot(!lane_fast) == 0ull) {
    if (!partial) {
      if constexpr (NK > 0) walk_fast<NK, true, MUL>(row, bm, NK, base, f);
      else walk_fast<NMAX, false, MUL>(row, bm, keep, base, f);
    } else {
      const uint4 ones = make_uint4(~0u, ~0u, ~0u, ~0u);
      const uint4 b = valid ? bm : ones;
      if constexpr (REDIRECT) {
        const uint32_t at = valid ? base : dump;
        if constexpr (NK > 0) walk_fast<NK, true, MUL>(row, b, NK, at, f);
        else walk_fast<NMAX, false, MUL>(row, b, keep, at, f);
      } else {
        uint32_t r[KW];
#pragma unroll
        for (int j = 0; j < KW; ++j) r[j] = valid ? row[j] : 0u;
        if constexpr (NK > 0) walk_fast<NK, true, MUL>(r, b, NK, base, f);
        else walk_fast<NMAX, false, MUL>(r, b, keep, base, f);
      }
    }
    return;
  }
  const uint32_t pc = valid ? pop : 0u;
  const uint32_t st = toff + wave_excl_scan(pc);
  const int iters = (int)wave_uniform(wave_max_u32(pc));
  GeneralWalk<MUL> walk(valid ? bm : make_uint4(0u, 0u, 0u, 0u), base);
  {
    const int n = iters < NMAX ? iters : NMAX;
    uint32_t r[KW];
    load_row<KW>(rs, st, row_chunks(n), true, r);
    mask_row<KW>(r, pc);
    patch(r);
    walk.template run<NMAX>(r, n, f);
  }
  // further rounds of at most NMAX values for rows holding more (rows may hold
  // more values than keep, e.g. after channel-wise pruning)
  if (__builtin_expect(iters > NMAX, 0)) {
    for (int done = NMAX; done < iters; done += NMAX) {
      const int n = iters - done < NMAX ? iters - done : NMAX;
      uint32_t r[KW];
      load_row<KW>(rs, st + (uint32_t)done, row_chunks(n), true, r);
      mask_row<KW>(r, pc > (uint32_t)done ? pc - (uint32_t)done : 0u);
      walk.template run<NMAX>(r, n, f);
    }
  }
}

}  // namespace mustafar
