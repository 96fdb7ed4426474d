// Decode-step attention computed directly over the bitmap-compressed key and
// value caches ([Summary] "Approach": a custom attention kernel over the bitmap
// format; [Abstract]; [README] "Part III": batched sparse attention kernel).
// This is mustafar_decode_attn: the stored entries of each 64-row tile are
// decoded into LDS and the two contractions over the decoded tile run on the
// matrix cores.
//
// Grid (splits, Hkv, B); 4 waves per block; tiles of a (batch, kv head) are
// divided among the splits * 4 waves; the block merges its waves into one
// partial per split and decode_reduce_kernel merges the splits.
//
// Per tile, lane t of a wave owns row t of both caches (bitmaps and kept
// entries in registers, loaded one tile ahead):
//   key tile    walk the key bitmap and write each kept entry into a zeroed
//               row-major fp16 tile K[t][c] in LDS (row stride 264 B).
//   scores      v_mfma_f32_16x16x32_f16: A = 16 tile rows x 32 channels read
//               from LDS, B = the G query heads as columns (registers), 4 row
//               blocks x 4 channel blocks; lane l ends with head l%16 of rows
//               16*mb + 4*(l/16) + i.
//   value tile  walk the value bitmap into a zeroed channel-major tile
//               V[c][t] in the same LDS buffer (row stride 136 B), while the
//               score MFMAs run.
//   softmax     tile_softmax.hpp: per head, online; with G <= 4 the scores
//               are first compacted onto the lanes of the padding heads; the
//               running reference max is raised (and the accumulators
//               rescaled) only when a score exceeds it by more than 8 in log2
//               units, so p <= 2^8; p to LDS as fp16 p[head][row].
//   P.V         v_mfma_f32_16x16x32_f16: A = 16 channels x 32 rows of V,
//               B = p[rows][heads]; accumulators out[channel][head] stay in
//               registers for the whole split (8 channel blocks x 2 row blocks).
// The MFMA operands are read with ds_wrxchg_rtn_b64, which returns the 8 bytes
// and leaves zeros: the operand reads of a tile cover every byte its walk can
// write, so the buffer is clean for the next tile without a clearing pass.
// Lanes past the end of the sequence therefore write zeros (into their own row
// or column), never data outside the operand area.  The strides are the ones
// at which a tile side's scatter and read-and-clear together cost the LDS
// least (measured: 264 B against 272 B key rows, 475 against 552 cycles per
// compute unit and wave-tile side; 136 B against 144 B value rows, 469 against
// 531): at the 16-byte-aligned strides the 8-byte exchanges meet bank conflicts
// that these 8-byte-aligned ones avoid.
#pragma once

#include "decode_walk.hpp"
#include "device_common.hpp"
#include "kernels.hpp"
#include "merge.hpp"
#include "tile_softmax.hpp"
#include "select_row.hpp"

#include <type_traits>

namespace mustafar {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kKRow = 264;  // key tile row: 128 fp16 + 8 B (the general walk's dump slot)
constexpr uint32_t kVRow = 136;  // value tile channel row: 64 fp16 + 8 B
// value tile + the general walk's dump row (channel 128), rounded up to 16 B;
// the key tile (64 x 264) fits too
constexpr int kTileBytes = (129 * kVRow + 15) / 16 * 16;
static_assert(64 * kKRow <= kTileBytes, "the key tile shares the value tile's buffer");


template <int G, int KW>
struct MfmaCfg {
  static constexpr int kPBytes = (G + 1) * 128;  // p[head][64] fp16; head row G stays zero
  // fused decode step: the new key and value rows, packed (bitmap words, then
  // the row registers' worth of values, zero past keep)
  static constexpr int kNewSide = 16 + 4 * KW;
  static constexpr int kNewBytes = 2 * kNewSide;
  static constexpr int kWaveBytes = (kTileBytes + kPBytes + kNewBytes + 15) / 16 * 16;
  static constexpr int kMergeBytes = kDecodeWaves * G * (2 + kHeadDim) * 4;
  static constexpr int kLdsBytes =
      kDecodeWaves * kWaveBytes > kMergeBytes ? kDecodeWaves * kWaveBytes : kMergeBytes;
};

// Fused decode step: one wave prunes the new row of one side (lane l holds
// channels l and l + 64 of `src`), stores it as row T of the compressed cache
// (values right after the stored ones, at the tile offsets' end entry, which
// then advances by keep) and keeps a packed copy at `copy` in LDS for the lane
// that owns the row in the tile walk.
// An empty sequence starts at value 0 whatever the offsets hold; an end entry
// that would put the row outside the unit's value region is not followed (the
// row is not stored, the status says so, the wave still attends over it).
template <int KW>
__device__ __forceinline__ void append_row(const uint16_t* src, int keep, int cap, uint64_t* bm_unit,
                                           uint16_t* val_unit, uint32_t* toff_unit, int T,
                                           char* copy, uint32_t* status) {
  const uint32_t lane = lane_id();
  constexpr int kChunks = (16 + 4 * KW) / 16;
  if (lane < (uint32_t)kChunks) *reinterpret_cast<uint4*>(copy + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t x0 = src[lane], x1 = src[lane + 64];
  const RowMask m = select_row(x0, x1, keep);
  const uint32_t pos = T == 0 ? 0u : wave_uniform(toff_unit[(T + kTile - 1) / kTile]);
  if (append_fits(pos, keep, cap)) {
    if (T == 0 && lane == 0) toff_unit[0] = 0;
    store_row(m, x0, x1, bm_unit + (int64_t)T * 2, val_unit + pos);
    if (lane == 0) toff_unit[(T + kTile) / kTile] = pos + (uint32_t)keep;
  } else if (lane == 0 && status) {
    atomicOr(status, MUSTAFAR_STATUS_BAD_OFFSETS);
  }
  wave_lds_sync();  // the zeroed copy before the packed row goes in
  store_row(m, x0, x1, reinterpret_cast<uint64_t*>(copy), reinterpret_cast<uint16_t*>(copy + 16));
  wave_lds_sync();
}

// Two waves per SIMD is what the LDS footprint allows.  The 64-value variants
// are held to the matching register budget (256 per lane, accumulation
// registers included), which they would otherwise exceed; the others fit it
// unasked (the hint measurably slows the 38-value variant's schedule), and
// rows of up to 128 values run at one wave per SIMD.
template <int G, int KMAX, int NK>
__global__ __launch_bounds__(kDecodeBlock) __attribute__((amdgpu_waves_per_eu(KMAX == 64 ? 2 : 1)))
void decode_sparse_mfma_kernel(SparseDecodeArgs a) {
  constexpr int NMAX = NK > 0 ? NK : KMAX;
  constexpr int KW = RowCfg<NMAX>::kW;
  using C = MfmaCfg<G, KW>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int unit = b * a.Hkv + h;
  const int wave = wave_uniform((int)(threadIdx.x / kWave));
  const uint32_t lane = lane_id();
  const uint32_t l16 = lane & 15u, grp = lane >> 4;
  int T_old = a.seq_lens[b];
  T_old = T_old < 0 ? 0 : (T_old > a.cap ? a.cap : T_old);
  const bool add = a.k_new != nullptr && T_old < a.cap;  // fused step adds row T_old
  const int T = add ? T_old + 1 : T_old;
  const int ntiles = (T + kTile - 1) / kTile;
  const int ntoff = a.cap / kTile + 1;

  char* tile_lds = smem + wave * C::kWaveBytes;
  uint16_t* p_lds = reinterpret_cast<uint16_t*>(tile_lds + kTileBytes);  // [G + 1][64]
  char* new_lds = tile_lds + kTileBytes + C::kPBytes;                    // new K row, new V row
  if (lane < 8u) *reinterpret_cast<uint4*>(p_lds + G * 64 + 8 * lane) = make_uint4(0u, 0u, 0u, 0u);

  // B operand of the score MFMA: query heads as columns (zero beyond G)
  half8 bq[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if ((int)l16 < G)
      x = *reinterpret_cast<const uint4*>(
          a.q + ((int64_t)b * a.Hq + h * G + l16) * kHeadDim + 32 * kb + 8 * grp);
    bq[kb] = __builtin_bit_cast(half8, x);
  }

  const float ninf = -__builtin_inff();
  float m = ninf, lsum = 0.f;  // softmax state (tile_softmax.hpp)
  floatx4 acc[8];              // out[channel 16*mb + 4*grp + i][head l16]
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int total_waves = a.splits * kDecodeWaves;
  const int wid = s * kDecodeWaves + wave;
  // tiles split as evenly as their count allows: wave w takes [w n / W, (w + 1) n / W),
  // so no wave has more than one tile above the average (a split by the rounded-up
  // average gave 30 of 32 waves 17 tiles of a 513-tile unit, two waves 3 and 0)
  const int tb = (int)((int64_t)wid * ntiles / total_waves);
  const int te = (int)((int64_t)(wid + 1) * ntiles / total_waves);
  const int tpw = te - tb;  // this wave's share

  constexpr uint32_t kKMapAt = offsetof(SparseDecodeArgs, kmap);
  constexpr uint32_t kVMapAt = offsetof(SparseDecodeArgs, vmap);
  const int kk = keep_of(a.kmap, kKMapAt, h), vk = keep_of(a.vmap, kVMapAt, h);
  const int64_t kreg = region_of(a.kmap, kKMapAt, b, h, a.cap);
  const int64_t vreg = region_of(a.vmap, kVMapAt, b, h, a.cap);
  const auto krs = make_rsrc(a.kval + kreg, (uint32_t)a.cap * kk * 2u);
  const auto vrs = make_rsrc(a.vval + vreg, (uint32_t)a.cap * vk * 2u);
  const auto kbrs = make_rsrc(a.kbm + (int64_t)unit * a.cap * 2, (uint32_t)a.cap * 16u);
  const auto vbrs = make_rsrc(a.vbm + (int64_t)unit * a.cap * 2, (uint32_t)a.cap * 16u);
  const auto ktrs = make_rsrc(a.ktoff + (int64_t)unit * ntoff, (uint32_t)ntoff * 4u);
  const auto vtrs = make_rsrc(a.vtoff + (int64_t)unit * ntoff, (uint32_t)ntoff * 4u);
  // chunks of each row's prefetch: a constant, so that no branch separates
  // the loads (without an exact keep, the whole register budget: the extra
  // bytes are the next rows' and hit the cache; a count taken from the keep
  // at run time measured slower)
  constexpr int kch = NK > 0 ? row_chunks(NK) : KW / 4;
  constexpr int vch = kch;
  const bool k_odd = (kk & 1) != 0, v_odd = (vk & 1) != 0;

  // fused step: the wave whose tiles include the new row stores it first; the
  // lane that owns the row in the walk then takes it from the LDS copy (its
  // prefetched bytes predate the store)
  const int tile_new = T_old / kTile;
  const bool owner = add && tile_new >= tb && tile_new < te;
  const uint32_t new_lane = (uint32_t)(T_old - tile_new * kTile);
  if (owner) {
    const int64_t ubase = (int64_t)unit * a.cap;
    append_row<KW>(a.k_new + (int64_t)unit * kHeadDim, kk, a.cap,
                   const_cast<uint64_t*>(a.kbm) + ubase * 2, const_cast<uint16_t*>(a.kval) + kreg,
                   const_cast<uint32_t*>(a.ktoff) + (int64_t)unit * ntoff, T_old, new_lds, a.status);
    append_row<KW>(a.v_new + (int64_t)unit * kHeadDim, vk, a.cap,
                   const_cast<uint64_t*>(a.vbm) + ubase * 2, const_cast<uint16_t*>(a.vval) + vreg,
                   const_cast<uint32_t*>(a.vtoff) + (int64_t)unit * ntoff, T_old,
                   new_lds + C::kNewSide, a.status);
  }
  // (only in the owner wave's last tile, which holds the new row: see the loop)
  auto take_new = [&](const char* copy, uint4& bm, uint32_t (&row)[KW]) {
    if (lane == new_lane) {
      bm = *reinterpret_cast<const uint4*>(copy);
#pragma unroll
      for (int j = 0; j < KW; ++j) row[j] = reinterpret_cast<const uint32_t*>(copy + 16)[j];
    }
  };

  // tile offsets of this wave's tiles, 64 at a time, one per lane
  // (tile 0 starts at value 0 by definition: its entry is not read, so a fused
  // step that starts an empty sequence does not read back its own write)
  int toff_base = tb;
  uint32_t ktv = buf_load4(ktrs, (uint32_t)(tb + lane) * 4u);
  uint32_t vtv = buf_load4(vtrs, (uint32_t)(tb + lane) * 4u);
  if (tb == 0 && lane == 0) ktv = vtv = 0u;
  auto offsets = [&](int tile, uint32_t& kt0, uint32_t& vt0) {
    if (tile - toff_base >= kWave) {
      toff_base = tile;
      ktv = buf_load4(ktrs, (uint32_t)(tile + lane) * 4u);
      vtv = buf_load4(vtrs, (uint32_t)(tile + lane) * 4u);
    }
    kt0 = __builtin_amdgcn_readlane(ktv, tile - toff_base);
    vt0 = __builtin_amdgcn_readlane(vtv, tile - toff_base);
  };

  // One register set per side, refilled for the next tile (the last tile
  // reloads itself, so the loads need no condition) as soon as the current
  // tile's walk over it is done.  With an even exact keep every row start is
  // even unless the caches break the format; such a start sends the tile to
  // the general path, so the fast loads skip the realignment.
  constexpr bool kEvenExact = NK > 0 && NK % 2 == 0;
  uint4 kb, vb;
  uint32_t krow[KW], vrow[KW];
  uint32_t kt0 = 0, vt0 = 0, kt0n = 0, vt0n = 0;
  // (rows starting at an odd value are realigned when their tile is walked)
  auto issue_k = [&](int tile, uint32_t t0) {
    kb = buf_load16(kbrs, ((uint32_t)(tile * kTile) + lane) * 16u);
    load_row_raw<KW>(krs, t0 + lane * (uint32_t)kk, kch, krow);
  };
  auto issue_v = [&](int tile, uint32_t t0) {
    vb = buf_load16(vbrs, ((uint32_t)(tile * kTile) + lane) * 16u);
    load_row_raw<KW>(vrs, t0 + lane * (uint32_t)vk, vch, vrow);
  };
  // The first tile's rows are requested at once, from where every cache the
  // library writes puts them (each earlier row holds exactly its head's
  // keep), instead of after the stored offsets arrive: a second dependent
  // memory round trip at kernel start.  A stored offset that differs (checked
  // once the buffer is clear) requests them again.  The requests are not
  // conditional (a wave without tiles reads in-range bytes or gets zeros from
  // the range check), so that waiting for the offsets does not also wait for
  // the rows.
  kt0 = (uint32_t)(tb * kTile) * (uint32_t)kk;
  vt0 = (uint32_t)(tb * kTile) * (uint32_t)vk;
  issue_k(tb, kt0);
  issue_v(tb, vt0);
  const uint32_t tile_base = (uint32_t)(tile_lds - smem);
  // the buffer starts clean; afterwards the operand reads clear it
  static_assert(kTileBytes % 16 == 0, "tile buffer cleared in 16-byte stores");
  constexpr int kClearFull = kTileBytes / (16 * kWave) * (16 * kWave);
#pragma unroll
  for (int o = 0; o < kClearFull; o += 16 * kWave)
    *reinterpret_cast<uint4*>(tile_lds + o + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
  if (kClearFull + 16 * (int)lane < kTileBytes)
    *reinterpret_cast<uint4*>(tile_lds + kClearFull + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
  wave_lds_sync();
  if (tb < te) {
    uint32_t kts, vts;
    offsets(tb, kts, vts);
    if (kts != kt0 || vts != vt0) {
      kt0 = kts;
      vt0 = vts;
      issue_k(tb, kt0);
      issue_v(tb, vt0);
    }
  }
  // An MFMA operand (16 bytes) read and cleared.
  auto take16 = [&](const char* p) {
    uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<char*>(p));
    const uint64_t lo = __hip_atomic_exchange(q, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    const uint64_t hi = __hip_atomic_exchange(q + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
  };
  auto scatter = [&](uint32_t addr, uint32_t vbits) {
    *reinterpret_cast<uint16_t*>(smem + addr) = (uint16_t)vbits;
  };

  // One tile.  Only the unit's last tile may end before its 64th row (TAIL);
  // PATCH (the owner wave's last tile) takes the new rows from LDS.
  auto do_tile = [&](int tile, auto patch_tag, auto tail_tag) {
    constexpr bool PATCH = decltype(patch_tag)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int nvalid = TAIL ? min(kTile, T - tile * kTile) : kTile;
    const bool valid = TAIL ? (int)lane < nvalid : true;
    const bool partial = TAIL && nvalid < kTile;
    const int nxt = min(tile + 1, te - 1);
    offsets(nxt, kt0n, vt0n);

    // ---- key tile K[t][c]
    wave_lds_sync();  // the previous tile's reads (and clears) of the buffer are done
    if (!kEvenExact && (k_odd || (kt0 & 1u))) realign_row<KW>(kt0 + lane * (uint32_t)kk, krow);
    if constexpr (PATCH) take_new(new_lds, kb, krow);
    decode_side<NMAX, NK, false, 2u>(krs, kt0, kk, valid, partial, !kEvenExact || !(kt0 & 1u), kb,
                                     krow, tile_base + lane * kKRow, 0u, scatter,
                                     [&](uint32_t (&r)[KW]) {
                                       if constexpr (PATCH) { uint4 t; take_new(new_lds, t, r); }
                                     });
    issue_k(nxt, kt0n);
    wave_lds_sync();

    // ---- scores: 4 row blocks x 4 channel blocks
    floatx4 cs[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      cs[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
      const char* rowp = tile_lds + (16 * mb + l16) * kKRow + 16 * grp;
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        const uint4 x = take16(rowp + 64 * kb4);
        cs[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, x), bq[kb4],
                                                        cs[mb], 0, 0, 0);
      }
    }

    // ---- value tile V[c][t] in the same buffer, walked while the score MFMAs
    // run: a wave's LDS operations execute in order, so its stores land after
    // the score operand reads (which cleared the buffer); only the compiler
    // must keep the order
    wave_lds_sync();
    if (!kEvenExact && (v_odd || (vt0 & 1u))) realign_row<KW>(vt0 + lane * (uint32_t)vk, vrow);
    if constexpr (PATCH) take_new(new_lds + C::kNewSide, vb, vrow);
    decode_side<NMAX, NK, false, kVRow>(
        vrs, vt0, vk, valid, partial, !kEvenExact || !(vt0 & 1u), vb, vrow, tile_base + 2u * lane,
        0u, scatter, [&](uint32_t (&r)[KW]) {
          if constexpr (PATCH) { uint4 t; take_new(new_lds + C::kNewSide, t, r); }
        });
    issue_v(nxt, vt0n);

    // ---- online softmax (tile_softmax.hpp); p to LDS
    tile_softmax<G>(cs, a.scale_log2, partial, nvalid, l16, grp, m, lsum, acc, p_lds);
    wave_lds_sync();  // p and the value tile written

    // ---- P.V: 8 channel blocks x 2 row blocks
    const uint16_t* prow = p_lds + (l16 < (uint32_t)G ? l16 : (uint32_t)G) * 64 + 8 * grp;
    const half8 pb0 = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(prow));
    const half8 pb1 = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(prow + 32));
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const char* vrowp = tile_lds + (16 * mb + l16) * kVRow + 16 * grp;
      const uint4 x0 = take16(vrowp);
      const uint4 x1 = take16(vrowp + 64);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, x0), pb0, acc[mb],
                                                       0, 0, 0);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, x1), pb1, acc[mb],
                                                       0, 0, 0);
    }
    kt0 = kt0n;
    vt0 = vt0n;
  };
  // The unit's last tile (which holds a fused step's new row, tile_new ==
  // te - 1 in the owner wave) runs on its own; the others need neither the
  // tail masks nor the patch.
  const bool has_last = tb < te && te == ntiles;
  const int te_plain = has_last ? te - 1 : te;
  for (int tile = tb; tile < te_plain; ++tile) {
    set_priority_by_tiles_left(te - tile, tpw);
    do_tile(tile, std::false_type{}, std::false_type{});
  }
  if (has_last) {
    set_priority_by_tiles_left(1, tpw);
    if (owner)
      do_tile(te - 1, std::true_type{}, std::true_type{});
    else
      do_tile(te - 1, std::false_type{}, std::true_type{});
  }

  lsum = tile_softmax_sum<G>(lsum);
  __syncthreads();  // the merge area overlaps the per-wave buffers
  float* lds_m = reinterpret_cast<float*>(smem);
  float* lds_l = lds_m + kDecodeWaves * G;
  float* lds_acc = lds_l + kDecodeWaves * G;
  if ((int)l16 < G) {
    if (grp == 0u) {
      lds_m[wave * G + l16] = m;
      lds_l[wave * G + l16] = lsum;
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lds_acc[(wave * G + l16) * kHeadDim + 16 * mb + 4 * grp + i] = acc[mb][i];
  }
  __syncthreads();
  store_split_partial<G>(lds_m, lds_l, lds_acc, G * kHeadDim, kHeadDim, unit, a.splits, s, a.part);
}

template <int G, int KMAX, int NK>
hipError_t launch_mfma_t(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  constexpr int lds = MfmaCfg<G, RowCfg<(NK > 0 ? NK : KMAX)>::kW>::kLdsBytes;
  if constexpr (lds > 65536) {
    hipError_t e = ensure_lds_limit<&decode_sparse_mfma_kernel<G, KMAX, NK>>(lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_sparse_mfma_kernel<G, KMAX, NK>), dim3(a.splits, a.Hkv, batch),
                     dim3(kDecodeBlock), lds, stream, a);
  return hipGetLastError();
}

// Straight-line walks when every head keeps the same number of values and it
// is that of one of the sparsities 50, 60, 65, 70, 75 or 80% at head_dim 128
// (keep 64, 51, 45, 38, 32, 26); bucketed walks for any other keep and for
// per-head keeps.
template <int G>
hipError_t launch_mfma_g(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  const bool uniform = !a.kmap.per_head && !a.vmap.per_head;
  if (uniform && a.kk == a.vk) {
    switch (a.kk) {
      case 26: return launch_mfma_t<G, 32, 26>(a, batch, stream);
      case 32: return launch_mfma_t<G, 32, 32>(a, batch, stream);
      case 38: return launch_mfma_t<G, 40, 38>(a, batch, stream);
      case 45: return launch_mfma_t<G, 48, 45>(a, batch, stream);
      case 51: return launch_mfma_t<G, 64, 51>(a, batch, stream);
      case 64: return launch_mfma_t<G, 64, 64>(a, batch, stream);
      default: break;
    }
  }
  const int kmax = a.kk > a.vk ? a.kk : a.vk;
  if (kmax <= 32) return launch_mfma_t<G, 32, 0>(a, batch, stream);
  if (kmax <= 48) return launch_mfma_t<G, 48, 0>(a, batch, stream);
  if (kmax <= 64) return launch_mfma_t<G, 64, 0>(a, batch, stream);
  return launch_mfma_t<G, 128, 0>(a, batch, stream);
}

}  // namespace
}  // namespace mustafar
