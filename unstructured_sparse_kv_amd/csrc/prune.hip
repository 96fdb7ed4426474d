// Per-token magnitude pruning and bitmap compression (prefill and decode-time
// append).  Sources: [Summary] "Approach" (per-token magnitude pruning of the
// key and value caches into a bitmap-based format), [Abstract] (runtime
// pruning and compression of the tokens produced during decode), [README]
// "Part II" (the token-wise, magnitude-based variant Kt_Mag / Vt_Mag).
//
// One wave owns one 128-channel row (select_row.hpp).
#include "device_common.hpp"
#include "kernels.hpp"
#include "select_lane.hpp"
#include "select_row.hpp"

namespace mustafar {
namespace {

constexpr int kPruneBlock = 256;
constexpr int kWavesPerBlock = kPruneBlock / kWave;
constexpr int kRowsPerWave = kTile / kWavesPerBlock;  // 16

// Grid (64-row tiles, units); wave w of a block prunes rows
// tile * 64 + 16w .. + 15 of its (batch, kv head) unit.  All 16 rows are
// loaded before the first is pruned: a row's selection takes far less time
// than a load's latency, so a wave that waited for each row in turn would
// spend most of its time stalled.  Units beyond gridDim.y are taken in steps
// of gridDim.y.  Row indices stay 32-bit within a unit.  Head h of a unit keeps
// keep_of(map, h) values per row.
// TWO_FOUR: the 2:4 comparator rule instead of the per-token top-keep rule
// (the map then holds keep = 64 for every head).
template <bool TWO_FOUR>
__global__ __launch_bounds__(kPruneBlock) void prune_compress_kernel(PruneArgs a) {
  constexpr uint32_t kMapAt = offsetof(PruneArgs, map);
  const uint32_t lane = lane_id();
  const int wave = wave_uniform((int)(threadIdx.x / kWave));
  const int tile = blockIdx.x;
  const int ntoff = a.cap / kTile + 1;
  for (int unit = blockIdx.y; unit < a.units; unit += gridDim.y) {
    const int b = unit / a.H, h = unit - b * a.H;
    const int keep = keep_of(a.map, kMapAt, h);
    int T = a.seq_lens[b];
    T = T < 0 ? 0 : (T > a.rows_per_unit ? a.rows_per_unit : T);
    uint32_t* toff = a.tile_off + (int64_t)unit * ntoff;
    if (tile == 0 && wave == 0 && lane == 0 && T == 0) toff[0] = 0;
    const int t0 = tile * kTile + wave * kRowsPerWave;
    const int tend = min(t0 + kRowsPerWave, T);
    if (t0 >= tend) continue;
    const uint16_t* src = a.dense + ((int64_t)unit * a.t_stride + t0) * kHeadDim;
    uint64_t* bm = a.bitmaps + ((int64_t)unit * a.cap + t0) * 2;
    uint16_t* vals = a.values + region_of(a.map, kMapAt, b, h, a.cap) + (int64_t)t0 * keep;
    const int n = tend - t0;  // 1 .. 16 rows
    uint32_t x0[kRowsPerWave], x1[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = i < n ? i : n - 1;  // rows past the end load the last one again
      x0[i] = src[r * kHeadDim + lane];
      x1[i] = src[r * kHeadDim + lane + 64];
    }
    // unrolled (each row under a uniform test) so that the rows stay in fixed
    // registers and their addresses are constant offsets
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (i < n) {
        const int t = t0 + i;
        const RowMask m = TWO_FOUR ? select_row_24(x0[i], x1[i]) : select_row(x0[i], x1[i], keep);
        store_row(m, x0[i], x1[i], bm + 2 * i, vals + (int64_t)i * keep);
        if (lane == 0) {
          if (t % kTile == 0) toff[t / kTile] = (uint32_t)(t * keep);
          if (t == T - 1) toff[(T + kTile - 1) / kTile] = (uint32_t)(T * keep);
        }
      }
    }
  }
}

// Per-token pruning with one row per lane (select_lane.hpp).  Each wave takes
// 64-row tiles of the (batch, kv head) units in turn: tile i of the
// unit-major order, then i + the number of waves in the grid, and so on.
//   stage    the tile's 64 dense rows (16 KB, contiguous) arrive as sixteen
//            coalesced 16-byte loads per lane into registers, issued while
//            the wave still works on its previous tile; they are written to
//            this wave's LDS tile (row stride 272 B) and lane t reads row t
//            into registers (16 reads of 16 B; each quarter wave touches 64
//            distinct banks).
//   select   lane_select_row: the row's survivors as a 128-bit mask, with
//            integer arithmetic on the lane's own keys only.
//   bitmaps  lane t stores row t's two words (consecutive lanes, consecutive
//            16 B).
//   pack     lane t walks its mask set bit by set bit and gathers the kept
//            values from its staged row (one 2-byte LDS read per kept value,
//            in channel order), then writes the packed row back to the LDS
//            tile at t * keep values; the tile's packed values (one contiguous
//            run of n * keep values, 16-byte aligned) are copied out with
//            coalesced 16-byte stores.
// The grid holds at most as many blocks as the chip keeps resident (two per
// CU), so that every wave works through several tiles and its loads overlap
// its own arithmetic.
constexpr int kLaneRow = 272;           // staged row: 256 B + 16 B
constexpr int kLaneWaves = 4;
constexpr int kLaneBlock = kLaneWaves * kWave;
constexpr int kLaneTileBytes = kTile * kLaneRow;
constexpr int kLaneBlocksPerCu = 2;     // LDS: 2 x 4 x 17 KB of the CU's 160 KB

// Gathers the values of the set bits of bm (channel order) from the lane's
// staged row at LDS address `row` into p (value 2i in the low half of p[i],
// value 2i + 1 in the high half), `steps` (wave-uniform) of them.  Without
// SPARE, bm holds at least `steps` set bits; with it, a lane whose bits run
// out reads channel 31 of its last word for the remaining steps (values never
// used).
template <bool SPARE>
__device__ __forceinline__ void gather_kept(const uint32_t (&bm)[4], int steps, const char* row,
                                            uint32_t (&p)[64]) {
  // empty words compacted away; each kept word carries the address of its channel 0
  uint32_t cw[4] = {bm[0], bm[1], bm[2], bm[3]};
  const char* cb[4] = {row, row + 64, row + 128, row + 192};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const bool sw = (cw[j] == 0u) && (cw[j + 1] != 0u);
      const uint32_t w = cw[j];
      const char* b = cb[j];
      cw[j] = sw ? cw[j + 1] : cw[j];
      cb[j] = sw ? cb[j + 1] : cb[j];
      cw[j + 1] = sw ? w : cw[j + 1];
      cb[j + 1] = sw ? b : cb[j + 1];
    }
  }
  uint32_t cur = cw[0], n1 = cw[1], n2 = cw[2], n3 = cw[3];
  const char *b0 = cb[0], *b1 = cb[1], *b2 = cb[2], *b3 = cb[3];
  auto step = [&](int i) {
    const uint32_t v = *reinterpret_cast<const uint16_t*>(
        b0 + 2u * (uint32_t)__builtin_ctz(SPARE ? (cur | 0x80000000u) : cur));
    p[i >> 1] = (i & 1) ? (p[i >> 1] | (v << 16)) : v;
    cur &= cur - 1u;
    const bool z = (cur == 0u);
    cur = z ? n1 : cur; b0 = z ? b1 : b0;
    n1 = z ? n2 : n1; b1 = z ? b2 : b1;
    n2 = z ? n3 : n2; b2 = z ? b3 : b2;
    n3 = z ? 0u : n3;
  };
  // (fully unrolled: p is indexed by the step number, so every step must be
  // straight-line code with a constant index)
  constexpr int kChunk = 8;
#pragma clang loop unroll(full)
  for (int i0 = 0; i0 < 128; i0 += kChunk) {
    if (i0 + kChunk <= steps) {
#pragma clang loop unroll(full)
      for (int j = 0; j < kChunk; ++j) step(i0 + j);
    } else if (i0 < steps) {
#pragma clang loop unroll(full)
      for (int j = 0; j < kChunk; ++j)
        if (i0 + j < steps) step(i0 + j);
    }
  }
}

// 64 x 64 bit transpose across the wave: lane l holds row l as the 64-bit
// value (w1:w0); afterwards bit j of lane l is what bit l of lane j was.  The
// usual recursive block swap: at distance d = 32, 16, 8, 4, 2, 1 a lane
// without bit d exchanges the columns with bit d set for its partner's
// (lane l ^ d) columns without it.  For d < 32 each 32-bit word is done on its
// own: the lower lane takes (P << d) in the positions with bit d set, the
// upper one (P >> d) in those without, as a byte permute (d = 16, 8) or a
// rotate and a bit-field insert (d = 4, 2, 1) with per-lane selectors.
__device__ __forceinline__ void wave_transpose64(uint32_t& w0, uint32_t& w1, uint32_t lane) {
  {
    const uint32_t p0 = (uint32_t)__shfl_xor((int)w0, 32, kWave), p1 = (uint32_t)__shfl_xor((int)w1, 32, kWave);
    if (lane & 32u) w0 = p1; else w1 = p0;
  }
  auto bytes = [&](uint32_t& w, int d, uint32_t sel) {
    const uint32_t pw = (uint32_t)__shfl_xor((int)w, d, kWave);
    w = byte_perm(pw, w, sel);
  };
  auto bits = [&](uint32_t& w, int d, uint32_t rot, uint32_t mask) {
    const uint32_t pw = (uint32_t)__shfl_xor((int)w, d, kWave);
    const uint32_t q = __builtin_amdgcn_alignbit(pw, pw, rot);  // rotate right
    w = (q & mask) | (w & ~mask);
  };
  const uint32_t s16 = (lane & 16u) ? 0x03020706u : 0x05040100u;
  const uint32_t s8 = (lane & 8u) ? 0x03070105u : 0x06020400u;
  const uint32_t r4 = (lane & 4u) ? 4u : 28u, m4 = (lane & 4u) ? 0x0F0F0F0Fu : 0xF0F0F0F0u;
  const uint32_t r2 = (lane & 2u) ? 2u : 30u, m2 = (lane & 2u) ? 0x33333333u : 0xCCCCCCCCu;
  const uint32_t r1 = (lane & 1u) ? 1u : 31u, m1 = (lane & 1u) ? 0x55555555u : 0xAAAAAAAAu;
  bytes(w0, 16, s16); bytes(w1, 16, s16);
  bytes(w0, 8, s8);   bytes(w1, 8, s8);
  bits(w0, 4, r4, m4); bits(w1, 4, r4, m4);
  bits(w0, 2, r2, m2); bits(w1, 2, r2, m2);
  bits(w0, 1, r1, m1); bits(w1, 1, r1, m1);
}

// One tile of the flattened unit-major order.  n <= 0: no row of it is inside
// its sequence.
struct LaneTile {
  int unit, b, h, tile, t0, n, T;
};

__device__ __forceinline__ LaneTile lane_tile(const PruneArgs& a, const int32_t* __restrict__ seq_lens,
                                              int item) {
  LaneTile t;
  t.unit = wave_uniform(item / a.tiles_per_unit);
  t.tile = item - t.unit * a.tiles_per_unit;
  t.b = t.unit / a.H;
  t.h = t.unit - t.b * a.H;
  int T = seq_lens[t.b];
  t.T = T < 0 ? 0 : (T > a.rows_per_unit ? a.rows_per_unit : T);
  t.t0 = t.tile * kTile;
  t.n = min(kTile, t.T - t.t0);
  return t;
}

// The 16 KB of tile t's rows, chunk c = 64 j + lane (row c / 16, bytes
// 16 (c % 16)) into r[j]; rows past the tile's n (all of them when n <= 0 or
// when `live` is false) read as zero without touching memory.
__device__ __forceinline__ void lane_fetch(const PruneArgs& a, const LaneTile& t, bool live,
                                           uint32_t lane, uint4 (&r)[16]) {
  const uint32_t rows = live && t.n > 0 ? (uint32_t)t.n : 0u;
  const auto src = make_rsrc(a.dense + ((int64_t)t.unit * a.t_stride + t.t0) * kHeadDim,
                             rows * (uint32_t)(2 * kHeadDim));
#pragma unroll
  for (int j = 0; j < 16; ++j) r[j] = buf_load16(src, 16u * (64u * (uint32_t)j + lane));
}

// seq_lens (a copy of a.seq_lens) as a restrict argument: the kernel never
// writes it, so its loads can go through the scalar unit.
// CHANNEL: the channel-wise rule for full tiles (the map then holds one even
// keep for every head): lane l reads channels 2l, 2l + 1 of the 64 staged rows
// (consecutive lanes, consecutive dwords of a row), lane_select_columns marks
// each channel's keep/2 kept rows, two 64 x 64 transposes across the wave turn
// the two column masks into row masks, and a bit shuffle interleaves them into
// row t's bitmap on lane t.  Rows then hold different numbers of values: each
// row's run starts at the prefix sum of the earlier rows' counts, and the walk
// takes as many steps as the longest row.  A partial tile takes the per-token
// rule.
template <bool CHANNEL>
__global__ __launch_bounds__(kLaneBlock) void prune_lane_kernel(PruneArgs a,
                                                               const int32_t* __restrict__ seq_lens) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr uint32_t kMapAt = offsetof(PruneArgs, map);
  const uint32_t lane = lane_id();
  const int wave = wave_uniform((int)(threadIdx.x / kWave));
  const int nwaves = (int)gridDim.x * kLaneWaves;
  const int ntoff = a.cap / kTile + 1;
  char* const tl = smem + wave * kLaneTileBytes;  // this wave's LDS tile
  int item = (int)blockIdx.x * kLaneWaves + wave;
  if (item >= a.items) return;
  const int share = (a.items - 1 - item) / nwaves + 1;  // this wave's tiles
  LaneTile cur = lane_tile(a, seq_lens, item);
  uint4 r[16];
  lane_fetch(a, cur, true, lane, r);
  for (;;) {
    // r: the rows of tile `item`
    const int next = item + nwaves;
    const bool more = next < a.items;
    set_priority_by_tiles_left((a.items - 1 - item) / nwaves + 1, share);
    uint32_t* toff = a.tile_off + (int64_t)cur.unit * ntoff;
    if (cur.tile == 0 && lane == 0 && cur.T == 0) toff[0] = 0;
    const int keep = keep_of(a.map, kMapAt, cur.h);
    const int n = cur.n, t0 = cur.t0;
    if (n > 0) {
      if (lane == 0) {
        toff[cur.tile] = (uint32_t)(t0 * keep);
        if (t0 + n == cur.T) toff[(cur.T + kTile - 1) / kTile] = (uint32_t)(cur.T * keep);
      }
      // ---- stage (the previous tile's copy-out reads of the LDS tile are
      // done: this wave's LDS operations run in order)
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t c = 64u * (uint32_t)j + lane;
        *reinterpret_cast<uint4*>(tl + (c >> 4) * kLaneRow + 16u * (c & 15u)) = r[j];
      }
    }
    // the next tile's loads, in flight while this one is processed
    const LaneTile nx = lane_tile(a, seq_lens, more ? next : item);
    lane_fetch(a, nx, more, lane, r);
    if (n > 0) {
      wave_lds_sync();
      uint32_t bm[4];
      int steps = keep;       // walk length (wave-uniform)
      uint32_t count = keep;  // this row's kept values
      uint32_t start = lane * (uint32_t)keep;  // its first value in the packed tile
      const bool by_channel = CHANNEL && n == kTile;
      if (by_channel) {
        uint32_t y[64];
#pragma unroll
        for (int r = 0; r < 64; ++r) y[r] = *reinterpret_cast<const uint32_t*>(tl + r * kLaneRow + 4u * lane);
        uint32_t lo[2], hi[2];
        lane_select_columns(y, (uint32_t)keep / 2u, lo, hi);
        wave_transpose64(lo[0], lo[1], lane);
        wave_transpose64(hi[0], hi[1], lane);
        bm[0] = shuffle32(byte_perm(hi[0], lo[0], 0x05040100u));
        bm[1] = shuffle32(byte_perm(hi[0], lo[0], 0x07060302u));
        bm[2] = shuffle32(byte_perm(hi[1], lo[1], 0x05040100u));
        bm[3] = shuffle32(byte_perm(hi[1], lo[1], 0x07060302u));
        count = popc32(bm[0]) + popc32(bm[1]) + popc32(bm[2]) + popc32(bm[3]);
        start = wave_excl_scan(count);
        steps = (int)wave_uniform(wave_max_u32(count));
      } else {
        uint32_t x[64];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint4 v = *reinterpret_cast<const uint4*>(tl + lane * kLaneRow + 16u * (uint32_t)j);
          x[4 * j] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
        }
        // lanes past the end take the lowest `keep` channels (never stored)
        lane_select_row(x, (uint32_t)keep, bm);
        if ((int)lane >= n) {
          bm[0] = bm[1] = bm[2] = bm[3] = ~0u;
          keep_lowest128(bm, (uint32_t)keep);
        }
      }
      if ((int)lane < n)
        *reinterpret_cast<uint4*>(a.bitmaps + ((int64_t)cur.unit * a.cap + t0 + lane) * 2) =
            make_uint4(bm[0], bm[1], bm[2], bm[3]);

      // ---- pack
      uint32_t p[64];  // (zeroed: left undefined, the unrolled walk's paths cost copies)
#pragma unroll
      for (int j = 0; j < 64; ++j) p[j] = 0u;
      gather_kept<CHANNEL>(bm, steps, tl + lane * kLaneRow, p);
      // the packed rows back to back in the same LDS tile (this wave's gathers
      // are done: its LDS operations run in order)
      wave_lds_sync();
      char* const prow = tl + 2u * start;  // packed row `lane`
      constexpr int kChunk = 8;
      if (!by_channel && (keep & 1) == 0) {
        const int nd = keep / 2;
#pragma clang loop unroll(full)
        for (int j0 = 0; j0 < 64; j0 += kChunk) {
          if (j0 + kChunk <= nd) {
#pragma clang loop unroll(full)
            for (int j = j0; j < j0 + kChunk; ++j) *reinterpret_cast<uint32_t*>(prow + 4 * j) = p[j];
          } else if (j0 < nd) {
#pragma clang loop unroll(full)
            for (int j = j0; j < j0 + kChunk; ++j)
              if (j < nd) *reinterpret_cast<uint32_t*>(prow + 4 * j) = p[j];
          }
        }
      } else {
        // rows that start at an odd value: value by value (`count` of them)
#pragma clang loop unroll(full)
        for (int i = 0; i < 128; ++i)
          if (i < steps && (uint32_t)i < count)
            *reinterpret_cast<uint16_t*>(prow + 2 * i) = (uint16_t)((i & 1) ? (p[i >> 1] >> 16) : p[i >> 1]);
      }
      wave_lds_sync();
      // coalesced copy-out of the n * keep values: 16-byte pieces in groups of
      // four (four LDS reads, then four stores: the reads stay inside this
      // wave's tile, the stores past the last whole piece fall outside the
      // buffer range and are dropped), then at most seven single values.  The
      // run starts 16-byte aligned: 64 * keep * 2 bytes per tile, regions of
      // capacity * keep values, capacity a multiple of 64.
      char* dst = reinterpret_cast<char*>(a.values + region_of(a.map, kMapAt, cur.b, cur.h, a.cap) +
                                          (int64_t)t0 * keep);
      const uint32_t bytes = (uint32_t)(n * keep) * 2u;
      const auto out = make_rsrc(dst, bytes & ~15u);
      for (uint32_t c0 = 0; c0 < bytes / 16u; c0 += 4u * kWave) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const uint4*>(tl + 16u * (c0 + 64u * k + lane));
#pragma unroll
        for (int k = 0; k < 4; ++k) buf_store16(out, 16u * (c0 + 64u * k + lane), v[k]);
      }
      const uint32_t tail = (bytes & ~15u) + 2u * lane;
      if (tail < bytes)
        *reinterpret_cast<uint16_t*>(dst + tail) = *reinterpret_cast<const uint16_t*>(tl + tail);
    }
    if (!more) break;
    item = next;
    cur = nx;
  }
}

// One block per batch row: its waves prune the new key and value rows of every
// kv head, then one thread advances seq_lens[b].
__global__ __launch_bounds__(1024) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const uint32_t lane = lane_id();
  const int wave = wave_uniform((int)(threadIdx.x / kWave)), nw = blockDim.x / kWave;
  const int H = a.H, cap = a.cap;
  int T = a.seq_lens[b];
  T = T < 0 ? 0 : T;
  const bool full = T >= cap;
  const int64_t ntoff = cap / kTile + 1;
  if (!full) {
    for (int row = wave; row < 2 * H; row += nw) {
      const bool is_v = row >= H;
      const int h = is_v ? row - H : row;
      const int64_t unit = (int64_t)b * H + h;
      const KeepMap& map = is_v ? a.vmap : a.kmap;
      const uint32_t at = is_v ? offsetof(AppendArgs, vmap) : offsetof(AppendArgs, kmap);
      const int keep = keep_of(map, at, h);
      const uint16_t* src = (is_v ? a.v_new : a.k_new) + unit * kHeadDim;
      const uint32_t x0 = src[lane], x1 = src[lane + 64];
      const RowMask m = select_row(x0, x1, keep);
      // the new row's values go right after the stored ones: the current end
      // entry of the tile offsets (T * keep when every row holds keep values);
      // an empty sequence starts at 0 whatever the offsets hold
      uint32_t* toff = (is_v ? a.vtoff : a.ktoff) + unit * ntoff;
      const uint32_t pos = T == 0 ? 0u : wave_uniform(toff[(T + kTile - 1) / kTile]);
      if (!append_fits(pos, keep, cap)) {
        if (lane == 0 && a.status) atomicOr(a.status, MUSTAFAR_STATUS_BAD_OFFSETS);
        continue;
      }
      if (T == 0 && lane == 0) toff[0] = 0;
      uint64_t* bm = (is_v ? a.vbm : a.kbm) + (unit * cap + T) * 2;
      uint16_t* vals = (is_v ? a.vval : a.kval) + region_of(map, at, b, h, cap) + pos;
      store_row(m, x0, x1, bm, vals);
      if (lane == 0) toff[(T + kTile) / kTile] = pos + (uint32_t)keep;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (full) {
      if (a.status) atomicOr(a.status, MUSTAFAR_STATUS_APPEND_FULL);
    } else {
      a.seq_lens[b] = T + 1;
    }
  }
}

}  // namespace

namespace {

// The per-lane kernel over every 64-row tile of the (batch, head) units.
hipError_t launch_lane(PruneArgs& a, int64_t units, int64_t tiles, bool channel, hipStream_t stream,
                       const int32_t* seq_lens) {
  constexpr int lds = kLaneWaves * kLaneTileBytes;
  hipError_t e = channel ? ensure_lds_limit<&prune_lane_kernel<true>>(lds)
                         : ensure_lds_limit<&prune_lane_kernel<false>>(lds);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = device_cu_count(&cus);
  if (e != hipSuccess) return e;
  const int64_t items = units * tiles;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  a.tiles_per_unit = (int32_t)tiles;
  a.items = (int32_t)items;
  const int64_t want = (items + kLaneWaves - 1) / kLaneWaves;
  const int64_t resident = (int64_t)cus * kLaneBlocksPerCu;
  const dim3 grid((unsigned)(want < resident ? want : resident));
  if (channel)
    hipLaunchKernelGGL(prune_lane_kernel<true>, grid, dim3(kLaneBlock), lds, stream, a, seq_lens);
  else
    hipLaunchKernelGGL(prune_lane_kernel<false>, grid, dim3(kLaneBlock), lds, stream, a, seq_lens);
  return hipGetLastError();
}

PruneArgs prune_args(const mustafar_kv_t& d, const KeepMap& map, const uint16_t* dense,
                     int64_t t_stride, const int32_t* seq_lens, int64_t rows_per_unit, int64_t units) {
  PruneArgs a;
  a.dense = dense;
  a.t_stride = t_stride;
  a.seq_lens = seq_lens;
  a.H = d.num_kv_heads;
  a.cap = d.capacity;
  a.rows_per_unit = (int32_t)rows_per_unit;
  a.units = (int32_t)units;
  a.bitmaps = d.bitmaps;
  a.values = d.values;
  a.tile_off = d.tile_offsets;
  a.map = map;
  a.tiles_per_unit = 0;
  a.items = 0;
  return a;
}

}  // namespace

hipError_t launch_prune_compress_channel(const mustafar_kv_t& d, const KeepMap& map,
                                         const uint16_t* dense, int64_t t_stride,
                                         const int32_t* seq_lens, hipStream_t stream) {
  const int64_t rows_per_unit = t_stride < d.capacity ? t_stride : d.capacity;
  const int64_t units = (int64_t)d.batch * d.num_kv_heads;
  const int64_t tiles = (rows_per_unit + kTile - 1) / kTile;
  if (units <= 0 || tiles <= 0) return hipSuccess;
  PruneArgs a = prune_args(d, map, dense, t_stride, seq_lens, rows_per_unit, units);
  return launch_lane(a, units, tiles, true, stream, seq_lens);
}

hipError_t launch_prune_compress(const mustafar_kv_t& d, const KeepMap& map, const uint16_t* dense,
                                 int64_t t_stride, const int32_t* seq_lens, hipStream_t stream,
                                 bool two_four) {
  const int64_t rows_per_unit = t_stride < d.capacity ? t_stride : d.capacity;
  const int64_t units = (int64_t)d.batch * d.num_kv_heads;
  const int64_t tiles = (rows_per_unit + kTile - 1) / kTile;
  if (units <= 0 || tiles <= 0) return hipSuccess;
  PruneArgs a = prune_args(d, map, dense, t_stride, seq_lens, rows_per_unit, units);
  if (!two_four) return launch_lane(a, units, tiles, false, stream, seq_lens);
  const unsigned gy = (unsigned)(units < 65535 ? units : 65535);
  hipLaunchKernelGGL(prune_compress_kernel<true>, dim3((unsigned)tiles, gy), dim3(kPruneBlock), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_append(const mustafar_kv_t& k, const KeepMap& kmap, const mustafar_kv_t& v,
                         const KeepMap& vmap, const uint16_t* k_new, const uint16_t* v_new,
                         int32_t* seq_lens, uint32_t* status, hipStream_t stream) {
  int rows = 2 * k.num_kv_heads;
  int threads = rows * kWave;
  if (threads > 1024) threads = 1024;
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.seq_lens = seq_lens;
  a.status = status;
  a.H = k.num_kv_heads;
  a.cap = k.capacity;
  a.kbm = k.bitmaps;
  a.kval = k.values;
  a.ktoff = k.tile_offsets;
  a.vbm = v.bitmaps;
  a.vval = v.values;
  a.vtoff = v.tile_offsets;
  a.kmap = kmap;
  a.vmap = vmap;
  hipLaunchKernelGGL(append_kernel, dim3(k.batch), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mustafar
