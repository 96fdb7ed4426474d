// Per-token magnitude pruning and bitmap compression (prefill and decode-time
// append).  Sources: [Summary] "Approach" (per-token magnitude pruning of the
// key and value caches into a bitmap-based format), [Abstract] (runtime
// pruning and compression of the tokens produced during decode), [README]
// "Part II" (the token-wise, magnitude-based variant Kt_Mag / Vt_Mag).
//
// One wave owns one 128-channel row (select_row.hpp).
#include "device_common.hpp"
#include "kernels.hpp"
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
      // entry of the tile offsets (T * keep when every row holds keep values)
      uint32_t* toff = (is_v ? a.vtoff : a.ktoff) + unit * ntoff;
      const uint32_t pos = toff[(T + kTile - 1) / kTile];
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

// Channel-wise pruning (the channel-wise direction of the pages' pruning
// variants, [README] "Part II"): in a full 64-row tile each channel keeps its
// keep/2 entries of largest magnitude over the tile's rows, ties to the
// earlier row, so the tile stores 64 * keep values; the rows of a final
// partial tile are pruned per token to keep.
//
// One wave per (tile, unit); grid (tiles, units), units beyond gridDim.y in
// steps of gridDim.y.  The tile is staged in LDS (row stride 260 B: a column
// read by the 64 lanes touches every bank twice).  For a full tile lane t owns
// row t: per channel, a ballot bisection over the 15 key bits finds the
// (keep/2)-th largest key of the column, ties go to the lower lanes (earlier
// rows), and each lane gathers its row's bits of the 128 channel ballots into
// its bitmap words.  The kept values are packed row after row in LDS and
// copied out with consecutive lanes on consecutive halves.  Every earlier tile
// is full, so this tile's values start at 64 * keep * tile.
constexpr int kChanRow = 130;  // staged row: 128 fp16 + 4 B

__global__ __launch_bounds__(kWave) void prune_channel_kernel(PruneArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);            // [64][kChanRow]
  uint16_t* packed = xs + kTile * kChanRow;                      // [64 * keep]
  const uint32_t lane = lane_id();
  const int tile = blockIdx.x;
  const int keep = a.map.keep, kc = keep / 2;
  const int ntoff = a.cap / kTile + 1;
  for (int unit = blockIdx.y; unit < a.units; unit += gridDim.y) {
    const int b = unit / a.H;
    int T = a.seq_lens[b];
    T = T < 0 ? 0 : (T > a.rows_per_unit ? a.rows_per_unit : T);
    uint32_t* toff = a.tile_off + (int64_t)unit * ntoff;
    if (tile == 0 && lane == 0 && T == 0) toff[0] = 0;
    const int t0 = tile * kTile;
    if (t0 >= T) continue;
    const int n = min(kTile, T - t0);
    const uint32_t v0 = (uint32_t)(t0 * keep);  // values before this tile
    uint64_t* bm = a.bitmaps + ((int64_t)unit * a.cap + t0) * 2;
    uint16_t* vals = a.values + (int64_t)unit * a.cap * keep + v0;
    if (lane == 0) {
      toff[tile] = v0;
      if (t0 + n == T) toff[(T + kTile - 1) / kTile] = v0 + (uint32_t)(n * keep);
    }
    // stage the tile's rows (lane t copies row t)
    const uint16_t* src = a.dense + ((int64_t)unit * a.t_stride + t0) * kHeadDim;
    __syncthreads();  // the previous unit's reads of the staging area are done
    if ((int)lane < n) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint4 c = *reinterpret_cast<const uint4*>(src + lane * kHeadDim + 8 * j);
        uint32_t* d = reinterpret_cast<uint32_t*>(xs + lane * kChanRow + 8 * j);
        d[0] = c.x; d[1] = c.y; d[2] = c.z; d[3] = c.w;
      }
    }
    __syncthreads();
    if (n < kTile) {
      // partial tile: per-token rule on each row
      for (int r = 0; r < n; ++r) {
        const uint32_t x0 = xs[r * kChanRow + lane], x1 = xs[r * kChanRow + 64 + lane];
        store_row(select_row(x0, x1, keep), x0, x1, bm + 2 * r, vals + r * keep);
      }
      continue;
    }
    // full tile: channel-wise selection, lane t = row t
    uint64_t w0 = 0, w1 = 0;
    for (int c = 0; c < kHeadDim; ++c) {
      const uint32_t key = xs[lane * kChanRow + c] & 0x7FFFu;
      uint32_t tau = 0;
      for (int bit = 14; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        const int cnt = __popcll(__ballot(key >= cand));
        if (cnt >= kc) tau = cand;
        if (cnt == kc) break;
      }
      const uint64_t gt = __ballot(key > tau), eq = __ballot(key == tau);
      const int need = kc - __popcll(gt);
      const bool kept = key > tau || (key == tau && (int)mbcnt64(eq, 0u) < need);
      const uint64_t bitc = kept ? 1ull : 0ull;
      if (c < 64) w0 |= bitc << c;
      else w1 |= bitc << (c - 64);
    }
    *reinterpret_cast<uint4*>(bm + 2 * lane) =
        make_uint4((uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32));
    // pack the row's kept values (ascending channel) after the earlier rows'
    const uint32_t pc = (uint32_t)(__popcll(w0) + __popcll(w1));
    uint32_t pos = wave_excl_scan(pc);
    const int most = (int)wave_uniform(wave_max_u32(pc));
    uint64_t cur = w0;
    uint32_t cbase = 0;
    for (int i = 0; i < most; ++i) {
      if (cur == 0ull && cbase == 0u) {
        cur = w1;
        cbase = 64u;
      }
      if (cur != 0ull) {
        const uint32_t c = cbase + (uint32_t)__builtin_ctzll(cur);
        cur &= cur - 1ull;
        packed[pos++] = xs[lane * kChanRow + c];
      }
    }
    __syncthreads();
    for (int i = (int)lane; i < kTile * keep; i += kWave) vals[i] = packed[i];
  }
}

}  // namespace

hipError_t launch_prune_compress_channel(const mustafar_kv_t& d, const KeepMap& map,
                                         const uint16_t* dense, int64_t t_stride,
                                         const int32_t* seq_lens, hipStream_t stream) {
  const int64_t rows_per_unit = t_stride < d.capacity ? t_stride : d.capacity;
  const int64_t units = (int64_t)d.batch * d.num_kv_heads;
  const int64_t tiles = (rows_per_unit + kTile - 1) / kTile;
  if (units <= 0 || tiles <= 0) return hipSuccess;
  const unsigned gy = (unsigned)(units < 65535 ? units : 65535);
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
  const int lds = (kTile * kChanRow + kTile * d.keep) * 2;
  hipLaunchKernelGGL(prune_channel_kernel, dim3((unsigned)tiles, gy), dim3(kWave), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_prune_compress(const mustafar_kv_t& d, const KeepMap& map, const uint16_t* dense,
                                 int64_t t_stride, const int32_t* seq_lens, hipStream_t stream,
                                 bool two_four) {
  const int64_t rows_per_unit = t_stride < d.capacity ? t_stride : d.capacity;
  const int64_t units = (int64_t)d.batch * d.num_kv_heads;
  const int64_t tiles = (rows_per_unit + kTile - 1) / kTile;
  if (units <= 0 || tiles <= 0) return hipSuccess;
  const unsigned gy = (unsigned)(units < 65535 ? units : 65535);
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
  if (two_four)
    hipLaunchKernelGGL(prune_compress_kernel<true>, dim3((unsigned)tiles, gy), dim3(kPruneBlock), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(prune_compress_kernel<false>, dim3((unsigned)tiles, gy), dim3(kPruneBlock), 0,
                       stream, a);
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
