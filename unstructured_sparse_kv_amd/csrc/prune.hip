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
// tile * 64 + 16w .. + 15 of its (batch, kv head) unit, one row at a time with
// the next row's loads in flight.  Units beyond gridDim.y are taken in steps
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
    uint32_t x0 = src[lane], x1 = src[lane + 64];
    for (int t = t0; t < tend; ++t) {
      // next row's loads (the last row reloads itself)
      const int64_t step = (t + 1 < tend) ? kHeadDim : 0;
      const uint32_t y0 = src[step + lane], y1 = src[step + lane + 64];
      const RowMask m = TWO_FOUR ? select_row_24(x0, x1) : select_row(x0, x1, keep);
      store_row(m, x0, x1, bm, vals);
      if (lane == 0) {
        if (t % kTile == 0) toff[t / kTile] = (uint32_t)(t * keep);
        if (t == T - 1) toff[(T + kTile - 1) / kTile] = (uint32_t)(T * keep);
      }
      src += step;
      bm += 2;
      vals += keep;
      x0 = y0;
      x1 = y1;
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

}  // namespace

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
