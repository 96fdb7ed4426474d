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
// of gridDim.y.  Row indices stay 32-bit within a unit.
__global__ __launch_bounds__(kPruneBlock) void prune_compress_kernel(
    const uint16_t* __restrict__ dense, int64_t t_stride, const int32_t* __restrict__ seq_lens,
    int32_t H, int32_t keep, int32_t cap, int32_t rows_per_unit, int32_t units,
    uint64_t* __restrict__ bitmaps, uint16_t* __restrict__ values,
    uint32_t* __restrict__ tile_off) {
  const uint32_t lane = lane_id();
  const int wave = wave_uniform((int)(threadIdx.x / kWave));
  const int tile = blockIdx.x;
  const int ntoff = cap / kTile + 1;
  for (int unit = blockIdx.y; unit < units; unit += gridDim.y) {
    int T = seq_lens[unit / H];
    T = T < 0 ? 0 : (T > rows_per_unit ? rows_per_unit : T);
    uint32_t* toff = tile_off + (int64_t)unit * ntoff;
    if (tile == 0 && wave == 0 && lane == 0 && T == 0) toff[0] = 0;
    const int t0 = tile * kTile + wave * kRowsPerWave;
    const int tend = min(t0 + kRowsPerWave, T);
    if (t0 >= tend) continue;
    const uint16_t* src = dense + ((int64_t)unit * t_stride + t0) * kHeadDim;
    uint64_t* bm = bitmaps + ((int64_t)unit * cap + t0) * 2;
    uint16_t* vals = values + (int64_t)unit * cap * keep + (int64_t)t0 * keep;
    uint32_t x0 = src[lane], x1 = src[lane + 64];
    for (int t = t0; t < tend; ++t) {
      // next row's loads (the last row reloads itself)
      const int64_t step = (t + 1 < tend) ? kHeadDim : 0;
      const uint32_t y0 = src[step + lane], y1 = src[step + lane + 64];
      const RowMask m = select_row(x0, x1, keep);
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
__global__ __launch_bounds__(1024) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    int32_t* __restrict__ seq_lens, uint32_t* __restrict__ status, int32_t H, int32_t cap,
    int32_t keep_k, uint64_t* __restrict__ kbm, uint16_t* __restrict__ kval,
    uint32_t* __restrict__ ktoff, int32_t keep_v, uint64_t* __restrict__ vbm,
    uint16_t* __restrict__ vval, uint32_t* __restrict__ vtoff) {
  const int b = blockIdx.x;
  const uint32_t lane = lane_id();
  const int wave = wave_uniform((int)(threadIdx.x / kWave)), nw = blockDim.x / kWave;
  int T = seq_lens[b];
  T = T < 0 ? 0 : T;
  const bool full = T >= cap;
  const int64_t ntoff = cap / kTile + 1;
  if (!full) {
    for (int row = wave; row < 2 * H; row += nw) {
      const bool is_v = row >= H;
      const int h = is_v ? row - H : row;
      const int64_t unit = (int64_t)b * H + h;
      const int keep = is_v ? keep_v : keep_k;
      const uint16_t* src = (is_v ? v_new : k_new) + unit * kHeadDim;
      const uint32_t x0 = src[lane], x1 = src[lane + 64];
      const RowMask m = select_row(x0, x1, keep);
      // the new row's values go right after the stored ones: the current end
      // entry of the tile offsets (T * keep when every row holds keep values)
      uint32_t* toff = (is_v ? vtoff : ktoff) + unit * ntoff;
      const uint32_t pos = toff[(T + kTile - 1) / kTile];
      uint64_t* bm = (is_v ? vbm : kbm) + (unit * cap + T) * 2;
      uint16_t* vals = (is_v ? vval : kval) + unit * (int64_t)cap * keep + pos;
      store_row(m, x0, x1, bm, vals);
      if (lane == 0) toff[(T + kTile) / kTile] = pos + (uint32_t)keep;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (full) {
      if (status) atomicOr(status, MUSTAFAR_STATUS_APPEND_FULL);
    } else {
      seq_lens[b] = T + 1;
    }
  }
}

}  // namespace

hipError_t launch_prune_compress(const mustafar_kv_t& d, const uint16_t* dense, int64_t t_stride,
                                 const int32_t* seq_lens, hipStream_t stream) {
  const int64_t rows_per_unit = t_stride < d.capacity ? t_stride : d.capacity;
  const int64_t units = (int64_t)d.batch * d.num_kv_heads;
  const int64_t tiles = (rows_per_unit + kTile - 1) / kTile;
  if (units <= 0 || tiles <= 0) return hipSuccess;
  const unsigned gy = (unsigned)(units < 65535 ? units : 65535);
  hipLaunchKernelGGL(prune_compress_kernel, dim3((unsigned)tiles, gy), dim3(kPruneBlock), 0, stream,
                     dense, t_stride, seq_lens, d.num_kv_heads, d.keep, d.capacity,
                     (int32_t)rows_per_unit, (int32_t)units, d.bitmaps, d.values, d.tile_offsets);
  return hipGetLastError();
}

hipError_t launch_append(const mustafar_kv_t& k, const mustafar_kv_t& v, const uint16_t* k_new,
                         const uint16_t* v_new, int32_t* seq_lens, uint32_t* status,
                         hipStream_t stream) {
  int rows = 2 * k.num_kv_heads;
  int threads = rows * kWave;
  if (threads > 1024) threads = 1024;
  hipLaunchKernelGGL(append_kernel, dim3(k.batch), dim3(threads), 0, stream, k_new, v_new,
                     seq_lens, status, k.num_kv_heads, k.capacity, k.keep, k.bitmaps, k.values,
                     k.tile_offsets, v.keep, v.bitmaps, v.values, v.tile_offsets);
  return hipGetLastError();
}

}  // namespace mustafar
