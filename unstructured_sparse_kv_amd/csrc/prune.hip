// Per-token magnitude pruning and bitmap compression (prefill and decode-time
// append).  Sources: [Summary] "Approach" (per-token magnitude pruning of the
// key and value caches into a bitmap-based format), [Abstract] (runtime
// pruning and compression of the tokens produced during decode), [README]
// "Part II" (the token-wise, magnitude-based variant Kt_Mag / Vt_Mag).
//
// One wave owns one 128-channel row: lane l holds channels l and l + 64, so
// "channel order" is "register 0 lanes, then register 1 lanes", which is the
// order ballot and mbcnt count in.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mustafar {
namespace {

struct RowMask {
  uint64_t w0, w1;  // kept channels 0..63 and 64..127
};

// Survivors of one row: the `keep` largest magnitude keys (bits & 0x7FFF; finite
// fp16 magnitudes order like these integers, and -0 == +0), ties to the lower
// channel.  tau is found by an MSB-first bisection over the 15 key bits: the
// largest value with #(key >= tau) >= keep, i.e. the keep-th largest key.  The
// loop stops early once exactly `keep` keys are >= the candidate.
__device__ __forceinline__ RowMask select_row(uint32_t x0, uint32_t x1, int keep) {
  const uint32_t k0 = x0 & 0x7FFFu, k1 = x1 & 0x7FFFu;
  uint32_t tau = 0;
#pragma unroll
  for (int b = 14; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    const int cnt = __popcll(__ballot(k0 >= cand)) + __popcll(__ballot(k1 >= cand));
    if (cnt >= keep) tau = cand;
    if (cnt == keep) break;
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
      uint64_t* bm = (is_v ? vbm : kbm) + (unit * cap + T) * 2;
      uint16_t* vals = (is_v ? vval : kval) + unit * (int64_t)cap * keep + (int64_t)T * keep;
      store_row(m, x0, x1, bm, vals);
      if (lane == 0) {
        uint32_t* toff = (is_v ? vtoff : ktoff) + unit * ntoff;
        if (T % kTile == 0) toff[T / kTile] = (uint32_t)((int64_t)T * keep);
        toff[(T + kTile) / kTile] = (uint32_t)((int64_t)(T + 1) * keep);
      }
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
