// Decode-step attention computed directly over the bitmap-compressed key and
// value caches ([Summary] "Approach": a custom attention kernel over the bitmap
// format; [Abstract]; [README] "Part III": batched sparse attention kernel),
// vector-unit-only variant (mustafar_decode_attn_valu).
//
// Grid (splits, Hkv, B); 4 waves per block.  The 64-row tiles of a
// (batch, kv head) are divided among the splits * 4 waves; each wave keeps an
// online-softmax state for the G = Hq/Hkv query heads that read this kv head.
// The block merges its waves into one partial per split; a second kernel
// (decode_reduce_kernel) merges the splits.
//
// Per tile, lane t of a wave owns row t of both caches: its two bitmaps (4
// dwords each) and its kept key and value entries, loaded into registers one
// tile ahead of use.
//   key side    walk the key bitmap set bit by set bit: the n-th set bit is
//               channel c and pairs with stored value n; every q head of the
//               group reuses the decoded element (q[c][g] from LDS).
//   softmax     per q head: wave max, exp2, running sums; p is kept as packed
//               fp16 pairs (p[t], p[t+1]) in LDS.
//   value side  walk the value bitmap the same way and write each stored
//               value into a zero-filled channel-major fp16 tile in LDS
//               (row c holds the 64 rows' entries of channel c); then lane l
//               owns channels l and l+64 and accumulates
//               acc[g][c] += v[c][t] p[g][t] + v[c][t+1] p[g][t+1]
//               with v_dot2_f32_f16 (fp32 accumulation) over the 32 row pairs.
// Every decoded element is touched once per side and no per-row bitmap is
// broadcast across lanes.  No matrix cores: the work is a memory-bound sparse
// matrix-vector product.
#include "device_common.hpp"
#include "kernels.hpp"
#include "merge.hpp"
#include "decode_walk.hpp"

namespace mustafar {
namespace {


constexpr int kTRowShift = 7;     // one channel row of the value tile: 64 fp16 = 128 B
constexpr uint32_t kTRowBytes = 1u << kTRowShift;
constexpr int kTRows = 129;       // 128 channels + a dump row for lanes past their last entry

template <int G>
struct SparseCfg {
  static constexpr int kQBytes = ((129 * 2 * G) + 15) / 16 * 16;  // q[c][g] fp16, c = 128 is zero
  static constexpr uint32_t kQMul = 2 * G;  // bytes per channel of the q table
  static constexpr int kTileBytes = kTRows << kTRowShift;
  // p pairs: 8 blocks of 4 row pairs; block stride (G | 1) * 4 dwords keeps the
  // 8 blocks on distinct banks when lanes read different blocks
  static constexpr int kP2Block = 4 * (G | 1);
  static constexpr int kP2Bytes = 8 * kP2Block * 4;
  static constexpr int kWaveBytes = (kTileBytes + kP2Bytes + 15) / 16 * 16;
  static constexpr int kMergeBytes = kDecodeWaves * G * (2 + kHeadDim) * 4;
  static constexpr int kLdsBytes =
      kQBytes + (kDecodeWaves * kWaveBytes > kMergeBytes ? kDecodeWaves * kWaveBytes : kMergeBytes);
};

// NK > 0: both caches keep exactly NK values per row (straight-line walks);
// NK == 0: any keep up to KMAX.
template <int G, int KMAX, int NK>
__global__ __launch_bounds__(kDecodeBlock) void decode_sparse_kernel(SparseDecodeArgs a) {
  using C = SparseCfg<G>;
  constexpr int NMAX = NK > 0 ? NK : KMAX;
  constexpr int KW = RowCfg<NMAX>::kW;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int unit = b * a.Hkv + h;
  const int wave = wave_uniform((int)(threadIdx.x / kWave));
  const uint32_t lane = lane_id();
  int T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > a.cap ? a.cap : T);
  const int ntiles = (T + kTile - 1) / kTile;
  const int ntoff = a.cap / kTile + 1;

  uint16_t* q_lds = reinterpret_cast<uint16_t*>(smem);
  char* wbase = smem + C::kQBytes + wave * C::kWaveBytes;
  char* vt_lds = wbase;                                   // [129][144 B] channel-major value tile
  uint32_t* p2_lds = reinterpret_cast<uint32_t*>(wbase + C::kTileBytes);  // [32][G] fp16 pairs

  for (int idx = threadIdx.x; idx < 129 * G; idx += kDecodeBlock) {
    const int c = idx / G, g = idx % G;
    q_lds[idx] = (c < kHeadDim) ? a.q[((int64_t)b * a.Hq + h * G + g) * kHeadDim + c] : (uint16_t)0;
  }
  __syncthreads();

  const float ninf = -__builtin_inff();
  float m[G], lsum[G], acc0[G], acc1[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m[g] = ninf; lsum[g] = 0.f; acc0[g] = 0.f; acc1[g] = 0.f; }

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
  // bytes are the next rows' and hit the cache)
  constexpr int kch = NK > 0 ? row_chunks(NK) : KW / 4;
  constexpr int vch = kch;
  const bool k_odd = (kk & 1) != 0, v_odd = (vk & 1) != 0;

  // tile offsets of this wave's tiles, 64 at a time, one per lane
  int toff_base = tb;
  uint32_t ktv = buf_load4(ktrs, (uint32_t)(tb + lane) * 4u);
  uint32_t vtv = buf_load4(vtrs, (uint32_t)(tb + lane) * 4u);
  auto offsets = [&](int tile, uint32_t& kt0, uint32_t& vt0) {
    if (tile - toff_base >= kWave) {
      toff_base = tile;
      ktv = buf_load4(ktrs, (uint32_t)(tile + lane) * 4u);
      vtv = buf_load4(vtrs, (uint32_t)(tile + lane) * 4u);
    }
    kt0 = __builtin_amdgcn_readlane(ktv, tile - toff_base);
    vt0 = __builtin_amdgcn_readlane(vtv, tile - toff_base);
  };

  // One register set per side, refilled for the next tile as soon as the
  // current tile's walk over it is done (keys after the key walk, values after
  // the value walk), so each side's loads overlap the rest of the tile.
  constexpr bool kEvenExact = NK > 0 && NK % 2 == 0;  // see the matrix-core kernel
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
  if (tb < te) {
    offsets(tb, kt0, vt0);
    issue_k(tb, kt0);
    issue_v(tb, vt0);
  }

  for (int tile = tb; tile < te; ++tile) {
    set_priority_by_tiles_left(te - tile, tpw);
    const int nvalid = min(kTile, T - tile * kTile);
    const bool valid = (int)lane < nvalid;
    const bool partial = nvalid < kTile;
    const int nxt = min(tile + 1, te - 1);  // the last tile reloads itself
    offsets(nxt, kt0n, vt0n);

    // ---- key side: scores for the G heads
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
    auto score = [&](uint32_t addr, uint32_t vbits) {
      uint32_t qh[G];
      load_q<G>(smem + addr, qh);
      const float v = half_bits_to_float(vbits);
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g] = fmaf(v, half_bits_to_float(qh[g]), sc[g]);
    };
    // lanes past the end read q entries like the others; their scores are masked
    if (!kEvenExact && (k_odd || (kt0 & 1u))) realign_row<KW>(kt0 + lane * (uint32_t)kk, krow);
    decode_side<NMAX, NK, true, C::kQMul>(krs, kt0, kk, valid, partial, !kEvenExact || !(kt0 & 1u),
                                          kb, krow, 0u, 0u, score);
    issue_k(nxt, kt0n);

    // ---- online softmax in log2 units; p as fp16 pairs for the dot2 P.V
    float p[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sv = valid ? sc[g] * a.scale_log2 : ninf;
      const float mn = fmaxf(m[g], wave_max(sv));
      const float alpha = exp2_raw(m[g] - mn);
      p[g] = exp2_raw(sv - mn);
      lsum[g] = lsum[g] * alpha + p[g];
      acc0[g] *= alpha;
      acc1[g] *= alpha;
      m[g] = mn;
    }

    // ---- value side: channel-major tile of this tile's stored values
    wave_lds_sync();  // the previous tile's reads of the tile and of p are done
#pragma unroll
    for (int j = 0; j < (kHeadDim * kTRowBytes) / (16 * kWave); ++j)
      *reinterpret_cast<uint4*>(vt_lds + 16 * (lane + kWave * j)) = make_uint4(0u, 0u, 0u, 0u);
    {
      uint16_t* p16 = reinterpret_cast<uint16_t*>(p2_lds);
      const uint32_t pair = lane >> 1;
      const uint32_t slot = (pair >> 2) * C::kP2Block + (pair & 3u) * G;
#pragma unroll
      for (int g = 0; g < G; ++g) p16[(slot + g) * 2 + (lane & 1u)] = float_to_half_bits(p[g]);
    }
    wave_lds_sync();  // zeros in place before any lane writes its entries
    auto scatter = [&](uint32_t addr, uint32_t vbits) {
      *reinterpret_cast<uint16_t*>(smem + addr) = (uint16_t)vbits;
    };
    const uint32_t col = (uint32_t)(vt_lds - smem) + 2u * lane;
    if (!kEvenExact && (v_odd || (vt0 & 1u))) realign_row<KW>(vt0 + lane * (uint32_t)vk, vrow);
    decode_side<NMAX, NK, false, kTRowBytes>(vrs, vt0, vk, valid, partial,
                                             !kEvenExact || !(vt0 & 1u), vb, vrow, col, 0u, scatter);
    issue_v(nxt, vt0n);
    wave_lds_sync();  // every lane's entries written before the channel-major reads

    // ---- P.V: lane owns channels lane and lane+64; 32 row pairs per tile, in
    // 8 blocks of 4 pairs visited in a lane-rotated order (conflict-free reads)
    const char* r0p = vt_lds + (lane << kTRowShift);
    const char* r1p = vt_lds + ((lane + 64) << kTRowShift);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t jr = (j + lane) & 7u;
      const uint4 x0 = *reinterpret_cast<const uint4*>(r0p + 16 * jr);
      const uint4 x1 = *reinterpret_cast<const uint4*>(r1p + 16 * jr);
      const uint32_t w0[4] = {x0.x, x0.y, x0.z, x0.w};
      const uint32_t w1[4] = {x1.x, x1.y, x1.z, x1.w};
      const uint32_t* pb = p2_lds + jr * C::kP2Block;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint32_t* pr = pb + pp * G;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const half2v pv = __builtin_bit_cast(half2v, pr[g]);
          acc0[g] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, w0[pp]), pv, acc0[g], false);
          acc1[g] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, w1[pp]), pv, acc1[g], false);
        }
      }
    }
    kt0 = kt0n;
    vt0 = vt0n;
  }

#pragma unroll
  for (int g = 0; g < G; ++g) lsum[g] = wave_sum(lsum[g]);
  __syncthreads();  // the merge area overlaps the per-wave regions
  float* lds_m = reinterpret_cast<float*>(smem + C::kQBytes);
  float* lds_l = lds_m + kDecodeWaves * G;
  float* lds_acc = lds_l + kDecodeWaves * G;
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) { lds_m[wave * G + g] = m[g]; lds_l[wave * G + g] = lsum[g]; }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lds_acc[(wave * G + g) * kHeadDim + lane] = acc0[g];
    lds_acc[(wave * G + g) * kHeadDim + 64 + lane] = acc1[g];
  }
  __syncthreads();
  store_split_partial<G>(lds_m, lds_l, lds_acc, G * kHeadDim, kHeadDim, unit, a.splits, s, a.part);
}

template <int G, int KMAX, int NK>
hipError_t launch_sparse_t(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  constexpr int lds = SparseCfg<G>::kLdsBytes;
  if constexpr (lds > 65536) {
    hipError_t e = ensure_lds_limit<&decode_sparse_kernel<G, KMAX, NK>>(lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_sparse_kernel<G, KMAX, NK>), dim3(a.splits, a.Hkv, batch),
                     dim3(kDecodeBlock), lds, stream, a);
  return hipGetLastError();
}

// Straight-line kernels for the keeps of 70% and 50% sparsity at head_dim 128
// (38 and 64) when every head keeps the same; bucketed kernels for any other
// keep and for per-head keeps.
template <int G>
hipError_t launch_sparse_g(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  const bool uniform = !a.kmap.per_head && !a.vmap.per_head;
  if (uniform && a.kk == a.vk && a.kk == 38) return launch_sparse_t<G, 40, 38>(a, batch, stream);
  if (uniform && a.kk == a.vk && a.kk == 64) return launch_sparse_t<G, 64, 64>(a, batch, stream);
  const int kmax = a.kk > a.vk ? a.kk : a.vk;
  if (kmax <= 32) return launch_sparse_t<G, 32, 0>(a, batch, stream);
  if (kmax <= 48) return launch_sparse_t<G, 48, 0>(a, batch, stream);
  if (kmax <= 64) return launch_sparse_t<G, 64, 0>(a, batch, stream);
  return launch_sparse_t<G, 128, 0>(a, batch, stream);
}

}  // namespace

hipError_t launch_decode_sparse_valu(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_sparse_g<1>(a, batch, stream);
    case 2: return launch_sparse_g<2>(a, batch, stream);
    case 4: return launch_sparse_g<4>(a, batch, stream);
    case 8: return launch_sparse_g<8>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mustafar
