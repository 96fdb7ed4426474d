// Decode-step attention computed directly over the bitmap-compressed key and
// value caches ([Summary] "Approach": a custom attention kernel over the bitmap
// format; [Abstract]; [README] "Part III": batched sparse attention kernel).
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

namespace mustafar {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kTRowBytes = 144;  // one channel row of the value tile: 64 fp16 + 16 B pad
constexpr int kTRows = 129;      // 128 channels + a dump row for lanes past their last entry

template <int G>
struct SparseCfg {
  static constexpr int kQBytes = ((129 * 2 * G) + 15) / 16 * 16;  // q[c][g] fp16, c = 128 is zero
  static constexpr int kTileBytes = kTRows * kTRowBytes;
  static constexpr int kP2Bytes = 32 * G * 4;                     // p pairs, [pair][g] fp16x2
  static constexpr int kWaveBytes = (kTileBytes + kP2Bytes + 15) / 16 * 16;
  static constexpr int kMergeBytes = kDecodeWaves * G * (2 + kHeadDim) * 4;
  static constexpr int kLdsBytes =
      kQBytes + (kDecodeWaves * kWaveBytes > kMergeBytes ? kDecodeWaves * kWaveBytes : kMergeBytes);
};

template <int KMAX>
struct RowCfg {
  static constexpr int kChunks = (KMAX / 2 + 1 + 3) / 4;  // 16 B chunks per row (+1 dword for realign)
  static constexpr int kW = kChunks * 4;                   // dwords of a row in registers
};

// q[c][g] for the G heads of the group, from the LDS table q_lds[c][g].
template <int G>
__device__ __forceinline__ void load_q(const uint16_t* q_lds, uint32_t ch, uint32_t (&qh)[G]) {
  const uint16_t* p = q_lds + ch * G;
  if constexpr (G == 1) {
    qh[0] = p[0];
  } else if constexpr (G == 2) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(p);
    qh[0] = x & 0xFFFFu;
    qh[1] = x >> 16;
  } else if constexpr (G == 4) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    qh[0] = x.x & 0xFFFFu; qh[1] = x.x >> 16; qh[2] = x.y & 0xFFFFu; qh[3] = x.y >> 16;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    qh[0] = x.x & 0xFFFFu; qh[1] = x.x >> 16; qh[2] = x.y & 0xFFFFu; qh[3] = x.y >> 16;
    qh[4] = x.z & 0xFFFFu; qh[5] = x.z >> 16; qh[6] = x.w & 0xFFFFu; qh[7] = x.w >> 16;
  }
}

template <int KW>
__device__ __forceinline__ uint32_t value_at(const uint32_t (&row)[KW], int i) {
  const uint32_t w = row[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Fast walk over the set bits of a row: every valid row holds exactly n set
// bits and all four bitmap dwords are non-zero (invalid lanes carry all-ones
// words and zero values), so the next dword is never empty and no lane runs
// out before the last step.  f(channel, value bits) is called for each set bit.
template <int KMAX, int KW, class F>
__device__ __forceinline__ void walk_fast(const uint32_t (&row)[KW], uint4 w, int n, F&& f) {
  uint32_t cur = w.x, n1 = w.y, n2 = w.z, n3 = w.w, base = 0;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i < n) {
      f(base + (uint32_t)__builtin_ctz(cur), value_at(row, i));
      cur &= cur - 1u;
      const bool z = (cur == 0u);
      cur = z ? n1 : cur;
      n1 = z ? n2 : n1;
      n2 = z ? n3 : n2;
      base += z ? 32u : 0u;
    }
  }
}

// General walk: empty dwords are compacted away (each kept dword carries its
// channel base) and a lane that has used all its set bits reports channel 128
// (the zero q entry / the dump accumulator); its remaining values are zero.
template <int KMAX, int KW, class F>
__device__ __forceinline__ void walk_general(const uint32_t (&row)[KW], uint4 w, int iters, F&& f) {
  uint32_t cw[4] = {w.x, w.y, w.z, w.w};
  uint32_t cb[4] = {0u, 32u, 64u, 96u};
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
  for (int j = 0; j < 4; ++j) cb[j] = cw[j] ? cb[j] : 128u;
  uint32_t cur = cw[0], b0 = cb[0], n1 = cw[1], b1 = cb[1], n2 = cw[2], b2 = cb[2], n3 = cw[3],
           b3 = cb[3];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i < iters) {
      f(cur ? b0 + (uint32_t)__builtin_ctz(cur) : 128u, value_at(row, i));
      cur &= cur - 1u;
      const bool z = (cur == 0u);
      cur = z ? n1 : cur; b0 = z ? b1 : b0;
      n1 = z ? n2 : n1; b1 = z ? b2 : b1;
      n2 = z ? n3 : n2; b2 = z ? b3 : b2;
      n3 = z ? 0u : n3; b3 = z ? 128u : b3;
    }
  }
}

// Loads dwords of the stored values from half index `start` of the region
// and shifts them so that row[i] holds values 2i and 2i+1 of the row.
template <int KW>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t rs, uint32_t start, int nchunks,
                                         bool odd_possible, uint32_t (&row)[KW]) {
  const uint32_t dw0 = start >> 1;
#pragma unroll
  for (int j = 0; j < KW / 4; ++j) {
    uint4 c = make_uint4(0u, 0u, 0u, 0u);
    if (j < nchunks) c = buf_load16(rs, (dw0 + 4u * j) * 4u);
    row[4 * j + 0] = c.x; row[4 * j + 1] = c.y; row[4 * j + 2] = c.z; row[4 * j + 3] = c.w;
  }
  if (odd_possible) {
    const bool odd = start & 1u;
#pragma unroll
    for (int j = 0; j < KW - 1; ++j)
      row[j] = odd ? __builtin_amdgcn_alignbit(row[j + 1], row[j], 16u) : row[j];
  }
}

// Chunks of 16 B covering n values starting at any half offset (+1 dword slack).
__device__ __forceinline__ int row_chunks(int n) { return (((n + 1) >> 1) + 1 + 3) >> 2; }

// Zeroes stored values beyond the first `count` of the row.
template <int KW>
__device__ __forceinline__ void mask_row(uint32_t (&row)[KW], uint32_t count) {
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    const uint32_t lo_ok = (2u * j < count) ? 0xFFFFu : 0u;
    const uint32_t hi_ok = (2u * j + 1u < count) ? 0xFFFF0000u : 0u;
    row[j] &= (lo_ok | hi_ok);
  }
}

__device__ __forceinline__ uint32_t pop4(uint4 w) {
  return __popc(w.x) + __popc(w.y) + __popc(w.z) + __popc(w.w);
}

// Prepares one side's rows for a walk and reports whether the fast walk applies
// to the whole wave.  Rows were loaded at the start each would have if every row
// held exactly `keep` values; when that does not hold the rows are reloaded from
// their exact starts (prefix sum of the popcounts).
template <int KW>
__device__ __forceinline__ bool prepare_rows(__amdgpu_buffer_rsrc_t rs, uint32_t toff, int keep,
                                             bool valid, bool partial, uint4& bm,
                                             uint32_t (&row)[KW], int& iters) {
  const uint32_t pop = pop4(bm);
  const bool lane_fast = !valid || (pop == (uint32_t)keep && bm.x && bm.y && bm.z && bm.w);
  if (__ballot(!lane_fast) == 0ull) {
    if (partial) {
      if (!valid) bm = make_uint4(~0u, ~0u, ~0u, ~0u);
#pragma unroll
      for (int j = 0; j < KW; ++j) row[j] = valid ? row[j] : 0u;
    }
    iters = keep;
    return true;
  }
  const uint32_t pc = valid ? pop : 0u;
  const uint32_t st = toff + wave_excl_scan(pc);
  iters = (int)wave_uniform(wave_max_u32(pc));
  load_row<KW>(rs, st, row_chunks(iters), true, row);
  mask_row<KW>(row, pc);
  if (!valid) bm = make_uint4(0u, 0u, 0u, 0u);
  return false;
}

template <int G, int KMAX>
__global__ __launch_bounds__(kDecodeBlock) void decode_sparse_kernel(SparseDecodeArgs a) {
  using C = SparseCfg<G>;
  constexpr int KW = RowCfg<KMAX>::kW;
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
  const int tpw = (ntiles + total_waves - 1) / total_waves;
  const int tb = min(wid * tpw, ntiles), te = min(tb + tpw, ntiles);

  const int kk = a.kk, vk = a.vk;
  const auto krs = make_rsrc(a.kval + (int64_t)unit * a.cap * kk, (uint32_t)a.cap * kk * 2u);
  const auto vrs = make_rsrc(a.vval + (int64_t)unit * a.cap * vk, (uint32_t)a.cap * vk * 2u);
  const auto kbrs = make_rsrc(a.kbm + (int64_t)unit * a.cap * 2, (uint32_t)a.cap * 16u);
  const auto vbrs = make_rsrc(a.vbm + (int64_t)unit * a.cap * 2, (uint32_t)a.cap * 16u);
  const auto ktrs = make_rsrc(a.ktoff + (int64_t)unit * ntoff, (uint32_t)ntoff * 4u);
  const auto vtrs = make_rsrc(a.vtoff + (int64_t)unit * ntoff, (uint32_t)ntoff * 4u);
  const int kch = row_chunks(kk), vch = row_chunks(vk);
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
  uint4 kb, vb;
  uint32_t krow[KW], vrow[KW];
  uint32_t kt0 = 0, vt0 = 0, kt0n = 0, vt0n = 0;
  auto issue_k = [&](int tile, uint32_t t0) {
    kb = buf_load16(kbrs, ((uint32_t)(tile * kTile) + lane) * 16u);
    load_row<KW>(krs, t0 + lane * (uint32_t)kk, kch, k_odd || (t0 & 1u), krow);
  };
  auto issue_v = [&](int tile, uint32_t t0) {
    vb = buf_load16(vbrs, ((uint32_t)(tile * kTile) + lane) * 16u);
    load_row<KW>(vrs, t0 + lane * (uint32_t)vk, vch, v_odd || (t0 & 1u), vrow);
  };
  if (tb < te) {
    offsets(tb, kt0, vt0);
    issue_k(tb, kt0);
    issue_v(tb, vt0);
  }

  for (int tile = tb; tile < te; ++tile) {
    const int nvalid = min(kTile, T - tile * kTile);
    const bool valid = (int)lane < nvalid;
    const bool partial = nvalid < kTile;
    const bool more = tile + 1 < te;
    if (more) offsets(tile + 1, kt0n, vt0n);

    // ---- key side: scores for the G heads
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
    auto score = [&](uint32_t ch, uint32_t vbits) {
      uint32_t qh[G];
      load_q<G>(q_lds, ch, qh);
      const float v = half_bits_to_float(vbits);
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g] = fmaf(v, half_bits_to_float(qh[g]), sc[g]);
    };
    int kit;
    if (prepare_rows<KW>(krs, kt0, kk, valid, partial, kb, krow, kit))
      walk_fast<KMAX, KW>(krow, kb, kit, score);
    else
      walk_general<KMAX, KW>(krow, kb, kit, score);
    if (more) issue_k(tile + 1, kt0n);

    // ---- online softmax in log2 units
    float p[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sv = valid ? sc[g] * a.scale_log2 : ninf;
      const float mn = fmaxf(m[g], wave_max(sv));
      const float alpha = exp2f(m[g] - mn);
      p[g] = exp2f(sv - mn);
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
    uint16_t* p16 = reinterpret_cast<uint16_t*>(p2_lds);
#pragma unroll
    for (int g = 0; g < G; ++g)
      p16[((lane >> 1) * G + g) * 2 + (lane & 1)] = float_to_half_bits(p[g]);
    wave_lds_sync();  // zeros in place before any lane writes its entries
    char* col = vt_lds + 2 * lane;
    auto scatter = [&](uint32_t ch, uint32_t vbits) {
      *reinterpret_cast<uint16_t*>(col + ch * kTRowBytes) = (uint16_t)vbits;
    };
    int vit;
    if (prepare_rows<KW>(vrs, vt0, vk, valid, partial, vb, vrow, vit))
      walk_fast<KMAX, KW>(vrow, vb, vit, scatter);
    else
      walk_general<KMAX, KW>(vrow, vb, vit, scatter);
    if (more) issue_v(tile + 1, vt0n);
    wave_lds_sync();  // every lane's entries written before the channel-major reads

    // ---- P.V: lane owns channels lane and lane+64; 32 row pairs per tile
    const char* r0p = vt_lds + lane * kTRowBytes;
    const char* r1p = vt_lds + (lane + 64) * kTRowBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(r0p + 16 * j);
      const uint4 x1 = *reinterpret_cast<const uint4*>(r1p + 16 * j);
      const uint32_t w0[4] = {x0.x, x0.y, x0.z, x0.w};
      const uint32_t w1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint32_t* pr = p2_lds + (4 * j + pp) * G;
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

template <int G, int KMAX>
hipError_t launch_sparse_t(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  constexpr int lds = SparseCfg<G>::kLdsBytes;
  if constexpr (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_sparse_kernel<G, KMAX>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_sparse_kernel<G, KMAX>), dim3(a.splits, a.Hkv, batch),
                     dim3(kDecodeBlock), lds, stream, a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_sparse_g(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  const int kmax = a.kk > a.vk ? a.kk : a.vk;
  if (kmax <= 32) return launch_sparse_t<G, 32>(a, batch, stream);
  if (kmax <= 40) return launch_sparse_t<G, 40>(a, batch, stream);
  if (kmax <= 48) return launch_sparse_t<G, 48>(a, batch, stream);
  if (kmax <= 64) return launch_sparse_t<G, 64>(a, batch, stream);
  return launch_sparse_t<G, 128>(a, batch, stream);
}

}  // namespace

hipError_t launch_decode_sparse(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_sparse_g<1>(a, batch, stream);
    case 2: return launch_sparse_g<2>(a, batch, stream);
    case 4: return launch_sparse_g<4>(a, batch, stream);
    case 8: return launch_sparse_g<8>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mustafar
