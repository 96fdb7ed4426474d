// Decode-step attention computed directly over the bitmap-compressed key and
// value caches ([Summary] "Approach": a custom attention kernel over the bitmap
// format; [Abstract]; [README] "Part III": batched sparse attention kernel).
//
// Grid (splits, Hkv, B); 4 waves per block.  The tiles (64 rows) of a
// (batch, kv head) are divided among the splits * 4 waves; each wave keeps an
// online-softmax state for the G = Hq/Hkv query heads that read this kv head,
// and the block epilogue merges waves, then splits.
//
// Per 64-row tile, one wave:
//   key side   lane t owns row t: its bitmap (4 dwords) and its kept values
//              (in registers) are walked set bit by set bit; channel c of
//              the n-th set bit pairs with value n, and q[g][c] comes from LDS.
//              Every q head of the group reuses each decoded element.
//   softmax    wave max / exp2 / running sum per q head.
//   value side lane l owns channels l and l+64; per row t the row's bitmap
//              words are scalar (SGPR) loads, the value index is
//              mbcnt(bitmap) + row start, the value is gathered from the
//              tile staged in LDS and zeroed by a v_cndmask on the bitmap.
// No matrix cores: this is a memory-bound sparse matrix-vector product.
#include "device_common.hpp"
#include "kernels.hpp"
#include "merge.hpp"

namespace mustafar {
namespace {

template <int G>
struct SparseLayout {
  static constexpr int kQBytes = ((129 * 2 * G) + 15) / 16 * 16;  // q[c][g] fp16, c = 128 is zero
};

template <int G, int KMAX>
struct SparseCfg {
  static constexpr int kKChunks = (KMAX / 2 + 1 + 3) / 4;  // 16 B chunks per key row (+1 dword)
  static constexpr int kKW = kKChunks * 4;                  // dwords of a key row in registers
  static constexpr int kVChunks = (KMAX * 8 + 1 + 63) / 64; // 16 B chunks per lane for a value tile
  static constexpr int kVStageBytes = ((64 * KMAX + 16) * 2 + 15) / 16 * 16;
  static constexpr int kWaveBytes = kVStageBytes + 64 * G * 4 + 64 * 8;
  static constexpr int kMergeBytes = kDecodeWaves * G * (2 + kHeadDim) * 4;
  static constexpr int kLdsBytes =
      SparseLayout<G>::kQBytes +
      (kDecodeWaves * kWaveBytes > kMergeBytes ? kDecodeWaves * kWaveBytes : kMergeBytes);
};

// q[g][ch] for the G heads of the group, from the LDS table q_lds[ch][g].
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
__device__ __forceinline__ uint32_t value_bits(const uint32_t (&row)[KW], int i) {
  const uint32_t w = row[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Fast walk: every valid row holds exactly `kk` set bits and all four bitmap
// dwords are non-zero (invalid lanes carry all-ones words and zero values), so
// the next dword is never empty and no lane runs out before the last step.
template <int G, int KMAX, int KW>
__device__ __forceinline__ void key_scores_fast(const uint32_t (&row)[KW], uint4 w, int kk,
                                                const uint16_t* q_lds, float (&s)[G]) {
  uint32_t cur = w.x, n1 = w.y, n2 = w.z, n3 = w.w, base = 0;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i < kk) {
      const uint32_t ch = base + (uint32_t)__builtin_ctz(cur);
      uint32_t qh[G];
      load_q<G>(q_lds, ch, qh);
      const float v = half_bits_to_float(value_bits(row, i));
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = fmaf(v, half_bits_to_float(qh[g]), s[g]);
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
// channel base) and a lane that has used all its set bits reads the zero q
// entry (channel 128); its remaining values are zero.
template <int G, int KMAX, int KW>
__device__ __forceinline__ void key_scores_general(const uint32_t (&row)[KW], uint4 w, int iters,
                                                   const uint16_t* q_lds, float (&s)[G]) {
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
      const uint32_t ch = cur ? b0 + (uint32_t)__builtin_ctz(cur) : 128u;
      uint32_t qh[G];
      load_q<G>(q_lds, ch, qh);
      const float v = half_bits_to_float(value_bits(row, i));
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = fmaf(v, half_bits_to_float(qh[g]), s[g]);
      cur &= cur - 1u;
      const bool z = (cur == 0u);
      cur = z ? n1 : cur; b0 = z ? b1 : b0;
      n1 = z ? n2 : n1; b1 = z ? b2 : b1;
      n2 = z ? n3 : n2; b2 = z ? b3 : b2;
      n3 = z ? 0u : n3; b3 = z ? 128u : b3;
    }
  }
}

// Loads dwords of the key values starting at half index `start` of the region
// and shifts them so that row[i] holds values 2i and 2i+1 of the row.
template <int KW>
__device__ __forceinline__ void load_key_row(__amdgpu_buffer_rsrc_t rs, uint32_t start, int nchunks,
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

template <int G, int KMAX>
__global__ __launch_bounds__(kDecodeBlock) void decode_sparse_kernel(SparseDecodeArgs a) {
  using C = SparseCfg<G, KMAX>;
  constexpr int KW = C::kKW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int last_flag;

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int unit = b * a.Hkv + h;
  const int wave = wave_uniform((int)(threadIdx.x / kWave));
  const uint32_t lane = lane_id();
  int T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > a.cap ? a.cap : T);
  const int ntiles = (T + kTile - 1) / kTile;
  const int64_t ntoff = a.cap / kTile + 1;

  uint16_t* q_lds = reinterpret_cast<uint16_t*>(smem);
  for (int idx = threadIdx.x; idx < 129 * G; idx += kDecodeBlock) {
    const int c = idx / G, g = idx % G;
    q_lds[idx] = (c < kHeadDim) ? a.q[((int64_t)b * a.Hq + h * G + g) * kHeadDim + c] : (uint16_t)0;
  }
  __syncthreads();

  char* wb = smem + SparseLayout<G>::kQBytes + wave * C::kWaveBytes;
  uint16_t* vstage = reinterpret_cast<uint16_t*>(wb);
  float* p_lds = reinterpret_cast<float*>(wb + C::kVStageBytes);
  uint2* rs_lds = reinterpret_cast<uint2*>(wb + C::kVStageBytes + 64 * G * 4);

  const float ninf = -__builtin_inff();
  float m[G], lsum[G], acc0[G], acc1[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m[g] = ninf; lsum[g] = 0.f; acc0[g] = 0.f; acc1[g] = 0.f; }

  const int total_waves = a.splits * kDecodeWaves;
  const int wid = s * kDecodeWaves + wave;
  const int tpw = (ntiles + total_waves - 1) / total_waves;
  const int tb = min(wid * tpw, ntiles), te = min(tb + tpw, ntiles);

  const int kk = a.kk;
  const uint64_t* kbm_u = a.kbm + (int64_t)unit * a.cap * 2;
  const uint64_t* vbm_u = a.vbm + (int64_t)unit * a.cap * 2;
  const auto krs = make_rsrc(a.kval + (int64_t)unit * a.cap * kk, (uint32_t)a.cap * kk * 2u);
  const auto vrs = make_rsrc(a.vval + (int64_t)unit * a.cap * a.vk, (uint32_t)a.cap * a.vk * 2u);
  const auto kbrs = make_rsrc(kbm_u, (uint32_t)a.cap * 16u);
  const auto vbrs = make_rsrc(vbm_u, (uint32_t)a.cap * 16u);
  ConstU32 ktoff_u = (ConstU32)(a.ktoff + unit * ntoff);
  ConstU32 vtoff_u = (ConstU32)(a.vtoff + unit * ntoff);
  const int kchunks_exact = (((kk + 1) >> 1) + 1 + 3) >> 2;

  for (int tile = tb; tile < te; ++tile) {
    const int row0 = tile * kTile;
    const int nvalid = min(kTile, T - row0);
    const bool valid = (int)lane < nvalid;
    const uint32_t kt0 = ktoff_u[tile];
    const uint32_t vt0 = vtoff_u[tile], vt1 = vtoff_u[tile + 1];

    // ---- issue the tile's loads: key bitmaps and rows first, value side after
    uint4 kb = buf_load16(kbrs, (uint32_t)(row0 + lane) * 16u);
    uint32_t krow[KW];
    const uint32_t kst = kt0 + lane * (uint32_t)kk;  // row start if every row holds kk values
    load_key_row<KW>(krs, kst, kchunks_exact, ((kt0 | (uint32_t)kk) & 1u) != 0u, krow);
    const uint4 vbv = buf_load16(vbrs, (uint32_t)(row0 + lane) * 16u);
    const uint32_t va = vt0 & ~7u;
    // chunks to stage; never more than the wave's stage holds, whatever the offsets say
    const int nvch = (int)min((vt1 - va + 7u) >> 3, (uint32_t)(C::kVStageBytes / 16));
    uint4 vch[C::kVChunks];
#pragma unroll
    for (int j = 0; j < C::kVChunks; ++j) {
      const int c = (int)lane + kWave * j;
      vch[j] = make_uint4(0u, 0u, 0u, 0u);
      if (c < nvch) vch[j] = buf_load16(vrs, (va + 8u * c) * 2u);
    }

    // ---- key side: scores for the G heads, lane = row
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
    const uint32_t kpop = __popc(kb.x) + __popc(kb.y) + __popc(kb.z) + __popc(kb.w);
    const bool lane_fast = !valid || (kpop == (uint32_t)kk && kb.x && kb.y && kb.z && kb.w);
    if (__ballot(!lane_fast) == 0ull) {
      if (nvalid < kTile) {
        if (!valid) kb = make_uint4(~0u, ~0u, ~0u, ~0u);
#pragma unroll
        for (int j = 0; j < KW; ++j) krow[j] = valid ? krow[j] : 0u;
      }
      key_scores_fast<G, KMAX, KW>(krow, kb, kk, q_lds, sc);
    } else {
      const uint32_t pc = valid ? kpop : 0u;
      const uint32_t st = kt0 + wave_excl_scan(pc);
      const int iters = (int)wave_uniform(wave_max_u32(pc));
      const int nch = (((iters + 1) >> 1) + 1 + 3) >> 2;
      load_key_row<KW>(krs, st, nch, true, krow);
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const uint32_t lo_ok = (2u * j < pc) ? 0xFFFFu : 0u;
        const uint32_t hi_ok = (2u * j + 1u < pc) ? 0xFFFF0000u : 0u;
        krow[j] &= (lo_ok | hi_ok);
      }
      if (!valid) kb = make_uint4(0u, 0u, 0u, 0u);
      key_scores_general<G, KMAX, KW>(krow, kb, iters, q_lds, sc);
    }

    // ---- online softmax (log2 units); p goes to LDS for the value side
    float pv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sv = valid ? sc[g] * a.scale_log2 : ninf;
      const float mt = wave_max(sv);
      const float mn = fmaxf(m[g], mt);
      const float alpha = exp2f(m[g] - mn);
      pv[g] = exp2f(sv - mn);
      lsum[g] = lsum[g] * alpha + pv[g];
      acc0[g] *= alpha;
      acc1[g] *= alpha;
      m[g] = mn;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) p_lds[lane * G + g] = pv[g];

    // ---- value side: stage the tile's values, row starts, then lane = channel
    wave_lds_sync();  // the previous tile's reads of the stage are done
#pragma unroll
    for (int j = 0; j < C::kVChunks; ++j) {
      const int c = (int)lane + kWave * j;
      if (c < nvch) *reinterpret_cast<uint4*>(vstage + 8 * c) = vch[j];
    }
    {
      const uint32_t p0 = valid ? (uint32_t)(__popc(vbv.x) + __popc(vbv.y)) : 0u;
      const uint32_t p1 = valid ? (uint32_t)(__popc(vbv.z) + __popc(vbv.w)) : 0u;
      const uint32_t r0 = (vt0 - va) + wave_excl_scan(p0 + p1);
      rs_lds[lane] = make_uint2(r0, r0 + p0);
    }
    wave_lds_sync();  // stage, p and row starts written by every lane before any lane reads
    ConstU64 vbs = (ConstU64)(vbm_u + (int64_t)row0 * 2);
#pragma unroll 8
    for (int t = 0; t < nvalid; ++t) {
      const uint64_t w0 = vbs[2 * t], w1 = vbs[2 * t + 1];
      const uint2 rs = rs_lds[t];
      const uint32_t x0 = keep_if_lane_bit(w0, vstage[mbcnt64(w0, rs.x)]);
      const uint32_t x1 = keep_if_lane_bit(w1, vstage[mbcnt64(w1, rs.y)]);
      const float v0 = half_bits_to_float(x0), v1 = half_bits_to_float(x1);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = p_lds[t * G + g];
        acc0[g] = fmaf(v0, p, acc0[g]);
        acc1[g] = fmaf(v1, p, acc1[g]);
      }
    }
  }

#pragma unroll
  for (int g = 0; g < G; ++g) lsum[g] = wave_sum(lsum[g]);
  __syncthreads();  // the merge area overlaps the per-wave regions
  float* lds_m = reinterpret_cast<float*>(smem + SparseLayout<G>::kQBytes);
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
  finish_split<G>(lds_m, lds_l, lds_acc, &last_flag, unit, b, h, a.Hq, a.splits, s, a.part,
                  a.counters, a.out);
}

template <int G, int KMAX>
hipError_t launch_sparse_t(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  constexpr int lds = SparseCfg<G, KMAX>::kLdsBytes;
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
