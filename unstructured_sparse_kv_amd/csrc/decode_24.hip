// 2:4 semi-structured comparator: decode attention over key and value caches
// in which every group of 4 consecutive channels of a row keeps exactly 2
// values -- one of the baselines the pages list ([Summary] "Experimental
// setup"), the structured kind of sparsity that unstructured pruning is shown
// to surpass ([Abstract]).  The caches are
// in the library's bitmap format at keep = 64: bitmap nibble g of a row marks
// the two kept channels of group g, and stored value dword g holds their
// values (lower channel in the low half).  mustafar_decode_attn reads the same
// bytes; this kernel uses the structure instead of walking the bitmap:
//   expand      each lane expands its row group by group in registers: the
//               group's nibble selects a pair of v_perm selectors from a
//               16-entry LDS table, which turn the group's value dword into
//               its 4 channels (8 bytes).  The dense rows go to a row-major
//               tile in LDS; every byte of it is written, so nothing is
//               cleared and nothing is scattered.
//   layout      8-byte chunk c of row t is stored at chunk c ^ s(t), where
//               s(t) swaps the two 2-bit fields of t mod 16.  The row writes
//               (16 rows, one chunk index), the key operand reads (16 rows)
//               and the transposed value reads (4 rows x 4 chunks) then each
//               touch 16 different bank pairs per 16 lanes.
//   scores      v_mfma_f32_16x16x32_f16, A = 16 key rows x 32 channels (two
//               8-byte reads), B = the G query heads as columns.
//   softmax     per head, online, with the reference max raised only when a
//               score exceeds it by more than 8 (log2 units), as in
//               mustafar_decode_attn.
//   P.V         v_mfma_f32_16x16x32_f16, A = 16 channels x 32 rows of the
//               value tile read transposed with ds_read_b64_tr_b16 (in each
//               16-lane group, lane i receives rows t0..t0+3 of channel c0 + i
//               when lane j addresses row t0 + j/4 at channels c0 + 4(j%4)),
//               B = p[rows][heads].
// Grid, splits and the cross-split merge are those of mustafar_decode_attn.
#include "device_common.hpp"
#include "kernels.hpp"
#include "merge.hpp"
#include "tile_softmax.hpp"

namespace mustafar {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;

constexpr int kRowBytes = 2 * kHeadDim;        // one dense row
constexpr int kTile24 = kTile * kRowBytes;     // 64 dense rows: the key tile, then the value tile
constexpr int kGroups = kHeadDim / 4;          // 32 groups of 4 channels per row

template <int G>
struct Cfg24 {
  static constexpr int kLutBytes = 16 * 8;     // (selector of channels 0-1, of channels 2-3) per nibble
  static constexpr int kPBytes = (G + 1) * 128;  // p[head][64] fp16; head row G stays zero
  static constexpr int kWaveBytes = kTile24 + kPBytes;
  static constexpr int kMergeBytes = kDecodeWaves * G * (2 + kHeadDim) * 4;
  static constexpr int kLdsBytes = kLutBytes + kDecodeWaves * kWaveBytes > kMergeBytes
                                       ? kLutBytes + kDecodeWaves * kWaveBytes
                                       : kMergeBytes;
};

__device__ __forceinline__ uint32_t swz(uint32_t t) { return ((t & 3u) << 2) | ((t >> 2) & 3u); }

// v_perm_b32(0, v, sel) selectors placing a group's two values (v: lower kept
// channel in bytes 0-1, higher in bytes 2-3) on their channels; selector byte
// 0x0C yields a zero byte.  Patterns without exactly two set bits give zeros.
__host__ __device__ constexpr uint64_t lut_entry(uint32_t n) {
  uint32_t hs[4] = {0x0C0Cu, 0x0C0Cu, 0x0C0Cu, 0x0C0Cu};
  int seen = 0, bits = 0;
  for (int c = 0; c < 4; ++c) bits += (n >> c) & 1u;
  if (bits == 2) {
    for (int c = 0; c < 4; ++c) {
      if ((n >> c) & 1u) {
        hs[c] = seen == 0 ? 0x0100u : 0x0302u;
        ++seen;
      }
    }
  }
  const uint32_t lo = hs[0] | (hs[1] << 16), hi = hs[2] | (hs[3] << 16);
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

// Two waves per SIMD (the LDS footprint allows no more): at most 256 registers
// per lane, accumulation registers included.
template <int G>
__global__ __launch_bounds__(kDecodeBlock) __attribute__((amdgpu_waves_per_eu(2)))
void decode_24_kernel(SparseDecodeArgs a) {
  using C = Cfg24<G>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int unit = b * a.Hkv + h;
  const int wave = wave_uniform((int)(threadIdx.x / kWave));
  const uint32_t lane = lane_id();
  const uint32_t l16 = lane & 15u, grp = lane >> 4;
  int T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > a.cap ? a.cap : T);
  const int ntiles = (T + kTile - 1) / kTile;

  uint2* lut = reinterpret_cast<uint2*>(smem);
  char* tile_lds = smem + C::kLutBytes + wave * C::kWaveBytes;
  uint16_t* p_lds = reinterpret_cast<uint16_t*>(tile_lds + kTile24);  // [G + 1][64]
  if (threadIdx.x < 16u) {
    const uint64_t e = lut_entry(threadIdx.x);
    lut[threadIdx.x] = make_uint2((uint32_t)e, (uint32_t)(e >> 32));
  }
  if (lane < 8u) *reinterpret_cast<uint4*>(p_lds + G * 64 + 8 * lane) = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

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

  // every row holds 64 values: row r of the unit starts at value 64 r
  const auto krs = make_rsrc(a.kval + (int64_t)unit * a.cap * 64, (uint32_t)a.cap * 128u);
  const auto vrs = make_rsrc(a.vval + (int64_t)unit * a.cap * 64, (uint32_t)a.cap * 128u);
  const auto kbrs = make_rsrc(a.kbm + (int64_t)unit * a.cap * 2, (uint32_t)a.cap * 16u);
  const auto vbrs = make_rsrc(a.vbm + (int64_t)unit * a.cap * 2, (uint32_t)a.cap * 16u);

  uint4 kb, vb;
  uint32_t krow[kGroups], vrow[kGroups];
  auto load_side = [&](__amdgpu_buffer_rsrc_t brs, __amdgpu_buffer_rsrc_t rs, int tile, uint4& bm,
                       uint32_t (&row)[kGroups]) {
    const uint32_t r = (uint32_t)(tile * kTile) + lane;
    bm = buf_load16(brs, r * 16u);
#pragma unroll
    for (int j = 0; j < kGroups / 4; ++j) {
      const uint4 c = buf_load16(rs, r * 128u + 16u * j);
      row[4 * j] = c.x; row[4 * j + 1] = c.y; row[4 * j + 2] = c.z; row[4 * j + 3] = c.w;
    }
  };
  if (tb < te) {
    load_side(kbrs, krs, tb, kb, krow);
    load_side(vbrs, vrs, tb, vb, vrow);
  }

  // The lane's row, expanded into the tile.  In a tile that ends the sequence
  // the rows past the end expand zero values (their bytes may be anything,
  // and P.V multiplies them by p = 0).
  const uint32_t lut_base = (uint32_t)((char*)lut - smem);
  char* my_row = tile_lds + lane * kRowBytes;
  const uint32_t my_swz = swz(lane);
  auto expand = [&](uint4 bm, uint32_t (&row)[kGroups], bool partial, bool valid) {
    if (partial) {
#pragma unroll
      for (int g = 0; g < kGroups; ++g) row[g] = valid ? row[g] : 0u;
    }
    const uint32_t w[4] = {bm.x, bm.y, bm.z, bm.w};
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const uint32_t nib = (w[g >> 3] >> (4 * (g & 7))) & 0xFu;
      const uint2 sel = *reinterpret_cast<const uint2*>(smem + lut_base + 8u * nib);
      const uint32_t v = row[g];
      const uint2 d = make_uint2(__builtin_amdgcn_perm(0u, v, sel.x), __builtin_amdgcn_perm(0u, v, sel.y));
      *reinterpret_cast<uint2*>(my_row + 8u * ((uint32_t)g ^ my_swz)) = d;
    }
  };

  for (int tile = tb; tile < te; ++tile) {
    set_priority_by_tiles_left(te - tile, tpw);
    const int nvalid = min(kTile, T - tile * kTile);
    const bool valid = (int)lane < nvalid;
    const bool partial = nvalid < kTile;
    const int nxt = min(tile + 1, te - 1);  // the last tile reloads itself

    // ---- key tile
    wave_lds_sync();  // the previous tile's reads of the buffer are done
    expand(kb, krow, partial, valid);
    load_side(kbrs, krs, nxt, kb, krow);
    wave_lds_sync();

    // ---- scores: 4 row blocks x 4 channel blocks
    floatx4 cs[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      cs[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
      const char* rowp = tile_lds + (16 * mb + l16) * kRowBytes;
      const uint32_t sw = swz(l16);
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        const uint32_t c0 = 8u * kb4 + 2u * grp;
        const uint2 x0 = *reinterpret_cast<const uint2*>(rowp + 8u * (c0 ^ sw));
        const uint2 x1 = *reinterpret_cast<const uint2*>(rowp + 8u * ((c0 + 1u) ^ sw));
        const uint4 x = make_uint4(x0.x, x0.y, x1.x, x1.y);
        cs[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, x), bq[kb4],
                                                        cs[mb], 0, 0, 0);
      }
    }

    // ---- online softmax (tile_softmax.hpp); p to LDS
    tile_softmax<G>(cs, a.scale_log2, partial, nvalid, l16, grp, m, lsum, acc, p_lds);

    // ---- value tile in the same buffer
    wave_lds_sync();  // score reads of the key tile done; p written
    expand(vb, vrow, partial, valid);
    load_side(vbrs, vrs, nxt, vb, vrow);
    wave_lds_sync();

    // ---- P.V: 8 channel blocks x 2 row blocks; A read transposed
    const uint16_t* prow = p_lds + (l16 < (uint32_t)G ? l16 : (uint32_t)G) * 64 + 8 * grp;
    const half8 pb0 = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(prow));
    const half8 pb1 = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(prow + 32));
    const uint32_t tr_dr = l16 >> 2;  // row of this lane's chunk within a 4-row read
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const uint32_t chunk = 4u * mb + (l16 & 3u);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        short4v r[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t t = 32u * kc + 8u * grp + 4u * hh + tr_dr;
          const uint32_t off = (uint32_t)(tile_lds - smem) + t * kRowBytes + 8u * (chunk ^ swz(t));
          r[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_short4*)((__attribute__((address_space(3))) char*)smem + off));
        }
        const half8 av = __builtin_bit_cast(
            half8, make_uint4(__builtin_bit_cast(uint2, r[0]).x, __builtin_bit_cast(uint2, r[0]).y,
                              __builtin_bit_cast(uint2, r[1]).x, __builtin_bit_cast(uint2, r[1]).y));
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, kc == 0 ? pb0 : pb1, acc[mb], 0, 0, 0);
      }
    }
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

template <int G>
hipError_t launch_24_g(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  constexpr int lds = Cfg24<G>::kLdsBytes;
  if constexpr (lds > 65536) {
    hipError_t e = ensure_lds_limit<&decode_24_kernel<G>>(lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_24_kernel<G>), dim3(a.splits, a.Hkv, batch), dim3(kDecodeBlock), lds,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_24(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_24_g<1>(a, batch, stream);
    case 2: return launch_24_g<2>(a, batch, stream);
    case 4: return launch_24_g<4>(a, batch, stream);
    case 8: return launch_24_g<8>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mustafar
