// Dense fp16 decode attention over unpruned caches: the comparison baseline
// (the pages measure the sparse kernel against dense attention, [Summary]
// "Key results" and "Experimental setup").  Same split / online-softmax /
// merge structure as the sparse kernel.
//
// Per 64-row tile, one wave:
//   scores  matrix cores: v_mfma_f32_16x16x32_f16 with A = 16 cache rows x 32
//           channels (lane l: row l%16, channels 8*(l/16)..+7, one 16 B load)
//           and B = the G query heads x 32 channels (zero columns for heads
//           >= G); C lane l holds head l%16 for rows 4*(l/16)+i.  4 row blocks
//           x 4 channel blocks = 16 MFMAs per tile.
//   P.V     vector units: lane l owns channels 8*(l%16)..+7 of rows 4i + l/16,
//           fp32 accumulators for every head; lane groups are summed at the end.
//           The probabilities enter rounded to fp16 (their sum stays fp32), as
//           in the sparse kernels, so that the two compare like for like.
#include "device_common.hpp"
#include "kernels.hpp"
#include "merge.hpp"

namespace mustafar {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int G>
struct DenseCfg {
  static constexpr int kWaveBytes = 64 * G * 4 + 64;  // p[row][g] + alpha[g]
  static constexpr int kMergeBytes = kDecodeWaves * G * (2 + kHeadDim) * 4;
  static constexpr int kLdsBytes =
      kDecodeWaves * kWaveBytes > kMergeBytes ? kDecodeWaves * kWaveBytes : kMergeBytes;
};

template <int G>
__global__ __launch_bounds__(kDecodeBlock) void decode_dense_kernel(DenseDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int unit = b * a.Hkv + h;
  const int wave = wave_uniform((int)(threadIdx.x / kWave));
  const uint32_t lane = lane_id();
  const uint32_t l16 = lane & 15u, grp = lane >> 4;
  int64_t T64 = a.seq_lens[b];
  T64 = T64 < 0 ? 0 : (T64 > a.t_stride ? a.t_stride : T64);
  const int T = (int)T64;
  const int ntiles = (T + kTile - 1) / kTile;

  float* p_lds = reinterpret_cast<float*>(smem + wave * DenseCfg<G>::kWaveBytes);
  float* alpha_lds = p_lds + 64 * G;

  // B operand: query heads as columns
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
  float m = ninf, lsum = 0.f;  // for head l16
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

  const int total_waves = a.splits * kDecodeWaves;
  const int wid = s * kDecodeWaves + wave;
  // tiles split as evenly as their count allows: wave w takes [w n / W, (w + 1) n / W),
  // so no wave has more than one tile above the average (a split by the rounded-up
  // average gave 30 of 32 waves 17 tiles of a 513-tile unit, two waves 3 and 0)
  const int tb = (int)((int64_t)wid * ntiles / total_waves);
  const int te = (int)((int64_t)(wid + 1) * ntiles / total_waves);
  const uint32_t region = (uint32_t)(a.t_stride * kHeadDim * 2);
  const auto krs = make_rsrc(a.k + (int64_t)unit * a.t_stride * kHeadDim, region);
  const auto vrs = make_rsrc(a.v + (int64_t)unit * a.t_stride * kHeadDim, region);

  for (int tile = tb; tile < te; ++tile) {
    const int row0 = tile * kTile;
    const int nvalid = min(kTile, T - row0);
    // the whole tile's loads first: 16 x 16 B of keys, 16 x 16 B of values per lane
    uint4 ka[16], vr[16];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        ka[4 * mb + kb] = buf_load16(krs, (uint32_t)(row0 + 16 * mb + l16) * (kHeadDim * 2) +
                                              (32 * kb + 8 * grp) * 2);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      vr[i] = buf_load16(vrs, (uint32_t)(row0 + 4 * i + grp) * (kHeadDim * 2) + 16 * l16);
    floatx4 cs[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      cs[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        cs[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ka[4 * mb + kb]),
                                                        bq[kb], cs[mb], 0, 0, 0);
    }
    // online softmax for head l16 over this lane's 16 rows, then across lane groups
    float sv[16];
    float mt = ninf;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mb + 4 * (int)grp + i;
        sv[4 * mb + i] = (r < nvalid) ? cs[mb][i] * a.scale_log2 : ninf;
        mt = fmaxf(mt, sv[4 * mb + i]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float mn = fmaxf(m, mt);
    const float alpha = exp2f(m - mn);
    float ps = 0.f;
    wave_lds_sync();  // the previous tile's reads of p and alpha are done
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sv[4 * mb + i] - mn);
        ps += p;
        // P.V takes p rounded to fp16, the sparse kernels' operand precision
        if ((int)l16 < G) p_lds[(16 * mb + 4 * grp + i) * G + l16] = (float)(_Float16)p;
      }
    lsum = lsum * alpha + ps;
    m = mn;
    if (lane < (uint32_t)G) alpha_lds[lane] = alpha;
    wave_lds_sync();  // p and alpha written before any lane reads them
    float al[G];
#pragma unroll
    for (int g = 0; g < G; ++g) al[g] = alpha_lds[g];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= al[g];
    // P.V on the vector units
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 4 * i + (int)grp;
      if (r < nvalid) {
        const half8 v = __builtin_bit_cast(half8, vr[i]);
        float pg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pg[g] = p_lds[r * G + g];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ve = (float)v[e];
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g][e] = fmaf(ve, pg[g], acc[g][e]);
        }
      }
    }
  }

  // sum the four lane groups
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[g][e] += __shfl_xor(acc[g][e], 16, kWave);
      acc[g][e] += __shfl_xor(acc[g][e], 32, kWave);
    }
  __syncthreads();
  float* lds_m = reinterpret_cast<float*>(smem);
  float* lds_l = lds_m + kDecodeWaves * G;
  float* lds_acc = lds_l + kDecodeWaves * G;
  if (lane < (uint32_t)G) {
    lds_m[wave * G + lane] = m;
    lds_l[wave * G + lane] = lsum;
  }
  if (lane < 16u) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) lds_acc[(wave * G + g) * kHeadDim + 8 * lane + e] = acc[g][e];
  }
  __syncthreads();
  store_split_partial<G>(lds_m, lds_l, lds_acc, G * kHeadDim, kHeadDim, unit, a.splits, s, a.part);
}

template <int G>
hipError_t launch_dense_g(const DenseDecodeArgs& a, int batch, hipStream_t stream) {
  constexpr int lds = DenseCfg<G>::kLdsBytes;
  hipLaunchKernelGGL(decode_dense_kernel<G>, dim3(a.splits, a.Hkv, batch), dim3(kDecodeBlock), lds,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_dense(const DenseDecodeArgs& a, int batch, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_dense_g<1>(a, batch, stream);
    case 2: return launch_dense_g<2>(a, batch, stream);
    case 4: return launch_dense_g<4>(a, batch, stream);
    case 8: return launch_dense_g<8>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mustafar
