// Split-K bookkeeping shared by the sparse and dense decode kernels.
//
// A (split, q head) state is (m, l, acc[128]) with scores in log2 units:
// m is a reference score, l = sum 2^(s - m), acc = sum 2^(s - m) v.  The
// waves of a block merge in LDS into one state per split, written to the
// workspace; the reduce kernel then merges the splits of each (batch, q head)
// and writes the output.  Splitting over the sequence keeps the GPU busy at
// small batch, where the pages report the sparse kernel under-using the GPU
// ([Summary] "Limitations").
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace mustafar {

// Merge the block's waves (after a __syncthreads) and store the split's partial.
// lds_m, lds_l: [kDecodeWaves][G]; the accumulator of wave w, head g, channel c
// is at acc[w * wave_stride + g * g_stride + c].
template <int G>
__device__ __forceinline__ void store_split_partial(const float* lds_m, const float* lds_l,
                                                    const float* acc, int wave_stride, int g_stride,
                                                    int unit, int splits, int s, float* part) {
  const float ninf = -__builtin_inff();
  float* pb = part + ((int64_t)(unit * splits + s) * G) * kPartStride;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kDecodeBlock) {
    const int g = idx / kHeadDim, c = idx % kHeadDim;
    float M = ninf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, lds_m[w * G + g]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float mw = lds_m[w * G + g];
      const float f = (mw == ninf) ? 0.f : exp2f(mw - M);
      A += acc[w * wave_stride + g * g_stride + c] * f;
      L += lds_l[w * G + g] * f;
    }
    pb[g * kPartStride + 2 + c] = A;
    if (c == 0) {
      pb[g * kPartStride + 0] = M;
      pb[g * kPartStride + 1] = L;
    }
  }
}

}  // namespace mustafar
