// Epilogue shared by the sparse and dense decode kernels: merge the online-
// softmax states of the block's waves, publish the block's partial for its
// split, and let the last block of each (batch, kv head) merge all splits and
// write the output.  A split's state for one q head is (m, l, acc[128]) with
// scores in log2 units: m = max score, l = sum 2^(s - m), acc = sum 2^(s - m) v.
// Splitting over the sequence keeps the GPU busy at small batch, where the
// pages report the sparse kernel under-using the GPU ([Summary] "Limitations").
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace mustafar {

// lds_m, lds_l: [kDecodeWaves][G]; lds_acc: [kDecodeWaves][G][128]; flag: one int.
template <int G>
__device__ __forceinline__ void finish_split(const float* lds_m, const float* lds_l,
                                             const float* lds_acc, int* flag, int unit, int b,
                                             int h, int Hq, int splits, int s, float* part,
                                             uint32_t* counters, uint16_t* out) {
  const int tid = threadIdx.x;
  const float ninf = -__builtin_inff();
  float* pb = part + ((int64_t)(unit * splits + s) * G) * kPartStride;
  for (int idx = tid; idx < G * kHeadDim; idx += kDecodeBlock) {
    const int g = idx / kHeadDim, c = idx % kHeadDim;
    float M = ninf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, lds_m[w * G + g]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float mw = lds_m[w * G + g];
      const float f = (mw == ninf) ? 0.f : exp2f(mw - M);
      A += lds_acc[(w * G + g) * kHeadDim + c] * f;
      L += lds_l[w * G + g] * f;
    }
    pb[g * kPartStride + 2 + c] = A;
    if (c == 0) {
      pb[g * kPartStride + 0] = M;
      pb[g * kPartStride + 1] = L;
    }
  }
  // Publish this split's partial, then count it; the block that completes the
  // count for this (batch, kv head) merges all splits.  Release/acquire at
  // device scope orders the partial stores with the counter across XCDs.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&counters[unit], 1u);
    *flag = (prev == (uint32_t)(splits - 1));
  }
  __syncthreads();
  if (!*flag) return;
  __threadfence();
  const float* pu = part + ((int64_t)unit * splits * G) * kPartStride;
  for (int idx = tid; idx < G * kHeadDim; idx += kDecodeBlock) {
    const int g = idx / kHeadDim, c = idx % kHeadDim;
    float M = ninf;
    for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, pu[(sp * G + g) * kPartStride]);
    float A = 0.f, L = 0.f;
    for (int sp = 0; sp < splits; ++sp) {
      const float* ps = pu + (sp * G + g) * kPartStride;
      const float ms = ps[0];
      const float f = (ms == ninf) ? 0.f : exp2f(ms - M);
      A += ps[2 + c] * f;
      L += ps[1] * f;
    }
    const float o = (L > 0.f) ? A / L : 0.f;
    out[((int64_t)b * Hq + h * G + g) * kHeadDim + c] = float_to_half_bits(o);
  }
  if (tid == 0) counters[unit] = 0u;  // leave the workspace ready for the next call
}

}  // namespace mustafar
