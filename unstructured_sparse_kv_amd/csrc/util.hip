// Small kernels: workspace clearing and the HBM stream-read probe.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mustafar {
namespace {

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Each block streams contiguous 4 KiB pages with coalesced 16 B loads; the XOR
// of everything read goes to *sink so the loads cannot be removed.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                          uint64_t pages, uint32_t* sink) {
  uint32_t x = 0;
  for (uint64_t pg = blockIdx.x; pg < pages; pg += gridDim.x) {
    const u32x4 v = __builtin_nontemporal_load(buf + pg * 256 + threadIdx.x);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9E3779B9u) atomicXor(sink, x);  // practically never taken
}

// Merge the split partials of one (batch, q head): block (b*Hq + hq).
// M = max m_s, L = sum l_s 2^(m_s - M), out = sum acc_s 2^(m_s - M) / L
// (0 for an empty sequence).  Thread t sums channel t % 128 over the splits of
// parity t / 128 (a wave-uniform value), and the two halves are added in LDS.
// The partials were written by the split kernel just before, so every load is
// a memory round trip: m and l of every split, then the accumulators of the
// first 2 * NV splits (they do not depend on M), are all requested at the
// start, and the factors 2^(m_s - M) go through LDS, so the merge waits for
// one round trip instead of one per batch of splits.  NV is the smallest of
// 4, 8, 16, 32 that covers the splits (more than 64 splits: the rest in a loop).
constexpr int kReduceThreads = 2 * kHeadDim;

template <int NV>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(
    const float* __restrict__ part, int hq_total, int g_size, int splits, uint16_t* __restrict__ out,
    int32_t* seq_lens, uint32_t* status, int32_t cap, int advance) {
  __shared__ float fs[kMaxSplits];  // 2^(m_s - M), 0 for an empty split
  __shared__ float red_m[kReduceThreads / kWave];
  __shared__ float red_l[kReduceThreads / kWave];
  __shared__ float half_a[kHeadDim];
  const int bq = blockIdx.x;
  const int b = bq / hq_total, hq = bq % hq_total;
  const int hkv = hq_total / g_size;
  const int h = hq / g_size, g = hq % g_size;
  const int unit = b * hkv + h;
  const int t = threadIdx.x, c = t % kHeadDim, par = wave_uniform(t / kHeadDim);
  const float ninf = -__builtin_inff();
  const float* pu = part + ((int64_t)unit * splits * g_size + g) * kPartStride;
  const int64_t sstride = (int64_t)g_size * kPartStride;

  // split t (splits <= kReduceThreads needs no other); clamped indices, so
  // that no load is conditional and waiting for one does not wait for later ones
  const float2 ml = *reinterpret_cast<const float2*>(pu + min(t, splits - 1) * sstride);
  const float m0 = t < splits ? ml.x : ninf, l0 = t < splits ? ml.y : 0.f;
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int sc = min(par + 2 * j, splits - 1);
    v[j] = pu[sc * sstride + 2 + c];
  }
  float mx = m0;
  for (int s = t + kReduceThreads; s < splits; s += kReduceThreads) mx = fmaxf(mx, pu[s * sstride]);
  mx = wave_max(mx);
  if (lane_id() == 0) red_m[t / kWave] = mx;
  __syncthreads();
  float M = red_m[0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / kWave; ++w) M = fmaxf(M, red_m[w]);

  float lp = 0.f;
  if (t < splits) {
    const float f = (m0 == ninf) ? 0.f : exp2f(m0 - M);
    fs[t] = f;
    lp = l0 * f;
  }
  for (int s = t + kReduceThreads; s < splits; s += kReduceThreads) {
    const float ms = pu[s * sstride];
    const float f = (ms == ninf) ? 0.f : exp2f(ms - M);
    fs[s] = f;
    lp += pu[s * sstride + 1] * f;
  }
  lp = wave_sum(lp);
  if (lane_id() == 0) red_l[t / kWave] = lp;
  __syncthreads();
  float L = red_l[0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / kWave; ++w) L += red_l[w];

  float A = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int s = par + 2 * j;
    if (s < splits) A += v[j] * fs[s];
  }
#pragma unroll 8
  for (int s = par + 2 * NV; s < splits; s += 2) A += pu[s * sstride + 2 + c] * fs[s];
  if (par == 1) half_a[c] = A;
  __syncthreads();
  if (par == 0) {
    A += half_a[c];
    out[(int64_t)bq * kHeadDim + c] = float_to_half_bits(L > 0.f ? A / L : 0.f);
  }
  // a fused decode step: the split kernel stored row seq_lens[b] (all its
  // blocks read the old length); one thread per sequence now advances it
  if (advance && hq == 0 && t == 0) {
    const int32_t tl = seq_lens[b] < 0 ? 0 : seq_lens[b];
    if (tl >= cap) {
      if (status) atomicOr(status, MUSTAFAR_STATUS_APPEND_FULL);
    } else {
      seq_lens[b] = tl + 1;
    }
  }
}

}  // namespace

hipError_t launch_decode_reduce(const float* part, int batch, int hq, int hkv, int splits,
                                uint16_t* out, hipStream_t stream, int32_t* seq_lens,
                                uint32_t* status, int32_t cap, bool advance) {
  auto kernel = splits <= 8    ? decode_reduce_kernel<4>
                : splits <= 16 ? decode_reduce_kernel<8>
                : splits <= 32 ? decode_reduce_kernel<16>
                               : decode_reduce_kernel<32>;
  hipLaunchKernelGGL(kernel, dim3(batch * hq), dim3(kReduceThreads), 0, stream, part, hq, hq / hkv,
                     splits, out, seq_lens, status, cap, advance ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, uint64_t n, hipStream_t stream) {
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
  const uint64_t pages = bytes / 4096;
  hipLaunchKernelGGL(stream_read_kernel, dim3(256 * 32), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(buf), pages, sink);
  return hipGetLastError();
}

}  // namespace mustafar
