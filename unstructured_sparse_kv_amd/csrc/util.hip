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
// (0 for an empty sequence).  The 256 threads first take the maximum over the
// splits together; then thread t sums channel t % 128 over the splits of
// parity t / 128, with the loop unrolled so that several splits' loads are in
// flight at once (the partials were just written and sit in the L2), and the
// two halves are added in LDS.
constexpr int kReduceThreads = 2 * kHeadDim;

__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(
    const float* __restrict__ part, int hq_total, int g_size, int splits, uint16_t* __restrict__ out,
    int32_t* seq_lens, uint32_t* status, int32_t cap, int advance) {
  __shared__ float red[kReduceThreads / kWave];
  __shared__ float half_a[kHeadDim];
  __shared__ float half_l;
  const int bq = blockIdx.x;
  const int b = bq / hq_total, hq = bq % hq_total;
  const int hkv = hq_total / g_size;
  const int h = hq / g_size, g = hq % g_size;
  const int unit = b * hkv + h;
  const int t = threadIdx.x, c = t % kHeadDim, par = t / kHeadDim;
  const float ninf = -__builtin_inff();
  const float* pu = part + ((int64_t)unit * splits * g_size + g) * kPartStride;
  const int64_t sstride = (int64_t)g_size * kPartStride;

  float mx = ninf;
  for (int s = t; s < splits; s += kReduceThreads) mx = fmaxf(mx, pu[s * sstride]);
  mx = wave_max(mx);
  if (lane_id() == 0) red[t / kWave] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / kWave; ++w) M = fmaxf(M, red[w]);

  float A = 0.f, L = 0.f;
#pragma unroll 8
  for (int s = par; s < splits; s += 2) {
    const float* ps = pu + s * sstride;
    const float ms = ps[0];
    const float f = (ms == ninf) ? 0.f : exp2f(ms - M);
    A += ps[2 + c] * f;
    L += ps[1] * f;
  }
  if (par == 1) {
    half_a[c] = A;
    if (c == 0) half_l = L;
  }
  __syncthreads();
  if (par == 0) {
    A += half_a[c];
    L += half_l;
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
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(batch * hq), dim3(kReduceThreads), 0, stream, part, hq,
                     hq / hkv, splits, out, seq_lens, status, cap, advance ? 1 : 0);
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
