// Internal launchers of the MUSTAFAR kernels (called by the C ABI in api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/mustafar.h"

namespace mustafar {

constexpr int kDecodeWaves = 4;        // waves per decode block
constexpr int kDecodeBlock = kDecodeWaves * 64;
constexpr int kPartStride = 132;       // floats per (unit, split, q head) partial: m, l, acc[128], pad

struct SparseDecodeArgs {
  const uint16_t* q;
  int32_t Hq, Hkv, cap, kk, vk, splits;
  const uint64_t* kbm;
  const uint16_t* kval;
  const uint32_t* ktoff;
  const uint64_t* vbm;
  const uint16_t* vval;
  const uint32_t* vtoff;
  const int32_t* seq_lens;
  float scale_log2;
  float* part;
  // fused decode step: when set, the new key and value rows [B][Hkv][128] are
  // pruned, compressed and stored as row seq_lens[b] before the attention,
  // which then covers that row too (matrix-core kernel only)
  const uint16_t* k_new;
  const uint16_t* v_new;
};

struct DenseDecodeArgs {
  const uint16_t* q;
  int32_t Hq, Hkv, splits;
  int64_t t_stride;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_lens;
  float scale_log2;
  float* part;
};

// Raises a kernel's dynamic LDS limit above the default 64 KB, once per device
// (the host call is not free, so launches skip it after the first).
template <auto Kernel>
hipError_t ensure_lds_limit(int bytes) {
  static std::atomic<uint64_t> configured{0};  // bit d: device d done (devices 0..63)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit && (configured.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) configured.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Workspace: the split partials, [batch][Hkv][splits][G][kPartStride] fp32.
inline uint64_t workspace_partial_bytes(int64_t batch, int64_t hq, int64_t splits) {
  return (uint64_t)(batch * hq * splits * kPartStride * 4);
}

hipError_t launch_prune_compress(const mustafar_kv_t& dst, const uint16_t* dense, int64_t t_stride,
                                 const int32_t* seq_lens, hipStream_t stream);
hipError_t launch_append(const mustafar_kv_t& k, const mustafar_kv_t& v, const uint16_t* k_new,
                         const uint16_t* v_new, int32_t* seq_lens, uint32_t* status,
                         hipStream_t stream);
hipError_t launch_decode_sparse(const SparseDecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_sparse_valu(const SparseDecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_dense(const DenseDecodeArgs& a, int batch, hipStream_t stream);
// Merges the split partials into out; with `advance` (a fused decode step) it
// also advances seq_lens[b] by one, or flags a full sequence in *status.
hipError_t launch_decode_reduce(const float* part, int batch, int hq, int hkv, int splits,
                                uint16_t* out, hipStream_t stream, int32_t* seq_lens = nullptr,
                                uint32_t* status = nullptr, int32_t cap = 0, bool advance = false);
hipError_t launch_zero_u32(uint32_t* p, uint64_t n, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace mustafar
