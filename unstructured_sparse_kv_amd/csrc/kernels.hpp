// Internal launchers of the MUSTAFAR kernels (called by the C ABI in api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stddef.h>

#include <atomic>

#include "../../include/mustafar.h"

namespace mustafar {

constexpr int kDecodeWaves = 4;        // waves per decode block
constexpr int kDecodeBlock = kDecodeWaves * 64;
constexpr int kPartStride = 132;       // floats per (unit, split, q head) partial: m, l, acc[128], pad
constexpr int kMaxSplits = 1024;       // sequence splits per (batch, kv head)

// Survivors per row of each kv head of one compressed tensor, and where the
// value region of (batch b, head h) starts: element cap * (b * sum + before(h)),
// which is unit * cap * keep when every head keeps `keep`.
struct KeepMap {
  int32_t keep;      // every head's keep, or the largest with per_head
  int32_t per_head;  // the tables hold each head's keep and prefix
  int32_t sum;       // keep summed over the kv heads
  uint8_t head[MUSTAFAR_MAX_HEAD_KEEP];     // keep of head h
  uint16_t before[MUSTAFAR_MAX_HEAD_KEEP];  // keep summed over heads 0 .. h-1
};

// A kernel reads its KeepMap tables through the kernel-argument segment
// pointer: indexing the by-value argument with a run-time head index would make
// the compiler copy the whole argument to scratch memory.  Every kernel that
// takes a KeepMap has one argument, a struct, which the code-object ABI places
// at offset 0 of the segment; `at` is the KeepMap's offset in that struct.
// h must be uniform across the wave (the loads are scalar).
typedef __attribute__((address_space(4))) const uint8_t kernarg_u8;
typedef __attribute__((address_space(4))) const uint32_t kernarg_u32;

// The aligned dword holding byte `at` of the kernel's argument struct, shifted
// so that byte `at` is its low byte; `at` is uniform, and so is the result.
__device__ __forceinline__ uint32_t kernarg_bytes_at(uint32_t at) {
  kernarg_u8* seg = (kernarg_u8*)__builtin_amdgcn_kernarg_segment_ptr();
  const uint32_t w = *reinterpret_cast<kernarg_u32*>(seg + (at & ~3u));
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(w >> (8u * (at & 3u))));
}

__device__ __forceinline__ int keep_of(const KeepMap& m, uint32_t at, int h) {
  if (!m.per_head) return m.keep;
  return (int)(kernarg_bytes_at(at + (uint32_t)offsetof(KeepMap, head) + (uint32_t)h) & 0xFFu);
}

__device__ __forceinline__ int64_t region_of(const KeepMap& m, uint32_t at, int64_t b, int h,
                                             int cap) {
  int64_t pre = (int64_t)h * m.keep;
  if (m.per_head)
    pre = kernarg_bytes_at(at + (uint32_t)offsetof(KeepMap, before) + 2u * (uint32_t)h) & 0xFFFFu;
  return (int64_t)cap * (b * m.sum + pre);
}

struct SparseDecodeArgs {
  const uint16_t* q;
  int32_t Hq, Hkv, cap, kk, vk, splits;  // kk, vk: the largest keep of K and V
  KeepMap kmap, vmap;
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
  uint32_t* status;  // fused step: MUSTAFAR_STATUS_BAD_OFFSETS (may be null)
};

struct PruneArgs {
  const uint16_t* dense;
  int64_t t_stride;
  const int32_t* seq_lens;
  int32_t H, cap, rows_per_unit, units;
  uint64_t* bitmaps;
  uint16_t* values;
  uint32_t* tile_off;
  KeepMap map;
  int32_t tiles_per_unit, items;  // the per-lane kernel's flattened tile order
};

struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int32_t* seq_lens;
  uint32_t* status;
  int32_t H, cap;
  uint64_t* kbm;
  uint16_t* kval;
  uint32_t* ktoff;
  uint64_t* vbm;
  uint16_t* vval;
  uint32_t* vtoff;
  KeepMap kmap, vmap;
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

// Compute units of the current device, looked up once per device.
inline hipError_t device_cu_count(int* cus) {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (c <= 0) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < 64) cached[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return hipSuccess;
}

// Workspace: the split partials, [batch][Hkv][splits][G][kPartStride] fp32.
inline uint64_t workspace_partial_bytes(int64_t batch, int64_t hq, int64_t splits) {
  return (uint64_t)(batch * hq * splits * kPartStride * 4);
}

hipError_t launch_prune_compress(const mustafar_kv_t& dst, const KeepMap& map, const uint16_t* dense,
                                 int64_t t_stride, const int32_t* seq_lens, hipStream_t stream,
                                 bool two_four = false);
hipError_t launch_prune_compress_channel(const mustafar_kv_t& dst, const KeepMap& map,
                                         const uint16_t* dense, int64_t t_stride,
                                         const int32_t* seq_lens, hipStream_t stream);
hipError_t launch_append(const mustafar_kv_t& k, const KeepMap& kmap, const mustafar_kv_t& v,
                         const KeepMap& vmap, const uint16_t* k_new, const uint16_t* v_new,
                         int32_t* seq_lens, uint32_t* status, hipStream_t stream);
hipError_t launch_decode_sparse(const SparseDecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_sparse_valu(const SparseDecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_24(const SparseDecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_dense(const DenseDecodeArgs& a, int batch, hipStream_t stream);
// Merges the split partials into out; with `advance` (a fused decode step) it
// also advances seq_lens[b] by one, or flags a full sequence in *status.
hipError_t launch_decode_reduce(const float* part, int batch, int hq, int hkv, int splits,
                                uint16_t* out, hipStream_t stream, int32_t* seq_lens = nullptr,
                                uint32_t* status = nullptr, int32_t cap = 0, bool advance = false);
hipError_t launch_zero_u32(uint32_t* p, uint64_t n, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace mustafar
