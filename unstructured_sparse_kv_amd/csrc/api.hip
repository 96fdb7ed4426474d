// C ABI of the MUSTAFAR library: host-side argument checks, launch geometry,
// workspace sizing and byte accounting.  Every check runs before any HIP call,
// so argument errors are reported without a device.
#include <math.h>
#include <string.h>

#include <atomic>

#include "device_common.hpp"
#include "kernels.hpp"

using namespace mustafar;

// Split partials of mustafar_decode_step_noalloc: a file-scope device array, so
// that the call allocates nothing.  Each device holds its own copy (from module
// load until the process ends) at its own address.  In host code the name is a
// host-side stand-in, never a device address: only the per-device pointer that
// hipGetSymbolAddress returns (scratch_of_current_device) is ever passed on.
static __device__ __align__(256) uint8_t scratch[MUSTAFAR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device (with that
// device current) and kept.
int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return MUSTAFAR_ENODEV;
  }
  if (dev < 0 || dev >= kMaxDevices) return MUSTAFAR_EUNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return MUSTAFAR_ELAUNCH;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MUSTAFAR_OK;
}

constexpr int64_t kMaxCapacity = 1 << 24;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Survivors per row of each kv head: head_keep[h] when the caller gives
// per-head keeps (keep must then be their maximum), else keep for every head.
int make_keep_map(const mustafar_kv_t* kv, KeepMap* m) {
  memset(m, 0, sizeof(*m));
  m->keep = kv->keep;
  if (!kv->head_keep) {
    const int64_t sum = (int64_t)kv->num_kv_heads * kv->keep;
    if (sum > INT32_MAX) return MUSTAFAR_EINVAL;
    m->sum = (int32_t)sum;
    return MUSTAFAR_OK;
  }
  if (kv->num_kv_heads > MUSTAFAR_MAX_HEAD_KEEP) return MUSTAFAR_EINVAL;
  int most = 0, sum = 0;
  for (int h = 0; h < kv->num_kv_heads; ++h) {
    const int k = kv->head_keep[h];
    if (k < 0 || k > kv->head_dim) return MUSTAFAR_EINVAL;
    m->head[h] = (uint8_t)k;
    m->before[h] = (uint16_t)sum;
    sum += k;
    most = k > most ? k : most;
  }
  if (most != kv->keep) return MUSTAFAR_EINVAL;
  m->per_head = 1;
  m->sum = sum;
  return MUSTAFAR_OK;
}

int check_kv_shape(const mustafar_kv_t* kv, KeepMap* map_out = nullptr) {
  if (!kv) return MUSTAFAR_EINVAL;
  if (kv->batch <= 0 || kv->num_kv_heads <= 0) return MUSTAFAR_EINVAL;
  if ((int64_t)kv->batch * kv->num_kv_heads > INT32_MAX) return MUSTAFAR_EINVAL;  // unit index is 32-bit
  if (kv->head_dim <= 0) return MUSTAFAR_EINVAL;
  if (kv->head_dim != kHeadDim) return MUSTAFAR_EUNSUPPORTED;
  if (kv->keep < 0 || kv->keep > kv->head_dim) return MUSTAFAR_EINVAL;
  if (kv->capacity <= 0 || kv->capacity % 64 != 0 || kv->capacity > kMaxCapacity)
    return MUSTAFAR_EINVAL;
  // per-(batch, head) value region must be addressable with 32-bit byte offsets
  if ((int64_t)kv->capacity * kv->keep * 2 >= (int64_t)1 << 31) return MUSTAFAR_EINVAL;
  KeepMap m;
  const int rc = make_keep_map(kv, &m);
  if (rc) return rc;
  if (map_out) *map_out = m;
  return MUSTAFAR_OK;
}

int check_kv(const mustafar_kv_t* kv, KeepMap* map_out = nullptr) {
  int rc = check_kv_shape(kv, map_out);
  if (rc) return rc;
  if (!kv->bitmaps || !kv->values || !kv->tile_offsets) return MUSTAFAR_EINVAL;
  if (!aligned16(kv->bitmaps) || !aligned16(kv->values) || !aligned4(kv->tile_offsets))
    return MUSTAFAR_EINVAL;
  return MUSTAFAR_OK;
}

int check_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return MUSTAFAR_ENODEV;
  }
  return MUSTAFAR_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? MUSTAFAR_OK : MUSTAFAR_ELAUNCH; }

// Sequence splits per (batch, kv head) when the caller passes 0: as many 4-wave
// blocks as fill the device once without a partial second round -- two per
// compute unit for the sparse kernels (their LDS footprint allows two), one
// for the dense kernel (measured fastest) -- with at least one 64-row tile
// per wave.
int auto_splits(int64_t batch, int64_t hkv, int64_t max_seq_len, int64_t target_blocks = 512) {
  const int64_t units = batch * hkv;
  const int64_t tiles = (max_seq_len + 63) / 64;
  int64_t s = target_blocks / units;
  const int64_t most = (tiles + kDecodeWaves - 1) / kDecodeWaves;  // >= 1 tile per wave
  if (s > most) s = most;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return (int)s;
}

int decode_common_checks(const uint16_t* q, int32_t hq, int32_t batch, int32_t hkv, int32_t max_seq_len,
                         float scale, int32_t splits, const uint16_t* out, const void* ws,
                         uint64_t ws_bytes, const int32_t* seq_lens, int* splits_out,
                         int64_t target_blocks = 512) {
  if (!q || !out || !ws || !seq_lens) return MUSTAFAR_EINVAL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws) || !aligned4(seq_lens))
    return MUSTAFAR_EINVAL;
  if (hq <= 0 || hkv <= 0 || batch <= 0) return MUSTAFAR_EINVAL;
  if (hq % hkv != 0) return MUSTAFAR_EINVAL;
  const int g = hq / hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8) return MUSTAFAR_EUNSUPPORTED;
  if (max_seq_len < 0 || splits < 0 || splits > kMaxSplits) return MUSTAFAR_EINVAL;
  if (!isfinite(scale)) return MUSTAFAR_EINVAL;
  if (batch > 65535 || hkv > 65535) return MUSTAFAR_EINVAL;  // grid z and y
  const int sp = splits ? splits : auto_splits(batch, hkv, max_seq_len, target_blocks);
  const uint64_t need = workspace_partial_bytes(batch, hq, sp);
  if (ws_bytes < need) return MUSTAFAR_ENOSPACE;
  *splits_out = sp;
  return MUSTAFAR_OK;
}

typedef hipError_t (*SparseLauncher)(const SparseDecodeArgs&, int, hipStream_t);

// Decode over the compressed caches; with k_new / v_new (the fused step) the
// split kernel first stores the new rows and the merge kernel advances seq_lens.
// workspace == kUseScratch: the partials go to the library's scratch array
// (workspace_bytes is then its size), looked up after the argument checks.
void* const kUseScratch = reinterpret_cast<void*>(uintptr_t{256});

int sparse_decode(SparseLauncher launch, const uint16_t* q, int32_t num_q_heads,
                  const mustafar_kv_t* k, const mustafar_kv_t* v, const int32_t* seq_lens,
                  int32_t max_seq_len, float scale, int32_t splits, uint16_t* out,
                  void* workspace, uint64_t workspace_bytes, void* stream,
                  const uint16_t* k_new = nullptr, const uint16_t* v_new = nullptr,
                  uint32_t* status = nullptr) {
  SparseDecodeArgs a;
  int rc = check_kv(k, &a.kmap);
  if (rc) return rc;
  if ((rc = check_kv(v, &a.vmap))) return rc;
  if (k->batch != v->batch || k->num_kv_heads != v->num_kv_heads || k->capacity != v->capacity)
    return MUSTAFAR_EINVAL;
  int sp = 0;
  rc = decode_common_checks(q, num_q_heads, k->batch, k->num_kv_heads, max_seq_len, scale, splits,
                            out, workspace, workspace_bytes, seq_lens, &sp);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  if (workspace == kUseScratch && (rc = scratch_of_current_device(&workspace))) return rc;
  a.q = q;
  a.Hq = num_q_heads;
  a.Hkv = k->num_kv_heads;
  a.cap = k->capacity;
  a.kk = k->keep;
  a.vk = v->keep;
  a.splits = sp;
  a.kbm = k->bitmaps;
  a.kval = k->values;
  a.ktoff = k->tile_offsets;
  a.vbm = v->bitmaps;
  a.vval = v->values;
  a.vtoff = v->tile_offsets;
  a.seq_lens = seq_lens;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  a.part = (float*)workspace;
  a.k_new = k_new;
  a.v_new = v_new;
  a.status = status;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = launched(launch(a, k->batch, st)))) return rc;
  return launched(launch_decode_reduce(a.part, k->batch, num_q_heads, k->num_kv_heads, sp, out, st,
                                       const_cast<int32_t*>(seq_lens), status, k->capacity,
                                       k_new != nullptr));
}

}  // namespace

extern "C" {

const char* mustafar_status_str(int status) {
  switch (status) {
    case MUSTAFAR_OK: return "ok";
    case MUSTAFAR_EINVAL: return "invalid argument";
    case MUSTAFAR_EUNSUPPORTED: return "unsupported configuration";
    case MUSTAFAR_ENODEV: return "no HIP device";
    case MUSTAFAR_ELAUNCH: return "kernel launch failed";
    case MUSTAFAR_ENOSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

int mustafar_keep_from_sparsity(double sparsity, int32_t head_dim) {
  if (!(sparsity >= 0.0 && sparsity <= 1.0) || head_dim <= 0) return MUSTAFAR_EINVAL;
  int k = (int)floor((1.0 - sparsity) * (double)head_dim + 0.5);
  if (k < 0) k = 0;
  if (k > head_dim) k = head_dim;
  return k;
}

int mustafar_kv_alloc_bytes(const mustafar_kv_t* kv, uint64_t* bitmaps_bytes,
                            uint64_t* values_bytes, uint64_t* offsets_bytes) {
  KeepMap m;
  const int rc = check_kv_shape(kv, &m);
  if (rc) return rc;
  if (!bitmaps_bytes || !values_bytes || !offsets_bytes) return MUSTAFAR_EINVAL;
  const uint64_t units = (uint64_t)kv->batch * kv->num_kv_heads;
  *bitmaps_bytes = units * kv->capacity * (kv->head_dim / 64) * 8;
  *values_bytes = (uint64_t)kv->batch * kv->capacity * (uint64_t)m.sum * 2 + 64;
  *offsets_bytes = units * (kv->capacity / 64 + 1) * 4;
  return MUSTAFAR_OK;
}

int mustafar_kv_used_bytes(const mustafar_kv_t* kv, const int32_t* seq_lens_host, int64_t* bytes) {
  KeepMap m;
  const int rc = check_kv_shape(kv, &m);
  if (rc) return rc;
  if (!seq_lens_host || !bytes) return MUSTAFAR_EINVAL;
  int64_t total = 0;
  for (int b = 0; b < kv->batch; ++b) {
    int64_t T = seq_lens_host[b];
    T = T < 0 ? 0 : (T > kv->capacity ? kv->capacity : T);
    total += (int64_t)kv->num_kv_heads * (T * (kv->head_dim / 8) + 4 * ((T + 63) / 64 + 1)) +
             2 * T * (int64_t)m.sum;
  }
  *bytes = total;
  return MUSTAFAR_OK;
}

int mustafar_prune_compress(const mustafar_kv_t* dst, const uint16_t* dense, int64_t t_stride,
                            const int32_t* seq_lens, void* stream) {
  KeepMap m;
  int rc = check_kv(dst, &m);
  if (rc) return rc;
  if (!dense || !seq_lens || !aligned16(dense) || !aligned4(seq_lens)) return MUSTAFAR_EINVAL;
  if (t_stride <= 0 || t_stride > kMaxCapacity * 64) return MUSTAFAR_EINVAL;
  if ((rc = check_device())) return rc;
  return launched(launch_prune_compress(*dst, m, dense, t_stride, seq_lens, (hipStream_t)stream));
}

int mustafar_prune_compress_channel(const mustafar_kv_t* dst, const uint16_t* dense,
                                    int64_t t_stride, const int32_t* seq_lens, void* stream) {
  KeepMap m;
  int rc = check_kv(dst, &m);
  if (rc) return rc;
  if (dst->keep % 2 != 0 || dst->head_keep) return MUSTAFAR_EINVAL;
  if (!dense || !seq_lens || !aligned16(dense) || !aligned4(seq_lens)) return MUSTAFAR_EINVAL;
  if (t_stride <= 0 || t_stride > kMaxCapacity * 64) return MUSTAFAR_EINVAL;
  if ((rc = check_device())) return rc;
  return launched(
      launch_prune_compress_channel(*dst, m, dense, t_stride, seq_lens, (hipStream_t)stream));
}

int mustafar_prune_compress_24(const mustafar_kv_t* dst, const uint16_t* dense, int64_t t_stride,
                               const int32_t* seq_lens, void* stream) {
  KeepMap m;
  int rc = check_kv(dst, &m);
  if (rc) return rc;
  if (dst->keep != kHeadDim / 2 || dst->head_keep) return MUSTAFAR_EINVAL;
  if (!dense || !seq_lens || !aligned16(dense) || !aligned4(seq_lens)) return MUSTAFAR_EINVAL;
  if (t_stride <= 0 || t_stride > kMaxCapacity * 64) return MUSTAFAR_EINVAL;
  if ((rc = check_device())) return rc;
  return launched(
      launch_prune_compress(*dst, m, dense, t_stride, seq_lens, (hipStream_t)stream, true));
}

int mustafar_append_token(const mustafar_kv_t* k, const mustafar_kv_t* v, const uint16_t* k_new,
                          const uint16_t* v_new, int32_t* seq_lens, uint32_t* status,
                          void* stream) {
  KeepMap km, vm;
  int rc = check_kv(k, &km);
  if (rc) return rc;
  if ((rc = check_kv(v, &vm))) return rc;
  if (k->batch != v->batch || k->num_kv_heads != v->num_kv_heads || k->capacity != v->capacity)
    return MUSTAFAR_EINVAL;
  if (!k_new || !v_new || !seq_lens) return MUSTAFAR_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned4(seq_lens)) return MUSTAFAR_EINVAL;
  if (status && !aligned4(status)) return MUSTAFAR_EINVAL;
  if (k->batch > 65535) return MUSTAFAR_EINVAL;
  if ((rc = check_device())) return rc;
  return launched(launch_append(*k, km, *v, vm, k_new, v_new, seq_lens, status, (hipStream_t)stream));
}

int mustafar_decode_auto_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  if (batch <= 0 || num_kv_heads <= 0 || max_seq_len < 0) return MUSTAFAR_EINVAL;
  return auto_splits(batch, num_kv_heads, max_seq_len);
}

int mustafar_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_seq_len, int32_t splits,
                                    uint64_t* bytes) {
  if (!bytes || batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
      splits < 0 || splits > kMaxSplits)
    return MUSTAFAR_EINVAL;
  if (head_dim != kHeadDim) return MUSTAFAR_EUNSUPPORTED;
  if (num_q_heads % num_kv_heads != 0) return MUSTAFAR_EINVAL;
  const int sp = splits ? splits : auto_splits(batch, num_kv_heads, max_seq_len);
  *bytes = workspace_partial_bytes(batch, num_q_heads, sp);
  return MUSTAFAR_OK;
}

int mustafar_decode_workspace_init(void* workspace, uint64_t bytes, void* stream) {
  if (!workspace || !aligned16(workspace) || bytes == 0 || bytes % 4 != 0) return MUSTAFAR_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  return launched(launch_zero_u32((uint32_t*)workspace, bytes / 4, (hipStream_t)stream));
}

int mustafar_decode_attn(const uint16_t* q, int32_t num_q_heads, const mustafar_kv_t* k,
                         const mustafar_kv_t* v, const int32_t* seq_lens, int32_t max_seq_len,
                         float scale, int32_t splits, uint16_t* out, void* workspace,
                         uint64_t workspace_bytes, void* stream) {
  return sparse_decode(launch_decode_sparse, q, num_q_heads, k, v, seq_lens, max_seq_len, scale,
                       splits, out, workspace, workspace_bytes, stream);
}

int mustafar_decode_attn_valu(const uint16_t* q, int32_t num_q_heads, const mustafar_kv_t* k,
                              const mustafar_kv_t* v, const int32_t* seq_lens, int32_t max_seq_len,
                              float scale, int32_t splits, uint16_t* out, void* workspace,
                              uint64_t workspace_bytes, void* stream) {
  return sparse_decode(launch_decode_sparse_valu, q, num_q_heads, k, v, seq_lens, max_seq_len,
                       scale, splits, out, workspace, workspace_bytes, stream);
}

int mustafar_decode_attn_24(const uint16_t* q, int32_t num_q_heads, const mustafar_kv_t* k,
                            const mustafar_kv_t* v, const int32_t* seq_lens, int32_t max_seq_len,
                            float scale, int32_t splits, uint16_t* out, void* workspace,
                            uint64_t workspace_bytes, void* stream) {
  for (const mustafar_kv_t* c : {k, v})
    if (c && (c->keep != kHeadDim / 2 || c->head_keep)) return MUSTAFAR_EINVAL;
  return sparse_decode(launch_decode_24, q, num_q_heads, k, v, seq_lens, max_seq_len, scale,
                       splits, out, workspace, workspace_bytes, stream);
}

int mustafar_decode_step(const uint16_t* q, int32_t num_q_heads, const mustafar_kv_t* k,
                         const mustafar_kv_t* v, const uint16_t* k_new, const uint16_t* v_new,
                         int32_t* seq_lens, uint32_t* status, int32_t max_seq_len, float scale,
                         int32_t splits, uint16_t* out, void* workspace, uint64_t workspace_bytes,
                         void* stream) {
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return MUSTAFAR_EINVAL;
  if (status && !aligned4(status)) return MUSTAFAR_EINVAL;
  return sparse_decode(launch_decode_sparse, q, num_q_heads, k, v, seq_lens, max_seq_len, scale,
                       splits, out, workspace, workspace_bytes, stream, k_new, v_new, status);
}

int mustafar_decode_step_noalloc(const uint16_t* q, int32_t num_q_heads, const mustafar_kv_t* k,
                                 const mustafar_kv_t* v, const uint16_t* k_new, const uint16_t* v_new,
                                 int32_t* seq_lens, uint32_t* status, int32_t max_seq_len,
                                 float scale, int32_t splits, uint16_t* out, void* stream) {
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return MUSTAFAR_EINVAL;
  if (status && !aligned4(status)) return MUSTAFAR_EINVAL;
  return sparse_decode(launch_decode_sparse, q, num_q_heads, k, v, seq_lens, max_seq_len, scale,
                       splits, out, kUseScratch, MUSTAFAR_NOALLOC_SCRATCH_BYTES, stream, k_new,
                       v_new, status);
}

int mustafar_dense_decode_attn(const uint16_t* q, int32_t num_q_heads, const uint16_t* k,
                               const uint16_t* v, int32_t batch, int32_t num_kv_heads,
                               int32_t head_dim, int64_t t_stride, const int32_t* seq_lens,
                               int32_t max_seq_len, float scale, int32_t splits, uint16_t* out,
                               void* workspace, uint64_t workspace_bytes, void* stream) {
  if (!k || !v || !aligned16(k) || !aligned16(v)) return MUSTAFAR_EINVAL;
  if (head_dim <= 0) return MUSTAFAR_EINVAL;
  if (head_dim != kHeadDim) return MUSTAFAR_EUNSUPPORTED;
  if (t_stride <= 0 || t_stride * kHeadDim * 2 >= ((int64_t)1 << 32)) return MUSTAFAR_EINVAL;
  int sp = 0;
  int rc = decode_common_checks(q, num_q_heads, batch, num_kv_heads, max_seq_len, scale, splits,
                                out, workspace, workspace_bytes, seq_lens, &sp, 256);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  DenseDecodeArgs a;
  a.q = q;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.splits = sp;
  a.t_stride = t_stride;
  a.k = k;
  a.v = v;
  a.seq_lens = seq_lens;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.part = (float*)workspace;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = launched(launch_decode_dense(a, batch, st)))) return rc;
  return launched(launch_decode_reduce(a.part, batch, num_q_heads, num_kv_heads, sp, out, st));
}

int mustafar_probe_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || !aligned16(buf) || !aligned4(sink)) return MUSTAFAR_EINVAL;
  if (bytes < 4096 || bytes % 4096 != 0) return MUSTAFAR_EINVAL;
  int rc = check_device();
  if (rc) return rc;
  return launched(launch_stream_read(buf, bytes, sink, (hipStream_t)stream));
}

}  // extern "C"
