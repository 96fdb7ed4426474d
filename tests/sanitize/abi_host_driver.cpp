// Host-side driver for the sanitizer build of the library's C ABI: every
// argument check, the byte accounting and the split / workspace sizing, run
// under AddressSanitizer and UndefinedBehaviorSanitizer (api.hip's host side
// built with them, kernel launchers stubbed).  Only paths that return before a
// launch are taken: argument errors, and -- when no device is visible -- the
// MUSTAFAR_ENODEV answer to otherwise valid calls.  Expected values are the
// closed forms stated in include/mustafar.h.  Exit status 0 = every check held.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/mustafar.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

alignas(16) static uint8_t arena[1 << 16];  // stands in for device buffers: never dereferenced

static mustafar_kv_t kv_of(int B, int H, int keep, int cap, const int32_t* head_keep = nullptr) {
  mustafar_kv_t kv;
  memset(&kv, 0, sizeof(kv));
  kv.batch = B;
  kv.num_kv_heads = H;
  kv.head_dim = 128;
  kv.keep = keep;
  kv.capacity = cap;
  kv.bitmaps = reinterpret_cast<uint64_t*>(arena);
  kv.values = reinterpret_cast<uint16_t*>(arena + 4096);
  kv.tile_offsets = reinterpret_cast<uint32_t*>(arena + 8192);
  kv.head_keep = head_keep;
  return kv;
}

static void sparsity() {
  CHECK(mustafar_keep_from_sparsity(0.0, 128) == 128);
  CHECK(mustafar_keep_from_sparsity(0.5, 128) == 64);
  CHECK(mustafar_keep_from_sparsity(0.7, 128) == 38);
  CHECK(mustafar_keep_from_sparsity(1.0, 128) == 0);
  CHECK(mustafar_keep_from_sparsity(-0.01, 128) == MUSTAFAR_EINVAL);
  CHECK(mustafar_keep_from_sparsity(1.01, 128) == MUSTAFAR_EINVAL);
  CHECK(mustafar_keep_from_sparsity(NAN, 128) == MUSTAFAR_EINVAL);
  CHECK(mustafar_keep_from_sparsity(0.5, 0) == MUSTAFAR_EINVAL);
  for (int s = 0; s <= 1000; ++s) {
    const int k = mustafar_keep_from_sparsity(s / 1000.0, 128);
    CHECK(k >= 0 && k <= 128);
  }
  for (int st = -7; st <= 7; ++st) CHECK(mustafar_status_str(st) != nullptr);
}

static void accounting() {
  uint64_t nb = 0, nv = 0, no = 0;
  int64_t used = -1;
  mustafar_kv_t kv = kv_of(8, 8, 38, 32768);
  CHECK(mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no) == MUSTAFAR_OK);
  CHECK(nb == 8ull * 8 * 32768 * 16);
  CHECK(nv == 8ull * 8 * 32768 * 38 * 2 + 64);
  CHECK(no == 8ull * 8 * (32768 / 64 + 1) * 4);
  std::vector<int32_t> seq(8, 32768);
  CHECK(mustafar_kv_used_bytes(&kv, seq.data(), &used) == MUSTAFAR_OK);
  CHECK(used == 64 * (16 * 32768 + 76 * 32768 + 4 * (512 + 1)));  // 193 069 312: one tensor, keep 38
  // lengths outside [0, capacity] are clamped
  int32_t odd[8] = {-5, 0, 1, 63, 64, 65, 32768, 1 << 30};
  CHECK(mustafar_kv_used_bytes(&kv, odd, &used) == MUSTAFAR_OK);
  int64_t expect = 0;
  for (int b = 0; b < 8; ++b) {
    int64_t T = odd[b] < 0 ? 0 : (odd[b] > 32768 ? 32768 : odd[b]);
    expect += 8 * (16 * T + 2 * 38 * T + 4 * ((T + 63) / 64 + 1));
  }
  CHECK(used == expect);
  // per-head keep: sizes follow the sum of the keeps
  int32_t hk[8] = {28, 32, 34, 38, 38, 42, 44, 48};
  kv = kv_of(2, 8, 48, 128, hk);
  CHECK(mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no) == MUSTAFAR_OK);
  CHECK(nv == 2ull * 128 * (28 + 32 + 34 + 38 + 38 + 42 + 44 + 48) * 2 + 64);
  int32_t two[2] = {128, 3};
  CHECK(mustafar_kv_used_bytes(&kv, two, &used) == MUSTAFAR_OK);
  CHECK(used == 8 * (16 * 128 + 4 * 3) + 8 * (16 * 3 + 4 * 2) + 2 * (128 + 3) * 304);
  // shape errors
  kv = kv_of(8, 8, 38, 32768);
  kv.keep = 48;
  kv.head_keep = hk;  // the keep must equal the largest head keep
  kv.keep = 47;
  CHECK(mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no) == MUSTAFAR_EINVAL);
  int32_t bad_hk[8] = {28, 32, 34, 38, 38, 42, 44, 129};
  kv = kv_of(2, 8, 129, 128, bad_hk);
  CHECK(mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no) == MUSTAFAR_EINVAL);
  std::vector<int32_t> many(129, 38);
  kv = kv_of(1, 129, 38, 128, many.data());
  CHECK(mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no) == MUSTAFAR_EINVAL);
  for (int cap : {0, -64, 63, 65, (1 << 24) + 64})
    CHECK((kv = kv_of(1, 1, 38, cap), mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no)) == MUSTAFAR_EINVAL);
  CHECK((kv = kv_of(1, 1, 38, 1 << 24), mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no)) == MUSTAFAR_OK);
  // capacity * keep * 2 must stay below 2^31 (32-bit byte offsets per value region)
  CHECK((kv = kv_of(1, 1, 64, 1 << 24), mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no)) == MUSTAFAR_EINVAL);
  CHECK((kv = kv_of(1, 1, 129, 64), mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no)) == MUSTAFAR_EINVAL);
  CHECK((kv = kv_of(1, 1, -1, 64), mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no)) == MUSTAFAR_EINVAL);
  CHECK((kv = kv_of(0, 1, 38, 64), mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no)) == MUSTAFAR_EINVAL);
  CHECK((kv = kv_of(65536, 65536, 38, 64), mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no)) == MUSTAFAR_EINVAL);
  kv = kv_of(1, 1, 38, 64);
  kv.head_dim = 64;
  CHECK(mustafar_kv_alloc_bytes(&kv, &nb, &nv, &no) == MUSTAFAR_EUNSUPPORTED);
  CHECK(mustafar_kv_alloc_bytes(nullptr, &nb, &nv, &no) == MUSTAFAR_EINVAL);
  kv = kv_of(1, 1, 38, 64);
  CHECK(mustafar_kv_alloc_bytes(&kv, nullptr, &nv, &no) == MUSTAFAR_EINVAL);
  CHECK(mustafar_kv_used_bytes(&kv, nullptr, &used) == MUSTAFAR_EINVAL);
}

static void splits_and_workspace() {
  CHECK(mustafar_decode_auto_splits(8, 8, 32768) == 8);
  CHECK(mustafar_decode_auto_splits(1, 8, 16384) == 64);
  CHECK(mustafar_decode_auto_splits(1, 1, 64) == 1);
  CHECK(mustafar_decode_auto_splits(64, 8, 16384) == 1);
  CHECK(mustafar_decode_auto_splits(0, 8, 64) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_auto_splits(1, 8, -1) == MUSTAFAR_EINVAL);
  for (int T : {0, 1, 63, 64, 65, 4096, 1 << 24}) {
    const int s = mustafar_decode_auto_splits(1, 1, T);
    CHECK(s >= 1 && s <= 1024);
  }
  uint64_t ws = 0;
  CHECK(mustafar_decode_workspace_bytes(8, 32, 8, 128, 32768, 0, &ws) == MUSTAFAR_OK);
  CHECK(ws == 8ull * 32 * 8 * 132 * 4);
  CHECK(mustafar_decode_workspace_bytes(8, 32, 8, 64, 32768, 0, &ws) == MUSTAFAR_EUNSUPPORTED);
  CHECK(mustafar_decode_workspace_bytes(8, 30, 8, 128, 32768, 0, &ws) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_workspace_bytes(8, 32, 8, 128, 32768, 1025, &ws) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_workspace_bytes(8, 32, 8, 128, 32768, 0, nullptr) == MUSTAFAR_EINVAL);
}

static void call_errors(bool have_device) {
  mustafar_kv_t k = kv_of(2, 2, 38, 128), v = kv_of(2, 2, 38, 128);
  const uint16_t* dense = reinterpret_cast<const uint16_t*>(arena + 16384);
  const uint16_t* q = reinterpret_cast<const uint16_t*>(arena + 20480);
  uint16_t* out = reinterpret_cast<uint16_t*>(arena + 24576);
  void* ws = arena + 32768;
  int32_t* seq = reinterpret_cast<int32_t*>(arena + 28672);
  uint32_t* status = reinterpret_cast<uint32_t*>(arena + 28800);
  const uint16_t* mis = reinterpret_cast<const uint16_t*>(arena + 16386);  // 2-byte aligned only
  const uint64_t wsb = 1 << 14;
  const float sc = 0.0883883f;
  // prune / append argument errors
  CHECK(mustafar_prune_compress(nullptr, dense, 128, seq, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_prune_compress(&k, nullptr, 128, seq, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_prune_compress(&k, mis, 128, seq, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_prune_compress(&k, dense, 0, seq, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_prune_compress_channel(&k, dense, 128, nullptr, nullptr) == MUSTAFAR_EINVAL);
  mustafar_kv_t odd = kv_of(2, 2, 37, 128);
  CHECK(mustafar_prune_compress_channel(&odd, dense, 128, seq, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_prune_compress_24(&k, dense, 128, seq, nullptr) == MUSTAFAR_EINVAL);  // keep != 64
  mustafar_kv_t other = kv_of(3, 2, 38, 128);
  CHECK(mustafar_append_token(&k, &other, dense, dense, seq, status, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_append_token(&k, &v, dense, mis, seq, status, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_append_token(&k, &v, dense, dense, nullptr, status, nullptr) == MUSTAFAR_EINVAL);
  mustafar_kv_t misk = k;
  misk.values = reinterpret_cast<uint16_t*>(arena + 4098);
  CHECK(mustafar_append_token(&misk, &v, dense, dense, seq, status, nullptr) == MUSTAFAR_EINVAL);
  // decode argument errors
  CHECK(mustafar_decode_attn(q, 8, &k, &v, seq, 128, sc, 0, out, nullptr, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_attn(q, 7, &k, &v, seq, 128, sc, 0, out, ws, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_attn(q, 6, &k, &v, seq, 128, sc, 0, out, ws, wsb, nullptr) == MUSTAFAR_EUNSUPPORTED);
  CHECK(mustafar_decode_attn(q, 32, &k, &v, seq, 128, sc, 0, out, ws, wsb, nullptr) == MUSTAFAR_EUNSUPPORTED);
  CHECK(mustafar_decode_attn(q, 8, &k, &v, seq, 128, NAN, 0, out, ws, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_attn(q, 8, &k, &v, seq, 128, sc, 1025, out, ws, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_attn(q, 8, &k, &v, seq, -1, sc, 0, out, ws, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_attn(q, 8, &k, &v, seq, 128, sc, 0, out, ws, 16, nullptr) == MUSTAFAR_ENOSPACE);
  CHECK(mustafar_decode_attn(q, 8, &k, &other, seq, 128, sc, 0, out, ws, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_attn_valu(mis, 8, &k, &v, seq, 128, sc, 0, out, ws, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_attn_24(q, 8, &k, &v, seq, 128, sc, 0, out, ws, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_step(q, 8, &k, &v, nullptr, dense, seq, status, 128, sc, 0, out, ws, wsb,
                             nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_dense_decode_attn(q, 8, dense, dense, 2, 2, 64, 128, seq, 128, sc, 0, out, ws, wsb,
                                   nullptr) == MUSTAFAR_EUNSUPPORTED);
  CHECK(mustafar_dense_decode_attn(q, 8, dense, mis, 2, 2, 128, 128, seq, 128, sc, 0, out, ws, wsb,
                                   nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_dense_decode_attn(q, 8, dense, dense, 2, 2, 128, int64_t(1) << 30, seq, 128, sc, 0, out,
                                   ws, wsb, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_decode_workspace_init(ws, 6, nullptr) == MUSTAFAR_EINVAL);
  CHECK(mustafar_probe_stream_read(ws, 100, status, nullptr) == MUSTAFAR_EINVAL);
  if (!have_device) {  // valid calls: no device here
    CHECK(mustafar_prune_compress(&k, dense, 128, seq, nullptr) == MUSTAFAR_ENODEV);
    CHECK(mustafar_append_token(&k, &v, dense, dense, seq, status, nullptr) == MUSTAFAR_ENODEV);
    CHECK(mustafar_decode_attn(q, 8, &k, &v, seq, 128, sc, 0, out, ws, wsb, nullptr) == MUSTAFAR_ENODEV);
    CHECK(mustafar_decode_step(q, 8, &k, &v, dense, dense, seq, status, 128, sc, 0, out, ws, wsb,
                               nullptr) == MUSTAFAR_ENODEV);
    CHECK(mustafar_dense_decode_attn(q, 8, dense, dense, 2, 2, 128, 128, seq, 128, sc, 0, out, ws, wsb,
                                     nullptr) == MUSTAFAR_ENODEV);
    CHECK(mustafar_decode_step_noalloc(q, 8, &k, &v, dense, dense, seq, status, 128, sc, 0, out,
                                       nullptr) == MUSTAFAR_ENODEV);
  }
  // the no-alloc step refuses partials beyond its scratch array before any device call
  mustafar_kv_t kb = kv_of(256, 8, 38, 64), vb = kv_of(256, 8, 38, 64);
  CHECK(mustafar_decode_step_noalloc(q, 64, &kb, &vb, dense, dense, seq, status, 64, sc, 0, out,
                                     nullptr) == MUSTAFAR_ENOSPACE);
  CHECK(mustafar_decode_step_noalloc(q, 8, &k, &v, nullptr, dense, seq, status, 128, sc, 0, out,
                                     nullptr) == MUSTAFAR_EINVAL);
}

int main() {
  int n = 0;
  const bool have_device = hipGetDeviceCount(&n) == hipSuccess && n > 0;
  (void)hipGetLastError();
  sparsity();
  accounting();
  splits_and_workspace();
  call_errors(have_device);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi host checks: all passed (device visible: %s)\n", have_device ? "yes" : "no");
  return 0;
}
