// MUSTAFAR hot path: CPU oracle.
//
// TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
// definition that the HIP library is checked against.  Only the tests, the
// smoke check and the benchmark's CPU-baseline leg may load it; the product
// path never does.  It shares no code, header, table or helper with the HIP
// library: its fp16 decoder, its top-k rule, its encoder and its attention are
// written here from their definitions, in fp64 for floating point and exact
// integers for everything else.
//
// Sources (web pages; cited by title and section):
//   [Summary]  "MUSTAFAR: Promoting Unstructured Sparsity for KV Cache Pruning
//              in LLM Inference", AI-written paper summary (research map page),
//              sections "Approach", "Key results", "Limitations".
//   [README]   "Mustafar: Promoting Unstructured Sparsity for KV Cache Pruning
//              in LLM Inference", repository README mirror, sections
//              "Part II: LongBench Evaluation", "Part III: Kernel Evaluation".
//   [Abstract] "Mustafar: Promoting Unstructured Sparsity for KV Cache Pruning
//              in LLM Inference", author abstract (author page).
//
// Readings where the pages are silent (each one also listed in the design doc):
//   R1 pruning unit: one (batch, kv-head, token) row of head_dim channels.
//   R2 survivors k = floor((1 - s) * d + 0.5), clamped to [0, d].
//   R3 magnitude: |x| of the fp16 value, compared through bits & 0x7FFF.
//   R4 ties: the lower channel index survives.
//   R5 the bitmap marks the k selected channels (so popcount == k).
//   R6 layout: two 64-bit words per 128-channel row, bit j of word w is
//      channel 64w + j; kept values in ascending channel order; one u32
//      offset per 64-row tile (plus an end entry).
//   R7 a pruned entry decompresses to +0.0.
//   R8 attention scale is passed in (1/sqrt(d) in the tests).
//   R9 q head hq reads kv head floor(hq / (Hq / Hkv)).
//   R14 an empty sequence gives an all-zero output.
//   R23 2:4 comparator: channels 4j..4j+3 of a row form a group; the 2 of
//       largest magnitude survive (ties to the lower channel), stored in the
//       same bitmap format with keep = d / 2.
//   R24 channel-wise pruning: in every full 64-row tile of a (b, h), each
//       channel keeps its keep/2 entries of largest magnitude over the tile's
//       rows (ties to the earlier row); rows of a final partial tile are pruned
//       per token to keep.  Same bitmap format; rows hold 0..d values.
//   R22 per-head keep: kv head h keeps head_keep[h] channels per row; the
//       values of (batch b, head h) start at element cap * (b * S + P_h),
//       S = the sum of head_keep over the heads, P_h = the sum over heads
//       before h (the uniform layout when every head keeps the same k).
//
// Parity status: every function here is pinned by the CPU tests (fp16
// decoder: exhaustive against IEEE-754 binary16; prune: brute force over all
// k-subsets and hand-worked fixtures; encode/decode: round trip and closed-form
// sizes; attention: torch's scaled_dot_product_attention in fp64, closed forms
// T=1 and q=0, GQA == MHA with repeated heads).  The pages print no worked
// example, so nothing here is pinned to a value printed on the pages.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

namespace {

// IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double half_to_double(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 0) {
    v = std::ldexp(static_cast<double>(m), -24);  // subnormal: m * 2^-24
  } else if (e == 31) {
    v = m ? std::nan("") : INFINITY;
  } else {
    v = std::ldexp(static_cast<double>(1024 + m), e - 25);  // (1 + m/2^10) * 2^(e-15)
  }
  return sign ? -v : v;
}

// R3: magnitude key of an fp16 value.  For finite values the ordering of
// (bits & 0x7FFF) as an unsigned integer is the ordering of |x|, and -0 == +0.
inline uint16_t mag_key(uint16_t h) { return static_cast<uint16_t>(h & 0x7FFF); }

// Per-token magnitude pruning of one row ([Summary] "Approach"; [Abstract];
// the token-wise, magnitude-based variant named in [README] "Part II"):
// keep the k channels of largest magnitude, ties to the lower channel (R4).
// Written as: stable sort of the channel indices by key, descending; the
// first k are the survivors.
void prune_row(const uint16_t* x, int d, int k, uint8_t* keep) {
  std::vector<int> idx(d);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int a, int b) { return mag_key(x[a]) > mag_key(x[b]); });
  std::memset(keep, 0, d);
  for (int i = 0; i < k && i < d; ++i) keep[idx[i]] = 1;
}

// 2:4 semi-structured pruning of one row (R23), a baseline the pages list
// ([Summary] "Experimental setup") and the structured kind of sparsity they
// argue against ([Abstract]): in every group of 4
// consecutive channels keep the 2 of largest magnitude, ties to the lower
// channel -- the per-token rule above applied to each group with k = 2.
void prune_row_24(const uint16_t* x, int d, uint8_t* keep) {
  for (int g = 0; g + 4 <= d; g += 4) prune_row(x + g, 4, 2, keep + g);
}

int clamp_len(int32_t t, int64_t cap) {
  if (t < 0) return 0;
  return static_cast<int>(std::min<int64_t>(t, cap));
}

template <class F>
void parallel_for(int64_t n, int nthreads, F&& f) {
  if (nthreads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  nthreads = static_cast<int>(std::min<int64_t>(nthreads, n));
  std::vector<std::thread> th;
  for (int w = 0; w < nthreads; ++w) {
    th.emplace_back([&, w] {
      for (int64_t i = w; i < n; i += nthreads) f(i);
    });
  }
  for (auto& t : th) t.join();
}

int hw_threads() {
  unsigned n = std::thread::hardware_concurrency();
  return n ? static_cast<int>(n) : 1;
}

// R22: survivors per row of each kv head and where each (b, h) value region
// starts.  head_keep == nullptr means every head keeps k.
struct Layout {
  std::vector<int64_t> keep, before;
  int64_t sum = 0, cap = 0;
  int64_t region(int64_t b, int64_t h) const { return cap * (b * sum + before[h]); }
};

bool make_layout(int H, const int32_t* head_keep, int k, int d, int64_t cap, Layout* L) {
  L->keep.assign(H, k);
  L->before.assign(H, 0);
  L->cap = cap;
  L->sum = 0;
  for (int h = 0; h < H; ++h) {
    if (head_keep) L->keep[h] = head_keep[h];
    if (L->keep[h] < 0 || L->keep[h] > d) return false;
    L->before[h] = L->sum;
    L->sum += L->keep[h];
  }
  return true;
}

}  // namespace

extern "C" {

double orc_half_to_double(uint16_t h) { return half_to_double(h); }

void orc_half_to_double_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = half_to_double(h[i]);
}

int orc_hardware_threads(void) { return hw_threads(); }

// R2: survivors per row for a pruned fraction s ([README] "Part II": the
// target sparsity is the fraction pruned, 0.5 or 0.7).  -1 for s outside [0,1].
int orc_keep_from_sparsity(double s, int d) {
  if (!(s >= 0.0 && s <= 1.0) || d <= 0) return -1;
  const double x = (1.0 - s) * static_cast<double>(d);
  int k = static_cast<int>(std::floor(x + 0.5));
  if (k < 0) k = 0;
  if (k > d) k = d;
  return k;
}

// Prune n rows of d channels; keep[r*d + c] = 1 for survivors.
void orc_prune_rows(const uint16_t* x, int64_t n, int d, int k, uint8_t* keep) {
  for (int64_t r = 0; r < n; ++r) prune_row(x + r * d, d, k, keep + r * d);
}

// The same with the 2:4 rule (R23); d must be a multiple of 4.
int orc_prune_rows_24(const uint16_t* x, int64_t n, int d, uint8_t* keep) {
  if (d <= 0 || d % 4 != 0) return -1;
  for (int64_t r = 0; r < n; ++r) prune_row_24(x + r * d, d, keep + r * d);
  return 0;
}

// Compress a dense cache [B][H][t_stride][d] (fp16 bits) into the bitmap format
// ([Summary] "Approach": a bitmap-based compressed format; [Abstract]):
//   bitmaps  [B][H][cap][d/64] u64   bit j of word w <=> channel 64w+j kept (R5, R6)
//   values   [B][H][cap*k]     fp16  kept values, ascending channel, rows in order
//   tile_off [B][H][cap/64+1]  u32   tile_off[j] = number of kept values in rows
//                                    r < min(64 j, T_b) of that (b, h)
// Rows r >= T_b = min(seq_lens[b], cap, t_stride) are not written; nor are
// tile_off entries j > ceil(T_b / 64).  Returns 0, or -1 on bad arguments.
// Channel-wise magnitude pruning (R24; the channel-wise direction of the
// pages' pruning variants, [README] "Part II"), compressed into the bitmap
// format: each channel of a full 64-row tile keeps its kc = keep / 2 largest
// entries over the tile's rows (the per-token rule applied to the column,
// ties to the earlier row), so a full tile stores 64 * keep values; rows of a
// final partial tile are pruned per token to keep.  keep must be even.
int orc_compress_channel(const uint16_t* dense, int B, int H, int64_t t_stride, int d,
                         const int32_t* seq_lens, int keep, int64_t cap, uint64_t* bitmaps,
                         uint16_t* values, uint32_t* tile_off, int nthreads) {
  if (d <= 0 || d % 64 != 0 || keep < 0 || keep > d || keep % 2 != 0 || cap <= 0 || cap % 64 != 0)
    return -1;
  const int words = d / 64;
  const int kc = keep / 2;
  const int64_t ntile_entries = cap / 64 + 1;
  if (nthreads <= 0) nthreads = hw_threads();
  parallel_for(static_cast<int64_t>(B) * H, nthreads, [&](int64_t u) {
    const int64_t b = u / H;
    const int T = clamp_len(seq_lens[b], std::min<int64_t>(cap, t_stride));
    const uint16_t* src = dense + u * t_stride * d;
    uint64_t* bm = bitmaps + u * cap * words;
    uint16_t* val = values + u * cap * keep;
    uint32_t* toff = tile_off + u * ntile_entries;
    std::vector<uint8_t> keep_mask(static_cast<size_t>(64) * d), col_keep(64);
    std::vector<uint16_t> col(64);
    uint32_t count = 0;
    for (int t0 = 0; t0 < T; t0 += 64) {
      toff[t0 / 64] = count;
      const int n = std::min(64, T - t0);
      if (n == 64) {
        for (int c = 0; c < d; ++c) {
          for (int r = 0; r < 64; ++r) col[r] = src[static_cast<int64_t>(t0 + r) * d + c];
          prune_row(col.data(), 64, kc, col_keep.data());
          for (int r = 0; r < 64; ++r) keep_mask[static_cast<size_t>(r) * d + c] = col_keep[r];
        }
      } else {
        for (int r = 0; r < n; ++r)
          prune_row(src + static_cast<int64_t>(t0 + r) * d, d, keep, &keep_mask[static_cast<size_t>(r) * d]);
      }
      for (int r = 0; r < n; ++r) {
        const uint16_t* x = src + static_cast<int64_t>(t0 + r) * d;
        uint64_t* w = bm + static_cast<int64_t>(t0 + r) * words;
        for (int i = 0; i < words; ++i) w[i] = 0;
        for (int c = 0; c < d; ++c) {
          if (keep_mask[static_cast<size_t>(r) * d + c]) {
            w[c / 64] |= uint64_t{1} << (c % 64);
            val[count++] = x[c];
          }
        }
      }
    }
    toff[(T + 63) / 64] = count;
  });
  return 0;
}

// With head_keep (R22) head h keeps head_keep[h] per row and the values of
// (b, h) start at Layout::region(b, h); values is then [B][cap * S].
static int compress_rule(const uint16_t* dense, int B, int H, int64_t t_stride, int d,
                         const int32_t* seq_lens, int k, const int32_t* head_keep, int64_t cap,
                         uint64_t* bitmaps, uint16_t* values, uint32_t* tile_off, int nthreads,
                         bool two_four) {
  if (d <= 0 || d % 64 != 0 || k < 0 || k > d || cap <= 0 || cap % 64 != 0) return -1;
  Layout L;
  if (!make_layout(H, head_keep, k, d, cap, &L)) return -1;
  const int words = d / 64;
  const int64_t ntile_entries = cap / 64 + 1;
  if (nthreads <= 0) nthreads = hw_threads();
  parallel_for(static_cast<int64_t>(B) * H, nthreads, [&](int64_t u) {
    const int64_t b = u / H, h = u % H;
    const int T = clamp_len(seq_lens[b], std::min<int64_t>(cap, t_stride));
    const uint16_t* src = dense + u * t_stride * d;
    uint64_t* bm = bitmaps + u * cap * words;
    uint16_t* val = values + L.region(b, h);
    uint32_t* toff = tile_off + u * ntile_entries;
    const int kh = static_cast<int>(L.keep[h]);
    std::vector<uint8_t> keep(d);
    uint32_t count = 0;
    for (int r = 0; r < T; ++r) {
      if (r % 64 == 0) toff[r / 64] = count;
      const uint16_t* x = src + static_cast<int64_t>(r) * d;
      if (two_four)
        prune_row_24(x, d, keep.data());
      else
        prune_row(x, d, kh, keep.data());
      for (int w = 0; w < words; ++w) bm[static_cast<int64_t>(r) * words + w] = 0;
      for (int c = 0; c < d; ++c) {
        if (keep[c]) {
          bm[static_cast<int64_t>(r) * words + c / 64] |= (uint64_t{1} << (c % 64));
          val[count++] = x[c];
        }
      }
    }
    toff[(T + 63) / 64] = count;
  });
  return 0;
}

int orc_compress_hk(const uint16_t* dense, int B, int H, int64_t t_stride, int d,
                    const int32_t* seq_lens, int k, const int32_t* head_keep, int64_t cap,
                    uint64_t* bitmaps, uint16_t* values, uint32_t* tile_off, int nthreads) {
  return compress_rule(dense, B, H, t_stride, d, seq_lens, k, head_keep, cap, bitmaps, values,
                       tile_off, nthreads, false);
}

int orc_compress(const uint16_t* dense, int B, int H, int64_t t_stride, int d,
                 const int32_t* seq_lens, int k, int64_t cap, uint64_t* bitmaps,
                 uint16_t* values, uint32_t* tile_off, int nthreads) {
  return orc_compress_hk(dense, B, H, t_stride, d, seq_lens, k, nullptr, cap, bitmaps, values,
                         tile_off, nthreads);
}

// 2:4 compression (R23) into the bitmap format with keep = d / 2: the layout
// of orc_compress, every 4-channel group of every row holding 2 set bits.
int orc_compress_24(const uint16_t* dense, int B, int H, int64_t t_stride, int d,
                    const int32_t* seq_lens, int64_t cap, uint64_t* bitmaps, uint16_t* values,
                    uint32_t* tile_off, int nthreads) {
  return compress_rule(dense, B, H, t_stride, d, seq_lens, d / 2, nullptr, cap, bitmaps, values,
                       tile_off, nthreads, true);
}

// Decode-time append of one new row per (b, h) to a compressed tensor
// ([Summary] "Approach" and [Abstract]: the tokens produced during decode are
// pruned and compressed at run time; R10: the new row is stored before the
// step's attention reads the cache).  The new row of (b, h) is rows[(b*H + h)*d ..]:
//   - it is pruned per token to keep (kept channels of that head, R22) by the
//     rule of prune_row, whatever rule wrote the rows before it (channel-wise
//     caches grow by per-token rows, R24);
//   - it becomes row T_b = seq_lens[b] (clamped to [0, cap]): its bitmap words
//     at that row, its kept values in ascending channel order right after the
//     values already stored for (b, h), i.e. from the tile-offset end entry
//     tile_off[ceil(T_b / 64)] (0 for an empty sequence, whose entry 0 is
//     written as 0);
//   - the end entry of the grown sequence, tile_off[ceil((T_b + 1) / 64)], is
//     set to that start plus keep.
// A sequence already at capacity is left unchanged and bit 0 of *status is
// set.  seq_lens is not changed here: the key and value tensors of a step
// share one length, which the caller advances once after appending to both.
int orc_append_rows(uint64_t* bitmaps, uint16_t* values, uint32_t* tile_off, int B, int H,
                    int64_t cap, int d, int k, const int32_t* head_keep, const uint16_t* rows,
                    const int32_t* seq_lens, uint32_t* status) {
  if (d <= 0 || d % 64 != 0 || cap <= 0 || cap % 64 != 0 || k < 0 || k > d) return -1;
  Layout L;
  if (!make_layout(H, head_keep, k, d, cap, &L)) return -1;
  const int words = d / 64;
  const int64_t ntile_entries = cap / 64 + 1;
  std::vector<uint8_t> keep(d);
  for (int64_t u = 0; u < static_cast<int64_t>(B) * H; ++u) {
    const int64_t b = u / H, h = u % H;
    const int T = clamp_len(seq_lens[b], cap);
    if (T >= cap) {
      if (status) *status |= 1u;
      continue;
    }
    const uint16_t* x = rows + u * d;
    uint64_t* bm = bitmaps + (u * cap + T) * words;
    uint16_t* val = values + L.region(b, h);
    uint32_t* toff = tile_off + u * ntile_entries;
    if (T == 0) toff[0] = 0;
    const uint32_t start = toff[(T + 63) / 64];
    prune_row(x, d, static_cast<int>(L.keep[h]), keep.data());
    for (int w = 0; w < words; ++w) bm[w] = 0;
    uint32_t n = 0;
    for (int c = 0; c < d; ++c) {
      if (keep[c]) {
        bm[c / 64] |= uint64_t{1} << (c % 64);
        val[start + n++] = x[c];
      }
    }
    toff[(T + 1 + 63) / 64] = start + n;
  }
  return 0;
}

// Decompress (R7): walk the bitmap; a set bit takes the next stored value, a
// clear bit gives +0.0.  Output [B][H][cap][d] fp16 bits; rows >= T_b are zero.
int orc_decompress_hk(const uint64_t* bitmaps, const uint16_t* values, const uint32_t* tile_off,
                      int B, int H, int64_t cap, int d, int k, const int32_t* head_keep,
                      const int32_t* seq_lens, uint16_t* out) {
  if (d <= 0 || d % 64 != 0 || cap <= 0 || cap % 64 != 0) return -1;
  Layout L;
  if (!make_layout(H, head_keep, k, d, cap, &L)) return -1;
  const int words = d / 64;
  const int64_t ntile_entries = cap / 64 + 1;
  for (int64_t u = 0; u < static_cast<int64_t>(B) * H; ++u) {
    const int64_t b = u / H, h = u % H;
    const int T = clamp_len(seq_lens[b], cap);
    const uint64_t* bm = bitmaps + u * cap * words;
    const uint16_t* val = values + L.region(b, h);
    const uint32_t* toff = tile_off + u * ntile_entries;
    uint16_t* dst = out + u * cap * d;
    std::memset(dst, 0, sizeof(uint16_t) * cap * d);
    for (int tile = 0; tile * 64 < T; ++tile) {
      uint32_t next = toff[tile];  // first value of the tile
      for (int r = tile * 64; r < std::min(T, tile * 64 + 64); ++r) {
        for (int c = 0; c < d; ++c) {
          const bool set = (bm[static_cast<int64_t>(r) * words + c / 64] >> (c % 64)) & 1u;
          dst[static_cast<int64_t>(r) * d + c] = set ? val[next++] : 0;
        }
      }
    }
  }
  return 0;
}

int orc_decompress(const uint64_t* bitmaps, const uint16_t* values, const uint32_t* tile_off,
                   int B, int H, int64_t cap, int d, int k, const int32_t* seq_lens,
                   uint16_t* out) {
  return orc_decompress_hk(bitmaps, values, tile_off, B, H, cap, d, k, nullptr, seq_lens, out);
}

// Bytes a compressed tensor occupies for the given lengths: per (b, h),
// bitmaps (d/8 bytes per row) + kept values (2 bytes each) + tile offsets
// (4 bytes per tile entry, ceil(T/64) + 1 entries).
// With head_keep, head h counts 2 * head_keep[h] bytes of values per row.
int64_t orc_used_bytes_hk(int B, int H, const int32_t* seq_lens, int64_t cap, int d, int k,
                          const int32_t* head_keep) {
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t T = clamp_len(seq_lens[b], cap);
    for (int h = 0; h < H; ++h) {
      const int64_t kh = head_keep ? head_keep[h] : k;
      total += T * (d / 8) + 2 * T * kh + 4 * ((T + 63) / 64 + 1);
    }
  }
  return total;
}

int64_t orc_used_bytes(int B, int H, const int32_t* seq_lens, int64_t cap, int d, int k) {
  return orc_used_bytes_hk(B, H, seq_lens, cap, d, k, nullptr);
}

// Decode-step attention, the plain definition, fp64 ([Summary] "Approach":
// attention computed over the pruned caches; [Abstract]):
//   s_t = scale * sum_c q[c] * K[t][c]
//   o[c] = sum_t exp(s_t - max s) V[t][c] / sum_t exp(s_t - max s)
// for each (b, hq) with kv head h = floor(hq / (Hq / Hkv)) (R9).  K, V are
// dense fp16 caches [B][Hkv][t_stride][d] (pass the zero-masked cache to get
// the sparse result).  T_b = min(seq_lens[b], t_stride); T_b = 0 gives zeros.
// out: [B][Hq][d] double.
int orc_attention_dense(const uint16_t* q, int B, int Hq, int Hkv, int d, const uint16_t* K,
                        const uint16_t* V, int64_t t_stride, const int32_t* seq_lens,
                        double scale, double* out, int nthreads) {
  if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0) return -1;
  const int G = Hq / Hkv;
  if (nthreads <= 0) nthreads = hw_threads();
  parallel_for(static_cast<int64_t>(B) * Hq, nthreads, [&](int64_t u) {
    const int64_t b = u / Hq, hq = u % Hq, h = hq / G;
    const int T = clamp_len(seq_lens[b], t_stride);
    double* o = out + u * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (T == 0) return;
    const uint16_t* qv = q + u * d;
    const uint16_t* Kb = K + (b * Hkv + h) * t_stride * d;
    const uint16_t* Vb = V + (b * Hkv + h) * t_stride * d;
    std::vector<double> qd(d), s(T);
    for (int c = 0; c < d; ++c) qd[c] = half_to_double(qv[c]);
    for (int t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += qd[c] * half_to_double(Kb[static_cast<int64_t>(t) * d + c]);
      s[t] = scale * acc;
    }
    const double m = *std::max_element(s.begin(), s.end());
    double l = 0.0;
    for (int t = 0; t < T; ++t) {
      const double w = std::exp(s[t] - m);
      l += w;
      for (int c = 0; c < d; ++c) o[c] += w * half_to_double(Vb[static_cast<int64_t>(t) * d + c]);
    }
    for (int c = 0; c < d; ++c) o[c] /= l;
  });
  return 0;
}

// The same attention read directly from the compressed caches: each row is
// decompressed by the rule of orc_decompress (R7) into fp64, then the plain
// definition above is applied.  Only the (b, hq) pairs listed in `units`
// (n_units entries of b*Hq + hq; all pairs when units == nullptr) are computed
// and written to out[b][hq][:].  kk and kv are the survivor counts of K and V.
// With kheads / vheads (R22) the value regions follow the per-head layout.
int orc_attention_compressed_hk(const uint16_t* q, int B, int Hq, int Hkv, int d,
                                const uint64_t* kbm, const uint16_t* kval, const uint32_t* ktoff,
                                int kk, const int32_t* kheads, const uint64_t* vbm,
                                const uint16_t* vval, const uint32_t* vtoff, int kvk,
                                const int32_t* vheads, int64_t cap, const int32_t* seq_lens,
                                double scale, const int64_t* units, int64_t n_units, double* out,
                                int nthreads) {
  if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || d % 64 != 0 || cap % 64 != 0) return -1;
  Layout KL, VL;
  if (!make_layout(Hkv, kheads, kk, d, cap, &KL) || !make_layout(Hkv, vheads, kvk, d, cap, &VL))
    return -1;
  const int G = Hq / Hkv;
  const int words = d / 64;
  const int64_t ntile_entries = cap / 64 + 1;
  if (nthreads <= 0) nthreads = hw_threads();
  const int64_t n = units ? n_units : static_cast<int64_t>(B) * Hq;
  auto decode_rows = [&](const uint64_t* bm, const uint16_t* val, const uint32_t* toff,
                         const Layout& L, int64_t b, int64_t h, int T, std::vector<double>& dst) {
    const int64_t unit = b * Hkv + h;
    const uint64_t* ub = bm + unit * cap * words;
    const uint16_t* uv = val + L.region(b, h);
    const uint32_t* ut = toff + unit * ntile_entries;
    dst.assign(static_cast<size_t>(T) * d, 0.0);
    for (int tile = 0; tile * 64 < T; ++tile) {
      uint32_t next = ut[tile];
      for (int r = tile * 64; r < std::min(T, tile * 64 + 64); ++r)
        for (int c = 0; c < d; ++c)
          if ((ub[static_cast<int64_t>(r) * words + c / 64] >> (c % 64)) & 1u)
            dst[static_cast<size_t>(r) * d + c] = half_to_double(uv[next++]);
    }
  };
  parallel_for(n, nthreads, [&](int64_t i) {
    const int64_t u = units ? units[i] : i;
    const int64_t b = u / Hq, hq = u % Hq, h = hq / G;
    const int T = clamp_len(seq_lens[b], cap);
    double* o = out + u * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (T == 0) return;
    std::vector<double> Kd, Vd, qd(d), s(T);
    decode_rows(kbm, kval, ktoff, KL, b, h, T, Kd);
    decode_rows(vbm, vval, vtoff, VL, b, h, T, Vd);
    for (int c = 0; c < d; ++c) qd[c] = half_to_double(q[u * d + c]);
    for (int t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += qd[c] * Kd[static_cast<size_t>(t) * d + c];
      s[t] = scale * acc;
    }
    const double m = *std::max_element(s.begin(), s.end());
    double l = 0.0;
    for (int t = 0; t < T; ++t) {
      const double w = std::exp(s[t] - m);
      l += w;
      for (int c = 0; c < d; ++c) o[c] += w * Vd[static_cast<size_t>(t) * d + c];
    }
    for (int c = 0; c < d; ++c) o[c] /= l;
  });
  return 0;
}

int orc_attention_compressed(const uint16_t* q, int B, int Hq, int Hkv, int d,
                             const uint64_t* kbm, const uint16_t* kval, const uint32_t* ktoff,
                             int kk, const uint64_t* vbm, const uint16_t* vval,
                             const uint32_t* vtoff, int kvk, int64_t cap,
                             const int32_t* seq_lens, double scale, const int64_t* units,
                             int64_t n_units, double* out, int nthreads) {
  return orc_attention_compressed_hk(q, B, Hq, Hkv, d, kbm, kval, ktoff, kk, nullptr, vbm, vval,
                                     vtoff, kvk, nullptr, cap, seq_lens, scale, units, n_units,
                                     out, nthreads);
}

}  // extern "C"
