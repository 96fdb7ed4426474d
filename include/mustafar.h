/*
 * mustafar.h -- C ABI of the MUSTAFAR hot path on AMD Instinct MI355X (gfx950).
 *
 * The library prunes the key and value caches of decode-time attention per
 * token by magnitude to an arbitrary unstructured sparsity, stores them in a
 * bitmap-compressed format, and computes the decode-step attention (q.K^T,
 * softmax, P.V) directly over the compressed caches.  A dense fp16 decode
 * attention is exported beside it as the comparison baseline.
 *
 * Sources (web pages; cited by title and section):
 *   [Summary]  "MUSTAFAR: Promoting Unstructured Sparsity for KV Cache Pruning in
 *              LLM Inference", AI-written paper summary (research-map page),
 *              sections "Approach", "Key results", "Limitations".
 *   [README]   "Mustafar: Promoting Unstructured Sparsity for KV Cache Pruning in
 *              LLM Inference", repository README mirror, sections
 *              "Part II: LongBench Evaluation", "Part III: Kernel Evaluation".
 *   [Abstract] "Mustafar: Promoting Unstructured Sparsity for KV Cache Pruning in
 *              LLM Inference", author abstract (author page).
 *
 * Conventions shared by every entry point
 *   - Pointers marked (device) are HIP device memory; (host) is host memory.
 *     The caller allocates and owns every buffer; the library never allocates,
 *     frees or synchronises.
 *   - fp16 data travels as its IEEE-754 binary16 bit patterns (uint16_t).
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Work is enqueued on it and the call returns without waiting.
 *   - Every call checks its arguments on the host first and returns a negative
 *     mustafar_status without launching anything when one is bad; only then
 *     does it look for a device (MUSTAFAR_ENODEV when there is none) and
 *     launch.  A launch failure returns MUSTAFAR_ELAUNCH.
 *   - head_dim must be 128.  Device pointers must be 16-byte aligned.
 *   - Lengths in seq_lens (device) are read by the kernels and clamped to
 *     [0, capacity]; the host cannot see them.
 *   - No global mutable state (except the device scratch array of
 *     mustafar_decode_step_noalloc): calls on different streams and buffers may
 *     run concurrently from any thread.
 */
#ifndef MUSTAFAR_H_
#define MUSTAFAR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUSTAFAR_OK = 0,
  MUSTAFAR_EINVAL = -1,       /* bad argument: null / misaligned pointer, size out of range */
  MUSTAFAR_EUNSUPPORTED = -2, /* valid but not built: head_dim != 128, Hq/Hkv not in {1,2,4,8} */
  MUSTAFAR_ENODEV = -3,       /* no HIP device visible */
  MUSTAFAR_ELAUNCH = -4,      /* kernel launch failed (hipGetLastError after the launch) */
  MUSTAFAR_ENOSPACE = -5      /* workspace smaller than the call needs */
} mustafar_status;

/* Sticky device status bits written by mustafar_append_token. */
#define MUSTAFAR_STATUS_APPEND_FULL 1u /* a sequence was already at capacity; its row was dropped */
#define MUSTAFAR_STATUS_BAD_OFFSETS 2u /* a tile-offset end entry would have placed a new row's values
                                          outside its (batch, head) value region; that row (bitmap,
                                          values, offsets) was not written */

/*
 * One compressed tensor (the key cache or the value cache of one layer) in the
 * bitmap-based sparse format ([Summary] "Approach"; [Abstract]).  The exact
 * layout is this library's design:
 *
 *   bitmaps      (device) uint64 [batch][num_kv_heads][capacity][2]
 *                bit j of word w is set <=> channel 64*w + j of that row was kept.
 *   values       (device) uint16 [batch][num_kv_heads][capacity * keep]
 *                the kept fp16 values of each row in ascending channel order,
 *                rows of a (batch, head) stored back to back from row 0.
 *   tile_offsets (device) uint32 [batch][num_kv_heads][capacity / 64 + 1]
 *                entry j = number of kept values stored before row 64*j of that
 *                (batch, head), for j = 0 .. ceil(T/64) (the last one is the end
 *                of the stored values); under per-token pruning entry j equals
 *                min(64*j, T) * keep.
 *
 * capacity is the number of rows allocated per (batch, head): a positive
 * multiple of 64, at most 2^24, with capacity * keep * 2 < 2^31.  keep
 * (0..head_dim) is the number of survivors per row.  head_dim must be 128.
 *
 * Per-head keep (the per-head sparsity the [Summary] "Limitations" section
 * leaves to future work): with head_keep set, kv head h keeps head_keep[h]
 * values per row, keep must equal the largest entry, and values becomes
 * uint16 [batch][capacity * S], S = the sum of head_keep, with the region of
 * (b, h) starting at element capacity * (b * S + head_keep[0] + ... +
 * head_keep[h - 1]); tile offsets count that head's values (min(64*j, T) *
 * head_keep[h]).  With every head at the same keep this is the layout above.
 * At most MUSTAFAR_MAX_HEAD_KEEP kv heads; entries outside 0..head_dim, or
 * keep different from their maximum, return MUSTAFAR_EINVAL.
 * batch * num_kv_heads must stay below 2^31.  Calls that break these limits
 * return MUSTAFAR_EINVAL (MUSTAFAR_EUNSUPPORTED for another head_dim).
 * The decode calls read any cache in this format: rows may hold any number of
 * values from 0 to head_dim (channel-wise pruning stores rows of varying
 * length) as long as the values are packed back to back, tile_offsets are
 * consistent with the popcounts and a (batch, head) stores at most
 * capacity * keep values.
 */
typedef struct {
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t keep;
  int32_t capacity;
  uint64_t *bitmaps;
  uint16_t *values;
  uint32_t *tile_offsets;
  const int32_t *head_keep; /* (host) NULL, or num_kv_heads survivors per row, one per kv head;
                               read during each call only */
} mustafar_kv_t;

#define MUSTAFAR_MAX_HEAD_KEEP 128 /* kv heads a per-head keep may describe */

/* Text for a status code (static storage; never NULL). */
const char *mustafar_status_str(int status);

/*
 * Survivors per row for a target sparsity s = fraction of entries pruned
 * ([README] "Part II": k_sparsity / v_sparsity, 0.5 means 50% pruned).
 * Returns floor((1 - s) * head_dim + 0.5) clamped to [0, head_dim]
 * (64 at s = 0.5, 38 at s = 0.7), or MUSTAFAR_EINVAL when s is not in [0, 1]
 * or head_dim <= 0.  Host only.
 */
int mustafar_keep_from_sparsity(double sparsity, int32_t head_dim);

/*
 * Bytes to allocate for each array of a compressed tensor described by `kv`
 * (its pointers are ignored).  values_bytes includes 64 bytes of tail padding.
 * Host only.  Returns MUSTAFAR_OK or MUSTAFAR_EINVAL/EUNSUPPORTED.
 */
int mustafar_kv_alloc_bytes(const mustafar_kv_t *kv, uint64_t *bitmaps_bytes,
                            uint64_t *values_bytes, uint64_t *offsets_bytes);

/*
 * Bytes the compressed tensor occupies for the given lengths (host array of
 * `batch` entries, clamped to [0, capacity]): per (batch, head) with T rows,
 * 16*T (bitmaps) + 2*keep*T (values; 2*head_keep[h]*T with per-head keep)
 * + 4*(ceil(T/64) + 1) (tile offsets).
 * This is the compressed size compared with the dense 256*T bytes
 * ([Summary] "Key results" gives 45% of dense at 70% sparsity and 65% at 50%
 * for the authors' own layout).  Host only.
 */
int mustafar_kv_used_bytes(const mustafar_kv_t *kv, const int32_t *seq_lens_host, int64_t *bytes);

/*
 * Prefill: prune every cached row of a dense cache per token by magnitude and
 * write it compressed into `dst` ([Summary] "Approach"; [Abstract]; the
 * token-wise, magnitude-based variant Kt_Mag / Vt_Mag of [README] "Part II").
 *
 *   dense     (device) uint16 [batch][num_kv_heads][t_stride][128] fp16 bits.
 *   seq_lens  (device) int32 [batch]; rows t < min(seq_lens[b], capacity, t_stride)
 *             are compressed, the rest of dst is left untouched except the
 *             tile-offset end entry.
 *
 * Row rule: the keep channels of largest |x| survive, compared through the
 * magnitude bits (bits & 0x7FFF, so -0 == +0); on equal magnitude the lower
 * channel survives.  Bitmaps, values and tile offsets are bit-exact
 * functions of the input.
 */
int mustafar_prune_compress(const mustafar_kv_t *dst, const uint16_t *dense, int64_t t_stride,
                            const int32_t *seq_lens, void *stream);

/*
 * Decode-time append: prune and compress the new key and value row of every
 * (batch, kv head) by the same rule and store them as row T_b = seq_lens[b] of
 * `k` and `v`, then increment seq_lens[b] once ([Summary] "Approach" and
 * [Abstract]: the tokens produced during decode are pruned and compressed at
 * run time).  The row's values go right after the stored ones (at the tile
 * offsets' end entry, T_b * keep when every row holds keep values) and the end
 * entry advances by keep.  k and v must agree in batch, num_kv_heads and
 * capacity and may differ in keep.
 *
 *   k_new, v_new (device) uint16 [batch][num_kv_heads][128] fp16 bits.
 *   seq_lens     (device) int32 [batch], incremented in place.
 *   status       (device) uint32, may be NULL; MUSTAFAR_STATUS_APPEND_FULL is
 *                OR-ed in when a sequence is already at capacity (that
 *                sequence is then left unchanged).
 *
 * Offsets precondition: for T_b > 0 the new row's values are placed at the
 * tile-offset end entry tile_offsets[ceil(T_b / 64)], which every call of this
 * library leaves consistent with the stored rows (prefill, append, fused
 * step).  For T_b = 0 the entries are not read: the row starts at value 0 and
 * entry 0 is written, so a never-prefilled cache (any contents) can be grown
 * from empty.  An end entry that would put the row's values past the
 * (batch, head) value region (capacity * keep values) is never followed: that
 * row is not written, MUSTAFAR_STATUS_BAD_OFFSETS is OR-ed into *status, and
 * the length still advances (the cache is inconsistent and must be refilled).
 */
int mustafar_append_token(const mustafar_kv_t *k, const mustafar_kv_t *v, const uint16_t *k_new,
                          const uint16_t *v_new, int32_t *seq_lens, uint32_t *status,
                          void *stream);

/*
 * Splits over the sequence that mustafar_decode_attn and mustafar_decode_attn_valu
 * use when called with splits = 0, for this shape: floor(512 / (batch *
 * num_kv_heads)) splits, so at most 512 blocks of 4 waves (two per compute
 * unit of an MI355X), at least 1, and at most ceil(tiles / 4) for the
 * ceil(max_seq_len / 64) 64-row tiles (every wave gets at least one tile).
 * mustafar_dense_decode_attn with splits = 0 uses the same rule with
 * 256 blocks (never more splits than this).  Host only.
 */
int mustafar_decode_auto_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len);

/*
 * Workspace bytes the decode calls need for `splits` splits (0 = automatic,
 * sized from max_seq_len).  Host only.
 */
int mustafar_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_seq_len, int32_t splits,
                                    uint64_t *bytes);

/*
 * Clear a decode workspace (device, `bytes` long, a multiple of 4).  The decode
 * calls need no particular workspace contents; clearing is only for callers
 * that want deterministic memory.  Calls that share a workspace must be
 * ordered (same stream); overlapping ones race.
 */
int mustafar_decode_workspace_init(void *workspace, uint64_t bytes, void *stream);

/*
 * Decode-step attention over the compressed caches ([Summary] "Approach": an
 * attention kernel that computes directly on the bitmap format; [Abstract];
 * [README] "Part III": the batched sparse attention kernel).  For every batch
 * row b and query head hq, with kv head h = floor(hq / (num_q_heads / num_kv_heads))
 * and T_b = min(seq_lens[b], capacity):
 *     s_t = scale * sum_c q[b][hq][c] * Khat[b][h][t][c]
 *     out[b][hq][c] = sum_t exp(s_t - max s) Vhat[b][h][t][c] / sum_t exp(s_t - max s)
 * where Khat/Vhat are the stored rows with pruned entries 0; T_b = 0 gives 0.
 *
 *   q    (device) uint16 [batch][num_q_heads][128] fp16 bits.
 *   k, v compressed caches with equal batch, num_kv_heads and capacity.
 *   seq_lens (device) int32 [batch].
 *   max_seq_len  host upper bound of seq_lens, used only to pick splits.
 *   scale        softmax scale (1/sqrt(128) for standard attention).
 *   splits       number of sequence splits per (batch, kv head); 0 = automatic.
 *   out  (device) uint16 [batch][num_q_heads][128] fp16 bits (round to nearest).
 *   workspace    (device) at least mustafar_decode_workspace_bytes long; it holds
 *                the per-split partial states between the two launches.
 * Arithmetic: fp16 inputs; each 64-row tile's stored entries are decoded
 * into a dense fp16 tile in LDS and both contractions run on the matrix cores
 * (v_mfma_f32_16x16x32_f16, fp32 accumulation): scores from the decoded key
 * tile, P.V with the probabilities rounded to fp16; fp32 online softmax per
 * split; a cross-split merge in fp32.
 * Two kernel launches on `stream`: the split kernel and the merge.
 * Errors: MUSTAFAR_EINVAL for null or misaligned pointers (q, out, workspace
 * 16 B; seq_lens 4 B), shape mismatches between k and v, num_q_heads not a
 * multiple of num_kv_heads, a non-finite scale or splits outside [0, 1024];
 * MUSTAFAR_EUNSUPPORTED for a group size other than 1, 2, 4, 8;
 * MUSTAFAR_ENOSPACE for a workspace smaller than needed; MUSTAFAR_ENODEV,
 * MUSTAFAR_ELAUNCH from the runtime.  Nothing is launched on an error.
 */
int mustafar_decode_attn(const uint16_t *q, int32_t num_q_heads, const mustafar_kv_t *k,
                         const mustafar_kv_t *v, const int32_t *seq_lens, int32_t max_seq_len,
                         float scale, int32_t splits, uint16_t *out, void *workspace,
                         uint64_t workspace_bytes, void *stream);

/*
 * The same operation, arguments and errors as mustafar_decode_attn, computed
 * on the vector units only: each decoded key entry is multiplied straight into
 * the G scores of its row (fp32 fma), and P.V accumulates from a channel-major
 * decoded value tile with the probabilities as fp16 pairs (v_dot2_f32_f16,
 * fp32 accumulation).  Kept as a second implementation of the same attention
 * for comparison.
 */
int mustafar_decode_attn_valu(const uint16_t *q, int32_t num_q_heads, const mustafar_kv_t *k,
                              const mustafar_kv_t *v, const int32_t *seq_lens, int32_t max_seq_len,
                              float scale, int32_t splits, uint16_t *out, void *workspace,
                              uint64_t workspace_bytes, void *stream);

/*
 * One fused decode step: mustafar_append_token followed by mustafar_decode_attn
 * in two kernel launches instead of three, with the same results bit for bit
 * (caches, seq_lens, status and out).  The pages ask that the attention over
 * the compressed caches pay for the run-time pruning and compression of the
 * tokens produced during decode ([Abstract]; [Summary] "Approach"); here the
 * wave whose tiles end the sequence prunes and stores the new key and value
 * rows itself and attends over them in the same pass, and the merge kernel
 * advances seq_lens.
 *
 *   k_new, v_new (device) uint16 [batch][num_kv_heads][128] fp16 bits (16 B aligned).
 *   seq_lens     (device) int32 [batch]: row seq_lens[b] is added, attention covers
 *                seq_lens[b] + 1 rows, and seq_lens[b] is incremented once.  A
 *                sequence already at capacity adds nothing, attends over its
 *                capacity rows and ORs MUSTAFAR_STATUS_APPEND_FULL into *status.
 *                The offsets precondition and MUSTAFAR_STATUS_BAD_OFFSETS are
 *                those of mustafar_append_token.
 *   status       (device) uint32, may be NULL.
 *   max_seq_len  host upper bound of the lengths after the step (picks splits).
 *   Other arguments and errors as mustafar_decode_attn; the caches are written.
 */
int mustafar_decode_step(const uint16_t *q, int32_t num_q_heads, const mustafar_kv_t *k,
                         const mustafar_kv_t *v, const uint16_t *k_new, const uint16_t *v_new,
                         int32_t *seq_lens, uint32_t *status, int32_t max_seq_len, float scale,
                         int32_t splits, uint16_t *out, void *workspace, uint64_t workspace_bytes,
                         void *stream);

/*
 * mustafar_decode_step without a workspace, for callers that cannot allocate
 * device memory around the call (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same operation, arguments (minus
 * workspace and workspace_bytes), results bit for bit and errors as
 * mustafar_decode_step; the call itself allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).
 *
 * The split partials go to a device array of the library,
 * MUSTAFAR_NOALLOC_SCRATCH_BYTES long, one per device, held from the library's
 * load on that device until the process ends.  A shape whose partials
 * (batch * num_q_heads * splits * 528 bytes, splits as for splits = 0 when 0 is
 * passed) exceed it returns MUSTAFAR_ENOSPACE and launches nothing.  Every call
 * on one device shares that device's array: calls that overlap in time on one
 * device (different streams, or threads without ordering) race and must be
 * serialised by the caller; calls on one stream are ordered and safe.  The
 * array's contents between calls are of no meaning (each call writes every
 * partial it reads).  The first call on each device looks up the array's
 * address once (hipGetSymbolAddress) and keeps it.
 */
#define MUSTAFAR_NOALLOC_SCRATCH_BYTES (8u << 20)
int mustafar_decode_step_noalloc(const uint16_t *q, int32_t num_q_heads, const mustafar_kv_t *k,
                                 const mustafar_kv_t *v, const uint16_t *k_new,
                                 const uint16_t *v_new, int32_t *seq_lens, uint32_t *status,
                                 int32_t max_seq_len, float scale, int32_t splits, uint16_t *out,
                                 void *stream);

/*
 * Channel-wise magnitude pruning, prefill (the channel-wise direction of the
 * pruning variants in [README] "Part II"; the pages give no grouping, so this
 * library groups by its 64-row tiles): in every full 64-row tile of a
 * (batch, head), each channel keeps its keep/2 entries of largest magnitude
 * over the tile's rows (ties to the earlier row), so the tile stores 64 * keep
 * values with rows of varying length; the rows of a final partial tile are
 * pruned per token to keep (like mustafar_prune_compress), and so are the rows
 * mustafar_append_token adds later.  The output is the bitmap format above;
 * the decode calls read it.  keep must be even and head_keep NULL
 * (MUSTAFAR_EINVAL otherwise); other arguments and errors as
 * mustafar_prune_compress.
 */
int mustafar_prune_compress_channel(const mustafar_kv_t *dst, const uint16_t *dense,
                                    int64_t t_stride, const int32_t *seq_lens, void *stream);

/*
 * 2:4 semi-structured comparator, prefill: prunes every row of `dense` so that
 * each group of 4 consecutive channels keeps its 2 entries of largest
 * magnitude (ties to the lower channel) and stores them in the bitmap format
 * above.  2:4 semi-structured sparsity is one of the baselines the pages list
 * ([Summary] "Experimental setup"); at 50% it stores exactly the bytes of
 * unstructured pruning at keep 64, so the two formats can be compared at equal
 * size.  dst->keep must be 64 (head_dim / 2) and dst->head_keep NULL, else
 * MUSTAFAR_EINVAL.  Other arguments, layout and errors as
 * mustafar_prune_compress.
 */
int mustafar_prune_compress_24(const mustafar_kv_t *dst, const uint16_t *dense, int64_t t_stride,
                               const int32_t *seq_lens, void *stream);

/*
 * 2:4 comparator, decode: the attention of mustafar_decode_attn over key and
 * value caches written by mustafar_prune_compress_24, computed with the
 * structure (each group's two values expanded in registers; no bitmap walk).
 * Both caches must have keep 64 and no head_keep (MUSTAFAR_EINVAL otherwise),
 * and every stored row must hold exactly two values in each group of 4
 * channels; for other contents the output is unspecified (mustafar_decode_attn
 * reads any cache).  Arguments, workspace and errors as mustafar_decode_attn.
 */
int mustafar_decode_attn_24(const uint16_t *q, int32_t num_q_heads, const mustafar_kv_t *k,
                            const mustafar_kv_t *v, const int32_t *seq_lens, int32_t max_seq_len,
                            float scale, int32_t splits, uint16_t *out, void *workspace,
                            uint64_t workspace_bytes, void *stream);

/*
 * The same attention over dense, unpruned fp16 caches: the comparison
 * baseline (the pages compare against dense attention, [Summary] "Key results"
 * and "Experimental setup").  q.K^T runs on the matrix cores (MFMA), P.V and
 * the softmax on the vector units: fp32 softmax, P.V with the probabilities
 * rounded to fp16 and fp32 accumulation (the operand precisions of
 * mustafar_decode_attn); two launches like mustafar_decode_attn.
 *
 *   k, v (device) uint16 [batch][num_kv_heads][t_stride][128] fp16 bits; rows
 *        t < min(seq_lens[b], t_stride) are attended.
 *   Other arguments as mustafar_decode_attn (the workspace rules are the same).
 */
int mustafar_dense_decode_attn(const uint16_t *q, int32_t num_q_heads, const uint16_t *k,
                               const uint16_t *v, int32_t batch, int32_t num_kv_heads,
                               int32_t head_dim, int64_t t_stride, const int32_t *seq_lens,
                               int32_t max_seq_len, float scale, int32_t splits, uint16_t *out,
                               void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * Measurement helper: read `bytes` (a multiple of 4096, >= 4096) from `buf`
 * (device, 16-byte aligned) with coalesced 16-byte loads and write a checksum
 * to *sink (device uint32) so the reads cannot be elided.  Used to measure
 * the achievable HBM read rate on the same device.
 */
int mustafar_probe_stream_read(const void *buf, uint64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MUSTAFAR_H_ */
