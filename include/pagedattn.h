/*
 * pagedattn.h -- C ABI of libpagedattn: paged-attention decode (v1 and the
 * partitioned v2) for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every sequence s of a decode batch (one query token
 * per sequence) and every query head h, attention over the sequence's cached
 * keys and values, which live in fixed-size blocks of a shared pool reached
 * through a per-sequence block table (page "BI-V100 PagedAttention V2
 * implementation" -- the commit page of paged_attention_v2_pytorch.py --
 * argument list of paged_attention_v2_pytorch and its per-block gather loop):
 *
 *   s[h,t]  = scale * k_scale * sum_d q[s,h,d] K[t,kv(h),d]  +  alibi[h] * t
 *   out[s,h] = sum_t softmax_t(s[h,:]) * v_scale * V[t,kv(h),:]
 *
 * with kv(h) = h / (num_heads / num_kv_heads) (same page, GQA expansion by
 * repeat_interleave) and t the absolute 0-based key position (same page,
 * "Alibi bias" step of Phase 1).
 *
 * v2 (same page, "Phase 1: Per-partition attention" and "Phase 2: Reduce
 * across partitions") splits each sequence into partitions of
 * PA_PARTITION_SIZE = 512 tokens; partition p covers tokens
 * [512p, min(512p + 512, L)).  Phase 1 stores, per (s, h, p),
 *   max_logits[s,h,p] = m_p = max over the partition of s[h,t]
 *   exp_sums[s,h,p]   = S_p = sum over the partition of exp(s[h,t] - m_p)
 *   tmp_out[s,h,p,:]  = O_p = sum exp(s[h,t] - m_p) v_scale V[t] / S_p
 * (O_p is normalised: the page's prose and its merge formula need that; its
 * printed code omits the division, which double counts S_p), and Phase 2
 * merges them with the log-sum-exp rescale
 *   M = max_p m_p,  r_p = exp(m_p - M) S_p,  out = sum_p (r_p / sum_q r_q) O_p.
 * v1 (same page, commit message and "Performance vs V1") processes the whole
 * sequence in one workgroup and writes only out.  Natural-log units
 * throughout.
 *
 * Layouts (all row-major, contiguous, device memory):
 *   query, out    [num_seqs, num_heads, head_size]                 dtype
 *   key_cache     [num_blocks, num_kv_heads, head_size/x, block_size, x]
 *   value_cache   [num_blocks, num_kv_heads, head_size, block_size]
 *                 x = 16 / sizeof(KV element): 4 (f32), 8 (f16, bf16),
 *                 16 (fp8); head dim d = c * x + j for K index [.., c, t, j].
 *                 KV elements have type dtype, or are OCP FP8 E4M3FN bytes
 *                 when kv_cache_dtype == PA_KV_FP8_E4M3.
 *   block_tables  int32 [num_seqs, max_num_blocks_per_seq]; token t of
 *                 sequence s is slot t % block_size of physical block
 *                 block_tables[s, t / block_size].  Entries at and after
 *                 ceil(seq_lens[s] / block_size) are never read.
 *   seq_lens      int32 [num_seqs]
 *   alibi_slopes  float [num_heads], or NULL for no ALiBi
 *   exp_sums, max_logits  float [num_seqs, num_heads, max_num_partitions]
 *   tmp_out       [num_seqs, num_heads, max_num_partitions, head_size]
 *                 float by default; the caller may choose the query /
 *                 output dtype instead (pa_decode_options.partial_dtype):
 *                 the V2 page's Phase 1 casts each partition's output to
 *                 the type of the caller's tmp_output buffer.  Partials are
 *                 accumulated in fp32 and rounded once to that type.
 *
 * Ownership.  Every buffer belongs to the caller.  The library allocates and
 * frees nothing and keeps no pointer after a call returns.  Its only global
 * state is a per-device cache of the compute-unit count, filled on first use
 * under a lock, and the per-thread profiling events of pa_set_timing_events.
 *
 * Streams.  Work is enqueued on `stream` (a hipStream_t; NULL is the null
 * stream) and runs asynchronously; no call synchronises or copies device
 * memory to the host (that is why max_seq_len is a host integer).
 *
 * Errors.  Every call returns a pa_status.  All argument checks run on the
 * host before any HIP call, so an error leaves every buffer untouched.  A
 * failed kernel launch returns PA_ERR_HIP.  Device data the host cannot see
 * is guarded in the kernels: a sequence whose seq_lens entry is negative or
 * above max_seq_len, or that reaches a block-table entry outside
 * [0, num_blocks), reads no memory through it and gets NaN in its outputs.
 *
 * Supported: dtype f32 / f16 / bf16; kv_cache_dtype AUTO (KV in dtype) or
 * FP8_E4M3 (dtype f16 or bf16); head_size 64 or 128; block_size 16 or 32;
 * num_heads any multiple of num_kv_heads; num_seqs <= 65535; max_seq_len
 * <= 65535 * 512 for v2 / auto.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_PARTITION_SIZE 512

/* The enums below are int-sized in C and C++ alike.  A C caller may pass any
 * int where one is expected; in C++ the fixed base type makes every int value
 * a valid value of the enum, so the library can reject unknown values
 * (PA_ERR_BAD_ARGUMENT) without undefined behaviour. */
#ifdef __cplusplus
#define PA_ENUM_BASE : int
#else
#define PA_ENUM_BASE
#endif

typedef enum pa_status PA_ENUM_BASE {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1, /* a required pointer is NULL                   */
  PA_ERR_BAD_SHAPE = 2,    /* sizes inconsistent or out of the valid range */
  PA_ERR_MISALIGNED = 3,   /* a cache / query / out pointer not 16-byte aligned */
  PA_ERR_UNSUPPORTED = 4,  /* valid but not built: head_size, block_size, dtype */
  PA_ERR_HIP = 5,          /* the HIP runtime reported an error            */
  PA_ERR_BAD_ARGUMENT = 6  /* non-finite scale, unknown enum value         */
} pa_status;

/* Element type of query and out (and of the KV cache when kv_cache_dtype is
 * PA_KV_AUTO). */
typedef enum pa_dtype PA_ENUM_BASE { PA_DTYPE_F32 = 0, PA_DTYPE_F16 = 1, PA_DTYPE_BF16 = 2 } pa_dtype;

/* "auto" = the cache holds dtype (V2 page, kv_cache_dtype argument);
 * FP8_E4M3 = the cache holds OCP FP8 E4M3FN bytes, dequantised as
 * value = decode(byte) * k_scale (keys) or * v_scale (values). */
typedef enum pa_kv_cache_dtype PA_ENUM_BASE { PA_KV_AUTO = 0, PA_KV_FP8_E4M3 = 1 } pa_kv_cache_dtype;

/* Which algorithm a sequence takes.  AUTO chooses per sequence, on the
 * device, with the rule of pa_should_use_v2. */
typedef enum pa_mode PA_ENUM_BASE { PA_MODE_V1 = 0, PA_MODE_V2 = 1, PA_MODE_AUTO = 2 } pa_mode;

/* Cache layouts a decode call reads.  DECODE is the V2 page's layout (K
 * [num_blocks, num_kv_heads, head_size/x, block_size, x], V [num_blocks,
 * num_kv_heads, head_size, block_size]).  BLOCK_ROWS is the dispatch page's
 * decode signature: K and V both [num_blocks, num_kv_heads, block_size,
 * head_size] (each token's head_size values contiguous); dtype f16 or bf16
 * and kv_cache_dtype AUTO only (others: PA_ERR_UNSUPPORTED). */
typedef enum pa_kv_layout PA_ENUM_BASE { PA_KV_LAYOUT_DECODE = 0, PA_KV_LAYOUT_BLOCK_ROWS = 1 } pa_kv_layout;

/* Element type of the v2 partial outputs in tmp_out (V2 page, "Phase 1:
 * Per-partition attention": each partition's output is cast to the dtype of
 * the caller's tmp_output buffer).  F32 is the default; OUT = the query /
 * output dtype (half the partial-row bytes for 16-bit queries; for f32
 * queries both are f32). */
typedef enum pa_partial_dtype PA_ENUM_BASE { PA_PARTIAL_F32 = 0, PA_PARTIAL_OUT = 1 } pa_partial_dtype;

/* Decode options of the *_ex entry points: the sliding window and the logit
 * soft cap of the dispatch page's decode configuration (AttnDispatchConfig
 * fields window_left and softcap, -1 and 0 meaning off), which the Neuron
 * page hands to a flash-attention call as window_size / softcap.  The pages
 * pass them on without defining them; the meaning taken is that call's:
 *
 *   window_left = W >= 0: the decode query, at position L - 1, attends to
 *     the keys t with L - 1 - W <= t <= L - 1 only (the last W + 1 tokens;
 *     W = 0 keeps the last token alone).  W = -1: every key.  A right window
 *     is moot for the last token and has no field.
 *   logits_soft_cap = c > 0: each scaled logit scale * k_scale * q.K becomes
 *     c * tanh(logit / c) before the ALiBi bias is added.  c = 0: off.
 *
 * Keys outside the window are neither weighted nor read when their whole
 * block lies outside it (their block-table entries may be stale).  In v2, a
 * partition with no key inside the window gets max_logits = -inf and
 * exp_sums = 0 (as the V2 page's unused partitions) and no tmp_out row;
 * the auto rule (pa_should_use_v2) is applied to the window-clipped length
 * min(L, W + 1).  kv_layout selects the cache layout (pa_kv_layout) and
 * partial_dtype the element type of tmp_out (pa_partial_dtype).  A NULL
 * options pointer means no window, no cap, the DECODE layout and fp32
 * partials (all fields zero but window_left = -1): the *_ex call is then the
 * plain call.  window_left < -1, a cap that is negative, infinite or NaN, or
 * an unknown layout or partial dtype returns PA_ERR_BAD_ARGUMENT. */
typedef struct pa_decode_options {
  int window_left;
  float logits_soft_cap;
  int kv_layout;      /* pa_kv_layout of key_cache / value_cache */
  int partial_dtype;  /* pa_partial_dtype of tmp_out */
} pa_decode_options;

/* ---------------------------------------------------------------------- */
/* Full calls                                                             */
/* ---------------------------------------------------------------------- */

/* v1: one workgroup per (sequence, KV head) walks the whole sequence and
 * writes out only (V2 page, commit message: v1 processes the entire KV
 * sequence in one kernel).  Unlike the page's v1 it has no shared-memory
 * ceiling on seq_len: it keeps a running max and sum. */
pa_status paged_attention_v1(
    void *out, const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, const float *alibi_slopes,
    pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
    void *stream);

/* v2: Phase 1 (one workgroup per (partition, KV head, sequence)) then
 * Phase 2 (one workgroup per (query head, sequence)); V2 page, "Phase 1" and
 * "Phase 2".  Writes out; max_logits / exp_sums for every partition slot
 * (slots p >= ceil(L/512) get -inf / 0, as the page's padding step); tmp_out
 * for p < ceil(L/512) only (later slots are untouched scratch).  A sequence
 * of length 0 gets out = 0 and padding statistics. */
pa_status paged_attention_v2(
    void *out, float *exp_sums, float *max_logits, void *tmp_out,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, void *stream);

/* Per-sequence choice between v1 and v2 (pa_should_use_v2, decided on the
 * device from seq_lens), same arguments as paged_attention_v2.  Sequences
 * sent down the v1 path get out only; their exp_sums / max_logits / tmp_out
 * rows are left as they were.  When the rule sends every sequence to v1
 * (it does at max_seq_len, and it is monotone in the length), the call runs
 * as plain v1: one workgroup per (sequence, KV head), no reduce phase.
 *
 * Batches with many (sequence, KV head) items on the narrow-group kernel
 * (pa_auto_uses_slots: no window, the default layout) run instead as one
 * persistent launch over equal shares of the batch's memory-load cost (the
 * PoD page's work estimate), then the reduce phase: piece j of a sequence's
 * (KV head, head group) item -- every piece of a cut item spans at least
 * 512 keys, so an item has no more pieces than partitions -- stores its
 * partials in partition slot j, the slots past the last piece get
 * max_logits = -inf / exp_sums = 0, and every sequence of two or more
 * partitions is merged.  out is the same softmax; the partial buffers are
 * then scratch (not the per-partition partials of v2).  A launch sized by
 * the longest sequence would otherwise dispatch a workgroup per partition
 * slot of every sequence. */
pa_status paged_attention_auto(
    void *out, float *exp_sums, float *max_logits, void *tmp_out,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, void *stream);

/* ---------------------------------------------------------------------- */
/* The two phases on their own (same arguments as paged_attention_v2 plus  */
/* the mode).  paged_attention_v2 == partition(V2) then reduce(V2), and    */
/* paged_attention_auto == partition(AUTO) then reduce(AUTO).  With        */
/* PA_MODE_V1 the partition phase is the whole of v1 (exp_sums, max_logits */
/* and tmp_out may then be NULL) and the reduce phase does nothing.        */
/* ---------------------------------------------------------------------- */

/* Phase 1 (V2 page, "Phase 1: Per-partition attention"). */
pa_status paged_attention_partition(
    pa_mode mode, void *out, float *exp_sums, float *max_logits, void *tmp_out,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, void *stream);

/* Phase 2 (V2 page, "Phase 2: Reduce across partitions (log-sum-exp)"):
 * reads exp_sums, max_logits and tmp_out of every sequence with more than
 * one partition on the v2 path and writes its out rows.  The cache pointers
 * and block_tables are not read and may be NULL. */
pa_status paged_attention_reduce(
    pa_mode mode, void *out, const float *exp_sums, const float *max_logits,
    const void *tmp_out, int num_seqs, int num_heads, int num_kv_heads, int head_size,
    const int32_t *seq_lens, int max_seq_len, int max_num_partitions, pa_dtype dtype,
    void *stream);

/* ---------------------------------------------------------------------- */
/* The same calls with decode options (sliding window, logit soft cap; see */
/* pa_decode_options).  Every other argument and every error is that of   */
/* the call without the suffix, which equals the *_ex call with NULL.     */
/* The two phases of one v2 / auto computation must be given the same     */
/* options: the reduce skips the partitions before the window.           */
/* ---------------------------------------------------------------------- */

pa_status paged_attention_v1_ex(
    void *out, const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, const float *alibi_slopes,
    pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
    const pa_decode_options *options, void *stream);

pa_status paged_attention_v2_ex(
    void *out, float *exp_sums, float *max_logits, void *tmp_out,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, const pa_decode_options *options, void *stream);

pa_status paged_attention_auto_ex(
    void *out, float *exp_sums, float *max_logits, void *tmp_out,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, const pa_decode_options *options, void *stream);

pa_status paged_attention_partition_ex(
    pa_mode mode, void *out, float *exp_sums, float *max_logits, void *tmp_out,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, const pa_decode_options *options, void *stream);

/* Only options->window_left and options->partial_dtype are used here (the
 * soft cap acts in Phase 1); both must be those the partition phase got. */
pa_status paged_attention_reduce_ex(
    pa_mode mode, void *out, const float *exp_sums, const float *max_logits,
    const void *tmp_out, int num_seqs, int num_heads, int num_kv_heads, int head_size,
    const int32_t *seq_lens, int max_seq_len, int max_num_partitions, pa_dtype dtype,
    const pa_decode_options *options, void *stream);

/* ---------------------------------------------------------------------- */
/* Balanced split (work decomposition for ragged batches)                 */
/* ---------------------------------------------------------------------- */

/* The decode of paged_attention_v2_ex with the work cut differently: each
 * sequence's window is split into k <= 64 equal pieces of at least 512 keys
 * (k = 1 for short sequences).  The piece size comes from the batch's shape
 * (num_seqs, KV heads, the window-clipped max_seq_len, the device's compute
 * units): a batch with at least two (sequence, KV head) items per compute
 * unit has its longest sequences cut in about four; a smaller one is cut so
 * that a full-length sequence gives about one piece per compute unit.  The
 * piece that finishes last merges the k partial results with the V2 page's
 * Phase 2 log-sum-exp rescale, inside the same kernel: one launch, no
 * reduce phase.  Compared with paged_attention_auto it pays off on long or
 * ragged batches (no tail of long single-workgroup sequences, no empty
 * partition slots); on a batch whose sequences already fill the device
 * once, the partial stores and merges cost more than they save.  The result equals the v1
 * / v2 result up to rounding (each partial is rounded to the partial dtype
 * of the options, fp32 by default, as tmp_out is).
 *
 * exp_sums, max_logits and tmp_out (shapes as for v2) serve as scratch for
 * the pieces: their contents after the call are unspecified.  counters is
 * int32 [num_seqs, num_heads] (pa_split_counters_size bytes, 4-byte
 * aligned) that must be all zero before the first call; every call leaves
 * it all zero again.  Calls that share a counters buffer must not run
 * concurrently.  Errors are those of paged_attention_v2_ex, plus
 * PA_ERR_NULL_POINTER for counters == NULL and PA_ERR_MISALIGNED for a
 * counters pointer that is not 4-byte aligned. */
pa_status paged_attention_split(
    void *out, float *exp_sums, float *max_logits, void *tmp_out, int32_t *counters,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, const pa_decode_options *options, void *stream);

/* ---------------------------------------------------------------------- */
/* Work list (persistent, cost-balanced scheduling for ragged batches)     */
/* ---------------------------------------------------------------------- */

/* The decode of paged_attention_v2_ex scheduled from a work list built on
 * the device, in one persistent launch of one workgroup per compute unit.
 * The workers are the workgroups, or their waves when the batch has at
 * least two (sequence, KV head) items per wave (many small items); none is
 * without work on a batch of at least 2048 keys per worker.  The items are
 * laid end to end by the work-cost model of the PoD page (FlashInfer PR
 * #967, qo_len + 2 * page_size * kv_len, a model of memory load): the K and
 * V rows of every key in the window, plus a per-item term standing for the
 * item's fixed cost (64 keys' worth, measured); worker w takes the w-th
 * equal share of that line, cutting an item only on 32-key steps and at
 * least 512 keys from either end (so a cut item has at most ceil(L / 512)
 * pieces, and at most 64).  Every worker builds its own entries of the list
 * from seq_lens; each walks its items in order, writes out directly for an
 * item it holds whole, and otherwise stores the piece's partials (slot =
 * piece) and arrives at the item's counter: the last piece merges them with
 * the V2 page's Phase 2 log-sum-exp rescale.  The result equals the v1 / v2
 * result up to rounding (partials rounded to the options' partial dtype,
 * fp32 by default).  Fastest on ragged batches of many short sequences;
 * paged_attention_split is faster on a few long ones.
 *
 * Buffers, counters contract and errors as for paged_attention_split
 * (exp_sums, max_logits and tmp_out are scratch; counters int32 [num_seqs,
 * num_heads], zero before the first call and left zero).  On the BLOCK_ROWS
 * layout only for groups of 3 or more query heads per KV head (the MFMA
 * form); smaller groups there return PA_ERR_UNSUPPORTED. */
pa_status paged_attention_worklist(
    void *out, float *exp_sums, float *max_logits, void *tmp_out, int32_t *counters,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, const pa_decode_options *options, void *stream);

/* The decode of paged_attention_auto_ex for callers that can hand the
 * library a counters buffer: with it, the call schedules the batch for
 * balance instead of by the per-sequence v1 / v2 rule -- the work list
 * (paged_attention_worklist) when the batch's (sequence, KV head group)
 * items fill the device's compute units at least once, else the balanced
 * split (paged_attention_split; also on the block-rows layout for groups
 * of 1 or 2 query heads per KV head, which the work list does not take).  Both run
 * in one launch and merge cut items with the V2 page's Phase 2 rescale
 * ("Phase 2: Reduce across partitions") inside it.  The result equals the
 * v1 / v2 result up to rounding (partials rounded to the options' partial
 * dtype, fp32 by default).  counters == NULL: exactly
 * paged_attention_auto_ex (exp_sums, max_logits and tmp_out then as there).
 * With counters: exp_sums, max_logits and tmp_out are scratch (contents
 * after the call unspecified), counters as for paged_attention_split (int32
 * [num_seqs, num_heads], zero before the first call, left zero; calls that
 * share it must not overlap).  Errors: those of the path taken, checked on
 * the host before any launch. */
pa_status paged_attention_auto_ws(
    void *out, float *exp_sums, float *max_logits, void *tmp_out, int32_t *counters,
    const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
    const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
    float k_scale, float v_scale, const pa_decode_options *options, void *stream);

/* Bytes of the counters buffer of paged_attention_split (0 for non-positive
 * sizes). */
size_t pa_split_counters_size(int num_seqs, int num_heads);

/* Size of the library's device array used by paged_attention_split_static. */
#define PA_SPLIT_STATIC_SCRATCH_BYTES (64u << 20)

/* paged_attention_split for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same decode, the same kernels and the same result, with no
 * exp_sums / max_logits / tmp_out / counters arguments.  The pieces' counters
 * and partials live in a device array the library owns,
 * PA_SPLIT_STATIC_SCRATCH_BYTES (64 MiB) per GPU, held from the first call on
 * that GPU until the process ends; the call allocates and frees nothing.
 * The array holds, each region rounded up to 256 bytes, num_seqs * num_heads
 * int32 counters and, for Z = the split's pieces per sequence at most (1 ..
 * 64, from the batch shape as in paged_attention_split), num_seqs * num_heads
 * * Z exp-sums and max-logits (fp32) and partial rows of head_size elements
 * (fp32, or 2 bytes with options->partial_dtype = PA_PARTIAL_OUT and a 16-bit
 * query).  A call needing more returns PA_ERR_BAD_SHAPE and launches
 * nothing.  Each call first clears its counters with a fill kernel (no
 * memset) on `stream`.  Every call on one GPU shares that GPU's array and
 * leaves its contents behind: calls that overlap on one GPU (different
 * streams, or host threads, without ordering between them) race and give
 * undefined results.  Arguments, options and errors otherwise as for
 * paged_attention_split; out is written, nothing else the caller owns. */
pa_status paged_attention_split_static(
    void *out, const void *query, const void *key_cache, const void *value_cache,
    int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
    int num_blocks, int block_size, int max_seq_len, const float *alibi_slopes,
    pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
    const pa_decode_options *options, void *stream);

/* ---------------------------------------------------------------------- */
/* Paged prefill                                                          */
/* ---------------------------------------------------------------------- */

/* Options of paged_prefill (the dispatch page's AttnDispatchConfig fields
 * is_causal, window_left, window_right, softcap; NULL = causal, no window,
 * no cap, the page's defaults). */
typedef struct pa_prefill_options {
  int causal;             /* nonzero: a query sees no key after its position */
  int window_left;        /* -1: unbounded; W >= 0: keys t >= p - W only     */
  int window_right;       /* -1: unbounded; W >= 0: keys t <= p + W only     */
  float logits_soft_cap;  /* 0: off; c > 0: logit -> c * tanh(logit / c)    */
} pa_prefill_options;

/* Prefill attention over a paged cache (dispatch page, dispatch_prefill:
 * flash attention with block tables and cumulative sequence offsets).
 * Sequence b owns the query rows cu_seq_q[b] .. cu_seq_q[b+1] - 1 (nq_b rows)
 * and nk_b = cu_seq_k[b+1] - cu_seq_k[b] keys, key t in slot t % block_size
 * of block block_tables[b, t / block_size].  The queries are the last nq_b
 * positions of the sequence: query i sits at p = nk_b - nq_b + i, and sees key
 * t iff (!causal || t <= p) and the window bounds hold.  Logits are
 * scale * q . k (soft-capped when asked); the output row is the softmax-
 * weighted sum of the visible values, or zero when no key is visible.
 * Query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Layouts (contiguous, device memory): query, out [total_q, num_heads,
 * head_size] dtype; key_cache, value_cache [num_blocks, num_kv_heads,
 * block_size, head_size] dtype (the page's prefill layout, different from
 * the decode layout); block_tables int32 [num_seqs, max_num_blocks_per_seq];
 * cu_seq_q, cu_seq_k int32 [num_seqs + 1].  max_seq_q / max_seq_k bound the
 * per-sequence query / key counts (host integers).
 *
 * Supported: dtype f16 / bf16 (f32: PA_ERR_UNSUPPORTED); head_size 64 or 128;
 * block_size 16 or 32; num_heads / num_kv_heads <= 128; scale finite and
 * >= 0 (a negative or non-finite scale: PA_ERR_BAD_ARGUMENT).  Errors as for
 * the decode calls; cu_seq_* entries that break max_seq_q / max_seq_k / total_q,
 * and block-table entries outside [0, num_blocks), give NaN rows for that
 * sequence (rows past max_seq_q are not written).  Accumulation is fp32. */
pa_status paged_prefill(
    void *out, const void *query, const void *key_cache, const void *value_cache,
    int total_q, int num_seqs, int num_heads, int num_kv_heads, int head_size, float scale,
    const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *cu_seq_q,
    const int32_t *cu_seq_k, int max_seq_q, int max_seq_k, int num_blocks, int block_size,
    pa_dtype dtype, const pa_prefill_options *options, void *stream);

/* ---------------------------------------------------------------------- */
/* Helpers                                                                */
/* ---------------------------------------------------------------------- */

/* 512 (V2 page, module constant _PARTITION_SIZE). */
int pa_partition_size(void);

/* ceil(max_seq_len / 512): the smallest valid max_num_partitions (0 -> 1). */
int pa_num_partitions(int max_seq_len);

/* The per-sequence v1/v2 rule of PA_MODE_AUTO, on the host.  It is the
 * dispatch page's should_use_paged_v2 ("ex_engine/factors/attn_dispatch.py":
 * tiles = num_kv_heads * ceil(seq_len / 512), v2 iff tiles > 2 * SM count)
 * re-sized to the GPU's compute units, plus one clause of ours for small
 * batches: v2 whenever num_seqs * num_kv_heads < cu_count, because v1 would
 * then leave compute units without a workgroup.  Returns 1 for v2, 0 for v1.
 * Under a sliding window of W >= 0 the auto call passes min(L, W + 1). */
int pa_should_use_v2(int num_seqs, int num_kv_heads, int seq_len, int cu_count);

/* Whether paged_attention_auto(_ex) and the AUTO phases run a batch of this
 * shape as the persistent slot form described at paged_attention_auto
 * (*uses_slots = 1; then its partial buffers are scratch) or by the
 * per-sequence rule (0).  The shape arguments are those of the call;
 * options as for the *_ex calls (NULL: none).  Reads the current device's
 * compute units.  PA_ERR_BAD_ARGUMENT / PA_ERR_BAD_SHAPE / PA_ERR_UNSUPPORTED
 * for arguments the call itself would refuse, PA_ERR_NULL_POINTER for a NULL
 * uses_slots; PA_ERR_HIP if the compute units cannot be read. */
pa_status pa_auto_uses_slots(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                             int block_size, int max_seq_len, pa_dtype dtype,
                             pa_kv_cache_dtype kv_cache_dtype,
                             const pa_decode_options *options, int *uses_slots);

/* Compute units of the current HIP device (cached per device); <= 0 and
 * PA_ERR_HIP if the runtime cannot tell. */
pa_status pa_device_cu_count(int *cu_count);

/* Profiling hook.  For launches made afterwards from the calling thread, the
 * partition-phase kernel records partition_start / partition_stop and the
 * reduce-phase kernel records reduce_start / reduce_stop (hipEvent_t handles
 * created by the caller), through hipExtLaunchKernelGGL: the events carry the
 * kernel's own start and end times, with no queue marker in between.  A
 * NULL pair switches its phase back to plain launches.  A reduce phase with
 * nothing to merge (an all-v1 auto call) records its pair back to back.  The
 * events are re-recorded by every call until replaced.  A pair with one NULL member
 * returns PA_ERR_NULL_POINTER and changes nothing. */
pa_status pa_set_timing_events(void *partition_start, void *partition_stop, void *reduce_start,
                               void *reduce_stop);

/* Measurement hook, not part of attention: the practical HBM read ceiling
 * that the decode kernels' bandwidth is reported against.  Reads `bytes`
 * bytes at `buf` with 16-byte nontemporal loads: num_workgroups workgroups
 * of 256 threads, workgroup w streaming the w-th contiguous share (the same
 * access shape as a partition workgroup's run of tiles), and writes the XOR
 * of the 32-bit words workgroup w read to sink[w].
 *   buf   device memory, 16-byte aligned, caller-owned; bytes a multiple of
 *         16 (0 is allowed: every sink word becomes 0)
 *   sink  device memory, num_workgroups uint32 words, caller-owned
 *   num_workgroups  1 .. 2^31 - 1
 * Errors: PA_ERR_NULL_POINTER (buf or sink NULL), PA_ERR_MISALIGNED (buf not
 * 16-byte aligned or bytes not a multiple of 16), PA_ERR_BAD_SHAPE
 * (num_workgroups < 1), PA_ERR_HIP (launch failure). */
pa_status pa_stream_read(const void *buf, size_t bytes, uint32_t *sink, int num_workgroups,
                         void *stream);

/* Static description of a status code. */
const char *pa_status_string(pa_status status);

/* Library version, "major.minor.patch". */
const char *pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
