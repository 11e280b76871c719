// Launch parameters shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Tokens per partition (page "BI-V100 PagedAttention V2 implementation",
// module constant _PARTITION_SIZE).
constexpr int kPartitionSize = 512;
// Every partition-phase workgroup is 4 wave64s; wave w takes logical blocks
// w, w+4, w+8, ... of its token range.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// kModeSplit: balanced split of each sequence into equal pieces sized from
// the batch's total length, merged in the partition kernel by the piece that
// finishes last (paged_attention_split).  kModeList: persistent launch over
// a work list balanced by memory-load cost (paged_attention_worklist); cut
// items are merged the same way.  Both are "piece" modes: out only, the
// partial buffers are scratch.
enum Mode : int { kModeV1 = 0, kModeV2 = 1, kModeAuto = 2, kModeSplit = 3, kModeList = 4 };

// Split mode: the piece target is at least this many keys, so every piece
// but a sequence's only one spans at least 512 keys.
constexpr int kSplitMinPiece = 1024;
// Split mode: at most this many pieces per sequence (the merge keeps their
// statistics in LDS).
constexpr int kSplitMaxPieces = 64;

// Minimum waves per SIMD the register allocator must allow (0: the kernel's
// own choice).
#ifndef PA_WAVES_PER_EU_MFMA
#define PA_WAVES_PER_EU_MFMA 0
#endif
#ifndef PA_WAVES_PER_EU_VALU
#define PA_WAVES_PER_EU_VALU 0
#endif
// KV tiles are read with the nontemporal (streaming) cache policy.
#ifndef PA_NONTEMPORAL
#define PA_NONTEMPORAL 1
#endif

struct Params {
  void *out;            // [B, H, D] dtype
  float *exp_sums;      // [B, H, P]
  float *max_logits;    // [B, H, P]
  void *tmp_out;        // [B, H, P, D] fp32 (tmp_f32) or the query dtype
  const void *query;    // [B, H, D] dtype
  const void *key_cache;    // [NB, Hkv, D/x, bs, x]
  const void *value_cache;  // [NB, Hkv, D, bs]
  const int32_t *block_tables;  // [B, max_num_blocks_per_seq]
  const int32_t *seq_lens;      // [B]
  const float *alibi_slopes;    // [H] or nullptr
  int num_seqs, num_heads, num_kv_heads, group;  // group = H / Hkv
  int max_num_blocks_per_seq, num_blocks, max_seq_len, max_num_partitions;
  int head_groups;      // query-head groups per KV head; grid.x = Hkv * head_groups
  int mode;             // Mode
  int auto_all_v2;      // AUTO: every sequence takes v2 (small batch clause)
  int auto_tile_limit;  // AUTO: v2 iff Hkv * ceil(L / 512) > auto_tile_limit
  int parts_reversed;   // grid z walks the partitions from the last to the first
  float scale_log2;     // scale * k_scale * log2(e): logits are kept in log2 units
  float v_scale;
  int window_left;      // -1: every key; W >= 0: keys t >= L - 1 - W only
  int cap_on;           // logit soft cap c > 0 in use
  float cap_in;         // 2 * log2(e) * scale * k_scale / c: exponent of exp(2 s / c)
  float cap_out;        // c * log2(e): the capped logit in log2 units
  float cap_in_nat;     // 2 * scale * k_scale / c: 2y of tanh(y) (fp32 kernels)
  int tmp_f32;          // partial outputs are stored as fp32 (else in the query dtype)
  int *counters;        // split mode: [B, H] arrival counters, zero between calls
  int split_target;     // split mode: keys per piece before equalising (multiple of 512)
  int item_cost;        // list mode: cost of an item beyond its keys (the query row)
  int list_wave;        // list mode, VALU kernel: 1 = one worker per wave, 2 = the same in
                        // the slot form (auto without counters), 0 = one per workgroup
};

// First key position inside the sliding window of a sequence of length
// L >= 1 (0 without a window).
__host__ __device__ inline int window_first_token(int window_left, int L) {
  return (window_left >= 0 && L - 1 - window_left > 0) ? L - 1 - window_left : 0;
}

}  // namespace pa
