// C ABI of libpagedattn: argument validation, the v1/v2 dispatch rule, kernel
// selection and launches.  Every check runs on the host before any HIP call.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/pagedattn.h"
#include "pa_launch.h"
#include "pa_params.h"
#include "pa_prefill.h"

namespace {

using pa::Params;

// ---------------------------------------------------------------------------
// Tunables.  Defaults are the shipped dispatch; the environment variables
// exist for tuning sweeps only.
// ---------------------------------------------------------------------------
struct Tunables {
  int mfma_min_group = 5;     // query heads per KV head from which the MFMA kernel is used
  // The same on the block-rows layout.  Measured on MI355X (long-context
  // batch, 4 x 100000 keys, 8 KV heads): the MFMA form ties the VALU form at
  // 2 heads per KV head (272 us each) and beats it from 3 (277 vs 321 us;
  // at 4: 274 vs 305 us); at 1 it loses (ragged batch: 2325 vs 2238 us).
  int rows_mfma_min_group = 3;
  int prefill_tiles = 0;      // prefill column tiles per wave: 0 = by shape, else 1 or 2
  int small_batch_factor = 1; // AUTO: v2 for all if B * Hkv < factor * CUs
  int tile_factor = 2;        // AUTO: v2 iff Hkv * ceil(L/512) > factor * CUs
  int parts_reversed = 1;     // all-v2 launches dispatch the last partition first
  int split_reversed = 0;     // split launches dispatch the last piece slice first
  int split_target = 0;       // split: fixed piece target in keys (0: the size rule)
  // List: an item's cost beyond its keys, in keys: the place of the PoD
  // page's qo_len term (the per-request work that does not scale with the
  // cache).  Here it stands for an item's fixed cost -- its epilogue and the
  // latency of its first loads -- which measures at about 64 keys' worth of
  // streaming: on MI355X the ragged ALiBi batch ran at 2104 / 2073 / 2085 /
  // 2088 / 2103 us for 16 / 64 / 128 / 256 / 511.
  int list_item_cost = 64;
  // List: workers per CU (0: as many workgroups as one CU holds at once).
  // One per CU already streams at the device's rate (one workgroup reads up
  // to ~48 GB/s, the device ~28 GB/s per CU); more workers only cut more
  // items into pieces.
  int list_per_cu = 1;
  int list_lds = 0;           // list: dynamic LDS bytes reserved per worker
  int list_wave = -1;         // list: 1 / 0 = one worker per wave / workgroup; -1: by shape
  int auto_slots = 1;         // AUTO: large VALU batches as the slot form of the work list
};

int env_int(const char *name, int fallback, int lo, int hi) {
  const char *s = getenv(name);
  if (!s || !*s) return fallback;
  char *end = nullptr;
  const long v = strtol(s, &end, 10);
  if (*end != '\0' || v < lo || v > hi) return fallback;
  return (int)v;
}

const Tunables &tunables() {
  static const Tunables t = [] {
    Tunables x;
    x.mfma_min_group = env_int("PA_MFMA_MIN_GROUP", x.mfma_min_group, 1, 1 << 20);
    x.rows_mfma_min_group =
        env_int("PA_ROWS_MFMA_MIN_GROUP", x.rows_mfma_min_group, 1, 1 << 20);
    x.prefill_tiles = env_int("PA_PREFILL_TILES", x.prefill_tiles, 0, 2);
    x.small_batch_factor = env_int("PA_AUTO_SMALL_BATCH_FACTOR", x.small_batch_factor, 0, 1 << 20);
    x.tile_factor = env_int("PA_AUTO_TILE_FACTOR", x.tile_factor, 0, 1 << 20);
    x.parts_reversed = env_int("PA_PARTS_REVERSED", x.parts_reversed, 0, 1);
    x.split_reversed = env_int("PA_SPLIT_REVERSED", x.split_reversed, 0, 1);
    x.split_target = env_int("PA_SPLIT_TARGET", x.split_target, 0, 1 << 30);
    x.list_item_cost = env_int("PA_LIST_ITEM_COST", x.list_item_cost, 0, 511);
    x.list_per_cu = env_int("PA_LIST_PER_CU", x.list_per_cu, 0, 16);
    x.list_lds = env_int("PA_LIST_LDS", x.list_lds, 0, 160 * 1024);
    x.list_wave = env_int("PA_LIST_WAVE", x.list_wave, -1, 1);
    x.auto_slots = env_int("PA_AUTO_SLOTS", x.auto_slots, 0, 1);
    return x;
  }();
  return t;
}

// ---------------------------------------------------------------------------
// Per-device compute-unit count, cached.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_cu_mutex;
int g_cu_count[kMaxDevices] = {0};

pa_status cu_count_current(int *cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (g_cu_count[dev] > 0) {
      *cu = g_cu_count[dev];
      return PA_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return PA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    g_cu_count[dev] = n;
  }
  *cu = n;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Profiling hook (pa_set_timing_events): per calling thread.
// ---------------------------------------------------------------------------
struct TimingEvents {
  hipEvent_t partition_start = nullptr, partition_stop = nullptr;
  hipEvent_t reduce_start = nullptr, reduce_stop = nullptr;
};
thread_local TimingEvents t_events;

// ---------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------
struct Call {
  pa_mode mode;
  void *out;
  float *exp_sums, *max_logits;
  void *tmp_out;
  const void *query, *key_cache, *value_cache;
  int num_seqs, num_heads, num_kv_heads, head_size;
  float scale;
  const int32_t *block_tables;
  int max_num_blocks_per_seq;
  const int32_t *seq_lens;
  int num_blocks, block_size, max_seq_len, max_num_partitions;
  const float *alibi_slopes;
  pa_dtype dtype;
  pa_kv_cache_dtype kv_cache_dtype;
  float k_scale, v_scale;
  int window_left;        // pa_decode_options (-1: no window)
  float logits_soft_cap;  // (0: no soft cap)
  int kv_layout;          // pa_kv_layout
  int partial_dtype;      // pa_partial_dtype of tmp_out
  int32_t *counters;      // paged_attention_split only (mode is then V2 for validation)
  bool split;             // a piece mode: split, or list (the work list)
  bool list;
  bool list_slots;        // list: the slot form (AUTO without counters; see auto_slots)
  bool static_scratch;    // the partial buffers and counters are the library's own array
  hipStream_t stream;
};

// Copies the decode options into the call (NULL: every option off, fp32
// partials).
pa_status apply_options(const pa_decode_options *o, Call &c) {
  c.window_left = -1;
  c.logits_soft_cap = 0.0f;
  c.kv_layout = PA_KV_LAYOUT_DECODE;
  c.partial_dtype = PA_PARTIAL_F32;
  if (!o) return PA_OK;
  if (o->window_left < -1) return PA_ERR_BAD_ARGUMENT;
  if (!isfinite(o->logits_soft_cap) || o->logits_soft_cap < 0.0f) return PA_ERR_BAD_ARGUMENT;
  if (o->kv_layout != PA_KV_LAYOUT_DECODE && o->kv_layout != PA_KV_LAYOUT_BLOCK_ROWS)
    return PA_ERR_BAD_ARGUMENT;
  if (o->partial_dtype != PA_PARTIAL_F32 && o->partial_dtype != PA_PARTIAL_OUT)
    return PA_ERR_BAD_ARGUMENT;
  c.window_left = o->window_left;
  c.logits_soft_cap = o->logits_soft_cap;
  c.kv_layout = o->kv_layout;
  c.partial_dtype = o->partial_dtype;
  return PA_OK;
}

// The length the auto rule sees for a sequence of length L: the
// window-clipped min(L, W + 1).
long long rule_length(const Call &c, long long L) {
  if (c.window_left >= 0 && L > (long long)c.window_left + 1) return (long long)c.window_left + 1;
  return L;
}

// Split mode: the piece target in keys, from host-known sizes only (the
// lengths live on the device; L = the window-clipped max_seq_len).  A large
// batch (B * gx >= 2 CUs: every CU already has two (sequence, head group)
// items) only needs its long poles cut: target L / 4.  A smaller batch is
// cut so that sequences of length L give about one piece per CU: target
// B * L * gx / CUs (no cut when the items already fill the CUs once).  At
// least kSplitMinPiece, rounded up to 512.  Measured on MI355X: cutting a
// batch that already fills the CUs once (the GQA and fp8 workloads) costs
// more in partial stores and merges than it gains in balance.
int split_target(const Call &c, long long grid_x, int cu) {
  if (tunables().split_target > 0)
    return (tunables().split_target + 511) / 512 * 512 > pa::kSplitMinPiece
               ? (tunables().split_target + 511) / 512 * 512
               : pa::kSplitMinPiece;
  const long long len = rule_length(c, c.max_seq_len);
  const long long items = (long long)c.num_seqs * grid_x;
  long long t = items >= 2LL * cu ? (len + 3) / 4 : (items * len + cu - 1) / cu;
  t = t > pa::kSplitMinPiece ? t : pa::kSplitMinPiece;
  t = (t + 511) / 512 * 512;
  return (int)(t < (1LL << 30) ? t : (1LL << 30));
}

// Split mode: grid slices per sequence, enough for the pieces of the
// longest window (its aligned start adds up to 31 keys); the kernel clamps
// its piece count to the grid's depth.
int split_grid_z(const Call &c, long long grid_x, int cu) {
  const long long len = rule_length(c, c.max_seq_len) + 31;
  const long long t = split_target(c, grid_x, cu);
  long long z = (len + t - 1) / t;
  if (z < 1) z = 1;
  if (z > pa::kSplitMaxPieces) z = pa::kSplitMaxPieces;
  return (int)z;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

constexpr int kMaxGridYZ = 65535;

pa_status validate_common(const Call &c, bool partition_phase) {
  if (c.mode != PA_MODE_V1 && c.mode != PA_MODE_V2 && c.mode != PA_MODE_AUTO)
    return PA_ERR_BAD_ARGUMENT;
  if (c.dtype != PA_DTYPE_F32 && c.dtype != PA_DTYPE_F16 && c.dtype != PA_DTYPE_BF16)
    return PA_ERR_BAD_ARGUMENT;
  if (c.num_seqs < 0 || c.num_heads <= 0 || c.num_kv_heads <= 0 || c.max_seq_len < 0)
    return PA_ERR_BAD_SHAPE;
  if (c.num_heads % c.num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
  if (c.head_size != 64 && c.head_size != 128) return PA_ERR_UNSUPPORTED;
  if (c.num_seqs > kMaxGridYZ) return PA_ERR_BAD_SHAPE;
  if (!c.out || !c.seq_lens) return PA_ERR_NULL_POINTER;
  if (!aligned16(c.out)) return PA_ERR_MISALIGNED;
  const bool partials = c.mode != PA_MODE_V1 && !c.static_scratch;
  if (partials) {
    if (!c.exp_sums || !c.max_logits || !c.tmp_out) return PA_ERR_NULL_POINTER;
    if (!aligned16(c.tmp_out)) return PA_ERR_MISALIGNED;
    if (c.max_num_partitions < 1 || c.max_num_partitions < pa_num_partitions(c.max_seq_len))
      return PA_ERR_BAD_SHAPE;
  }
  if (c.split && !c.static_scratch) {
    if (!c.counters) return PA_ERR_NULL_POINTER;
    if (((uintptr_t)c.counters & 3u) != 0) return PA_ERR_MISALIGNED;
  }
  if (!partition_phase) return PA_OK;

  if (c.kv_cache_dtype != PA_KV_AUTO && c.kv_cache_dtype != PA_KV_FP8_E4M3)
    return PA_ERR_BAD_ARGUMENT;
  if (c.kv_cache_dtype == PA_KV_FP8_E4M3 && c.dtype == PA_DTYPE_F32) return PA_ERR_UNSUPPORTED;
  // The block-rows layout: 16-bit caches only; the work list only in the
  // MFMA form (groups of rows_mfma_min_group or more query heads).
  if (c.kv_layout == PA_KV_LAYOUT_BLOCK_ROWS &&
      (c.dtype == PA_DTYPE_F32 || c.kv_cache_dtype != PA_KV_AUTO ||
       (c.list && c.num_heads / c.num_kv_heads < tunables().rows_mfma_min_group)))
    return PA_ERR_UNSUPPORTED;
  if (c.block_size != 16 && c.block_size != 32) return PA_ERR_UNSUPPORTED;
  if (pa::kPartitionSize % c.block_size != 0) return PA_ERR_UNSUPPORTED;
  if (!isfinite(c.scale) || !isfinite(c.k_scale) || !isfinite(c.v_scale))
    return PA_ERR_BAD_ARGUMENT;
  // A soft cap so small that scale * k_scale / cap leaves the float range.
  if (c.logits_soft_cap > 0.0f &&
      !isfinite((float)((double)c.scale * (double)c.k_scale / (double)c.logits_soft_cap)))
    return PA_ERR_BAD_ARGUMENT;
  if (!c.query || !c.key_cache || !c.value_cache || !c.block_tables) return PA_ERR_NULL_POINTER;
  if (!aligned16(c.query) || !aligned16(c.key_cache) || !aligned16(c.value_cache))
    return PA_ERR_MISALIGNED;
  if (c.max_num_blocks_per_seq < 0 || c.num_blocks < 0) return PA_ERR_BAD_SHAPE;
  if ((long long)c.max_num_blocks_per_seq * c.block_size < c.max_seq_len) return PA_ERR_BAD_SHAPE;
  if (c.max_seq_len > 0 && c.num_blocks < 1) return PA_ERR_BAD_SHAPE;
  return PA_OK;
}

// Kernel choice for the partition phase.
struct Plan {
  bool mfma;
  int gp;           // query-head slots per workgroup (VALU) / 16 (MFMA)
  int head_groups;  // workgroups per KV head along grid.x
};

Plan make_plan(const Call &c) {
  const int group = c.num_heads / c.num_kv_heads;
  Plan pl{};
  const int min_group = c.kv_layout == PA_KV_LAYOUT_BLOCK_ROWS ? tunables().rows_mfma_min_group
                                                               : tunables().mfma_min_group;
  pl.mfma = c.dtype != PA_DTYPE_F32 && group >= min_group;
  if (pl.mfma) {
    pl.gp = 16;
  } else if (c.kv_layout == PA_KV_LAYOUT_BLOCK_ROWS) {
    const int gmax = pa::nhd_max_group(c.head_size, c.block_size);
    int p2 = 1;
    while (p2 < group && p2 < gmax) p2 *= 2;
    pl.gp = p2;
  } else {
    const int kv_bytes = c.kv_cache_dtype == PA_KV_FP8_E4M3 ? 1 : (c.dtype == PA_DTYPE_F32 ? 4 : 2);
    const int gmax = pa::valu_max_group(kv_bytes, c.head_size, c.block_size);
    int p2 = 1;
    while (p2 < group && p2 < gmax) p2 *= 2;
    pl.gp = p2;
  }
  pl.head_groups = ceil_div(group, pl.gp);
  return pl;
}

Params make_params(const Call &c, int cu, int head_groups) {
  Params p{};
  p.out = c.out;
  p.exp_sums = c.exp_sums;
  p.max_logits = c.max_logits;
  p.tmp_out = c.tmp_out;
  p.query = c.query;
  p.key_cache = c.key_cache;
  p.value_cache = c.value_cache;
  p.block_tables = c.block_tables;
  p.seq_lens = c.seq_lens;
  p.alibi_slopes = c.alibi_slopes;
  p.num_seqs = c.num_seqs;
  p.num_heads = c.num_heads;
  p.num_kv_heads = c.num_kv_heads;
  p.group = c.num_heads / c.num_kv_heads;
  p.max_num_blocks_per_seq = c.max_num_blocks_per_seq;
  p.num_blocks = c.num_blocks;
  p.max_seq_len = c.max_seq_len;
  p.max_num_partitions = c.max_num_partitions;
  p.head_groups = head_groups;
  p.mode = c.list ? pa::kModeList : c.split ? pa::kModeSplit : (int)c.mode;
  p.item_cost = tunables().list_item_cost;
  // List workers: one per wave when the batch has at least two items
  // (sequence, head group) per wave worker -- many small items, where a
  // workgroup-wide epilogue per item would idle the CU -- else one per
  // workgroup.  (VALU kernels only; the MFMA kernels' batches have few,
  // large items per worker.)
  if (c.list) {
    const long long waves = 4LL * cu * (tunables().list_per_cu > 0 ? tunables().list_per_cu : 1);
    p.list_wave = tunables().list_wave >= 0
                      ? tunables().list_wave
                      : ((long long)c.num_seqs * c.num_kv_heads * head_groups >= 2 * waves ? 1 : 0);
    if (c.list_slots) p.list_wave = 2;  // the slot form: wave workers
  }
  p.counters = c.counters;
  p.split_target = c.split ? split_target(c, (long long)c.num_kv_heads * head_groups, cu) : 0;
  const long long b_hkv = (long long)c.num_seqs * c.num_kv_heads;
  p.auto_all_v2 = b_hkv < (long long)tunables().small_batch_factor * cu ? 1 : 0;
  p.auto_tile_limit = tunables().tile_factor * cu;
  p.parts_reversed = c.split ? tunables().split_reversed
                             : tunables().parts_reversed &&
                                       (c.mode == PA_MODE_V2 ||
                                        (c.mode == PA_MODE_AUTO && p.auto_all_v2))
                                   ? 1
                                   : 0;
  p.tmp_f32 = (c.dtype == PA_DTYPE_F32 || c.partial_dtype == PA_PARTIAL_F32) ? 1 : 0;
  p.scale_log2 = c.scale * c.k_scale * 1.4426950408889634f;
  p.v_scale = c.v_scale;
  // A window no sequence outgrows (W >= max_seq_len - 1) clips nothing: the
  // kernels then run their window-free form.
  p.window_left = (c.window_left >= 0 && c.window_left < c.max_seq_len - 1) ? c.window_left : -1;
  p.cap_on = c.logits_soft_cap > 0.0f ? 1 : 0;
  if (p.cap_on) {
    p.cap_in = (float)(2.0 * 1.4426950408889634 * (double)c.scale * (double)c.k_scale /
                       (double)c.logits_soft_cap);
    p.cap_out = (float)((double)c.logits_soft_cap * 1.4426950408889634);
    p.cap_in_nat =
        (float)(2.0 * (double)c.scale * (double)c.k_scale / (double)c.logits_soft_cap);
  }
  return p;
}

// AUTO launches in which every sequence takes v1: the rule is monotone in the
// length, so v1 at max_seq_len (window-clipped) means v1 for every valid
// length (an invalid length also takes the v1 path).  Such a launch runs as
// plain v1: one grid slice instead of one per partition, and no reduce.
bool auto_all_v1(const Call &c, int cu) {
  if (c.mode != PA_MODE_AUTO) return false;
  const Tunables &t = tunables();
  if ((long long)c.num_seqs * c.num_kv_heads < (long long)t.small_batch_factor * cu) return false;
  const int len = (int)rule_length(c, c.max_seq_len);
  return (long long)c.num_kv_heads * pa_num_partitions(len) <= (long long)t.tile_factor * cu;
}

// AUTO calls whose grid would be one workgroup per partition slot of the
// longest sequence for many (sequence, KV head) items -- most of them empty
// in a ragged batch, and the launch then costs their dispatch -- run as the
// slot form of the work list: one worker per wave over equal shares of the
// batch's memory-load cost, piece j of an item stored as the v2 partials of
// partition slot j (an item has no more pieces than partitions; the slots
// past its last piece padded) and merged by the reduce kernel for every
// sequence of two or more partitions.  VALU plans (the MFMA kernel has no
// wave-worker form), the decode layout, no window, and at least two items
// per wave worker.  Both phases decide it alike.
bool auto_slots(const Call &c, int cu) {
  if (c.mode != PA_MODE_AUTO || c.split || c.list || !tunables().auto_slots) return false;
  if (c.kv_layout != PA_KV_LAYOUT_DECODE) return false;
  if (c.window_left >= 0 && c.window_left < c.max_seq_len - 1) return false;
  if (auto_all_v1(c, cu)) return false;
  const Plan pl = make_plan(c);
  if (pl.mfma) return false;
  const long long items = (long long)c.num_seqs * c.num_kv_heads * pl.head_groups;
  return items >= 2LL * pa::kWaves * cu;
}

pa_status run_partition(const Call &c_in) {
  pa_status st = validate_common(c_in, true);
  if (st != PA_OK) return st;
  Call c = c_in;
  if (c.num_seqs > 0 && c.mode == PA_MODE_AUTO && !c.split && !c.list) {
    int cu_a = 0;
    st = cu_count_current(&cu_a);
    if (st != PA_OK) return st;
    if (auto_slots(c, cu_a)) {
      c.list = true;
      c.list_slots = true;
    }
  }
  const Plan pl = make_plan(c);
  const long long grid_x = (long long)c.num_kv_heads * pl.head_groups;
  if (grid_x > 0x7fffffffLL || pa_num_partitions(c.max_seq_len) > kMaxGridYZ)
    return PA_ERR_BAD_SHAPE;
  if (c.num_seqs == 0) return PA_OK;
  int cu = 0;
  if (c.mode == PA_MODE_AUTO || c.split) {  // also the list
    st = cu_count_current(&cu);
    if (st != PA_OK) return st;
  }
  const int gz = c.list    ? 1
                 : c.split ? split_grid_z(c, grid_x, cu)
                 : (c.mode == PA_MODE_V1 || auto_all_v1(c, cu)) ? 1
                                                                : pa_num_partitions(c.max_seq_len);
  const Params p = make_params(c, cu, pl.head_groups);
  pa::Launch l{dim3((unsigned)grid_x, c.num_seqs, gz), c.stream, t_events.partition_start,
               t_events.partition_stop};
  if (c.list) {
    l.list_cus = cu;
    l.list_per_cu = tunables().list_per_cu;
    l.list_lds = tunables().list_lds;
  }
  const bool fp8 = c.kv_cache_dtype == PA_KV_FP8_E4M3;
  hipError_t e;
  if (c.kv_layout == PA_KV_LAYOUT_BLOCK_ROWS) {
    e = pl.mfma ? pa::launch_partition_mfma_rows(p, (int)c.dtype, c.head_size, c.block_size, l)
                : pa::launch_partition_nhd(p, (int)c.dtype, c.head_size, c.block_size, pl.gp, l);
  } else if (pl.mfma) {
    e = pa::launch_partition_mfma(p, (int)c.dtype, fp8, c.head_size, c.block_size, l);
  } else if (fp8) {
    e = pa::launch_partition_valu_fp8(p, (int)c.dtype, c.head_size, c.block_size, pl.gp, l);
  } else if (c.dtype == PA_DTYPE_F32) {
    e = pa::launch_partition_valu_f32(p, c.head_size, c.block_size, pl.gp, l);
  } else if (c.dtype == PA_DTYPE_F16) {
    e = pa::launch_partition_valu_f16(p, c.head_size, c.block_size, pl.gp, l);
  } else {
    e = pa::launch_partition_valu_bf16(p, c.head_size, c.block_size, pl.gp, l);
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status run_reduce(const Call &c) {
  pa_status st = validate_common(c, false);
  if (st != PA_OK) return st;
  if (c.mode == PA_MODE_V1 || c.num_seqs == 0) return PA_OK;
  if ((long long)c.num_heads > 0x7fffffffLL) return PA_ERR_BAD_SHAPE;
  int cu = 0;
  if (c.mode == PA_MODE_AUTO) {
    st = cu_count_current(&cu);
    if (st != PA_OK) return st;
  }
  if (!c.split && !c.list && auto_slots(c, cu)) {
    // The slot form of the partition phase: every sequence of two or more
    // partitions has its slots merged (the v2 rule for all).
    Call cv = c;
    cv.mode = PA_MODE_V2;
    const Params p = make_params(cv, cu, 1);
    const pa::Launch l{dim3(c.num_heads, c.num_seqs, 1), c.stream, t_events.reduce_start,
                       t_events.reduce_stop};
    const hipError_t e = pa::launch_reduce(p, (int)c.dtype, c.head_size, l);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  if (auto_all_v1(c, cu)) {
    // Nothing to merge.  The profiling events still mark an (empty) phase.
    if (t_events.reduce_start && t_events.reduce_stop &&
        (hipEventRecord(t_events.reduce_start, c.stream) != hipSuccess ||
         hipEventRecord(t_events.reduce_stop, c.stream) != hipSuccess))
      return PA_ERR_HIP;
    return PA_OK;
  }
  const Params p = make_params(c, cu, 1);
  const pa::Launch l{dim3(c.num_heads, c.num_seqs, 1), c.stream, t_events.reduce_start,
                     t_events.reduce_stop};
  const hipError_t e = pa::launch_reduce(p, (int)c.dtype, c.head_size, l);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

Call make_call(pa_mode mode, void *out, float *exp_sums, float *max_logits, void *tmp_out,
               const void *query, const void *key_cache, const void *value_cache, int num_seqs,
               int num_heads, int num_kv_heads, int head_size, float scale,
               const int32_t *block_tables, int max_num_blocks_per_seq, const int32_t *seq_lens,
               int num_blocks, int block_size, int max_seq_len, int max_num_partitions,
               const float *alibi_slopes, pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
               float k_scale, float v_scale, void *stream) {
  Call c;
  c.mode = mode;
  c.out = out;
  c.exp_sums = exp_sums;
  c.max_logits = max_logits;
  c.tmp_out = tmp_out;
  c.query = query;
  c.key_cache = key_cache;
  c.value_cache = value_cache;
  c.num_seqs = num_seqs;
  c.num_heads = num_heads;
  c.num_kv_heads = num_kv_heads;
  c.head_size = head_size;
  c.scale = scale;
  c.block_tables = block_tables;
  c.max_num_blocks_per_seq = max_num_blocks_per_seq;
  c.seq_lens = seq_lens;
  c.num_blocks = num_blocks;
  c.block_size = block_size;
  c.max_seq_len = max_seq_len;
  c.max_num_partitions = max_num_partitions;
  c.alibi_slopes = alibi_slopes;
  c.dtype = dtype;
  c.kv_cache_dtype = kv_cache_dtype;
  c.k_scale = k_scale;
  c.v_scale = v_scale;
  c.window_left = -1;
  c.logits_soft_cap = 0.0f;
  c.kv_layout = PA_KV_LAYOUT_DECODE;
  c.partial_dtype = PA_PARTIAL_F32;
  c.counters = nullptr;
  c.split = false;
  c.list = false;
  c.list_slots = false;
  c.static_scratch = false;
  c.stream = reinterpret_cast<hipStream_t>(stream);
  return c;
}

}  // namespace

extern "C" {

pa_status paged_attention_partition_ex(pa_mode mode, void *out, float *exp_sums,
                                       float *max_logits, void *tmp_out, const void *query,
                                       const void *key_cache, const void *value_cache,
                                       int num_seqs, int num_heads, int num_kv_heads,
                                       int head_size, float scale, const int32_t *block_tables,
                                       int max_num_blocks_per_seq, const int32_t *seq_lens,
                                       int num_blocks, int block_size, int max_seq_len,
                                       int max_num_partitions, const float *alibi_slopes,
                                       pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
                                       float k_scale, float v_scale,
                                       const pa_decode_options *options, void *stream) {
  Call c = make_call(mode, out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                     num_seqs, num_heads, num_kv_heads, head_size, scale, block_tables,
                     max_num_blocks_per_seq, seq_lens, num_blocks, block_size, max_seq_len,
                     max_num_partitions, alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                     stream);
  const pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  return run_partition(c);
}

pa_status paged_attention_partition(pa_mode mode, void *out, float *exp_sums, float *max_logits,
                                    void *tmp_out, const void *query, const void *key_cache,
                                    const void *value_cache, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_size, float scale,
                                    const int32_t *block_tables, int max_num_blocks_per_seq,
                                    const int32_t *seq_lens, int num_blocks, int block_size,
                                    int max_seq_len, int max_num_partitions,
                                    const float *alibi_slopes, pa_dtype dtype,
                                    pa_kv_cache_dtype kv_cache_dtype, float k_scale,
                                    float v_scale, void *stream) {
  return paged_attention_partition_ex(mode, out, exp_sums, max_logits, tmp_out, query, key_cache,
                                      value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                                      scale, block_tables, max_num_blocks_per_seq, seq_lens,
                                      num_blocks, block_size, max_seq_len, max_num_partitions,
                                      alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                                      nullptr, stream);
}

pa_status paged_attention_reduce_ex(pa_mode mode, void *out, const float *exp_sums,
                                    const float *max_logits, const void *tmp_out, int num_seqs,
                                    int num_heads, int num_kv_heads, int head_size,
                                    const int32_t *seq_lens, int max_seq_len,
                                    int max_num_partitions, pa_dtype dtype,
                                    const pa_decode_options *options, void *stream) {
  Call c = make_call(mode, out, const_cast<float *>(exp_sums), const_cast<float *>(max_logits),
                     const_cast<void *>(tmp_out), nullptr, nullptr, nullptr, num_seqs, num_heads,
                     num_kv_heads, head_size, 1.0f, nullptr, 0, seq_lens, 0, 16, max_seq_len,
                     max_num_partitions, nullptr, dtype, PA_KV_AUTO, 1.0f, 1.0f, stream);
  const pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  return run_reduce(c);
}

pa_status paged_attention_reduce(pa_mode mode, void *out, const float *exp_sums,
                                 const float *max_logits, const void *tmp_out, int num_seqs,
                                 int num_heads, int num_kv_heads, int head_size,
                                 const int32_t *seq_lens, int max_seq_len, int max_num_partitions,
                                 pa_dtype dtype, void *stream) {
  return paged_attention_reduce_ex(mode, out, exp_sums, max_logits, tmp_out, num_seqs, num_heads,
                                   num_kv_heads, head_size, seq_lens, max_seq_len,
                                   max_num_partitions, dtype, nullptr, stream);
}

static pa_status two_phase(pa_mode mode, void *out, float *exp_sums, float *max_logits,
                           void *tmp_out, const void *query, const void *key_cache,
                           const void *value_cache, int num_seqs, int num_heads, int num_kv_heads,
                           int head_size, float scale, const int32_t *block_tables,
                           int max_num_blocks_per_seq, const int32_t *seq_lens, int num_blocks,
                           int block_size, int max_seq_len, int max_num_partitions,
                           const float *alibi_slopes, pa_dtype dtype,
                           pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                           const pa_decode_options *options, void *stream) {
  Call c = make_call(mode, out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                     num_seqs, num_heads, num_kv_heads, head_size, scale, block_tables,
                     max_num_blocks_per_seq, seq_lens, num_blocks, block_size, max_seq_len,
                     max_num_partitions, alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                     stream);
  // Validate both phases before launching either.
  pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  st = validate_common(c, true);
  if (st != PA_OK) return st;
  st = run_partition(c);
  if (st != PA_OK) return st;
  return run_reduce(c);
}

pa_status paged_attention_v1_ex(void *out, const void *query, const void *key_cache,
                                const void *value_cache, int num_seqs, int num_heads,
                                int num_kv_heads, int head_size, float scale,
                                const int32_t *block_tables, int max_num_blocks_per_seq,
                                const int32_t *seq_lens, int num_blocks, int block_size,
                                int max_seq_len, const float *alibi_slopes, pa_dtype dtype,
                                pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                                const pa_decode_options *options, void *stream) {
  Call c = make_call(PA_MODE_V1, out, nullptr, nullptr, nullptr, query, key_cache, value_cache,
                     num_seqs, num_heads, num_kv_heads, head_size, scale, block_tables,
                     max_num_blocks_per_seq, seq_lens, num_blocks, block_size, max_seq_len, 1,
                     alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale, stream);
  const pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  return run_partition(c);
}

pa_status paged_attention_v1(void *out, const void *query, const void *key_cache,
                             const void *value_cache, int num_seqs, int num_heads,
                             int num_kv_heads, int head_size, float scale,
                             const int32_t *block_tables, int max_num_blocks_per_seq,
                             const int32_t *seq_lens, int num_blocks, int block_size,
                             int max_seq_len, const float *alibi_slopes, pa_dtype dtype,
                             pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                             void *stream) {
  return paged_attention_v1_ex(out, query, key_cache, value_cache, num_seqs, num_heads,
                               num_kv_heads, head_size, scale, block_tables,
                               max_num_blocks_per_seq, seq_lens, num_blocks, block_size,
                               max_seq_len, alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                               nullptr, stream);
}

pa_status paged_attention_v2_ex(void *out, float *exp_sums, float *max_logits, void *tmp_out,
                                const void *query, const void *key_cache,
                                const void *value_cache, int num_seqs, int num_heads,
                                int num_kv_heads, int head_size, float scale,
                                const int32_t *block_tables, int max_num_blocks_per_seq,
                                const int32_t *seq_lens, int num_blocks, int block_size,
                                int max_seq_len, int max_num_partitions,
                                const float *alibi_slopes, pa_dtype dtype,
                                pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                                const pa_decode_options *options, void *stream) {
  return two_phase(PA_MODE_V2, out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                   num_seqs, num_heads, num_kv_heads, head_size, scale, block_tables,
                   max_num_blocks_per_seq, seq_lens, num_blocks, block_size, max_seq_len,
                   max_num_partitions, alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                   options, stream);
}

pa_status paged_attention_v2(void *out, float *exp_sums, float *max_logits, void *tmp_out,
                             const void *query, const void *key_cache, const void *value_cache,
                             int num_seqs, int num_heads, int num_kv_heads, int head_size,
                             float scale, const int32_t *block_tables, int max_num_blocks_per_seq,
                             const int32_t *seq_lens, int num_blocks, int block_size,
                             int max_seq_len, int max_num_partitions, const float *alibi_slopes,
                             pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype, float k_scale,
                             float v_scale, void *stream) {
  return two_phase(PA_MODE_V2, out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                   num_seqs, num_heads, num_kv_heads, head_size, scale, block_tables,
                   max_num_blocks_per_seq, seq_lens, num_blocks, block_size, max_seq_len,
                   max_num_partitions, alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                   nullptr, stream);
}

pa_status paged_attention_auto_ex(void *out, float *exp_sums, float *max_logits, void *tmp_out,
                                  const void *query, const void *key_cache,
                                  const void *value_cache, int num_seqs, int num_heads,
                                  int num_kv_heads, int head_size, float scale,
                                  const int32_t *block_tables, int max_num_blocks_per_seq,
                                  const int32_t *seq_lens, int num_blocks, int block_size,
                                  int max_seq_len, int max_num_partitions,
                                  const float *alibi_slopes, pa_dtype dtype,
                                  pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                                  const pa_decode_options *options, void *stream) {
  return two_phase(PA_MODE_AUTO, out, exp_sums, max_logits, tmp_out, query, key_cache,
                   value_cache, num_seqs, num_heads, num_kv_heads, head_size, scale, block_tables,
                   max_num_blocks_per_seq, seq_lens, num_blocks, block_size, max_seq_len,
                   max_num_partitions, alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                   options, stream);
}

pa_status paged_attention_auto(void *out, float *exp_sums, float *max_logits, void *tmp_out,
                               const void *query, const void *key_cache, const void *value_cache,
                               int num_seqs, int num_heads, int num_kv_heads, int head_size,
                               float scale, const int32_t *block_tables,
                               int max_num_blocks_per_seq, const int32_t *seq_lens,
                               int num_blocks, int block_size, int max_seq_len,
                               int max_num_partitions, const float *alibi_slopes, pa_dtype dtype,
                               pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                               void *stream) {
  return two_phase(PA_MODE_AUTO, out, exp_sums, max_logits, tmp_out, query, key_cache,
                   value_cache, num_seqs, num_heads, num_kv_heads, head_size, scale, block_tables,
                   max_num_blocks_per_seq, seq_lens, num_blocks, block_size, max_seq_len,
                   max_num_partitions, alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                   nullptr, stream);
}

pa_status paged_attention_split(void *out, float *exp_sums, float *max_logits, void *tmp_out,
                                int32_t *counters, const void *query, const void *key_cache,
                                const void *value_cache, int num_seqs, int num_heads,
                                int num_kv_heads, int head_size, float scale,
                                const int32_t *block_tables, int max_num_blocks_per_seq,
                                const int32_t *seq_lens, int num_blocks, int block_size,
                                int max_seq_len, int max_num_partitions,
                                const float *alibi_slopes, pa_dtype dtype,
                                pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                                const pa_decode_options *options, void *stream) {
  Call c = make_call(PA_MODE_V2, out, exp_sums, max_logits, tmp_out, query, key_cache,
                     value_cache, num_seqs, num_heads, num_kv_heads, head_size, scale,
                     block_tables, max_num_blocks_per_seq, seq_lens, num_blocks, block_size,
                     max_seq_len, max_num_partitions, alibi_slopes, dtype, kv_cache_dtype,
                     k_scale, v_scale, stream);
  c.split = true;
  c.counters = counters;
  const pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  return run_partition(c);
}

pa_status paged_attention_worklist(void *out, float *exp_sums, float *max_logits,
                                   void *tmp_out, int32_t *counters, const void *query,
                                   const void *key_cache, const void *value_cache, int num_seqs,
                                   int num_heads, int num_kv_heads, int head_size, float scale,
                                   const int32_t *block_tables, int max_num_blocks_per_seq,
                                   const int32_t *seq_lens, int num_blocks, int block_size,
                                   int max_seq_len, int max_num_partitions,
                                   const float *alibi_slopes, pa_dtype dtype,
                                   pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                                   const pa_decode_options *options, void *stream) {
  Call c = make_call(PA_MODE_V2, out, exp_sums, max_logits, tmp_out, query, key_cache,
                     value_cache, num_seqs, num_heads, num_kv_heads, head_size, scale,
                     block_tables, max_num_blocks_per_seq, seq_lens, num_blocks, block_size,
                     max_seq_len, max_num_partitions, alibi_slopes, dtype, kv_cache_dtype,
                     k_scale, v_scale, stream);
  c.split = true;
  c.list = true;
  c.counters = counters;
  const pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  return run_partition(c);
}

pa_status paged_attention_auto_ws(void *out, float *exp_sums, float *max_logits, void *tmp_out,
                                  int32_t *counters, const void *query, const void *key_cache,
                                  const void *value_cache, int num_seqs, int num_heads,
                                  int num_kv_heads, int head_size, float scale,
                                  const int32_t *block_tables, int max_num_blocks_per_seq,
                                  const int32_t *seq_lens, int num_blocks, int block_size,
                                  int max_seq_len, int max_num_partitions,
                                  const float *alibi_slopes, pa_dtype dtype,
                                  pa_kv_cache_dtype kv_cache_dtype, float k_scale, float v_scale,
                                  const pa_decode_options *options, void *stream) {
  if (!counters)
    return paged_attention_auto_ex(out, exp_sums, max_logits, tmp_out, query, key_cache,
                                   value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                                   scale, block_tables, max_num_blocks_per_seq, seq_lens,
                                   num_blocks, block_size, max_seq_len, max_num_partitions,
                                   alibi_slopes, dtype, kv_cache_dtype, k_scale, v_scale,
                                   options, stream);
  Call c = make_call(PA_MODE_V2, out, exp_sums, max_logits, tmp_out, query, key_cache,
                     value_cache, num_seqs, num_heads, num_kv_heads, head_size, scale,
                     block_tables, max_num_blocks_per_seq, seq_lens, num_blocks, block_size,
                     max_seq_len, max_num_partitions, alibi_slopes, dtype, kv_cache_dtype,
                     k_scale, v_scale, stream);
  c.split = true;
  c.counters = counters;
  pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  st = validate_common(c, true);
  if (st != PA_OK || num_seqs == 0) return st;
  int cu = 0;
  st = cu_count_current(&cu);
  if (st != PA_OK) return st;
  // The work list where the items fill the CUs at least once; the split
  // for fewer, longer items, and for the block-rows layout's VALU form,
  // which has no list form.
  const Plan pl = make_plan(c);
  const long long items = (long long)num_seqs * num_kv_heads * pl.head_groups;
  c.list = items >= cu && (c.kv_layout == PA_KV_LAYOUT_DECODE || pl.mfma);
  return run_partition(c);
}

pa_status paged_attention_split_static(void *out, const void *query, const void *key_cache,
                                       const void *value_cache, int num_seqs, int num_heads,
                                       int num_kv_heads, int head_size, float scale,
                                       const int32_t *block_tables, int max_num_blocks_per_seq,
                                       const int32_t *seq_lens, int num_blocks, int block_size,
                                       int max_seq_len, const float *alibi_slopes,
                                       pa_dtype dtype, pa_kv_cache_dtype kv_cache_dtype,
                                       float k_scale, float v_scale,
                                       const pa_decode_options *options, void *stream) {
  Call c = make_call(PA_MODE_V2, out, nullptr, nullptr, nullptr, query, key_cache, value_cache,
                     num_seqs, num_heads, num_kv_heads, head_size, scale, block_tables,
                     max_num_blocks_per_seq, seq_lens, num_blocks, block_size, max_seq_len,
                     pa_num_partitions(max_seq_len), alibi_slopes, dtype, kv_cache_dtype, k_scale,
                     v_scale, stream);
  c.split = true;
  c.static_scratch = true;
  pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  st = validate_common(c, true);
  if (st != PA_OK) return st;
  if (c.num_seqs == 0) return PA_OK;
  // The pieces' scratch, laid out in the library's array: counters
  // [B, H] int32, then exp_sums and max_logits [B, H, Z] and tmp_out
  // [B, H, Z, D], Z = the split grid's depth (a piece's slot is its index,
  // below Z), each region 256-byte aligned.
  const Plan pl = make_plan(c);
  const long long grid_x = (long long)c.num_kv_heads * pl.head_groups;
  int cu = 0;
  st = cu_count_current(&cu);
  if (st != PA_OK) return st;
  const int gz = split_grid_z(c, grid_x, cu);
  const size_t tsz = (c.dtype == PA_DTYPE_F32 || c.partial_dtype == PA_PARTIAL_F32) ? 4 : 2;
  const size_t rows = (size_t)c.num_seqs * (size_t)c.num_heads;
  auto up = [](size_t n) { return (n + 255) / 256 * 256; };
  const size_t off_es = up(rows * 4);
  const size_t off_ml = off_es + up(rows * gz * 4);
  const size_t off_to = off_ml + up(rows * gz * 4);
  const size_t need = off_to + up(rows * gz * (size_t)c.head_size * tsz);
  if (need > (size_t)PA_SPLIT_STATIC_SCRATCH_BYTES) return PA_ERR_BAD_SHAPE;
  char *base = nullptr;
  st = pa::static_scratch(reinterpret_cast<void **>(&base));
  if (st != PA_OK) return st;
  c.counters = reinterpret_cast<int32_t *>(base);
  c.exp_sums = reinterpret_cast<float *>(base + off_es);
  c.max_logits = reinterpret_cast<float *>(base + off_ml);
  c.tmp_out = base + off_to;
  c.max_num_partitions = gz;
  // Counters start at zero on every call (a fill kernel, no memset node).
  if (pa::launch_fill_zero(c.counters, rows, c.stream) != hipSuccess) return PA_ERR_HIP;
  return run_partition(c);
}

pa_status paged_prefill(void *out, const void *query, const void *key_cache,
                        const void *value_cache, int total_q, int num_seqs, int num_heads,
                        int num_kv_heads, int head_size, float scale, const int32_t *block_tables,
                        int max_num_blocks_per_seq, const int32_t *cu_seq_q,
                        const int32_t *cu_seq_k, int max_seq_q, int max_seq_k, int num_blocks,
                        int block_size, pa_dtype dtype, const pa_prefill_options *options,
                        void *stream) {
  pa_prefill_options o{1, -1, -1, 0.0f};
  if (options) o = *options;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16)
    return PA_ERR_BAD_ARGUMENT;
  // A negative scale is refused: the kernel's step max is the max of the raw
  // dot products scaled once, the max logit only for scale >= 0.
  if (o.window_left < -1 || o.window_right < -1 || !isfinite(o.logits_soft_cap) ||
      o.logits_soft_cap < 0.0f || !isfinite(scale) || scale < 0.0f)
    return PA_ERR_BAD_ARGUMENT;
  if (o.logits_soft_cap > 0.0f &&
      !isfinite((float)((double)scale / (double)o.logits_soft_cap)))
    return PA_ERR_BAD_ARGUMENT;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || total_q < 0 || max_seq_q < 0 ||
      max_seq_k < 0 || max_num_blocks_per_seq < 0 || num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  if (num_heads % num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
  const int group = num_heads / num_kv_heads;
  if (group > pa::kPrefillMaxCols) return PA_ERR_UNSUPPORTED;
  if (num_seqs > kMaxGridYZ || num_kv_heads > kMaxGridYZ) return PA_ERR_BAD_SHAPE;
  if (dtype == PA_DTYPE_F32) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !cu_seq_q || !cu_seq_k)
    return PA_ERR_NULL_POINTER;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return PA_ERR_MISALIGNED;
  if ((long long)max_num_blocks_per_seq * block_size < max_seq_k) return PA_ERR_BAD_SHAPE;
  if (max_seq_k > 0 && num_blocks < 1) return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0 || total_q == 0 || max_seq_q == 0) return PA_OK;
  pa::PrefillParams p{};
  p.out = out;
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.cu_seq_q = cu_seq_q;
  p.cu_seq_k = cu_seq_k;
  p.total_q = total_q;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.max_num_blocks_per_seq = max_num_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.max_seq_q = max_seq_q;
  p.max_seq_k = max_seq_k;
  // Two column tiles per wave (each K / V fragment read from LDS feeds
  // both) when each query sees many keys (chunked prefill), or when the
  // two-tile grid still gives every CU two workgroups; one otherwise (small
  // fresh batches: more, shorter workgroups fill the CUs).  A group wider
  // than one tile's worth of columns needs two.  Measured on MI355X with the
  // XCD mapping: 8 fresh 2048-token prompts 0.495 ms with two tiles vs 0.543
  // with one; 16 chunks of 512 over 8192 keys 1.62 vs 1.86 ms.
  int cu = 0;
  const pa_status cst = cu_count_current(&cu);
  if (cst != PA_OK) return cst;
  const int q_tile2 = 16 * 2 * pa::kWaves / group;
  const long long grid2 = ((long long)max_seq_q + q_tile2 - 1) / q_tile2 * num_kv_heads * num_seqs;
  p.tiles_per_wave =
      (max_seq_k >= 2LL * max_seq_q || group > 16 * pa::kWaves || grid2 >= 2LL * cu) ? 2 : 1;
  if (tunables().prefill_tiles > 0 && group <= 16 * pa::kWaves)
    p.tiles_per_wave = tunables().prefill_tiles;
  p.q_tile = 16 * p.tiles_per_wave * pa::kWaves / group;
  const long long tiles = ((long long)max_seq_q + p.q_tile - 1) / p.q_tile;
  if (tiles > 0x7fffffffLL) return PA_ERR_BAD_SHAPE;
  p.num_q_tiles = (int)tiles;
  p.causal = o.causal ? 1 : 0;
  // Tile-major order when the tiles' costs differ widely: causal, with
  // fewer than twice as many keys as queries (tile t of a prompt sees the
  // prefix plus t + 1 tiles of keys, so costs span more than 2:1).
  p.tile_major = (o.causal && (long long)max_seq_k < 2LL * max_seq_q) ? 1 : 0;
  p.window_left = o.window_left;
  p.window_right = o.window_right;
  p.scale_log2 = scale * 1.4426950408889634f;
  // The uncapped kernel folds the scale into each weight's fma and masks a
  // key by giving it a raw logit of -inf, which needs scale_log2 > 0.  A
  // zero scale makes every logit 0, as c tanh(0 / c) = 0 does for any cap
  // c: it runs the capped kernel with c = 1.
  const bool cap = o.logits_soft_cap > 0.0f || p.scale_log2 == 0.0f;
  if (cap) {
    const double c = o.logits_soft_cap > 0.0f ? (double)o.logits_soft_cap : 1.0;
    p.cap_in = (float)(2.0 * 1.4426950408889634 * (double)scale / c);
    p.cap_out = (float)(c * 1.4426950408889634);
  }
  const pa::Launch l{dim3((unsigned)tiles, num_kv_heads, num_seqs),
                     reinterpret_cast<hipStream_t>(stream), t_events.partition_start,
                     t_events.partition_stop};
  const hipError_t e = pa::launch_prefill(p, (int)dtype, head_size, block_size, cap, l);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t pa_split_counters_size(int num_seqs, int num_heads) {
  if (num_seqs <= 0 || num_heads <= 0) return 0;
  return (size_t)num_seqs * (size_t)num_heads * sizeof(int32_t);
}

pa_status pa_set_timing_events(void *partition_start, void *partition_stop, void *reduce_start,
                               void *reduce_stop) {
  if ((partition_start == nullptr) != (partition_stop == nullptr) ||
      (reduce_start == nullptr) != (reduce_stop == nullptr))
    return PA_ERR_NULL_POINTER;
  t_events.partition_start = reinterpret_cast<hipEvent_t>(partition_start);
  t_events.partition_stop = reinterpret_cast<hipEvent_t>(partition_stop);
  t_events.reduce_start = reinterpret_cast<hipEvent_t>(reduce_start);
  t_events.reduce_stop = reinterpret_cast<hipEvent_t>(reduce_stop);
  return PA_OK;
}

int pa_partition_size(void) { return pa::kPartitionSize; }

int pa_num_partitions(int max_seq_len) {
  if (max_seq_len <= 0) return 1;
  return ceil_div(max_seq_len, pa::kPartitionSize);
}

int pa_should_use_v2(int num_seqs, int num_kv_heads, int seq_len, int cu_count) {
  const Tunables &t = tunables();
  if ((long long)num_seqs * num_kv_heads < (long long)t.small_batch_factor * cu_count) return 1;
  const long long tiles = (long long)num_kv_heads * (seq_len <= 0 ? 0 : ceil_div(seq_len, pa::kPartitionSize));
  return tiles > (long long)t.tile_factor * cu_count ? 1 : 0;
}

pa_status pa_auto_uses_slots(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                             int block_size, int max_seq_len, pa_dtype dtype,
                             pa_kv_cache_dtype kv_cache_dtype, const pa_decode_options *options,
                             int *uses_slots) {
  if (!uses_slots) return PA_ERR_NULL_POINTER;
  *uses_slots = 0;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16)
    return PA_ERR_BAD_ARGUMENT;
  if (kv_cache_dtype != PA_KV_AUTO && kv_cache_dtype != PA_KV_FP8_E4M3) return PA_ERR_BAD_ARGUMENT;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
      num_heads % num_kv_heads != 0)
    return PA_ERR_BAD_SHAPE;
  if ((head_size != 64 && head_size != 128) || (block_size != 16 && block_size != 32))
    return PA_ERR_UNSUPPORTED;
  Call c = make_call(PA_MODE_AUTO, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     num_seqs, num_heads, num_kv_heads, head_size, 1.0f, nullptr, 0, nullptr, 0,
                     block_size, max_seq_len, pa_num_partitions(max_seq_len), nullptr, dtype,
                     kv_cache_dtype, 1.0f, 1.0f, nullptr);
  const pa_status st = apply_options(options, c);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  int cu = 0;
  const pa_status cs = cu_count_current(&cu);
  if (cs != PA_OK) return cs;
  *uses_slots = auto_slots(c, cu) ? 1 : 0;
  return PA_OK;
}

pa_status pa_device_cu_count(int *cu_count) {
  if (!cu_count) return PA_ERR_NULL_POINTER;
  *cu_count = 0;
  return cu_count_current(cu_count);
}

pa_status pa_stream_read(const void *buf, size_t bytes, uint32_t *sink, int num_workgroups,
                         void *stream) {
  if (!buf || !sink) return PA_ERR_NULL_POINTER;
  if (!aligned16(buf) || bytes % 16 != 0) return PA_ERR_MISALIGNED;
  if (num_workgroups < 1) return PA_ERR_BAD_SHAPE;
  const hipError_t e = pa::launch_stream_read(buf, bytes, sink, num_workgroups,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

const char *pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case PA_ERR_BAD_SHAPE: return "sizes are inconsistent or out of range";
    case PA_ERR_MISALIGNED: return "a cache, query, out or tmp_out pointer is not 16-byte aligned";
    case PA_ERR_UNSUPPORTED: return "unsupported head_size, block_size or dtype combination";
    case PA_ERR_HIP: return "the HIP runtime reported an error";
    case PA_ERR_BAD_ARGUMENT: return "non-finite scale or unknown enum value";
  }
  return "unknown status";
}

const char *pa_version(void) { return "0.2.0"; }

}  // extern "C"
