// Launch parameters of the paged prefill kernel (shared by the host library
// and the kernel).
#pragma once

#include "pa_launch.h"

namespace pa {

// Query columns of one workgroup: (query token, query head) pairs of one KV
// head, one or two 16-column MFMA tiles per wave (tiles_per_wave).
constexpr int kPrefillMaxCols = 16 * 2 * kWaves;
// Keys per step of the prefill loop (16-key MFMA sub-tiles; a multiple of 32).
constexpr int kPrefillStep = 32;

struct PrefillParams {
  void *out;                  // [total_q, H, D] dtype
  const void *query;          // [total_q, H, D] dtype
  const void *key_cache;      // [NB, Hkv, bs, D] dtype
  const void *value_cache;    // [NB, Hkv, bs, D] dtype
  const int32_t *block_tables;  // [B, max_blocks]
  const int32_t *cu_seq_q;      // [B + 1]
  const int32_t *cu_seq_k;      // [B + 1]
  int total_q, num_seqs, num_heads, num_kv_heads, group;
  int max_num_blocks_per_seq, num_blocks, max_seq_q, max_seq_k;
  int tiles_per_wave;  // 1 or 2 column tiles per wave
  int q_tile;        // query tokens per workgroup: 16 * tiles_per_wave * waves / group
  int num_q_tiles;   // ceil(max_seq_q / q_tile) = grid.x
  int tile_major;    // workgroup order: 1 heaviest tiles of all pairs first, 0 pair by pair
  int causal, window_left, window_right;
  float scale_log2;  // scale * log2(e)
  float cap_in;      // 2 * log2(e) * scale / c
  float cap_out;     // c * log2(e)
};

// Grid: x = query tile (heaviest first), y = KV head, z = sequence.
hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_size, int block_size,
                          bool cap, const Launch &l);

}  // namespace pa
