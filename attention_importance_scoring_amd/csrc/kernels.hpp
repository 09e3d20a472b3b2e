// Internal launch interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

// One scoring problem: units u = (layer, KV head); each unit has R query
// rows (G query heads x rows_per_qhead) and n_keys scored keys.
struct ScoreArgs {
  const void* q;            // [layers][Hq][rows_per_qhead][D]
  const void* k;            // [layers][Hkv][k_head_stride]
  int64_t q_layer_stride;   // elements
  int64_t q_head_stride;    // elements
  int64_t k_layer_stride;   // elements
  int64_t k_head_stride;    // elements
  int32_t layer0;           // first layer scored (SpecPC: l_skip)
  int32_t n_units;          // (layers - layer0) * heads per layer
  int32_t n_kv_heads;       // heads per layer (unit % n_kv_heads is the head)
  int32_t kv_repeat;        // heads per KV head (>1: one unit per query head); KV head = head / kv_repeat
  int32_t agg_max;          // pass 2 aggregates the rows by max instead of sum
  int32_t group;            // G = Hq / Hkv
  int32_t rows_per_qhead;   // SpecKV: n_window + n_lookahead; SpecPC: W
  int32_t n_rows;           // R = G * rows_per_qhead
  int32_t n_keys;           // SpecKV: n_pre; SpecPC: n_in
  int32_t n_chunks;         // key chunks per unit (pass 1 partial count)
  int32_t n_sub;            // groups of resident keys per chunk (score_plan)
  int32_t rows_per_part;    // query rows a block holds in LDS (multiple of 32)
  int32_t n_parts;          // ceil(n_rows / rows_per_part); one block per (unit, chunk, part)
  int32_t causal;           // SpecPC: row i sees keys j <= pos_base + i
  int64_t pos_base;         // SpecPC: n_in - W
  float c;                  // logit scale * log2(e)
  float2* part;             // pass 1 output: [n_units][n_chunks][R] (max, sum) in log2 units
  float* lam;               // combine output / pass 2 input: [n_units][R] log2-domain lse
  float* scores;            // pass 2 output: [n_units][n_keys]
  float* colpart;           // pass 2, parts 1 ..: [n_parts - 1][n_units][n_keys] column sums (or maxima)
  const int32_t* key_rows;  // NULL, or key j is row key_rows[j] (clamped to [0, key_row_limit)) of the head slab
  int32_t key_row_limit;
};

// Work plan of the two scoring passes for one problem size.
struct ScorePlan {
  int32_t n_sub, n_chunks, rows_per_part, n_parts;
  int32_t kt;                   // key tiles of 32 per wave (2 or 4)
  size_t lds_pass1, lds_pass2;  // dynamic LDS bytes per block
};
void score_plan(int dtype, int head_dim, int64_t n_units, int64_t n_rows, int64_t n_keys, ScorePlan* pl);
int64_t score_plan_target_blocks();  // blocks per launch the planner aims at
hipError_t launch_score_pass1(int dtype, int head_dim, int kt, const ScoreArgs& a, size_t lds, hipStream_t s);
hipError_t launch_lse_combine(const ScoreArgs& a, hipStream_t s);
hipError_t launch_score_pass2(int dtype, int head_dim, int kt, const ScoreArgs& a, size_t lds, hipStream_t s);
hipError_t launch_colsum_combine(const ScoreArgs& a, hipStream_t s);  // when n_parts > 1

// SpecPC pass 2: mean over (layer, query head) of the causal probabilities,
// weighted max over window rows, per key.
struct SpecPCArgs {
  ScoreArgs sc;             // same problem description (causal), lam filled
  const float* weights;     // [W] or nullptr (linear 0.1 .. 1)
  float* rowblock_max;      // [n_rowblocks][n_in] partial maxima (workspace)
  float* token_scores;      // [n_in]
  int32_t n_rowblocks;
  int32_t maps_per_stage;   // set by the launcher
  float inv_maps;           // 1 / ((L - l_skip) * Hq)
};
int specpc_rows_per_block(int dtype, int head_dim);
int specpc_keys_per_block(int dtype, int head_dim);
hipError_t launch_specpc_pass2(int dtype, int head_dim, const SpecPCArgs& a, hipStream_t s);
hipError_t launch_specpc_reduce(const SpecPCArgs& a, hipStream_t s);

// Pooling + top-k selection, one block per unit.
struct SelectArgs {
  const float* scores;      // [n_units][n_pre]
  float* pooled;            // [n_units][n_pre]
  int32_t* kept;            // [n_units][n_keep]
  int32_t n_units;
  int32_t n_pre;
  int32_t n_window;
  int32_t n_top;            // min(C_max, n_pre)
  int32_t pool;             // skv_pool
  int32_t pool_radius;      // pool_kernel / 2
  int32_t write_pooled;     // 0: `pooled` is workspace that only the run-time pool path needs
  // Two-stage form for long units with few heads: n_seg segments of seg_len
  // keys each keep their local top n_top as (key, index) candidates in
  // [n_units][n_seg][n_top] (workspace); a second kernel selects among them.
  int32_t n_seg;
  int32_t seg_len;
  uint32_t* cand_key;
  int32_t* cand_idx;
};
// Segments per unit for the two-stage form (1: single stage) and its workspace bytes.
int select_segments(int64_t n_units, int64_t n_pre, int64_t n_top);
size_t select_candidate_bytes(int64_t n_units, int64_t n_pre, int64_t n_top);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

// Row gather: dst[u][t] = src[u][idx[u * idx_unit_stride + t]] (or src[u][t] when idx is null);
// with src2 set, the same gather from src2 into dst2 in the same launch (K and V together).
struct GatherArgs {
  const void* src;
  void* dst;
  const void* src2;         // NULL, or a second tensor gathered with the same indices
  void* dst2;
  const int32_t* idx;       // per-unit lists (idx_unit_stride = n_rows), one shared list (0), or nullptr
  const int32_t* idx2;      // NULL, or a shared list the first index goes through: row idx2[idx[...]]
  int32_t n_idx2;           // entries of idx2 (a first index outside [0, n_idx2) gives a zero row)
  int64_t idx_unit_stride;  // elements
  int64_t src_unit_stride;  // bytes
  int64_t dst_unit_stride;  // bytes
  int32_t n_units;          // destination units
  int32_t units_per_layer;  // destination units per layer
  int32_t src_units_per_layer;
  int32_t src_repeat;       // destination units per source unit within a layer
  int32_t n_rows;           // rows per unit to write
  int32_t n_src_rows;       // valid source rows per unit (bounds check)
  int32_t row_bytes;        // multiple of 16
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

// Decode attention: units u = (layer, cache head); each unit's `group`
// query heads attend over its first n_rows cached rows.
struct DecodeArgs {
  const void* q;              // [layers * q_heads_per_layer][D] (cache dtype)
  const void* k;              // [n_units][head_stride] (bf16 or fp32)
  const void* v;
  int64_t head_stride;        // elements between cache head slabs
  int64_t n_rows;             // attended rows per head
  int32_t n_units;            // layers * heads_per_layer
  int32_t heads_per_layer;    // cache heads per layer (KV heads, or query heads)
  int32_t q_heads_per_layer;
  int32_t group;              // query heads per cache head, <= decode_max_group()
  int32_t n_chunks;           // blocks per unit (decode_plan)
  int32_t n_sub;              // 512-key sub-chunks per block (decode_plan)
  float c;                    // scale * log2(e)
  float* out;                 // [layers * q_heads_per_layer][D] fp32
  float2* part_ml;            // n_chunks > 1: [n_units][n_chunks][16] (max, sum) in log2 units
  float* part_acc;            // n_chunks > 1: [n_units][n_chunks][16][D]
};
void decode_plan(int dtype, int64_t n_units, int64_t n_rows, int32_t* n_sub, int32_t* n_chunks);
int decode_max_group();
hipError_t launch_decode_attention(int dtype, int head_dim, const DecodeArgs& a, hipStream_t s);

}  // namespace skv
