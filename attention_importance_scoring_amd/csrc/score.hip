// Two-pass importance scoring on gfx950 (paper notes "Draft-based
// Approximate Inference for LLMs", section "Key designs": SpecKV scores each
// remaining input key by the cross-attention of the observation queries;
// SpecPC reads the draft's causal attention rows).
//
// Pass 1 (row statistics): for every query row r, the log2-domain
//   lse_r = log2 sum_j 2^(c * <q_r, k_j>),  c = scale * log2(e),
// built from per-block (max, sum) partials so that the score matrix is never
// stored.  Pass 2 (column sums): score_j = sum_r 2^(c * <q_r, k_j> - lse_r)
// (or the maximum over r, in the max-aggregation variant).
//
// Work split: one block per CU (8 waves; 12 at head_dim 64, where the vector
// work dominates) owns a chunk of consecutive keys of one unit (layer, KV
// head, or, in pass 2, query head when each has its own kept set) and one
// "part" of the unit's query rows: as many 32-row tiles as fit in LDS (up to
// ~156 KB), copied there once.  The parts of a chunk are neighbouring blocks
// on one XCD, so K comes from HBM about once and from L2 for the other parts
// (in pass 1 every part walks the same number of tiles to stay in step);
// pass 2 writes one column-sum row per part and a small kernel adds them in
// part order.  Keys may also be read through a row list (the ROWS instances).  Every wave walks its
// share of the chunk, kKT tiles of 32 keys at a time held in registers as an
// MFMA operand, against every row tile of the part.  The main loop has no
// barriers: the rows are read-only in LDS, each wave keeps its own row
// statistics (pass 1) or column sums (pass 2), and the waves that share a
// SIMD walk the row tiles half a sub-chunk apart, so that while one waits on
// its MFMAs (or its next keys) another runs its exp / sum work.  Pass 1 puts keys on
// the MFMA M dimension and rows on N, so each lane reduces one row in-lane;
// pass 2 swaps the operands so that each lane owns one key column.  Every sum
// has a fixed order (no floating-point atomics): results are run-to-run
// identical.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace skv {

constexpr int kScoreLdsBudget = 156 * 1024;  // dynamic LDS per block (one block per CU)
#ifndef SKV_MAX_SUB
#define SKV_MAX_SUB 32
#endif
#ifndef SKV_TARGET_BLOCKS
#define SKV_TARGET_BLOCKS 768
#endif
constexpr int kMaxSubPerChunk = SKV_MAX_SUB;  // groups of resident keys per block
// With two waves per SIMD, the wave that reads its row fragment and issues
// its MFMAs runs at raised issue priority, so the matrix unit is fed first
// and the other wave's exp/sum work takes the remaining issue cycles.  (At
// three waves per SIMD, head_dim 64, it gained nothing and is not used.)
template <int P>
__device__ __forceinline__ void mfma_prio() {
  __builtin_amdgcn_s_setprio(P);
}

template <typename T, int D, int KT>
struct ScoreGeom {
  using RF = RowFrag<T, D>;
  static constexpr int kNV = RF::kNV;
  static constexpr int kKT = KT;  // key tiles (of 32) held per wave
  static_assert(KT * 4 * kNV <= 128, "resident keys must fit in 128 VGPRs");
  // Waves per block (one block per CU, kWaves / 4 per SIMD).  At head_dim 64
  // the vector work outweighs the MFMAs, and with at most 64 VGPRs of
  // resident keys three waves per SIMD fit and raise the issue rate.  (Three
  // waves with two key tiles at head_dim 128 measured 8-10 % slower on the
  // 128K in-place workload, whose layers arrive cold, and 10 % slower at 64K.)
  static constexpr int kWaves = (D == 64 && KT * 4 * kNV <= 64) ? 12 : 8;
  static constexpr bool kPrio = kWaves == 8;  // the MFMA issue priority (nothing gained at 64)
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKeysPerWave = 32 * kKT;
  static constexpr int kKeysPerSub = kWaves * kKeysPerWave;  // keys resident in one block at a time
  static constexpr int kRowPitch = RF::kRowBytes + 16;       // LDS pitch, padded against bank conflicts
  static constexpr int kVecPerRow = RF::kRowBytes / 16;
};

struct RowStat {
  float m;  // max (log2 units)
  float s;  // sum of 2^(x - m)
};

__device__ __forceinline__ RowStat merge_stat(RowStat a, RowStat b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return {-INFINITY, 0.f};
  return {M, a.s * fast_exp2(a.m - M) + b.s * fast_exp2(b.m - M)};
}

// The query rows of one unit are contiguous: [group][rows_per_qhead][D] (the
// unit's query heads), so row r of the unit sits at r * D elements from the
// unit's first row.
template <typename T>
__device__ __forceinline__ const char* unit_rows(const ScoreArgs& a, int unit) {
  const int layer = a.layer0 + unit / a.n_kv_heads;
  const int head = unit % a.n_kv_heads;
  return static_cast<const char*>(a.q) +
         (layer * a.q_layer_stride + (int64_t)head * a.group * a.q_head_stride) * Elem<T>::kBytes;
}

// Copies rows [0, n_rows) starting at `src` into LDS (padded pitch) and zeroes
// rows [n_rows, n_pad).  All threads of the block take part.
template <typename T, int D, int KT>
__device__ __forceinline__ void stage_rows(char* s_q, const char* src, int n_rows, int n_pad) {
  using Gm = ScoreGeom<T, D, KT>;
  const int total = n_pad * Gm::kVecPerRow;
  for (int base = 0; base < total; base += 4 * Gm::kThreads) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + u * Gm::kThreads + threadIdx.x;
      const int row = idx / Gm::kVecPerRow, col = idx % Gm::kVecPerRow;
      v[u] = (idx < total && row < n_rows) ? ldg16(src + (int64_t)row * Gm::RF::kRowBytes + col * 16)
                                           : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + u * Gm::kThreads + threadIdx.x;
      const int row = idx / Gm::kVecPerRow, col = idx % Gm::kVecPerRow;
      if (idx < total) *reinterpret_cast<u32x4*>(s_q + row * Gm::kRowPitch + col * 16) = v[u];
    }
  }
}

// This lane's MFMA operand vectors of row tile rt: vector v of the lane's
// half row (row 32 rt + lane % 32).
template <typename T, int D, int KT>
__device__ __forceinline__ void read_q_frag(const char* s_q, int rt, int lane, u32x4 (&qf)[ScoreGeom<T, D, KT>::kNV]) {
  using Gm = ScoreGeom<T, D, KT>;
  const char* p = s_q + (rt * 32 + lane % 32) * Gm::kRowPitch + (lane / 32) * Gm::RF::kHalfBytes;
#pragma unroll
  for (int v = 0; v < Gm::kNV; ++v) qf[v] = *reinterpret_cast<const u32x4*>(p + v * 16);
}

// Resident keys of this wave: kst[kt][v] = 16-byte vector v of the lane's
// half row of key (kbase + 32 kt + lane % 32).  Keys at or beyond n_keys read
// the last key's row instead (clamped address, no branch): pass 1 masks them
// through the accumulator's initial value and pass 2 never stores their
// columns, so their contents do not matter.  With a row list, key j is row
// key_rows[j] of the head slab (clamped into the slab); ROWS selects that
// form at compile time, so the plain kernels carry no trace of it.
template <typename T, int D, int KT, bool ROWS>
__device__ __forceinline__ void load_keys(const ScoreArgs& a, int unit, int kbase,
                                          u32x4 (&kst)[ScoreGeom<T, D, KT>::kKT][ScoreGeom<T, D, KT>::kNV]) {
  using Gm = ScoreGeom<T, D, KT>;
  const int lane = threadIdx.x % kWave, half = lane / 32;
  const int layer = a.layer0 + unit / a.n_kv_heads;
  const int kvh = (unit % a.n_kv_heads) / a.kv_repeat;
  const char* kb = static_cast<const char*>(a.k) + (layer * a.k_layer_stride + kvh * a.k_head_stride) * Elem<T>::kBytes;
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) {
    int key = min(kbase + kt * 32 + (lane % 32), a.n_keys - 1);
    if constexpr (ROWS) key = min(max(a.key_rows[key], 0), a.key_row_limit - 1);
    const char* row = kb + (int64_t)key * Gm::RF::kRowBytes + half * Gm::RF::kHalfBytes;
#pragma unroll
    for (int v = 0; v < Gm::kNV; ++v) kst[kt][v] = ldg16(row + v * 16);
  }
}

// A wave's walk over (sub-chunk, row tile) starts rot tiles into sub-chunk 0
// and ends with sub-chunk 0's first rot tiles.  The waves that share a SIMD
// (w, w + 4, ...) take rot = 0, n_tiles / 2 (or thirds at 12 waves): they
// work on different row tiles at any time, and one reloads its keys at a
// sub-chunk boundary while the other is mid-way through its sub-chunk.
template <int WAVES>
__device__ __forceinline__ int wave_phase(int wave, int n_tiles) {
  return (wave / 4) * n_tiles / (WAVES / 4);
}

// Pass-1 key mask of one wave for one row: keys past `rel` (offset in the
// wave's range, half-wave offset removed) are masked; 4096 = none masked.
__device__ __forceinline__ int pass1_rel(const ScoreArgs& a, int kbase, int row, int half) {
  int64_t lim = (int64_t)a.n_keys - 1;
  if (a.causal) {
    const int g = row / a.rows_per_qhead;
    const int64_t pos = a.pos_base + (row - g * a.rows_per_qhead);
    lim = pos < lim ? pos : lim;
  }
  int64_t rel = lim - kbase - 4 * half;
  return (int)(rel < -4096 ? -4096 : (rel > 4096 ? 4096 : rel));
}

// Block -> (unit, key chunk, row part).  The parts of one chunk are adjacent
// logical blocks, which the XCD-contiguous remap puts on the same XCD at about
// the same time, so the keys the first part reads from HBM reach the others
// from that XCD's L2.
struct BlockPos {
  int unit, chunk, part;
};
__device__ __forceinline__ BlockPos block_pos(const ScoreArgs& a) {
  const int logical = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int part = logical % a.n_parts, uc = logical / a.n_parts;
  return {uc / a.n_chunks, uc % a.n_chunks, part};
}

// ---------------------------------------------------------------------------
// Pass 1

// acc = K_tile x Q_tile^T for the wave's keys (M) and the tile's rows (N).
template <typename T, int D, int KT, bool MASKED>
__device__ __forceinline__ void pass1_mfma(const u32x4 (&kst)[ScoreGeom<T, D, KT>::kKT][ScoreGeom<T, D, KT>::kNV],
                                           const u32x4 (&qf)[ScoreGeom<T, D, KT>::kNV], int rel,
                                           f32x16 (&acc)[ScoreGeom<T, D, KT>::kKT]) {
  using Gm = ScoreGeom<T, D, KT>;
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) {
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[kt][i] = (kt * 32 + 8 * (i >> 2) + (i & 3) <= rel) ? 0.f : -INFINITY;
    } else {
      acc[kt] = f32x16{};
    }
  }
#pragma unroll
  for (int v = 0; v < Gm::kNV; ++v)
#pragma unroll
    for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = Mfma<T>::step(kst[kt][v], qf[v], acc[kt]);
}

// Per-lane (max, sum) of the lane's row over the wave's keys, both half-waves merged.
template <typename T, int D, int KT, bool MASKED>
__device__ __forceinline__ RowStat pass1_stats(const f32x16 (&acc)[ScoreGeom<T, D, KT>::kKT], float c) {
  using Gm = ScoreGeom<T, D, KT>;
  float m4[4] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) m4[i & 3] = fmaxf(m4[i & 3], acc[kt][i]);
  const float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  const bool empty = MASKED && (mx == -INFINITY);
  const float my = empty ? 0.f : mx * c;
  float s4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = fast_exp2(__builtin_fmaf(acc[0][i], c, -my));
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt)
#pragma unroll
    for (int i = (kt == 0 ? 4 : 0); i < 16; ++i) s4[i & 3] += fast_exp2(__builtin_fmaf(acc[kt][i], c, -my));
  RowStat rs = {empty ? -INFINITY : my, (s4[0] + s4[1]) + (s4[2] + s4[3])};
  // Lanes l and l ^ 32 hold the same row over different keys.
  return merge_stat(rs, {shfl_xor32(rs.m), shfl_xor32(rs.s)});
}

// Sum of 2^(c x - ref) over the wave's keys for the lane's row, both
// half-waves added.  Masked entries (-inf) add 0 when ref is finite.
template <typename T, int D, int KT>
__device__ __forceinline__ float pass1_sum_ref(const f32x16 (&acc)[ScoreGeom<T, D, KT>::kKT], float c, float ref) {
  using Gm = ScoreGeom<T, D, KT>;
  float s4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = fast_exp2(__builtin_fmaf(acc[0][i], c, -ref));
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt)
#pragma unroll
    for (int i = (kt == 0 ? 4 : 0); i < 16; ++i) s4[i & 3] += fast_exp2(__builtin_fmaf(acc[kt][i], c, -ref));
  const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  return s + shfl_xor32(s);
}

template <typename T, int D, int KT, bool ROWS>
__global__ __launch_bounds__((ScoreGeom<T, D, KT>::kThreads), 1) void score_pass1_kernel(ScoreArgs a) {
  using Gm = ScoreGeom<T, D, KT>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* s_q = smem;                                                                      // [rows_per_part][pitch]
  RowStat* s_ws = reinterpret_cast<RowStat*>(smem + (size_t)a.rows_per_part * Gm::kRowPitch);  // [waves][rows_per_part]

  const BlockPos bp = block_pos(a);
  const int unit = bp.unit, chunk = bp.chunk;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, half = lane / 32;
  const int key0 = chunk * a.n_sub * Gm::kKeysPerSub;
  const int n_sub = min(a.n_sub, (a.n_keys - key0 + Gm::kKeysPerSub - 1) / Gm::kKeysPerSub);
  const float c = a.c;
  const char* qrows = unit_rows<T>(a, unit);
  float2* part_out = a.part + ((int64_t)unit * a.n_chunks + chunk) * a.n_rows;
  RowStat* ws = s_ws + wave * a.rows_per_part;

  auto wave_kbase = [&](int sc) { return key0 + sc * Gm::kKeysPerSub + wave * Gm::kKeysPerWave; };
  auto sub_masked = [&](int sc) {
    const int kb = wave_kbase(sc);
    return (kb + Gm::kKeysPerWave > a.n_keys) || (a.causal && (int64_t)kb + Gm::kKeysPerWave - 1 > a.pos_base);
  };

  {
    const int row0 = bp.part * a.rows_per_part;
    const int prow = min(a.rows_per_part, a.n_rows - row0);
    // Every part walks the same number of row tiles (a shorter last part
    // pads with zero rows, whose statistics are never written), so the parts
    // of a chunk read each key group at the same pace and share it in L2.
    const int n_tiles = a.rows_per_part / 32;
    const int rot = wave_phase<Gm::kWaves>(wave, n_tiles);
    const int n_iter = n_sub * n_tiles;
    stage_rows<T, D, KT>(s_q, qrows + (int64_t)row0 * Gm::RF::kRowBytes, prow, n_tiles * 32);
    __syncthreads();

    u32x4 kst[Gm::kKT][Gm::kNV];  // resident keys of the current sub-chunk
    load_keys<T, D, KT, ROWS>(a, unit, wave_kbase(0), kst);
    int sc = 0, rt = rot;  // current sub-chunk and row tile
    bool masked = sub_masked(0);
    for (int it = 0; it < n_iter; ++it, ++rt) {
      if (rt == n_tiles) {  // next sub-chunk; after the last one, back to sub-chunk 0 for its first rot tiles
        rt = 0;
        const int nsc = sc + 1 == n_sub ? 0 : sc + 1;
        if (nsc != sc) {
          sc = nsc;
          load_keys<T, D, KT, ROWS>(a, unit, wave_kbase(sc), kst);
          masked = sub_masked(sc);
        }
      }
      u32x4 qf[Gm::kNV];
      if constexpr (Gm::kPrio) mfma_prio<1>();
      read_q_frag<T, D, KT>(s_q, rt, lane, qf);
      f32x16 acc[Gm::kKT];
      const int r = rt * 32 + lane % 32;
      if (masked)
        pass1_mfma<T, D, KT, true>(kst, qf, pass1_rel(a, wave_kbase(sc), row0 + r, half), acc);
      else
        pass1_mfma<T, D, KT, false>(kst, qf, 0, acc);
      if constexpr (Gm::kPrio) mfma_prio<0>();
      RowStat st;
      if (it < n_tiles) {  // first visit of the row in this part: exact (max, sum)
        st = masked ? pass1_stats<T, D, KT, true>(acc, c) : pass1_stats<T, D, KT, false>(acc, c);
      } else {
        // Later visits sum against the row's reference (the maximum of its
        // first visit, raised only by an exact merge): no per-tile max and no
        // rescaling.  A wave falls back to the exact merge when a row has no
        // reference yet or a tile would exceed it by 2^64; the running sum
        // then stays below 2^64 times the keys visited, far inside fp32.
        const RowStat cur = ws[r];  // lanes l and l ^ 32 read the same row
        const float add = pass1_sum_ref<T, D, KT>(acc, c, cur.m);
        if (__any(!(add <= 0x1p64f)))
          st = merge_stat(cur, pass1_stats<T, D, KT, true>(acc, c));
        else
          st = {cur.m, cur.s + add};
      }
      if (lane < 32) ws[r] = st;  // this wave's own slice: no other wave touches it
    }
    __syncthreads();
    for (int r = threadIdx.x; r < prow; r += Gm::kThreads) {
      RowStat m = s_ws[r];
      for (int w = 1; w < Gm::kWaves; ++w) m = merge_stat(m, s_ws[w * a.rows_per_part + r]);
      part_out[row0 + r] = make_float2(m.m, m.s);
    }
  }
}

__global__ __launch_bounds__(256) void lse_combine_kernel(ScoreArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.n_units * a.n_rows) return;
  const int64_t unit = idx / a.n_rows, r = idx % a.n_rows;
  const float2* p = a.part + unit * a.n_chunks * a.n_rows + r;
  // One pass over the chunk partials, eight loads in flight, merged in chunk
  // order with a running maximum (fixed order: run-to-run identical).
  constexpr int kBatch = 8;
  float M = -INFINITY, S = 0.f;
  for (int ch0 = 0; ch0 < a.n_chunks; ch0 += kBatch) {
    float2 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      v[u] = p[(int64_t)min(ch0 + u, a.n_chunks - 1) * a.n_rows];  // clamped; extra ones dropped below
      if (ch0 + u >= a.n_chunks) v[u] = make_float2(-INFINITY, 0.f);
    }
    float mb = v[0].x;
#pragma unroll
    for (int u = 1; u < kBatch; ++u) mb = fmaxf(mb, v[u].x);
    if (mb == -INFINITY) continue;
    if (mb > M) {
      S = (M == -INFINITY) ? 0.f : S * exp2f(M - mb);
      M = mb;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (v[u].x != -INFINITY) S += v[u].y * exp2f(v[u].x - M);
  }
  a.lam[idx] = M + log2f(S);
}

// scores += column sums of parts 1 .. n_parts - 1, in part order (or their
// maximum, for the max aggregation).  Four consecutive elements per thread:
// 16-byte accesses when both buffers are 16-byte aligned, else one by one.
__global__ __launch_bounds__(256) void colsum_combine_kernel(ScoreArgs a, int vec) {
  const int64_t n = (int64_t)a.n_units * a.n_keys;
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i0 >= n) return;
  if (vec && i0 + 4 <= n) {
    f32x4 v = *reinterpret_cast<const f32x4*>(a.scores + i0);
    for (int p = 1; p < a.n_parts; ++p) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(a.colpart + (int64_t)(p - 1) * n + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = a.agg_max ? fmaxf(v[e], x[e]) : v[e] + x[e];
    }
    *reinterpret_cast<f32x4*>(a.scores + i0) = v;
    return;
  }
  for (int64_t idx = i0; idx < i0 + 4 && idx < n; ++idx) {
    float v = a.scores[idx];
    for (int p = 1; p < a.n_parts; ++p) {
      const float x = a.colpart[(int64_t)(p - 1) * n + idx];
      v = a.agg_max ? fmaxf(v, x) : v + x;
    }
    a.scores[idx] = v;
  }
}

// ---------------------------------------------------------------------------
// Pass 2

template <typename T, int D, int KT>
__device__ __forceinline__ void pass2_mfma(const u32x4 (&kst)[ScoreGeom<T, D, KT>::kKT][ScoreGeom<T, D, KT>::kNV],
                                           const u32x4 (&qf)[ScoreGeom<T, D, KT>::kNV],
                                           f32x16 (&acc)[ScoreGeom<T, D, KT>::kKT]) {
  using Gm = ScoreGeom<T, D, KT>;
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = f32x16{};
#pragma unroll
  for (int v = 0; v < Gm::kNV; ++v)
#pragma unroll
    for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = Mfma<T>::step(qf[v], kst[kt][v], acc[kt]);
}

// Row aggregation of pass 2: sum (the default) or max of the probabilities.
template <bool MAX>
__device__ __forceinline__ float agg2(float x, float y) {
  if constexpr (MAX) return fmaxf(x, y);
  return x + y;
}

template <typename T, int D, int KT, bool MAX, bool ROWS>
__global__ __launch_bounds__((ScoreGeom<T, D, KT>::kThreads), 1) void score_pass2_kernel(ScoreArgs a) {
  using Gm = ScoreGeom<T, D, KT>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* s_q = smem;                                                                    // [rows_per_part][pitch]
  float* s_lam = reinterpret_cast<float*>(smem + (size_t)a.rows_per_part * Gm::kRowPitch);  // [rows_per_part]

  const BlockPos bp = block_pos(a);
  const int unit = bp.unit, chunk = bp.chunk;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, half = lane / 32;
  const int key0 = chunk * a.n_sub * Gm::kKeysPerSub;
  const int n_sub = min(a.n_sub, (a.n_keys - key0 + Gm::kKeysPerSub - 1) / Gm::kKeysPerSub);
  const float c = a.c;
  const char* qrows = unit_rows<T>(a, unit);
  const float* lam_unit = a.lam + (int64_t)unit * a.n_rows;
  // part 0 writes the scores, part p > 0 its own partial column sums
  float* out = (bp.part == 0 ? a.scores : a.colpart + (int64_t)(bp.part - 1) * a.n_units * a.n_keys) +
               (int64_t)unit * a.n_keys;
  auto wave_kbase = [&](int sc) { return key0 + sc * Gm::kKeysPerSub + wave * Gm::kKeysPerWave; };
  // lse of row tile rt's rows m(i) = acc_row(i, half), for the lane's half-wave.
  auto read_lam = [&](int rt, float (&lam)[16]) {
    const float* lrow = s_lam + rt * 32;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lrow[8 * g4 + 4 * half]);
      lam[4 * g4 + 0] = l4[0];
      lam[4 * g4 + 1] = l4[1];
      lam[4 * g4 + 2] = l4[2];
      lam[4 * g4 + 3] = l4[3];
    }
  };

  {
    const int row0 = bp.part * a.rows_per_part;
    const int prow = min(a.rows_per_part, a.n_rows - row0);
    const int n_tiles = (prow + 31) / 32;
    const int rot = wave_phase<Gm::kWaves>(wave, n_tiles);
    const int n_iter = n_sub * n_tiles;
    stage_rows<T, D, KT>(s_q, qrows + (int64_t)row0 * Gm::RF::kRowBytes, prow, n_tiles * 32);
    for (int r = threadIdx.x; r < n_tiles * 32; r += Gm::kThreads) s_lam[r] = (r < prow) ? lam_unit[row0 + r] : INFINITY;
    __syncthreads();

    u32x4 kst[Gm::kKT][Gm::kNV];  // resident keys of the current sub-chunk
    load_keys<T, D, KT, ROWS>(a, unit, wave_kbase(0), kst);
    float colsum[Gm::kKT];
#pragma unroll
    for (int kt = 0; kt < Gm::kKT; ++kt) colsum[kt] = 0.f;
    // Column sums of sub-chunk sc for this part: stored, or (the second
    // stretch of sub-chunk 0, after the wrap) combined with the first one.
    auto flush = [&](int sc, bool combine) {
      const int kbase = wave_kbase(sc);
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) {
        const float tot = agg2<MAX>(colsum[kt], shfl_xor32(colsum[kt]));
        const int key = kbase + kt * 32 + lane;
        if (lane < 32 && key < a.n_keys) out[key] = combine ? agg2<MAX>(out[key], tot) : tot;
        colsum[kt] = 0.f;
      }
    };
    int sc = 0, rt = rot;  // current sub-chunk and row tile
    for (int it = 0; it < n_iter; ++it, ++rt) {
      if (rt == n_tiles) {  // next sub-chunk; after the last one, back to sub-chunk 0 for its first rot tiles
        rt = 0;
        const int nsc = sc + 1 == n_sub ? 0 : sc + 1;
        if (nsc != sc) {
          flush(sc, false);
          sc = nsc;
          load_keys<T, D, KT, ROWS>(a, unit, wave_kbase(sc), kst);
        }
      }
      float lam[16];
      read_lam(rt, lam);
      f32x16 acc[Gm::kKT];
      u32x4 qf[Gm::kNV];
      if constexpr (Gm::kPrio) mfma_prio<1>();
      read_q_frag<T, D, KT>(s_q, rt, lane, qf);
      pass2_mfma<T, D, KT>(kst, qf, acc);
      if constexpr (Gm::kPrio) mfma_prio<0>();
      // acc[kt][i] = <q_(row0 + 32 rt + acc_row(i, half)), k_(kbase + 32 kt + lane % 32)>
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) {
        float s4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[i] = fast_exp2(__builtin_fmaf(acc[kt][i], c, -lam[i]));
#pragma unroll
        for (int i = 4; i < 16; ++i) s4[i & 3] = agg2<MAX>(s4[i & 3], fast_exp2(__builtin_fmaf(acc[kt][i], c, -lam[i])));
        colsum[kt] = agg2<MAX>(colsum[kt], agg2<MAX>(agg2<MAX>(s4[0], s4[1]), agg2<MAX>(s4[2], s4[3])));
      }
    }
    flush(sc, rot > 0 && n_sub > 1);
  }
}

// ---------------------------------------------------------------------------

template <typename T, int D, int KT>
static void plan_for(int64_t n_units, int64_t n_rows, int64_t n_keys, ScorePlan* pl,
                     int64_t target_blocks = SKV_TARGET_BLOCKS, int64_t extra_parts = 0) {
  using Gm = ScoreGeom<T, D, KT>;
  // Row parts: as many 32-row tiles as the LDS budget holds (or extra_parts
  // more parts than that needs), split evenly.
  const int64_t tiles = (n_rows + 31) / 32;
  const int64_t per_row1 = Gm::kRowPitch + (int64_t)Gm::kWaves * (int64_t)sizeof(RowStat);
  const int64_t per_row2 = Gm::kRowPitch + 4;
  int64_t fit = kScoreLdsBudget / (32 * per_row1);
  const int64_t fit2 = kScoreLdsBudget / (32 * per_row2);
  fit = fit < fit2 ? fit : fit2;
  if (fit < 1) fit = 1;
  int64_t parts = (tiles + fit - 1) / fit + extra_parts;
  parts = parts > tiles ? tiles : parts;
  const int64_t tpp = (tiles + parts - 1) / parts;
  pl->rows_per_part = (int32_t)(tpp * 32);
  pl->n_parts = (int32_t)((tiles + tpp - 1) / tpp);
  pl->lds_pass1 = (size_t)(pl->rows_per_part * per_row1);
  pl->lds_pass2 = (size_t)(pl->rows_per_part * per_row2);
  // Key chunks: enough blocks (units x chunks x parts) for several rounds over
  // the 256 CUs, one block per CU; at most kMaxSubPerChunk groups of resident
  // keys per block, so the parts of a chunk stay close together in time.
  const int64_t subs = (n_keys + Gm::kKeysPerSub - 1) / Gm::kKeysPerSub;
  const int64_t ups = n_units * pl->n_parts;
  int64_t chunks = (target_blocks + ups - 1) / ups;
  chunks = chunks < 1 ? 1 : (chunks > subs ? subs : chunks);
  int64_t per = (subs + chunks - 1) / chunks;
  if (per > kMaxSubPerChunk) per = kMaxSubPerChunk;
  pl->n_sub = (int32_t)per;
  pl->n_chunks = (int32_t)((subs + per - 1) / per);
  pl->kt = KT;
}

// Four key tiles per wave halve the LDS reads of the row operand per MFMA,
// but coarsen the key split: they are taken where the resident-key
// registers allow them and every block still walks at least 16 key groups at
// the usual target.  Otherwise (few units, or few keys per unit) four tiles
// still win where the blocks make whole rounds over the CUs, with no partly
// filled last round, and every block walks at least 4 key groups: the row
// parts may then be cut up to two finer than the LDS budget needs, and the
// plan with the fewest rounds (the longest blocks) is taken.
template <typename T, int D>
static void plan_pick(int64_t n_units, int64_t n_rows, int64_t n_keys, ScorePlan* pl) {
  plan_for<T, D, 2>(n_units, n_rows, n_keys, pl);
  if constexpr (4 * 4 * RowFrag<T, D>::kNV <= 128) {
    constexpr int64_t kCUs = 256;
    ScorePlan p4;
    plan_for<T, D, 4>(n_units, n_rows, n_keys, &p4);
    if (p4.n_sub >= 16) {
      *pl = p4;
      return;
    }
    int64_t best_rounds = 0;
    for (int64_t extra = 0; extra <= 2; ++extra) {
      for (int64_t rounds = 1; rounds <= 8; ++rounds) {
        plan_for<T, D, 4>(n_units, n_rows, n_keys, &p4, rounds * kCUs, extra);
        const int64_t blocks = n_units * p4.n_parts * p4.n_chunks;
        if (p4.n_sub < 4 || blocks % kCUs != 0) continue;
        if (best_rounds == 0 || blocks / kCUs < best_rounds) {
          best_rounds = blocks / kCUs;
          *pl = p4;
        }
        break;
      }
    }
  }
}

int64_t score_plan_target_blocks() { return SKV_TARGET_BLOCKS; }

void score_plan(int dtype, int head_dim, int64_t n_units, int64_t n_rows, int64_t n_keys, ScorePlan* pl) {
  if (dtype == 0) {
    if (head_dim == 64) plan_pick<float, 64>(n_units, n_rows, n_keys, pl);
    else plan_pick<float, 128>(n_units, n_rows, n_keys, pl);
  } else {
    if (head_dim == 64) plan_pick<bf16_t, 64>(n_units, n_rows, n_keys, pl);
    else plan_pick<bf16_t, 128>(n_units, n_rows, n_keys, pl);
  }
}

template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

// ROWS: keys through the row list (a.key_rows), a separate instance so the
// plain kernels are unchanged.
template <typename T, int D, int KT, bool ROWS>
static hipError_t launch_p1_form(const ScoreArgs& a, size_t lds, hipStream_t s) {
  hipError_t e = allow_lds(score_pass1_kernel<T, D, KT, ROWS>, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((int64_t)a.n_units * a.n_chunks * a.n_parts)), block(ScoreGeom<T, D, KT>::kThreads);
  score_pass1_kernel<T, D, KT, ROWS><<<grid, block, lds, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int KT>
static hipError_t launch_p1(const ScoreArgs& a, size_t lds, hipStream_t s) {
  return a.key_rows ? launch_p1_form<T, D, KT, true>(a, lds, s) : launch_p1_form<T, D, KT, false>(a, lds, s);
}

template <typename T, int D, int KT, bool MAX, bool ROWS>
static hipError_t launch_p2_form(const ScoreArgs& a, size_t lds, hipStream_t s) {
  hipError_t e = allow_lds(score_pass2_kernel<T, D, KT, MAX, ROWS>, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((int64_t)a.n_units * a.n_chunks * a.n_parts)), block(ScoreGeom<T, D, KT>::kThreads);
  score_pass2_kernel<T, D, KT, MAX, ROWS><<<grid, block, lds, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int KT>
static hipError_t launch_p2(const ScoreArgs& a, size_t lds, hipStream_t s) {
  if (a.key_rows)
    return a.agg_max ? launch_p2_form<T, D, KT, true, true>(a, lds, s) : launch_p2_form<T, D, KT, false, true>(a, lds, s);
  return a.agg_max ? launch_p2_form<T, D, KT, true, false>(a, lds, s) : launch_p2_form<T, D, KT, false, false>(a, lds, s);
}

hipError_t launch_score_pass1(int dtype, int head_dim, int kt, const ScoreArgs& a, size_t lds, hipStream_t s) {
  if (dtype == 0) {
    if (head_dim == 64) return kt == 4 ? launch_p1<float, 64, 4>(a, lds, s) : launch_p1<float, 64, 2>(a, lds, s);
    return launch_p1<float, 128, 2>(a, lds, s);
  }
  if (head_dim == 64) return kt == 4 ? launch_p1<bf16_t, 64, 4>(a, lds, s) : launch_p1<bf16_t, 64, 2>(a, lds, s);
  return kt == 4 ? launch_p1<bf16_t, 128, 4>(a, lds, s) : launch_p1<bf16_t, 128, 2>(a, lds, s);
}

hipError_t launch_lse_combine(const ScoreArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_units * a.n_rows;
  lse_combine_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_colsum_combine(const ScoreArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_units * a.n_keys;
  const int vec = (reinterpret_cast<uintptr_t>(a.scores) % 16 == 0) && (reinterpret_cast<uintptr_t>(a.colpart) % 16 == 0) &&
                  (n % 4 == 0);
  const int64_t threads = (n + 3) / 4;
  colsum_combine_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(a, vec);
  return hipGetLastError();
}

hipError_t launch_score_pass2(int dtype, int head_dim, int kt, const ScoreArgs& a, size_t lds, hipStream_t s) {
  if (dtype == 0) {
    if (head_dim == 64) return kt == 4 ? launch_p2<float, 64, 4>(a, lds, s) : launch_p2<float, 64, 2>(a, lds, s);
    return launch_p2<float, 128, 2>(a, lds, s);
  }
  if (head_dim == 64) return kt == 4 ? launch_p2<bf16_t, 64, 4>(a, lds, s) : launch_p2<bf16_t, 64, 2>(a, lds, s);
  return kt == 4 ? launch_p2<bf16_t, 128, 4>(a, lds, s) : launch_p2<bf16_t, 128, 2>(a, lds, s);
}

}  // namespace skv
