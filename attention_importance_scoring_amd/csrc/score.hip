// Two-pass importance scoring on gfx950 (paper notes "Draft-based
// Approximate Inference for LLMs", section "Key designs": SpecKV scores each
// remaining input key by the cross-attention of the observation queries;
// SpecPC reads the draft's causal attention rows).
//
// Pass 1 (row statistics): for every query row r, the log2-domain
//   lse_r = log2 sum_j 2^(c * <q_r, k_j>),  c = scale * log2(e),
// built from per-block (max, sum) partials so that the score matrix is never
// stored.  Pass 2 (column sums): score_j = sum_r 2^(c * <q_r, k_j> - lse_r).
//
// Work split: a block owns a chunk of consecutive keys of one unit (layer,
// KV head) and walks it in "sub-chunks" of kKeysPerSub keys; for each, every
// wave keeps its kKT tiles of 32 keys resident in registers as an MFMA
// operand while all query rows of the unit stream past, 32 rows per tile,
// through a three-buffer LDS ring (one barrier per tile; the global loads of a
// tile are issued three iterations ahead into one of two register sets).  Inside a wave the loop is software-pipelined: the MFMAs of
// tile t+1 are issued next to the exp / sum work of tile t, so the matrix
// cores and the vector ALUs run at the same time.  Pass 1 puts keys on the
// MFMA M dimension and rows on N, so each lane reduces one row in-lane; pass 2
// swaps the operands so that each lane owns one key column.  Every sum has a
// fixed order (no floating-point atomics): results are run-to-run identical.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace skv {

// Registers per lane that hold resident keys, and target waves per SIMD.
#ifndef SKV_KEY_VGPRS
#define SKV_KEY_VGPRS 64
#endif
#ifndef SKV_SCORE_OCC
#define SKV_SCORE_OCC 2
#endif
// Vector instructions scheduled after each MFMA in the pipelined loops.
#ifndef SKV_P1_VALU_PER
#define SKV_P1_VALU_PER 8
#endif
#ifndef SKV_P2_VALU_PER
#define SKV_P2_VALU_PER 5
#endif
// Vector instructions scheduled before the first MFMA (covering LDS latency).
#ifndef SKV_P2_VALU_LEAD
#define SKV_P2_VALU_LEAD 16
#endif
#ifndef SKV_P1_VALU_LEAD
#define SKV_P1_VALU_LEAD 24
#endif

template <typename T, int D>
struct ScoreGeom {
  using RF = RowFrag<T, D>;
  static constexpr int kNV = RF::kNV;
  static constexpr int kKT = (SKV_KEY_VGPRS / (4 * kNV)) > 0 ? SKV_KEY_VGPRS / (4 * kNV) : 1;  // key tiles per wave
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKeysPerWave = 32 * kKT;
  static constexpr int kKeysPerSub = kWaves * kKeysPerWave;  // keys resident in one block at a time
  static constexpr int kRowPitch = RF::kRowBytes + 16;       // LDS pitch, padded against bank conflicts
  static constexpr int kTileBytes = 32 * kRowPitch;
  static constexpr int kVecPerRow = RF::kRowBytes / 16;
  static constexpr int kStageVecs = 32 * kVecPerRow / kThreads;  // 16-byte loads per thread per tile
  static constexpr int kRing = 3;                                // LDS tile buffers
  static_assert((32 * kVecPerRow) % kThreads == 0, "tile must split evenly over the block");
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

// The query rows of one unit are contiguous: [G][rows_per_qhead][D], so row
// r of the unit sits at r * D elements from the unit's first row.
template <typename T>
__device__ __forceinline__ const char* unit_rows(const ScoreArgs& a, int unit) {
  const int layer = a.layer0 + unit / a.n_kv_heads;
  const int kvh = unit % a.n_kv_heads;
  return static_cast<const char*>(a.q) +
         (layer * a.q_layer_stride + (int64_t)kvh * a.group * a.q_head_stride) * Elem<T>::kBytes;
}

// This thread's share of query row tile `rt` (zero rows past n_rows).
template <typename T, int D>
__device__ __forceinline__ void load_q_tile(const char* rows, int n_rows, int rt,
                                            u32x4 (&st)[ScoreGeom<T, D>::kStageVecs]) {
  using Gm = ScoreGeom<T, D>;
  // Loads are unconditional (rows past n_rows read row 0 and are zeroed
  // afterwards), so the wait counters stay exact and no branch is emitted.
  const char* tile = rows + (int64_t)rt * 32 * Gm::RF::kRowBytes;
  const int rows_left = n_rows - rt * 32;
#pragma unroll
  for (int p = 0; p < Gm::kStageVecs; ++p) {
    const int idx = p * Gm::kThreads + threadIdx.x;
    const bool ok = idx / Gm::kVecPerRow < rows_left;
    const u32x4 v = ldg16(ok ? tile + idx * 16 : rows + (idx % Gm::kVecPerRow) * 16);
    st[p] = ok ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

template <typename T, int D>
__device__ __forceinline__ void store_q_tile(char* tile, const u32x4 (&st)[ScoreGeom<T, D>::kStageVecs]) {
  using Gm = ScoreGeom<T, D>;
#pragma unroll
  for (int p = 0; p < Gm::kStageVecs; ++p) {
    const int idx = p * Gm::kThreads + threadIdx.x;
    const int row = idx / Gm::kVecPerRow, col = idx % Gm::kVecPerRow;
    *reinterpret_cast<u32x4*>(tile + row * Gm::kRowPitch + col * 16) = st[p];
  }
}

// This lane's MFMA operand vectors of the staged tile: vector v of the lane's
// half row (row lane % 32).
template <typename T, int D>
__device__ __forceinline__ void read_q_frag(const char* tile, int lane, u32x4 (&qf)[ScoreGeom<T, D>::kNV]) {
  using Gm = ScoreGeom<T, D>;
  const char* p = tile + (lane % 32) * Gm::kRowPitch + (lane / 32) * Gm::RF::kHalfBytes;
#pragma unroll
  for (int v = 0; v < Gm::kNV; ++v) qf[v] = *reinterpret_cast<const u32x4*>(p + v * 16);
}

// Resident keys of this wave: kst[kt][v] = 16-byte vector v of the lane's
// half row of key (kbase + 32 kt + lane % 32); zero beyond n_keys.
template <typename T, int D>
__device__ __forceinline__ void load_keys(const ScoreArgs& a, int unit, int kbase,
                                          u32x4 (&kst)[ScoreGeom<T, D>::kKT][ScoreGeom<T, D>::kNV]) {
  using Gm = ScoreGeom<T, D>;
  const int lane = threadIdx.x % kWave, half = lane / 32;
  const int layer = a.layer0 + unit / a.n_kv_heads;
  const int kvh = unit % a.n_kv_heads;
  const char* kb = static_cast<const char*>(a.k) + (layer * a.k_layer_stride + kvh * a.k_head_stride) * Elem<T>::kBytes;
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) {
    const int key = kbase + kt * 32 + (lane % 32);
    const bool ok = key < a.n_keys;
    const char* row = kb + (int64_t)(ok ? key : a.n_keys - 1) * Gm::RF::kRowBytes + half * Gm::RF::kHalfBytes;
#pragma unroll
    for (int v = 0; v < Gm::kNV; ++v) {
      const u32x4 x = ldg16(row + v * 16);  // unconditional: keeps the wait counters exact
      kst[kt][v] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Iteration it of a block walks sub-chunk it / n_tiles and row tile it % n_tiles.
struct IterPos {
  int sc, rt;
};
__device__ __forceinline__ IterPos iter_pos(int it, int n_tiles) {
  const int sc = it / n_tiles;
  return {sc, it - sc * n_tiles};
}

// Pass-1 key mask of one wave for one row tile: keys past `rel` (offset in the
// wave's range, half-wave offset removed) are masked; 4096 = none masked.
__device__ __forceinline__ int pass1_rel(const ScoreArgs& a, int kbase, int rt, int lane) {
  int64_t lim = (int64_t)a.n_keys - 1;
  if (a.causal) {
    const int rr = rt * 32 + (lane % 32);
    const int g = rr / a.rows_per_qhead;
    const int64_t pos = a.pos_base + (rr - g * a.rows_per_qhead);
    lim = pos < lim ? pos : lim;
  }
  int64_t rel = lim - kbase - 4 * (lane / 32);
  return (int)(rel < -4096 ? -4096 : (rel > 4096 ? 4096 : rel));
}

// ---------------------------------------------------------------------------
// Pass 1

// acc = K_tile x Q_tile^T for the wave's keys (M) and the tile's rows (N).
template <typename T, int D, bool MASKED>
__device__ __forceinline__ void pass1_mfma(const u32x4 (&kst)[ScoreGeom<T, D>::kKT][ScoreGeom<T, D>::kNV],
                                           const u32x4 (&qf)[ScoreGeom<T, D>::kNV], int rel,
                                           f32x16 (&acc)[ScoreGeom<T, D>::kKT]) {
  using Gm = ScoreGeom<T, D>;
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
template <typename T, int D, bool MASKED>
__device__ __forceinline__ RowStat pass1_stats(const f32x16 (&acc)[ScoreGeom<T, D>::kKT], float c) {
  using Gm = ScoreGeom<T, D>;
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

template <typename T, int D>
__global__ __launch_bounds__(256, SKV_SCORE_OCC) void score_pass1_kernel(ScoreArgs a) {
  using Gm = ScoreGeom<T, D>;
  extern __shared__ float2 s_rowstat[];  // [n_rows] running (max, sum) over this block's keys
  __shared__ __attribute__((aligned(16))) char s_tile[Gm::kRing][Gm::kTileBytes];
  __shared__ RowStat s_stat[2][Gm::kWaves][32];

  const int logical = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int unit = logical / a.n_chunks, chunk = logical % a.n_chunks;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int key0 = chunk * a.n_sub * Gm::kKeysPerSub;
  const int n_sub = min(a.n_sub, (a.n_keys - key0 + Gm::kKeysPerSub - 1) / Gm::kKeysPerSub);
  const int n_tiles = (a.n_rows + 31) / 32;
  const int n_iter = n_sub * n_tiles;
  const float c = a.c;
  const char* qrows = unit_rows<T>(a, unit);

  auto wave_kbase = [&](int sc) { return key0 + sc * Gm::kKeysPerSub + wave * Gm::kKeysPerWave; };
  auto sub_masked = [&](int sc) {
    const int kb = wave_kbase(sc);
    return (kb + Gm::kKeysPerWave > a.n_keys) || (a.causal && (int64_t)kb + Gm::kKeysPerWave - 1 > a.pos_base);
  };
  // Folds the four waves' statistics of iteration `it` into the block's rows.
  auto merge_tile = [&](int it) {
    const IterPos p = iter_pos(it, n_tiles);
    const int rr = p.rt * 32 + lane;
    if (lane < 32 && rr < a.n_rows) {
      RowStat m = s_stat[it & 1][0][lane];
#pragma unroll
      for (int w = 1; w < Gm::kWaves; ++w) m = merge_stat(m, s_stat[it & 1][w][lane]);
      if (p.sc > 0) {
        const float2 old = s_rowstat[rr];
        m = merge_stat({old.x, old.y}, m);
      }
      s_rowstat[rr] = make_float2(m.m, m.s);
    }
  };

  // Prologue: tiles of iterations 0 and 1 staged in LDS, tile 2 in flight to
  // registers; keys of sub-chunk 0 resident; MFMAs of iteration 0 issued.
  u32x4 st_a[Gm::kStageVecs], st_b[Gm::kStageVecs];
  load_q_tile<T, D>(qrows, a.n_rows, 0, st_a);
  store_q_tile<T, D>(s_tile[0], st_a);
  load_q_tile<T, D>(qrows, a.n_rows, iter_pos(1, n_tiles).rt, st_a);
  store_q_tile<T, D>(s_tile[1], st_a);
  u32x4 kst[Gm::kKT][Gm::kNV];
  load_keys<T, D>(a, unit, wave_kbase(0), kst);
  load_q_tile<T, D>(qrows, a.n_rows, iter_pos(2, n_tiles).rt, st_a);
  bool mask_cur = sub_masked(0);
  __syncthreads();

  u32x4 qf[Gm::kNV];
  f32x16 acc_a[Gm::kKT], acc_b[Gm::kKT];
  read_q_frag<T, D>(s_tile[0], lane, qf);
  if (mask_cur) pass1_mfma<T, D, true>(kst, qf, pass1_rel(a, wave_kbase(0), 0, lane), acc_a);
  else pass1_mfma<T, D, false>(kst, qf, 0, acc_a);

  // One pipeline step: MFMAs of iteration it + 1 into acc_next, statistics of
  // iteration it from acc_cur; tile it + 2 goes from st_ready to LDS and the
  // loads of tile it + 3 start into st_fill.
  auto step = [&](int it, f32x16 (&acc_cur)[Gm::kKT], f32x16 (&acc_next)[Gm::kKT],
                  u32x4 (&st_ready)[Gm::kStageVecs], u32x4 (&st_fill)[Gm::kStageVecs]) {
    const IterPos nx = iter_pos(it + 1, n_tiles);
    bool mask_next = mask_cur;
    if (it + 1 < n_iter && nx.rt == 0) {  // next sub-chunk: new resident keys
      load_keys<T, D>(a, unit, wave_kbase(nx.sc), kst);
      mask_next = sub_masked(nx.sc);
    }
    store_q_tile<T, D>(s_tile[(it + 2) % Gm::kRing], st_ready);
    load_q_tile<T, D>(qrows, a.n_rows, iter_pos(it + 3, n_tiles).rt, st_fill);
    if (it > 0 && wave == ((it - 1) & 3)) merge_tile(it - 1);
    read_q_frag<T, D>(s_tile[(it + 1) % Gm::kRing], lane, qf);
    RowStat rs;
    constexpr int kMfmas = Gm::kKT * Gm::kNV * (sizeof(T) == 4 ? 4 : 1);
    if (mask_cur || mask_next) {
      pass1_mfma<T, D, true>(kst, qf, pass1_rel(a, wave_kbase(nx.sc), nx.rt, lane), acc_next);
      rs = pass1_stats<T, D, true>(acc_cur, c);
      __builtin_amdgcn_sched_group_barrier(0x100, Gm::kNV, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, SKV_P1_VALU_LEAD, 0);
      interleave_mfma_valu<kMfmas, SKV_P1_VALU_PER>();
    } else {
      pass1_mfma<T, D, false>(kst, qf, 0, acc_next);
      rs = pass1_stats<T, D, false>(acc_cur, c);
      __builtin_amdgcn_sched_group_barrier(0x100, Gm::kNV, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, SKV_P1_VALU_LEAD, 0);
      interleave_mfma_valu<kMfmas, SKV_P1_VALU_PER>();
    }
    if (lane < 32) s_stat[it & 1][wave][lane] = rs;
    __syncthreads();
    mask_cur = mask_next;
  };
  int it = 0;
  for (; it + 1 < n_iter; it += 2) {
    step(it, acc_a, acc_b, st_a, st_b);
    step(it + 1, acc_b, acc_a, st_b, st_a);
  }
  if (it < n_iter) step(it, acc_a, acc_b, st_a, st_b);
  if (wave == ((n_iter - 1) & 3)) merge_tile(n_iter - 1);
  __syncthreads();
  float2* part = a.part + ((int64_t)unit * a.n_chunks + chunk) * a.n_rows;
  for (int r = threadIdx.x; r < a.n_rows; r += Gm::kThreads) part[r] = s_rowstat[r];
}

__global__ __launch_bounds__(256) void lse_combine_kernel(ScoreArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.n_units * a.n_rows) return;
  const int64_t unit = idx / a.n_rows, r = idx % a.n_rows;
  const float2* p = a.part + unit * a.n_chunks * a.n_rows + r;
  float M = -INFINITY;
  for (int ch = 0; ch < a.n_chunks; ++ch) M = fmaxf(M, p[(int64_t)ch * a.n_rows].x);
  float S = 0.f;
  if (M != -INFINITY)
    for (int ch = 0; ch < a.n_chunks; ++ch) {
      const float2 v = p[(int64_t)ch * a.n_rows];
      if (v.x != -INFINITY) S += v.y * exp2f(v.x - M);
    }
  a.lam[idx] = M + log2f(S);
}

// ---------------------------------------------------------------------------
// Pass 2

template <typename T, int D>
__device__ __forceinline__ void pass2_mfma(const u32x4 (&kst)[ScoreGeom<T, D>::kKT][ScoreGeom<T, D>::kNV],
                                           const u32x4 (&qf)[ScoreGeom<T, D>::kNV],
                                           f32x16 (&acc)[ScoreGeom<T, D>::kKT]) {
  using Gm = ScoreGeom<T, D>;
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = f32x16{};
#pragma unroll
  for (int v = 0; v < Gm::kNV; ++v)
#pragma unroll
    for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = Mfma<T>::step(qf[v], kst[kt][v], acc[kt]);
}

template <typename T, int D>
__global__ __launch_bounds__(256, SKV_SCORE_OCC) void score_pass2_kernel(ScoreArgs a) {
  using Gm = ScoreGeom<T, D>;
  __shared__ __attribute__((aligned(16))) char s_tile[Gm::kRing][Gm::kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_lam[Gm::kRing][32];

  const int logical = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int unit = logical / a.n_chunks, chunk = logical % a.n_chunks;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, half = lane / 32;
  const int key0 = chunk * a.n_sub * Gm::kKeysPerSub;
  const int n_sub = min(a.n_sub, (a.n_keys - key0 + Gm::kKeysPerSub - 1) / Gm::kKeysPerSub);
  const int n_tiles = (a.n_rows + 31) / 32;
  const int n_iter = n_sub * n_tiles;
  const float* lam_unit = a.lam + (int64_t)unit * a.n_rows;
  float* out = a.scores + (int64_t)unit * a.n_keys;
  const float c = a.c;
  const char* qrows = unit_rows<T>(a, unit);
  auto wave_kbase = [&](int sc) { return key0 + sc * Gm::kKeysPerSub + wave * Gm::kKeysPerWave; };
  auto lam_of = [&](int rt) {
    const int rr = rt * 32 + threadIdx.x;
    const float v = lam_unit[rr < a.n_rows ? rr : 0];
    return (rr < a.n_rows) ? v : INFINITY;
  };

  u32x4 st_a[Gm::kStageVecs], st_b[Gm::kStageVecs];
  float lst_a = INFINITY, lst_b = INFINITY;
  load_q_tile<T, D>(qrows, a.n_rows, 0, st_a);
  store_q_tile<T, D>(s_tile[0], st_a);
  if (threadIdx.x < 32) s_lam[0][threadIdx.x] = lam_of(0);
  load_q_tile<T, D>(qrows, a.n_rows, iter_pos(1, n_tiles).rt, st_a);
  store_q_tile<T, D>(s_tile[1], st_a);
  if (threadIdx.x < 32) s_lam[1][threadIdx.x] = lam_of(iter_pos(1, n_tiles).rt);
  u32x4 kst[Gm::kKT][Gm::kNV];
  load_keys<T, D>(a, unit, wave_kbase(0), kst);
  load_q_tile<T, D>(qrows, a.n_rows, iter_pos(2, n_tiles).rt, st_a);
  if (threadIdx.x < 32) lst_a = lam_of(iter_pos(2, n_tiles).rt);
  __syncthreads();

  u32x4 qf[Gm::kNV];
  f32x16 acc_a[Gm::kKT], acc_b[Gm::kKT];
  read_q_frag<T, D>(s_tile[0], lane, qf);
  pass2_mfma<T, D>(kst, qf, acc_a);
  float colsum[Gm::kKT];
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) colsum[kt] = 0.f;
  int kbase_cur = wave_kbase(0);

  // lse of a tile's rows m(i) = acc_row(i, half), for the lane's half-wave.
  auto read_lam = [&](int ring, float (&lam)[16]) {
    const float* lrow = s_lam[ring];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lrow[8 * g4 + 4 * half]);
      lam[4 * g4 + 0] = l4[0];
      lam[4 * g4 + 1] = l4[1];
      lam[4 * g4 + 2] = l4[2];
      lam[4 * g4 + 3] = l4[3];
    }
  };
  float lam_a[16], lam_b[16];
  read_lam(0, lam_a);

  // One pipeline step: MFMAs of iteration it + 1 into acc_next, column sums of
  // iteration it from acc_cur (whose lse values are already in lam_cur); tile
  // it + 2 goes from the ready staging set to LDS, the loads of tile it + 3
  // start into the other set, and the lse values of tile it + 1 are read for
  // the next step.
  auto step = [&](int it, f32x16 (&acc_cur)[Gm::kKT], f32x16 (&acc_next)[Gm::kKT], float (&lam_cur)[16],
                  float (&lam_next)[16], u32x4 (&st_ready)[Gm::kStageVecs], float& lst_ready,
                  u32x4 (&st_fill)[Gm::kStageVecs], float& lst_fill) {
    const IterPos cu = iter_pos(it, n_tiles), nx = iter_pos(it + 1, n_tiles);
    if (it + 1 < n_iter && nx.rt == 0) load_keys<T, D>(a, unit, wave_kbase(nx.sc), kst);
    store_q_tile<T, D>(s_tile[(it + 2) % Gm::kRing], st_ready);
    if (threadIdx.x < 32) s_lam[(it + 2) % Gm::kRing][threadIdx.x] = lst_ready;
    const int ahead = iter_pos(it + 3, n_tiles).rt;
    load_q_tile<T, D>(qrows, a.n_rows, ahead, st_fill);
    if (threadIdx.x < 32) lst_fill = lam_of(ahead);
    read_q_frag<T, D>(s_tile[(it + 1) % Gm::kRing], lane, qf);
    pass2_mfma<T, D>(kst, qf, acc_next);
    // acc_cur[kt][i] = <q_(32 rt + acc_row(i, half)), k_(kbase_cur + 32 kt + lane % 32)>
#pragma unroll
    for (int kt = 0; kt < Gm::kKT; ++kt) {
      float s4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s4[i] = fast_exp2(__builtin_fmaf(acc_cur[kt][i], c, -lam_cur[i]));
#pragma unroll
      for (int i = 4; i < 16; ++i) s4[i & 3] += fast_exp2(__builtin_fmaf(acc_cur[kt][i], c, -lam_cur[i]));
      colsum[kt] += (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    constexpr int kMfmas = Gm::kKT * Gm::kNV * (sizeof(T) == 4 ? 4 : 1);
    __builtin_amdgcn_sched_group_barrier(0x100, Gm::kNV, 0);        // MFMA operands from LDS
    __builtin_amdgcn_sched_group_barrier(0x002, SKV_P2_VALU_LEAD, 0);  // vector work while they arrive
    interleave_mfma_valu<kMfmas, SKV_P2_VALU_PER>();
    read_lam((it + 1) % Gm::kRing, lam_next);
    if (cu.rt + 1 == n_tiles) {  // sub-chunk complete: write its column sums
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) {
        const float tot = colsum[kt] + shfl_xor32(colsum[kt]);
        const int key = kbase_cur + kt * 32 + lane;
        if (lane < 32 && key < a.n_keys) out[key] = tot;
        colsum[kt] = 0.f;
      }
      kbase_cur = wave_kbase(nx.sc);
    }
    __syncthreads();
  };
  int it = 0;
  for (; it + 1 < n_iter; it += 2) {
    step(it, acc_a, acc_b, lam_a, lam_b, st_a, lst_a, st_b, lst_b);
    step(it + 1, acc_b, acc_a, lam_b, lam_a, st_b, lst_b, st_a, lst_a);
  }
  if (it < n_iter) step(it, acc_a, acc_b, lam_a, lam_b, st_a, lst_a, st_b, lst_b);
}

// ---------------------------------------------------------------------------

int score_keys_per_sub(int dtype, int head_dim) {
  if (dtype == 0) return head_dim == 64 ? ScoreGeom<float, 64>::kKeysPerSub : ScoreGeom<float, 128>::kKeysPerSub;
  return head_dim == 64 ? ScoreGeom<bf16_t, 64>::kKeysPerSub : ScoreGeom<bf16_t, 128>::kKeysPerSub;
}

void score_plan(int dtype, int head_dim, int64_t n_units, int64_t n_keys, int32_t* n_sub, int32_t* n_chunks) {
  // Enough blocks to fill 256 CUs several times over; as few partials as that allows.
  constexpr int64_t kTargetBlocks = 4096;
  const int64_t kps = score_keys_per_sub(dtype, head_dim);
  const int64_t subs = (n_keys + kps - 1) / kps;
  int64_t chunks = (kTargetBlocks + n_units - 1) / n_units;
  chunks = chunks < 1 ? 1 : (chunks > subs ? subs : chunks);
  const int64_t per = (subs + chunks - 1) / chunks;
  *n_sub = (int32_t)per;
  *n_chunks = (int32_t)((subs + per - 1) / per);
}

static size_t score_pass1_lds_bytes(int32_t n_rows) { return (size_t)n_rows * sizeof(float2); }

template <typename T, int D>
static hipError_t launch_p1(const ScoreArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_units * a.n_chunks)), block(ScoreGeom<T, D>::kThreads);
  score_pass1_kernel<T, D><<<grid, block, score_pass1_lds_bytes(a.n_rows), s>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_p2(const ScoreArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_units * a.n_chunks)), block(ScoreGeom<T, D>::kThreads);
  score_pass2_kernel<T, D><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_score_pass1(int dtype, int head_dim, const ScoreArgs& a, hipStream_t s) {
  if (dtype == 0) return head_dim == 64 ? launch_p1<float, 64>(a, s) : launch_p1<float, 128>(a, s);
  return head_dim == 64 ? launch_p1<bf16_t, 64>(a, s) : launch_p1<bf16_t, 128>(a, s);
}

hipError_t launch_lse_combine(const ScoreArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_units * a.n_rows;
  lse_combine_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_score_pass2(int dtype, int head_dim, const ScoreArgs& a, hipStream_t s) {
  if (dtype == 0) return head_dim == 64 ? launch_p2<float, 64>(a, s) : launch_p2<float, 128>(a, s);
  return head_dim == 64 ? launch_p2<bf16_t, 64>(a, s) : launch_p2<bf16_t, 128>(a, s);
}

}  // namespace skv
