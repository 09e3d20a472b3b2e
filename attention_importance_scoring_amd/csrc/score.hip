// Two-pass importance scoring on gfx950 (paper notes "Draft-based
// Approximate Inference for LLMs", section "Key designs": SpecKV scores each
// remaining input key by the cross-attention of the observation queries;
// SpecPC reads the draft's causal attention rows).
//
// Pass 1 (row statistics): for every query row r, the log2-domain
//   lse_r = log2 sum_j 2^(c * <q_r, k_j>),  c = scale * log2(e),
// built from per-chunk (max, sum) partials so that the score matrix is never
// stored.  Pass 2 (column sums): score_j = sum_r 2^(c * <q_r, k_j> - lse_r).
//
// Work split: a block owns kKeysPerBlock consecutive keys of one unit
// (layer, KV head); each of its four waves keeps kKT tiles of 32 keys
// resident in registers as an MFMA operand for the whole block lifetime,
// and the block streams the unit's query rows through LDS 32 rows at a time
// (double buffered, one barrier per row tile).  Pass 1 puts keys on the MFMA
// M dimension and rows on N so that each lane reduces one row in-lane;
// pass 2 swaps the operands so that each lane owns one key column.  No
// floating-point atomics: every sum has a fixed order.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace skv {

template <typename T, int D>
struct ScoreGeom {
  using RF = RowFrag<T, D>;
  static constexpr int kNV = RF::kNV;
  static constexpr int kKT = (RF::kHalfBytes <= 128) ? 4 : 2;  // resident key tiles per wave
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKeysPerWave = 32 * kKT;
  static constexpr int kKeysPerBlock = kWaves * kKeysPerWave;
  static constexpr int kRowPitch = RF::kRowBytes + 16;  // LDS pitch, padded against bank conflicts
  static constexpr int kTileBytes = 32 * kRowPitch;
  static constexpr int kVecPerRow = RF::kRowBytes / 16;
  static constexpr int kStageVecs = 32 * kVecPerRow / kThreads;  // 16-byte loads per thread per tile
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

// Loads this thread's share of query row tile `rt` of `unit` into registers.
template <typename T, int D>
__device__ __forceinline__ void load_q_tile(const ScoreArgs& a, int unit, int rt, u32x4 (&st)[ScoreGeom<T, D>::kStageVecs]) {
  using Gm = ScoreGeom<T, D>;
  const int layer = a.layer0 + unit / a.n_kv_heads;
  const int kvh = unit % a.n_kv_heads;
  const char* qbase = static_cast<const char*>(a.q) +
                      (layer * a.q_layer_stride + (int64_t)kvh * a.group * a.q_head_stride) * Elem<T>::kBytes;
#pragma unroll
  for (int p = 0; p < Gm::kStageVecs; ++p) {
    const int idx = p * Gm::kThreads + threadIdx.x;
    const int row = idx / Gm::kVecPerRow, col = idx % Gm::kVecPerRow;
    const int rr = rt * 32 + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (rr < a.n_rows) {
      const int g = rr / a.rows_per_qhead, i = rr - g * a.rows_per_qhead;
      v = ldg16(qbase + ((int64_t)g * a.q_head_stride + (int64_t)i * D) * Elem<T>::kBytes + col * 16);
    }
    st[p] = v;
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
    const char* row = kb + (int64_t)key * Gm::RF::kRowBytes + half * Gm::RF::kHalfBytes;
#pragma unroll
    for (int v = 0; v < Gm::kNV; ++v) kst[kt][v] = (key < a.n_keys) ? ldg16(row + v * 16) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void score_pass1_kernel(ScoreArgs a) {
  using Gm = ScoreGeom<T, D>;
  __shared__ __attribute__((aligned(16))) char s_tile[2][Gm::kTileBytes];
  __shared__ RowStat s_stat[2][Gm::kWaves][32];

  const int logical = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int unit = logical / a.n_chunks, chunk = logical % a.n_chunks;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, half = lane / 32;
  const int kbase = chunk * Gm::kKeysPerBlock + wave * Gm::kKeysPerWave;
  const int n_tiles = (a.n_rows + 31) / 32;

  u32x4 kst[Gm::kKT][Gm::kNV];
  load_keys<T, D>(a, unit, kbase, kst);

  // Keys of this wave beyond n_keys, or (causal) beyond the earliest row position, need masking.
  const bool wave_needs_mask =
      (kbase + Gm::kKeysPerWave > a.n_keys) || (a.causal && (int64_t)kbase + Gm::kKeysPerWave - 1 > a.pos_base);

  u32x4 st[Gm::kStageVecs];
  load_q_tile<T, D>(a, unit, 0, st);
  store_q_tile<T, D>(s_tile[0], st);
  __syncthreads();

  float2* part = a.part + ((int64_t)unit * a.n_chunks + chunk) * a.n_rows;
  const float c = a.c;

  for (int rt = 0; rt < n_tiles; ++rt) {
    const int buf = rt & 1;
    if (rt + 1 < n_tiles) load_q_tile<T, D>(a, unit, rt + 1, st);

    // Merge the previous tile's per-wave statistics (visible since the last barrier).
    if (rt > 0 && wave == ((rt - 1) & 3) && lane < 32) {
      RowStat m = s_stat[buf ^ 1][0][lane];
#pragma unroll
      for (int w = 1; w < Gm::kWaves; ++w) m = merge_stat(m, s_stat[buf ^ 1][w][lane]);
      const int rr = (rt - 1) * 32 + lane;
      if (rr < a.n_rows) part[rr] = make_float2(m.m, m.s);
    }

    // Masked keys start the accumulator at -inf, so they drop out of the max and the sum.
    f32x16 acc[Gm::kKT];
    if (!wave_needs_mask) {
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = f32x16{};
    } else {
      int64_t lim = (int64_t)a.n_keys - 1;
      if (a.causal) {
        const int rr = rt * 32 + (lane % 32);
        const int g = rr / a.rows_per_qhead;
        const int64_t pos = a.pos_base + (rr - g * a.rows_per_qhead);
        lim = pos < lim ? pos : lim;
      }
      int64_t rel64 = lim - kbase - 4 * half;  // key offset within the wave's range, half removed
      rel64 = rel64 < -4096 ? -4096 : (rel64 > 4096 ? 4096 : rel64);
      const int rel = (int)rel64;
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[kt][i] = (kt * 32 + 8 * (i >> 2) + (i & 3) <= rel) ? 0.f : -INFINITY;
    }
    const char* trow = s_tile[buf] + (lane % 32) * Gm::kRowPitch + half * Gm::RF::kHalfBytes;
#pragma unroll
    for (int v = 0; v < Gm::kNV; ++v) {
      const u32x4 qv = *reinterpret_cast<const u32x4*>(trow + v * 16);
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = Mfma<T>::step(kst[kt][v], qv, acc[kt]);
    }

    // acc[kt][i] = <k_(kbase + 32 kt + acc_row(i, half)), q_(32 rt + lane % 32)>
    RowStat rs;
    {
      float mx = acc[0][0];
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[kt][i]);
      const bool empty = (mx == -INFINITY);  // every key of this lane masked
      const float my = empty ? 0.f : mx * c;
      float s = 0.f;
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += fast_exp2(__builtin_fmaf(acc[kt][i], c, -my));
      rs = {empty ? -INFINITY : my, s};
    }
    // Lanes l and l ^ 32 hold the same row over different keys.
    const RowStat other = {shfl_xor32(rs.m), shfl_xor32(rs.s)};
    rs = merge_stat(rs, other);
    if (lane < 32) s_stat[buf][wave][lane] = rs;

    if (rt + 1 < n_tiles) store_q_tile<T, D>(s_tile[buf ^ 1], st);
    __syncthreads();
  }
  {
    const int rt = n_tiles;  // merge the last tile
    if (wave == ((rt - 1) & 3) && lane < 32) {
      const int buf = (rt - 1) & 1;
      RowStat m = s_stat[buf][0][lane];
#pragma unroll
      for (int w = 1; w < Gm::kWaves; ++w) m = merge_stat(m, s_stat[buf][w][lane]);
      const int rr = (rt - 1) * 32 + lane;
      if (rr < a.n_rows) part[rr] = make_float2(m.m, m.s);
    }
  }
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

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void score_pass2_kernel(ScoreArgs a) {
  using Gm = ScoreGeom<T, D>;
  __shared__ __attribute__((aligned(16))) char s_tile[2][Gm::kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_lam[2][32];

  const int logical = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  const int unit = logical / a.n_chunks, chunk = logical % a.n_chunks;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, half = lane / 32;
  const int kbase = chunk * Gm::kKeysPerBlock + wave * Gm::kKeysPerWave;
  const int n_tiles = (a.n_rows + 31) / 32;
  const float* lam_unit = a.lam + (int64_t)unit * a.n_rows;

  u32x4 kst[Gm::kKT][Gm::kNV];
  load_keys<T, D>(a, unit, kbase, kst);

  u32x4 st[Gm::kStageVecs];
  float lst = INFINITY;
  load_q_tile<T, D>(a, unit, 0, st);
  if (threadIdx.x < 32) lst = (threadIdx.x < a.n_rows) ? lam_unit[threadIdx.x] : INFINITY;
  store_q_tile<T, D>(s_tile[0], st);
  if (threadIdx.x < 32) s_lam[0][threadIdx.x] = lst;
  __syncthreads();

  float colsum[Gm::kKT];
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) colsum[kt] = 0.f;
  const float c = a.c;

  for (int rt = 0; rt < n_tiles; ++rt) {
    const int buf = rt & 1;
    if (rt + 1 < n_tiles) {
      load_q_tile<T, D>(a, unit, rt + 1, st);
      if (threadIdx.x < 32) {
        const int rr = (rt + 1) * 32 + threadIdx.x;
        lst = (rr < a.n_rows) ? lam_unit[rr] : INFINITY;
      }
    }
    f32x16 acc[Gm::kKT];
#pragma unroll
    for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = f32x16{};
    const char* trow = s_tile[buf] + (lane % 32) * Gm::kRowPitch + half * Gm::RF::kHalfBytes;
#pragma unroll
    for (int v = 0; v < Gm::kNV; ++v) {
      const u32x4 qv = *reinterpret_cast<const u32x4*>(trow + v * 16);
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) acc[kt] = Mfma<T>::step(qv, kst[kt][v], acc[kt]);
    }
    // acc[kt][i] = <q_(32 rt + acc_row(i, half)), k_(kbase + 32 kt + lane % 32)>
    float lam[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&s_lam[buf][8 * g4 + 4 * half]);
      lam[4 * g4 + 0] = l4[0];
      lam[4 * g4 + 1] = l4[1];
      lam[4 * g4 + 2] = l4[2];
      lam[4 * g4 + 3] = l4[3];
    }
#pragma unroll
    for (int kt = 0; kt < Gm::kKT; ++kt) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += fast_exp2(__builtin_fmaf(acc[kt][i], c, -lam[i]));
      colsum[kt] += s;
    }
    if (rt + 1 < n_tiles) {
      store_q_tile<T, D>(s_tile[buf ^ 1], st);
      if (threadIdx.x < 32) s_lam[buf ^ 1][threadIdx.x] = lst;
    }
    __syncthreads();
  }
  float* out = a.scores + (int64_t)unit * a.n_keys;
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) {
    const float tot = colsum[kt] + shfl_xor32(colsum[kt]);
    const int key = kbase + kt * 32 + lane;
    if (lane < 32 && key < a.n_keys) out[key] = tot;
  }
}

int score_keys_per_block(int dtype, int head_dim) {
  if (dtype == 0) return head_dim == 64 ? ScoreGeom<float, 64>::kKeysPerBlock : ScoreGeom<float, 128>::kKeysPerBlock;
  return head_dim == 64 ? ScoreGeom<bf16_t, 64>::kKeysPerBlock : ScoreGeom<bf16_t, 128>::kKeysPerBlock;
}

hipError_t launch_score_pass1(int dtype, int head_dim, const ScoreArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_units * a.n_chunks)), block(256);
  if (dtype == 0 && head_dim == 64) score_pass1_kernel<float, 64><<<grid, block, 0, s>>>(a);
  else if (dtype == 0) score_pass1_kernel<float, 128><<<grid, block, 0, s>>>(a);
  else if (head_dim == 64) score_pass1_kernel<bf16_t, 64><<<grid, block, 0, s>>>(a);
  else score_pass1_kernel<bf16_t, 128><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_lse_combine(const ScoreArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_units * a.n_rows;
  lse_combine_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_score_pass2(int dtype, int head_dim, const ScoreArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_units * a.n_chunks)), block(256);
  if (dtype == 0 && head_dim == 64) score_pass2_kernel<float, 64><<<grid, block, 0, s>>>(a);
  else if (dtype == 0) score_pass2_kernel<float, 128><<<grid, block, 0, s>>>(a);
  else if (head_dim == 64) score_pass2_kernel<bf16_t, 64><<<grid, block, 0, s>>>(a);
  else score_pass2_kernel<bf16_t, 128><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace skv
