// Pooling and top-C_max selection (paper notes "Draft-based Approximate
// Inference for LLMs": section "Key designs", SpecKV keeps the top C_max KV
// pairs plus the window pairs; section "Loss / training strategy", local
// pooling keeps the kept tokens contiguous).
//
// One 1024-thread block per unit (layer, KV head), working on the
// order-preserving uint32 image of the fp32 pooled values.  For n_pre up to
// 64K the keys stay in registers: wave w owns a contiguous index span, lane l
// step i holds index w S + 64 i + l.
//   1. pooled[j] = max (or in-range mean) of scores over |j' - j| <= r; max
//      pools up to width 65 (and no pooling) are computed in registers from
//      one coalesced load per score, with lane rotations for the neighbours;
//   2. the n_top-th largest key T is found bit by bit from the top
//      (T | bit is kept when at least n_top keys are >= it), each count a
//      per-lane sum, seven ballots and one sum over the 16 waves; the search
//      ends early once the top set is known exactly or T's remaining range
//      holds it as its largest key;
//   3. keys > T are all taken, and of the keys equal to T the lowest-index
//      k_rem ones; wave-level counts and scans over the waves give each wave
//      its output offset, so one in-order sweep writes the kept list
//      ascending; the window keys are appended after it.
// Units that are long for their number (few heads, long context) run in two
// stages: segments keep their own top n_top as candidates, then one block per
// unit applies the same rule to the candidates.  Longer units still use an
// LDS-histogram radix select with a tile-by-tile block scan.  Integer
// decisions only: bit-exact and run-to-run deterministic.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace skv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// Exclusive prefix count of `flag` over the block (thread order); also the total.
__device__ __forceinline__ uint32_t block_prefix(bool flag, uint32_t* s_tot, uint32_t& total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const uint64_t m = __ballot(flag);
  const uint32_t lane_pre = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_tot[wave] = __popcll(m);
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t t = s_tot[w];
    pre += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return pre + lane_pre;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_tot[kSelWaves];
  __shared__ uint32_t s_pick[2];

  const int unit = blockIdx.x;
  const int n = a.n_pre, tid = threadIdx.x;
  const float* sc = a.scores + (int64_t)unit * n;
  float* pl = a.pooled + (int64_t)unit * n;
  int32_t* kept = a.kept + (int64_t)unit * (a.n_top + a.n_window);

  // 1. pooling (stride 1, windows truncated at both ends)
  const int r = a.pool_radius;
  for (int j = tid; j < n; j += kSelThreads) {
    float v = sc[j];
    if (a.pool == 1) {
      for (int o = 1; o <= r; ++o) {
        if (j - o >= 0) v = fmaxf(v, sc[j - o]);
        if (j + o < n) v = fmaxf(v, sc[j + o]);
      }
    } else if (a.pool == 2 && r > 0) {
      const int lo = j - r < 0 ? 0 : j - r, hi = j + r >= n ? n - 1 : j + r;
      float s = 0.f;
      for (int t = lo; t <= hi; ++t) s += sc[t];
      v = s / (float)(hi - lo + 1);
    }
    pl[j] = v;
  }
  for (int t = tid; t < a.n_window; t += kSelThreads) kept[a.n_top + t] = n + t;
  if (a.n_top >= n) {
    for (int j = tid; j < n; j += kSelThreads) kept[j] = j;
    return;
  }
  if (a.n_top == 0) return;
  __syncthreads();  // pooled values visible to the whole block

  // 2. radix select of the n_top-th largest key
  uint32_t prefix = 0u, mask = 0u, k_rem = (uint32_t)a.n_top;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) s_hist[tid] = 0u;
    __syncthreads();
    for (int j = tid; j < n; j += kSelThreads) {
      const uint32_t key = ordered_key(pl[j]);
      if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0u;
      int d = 255;
      for (; d > 0; --d) {
        if (cum + s_hist[d] >= k_rem) break;
        cum += s_hist[d];
      }
      s_pick[0] = (uint32_t)d;
      s_pick[1] = k_rem - cum;
    }
    __syncthreads();
    prefix |= s_pick[0] << shift;
    mask |= 255u << shift;
    k_rem = s_pick[1];
  }
  const uint32_t T = prefix;  // ordered key of the n_top-th largest value; take k_rem keys equal to it

  // 3. ascending emission
  uint32_t run_eq = 0u, run_sel = 0u;
  for (int base = 0; base < n && run_sel < (uint32_t)a.n_top; base += kSelThreads) {
    const int j = base + tid;
    const uint32_t key = (j < n) ? ordered_key(pl[j]) : 0u;
    const bool gt = j < n && key > T;
    const bool eq = j < n && key == T;
    uint32_t eq_tot, sel_tot;
    const uint32_t eq_rank = run_eq + block_prefix(eq, s_tot, eq_tot);
    const bool take = gt || (eq && eq_rank < k_rem);
    const uint32_t pos = run_sel + block_prefix(take, s_tot, sel_tot);
    if (take && pos < (uint32_t)a.n_top) kept[pos] = j;
    run_eq += eq_tot;
    run_sel += sel_tot;
  }
}

// Pooled value at j (pool 0: none, 1: max, 2: in-range mean; radius r).
// Max pooling reads clamped neighbours: a truncated window only repeats
// in-range values, which leaves the max unchanged, and the loads carry no
// branches.
__device__ __forceinline__ float pooled_at(const float* sc, int j, int n, int pool, int r) {
  if (pool == 1) {
    float v = sc[j];
    for (int o = 1; o <= r; ++o) v = fmaxf(v, fmaxf(sc[max(j - o, 0)], sc[min(j + o, n - 1)]));
    return v;
  }
  if (pool == 2 && r > 0) {
    const int lo = j - r < 0 ? 0 : j - r, hi = j + r >= n ? n - 1 : j + r;
    float s = 0.f;
    for (int t = lo; t <= hi; ++t) s += sc[t];
    return s / (float)(hi - lo + 1);
  }
  return sc[j];
}

// Value held by lane (lane + o) mod 64.
__device__ __forceinline__ float lane_rot(float v, int lane, int o) { return __shfl(v, (lane + o) & (kWave - 1)); }

// Max pool of width 2r + 1 (0 <= r <= 32) at the wave's positions
// first + 64 i + lane, i < E, held in registers.  at(i) is the score at step
// i's position, for i in [-1, E]: the caller clamps positions to [0, n), so
// that a clamped neighbour repeats an in-range value, which leaves a max
// unchanged (windows truncated at both ends), and a padding position next to
// a valid one holds its real neighbour.  Each score is loaded once,
// coalesced.  Maxima over the L positions starting at p are built by
// doubling L; the window [p - r, p + r] is then the max of the L-window
// starting at p - r and the one starting at p + r + 1 - L, for the largest
// power of two L <= 2r + 1.  Every shift is one lane rotation: the lanes it
// wraps take the rotated value of the adjacent step, and a wrapped lane of
// the last step only reaches positions past the ones pooled.
// R >= 0 fixes r at compile time; R = -2 takes r_rt.
template <int E, int R, class At>
__device__ __forceinline__ void pool_regs(At at, int lane, int r_rt, float (&out)[E]) {
  const int r = R >= 0 ? R : r_rt;
  float F[E + 2];  // F[j]: step j - 1, j = 0 .. E + 1
#pragma unroll
  for (int j = 0; j < E + 2; ++j) F[j] = at(j - 1);
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < E; ++i) out[i] = F[i + 1];
    return;
  }
  if constexpr (R == 3) {
    // Width 7: the max over pairs, then fours, then the four ending at p
    // and the four starting at p (fewer live values than the general form).
    float rx[E + 2], m2[E + 2];
#pragma unroll
    for (int j = 0; j < E + 2; ++j) rx[j] = lane_rot(F[j], lane, 1);
#pragma unroll
    for (int j = 0; j < E + 2; ++j) {
      const float nxt = rx[j + 1 < E + 2 ? j + 1 : j];  // the last step's lane 63 is never used
      m2[j] = fmaxf(F[j], lane < kWave - 1 ? rx[j] : nxt);
    }
    float rm2[E + 2], m4[E + 1];
#pragma unroll
    for (int j = 0; j < E + 2; ++j) rm2[j] = lane_rot(m2[j], lane, 2);
#pragma unroll
    for (int j = 0; j < E + 1; ++j) m4[j] = fmaxf(m2[j], lane < kWave - 2 ? rm2[j] : rm2[j + 1]);
    float rm4[E + 1];
#pragma unroll
    for (int j = 0; j < E + 1; ++j) rm4[j] = lane_rot(m4[j], lane, kWave - 3);
#pragma unroll
    for (int i = 0; i < E; ++i) out[i] = fmaxf(m4[i + 1], lane >= 3 ? rm4[i + 1] : rm4[i]);
    return;
  }
  int L = 1;
  for (; 2 * L <= 2 * r + 1; L *= 2) {  // F: max over [p, p + L) -> over [p, p + 2L)
    float nxt = lane_rot(F[0], lane, L);
#pragma unroll
    for (int j = 0; j < E + 2; ++j) {
      const float cur = nxt;
      if (j + 1 < E + 2) nxt = lane_rot(F[j + 1], lane, L);
      F[j] = fmaxf(F[j], lane + L < kWave ? cur : nxt);
    }
  }
  const int s = r + 1 - L;  // second window's start relative to p, in (-r, L)
  float RA[E + 1], RS[E + 2];
#pragma unroll
  for (int j = 0; j < E + 1; ++j) RA[j] = lane_rot(F[j], lane, kWave - r);
  if (s == 0) {
#pragma unroll
    for (int j = 0; j < E + 2; ++j) RS[j] = F[j];
  } else {
#pragma unroll
    for (int j = 0; j < E + 2; ++j) RS[j] = lane_rot(F[j], lane, s);
  }
  const bool a_here = lane >= r, b_here = (unsigned)(lane + s) < (unsigned)kWave;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int j = i + 1;
    const float a = a_here ? RA[j] : RA[j - 1];                               // window at p - r
    const float b = b_here ? RS[j] : (s >= 0 ? RS[j + 1] : RS[j - 1]);        // window at p + s
    out[i] = fmaxf(a, b);
  }
}

// Sum of one value per wave over the block's 16 waves (every thread gets it).
// Also returns the sum over the waves before this one.
__device__ __forceinline__ uint32_t waves_sum(uint32_t v, uint32_t* s_red, uint32_t& before) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  uint32_t tot = 0, pre = 0;
#pragma unroll
  for (int w4 = 0; w4 < kSelWaves / 4; ++w4) {
    const u32x4 t4 = reinterpret_cast<const u32x4*>(s_red)[w4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pre += (4 * w4 + q < wave) ? t4[q] : 0u;
      tot += t4[q];
    }
  }
  __syncthreads();
  before = pre;
  return tot;
}

// Maximum over the wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Maximum of one wave-uniform value per wave over the block's 16 waves.
__device__ __forceinline__ uint32_t waves_max(uint32_t v, uint32_t* s_red) {
  if (threadIdx.x % kWave == 0) s_red[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t m = 0u;
#pragma unroll
  for (int w4 = 0; w4 < kSelWaves / 4; ++w4) {
    const u32x4 t4 = reinterpret_cast<const u32x4*>(s_red)[w4];
    m = max(max(m, max(t4[0], t4[1])), max(t4[2], t4[3]));
  }
  __syncthreads();
  return m;
}

// Sum over the wave of a per-lane count below 128, as seven ballots over
// its bits (the result is wave-uniform).
__device__ __forceinline__ uint32_t wave_count(uint32_t c) {
  uint32_t t = 0u;
#pragma unroll
  for (int b = 0; b < 7; ++b) t += (uint32_t)__popcll(__ballot((c >> b) & 1u)) << b;
  return t;
}

enum SelMode { kSelDirect = 0, kSelSegment = 1, kSelMerge = 2 };

// Selection with the keys of one block in registers (up to 64 per lane).
//   direct : block = unit; keys = pooled scores; writes the kept list.
//   segment: block = (unit, segment); keys = pooled scores of the segment;
//            writes the segment's own top n_top as (key, index) candidates.
//   merge  : block = unit; keys = the segments' candidates in segment order
//            (so in index order); writes the kept list.
// The unit's top n_top is contained in the union of the segments' own top
// n_top (lowest indices first on ties in both), so the merge is exact.
// R: 0 or 3 pools in registers with that radius (no pooling, the width-7 max
// pool), -2 the max pool of the run-time radius (at most 32) in registers,
// -1 any pool mode and radius through the pooled buffer.
template <int E, int R, int MODE>
__global__ __launch_bounds__(kSelThreads) void select_reg_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t s_red[kSelWaves];
  __shared__ __attribute__((aligned(16))) uint32_t s_cnt[2][kSelWaves];  // the threshold search's counts
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n = a.n_pre;
  int unit = blockIdx.x, s0 = 0, len = n, n_top = a.n_top;
  if (MODE == kSelSegment) {
    unit = blockIdx.x / a.n_seg;
    s0 = (blockIdx.x % a.n_seg) * a.seg_len;
    len = min(a.seg_len, n - s0);
    n_top = min(a.n_top, len);
  } else if (MODE == kSelMerge) {
    len = a.n_seg * a.n_top;
  }
  const float* sc = a.scores + (int64_t)unit * n;
  float* pl = a.pooled + (int64_t)unit * n;
  int32_t* kept = a.kept + (int64_t)unit * (a.n_top + a.n_window);
  const int64_t cbase = (int64_t)unit * a.n_seg * a.n_top + (MODE == kSelSegment ? (int64_t)(blockIdx.x % a.n_seg) * a.n_top : 0);
  uint32_t* cand_key = a.cand_key + cbase;
  int32_t* cand_idx = a.cand_idx + cbase;
  const int span = (len + kSelThreads - 1) / kSelThreads * kWave;  // positions per wave (contiguous)
  const int base = wave * span;
  const int lim = min(span, len - base) - lane;  // this lane's step i holds a position iff i * 64 < lim

  if (MODE != kSelSegment)
    for (int t = tid; t < a.n_window; t += kSelThreads) kept[a.n_top + t] = n + t;
  if (len <= 0) return;  // nothing to select (an empty prefix keeps the window only); block-uniform

  // 1. keys; key 0 marks padding (every non-negative score maps above 2^31)
  uint32_t key[E];
  if constexpr (MODE == kSelMerge) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int p = base + i * kWave + lane;
      const int pc = min(p, len - 1);
      const int seg = pc / a.n_top;
      const int seg_keep = min(a.n_top, min(a.seg_len, n - seg * a.seg_len));
      const uint32_t k = cand_key[pc];
      key[i] = (i * kWave < lim && pc - seg * a.n_top < seg_keep) ? k : 0u;
    }
  } else if constexpr (R != -1) {  // max pool in registers
    // Chunks of steps, each with its own neighbour loads, bound the registers
    // in flight next to the keys already made.
    constexpr int C = E <= 32 ? E : (R >= 0 ? 32 : (MODE == kSelDirect ? 16 : 8));
#pragma unroll
    for (int c = 0; c < E; c += C) {
      float v[C];
      const int first = s0 + base + c * kWave;
      if (first >= kWave && first + (C + 1) * kWave <= n) {  // every load in range (wave-uniform)
        const float* p = sc + first + lane;
        pool_regs<C, R>([&](int i) { return p[i * kWave]; }, lane, a.pool_radius, v);
      } else {
        pool_regs<C, R>([&](int i) { return sc[min(max(first + i * kWave + lane, 0), n - 1)]; }, lane,
                        a.pool_radius, v);
      }
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const int st = c + i;
        if (a.write_pooled && st * kWave < lim) pl[s0 + base + st * kWave + lane] = v[i];
        key[st] = (st * kWave < lim) ? ordered_key(v[i]) : 0u;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll 8
    for (int i = 0; i < E; ++i) {
      const int p = base + i * kWave + lane;
      if (i * kWave < lim) pl[s0 + p] = pooled_at(sc, s0 + p, n, a.pool, a.pool_radius);
    }
    __syncthreads();  // the block's pooled values are visible to all its threads
    const float* pl_lane = pl + s0 + base + lane;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float v = pl_lane[min(i * kWave, len - 1 - base - lane)];  // clamped: no branch, padding dropped
      key[i] = (i * kWave < lim) ? ordered_key(v) : 0u;
    }
  }
  // Index (in the unit) of the element at step i of this lane.
  auto index_of = [&](int i) -> int {
    const int p = base + i * kWave + lane;
    if constexpr (MODE == kSelMerge) return cand_idx[p];
    return s0 + p;
  };
  auto emit = [&](uint32_t pos, int i) {
    if constexpr (MODE == kSelSegment) {
      cand_key[pos] = key[i];
      cand_idx[pos] = index_of(i);
    } else {
      kept[pos] = index_of(i);
    }
  };

  if (n_top == 0) return;
  if (n_top >= len) {  // everything is kept (direct or segment only: a merge always has more candidates)
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (i * kWave < lim) emit((uint32_t)(base + i * kWave + lane), i);
    return;
  }

  // 2. T = the n_top-th largest key, bit by bit from the top: T keeps the
  //    bits found so far, at least n_top keys are >= T, fewer than n_top lie
  //    above T's range [T, T + 2^(b+1)).  Two exits end the search early:
  //    * exactly n_top keys are >= a candidate: they are the top n_top with
  //      no tie across the boundary, and T = candidate - 1 takes nothing
  //      equal to it (usual for distinct scores, about halfway down);
  //    * after 16 and after 24 bits, the largest key m in T's range: if at
  //      least n_top keys are >= m, T is m (usual when max pooling has spread
  //      the boundary value over neighbouring positions).
  //    Each count adds vector compares for 3/8 of the keys and wave ballots
  //    with scalar popcounts for the rest (the two issue side by side), then
  //    one sum over the waves through a double-buffered LDS row: one barrier
  //    per bit (a wave writes a row only after every wave has passed the
  //    barrier that followed its previous reads of that row).
  constexpr int kVecCount = (3 * E) / 8;
  uint32_t T = 0u, before;
  int round = 0;
  for (int b = 31; b >= 0; --b) {
    if (b == 15 || b == 7) {
      uint32_t m = 0u;  // the range holds a key (at least n_top keys are >= T, fewer above the range)
#pragma unroll
      for (int i = 0; i < E; ++i) m = (key[i] - T < (2u << b)) ? max(m, key[i]) : m;
      m = waves_max(wave_max(m), s_red);
      uint32_t c = 0u;
#pragma unroll
      for (int i = 0; i < E; ++i) c += key[i] >= m ? 1u : 0u;
      if (waves_sum(wave_count(c), s_red, before) >= (uint32_t)n_top) {
        T = m;
        break;
      }
    }
    const uint32_t cand = T | (1u << b);
    uint32_t c = 0u, cs = 0u;
#pragma unroll
    for (int i = 0; i < kVecCount; ++i) c += key[i] >= cand ? 1u : 0u;
#pragma unroll
    for (int i = kVecCount; i < E; ++i) cs += (uint32_t)__popcll(__ballot(key[i] >= cand));
    const uint32_t wc = wave_count(c) + cs;  // ballots: every lane active
    uint32_t* row = s_cnt[round & 1];
    ++round;
    if (lane == 0) row[wave] = wc;
    __syncthreads();
    uint32_t cnt = 0u;  // block-uniform
#pragma unroll
    for (int w4 = 0; w4 < kSelWaves / 4; ++w4) {
      const u32x4 t4 = reinterpret_cast<const u32x4*>(row)[w4];
      cnt += (t4[0] + t4[1]) + (t4[2] + t4[3]);
    }
    if (cnt == (uint32_t)n_top) {
      T = cand - 1u;
      break;
    }
    if (cnt > (uint32_t)n_top) T = cand;
  }

  // 3. ascending emission: every key > T, and the k_rem lowest-index keys == T
  uint32_t gt_l = 0u, eq_l = 0u;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    gt_l += key[i] > T ? 1u : 0u;
    eq_l += key[i] == T ? 1u : 0u;
  }
  const uint32_t gt = wave_count(gt_l), eq = wave_count(eq_l);
  uint32_t gt_before, eq_before;
  const uint32_t k_rem = (uint32_t)n_top - waves_sum(gt, s_red, gt_before);
  waves_sum(eq, s_red, eq_before);
  const uint32_t eq_take = eq_before >= k_rem ? 0u : (k_rem - eq_before < eq ? k_rem - eq_before : eq);
  uint32_t run_sel;
  waves_sum(gt + eq_take, s_red, run_sel);
  uint32_t run_eq = eq_before;
  const uint64_t lower = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const uint64_t m_eq = __ballot(key[i] == T);
    const bool is_eq = key[i] == T;
    const bool take = key[i] > T || (is_eq && run_eq + (uint32_t)__popcll(m_eq & lower) < k_rem);
    const uint64_t m_take = __ballot(take);
    if (take) emit(run_sel + (uint32_t)__popcll(m_take & lower), i);
    run_eq += (uint32_t)__popcll(m_eq);
    run_sel += (uint32_t)__popcll(m_take);
  }
}

constexpr int kSelMaxPerLane = 64;
constexpr int kRegPoolMaxRadius = 32;  // register pools reach one step (64 positions) to either side

static int per_lane(int64_t len) { return (int)((len + kSelThreads - 1) / kSelThreads); }

int select_segments(int64_t n_units, int64_t n_pre, int64_t n_top) {
  if (n_top <= 0 || n_top >= n_pre) return 1;
  if (n_units >= 128 && per_lane(n_pre) <= kSelMaxPerLane) return 1;  // one block per unit fills the GPU
  // Balance segment length against candidate count (B ~ sqrt(n / n_top)),
  // within the register capacity of both stages.
  int64_t b = (int64_t)(sqrt((double)n_pre / (double)n_top) + 0.5);
  if (b < 2) b = 2;
  while (b > 2 && b * n_top > (int64_t)kSelThreads * kSelMaxPerLane) --b;
  while (per_lane((n_pre + b - 1) / b) > kSelMaxPerLane) ++b;
  if (b * n_top > (int64_t)kSelThreads * kSelMaxPerLane) return 1;  // too many candidates: single stage
  return (int)b;
}

size_t select_candidate_bytes(int64_t n_units, int64_t n_pre, int64_t n_top) {
  const int b = select_segments(n_units, n_pre, n_top);
  return b > 1 ? (size_t)(n_units * b * n_top) * 8 : 0;
}

template <int MODE, int R>
static void launch_mode(const SelectArgs& a, dim3 grid, int len, hipStream_t s) {
  const dim3 block(kSelThreads);
  const int e = per_lane(len);
  if (e <= 4) select_reg_kernel<4, R, MODE><<<grid, block, 0, s>>>(a);
  else if (e <= 8) select_reg_kernel<8, R, MODE><<<grid, block, 0, s>>>(a);
  else if (e <= 16) select_reg_kernel<16, R, MODE><<<grid, block, 0, s>>>(a);
  else if (e <= 32) select_reg_kernel<32, R, MODE><<<grid, block, 0, s>>>(a);
  else if constexpr (R == -2 && MODE == kSelSegment)  // the register pool of a run-time radius
    select_reg_kernel<64, -1, MODE><<<grid, block, 0, s>>>(a);  // would not fit beside 64 segment keys
  else select_reg_kernel<64, R, MODE><<<grid, block, 0, s>>>(a);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const bool r3 = a.pool == 1 && a.pool_radius == 3;                       // the width-7 max pool
  const bool r0 = a.pool_radius == 0;                                       // no pooling (or width 1)
  const bool rmax = a.pool == 1 && a.pool_radius <= kRegPoolMaxRadius;      // other max pools in registers
  if (a.n_seg > 1) {
    const dim3 g1((unsigned)((int64_t)a.n_units * a.n_seg));
    if (r3) launch_mode<kSelSegment, 3>(a, g1, a.seg_len, s);
    else if (r0) launch_mode<kSelSegment, 0>(a, g1, a.seg_len, s);
    else if (rmax) launch_mode<kSelSegment, -2>(a, g1, a.seg_len, s);
    else launch_mode<kSelSegment, -1>(a, g1, a.seg_len, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_mode<kSelMerge, -1>(a, dim3((unsigned)a.n_units), a.n_seg * a.n_top, s);
    return hipGetLastError();
  }
  if (per_lane(a.n_pre) <= kSelMaxPerLane) {
    if (r3) launch_mode<kSelDirect, 3>(a, dim3((unsigned)a.n_units), a.n_pre, s);
    else if (r0) launch_mode<kSelDirect, 0>(a, dim3((unsigned)a.n_units), a.n_pre, s);
    else if (rmax) launch_mode<kSelDirect, -2>(a, dim3((unsigned)a.n_units), a.n_pre, s);
    else launch_mode<kSelDirect, -1>(a, dim3((unsigned)a.n_units), a.n_pre, s);
  } else {
    select_kernel<<<dim3((unsigned)a.n_units), dim3(kSelThreads), 0, s>>>(a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row gather for compaction (paper notes, "Key designs", SpecKV: the kept KV
// pairs form the compressed cache; SpecKV-PC: the target cache over the
// SpecPC kept tokens, one token list for every head; or the kept rows of
// a cache addressed through that list).  One thread copies one 16-byte
// vector; consecutive threads cover consecutive bytes of a row.  Source
// indices outside [0, n_src_rows) produce zero rows instead of faulting.

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int vpr = a.row_bytes / 16;
  const int64_t per_unit = (int64_t)a.n_rows * vpr;
  const int64_t blocks_per_unit = (per_unit + 255) / 256;
  const int64_t unit = blockIdx.x / blocks_per_unit;
  const int64_t t = (blockIdx.x % blocks_per_unit) * 256 + threadIdx.x;
  if (unit >= a.n_units || t >= per_unit) return;
  const int row = (int)(t / vpr), col = (int)(t % vpr);
  int src_row = a.idx ? a.idx[unit * a.idx_unit_stride + row] : row;
  if (a.idx2) src_row = (src_row >= 0 && src_row < a.n_idx2) ? a.idx2[src_row] : -1;
  // source unit: same layer, head (unit % units_per_layer) / src_repeat
  const int64_t src_unit = (unit / a.units_per_layer) * a.src_units_per_layer + (unit % a.units_per_layer) / a.src_repeat;
  const char* src = static_cast<const char*>(blockIdx.y ? a.src2 : a.src);  // grid row 1: the second tensor
  char* dst = static_cast<char*>(blockIdx.y ? a.dst2 : a.dst) + unit * a.dst_unit_stride + (int64_t)row * a.row_bytes +
              col * 16;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (src_row >= 0 && src_row < a.n_src_rows)
    v = ldg16(src + src_unit * a.src_unit_stride + (int64_t)src_row * a.row_bytes + col * 16);
  *reinterpret_cast<u32x4*>(dst) = v;
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const int64_t per_unit = (int64_t)a.n_rows * (a.row_bytes / 16);
  const int64_t blocks = (per_unit + 255) / 256 * a.n_units;
  gather_kernel<<<dim3((unsigned)blocks, a.src2 ? 2u : 1u), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace skv
