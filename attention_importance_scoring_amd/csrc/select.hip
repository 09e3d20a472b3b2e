// Pooling and top-C_max selection (paper notes "Draft-based Approximate
// Inference for LLMs": section "Key designs", SpecKV keeps the top C_max KV
// pairs plus the window pairs; section "Loss / training strategy", local
// pooling keeps the kept tokens contiguous).
//
// One 1024-thread block per unit (layer, KV head):
//   1. pooled[j] = max (or in-range mean) of scores over |j' - j| <= r;
//   2. radix select, four 8-bit digits from the most significant, on the
//      order-preserving uint32 image of the fp32 pooled values, finds the
//      n_top-th largest value T and how many keys equal to T are taken;
//   3. one ascending sweep emits keys with value > T, and the lowest-index
//      keys equal to T, in index order (ballot prefix sums), so the kept
//      list comes out sorted; the window keys are appended after them.
// Integer decisions only: bit-exact and run-to-run deterministic.
#include "common.hpp"
#include "kernels.hpp"

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

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  select_kernel<<<dim3((unsigned)a.n_units), dim3(kSelThreads), 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row gather for compaction (paper notes, "Key designs", SpecKV: the kept KV
// pairs form the compressed cache).  One thread copies one 16-byte vector;
// consecutive threads cover consecutive bytes of a row.  Source indices
// outside [0, n_src_rows) produce zero rows instead of faulting.

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int vpr = a.row_bytes / 16;
  const int64_t per_unit = (int64_t)a.n_rows * vpr;
  const int64_t blocks_per_unit = (per_unit + 255) / 256;
  const int64_t unit = blockIdx.x / blocks_per_unit;
  const int64_t t = (blockIdx.x % blocks_per_unit) * 256 + threadIdx.x;
  if (unit >= a.n_units || t >= per_unit) return;
  const int row = (int)(t / vpr), col = (int)(t % vpr);
  const int src_row = a.idx ? a.idx[unit * a.n_rows + row] : row;
  char* dst = static_cast<char*>(a.dst) + unit * a.dst_unit_stride + (int64_t)row * a.row_bytes + col * 16;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (src_row >= 0 && src_row < a.n_src_rows)
    v = ldg16(static_cast<const char*>(a.src) + unit * a.src_unit_stride + (int64_t)src_row * a.row_bytes + col * 16);
  *reinterpret_cast<u32x4*>(dst) = v;
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const int64_t per_unit = (int64_t)a.n_rows * (a.row_bytes / 16);
  const int64_t blocks = (per_unit + 255) / 256 * a.n_units;
  gather_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace skv
