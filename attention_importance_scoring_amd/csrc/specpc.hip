// SpecPC token scoring, pass 2 (paper notes "Draft-based Approximate
// Inference for LLMs", section "Key designs", SpecPC: the draft's attention
// rows over a window of queries, layers below l_skip skipped, mean over
// layers and heads first, then a weighted max over the window rows).
//
// The mean must be complete before the max, so each block keeps its
// (window rows x keys) tile of the running sum
//   acc[i][j] = sum over (layer, query head) of 2^(c <q_i, k_j> - lse_i)
// in registers across all (layer, query head) pairs, with the keys of the
// current (layer, KV head) resident as MFMA operands (shared by the G query
// heads of the group) and the query rows streamed through LDS, a whole GQA
// group per barrier where it fits.  The attention tensor itself is never
// stored.  At the end each lane owns one key
// column: it takes the weighted max over its rows; a tiny second kernel
// takes the max over row blocks and applies the 1 / (layers x heads) mean.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace skv {

#ifndef SKV_PC_RT
#define SKV_PC_RT 2
#endif
#ifndef SKV_PC_WAVES
#define SKV_PC_WAVES 8
#endif

constexpr int kPcLdsBudget = 150 * 1024;  // dynamic LDS per block (one block per CU)

template <typename T, int D>
struct PcGeom {
  using RF = RowFrag<T, D>;
  static constexpr int kNV = RF::kNV;
  static constexpr int kKT = kNV >= 8 ? 1 : 2;  // key tiles per wave (resident keys at most 32 VGPRs)
  static constexpr int kRT = SKV_PC_RT;          // row tiles per block
  static constexpr int kWaves = SKV_PC_WAVES;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKeysPerWave = 32 * kKT;
  static constexpr int kKeysPerBlock = kWaves * kKeysPerWave;
  static constexpr int kRowsPerBlock = 32 * kRT;
  static constexpr int kRowPitch = RF::kRowBytes + 16;
  static constexpr int kMapBytes = kRowsPerBlock * kRowPitch;       // one (layer, query head) map's rows
  static constexpr int kMapLds = kMapBytes + kRowsPerBlock * 4;     // rows + their lse values
  static constexpr int kVecPerRow = RF::kRowBytes / 16;
  static constexpr int kVecsPerMap = kRowsPerBlock * kVecPerRow;
  static constexpr int kStageVecs = (kVecsPerMap + kThreads - 1) / kThreads;  // per thread per map
};

// Maps staged per barrier: a whole GQA group when it fits (double-buffered).
template <typename T, int D>
static int pc_maps_per_stage(int group) {
  const int fit = kPcLdsBudget / (2 * PcGeom<T, D>::kMapLds);
  return group < fit ? group : (fit < 1 ? 1 : fit);
}

// Block = (32 kRT window rows, 8 waves x 32 kKT keys).  The block walks the (layer, KV head)
// units; per unit its waves hold their keys as MFMA operands and the G query
// heads' rows stream through LDS, several maps per barrier, the next stage's
// rows loading while the current one is computed.
// The block of key block kblk and row block rb; MASKED blocks hold keys past
// the first window position (the causal diagonal).
template <typename T, int D, bool MASKED>
__device__ __forceinline__ void specpc_pass2_block(const SpecPCArgs& pa, int rb, int kblk, char* smem) {
  using Gm = PcGeom<T, D>;
  const ScoreArgs& a = pa.sc;
  const int mps = pa.maps_per_stage;
  char* s_rows = smem;                                                          // [2][mps][kMapBytes]
  float* s_lam = reinterpret_cast<float*>(smem + (size_t)2 * mps * Gm::kMapBytes);  // [2][mps][kRowsPerBlock]
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, half = lane / 32;
  const int W = a.rows_per_qhead, G = a.group;
  const int row0 = rb * Gm::kRowsPerBlock;                    // first window row of the block
  const int kbase = kblk * Gm::kKeysPerBlock + wave * Gm::kKeysPerWave;
  const int spu = (G + mps - 1) / mps;                        // stages per (layer, KV head)
  const int n_stages = a.n_units * spu;
  const float c = a.c;

  // Waves whose keys all lie after the last row's position see nothing (causal).
  const int64_t last_pos = a.pos_base + (int64_t)(row0 + Gm::kRowsPerBlock - 1);
  const bool wave_active = (int64_t)kbase <= last_pos && kbase < a.n_keys;

  auto stage_maps = [&](int st) { return min(mps, G - (st % spu) * mps); };
  // Rows (clamped to the window: rows past it get lse = +inf and add 0) and
  // lse values of map m of stage st.
  auto load_map = [&](int st, int m, u32x4 (&v)[Gm::kStageVecs], float& l) {
    const int unit = st / spu, g = (st % spu) * mps + m;
    const int layer = a.layer0 + unit / a.n_kv_heads, kvh = unit % a.n_kv_heads;
    const char* qh = static_cast<const char*>(a.q) +
                     (layer * a.q_layer_stride + (int64_t)(kvh * G + g) * a.q_head_stride) * Elem<T>::kBytes;
#pragma unroll
    for (int p = 0; p < Gm::kStageVecs; ++p) {
      const int idx = min(p * Gm::kThreads + tid, Gm::kVecsPerMap - 1);
      const int row = idx / Gm::kVecPerRow, col = idx % Gm::kVecPerRow;
      v[p] = ldg16(qh + (int64_t)min(row0 + row, W - 1) * Gm::RF::kRowBytes + col * 16);
    }
    if (tid < Gm::kRowsPerBlock) {
      const int i = row0 + tid;
      l = (i < W) ? a.lam[(int64_t)unit * a.n_rows + (int64_t)g * W + i] : INFINITY;
    }
  };
  auto store_map = [&](int buf, int m, const u32x4 (&v)[Gm::kStageVecs], float l) {
    char* dst = s_rows + (size_t)(buf * mps + m) * Gm::kMapBytes;
#pragma unroll
    for (int p = 0; p < Gm::kStageVecs; ++p) {
      const int idx = p * Gm::kThreads + tid;
      const int row = idx / Gm::kVecPerRow, col = idx % Gm::kVecPerRow;
      if (idx < Gm::kVecsPerMap) *reinterpret_cast<u32x4*>(dst + row * Gm::kRowPitch + col * 16) = v[p];
    }
    if (tid < Gm::kRowsPerBlock) s_lam[(buf * mps + m) * Gm::kRowsPerBlock + tid] = l;
  };

  f32x16 acc[Gm::kRT][Gm::kKT];
#pragma unroll
  for (int r = 0; r < Gm::kRT; ++r)
#pragma unroll
    for (int kt = 0; kt < Gm::kKT; ++kt) acc[r][kt] = f32x16{};
  u32x4 kst[Gm::kKT][Gm::kNV];

  // acc[r][kt][i] += 2^(c <q_(row0 + 32 r + acc_row(i, half)), k_(kbase + 32 kt + lane % 32)> - lse)
  auto compute_map = [&](int buf, int m) {
    const char* rows = s_rows + (size_t)(buf * mps + m) * Gm::kMapBytes;
    const float* lams = s_lam + (buf * mps + m) * Gm::kRowsPerBlock;
#pragma unroll
    for (int r = 0; r < Gm::kRT; ++r) {
      // Keys after a row's position start at -inf (causal mask), so they add 0.
      int rel = 4096;
      if constexpr (MASKED) {
        int64_t rel64 = a.pos_base + row0 + r * 32 + 4 * half - (kbase + (lane % 32));
        rel64 = rel64 < -4096 ? -4096 : (rel64 > 4096 ? 4096 : rel64);
        rel = (int)rel64;
      }
      const char* trow = rows + (r * 32 + lane % 32) * Gm::kRowPitch + half * Gm::RF::kHalfBytes;
      u32x4 qv[Gm::kNV];
#pragma unroll
      for (int v = 0; v < Gm::kNV; ++v) qv[v] = *reinterpret_cast<const u32x4*>(trow + v * 16);
      float lam[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lams[r * 32 + 8 * g4 + 4 * half]);
        lam[4 * g4 + 0] = l4[0];
        lam[4 * g4 + 1] = l4[1];
        lam[4 * g4 + 2] = l4[2];
        lam[4 * g4 + 3] = l4[3];
      }
      // One key tile at a time: its MFMAs, then its exp / add work.
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) {
        f32x16 sacc;
        if constexpr (!MASKED) {
          sacc = f32x16{};
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[i] = (kt * 32 - 8 * (i >> 2) - (i & 3) <= rel) ? 0.f : -INFINITY;
        }
#pragma unroll
        for (int v = 0; v < Gm::kNV; ++v) sacc = Mfma<T>::step(qv[v], kst[kt][v], sacc);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][kt][i] += fast_exp2(__builtin_fmaf(sacc[i], c, -lam[i]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  u32x4 sv[Gm::kStageVecs];
  float sl = INFINITY;
  for (int m = 0; m < stage_maps(0); ++m) {
    load_map(0, m, sv, sl);
    store_map(0, m, sv, sl);
  }
  __syncthreads();

  for (int st = 0; st < n_stages; ++st) {
    const int buf = st & 1;
    if (st % spu == 0 && wave_active) {
      // New (layer, KV head): this wave's resident keys (clamped rows past n_keys are never stored).
      const int unit = st / spu;
      const int layer = a.layer0 + unit / a.n_kv_heads, kvh = unit % a.n_kv_heads;
      const char* kb = static_cast<const char*>(a.k) + (layer * a.k_layer_stride + kvh * a.k_head_stride) * Elem<T>::kBytes;
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) {
        const int key = min(kbase + kt * 32 + (lane % 32), a.n_keys - 1);
        const char* row = kb + (int64_t)key * Gm::RF::kRowBytes + half * Gm::RF::kHalfBytes;
#pragma unroll
        for (int v = 0; v < Gm::kNV; ++v) kst[kt][v] = ldg16(row + v * 16);
      }
    }
    const int n_cur = stage_maps(st);
    const int n_nxt = st + 1 < n_stages ? stage_maps(st + 1) : 0;
    const int n_m = n_cur > n_nxt ? n_cur : n_nxt;
    for (int m = 0; m < n_m; ++m) {
      if (m < n_nxt) load_map(st + 1, m, sv, sl);  // into the buffer nobody reads this stage
      if (m < n_cur && wave_active) compute_map(buf, m);
      if (m < n_nxt) store_map(buf ^ 1, m, sv, sl);
    }
    __syncthreads();
  }

  // Weighted max over this block's window rows, per key.
  float wmax[Gm::kKT];
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) wmax[kt] = 0.f;
#pragma unroll
  for (int r = 0; r < Gm::kRT; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int wi = row0 + r * 32 + acc_row(i, half);
      float w = 0.f;
      if (wi < W) w = pa.weights ? pa.weights[wi] : (W == 1 ? 1.f : 0.1f + 0.9f * (float)wi / (float)(W - 1));
#pragma unroll
      for (int kt = 0; kt < Gm::kKT; ++kt) wmax[kt] = fmaxf(wmax[kt], w * acc[r][kt][i]);
    }
  float* out = pa.rowblock_max + (int64_t)rb * a.n_keys;
#pragma unroll
  for (int kt = 0; kt < Gm::kKT; ++kt) {
    const float m = fmaxf(wmax[kt], shfl_xor32(wmax[kt]));
    const int key = kbase + kt * 32 + lane;
    if (lane < 32 && key < a.n_keys) out[key] = m;
  }
}

// One launch covers every (key block, row block): blocks whose keys all
// precede the first window position (kblk < n_plain) need no causal mask.
// Every block walks all (layer, query head) maps, so plain and masked
// blocks take about the same time and share the rounds of the launch.
template <typename T, int D>
__global__ __launch_bounds__(SKV_PC_WAVES * 64, 1) void specpc_pass2_kernel(SpecPCArgs pa, int n_plain) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int logical = (int)xcd_contiguous_block(blockIdx.x, gridDim.x);
  // The row blocks of one key block are neighbours (same XCD, same time): the keys come from L2 after the first.
  const int rb = logical % pa.n_rowblocks, kblk = logical / pa.n_rowblocks;
  if (kblk < n_plain) specpc_pass2_block<T, D, false>(pa, rb, kblk, smem);  // block-uniform
  else specpc_pass2_block<T, D, true>(pa, rb, kblk, smem);
}

__global__ __launch_bounds__(256) void specpc_reduce_kernel(SpecPCArgs pa) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= pa.sc.n_keys) return;
  float m = 0.f;
  for (int rb = 0; rb < pa.n_rowblocks; ++rb) m = fmaxf(m, pa.rowblock_max[(int64_t)rb * pa.sc.n_keys + j]);
  pa.token_scores[j] = m * pa.inv_maps;
}

int specpc_rows_per_block(int, int) { return PcGeom<bf16_t, 64>::kRowsPerBlock; }

int specpc_keys_per_block(int dtype, int head_dim) {
  if (dtype == 0) return head_dim == 64 ? PcGeom<float, 64>::kKeysPerBlock : PcGeom<float, 128>::kKeysPerBlock;
  return head_dim == 64 ? PcGeom<bf16_t, 64>::kKeysPerBlock : PcGeom<bf16_t, 128>::kKeysPerBlock;
}

template <typename T, int D>
static hipError_t launch_pc2(const SpecPCArgs& args, hipStream_t s) {
  using Gm = PcGeom<T, D>;
  SpecPCArgs a = args;
  a.maps_per_stage = pc_maps_per_stage<T, D>(a.sc.group);
  const size_t lds = (size_t)2 * a.maps_per_stage * Gm::kMapLds;
  const int n_kblocks = (a.sc.n_keys + Gm::kKeysPerBlock - 1) / Gm::kKeysPerBlock;
  // Key blocks whose every key precedes the first window position need no causal mask.
  int64_t n_plain = (a.sc.pos_base + 1) / Gm::kKeysPerBlock;
  if (n_plain > n_kblocks) n_plain = n_kblocks;
  if ((int64_t)n_kblocks * Gm::kKeysPerBlock > a.sc.n_keys && n_plain == n_kblocks) n_plain = n_kblocks - 1;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(specpc_pass2_kernel<T, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  specpc_pass2_kernel<T, D><<<dim3((unsigned)(n_kblocks * a.n_rowblocks)), dim3(Gm::kThreads), lds, s>>>(
      a, (int)n_plain);
  return hipGetLastError();
}

hipError_t launch_specpc_pass2(int dtype, int head_dim, const SpecPCArgs& a, hipStream_t s) {
  if (dtype == 0 && head_dim == 64) return launch_pc2<float, 64>(a, s);
  if (dtype == 0) return launch_pc2<float, 128>(a, s);
  if (head_dim == 64) return launch_pc2<bf16_t, 64>(a, s);
  return launch_pc2<bf16_t, 128>(a, s);
}

hipError_t launch_specpc_reduce(const SpecPCArgs& a, hipStream_t s) {
  specpc_reduce_kernel<<<dim3((unsigned)((a.sc.n_keys + 255) / 256)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace skv
