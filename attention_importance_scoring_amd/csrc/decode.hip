// Decode attention over a (compacted) KV cache: each query head's new query
// attends over the first n_rows cached rows of its KV head (paper notes
// "Draft-based Approximate Inference for LLMs", section "Background":
// attention and KV cache cost grow with the context; section "Key designs",
// SpecKV: generation runs over the kept pairs).
//
// The work is HBM-bound: every cached K and V byte is read once and feeds
// only G (query heads per cache head) dot products.  The G x n_rows x D
// contractions still run on MFMA (v_mfma_f32_16x16x32_bf16), which leaves
// the vector units free for the softmax:
//
//   S^T = K Q^T : A = 16 keys x 32 head-dim elements, B = Q^T (queries on N,
//                 padded to 16).  Lane l gets query l % 16 and keys
//                 4 (l / 16) + i, i < 4, of the 16-key half tile.
//   O   = P V   : A = P (queries on M, keys on K).  The contraction order is
//                 free as long as A and B agree, so a lane's eight S values
//                 of a 32-key tile (four per half) ARE its A operand: element
//                 e < 4 is key 4 (l / 16) + e, element e >= 4 is key
//                 16 + 4 (l / 16) + e - 4.  B = V read with the same key
//                 order, one 16-column slice of the head dim per MFMA, from
//                 a padded LDS copy of the tile (the transposed access).
//
// P enters the MFMA as two bf16 terms, p = hi + lo (hi = bf16(p),
// lo = bf16(p - hi)), so the product carries about 16 bits of P; the second
// MFMA is free in an HBM-bound kernel.  fp32 caches use
// v_mfma_f32_16x16x4f32 with the same lane layout (one contraction element
// per lane and step), exact fp32 P and two tiles per wave per sub-chunk.
//
// A block walks n_sub sub-chunks of 512 keys (256 for fp32).  In each, a
// wave first computes all scores of its four tiles (kept in registers) and
// their exact maximum, then the probabilities and P V; its running (max,
// sum, acc) is rescaled once per sub-chunk, only when the maximum grows.
// The four waves merge in LDS; when a cache is split over several blocks
// they write partials that decode_combine_kernel merges.  Longer blocks
// (n_sub > 1) amortize the per-block start-up and merge: the host picks
// n_sub so that a launch has about SKV_DEC_TARGET_BLOCKS blocks.
#include "common.hpp"
#include "kernels.hpp"

namespace skv {

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kDecMaxGroup = 16;  // queries per cache head (MFMA N)

template <typename T, int D>
struct DecGeom {
  static constexpr bool kF32 = Elem<T>::kBytes == 4;
  static constexpr int kTiles = kF32 ? 2 : 4;                // 32-key tiles per wave per sub-chunk
  static constexpr int kSubKeys = kDecWaves * kTiles * 32;   // keys per sub-chunk
  static constexpr int kRowBytes = D * Elem<T>::kBytes;
  // Q and K operand: in vector s, lane (row r, group g) holds bytes
  // [64 s + 16 g, 64 s + 16 g + 16) of its row, so the four lanes of a row
  // read 64 contiguous bytes per vector.
  static constexpr int kQV = kRowBytes / 64;
  static constexpr int kDGroups = D / 16;                    // PV MFMAs (16 head-dim columns each) per term
  // LDS V row pitch: the four key groups of one transposed read hit distinct banks
  static constexpr int kPitch = kRowBytes + (kF32 ? 16 : 8);
  static constexpr int kVecPerRow = kRowBytes / 16;
  static constexpr int kVLoads = 32 * kVecPerRow / kWave;    // 16-byte V loads per lane per tile
  static constexpr int kWaveLds = 32 * kPitch;               // V tile bytes per wave
  static constexpr int kMergeLds = kDecWaves * (kDecMaxGroup * D + 2 * kDecMaxGroup) * 4;
  static constexpr int kLds = kDecWaves * kWaveLds > kMergeLds ? kDecWaves * kWaveLds : kMergeLds;
};

__device__ __forceinline__ f32x4_t mfma16(bf16x8 a, bf16x8 b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// acc += A B over one 16-byte vector of each operand: one bf16 MFMA (8
// contraction elements per lane), or four fp32 MFMAs (one element each).
template <typename T>
__device__ __forceinline__ f32x4_t mfma_vec(u32x4 a, u32x4 b, f32x4_t acc) {
  if constexpr (Elem<T>::kBytes == 2) {
    return mfma16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
    return acc;
  }
}

__device__ __forceinline__ float xor16(float v) { return __shfl_xor(v, 16); }

// Key (within a 32-key tile) of P/V contraction element e for key group g = lane / 16.
__device__ __forceinline__ int tile_key(int g, int e) { return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4); }

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads, 2) void decode_attention_kernel(DecodeArgs a) {
  using Geo = DecGeom<T, D>;
  constexpr int TW = Geo::kTiles;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t unit = blockIdx.x / a.n_chunks;
  const int chunk = blockIdx.x % a.n_chunks;
  const int G = a.group;
  const int64_t layer = unit / a.heads_per_layer, head = unit % a.heads_per_layer;
  const int64_t q_row0 = layer * a.q_heads_per_layer + head * G;  // first query (and output) row of the unit
  const char* kp = static_cast<const char*>(a.k) + unit * a.head_stride * Elem<T>::kBytes;
  const char* vp = static_cast<const char*>(a.v) + unit * a.head_stride * Elem<T>::kBytes;

  // Q^T operand (queries on N); padded queries are zero.
  u32x4 qf[Geo::kQV];
  {
    const char* qp = static_cast<const char*>(a.q) + (q_row0 + (r < G ? r : 0)) * Geo::kRowBytes + 16 * g;
#pragma unroll
    for (int s = 0; s < Geo::kQV; ++s) {
      qf[s] = ldg16(qp + 64 * s);
      if (r >= G) qf[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int64_t last = a.n_rows - 1;
  char* vl = lds + wave * Geo::kWaveLds;
  f32x4_t acc[Geo::kDGroups];
#pragma unroll
  for (int i = 0; i < Geo::kDGroups; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;           // this lane's part of the sum for query r
  float m = -INFINITY;     // running maximum for query r (log2 units), the same in the four lanes of r

  for (int sub = 0; sub < a.n_sub; ++sub) {
    const int64_t sub_base = ((int64_t)chunk * a.n_sub + sub) * Geo::kSubKeys;
    if (sub_base > last) break;  // block-uniform

    // ---- phase 1: scores of this wave's tiles (tile t = wave + 4 j of the sub-chunk) ----
    // Every load is issued before the first MFMA; rows past the cache end are
    // clamped to its last row (in bounds) and masked below.
    u32x4 kf[TW][2][Geo::kQV];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int64_t kbase = sub_base + 32 * (wave + kDecWaves * j);
      const int64_t ra = kbase + r < last ? kbase + r : last;
      const int64_t rb = kbase + 16 + r < last ? kbase + 16 + r : last;
#pragma unroll
      for (int s = 0; s < Geo::kQV; ++s) {
        kf[j][0][s] = ldg16(kp + ra * Geo::kRowBytes + 16 * g + 64 * s);
        kf[j][1][s] = ldg16(kp + rb * Geo::kRowBytes + 16 * g + 64 * s);
      }
    }
    float sc[TW][8];
    float m_sub = -INFINITY;
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int64_t kbase = sub_base + 32 * (wave + kDecWaves * j);
      f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < Geo::kQV; ++s) {
        sa = mfma_vec<T>(kf[j][0][s], qf[s], sa);
        sb = mfma_vec<T>(kf[j][1][s], qf[s], sb);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t key = kbase + tile_key(g, e);
        const float t = (e < 4 ? sa[e] : sb[e - 4]) * a.c;
        sc[j][e] = key <= last ? t : -INFINITY;
        m_sub = fmaxf(m_sub, sc[j][e]);
      }
    }
    // the four lanes of a query (same r) hold disjoint keys
    m_sub = fmaxf(m_sub, xor16(m_sub));
    m_sub = fmaxf(m_sub, shfl_xor32(m_sub));
    if (m_sub == -INFINITY) continue;  // wave-uniform: no key of this wave in the sub-chunk

    // ---- rescale the running sums to the new maximum ----
    const float m_new = fmaxf(m, m_sub);
    const float f = fast_exp2(m - m_new);  // 0 on the first visit (m = -inf)
    l *= f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float fi = __shfl(f, 4 * g + i);  // acc register i holds query 4 g + i
#pragma unroll
      for (int dg = 0; dg < Geo::kDGroups; ++dg) acc[dg][i] *= fi;
    }
    m = m_new;

    // ---- phase 2: probabilities and P V ----
    // All V tiles of the wave are requested at once (16-byte vectors,
    // consecutive lanes along a row: fully used lines), then staged through
    // LDS one tile at a time for the transposed reads.
    u32x4 vv[TW][Geo::kVLoads];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int64_t kbase = sub_base + 32 * (wave + kDecWaves * j);
#pragma unroll
      for (int t = 0; t < Geo::kVLoads; ++t) {
        const int c = lane + kWave * t;
        const int row = c / Geo::kVecPerRow, col = c % Geo::kVecPerRow;
        const int64_t src = kbase + row < last ? kbase + row : last;
        vv[j][t] = ldg16(vp + src * Geo::kRowBytes + col * 16);
      }
    }
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int64_t kbase = sub_base + 32 * (wave + kDecWaves * j);
      if (kbase > last) continue;  // wave-uniform: a tile past the end holds no key
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(sc[j][e] - m);  // 0 for masked keys
        l += p[e];
      }
#pragma unroll
      for (int t = 0; t < Geo::kVLoads; ++t) {
        const int c = lane + kWave * t;
        const int row = c / Geo::kVecPerRow, col = c % Geo::kVecPerRow;
        uint2* dst = reinterpret_cast<uint2*>(vl + row * Geo::kPitch + col * 16);
        dst[0] = uint2{vv[j][t][0], vv[j][t][1]};
        dst[1] = uint2{vv[j][t][2], vv[j][t][3]};
      }
      // LDS operations of one wave complete in issue order: the reads below see the writes above
      __builtin_amdgcn_wave_barrier();
      if constexpr (Geo::kF32) {
        const float* vt = reinterpret_cast<const float*>(vl);
#pragma unroll
        for (int dg = 0; dg < Geo::kDGroups; ++dg)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[dg] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                p[e], vt[tile_key(g, e) * (Geo::kPitch / 4) + 16 * dg + r], acc[dg], 0, 0, 0);
      } else {
        bf16x8 phi, plo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 h = (__bf16)p[e];
          phi[e] = h;
          plo[e] = (__bf16)(p[e] - (float)h);
        }
        const __bf16* vt = reinterpret_cast<const __bf16*>(vl);
#pragma unroll
        for (int dg = 0; dg < Geo::kDGroups; ++dg) {
          bf16x8 vb;
#pragma unroll
          for (int e = 0; e < 8; ++e) vb[e] = vt[tile_key(g, e) * (Geo::kPitch / 2) + 16 * dg + r];
          acc[dg] = mfma16(phi, vb, acc[dg]);
          acc[dg] = mfma16(plo, vb, acc[dg]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  l += xor16(l);
  l += shfl_xor32(l);
  const bool any = m != -INFINITY;  // the wave saw at least one key

  // ---- merge the four waves in LDS ----
  __syncthreads();  // every wave is done with its V tiles
  float* macc = reinterpret_cast<float*>(lds);                         // [wave][16][D]
  float* mml = macc + kDecWaves * kDecMaxGroup * D;                    // [wave][16] max, then [wave][16] sum
  if (lane < 16) {
    mml[wave * kDecMaxGroup + lane] = any ? m : -INFINITY;
    mml[kDecWaves * kDecMaxGroup + wave * kDecMaxGroup + lane] = l;
  }
#pragma unroll
  for (int dg = 0; dg < Geo::kDGroups; ++dg)
#pragma unroll
    for (int i = 0; i < 4; ++i) macc[(wave * kDecMaxGroup + 4 * g + i) * D + 16 * dg + r] = acc[dg][i];
  __syncthreads();
  for (int o = threadIdx.x; o < G * D; o += kDecThreads) {
    const int q = o / D, d = o % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, mml[w * kDecMaxGroup + q]);
    float num = 0.f, den = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = mml[w * kDecMaxGroup + q];
        if (mw == -INFINITY) continue;
        const float f = fast_exp2(mw - mx);
        num += f * macc[(w * kDecMaxGroup + q) * D + d];
        den += f * mml[kDecWaves * kDecMaxGroup + w * kDecMaxGroup + q];
      }
    }
    if (a.n_chunks == 1) {
      a.out[(q_row0 + q) * D + d] = num / den;
    } else {
      const int64_t pc = unit * a.n_chunks + chunk;
      a.part_acc[(pc * kDecMaxGroup + q) * D + d] = num;
      if (d == 0) a.part_ml[pc * kDecMaxGroup + q] = float2{mx, den};
    }
  }
}

// Merge of the chunk partials of one unit: out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int64_t unit = blockIdx.x;
  const int G = a.group;
  const int64_t layer = unit / a.heads_per_layer, head = unit % a.heads_per_layer;
  const int64_t q_row0 = layer * a.q_heads_per_layer + head * G;
  for (int o = threadIdx.x; o < G * D; o += 256) {
    const int q = o / D, d = o % D;
    const float2* ml = a.part_ml + unit * a.n_chunks * kDecMaxGroup + q;
    float mx = -INFINITY;
    for (int c = 0; c < a.n_chunks; ++c) mx = fmaxf(mx, ml[c * kDecMaxGroup].x);
    float num = 0.f, den = 0.f;
    for (int c = 0; c < a.n_chunks; ++c) {
      const float2 v = ml[c * kDecMaxGroup];
      if (v.x == -INFINITY) continue;
      const float f = fast_exp2(v.x - mx);
      num += f * a.part_acc[((unit * a.n_chunks + c) * kDecMaxGroup + q) * D + d];
      den += f * v.y;
    }
    a.out[(q_row0 + q) * D + d] = num / den;
  }
}

}  // namespace

#ifndef SKV_DEC_TARGET_BLOCKS
#define SKV_DEC_TARGET_BLOCKS 4096
#endif

void decode_plan(int dtype, int64_t n_units, int64_t n_rows, int32_t* n_sub, int32_t* n_chunks) {
  const int64_t sub_keys = dtype == 0 ? DecGeom<float, 64>::kSubKeys : DecGeom<bf16_t, 64>::kSubKeys;
  const int64_t subs = (n_rows + sub_keys - 1) / sub_keys;  // sub-chunks per unit
  int64_t ns = n_units * subs / SKV_DEC_TARGET_BLOCKS;
  ns = ns < 1 ? 1 : (ns > 64 ? 64 : ns);
  if (ns > subs) ns = subs;
  const int64_t chunks = (subs + ns - 1) / ns;
  *n_chunks = (int32_t)chunks;
  *n_sub = (int32_t)((subs + chunks - 1) / chunks);  // balanced: every block but the last walks n_sub
}
int decode_max_group() { return kDecMaxGroup; }

template <typename T, int D>
static hipError_t launch_dec(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_units * a.n_chunks)), block(kDecThreads);
  constexpr int lds = DecGeom<T, D>::kLds;  // fp32 at head_dim 128 needs more than the default 64 KB
  hipError_t e0 = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_attention_kernel<T, D>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e0 != hipSuccess) return e0;
  decode_attention_kernel<T, D><<<grid, block, lds, s>>>(a);
  if (a.n_chunks > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decode_combine_kernel<D><<<dim3((unsigned)a.n_units), dim3(256), 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_attention(int dtype, int head_dim, const DecodeArgs& a, hipStream_t s) {
  if (dtype == 0) return head_dim == 128 ? launch_dec<float, 128>(a, s) : launch_dec<float, 64>(a, s);
  return head_dim == 128 ? launch_dec<bf16_t, 128>(a, s) : launch_dec<bf16_t, 64>(a, s);
}

}  // namespace skv
