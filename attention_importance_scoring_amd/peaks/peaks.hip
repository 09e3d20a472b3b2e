// Measured ceilings of the units the scoring path leans on, beside the
// datasheet figures the rooflines use: HBM read and copy bandwidth, dense
// bf16 MFMA throughput (v_mfma_f32_32x32x16_bf16) and v_exp_f32 throughput,
// each with the core clock it ran at.
//
// The clock comes from the kernel itself: thread 0 of block 0 reads the
// shader clock counter (clock64) and the constant-rate wall clock
// (wall_clock64) at its start and end; with one block per CU every block
// runs for about the whole launch.  Timing is by HIP events over one launch
// after a warm-up launch, best of three.  Prints one line per test and a
// JSON line.  A stand-alone program, not part of libspeckv.so.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#define CK(x)                                                                              \
  do {                                                                                     \
    hipError_t e_ = (x);                                                                   \
    if (e_ != hipSuccess) {                                                                \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);  \
      std::exit(1);                                                                        \
    }                                                                                      \
  } while (0)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// clk[0..1]: shader clock at start and end, clk[2..3]: wall clock.
__device__ __forceinline__ void clock_mark(unsigned long long* clk, int end) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[end] = clock64();
    clk[2 + end] = wall_clock64();
  }
}

__device__ __forceinline__ unsigned fold(uint4 v) { return (v.x ^ v.y) ^ (v.z ^ v.w); }

// Each block reads its own contiguous chunk of the n16 16-byte words, eight
// loads in flight per thread.
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, size_t n16, unsigned* sink,
                                                   unsigned long long* clk) {
  clock_mark(clk, 0);
  const size_t per_block = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per_block;
  const size_t end = beg + per_block < n16 ? beg + per_block : n16;
  unsigned acc = 0u;
  size_t i = beg + threadIdx.x;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[i + k * 256];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += fold(v[k]);
  }
  for (; i < end; i += 256) acc += fold(p[i]);
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; the data never makes it true
  clock_mark(clk, 1);
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n16,
                                                   unsigned long long* clk) {
  clock_mark(clk, 0);
  const size_t per_block = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per_block;
  const size_t end = beg + per_block < n16 ? beg + per_block : n16;
  size_t i = beg + threadIdx.x;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = src[i + k * 256];
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[i + k * 256] = v[k];
  }
  for (; i < end; i += 256) dst[i] = src[i];
  clock_mark(clk, 1);
}

// Four independent accumulation chains of 32x32x16 bf16 MFMAs per wave.
__global__ __launch_bounds__(1024) void mfma_kernel(int iters, float seed, float* sink, unsigned long long* clk) {
  clock_mark(clk, 0);
  const int lane = threadIdx.x % 64;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(lane + i));
    b[i] = (__bf16)(seed * (float)(lane - i));
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) t += acc[j][i];
  if (t == 1234.5f) sink[0] = t;
  clock_mark(clk, 1);
}

// Eight independent chains x <- 2^(-x) per thread (the negation is an input
// modifier of v_exp_f32, so the loop is exponentials only).
__global__ __launch_bounds__(1024) void exp_kernel(int iters, float seed, float* sink, unsigned long long* clk) {
  clock_mark(clk, 0);
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = seed * (float)(threadIdx.x % 7 + j);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) t += x[j];
  if (t == 1234.5f) sink[0] = t;
  clock_mark(clk, 1);
}

struct Result {
  float ms;
  double ghz;
};

static double g_wall_khz = 0.0;

template <typename Launch>
static Result time_best(Launch launch, unsigned long long* d_clk) {
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  launch();
  CK(hipDeviceSynchronize());
  Result best{1e30f, 0.0};
  for (int r = 0; r < 3; ++r) {
    CK(hipEventRecord(e0));
    launch();
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float ms = 0.f;
    CK(hipEventElapsedTime(&ms, e0, e1));
    unsigned long long clk[4];
    CK(hipMemcpy(clk, d_clk, sizeof(clk), hipMemcpyDeviceToHost));
    const double wall_s = (double)(clk[3] - clk[2]) / (g_wall_khz * 1e3);
    const double ghz = wall_s > 0 ? (double)(clk[1] - clk[0]) / wall_s * 1e-9 : 0.0;
    if (ms < best.ms) best = {ms, ghz};
  }
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  return best;
}

int main(int argc, char** argv) {
  // --small: a quick run with small sizes (checks that every test runs).
  const bool small = argc > 1 && std::strcmp(argv[1], "--small") == 0;
  int dev = 0, cus = 0, wall_khz = 0;
  CK(hipGetDevice(&dev));
  CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  CK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev));
  g_wall_khz = wall_khz;
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, dev));

  const size_t bytes = small ? ((size_t)64 << 20) : ((size_t)4 << 30);
  const size_t n16 = bytes / 16;
  uint4 *src = nullptr, *dst = nullptr;
  unsigned* usink = nullptr;
  float* fsink = nullptr;
  unsigned long long* d_clk = nullptr;
  CK(hipMalloc(&src, bytes));
  CK(hipMalloc(&dst, bytes));
  CK(hipMalloc(&usink, 64));
  CK(hipMalloc(&fsink, 64));
  CK(hipMalloc(&d_clk, 4 * sizeof(unsigned long long)));
  CK(hipMemset(src, 1, bytes));
  CK(hipMemset(dst, 0, bytes));

  const int mem_blocks = cus * 8;  // one round: 8 blocks of 4 waves per CU
  const Result rd = time_best([&] { read_kernel<<<mem_blocks, 256>>>(src, n16, usink, d_clk); }, d_clk);
  const Result cp = time_best([&] { copy_kernel<<<mem_blocks, 256>>>(src, dst, n16, d_clk); }, d_clk);
  const double rd_gbs = (double)bytes / (rd.ms * 1e-3) * 1e-9;
  const double cp_gbs = 2.0 * (double)bytes / (cp.ms * 1e-3) * 1e-9;

  // One block per CU; 8 or 16 waves per block (2 or 4 per SIMD).
  const int mfma_iters = small ? 200 : 200000;
  double mfma_tf[2];
  Result mfma_r[2];
  for (int k = 0; k < 2; ++k) {
    const int threads = k == 0 ? 512 : 1024;
    mfma_r[k] = time_best([&] { mfma_kernel<<<cus, threads>>>(mfma_iters, 1e-3f, fsink, d_clk); }, d_clk);
    const double flops = (double)cus * (threads / 64) * mfma_iters * 4 * (2.0 * 32 * 32 * 16);
    mfma_tf[k] = flops / (mfma_r[k].ms * 1e-3) * 1e-12;
  }
  const int exp_iters = small ? 200 : 200000;
  double exp_t[2];
  Result exp_r[2];
  for (int k = 0; k < 2; ++k) {
    const int threads = k == 0 ? 512 : 1024;
    exp_r[k] = time_best([&] { exp_kernel<<<cus, threads>>>(exp_iters, 0.1f, fsink, d_clk); }, d_clk);
    exp_t[k] = (double)cus * threads * exp_iters * 8 / (exp_r[k].ms * 1e-3) * 1e-12;
  }
  CK(hipDeviceSynchronize());

  std::printf("device %s, %d CUs, wall clock %d kHz\n", prop.gcnArchName, cus, wall_khz);
  std::printf("hbm read   %6.2f GiB  %8.3f ms  %7.0f GB/s  (datasheet 8000 GB/s)  clock %.2f GHz\n",
              bytes / 1073741824.0, rd.ms, rd_gbs, rd.ghz);
  std::printf("hbm copy   %6.2f GiB  %8.3f ms  %7.0f GB/s  (read + write)          clock %.2f GHz\n",
              bytes / 1073741824.0, cp.ms, cp_gbs, cp.ghz);
  for (int k = 0; k < 2; ++k)
    std::printf("mfma bf16  %d waves/SIMD %8.3f ms  %7.1f TFLOP/s (datasheet 2500, dense)  clock %.2f GHz\n",
                k == 0 ? 2 : 4, mfma_r[k].ms, mfma_tf[k], mfma_r[k].ghz);
  for (int k = 0; k < 2; ++k)
    std::printf("v_exp_f32  %d waves/SIMD %8.3f ms  %7.2f T exp/s                      clock %.2f GHz\n",
                k == 0 ? 2 : 4, exp_r[k].ms, exp_t[k], exp_r[k].ghz);
  std::printf("{\"hbm_read_GBps\": %.1f, \"hbm_copy_GBps\": %.1f, \"mfma_bf16_TFLOPs\": [%.1f, %.1f], "
              "\"exp_T_per_s\": [%.3f, %.3f], \"clock_GHz\": {\"read\": %.3f, \"copy\": %.3f, \"mfma\": [%.3f, %.3f], "
              "\"exp\": [%.3f, %.3f]}, \"small\": %s}\n",
              rd_gbs, cp_gbs, mfma_tf[0], mfma_tf[1], exp_t[0], exp_t[1], rd.ghz, cp.ghz, mfma_r[0].ghz,
              mfma_r[1].ghz, exp_r[0].ghz, exp_r[1].ghz, small ? "true" : "false");
  CK(hipFree(src));
  CK(hipFree(dst));
  CK(hipFree(usink));
  CK(hipFree(fsink));
  CK(hipFree(d_clk));
  return 0;
}
