// Host-side check of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_capi_sanitize.py with the
// sanitizers on the host code only).  It calls every entry point with
// arguments that validation must reject, plus the pure host queries
// (workspace sizes, kept counts, profiling state) over a grid of shapes that
// includes the largest sizes the checks admit.  Pointers are fake and are
// never dereferenced: no call here may pass validation, so nothing is ever
// launched.  Exit status 0 means every status matched; any sanitizer report
// aborts the run.
#include "../include/speckv.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

static int g_fail = 0;

#define EXPECT(call, want)                                                                          \
  do {                                                                                              \
    const int got_ = (int)(call);                                                                   \
    if (got_ != (int)(want)) {                                                                      \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
      ++g_fail;                                                                                     \
    }                                                                                               \
  } while (0)

static void* P(uint64_t a) { return reinterpret_cast<void*>(a); }

static skv_shape shape(int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int64_t n_in, int32_t win, int32_t look,
                       int32_t dtype = SKV_BF16, int64_t stride = 0) {
  skv_shape s{};
  s.n_layers = L;
  s.n_q_heads = Hq;
  s.n_kv_heads = Hkv;
  s.head_dim = D;
  s.n_in = n_in;
  s.kv_head_stride = stride;
  s.n_window = win;
  s.n_lookahead = look;
  s.scale = 0.f;
  s.dtype = dtype;
  s.aggregation = SKV_AGG_SUM;
  s.per_query_head = 0;
  return s;
}

// Size queries over many shapes: every one must either succeed or return a
// shape/parameter error, never trip a sanitizer.
static void query_grid() {
  const int32_t Ls[] = {1, 2, 24, 64, 4096, 1 << 16};
  const int32_t heads[][2] = {{1, 1}, {4, 1}, {14, 2}, {40, 8}, {64, 1}, {1 << 14, 1 << 14}};
  const int32_t dims[] = {64, 128, 96};  // 96 is rejected
  const int64_t n_ins[] = {1, 2, 7, 2048, 65536, 131072, (int64_t)1 << 24, (int64_t)INT32_MAX - 1024,
                           (int64_t)INT32_MAX};
  const int32_t wins[] = {0, 32, 512};
  const int32_t looks[] = {0, 128, 1 << 20};
  const int32_t cmaxes[] = {0, 256, INT32_MAX};
  size_t n_queries = 0;
  for (int32_t L : Ls)
    for (auto& h : heads)
      for (int32_t D : dims)
        for (int64_t n_in : n_ins)
          for (int32_t w : wins)
            for (int32_t la : looks)
              for (int dt = 0; dt < 2; ++dt)
                for (int pq = 0; pq < 2; ++pq) {
                  skv_shape s = shape(L, h[0], h[1], D, n_in, w, la, dt);
                  s.per_query_head = pq;
                  s.aggregation = pq;
                  for (int32_t c : cmaxes) {
                    size_t ws = 0;
                    int64_t keep = 0;
                    const skv_status a = speckv_workspace_bytes(&s, c, &ws);
                    const skv_status b = speckv_n_keep(&s, c, &keep);
                    if (a != SKV_OK && a != SKV_ERR_SHAPE && a != SKV_ERR_PARAM) {
                      std::fprintf(stderr, "workspace query: unexpected status %d\n", (int)a);
                      ++g_fail;
                    }
                    if (b == SKV_OK && (keep < 0 || keep > n_in)) {
                      std::fprintf(stderr, "n_keep %lld out of range\n", (long long)keep);
                      ++g_fail;
                    }
                    ++n_queries;
                  }
                  size_t dws = 0;
                  (void)speckv_decode_workspace_bytes(&s, n_in, &dws);
                  (void)speckv_decode_workspace_bytes(&s, 1, &dws);
                }
  std::printf("size queries: %zu\n", n_queries);
}

static void shape_checks() {
  size_t ws = 0;
  int64_t keep = 0;
  EXPECT(speckv_workspace_bytes(nullptr, 1, &ws), SKV_ERR_NULL);
  skv_shape s = shape(2, 8, 2, 128, 1000, 16, 8);
  EXPECT(speckv_workspace_bytes(&s, 64, nullptr), SKV_ERR_NULL);
  EXPECT(speckv_workspace_bytes(&s, -1, &ws), SKV_ERR_PARAM);
  EXPECT(speckv_n_keep(&s, 64, &keep), SKV_OK);
  EXPECT(keep, 80);
  skv_shape bad = s;
  bad.dtype = 7;
  EXPECT(speckv_workspace_bytes(&bad, 64, &ws), SKV_ERR_DTYPE);
  bad = s;
  bad.head_dim = 96;
  EXPECT(speckv_workspace_bytes(&bad, 64, &ws), SKV_ERR_SHAPE);
  bad = s;
  bad.kv_head_stride = INT64_MAX;  // head slabs beyond any address space
  EXPECT(speckv_workspace_bytes(&bad, 64, &ws), SKV_ERR_SHAPE);
  bad = s;
  bad.kv_head_stride = -128;
  EXPECT(speckv_workspace_bytes(&bad, 64, &ws), SKV_ERR_SHAPE);
  bad = s;
  bad.n_in = INT64_MAX;
  EXPECT(speckv_workspace_bytes(&bad, 64, &ws), SKV_ERR_SHAPE);
  bad = s;
  bad.scale = -1.f;
  EXPECT(speckv_workspace_bytes(&bad, 64, &ws), SKV_ERR_PARAM);
  bad = shape(1 << 30, 4, 1, 128, 1000, 16, 8);  // layers x heads beyond int32 indexing
  EXPECT(speckv_workspace_bytes(&bad, 64, &ws), SKV_ERR_SHAPE);
  bad = shape(1 << 20, 1 << 14, 1 << 14, 128, (int64_t)INT32_MAX - 1024, 0, 1);  // 2^59 bytes of K
  EXPECT(speckv_workspace_bytes(&bad, 64, &ws), SKV_ERR_SHAPE);
}

static void entry_point_rejections() {
  skv_shape s = shape(2, 8, 2, 128, 1000, 16, 8);
  size_t ws = 0;
  EXPECT(speckv_workspace_bytes(&s, 64, &ws), SKV_OK);
  const uint64_t q = 1ull << 30, k = 2ull << 30, sc = 3ull << 30, w = 4ull << 30, kept = 5ull << 30,
                 pooled = 6ull << 30, ko = 7ull << 30, vo = 8ull << 30, v = 9ull << 30;
  // scores
  EXPECT(speckv_scores(&s, nullptr, P(k), (float*)P(sc), P(w), ws, nullptr), SKV_ERR_NULL);
  EXPECT(speckv_scores(&s, P(q + 2), P(k), (float*)P(sc), P(w), ws, nullptr), SKV_ERR_ALIGN);
  EXPECT(speckv_scores(&s, P(q), P(k), (float*)P(sc), P(w), 16, nullptr), SKV_ERR_WORKSPACE);
  EXPECT(speckv_scores(&s, P(q), P(k), (float*)P(q + 4096), P(w), ws, nullptr), SKV_ERR_ALIAS);
  EXPECT(speckv_scores(&s, P(q), P(k), (float*)P(sc), P(k + 64), ws, nullptr), SKV_ERR_ALIAS);
  EXPECT(speckv_scores_rows(&s, P(q), P(k), nullptr, 1000, (float*)P(sc), P(w), ws, nullptr), SKV_ERR_NULL);
  EXPECT(speckv_scores_rows(&s, P(q), P(k), (const int32_t*)P(kept), 1001, (float*)P(sc), P(w), ws, nullptr),
         SKV_ERR_SHAPE);
  EXPECT(speckv_scores_rows(&s, P(q), P(k), (const int32_t*)P(sc + 64), 1000, (float*)P(sc), P(w), ws, nullptr),
         SKV_ERR_ALIAS);
  // select
  EXPECT(speckv_select(&s, (float*)P(sc), -1, SKV_POOL_MAX, 7, (int32_t*)P(kept), nullptr, P(w), ws, nullptr),
         SKV_ERR_PARAM);
  EXPECT(speckv_select(&s, (float*)P(sc), 64, SKV_POOL_MAX, 4, (int32_t*)P(kept), nullptr, P(w), ws, nullptr),
         SKV_ERR_PARAM);
  EXPECT(speckv_select(&s, (float*)P(sc), 64, 9, 7, (int32_t*)P(kept), nullptr, P(w), ws, nullptr), SKV_ERR_PARAM);
  EXPECT(speckv_select(&s, (float*)P(sc), 64, SKV_POOL_MAX, 7, (int32_t*)P(kept), (float*)P(sc + 4), P(w), ws,
                       nullptr),
         SKV_ERR_ALIAS);
  EXPECT(speckv_select(&s, (float*)P(sc), 64, SKV_POOL_MAX, 7, (int32_t*)P(kept), (float*)P(kept + 16), P(w), ws,
                       nullptr),
         SKV_ERR_ALIAS);
  EXPECT(speckv_select(&s, (float*)P(sc), 64, SKV_POOL_AVG, 7, (int32_t*)P(kept), nullptr, P(sc + 64), ws, nullptr),
         SKV_ERR_ALIAS);
  EXPECT(speckv_select(&s, (float*)P(sc), 64, SKV_POOL_AVG, 7, (int32_t*)P(kept), nullptr, nullptr, 0, nullptr),
         SKV_ERR_WORKSPACE);
  EXPECT(speckv_select(&s, nullptr, 64, SKV_POOL_MAX, 7, (int32_t*)P(kept), nullptr, P(w), ws, nullptr),
         SKV_ERR_NULL);
  (void)pooled;
  // compact
  EXPECT(speckv_compact(&s, P(k), P(v), (int32_t*)P(kept), 0, P(ko), P(vo), P(w), ws, nullptr), SKV_ERR_PARAM);
  EXPECT(speckv_compact(&s, P(k), P(v), (int32_t*)P(kept), 80, P(k), P(vo), P(w), ws, nullptr), SKV_ERR_ALIAS);
  EXPECT(speckv_compact(&s, P(k), P(k), (int32_t*)P(kept), 80, P(ko), P(vo), P(w), ws, nullptr), SKV_ERR_ALIAS);
  EXPECT(speckv_compact(&s, P(k), P(v), (int32_t*)P(kept), 80, P(k), P(v), nullptr, 0, nullptr), SKV_ERR_WORKSPACE);
  EXPECT(speckv_compact(&s, P(k), P(v), (int32_t*)P(w + 256), 80, P(k), P(v), P(w), ws, nullptr), SKV_ERR_ALIAS);
  EXPECT(speckv_compact(&s, P(k + 8), P(v), (int32_t*)P(kept), 80, P(ko), P(vo), P(w), ws, nullptr), SKV_ERR_ALIGN);
  EXPECT(speckv_compact_rows(&s, P(k), P(v), (const int32_t*)P(pooled), 1000, (int32_t*)P(kept), 80, P(k), P(v),
                             nullptr),
         SKV_ERR_ALIAS);
  EXPECT(specpc_gather_tokens(&s, P(k), P(v), (const int32_t*)P(kept), 0, P(ko), P(vo), nullptr), SKV_ERR_PARAM);
  EXPECT(specpc_gather_tokens(&s, P(k), P(v), (const int32_t*)P(kept), 10, P(k), P(v), nullptr), SKV_ERR_ALIAS);
  // SpecPC: the size the query returns is accepted for every l_skip (the
  // unaligned workspace then stops the call at the alignment check)
  skv_shape pc = shape(3, 2, 2, 64, 65536, 1024, 1);
  size_t pcws = 0;
  EXPECT(speckv_workspace_bytes(&pc, 0, &pcws), SKV_OK);
  for (int ls = 0; ls < 3; ++ls)
    EXPECT(specpc_token_scores(&pc, ls, P(q), P(k), nullptr, (float*)P(sc), P(w + 4), pcws, nullptr), SKV_ERR_ALIGN);
  EXPECT(specpc_token_scores(&pc, 3, P(q), P(k), nullptr, (float*)P(sc), P(w), pcws, nullptr), SKV_ERR_PARAM);
  EXPECT(specpc_token_scores(&pc, -1, P(q), P(k), nullptr, (float*)P(sc), P(w), pcws, nullptr), SKV_ERR_PARAM);
  // decode
  skv_shape dec = shape(2, 8, 2, 128, 4096, 16, 8);
  size_t dws = 0;
  EXPECT(speckv_decode_workspace_bytes(&dec, 4096, &dws), SKV_OK);
  if (dws == 0) {  // a 4096-row cache is split over several blocks per head: it needs a workspace
    std::fprintf(stderr, "decode workspace of a 4096-row cache is 0\n");
    ++g_fail;
  } else {
    EXPECT(speckv_decode_attention(&dec, 4096, P(q), P(k), P(v), (float*)P(sc), nullptr, 0, nullptr),
           SKV_ERR_WORKSPACE);
  }
  EXPECT(speckv_decode_attention(&dec, 0, P(q), P(k), P(v), (float*)P(sc), P(w), dws, nullptr), SKV_ERR_PARAM);
  EXPECT(speckv_decode_attention(&dec, 4096, P(q), P(k), P(v), (float*)P(k + 64), P(w), dws, nullptr),
         SKV_ERR_ALIAS);
}

static void profiling_state() {
  EXPECT(speckv_profile_enable(1), SKV_OK);
  EXPECT(speckv_profile_count(), 0);
  const char* name = nullptr;
  int64_t n = 0;
  double ms = 0.0;
  EXPECT(speckv_profile_read(0, &name, &n, &ms), SKV_ERR_PARAM);
  skv_shape s = shape(2, 8, 2, 128, 1000, 16, 8);
  EXPECT(speckv_scores(&s, nullptr, P(1), nullptr, nullptr, 0, nullptr), SKV_ERR_NULL);  // records nothing
  EXPECT(speckv_profile_count(), 0);
  EXPECT(speckv_profile_enable(0), SKV_OK);
  for (int st = -1; st < 12; ++st)
    if (!speckv_status_string((skv_status)st)) ++g_fail;
}

int main() {
  shape_checks();
  entry_point_rejections();
  profiling_state();
  query_grid();
  std::printf("%s: %d mismatches\n", g_fail ? "FAIL" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
