// C ABI of the scoring library: argument validation, workspace layout,
// launch sequencing on the caller's stream, status mapping and optional
// per-kernel event timing.  Every check runs on the host before anything is
// enqueued, and no HIP call is made on an invalid argument.
#include "../../include/speckv.h"
#include "kernels.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

using namespace skv;

namespace {

constexpr size_t kAlign = 256;
// Query rows per KV head (G x observation rows), kept well inside int32 indexing.
constexpr int64_t kMaxRows = 1 << 20;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Dims {
  int64_t L, Hq, Hkv, D, n_in, stride, n_window, n_lookahead, esize;
  float scale;
  int dtype;
  int agg;   // skv_agg
  bool pqh;  // per_query_head: SpecKV heads are the query heads
  int64_t heads() const { return pqh ? Hq : Hkv; }     // SpecKV heads H per layer
  int64_t group() const { return pqh ? 1 : Hq / Hkv; }  // query heads per SpecKV head
  int64_t repeat() const { return pqh ? Hq / Hkv : 1; } // SpecKV heads per KV head
};

skv_status check_shape(const skv_shape* s, Dims* d) {
  if (!s) return SKV_ERR_NULL;
  if (s->dtype != SKV_F32 && s->dtype != SKV_BF16) return SKV_ERR_DTYPE;
  if (s->n_layers < 1 || s->n_kv_heads < 1 || s->n_q_heads < 1 || s->n_q_heads % s->n_kv_heads != 0)
    return SKV_ERR_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return SKV_ERR_SHAPE;
  if (s->n_in < 1 || s->n_in > INT32_MAX - 1024) return SKV_ERR_SHAPE;
  if (s->n_window < 0 || s->n_lookahead < 0 || s->n_window > s->n_in) return SKV_ERR_SHAPE;
  if (!(s->scale >= 0.f) || std::isinf(s->scale)) return SKV_ERR_PARAM;
  if (s->aggregation != SKV_AGG_SUM && s->aggregation != SKV_AGG_MAX) return SKV_ERR_PARAM;
  if (s->per_query_head != 0 && s->per_query_head != 1) return SKV_ERR_PARAM;
  d->agg = s->aggregation;
  d->pqh = s->per_query_head != 0;
  d->L = s->n_layers;
  d->Hq = s->n_q_heads;
  d->Hkv = s->n_kv_heads;
  d->D = s->head_dim;
  d->n_in = s->n_in;
  d->esize = (s->dtype == SKV_F32) ? 4 : 2;
  // unit counts must stay inside int32 for the kernels
  if (d->L * d->Hq > INT32_MAX / 2) return SKV_ERR_SHAPE;
  d->stride = s->kv_head_stride ? s->kv_head_stride : s->n_in * s->head_dim;
  if (d->stride < d->n_in * d->D) return SKV_ERR_SHAPE;
  // Every size the library forms (buffer spans, workspace pieces) stays far
  // inside int64: the K/V span below 2^60 bytes, L * Hq * n_in below 2^56 and
  // the query rows L * Hq * (n_window + n_lookahead) below 2^40.
  constexpr int64_t kSpan = INT64_C(1) << 60;
  if (d->stride > kSpan / (d->L * d->Hkv * d->esize)) return SKV_ERR_SHAPE;
  if (d->n_in > (INT64_C(1) << 56) / (d->L * d->Hq)) return SKV_ERR_SHAPE;
  if ((int64_t)s->n_window + s->n_lookahead > (INT64_C(1) << 40) / (d->L * d->Hq)) return SKV_ERR_SHAPE;
  if ((d->stride * d->esize) % 16 != 0) return SKV_ERR_ALIGN;
  d->n_window = s->n_window;
  d->n_lookahead = s->n_lookahead;
  d->scale = s->scale > 0.f ? s->scale : (float)(1.0 / std::sqrt((double)s->head_dim));
  d->dtype = s->dtype;
  const int64_t G = d->Hq / d->Hkv;
  // query rows per unit must stay inside int32 for the kernels
  if (G * (d->n_window + d->n_lookahead) > INT32_MAX / 2) return SKV_ERR_SHAPE;
  return SKV_OK;
}

// ---- workspace layouts -------------------------------------------------
struct ScoreWs {
  size_t part, lam, colpart, end;
};
ScoreWs score_ws(const Dims& d, int64_t units, int64_t rows, int64_t keys) {
  ScorePlan pl{1, 1, 32, 1, 2, 0, 0};
  if (keys > 0 && rows > 0) score_plan(d.dtype, (int)d.D, units, rows, keys, &pl);
  const int64_t chunks = pl.n_chunks;
  ScoreWs w;
  w.part = 0;
  w.lam = round_up((size_t)(units * chunks * rows) * sizeof(float2));
  w.colpart = w.lam + round_up((size_t)(units * rows) * sizeof(float));
  w.end = w.colpart + round_up((size_t)((pl.n_parts - 1) * units * keys) * sizeof(float));
  return w;
}

// SpecKV scoring runs pass 1 over the rows of a whole GQA group per KV head
// in both selection granularities: every row's normaliser is the same, and
// the per-query-head row order ([query head][row] per KV head) is the
// grouped order, so the row statistics land where a per-query-head pass 2
// reads them, while each K row is read once per pass-1 block instead of once
// per query head.  Pass 2 runs one unit per SpecKV head (KV or query head):
// the query heads of one KV head are neighbouring blocks and share its keys
// through L2.
struct SpecKVPlans {
  int64_t units1, rows1, units2, rows2;
  ScorePlan pl1, pl2;
  ScoreWs ws;
};
SpecKVPlans speckv_plans(const Dims& d, int64_t n_pre) {
  const int64_t n_obs = d.n_window + d.n_lookahead;
  SpecKVPlans p;
  p.units1 = d.L * d.Hkv;
  p.rows1 = (d.Hq / d.Hkv) * n_obs;
  p.units2 = d.L * d.heads();
  p.rows2 = d.group() * n_obs;
  p.pl1 = ScorePlan{1, 1, 32, 1, 2, 0, 0};
  p.pl2 = p.pl1;
  if (n_pre > 0 && n_obs > 0) {
    score_plan(d.dtype, (int)d.D, p.units1, p.rows1, n_pre, &p.pl1);
    score_plan(d.dtype, (int)d.D, p.units2, p.rows2, n_pre, &p.pl2);
  }
  const int64_t partials = p.pl2.n_parts - 1;
  p.ws.part = 0;
  p.ws.lam = round_up((size_t)(p.units1 * p.pl1.n_chunks * p.rows1) * sizeof(float2));
  p.ws.colpart = p.ws.lam + round_up((size_t)(p.units1 * p.rows1) * sizeof(float));
  p.ws.end = p.ws.colpart + round_up((size_t)(partials * p.units2 * n_pre) * sizeof(float));
  return p;
}

struct PcWs {
  ScoreWs sc;
  size_t rowmax, end;
};
// SpecPC keys: the n_in input tokens, then the n_lookahead - 1 draft tokens
// the window's draft rows attend (none when n_lookahead <= 1).
int64_t specpc_keys(const Dims& d) { return d.n_in + (d.n_lookahead > 1 ? d.n_lookahead - 1 : 0); }

PcWs specpc_ws(const Dims& d, int64_t units) {
  const int64_t G = d.Hq / d.Hkv, W = d.n_window;
  PcWs w;
  w.sc = score_ws(d, units, G * W, specpc_keys(d));
  const int64_t rpb = specpc_rows_per_block(d.dtype, (int)d.D);
  const int64_t nrb = (W + rpb - 1) / rpb;
  w.rowmax = w.sc.end;
  w.end = w.rowmax + round_up((size_t)(nrb * d.n_in) * sizeof(float));
  return w;
}

// Workspace of specpc_token_scores for any l_skip: the planner may give fewer
// units (a larger l_skip) more key chunks, hence larger pass-1 partials, so
// the size is the maximum over every l_skip in [0, L).
//
// The planner gives a unit more than one key chunk only while the launch has
// fewer blocks than its target; past that the plan of a unit no longer
// depends on the unit count and the workspace grows with it, so l_skip = 0
// is the largest of those.  Only the l_skip values with fewer units than a
// few times the target need a look.
size_t specpc_ws_any_lskip(const Dims& d) {
  const int64_t few = 4 * score_plan_target_blocks();
  size_t need = specpc_ws(d, d.L * d.Hkv).end;
  for (int64_t ls = std::max<int64_t>(1, d.L - few / d.Hkv - 1); ls < d.L; ++ls)
    need = std::max(need, specpc_ws(d, (d.L - ls) * d.Hkv).end);
  return need;
}

int64_t keep_count(const Dims& d, int64_t C_max) {
  const int64_t n_pre = d.n_in - d.n_window;
  return (C_max < n_pre ? C_max : n_pre) + d.n_window;
}

// ---- optional event profiling -----------------------------------------
struct ProfEntry {
  const char* name;
  int64_t launches;
  double ms;
};
struct ProfPending {
  int entry;
  hipEvent_t start, stop;
};
bool g_prof_on = false;
std::vector<ProfEntry> g_prof;
std::vector<ProfPending> g_pending;
std::vector<hipEvent_t> g_spare;

hipEvent_t take_event() {
  if (!g_spare.empty()) {
    hipEvent_t e = g_spare.back();
    g_spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Returns an event to the spare list, or destroys it when the list cannot grow.
void give_event(hipEvent_t e) {
  try {
    g_spare.push_back(e);
  } catch (...) {
    (void)hipEventDestroy(e);
  }
}

// The profiling lists grow while profiling is on; a host allocation failure
// drops that sample and marks the profile incomplete instead of throwing
// (the scope's destructor runs inside the C ABI).
bool g_prof_lost = false;

struct ProfScope {
  int entry = -1;
  hipEvent_t start = nullptr;
  hipStream_t stream;
  ProfScope(const char* name, hipStream_t s) : stream(s) {
    if (!g_prof_on) return;
    try {
      for (size_t i = 0; i < g_prof.size(); ++i)
        if (std::strcmp(g_prof[i].name, name) == 0) entry = (int)i;
      if (entry < 0) {
        g_prof.push_back({name, 0, 0.0});
        entry = (int)g_prof.size() - 1;
      }
      g_pending.reserve(g_pending.size() + 1);
    } catch (...) {
      g_prof_lost = true;
      entry = -1;
      return;
    }
    start = take_event();
    if (start) (void)hipEventRecord(start, stream);
  }
  ~ProfScope() {
    if (!g_prof_on || !start || entry < 0) return;
    hipEvent_t stop = take_event();
    if (!stop) return;
    (void)hipEventRecord(stop, stream);
    g_pending.push_back({entry, start, stop});  // capacity reserved by the constructor: does not throw
  }
};

skv_status hip_status(hipError_t e) { return e == hipSuccess ? SKV_OK : SKV_ERR_HIP; }

#define SKV_TRY(expr)                 \
  do {                                \
    skv_status st_ = (expr);          \
    if (st_ != SKV_OK) return st_;    \
  } while (0)

void apply_plan(ScoreArgs& a, const ScorePlan& pl) {
  a.n_sub = pl.n_sub;
  a.n_chunks = pl.n_chunks;
  a.rows_per_part = pl.rows_per_part;
  a.n_parts = pl.n_parts;
}

skv_status run_scoring(const Dims& d, ScoreArgs& a, const ScorePlan& pl, hipStream_t s) {
  {
    ProfScope p("score_pass1", s);
    SKV_TRY(hip_status(launch_score_pass1(d.dtype, (int)d.D, pl.kt, a, pl.lds_pass1, s)));
  }
  {
    ProfScope p("lse_combine", s);
    SKV_TRY(hip_status(launch_lse_combine(a, s)));
  }
  return SKV_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Every extern "C" body runs through this: a C++ exception (a host
// allocation failure in the library or the HIP runtime) becomes a status.
template <typename F>
skv_status guard(F&& body) {
  try {
    return body();
  } catch (...) {
    return SKV_ERR_INTERNAL;
  }
}

// Bytes spanned by the K (or V) buffer: every head slab but the last in full,
// then the rows of the last one.
size_t kv_span(const Dims& d, int64_t rows_last) {
  return (size_t)((d.L * d.Hkv - 1) * d.stride * d.esize + rows_last * d.D * d.esize);
}

}  // namespace

extern "C" {

const char* speckv_status_string(int32_t status) {
  switch (status) {
    case SKV_OK: return "ok";
    case SKV_ERR_NULL: return "required pointer is NULL";
    case SKV_ERR_SHAPE: return "inconsistent or unsupported shape";
    case SKV_ERR_DTYPE: return "unsupported element type";
    case SKV_ERR_PARAM: return "parameter out of range";
    case SKV_ERR_WORKSPACE: return "workspace missing or too small";
    case SKV_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case SKV_ERR_ALIAS: return "output overlaps an input";
    case SKV_ERR_HIP: return "HIP runtime error";
    case SKV_ERR_INTERNAL: return "host-side failure inside the library";
  }
  return "unknown status";
}

skv_status speckv_n_keep(const skv_shape* shape, int32_t C_max, int64_t* out) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!out) return SKV_ERR_NULL;
    if (C_max < 0) return SKV_ERR_PARAM;
    *out = keep_count(d, C_max);
    return SKV_OK;
  });
}

skv_status speckv_workspace_bytes(const skv_shape* shape, int32_t C_max, size_t* out) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!out) return SKV_ERR_NULL;
    if (C_max < 0) return SKV_ERR_PARAM;
    const int64_t units = d.L * d.heads();
    const int64_t n_pre = d.n_in - d.n_window;
    size_t need = speckv_plans(d, n_pre).ws.end;                                               // speckv_scores
    need = std::max(need, round_up((size_t)(units * n_pre) * sizeof(float)) +                   // speckv_select
                              select_candidate_bytes(units, n_pre, keep_count(d, C_max) - d.n_window));
    need = std::max(need, 2 * round_up((size_t)(units * keep_count(d, C_max) * d.D * d.esize)));  // in-place compact
    if (d.n_window >= 1) need = std::max(need, specpc_ws_any_lskip(d));                          // specpc_token_scores
    *out = need;
    return SKV_OK;
  });
}

}  // extern "C"

namespace {

// speckv_scores, with keys optionally taken through a row list (rows != NULL:
// key j is row rows[j] of each head slab, which holds n_src_rows rows).
skv_status scores_impl(const skv_shape* shape, const void* q_obs, const void* k, const int32_t* rows,
                       int64_t n_src_rows, float* scores, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  SKV_TRY(check_shape(shape, &d));
  const int64_t n_obs = d.n_window + d.n_lookahead, n_pre = d.n_in - d.n_window;
  if (!q_obs || !k || (!scores && n_pre > 0)) return SKV_ERR_NULL;  // an empty prefix has no scores
  if (n_obs < 1) return SKV_ERR_SHAPE;
  if ((d.Hq / d.Hkv) * n_obs > kMaxRows) return SKV_ERR_SHAPE;
  if (!aligned(q_obs, 16) || !aligned(k, 16) || !aligned(scores, 4)) return SKV_ERR_ALIGN;
  const SpecKVPlans pp = speckv_plans(d, n_pre);
  const ScoreWs& w = pp.ws;
  if (n_pre == 0) return SKV_OK;
  const size_t q_bytes = (size_t)(d.L * d.Hq * n_obs * d.D * d.esize);
  const size_t k_bytes = kv_span(d, rows ? n_src_rows : d.n_in);
  const size_t s_bytes = (size_t)(d.L * d.heads() * n_pre) * sizeof(float);
  if (ranges_overlap(scores, s_bytes, q_obs, q_bytes) || ranges_overlap(scores, s_bytes, k, k_bytes) ||
      (rows && ranges_overlap(rows, (size_t)d.n_in * 4, scores, s_bytes)))
    return SKV_ERR_ALIAS;
  // the workspace checks come last (the allocation-free variant relies on it)
  if (!ws || ws_bytes < w.end) return SKV_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return SKV_ERR_ALIGN;
  if (ranges_overlap(scores, s_bytes, ws, w.end) || ranges_overlap(ws, w.end, q_obs, q_bytes) ||
      ranges_overlap(ws, w.end, k, k_bytes) || (rows && ranges_overlap(rows, (size_t)d.n_in * 4, ws, w.end)))
    return SKV_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ScoreArgs a{};
  a.q = q_obs;
  a.k = k;
  a.q_head_stride = n_obs * d.D;
  a.q_layer_stride = d.Hq * a.q_head_stride;
  a.k_head_stride = d.stride;
  a.k_layer_stride = d.Hkv * d.stride;
  a.layer0 = 0;
  a.agg_max = d.agg == SKV_AGG_MAX;
  a.rows_per_qhead = (int32_t)n_obs;
  a.n_keys = (int32_t)n_pre;
  a.causal = 0;
  a.pos_base = 0;
  a.c = d.scale * 1.4426950408889634f;
  char* base = static_cast<char*>(ws);
  a.part = reinterpret_cast<float2*>(base + w.part);
  a.lam = reinterpret_cast<float*>(base + w.lam);
  a.colpart = reinterpret_cast<float*>(base + w.colpart);
  a.scores = scores;
  a.key_rows = rows;
  a.key_row_limit = (int32_t)(rows ? n_src_rows : 0);
  ScoreArgs a1 = a;  // pass 1: one unit per (layer, KV head), the whole group's rows
  a1.n_units = (int32_t)pp.units1;
  a1.n_kv_heads = (int32_t)d.Hkv;
  a1.kv_repeat = 1;
  a1.group = (int32_t)(d.Hq / d.Hkv);
  a1.n_rows = (int32_t)pp.rows1;
  apply_plan(a1, pp.pl1);
  SKV_TRY(run_scoring(d, a1, pp.pl1, s));
  ScoreArgs a2 = a;  // pass 2: one unit per SpecKV head
  a2.n_units = (int32_t)pp.units2;
  a2.n_kv_heads = (int32_t)d.heads();
  a2.kv_repeat = (int32_t)d.repeat();
  a2.group = (int32_t)d.group();
  a2.n_rows = (int32_t)pp.rows2;
  apply_plan(a2, pp.pl2);
  {
    ProfScope p("score_pass2", s);
    SKV_TRY(hip_status(launch_score_pass2(d.dtype, (int)d.D, pp.pl2.kt, a2, pp.pl2.lds_pass2, s)));
  }
  if (a2.n_parts == 1) return SKV_OK;
  ProfScope p("colsum_combine", s);
  return hip_status(launch_colsum_combine(a2, s));
}

}  // namespace

extern "C" {

skv_status speckv_scores(const skv_shape* shape, const void* q_obs, const void* k, float* scores, void* ws,
                         size_t ws_bytes, void* stream) {
  return guard([&]() -> skv_status {
    return scores_impl(shape, q_obs, k, nullptr, 0, scores, ws, ws_bytes, stream);
  });
}

}  // extern "C"

// Scratch of speckv_scores_noalloc: a fixed device array instead of a
// caller workspace, one copy per GPU (each GPU that runs the library holds
// it until the process ends).  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is looked up once
// per GPU and only that address is used.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the current device (looked up on
// the first call there, with that device current).
skv_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SKV_ERR_HIP;
  if (dev >= kMaxDevices) return SKV_ERR_PARAM;
  if (stream) {  // the scratch belongs to the current device: the stream must too
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SKV_ERR_HIP;
    if (sdev != dev) return SKV_ERR_PARAM;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SKV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SKV_OK;
}

}  // namespace

extern "C" {

skv_status speckv_scores_noalloc(const skv_shape* shape, const void* q_obs, const void* k, float* scores,
                                 void* stream) {
  return guard([&]() -> skv_status {
    // Argument checks first (no HIP call on an invalid argument): the
    // scratch then stands in for the workspace, with the same layout.  The
    // pass-1 partials, the row normalisers and the extra column sums are all
    // written before they are read, so the previous call's contents need no
    // clearing.
    const skv_status pre = scores_impl(shape, q_obs, k, nullptr, 0, scores, nullptr, 0, nullptr);
    if (pre != SKV_ERR_WORKSPACE) return pre;  // an argument error, or nothing to score (SKV_OK)
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (speckv_plans(d, d.n_in - d.n_window).ws.end > kNoAllocScratchBytes)
      return SKV_ERR_WORKSPACE;  // needs more than the fixed scratch
    void* ws = nullptr;
    SKV_TRY(scratch_address(static_cast<hipStream_t>(stream), &ws));
    return scores_impl(shape, q_obs, k, nullptr, 0, scores, ws, kNoAllocScratchBytes, stream);
  });
}

skv_status speckv_scores_rows(const skv_shape* shape, const void* q_obs, const void* k, const int32_t* rows,
                              int64_t n_src_rows, float* scores, void* ws, size_t ws_bytes, void* stream) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!rows) return SKV_ERR_NULL;
    if (!aligned(rows, 4)) return SKV_ERR_ALIGN;
    if (n_src_rows < 1 || n_src_rows > INT32_MAX || n_src_rows * d.D > d.stride) return SKV_ERR_SHAPE;
    return scores_impl(shape, q_obs, k, rows, n_src_rows, scores, ws, ws_bytes, stream);
  });
}

skv_status speckv_compact_rows(const skv_shape* shape, const void* k, const void* v, const int32_t* rows,
                               int64_t n_src_rows, const int32_t* kept, int64_t n_keep, void* k_out, void* v_out,
                               void* stream) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!k || !v || !rows || !kept || !k_out || !v_out) return SKV_ERR_NULL;
    if (n_keep < 1 || n_keep > d.n_in) return SKV_ERR_PARAM;
    if (n_src_rows < 1 || n_src_rows > INT32_MAX || n_src_rows * d.D > d.stride) return SKV_ERR_SHAPE;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(kept, 4) ||
        !aligned(rows, 4))
      return SKV_ERR_ALIGN;
    const int64_t kv_units = d.L * d.Hkv, units = d.L * d.heads(), row_bytes = d.D * d.esize;
    const size_t in_bytes = (size_t)((kv_units - 1) * d.stride * d.esize + n_src_rows * row_bytes);
    const size_t out_bytes = (size_t)(units * n_keep * row_bytes);
    const size_t kept_bytes = (size_t)(units * n_keep) * 4, rows_bytes = (size_t)d.n_in * 4;
    if (k == v || ranges_overlap(k_out, out_bytes, k, in_bytes) || ranges_overlap(k_out, out_bytes, v, in_bytes) ||
        ranges_overlap(v_out, out_bytes, k, in_bytes) || ranges_overlap(v_out, out_bytes, v, in_bytes) ||
        ranges_overlap(k_out, out_bytes, v_out, out_bytes) || ranges_overlap(kept, kept_bytes, k_out, out_bytes) ||
        ranges_overlap(kept, kept_bytes, v_out, out_bytes) || ranges_overlap(rows, rows_bytes, k_out, out_bytes) ||
        ranges_overlap(rows, rows_bytes, v_out, out_bytes))
      return SKV_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    GatherArgs g{};
    g.n_units = (int32_t)units;
    g.units_per_layer = (int32_t)d.heads();
    g.src_units_per_layer = (int32_t)d.Hkv;
    g.src_repeat = (int32_t)d.repeat();
    g.n_rows = (int32_t)n_keep;
    g.n_src_rows = (int32_t)n_src_rows;
    g.row_bytes = (int32_t)row_bytes;
    g.src_unit_stride = d.stride * d.esize;
    g.dst_unit_stride = n_keep * row_bytes;
    g.idx = kept;
    g.idx_unit_stride = n_keep;
    g.idx2 = rows;
    g.n_idx2 = (int32_t)d.n_in;
    ProfScope p("compact_gather", s);
    g.src = k;
    g.dst = k_out;
    g.src2 = v;
    g.dst2 = v_out;
    return hip_status(launch_gather(g, s));
  });
}

skv_status speckv_select(const skv_shape* shape, const float* scores, int32_t C_max, int32_t pool, int32_t pool_kernel,
                         int32_t* kept, float* pooled, void* ws, size_t ws_bytes, void* stream) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!kept || (!scores && d.n_in > d.n_window)) return SKV_ERR_NULL;  // an empty prefix has no scores
    if (C_max < 0) return SKV_ERR_PARAM;
    if (pool != SKV_POOL_NONE && pool != SKV_POOL_MAX && pool != SKV_POOL_AVG) return SKV_ERR_PARAM;
    if (pool != SKV_POOL_NONE && (pool_kernel < 1 || pool_kernel % 2 == 0 || pool_kernel > 4097)) return SKV_ERR_PARAM;
    if (!aligned(scores, 4) || !aligned(kept, 4) || (pooled && !aligned(pooled, 4))) return SKV_ERR_ALIGN;
    const int64_t units = d.L * d.heads(), n_pre = d.n_in - d.n_window;
    const int64_t n_keep = keep_count(d, C_max);
    const size_t s_bytes = (size_t)(units * n_pre) * 4, kept_bytes = (size_t)(units * n_keep) * 4;
    if (pooled && ranges_overlap(pooled, s_bytes, scores, s_bytes)) return SKV_ERR_ALIAS;
    if (pooled && ranges_overlap(pooled, s_bytes, kept, kept_bytes)) return SKV_ERR_ALIAS;
    if (ranges_overlap(kept, kept_bytes, scores, s_bytes)) return SKV_ERR_ALIAS;
    const int64_t n_top = n_keep - d.n_window;
    const int n_seg = select_segments(units, n_pre, n_top);
    const size_t pool_bytes = pooled ? 0 : round_up((size_t)(units * n_pre) * sizeof(float));
    const size_t cand_bytes = select_candidate_bytes(units, n_pre, n_top);
    float* pl = pooled;
    char* cand = nullptr;
    if (pool_bytes + cand_bytes > 0) {
      if (!ws || ws_bytes < pool_bytes + cand_bytes) return SKV_ERR_WORKSPACE;
      if (!aligned(ws, 16)) return SKV_ERR_ALIGN;
      const size_t used = pool_bytes + cand_bytes;
      if (ranges_overlap(ws, used, scores, s_bytes) || ranges_overlap(ws, used, kept, kept_bytes) ||
          (pooled && ranges_overlap(ws, used, pooled, s_bytes)))
        return SKV_ERR_ALIAS;
      if (!pooled) pl = static_cast<float*>(ws);
      cand = static_cast<char*>(ws) + pool_bytes;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    SelectArgs a{};
    a.n_seg = n_seg;
    a.seg_len = (int32_t)((n_pre + n_seg - 1) / n_seg);
    if (n_seg > 1) {
      a.cand_key = reinterpret_cast<uint32_t*>(cand);
      a.cand_idx = reinterpret_cast<int32_t*>(cand + (size_t)(units * n_seg * n_top) * 4);
    }
    a.scores = scores;
    a.pooled = pl;
    a.kept = kept;
    a.n_units = (int32_t)units;
    a.n_pre = (int32_t)n_pre;
    a.n_window = (int32_t)d.n_window;
    a.n_top = (int32_t)n_top;
    a.pool = pool;
    a.pool_radius = pool == SKV_POOL_NONE ? 0 : pool_kernel / 2;
    a.write_pooled = pooled != nullptr;
    ProfScope p("select", s);
    return hip_status(launch_select(a, s));
  });
}

skv_status speckv_compact(const skv_shape* shape, const void* k, const void* v, const int32_t* kept, int64_t n_keep,
                          void* k_out, void* v_out, void* ws, size_t ws_bytes, void* stream) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!k || !v || !kept || !k_out || !v_out) return SKV_ERR_NULL;
    if (n_keep < 1 || n_keep > d.n_in) return SKV_ERR_PARAM;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(kept, 4))
      return SKV_ERR_ALIGN;
    const int64_t kv_units = d.L * d.Hkv, units = d.L * d.heads(), row_bytes = d.D * d.esize;
    const size_t in_bytes = (size_t)((kv_units - 1) * d.stride * d.esize + d.n_in * row_bytes);
    const size_t out_bytes = (size_t)(units * n_keep * row_bytes);
    const bool k_inplace = (k_out == k), v_inplace = (v_out == v);
    if (k_inplace != v_inplace) return SKV_ERR_ALIAS;
    if (k == v) return SKV_ERR_ALIAS;
    if (k_inplace && units != kv_units) return SKV_ERR_PARAM;  // per-query-head caches do not fit the KV slabs
    hipStream_t s = static_cast<hipStream_t>(stream);
    GatherArgs g{};
    g.n_units = (int32_t)units;
    g.units_per_layer = (int32_t)d.heads();
    g.src_units_per_layer = (int32_t)d.Hkv;
    g.src_repeat = (int32_t)d.repeat();
    g.n_rows = (int32_t)n_keep;
    g.n_src_rows = (int32_t)d.n_in;
    g.row_bytes = (int32_t)row_bytes;
    g.src_unit_stride = d.stride * d.esize;
    if (!k_inplace) {
      if (ranges_overlap(k_out, out_bytes, k, in_bytes) || ranges_overlap(k_out, out_bytes, v, in_bytes) ||
          ranges_overlap(v_out, out_bytes, k, in_bytes) || ranges_overlap(v_out, out_bytes, v, in_bytes) ||
          ranges_overlap(k_out, out_bytes, v_out, out_bytes) ||
          ranges_overlap(kept, (size_t)(units * n_keep) * 4, k_out, out_bytes) ||
          ranges_overlap(kept, (size_t)(units * n_keep) * 4, v_out, out_bytes))
        return SKV_ERR_ALIAS;
      ProfScope p("compact_gather", s);
      g.idx = kept;
      g.idx_unit_stride = n_keep;
      g.dst_unit_stride = n_keep * row_bytes;
      g.src = k;
      g.dst = k_out;
      g.src2 = v;
      g.dst2 = v_out;
      return hip_status(launch_gather(g, s));
    }
    // In place: gather K and V into the workspace, then copy back to rows [0, n_keep).
    if (ranges_overlap(kept, (size_t)(units * n_keep) * 4, k, in_bytes) ||
        ranges_overlap(kept, (size_t)(units * n_keep) * 4, v, in_bytes) || ranges_overlap(k, in_bytes, v, in_bytes))
      return SKV_ERR_ALIAS;
    const size_t stage = round_up(out_bytes);
    if (!ws || ws_bytes < 2 * stage) return SKV_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return SKV_ERR_ALIGN;
    if (ranges_overlap(ws, 2 * stage, k, in_bytes) || ranges_overlap(ws, 2 * stage, v, in_bytes) ||
        ranges_overlap(ws, 2 * stage, kept, (size_t)(units * n_keep) * 4))
      return SKV_ERR_ALIAS;
    char* ks = static_cast<char*>(ws);
    char* vs = ks + stage;
    {
      ProfScope p("compact_gather", s);
      g.idx = kept;
      g.idx_unit_stride = n_keep;
      g.dst_unit_stride = n_keep * row_bytes;
      g.src = k;
      g.dst = ks;
      g.src2 = v;
      g.dst2 = vs;
      SKV_TRY(hip_status(launch_gather(g, s)));
    }
    ProfScope p("compact_copyback", s);
    GatherArgs b{};
    b.n_units = (int32_t)units;
    b.units_per_layer = b.src_units_per_layer = (int32_t)d.Hkv;
    b.src_repeat = 1;
    b.n_rows = (int32_t)n_keep;
    b.n_src_rows = (int32_t)n_keep;
    b.row_bytes = (int32_t)row_bytes;
    b.idx = nullptr;
    b.src_unit_stride = n_keep * row_bytes;
    b.dst_unit_stride = d.stride * d.esize;
    b.src = ks;
    b.dst = const_cast<void*>(k);
    b.src2 = vs;
    b.dst2 = const_cast<void*>(v);
    return hip_status(launch_gather(b, s));
  });
}

skv_status specpc_gather_tokens(const skv_shape* shape, const void* k, const void* v, const int32_t* tokens,
                                int64_t n_tokens, void* k_out, void* v_out, void* stream) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!k || !v || !tokens || !k_out || !v_out) return SKV_ERR_NULL;
    if (n_tokens < 1 || n_tokens > d.n_in) return SKV_ERR_PARAM;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(tokens, 4))
      return SKV_ERR_ALIGN;
    const int64_t units = d.L * d.Hkv, row_bytes = d.D * d.esize;
    const size_t in_bytes = (size_t)((units - 1) * d.stride * d.esize + d.n_in * row_bytes);
    const size_t out_bytes = (size_t)(units * n_tokens * row_bytes);
    const size_t tok_bytes = (size_t)n_tokens * 4;
    if (k == v || ranges_overlap(k_out, out_bytes, k, in_bytes) || ranges_overlap(k_out, out_bytes, v, in_bytes) ||
        ranges_overlap(v_out, out_bytes, k, in_bytes) || ranges_overlap(v_out, out_bytes, v, in_bytes) ||
        ranges_overlap(k_out, out_bytes, v_out, out_bytes) || ranges_overlap(tokens, tok_bytes, k_out, out_bytes) ||
        ranges_overlap(tokens, tok_bytes, v_out, out_bytes))
      return SKV_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    GatherArgs g{};
    g.n_units = (int32_t)units;
    g.units_per_layer = g.src_units_per_layer = (int32_t)d.Hkv;
    g.src_repeat = 1;
    g.n_rows = (int32_t)n_tokens;
    g.n_src_rows = (int32_t)d.n_in;
    g.row_bytes = (int32_t)row_bytes;
    g.src_unit_stride = d.stride * d.esize;
    g.dst_unit_stride = n_tokens * row_bytes;
    g.idx = tokens;
    g.idx_unit_stride = 0;  // one token list for every (layer, KV head)
    ProfScope p("gather_tokens", s);
    g.src = k;
    g.dst = k_out;
    g.src2 = v;
    g.dst2 = v_out;
    return hip_status(launch_gather(g, s));
  });
}

skv_status specpc_token_scores(const skv_shape* shape, int32_t l_skip, const void* q_win, const void* k,
                               const float* query_weights, float* token_scores, void* ws, size_t ws_bytes,
                               void* stream) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!q_win || !k || !token_scores) return SKV_ERR_NULL;
    if (l_skip < 0 || l_skip >= d.L) return SKV_ERR_PARAM;
    if (d.agg != SKV_AGG_SUM || d.pqh) return SKV_ERR_PARAM;  // SpecPC has its own aggregation
    const int64_t W = d.n_window;
    if (W < 1) return SKV_ERR_SHAPE;
    if ((d.Hq / d.Hkv) * W > kMaxRows) return SKV_ERR_SHAPE;
    if (!aligned(q_win, 16) || !aligned(k, 16) || !aligned(token_scores, 4) ||
        (query_weights && !aligned(query_weights, 4)))
      return SKV_ERR_ALIGN;
    const int64_t G = d.Hq / d.Hkv, units = (d.L - l_skip) * d.Hkv;
    const int64_t n_keys = specpc_keys(d);  // keys in the causal normaliser
    if (d.stride < n_keys * d.D) return SKV_ERR_SHAPE;  // head slabs must hold the draft keys too
    const PcWs w = specpc_ws(d, units);
    if (!ws || ws_bytes < w.end) return SKV_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return SKV_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    SpecPCArgs pa{};
    ScoreArgs& a = pa.sc;
    a.q = q_win;
    a.k = k;
    a.q_head_stride = W * d.D;
    a.q_layer_stride = d.Hq * a.q_head_stride;
    a.k_head_stride = d.stride;
    a.k_layer_stride = d.Hkv * d.stride;
    a.layer0 = l_skip;
    a.n_units = (int32_t)units;
    a.n_kv_heads = (int32_t)d.Hkv;
    a.kv_repeat = 1;
    a.agg_max = 0;
    a.group = (int32_t)G;
    a.rows_per_qhead = (int32_t)W;
    a.n_rows = (int32_t)(G * W);
    a.n_keys = (int32_t)n_keys;
    ScorePlan pl;
    score_plan(d.dtype, (int)d.D, units, G * W, n_keys, &pl);
    apply_plan(a, pl);
    a.causal = 1;
    a.pos_base = n_keys - W;  // window row i sits at position n_keys - W + i
    a.c = d.scale * 1.4426950408889634f;
    char* base = static_cast<char*>(ws);
    a.part = reinterpret_cast<float2*>(base + w.sc.part);
    a.lam = reinterpret_cast<float*>(base + w.sc.lam);
    a.scores = nullptr;
    a.colpart = nullptr;
    pa.weights = query_weights;
    pa.rowblock_max = reinterpret_cast<float*>(base + w.rowmax);
    pa.token_scores = token_scores;
    const int rpb = specpc_rows_per_block(d.dtype, (int)d.D);
    pa.n_rowblocks = (int32_t)((W + rpb - 1) / rpb);
    pa.inv_maps = (float)(1.0 / (double)(units * G));
    SKV_TRY(run_scoring(d, a, pl, s));
    a.n_keys = (int32_t)d.n_in;  // the mean and max cover the input tokens only
    {
      ProfScope p("specpc_pass2", s);
      SKV_TRY(hip_status(launch_specpc_pass2(d.dtype, (int)d.D, pa, s)));
    }
    ProfScope p("specpc_reduce", s);
    return hip_status(launch_specpc_reduce(pa, s));
  });
}

size_t decode_ws_bytes(const Dims& d, int64_t n_rows) {
  const int64_t units = d.L * d.heads();
  int32_t n_sub = 1, chunks = 1;
  decode_plan(d.dtype, units, n_rows, &n_sub, &chunks);
  if (chunks <= 1) return 0;
  const int64_t slots = units * chunks * decode_max_group();
  return round_up((size_t)slots * sizeof(float2)) + round_up((size_t)(slots * d.D) * sizeof(float));
}

skv_status speckv_decode_workspace_bytes(const skv_shape* shape, int64_t n_rows, size_t* out_bytes) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!out_bytes) return SKV_ERR_NULL;
    if (n_rows < 1 || n_rows > d.n_in) return SKV_ERR_PARAM;
    *out_bytes = decode_ws_bytes(d, n_rows);
    return SKV_OK;
  });
}

skv_status speckv_decode_attention(const skv_shape* shape, int64_t n_rows, const void* q, const void* k,
                                   const void* v, float* out, void* ws, size_t ws_bytes, void* stream) {
  return guard([&]() -> skv_status {
    Dims d;
    SKV_TRY(check_shape(shape, &d));
    if (!q || !k || !v || !out) return SKV_ERR_NULL;
    if (n_rows < 1 || n_rows > d.n_in) return SKV_ERR_PARAM;
    if (d.group() > decode_max_group()) return SKV_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4)) return SKV_ERR_ALIGN;
    const int64_t units = d.L * d.heads();
    const size_t cache_bytes = (size_t)((units - 1) * d.stride * d.esize + d.n_in * d.D * d.esize);
    const size_t out_bytes = (size_t)(d.L * d.Hq * d.D) * sizeof(float);
    if (ranges_overlap(out, out_bytes, q, (size_t)(d.L * d.Hq * d.D * d.esize)) ||
        ranges_overlap(out, out_bytes, k, cache_bytes) || ranges_overlap(out, out_bytes, v, cache_bytes))
      return SKV_ERR_ALIAS;
    const size_t need = decode_ws_bytes(d, n_rows);
    DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.head_stride = d.stride;
    a.n_rows = n_rows;
    a.n_units = (int32_t)units;
    a.heads_per_layer = (int32_t)d.heads();
    a.q_heads_per_layer = (int32_t)d.Hq;
    a.group = (int32_t)d.group();
    decode_plan(d.dtype, units, n_rows, &a.n_sub, &a.n_chunks);
    a.c = d.scale * 1.4426950408889634f;
    a.out = out;
    if (need > 0) {
      if (!ws || ws_bytes < need) return SKV_ERR_WORKSPACE;
      if (!aligned(ws, 16)) return SKV_ERR_ALIGN;
      if (ranges_overlap(ws, need, out, out_bytes) || ranges_overlap(ws, need, k, cache_bytes) ||
          ranges_overlap(ws, need, v, cache_bytes))
        return SKV_ERR_ALIAS;
      const int64_t slots = units * a.n_chunks * decode_max_group();
      a.part_ml = static_cast<float2*>(ws);
      a.part_acc = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up((size_t)slots * sizeof(float2)));
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    ProfScope p("decode_attention", s);
    return hip_status(launch_decode_attention(d.dtype, (int)d.D, a, s));
  });
}

skv_status speckv_profile_enable(int32_t on) {
  return guard([&]() -> skv_status {
    if (on) {
      g_prof.clear();
      for (auto& p : g_pending) {
        give_event(p.start);
        give_event(p.stop);
      }
      g_pending.clear();
      g_prof_lost = false;
    }
    g_prof_on = on != 0;
    return SKV_OK;
  });
}

int32_t speckv_profile_count(void) { return (int32_t)g_prof.size(); }

skv_status speckv_profile_read(int32_t index, const char** name, int64_t* launches, double* total_ms) {
  return guard([&]() -> skv_status {
    // Samples are folded into the totals in order; one that cannot be read
    // yet stays pending (the ones before it are not counted twice).
    size_t done = 0;
    skv_status st = SKV_OK;
    for (; done < g_pending.size(); ++done) {
      const ProfPending& p = g_pending[done];
      float ms = 0.f;
      if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
        st = SKV_ERR_HIP;
        break;
      }
      g_prof[p.entry].launches += 1;
      g_prof[p.entry].ms += ms;
      give_event(p.start);
      give_event(p.stop);
    }
    g_pending.erase(g_pending.begin(), g_pending.begin() + (std::ptrdiff_t)done);
    if (st != SKV_OK) return st;
    if (index < 0 || index >= (int32_t)g_prof.size()) return SKV_ERR_PARAM;
    if (name) *name = g_prof[index].name;
    if (launches) *launches = g_prof[index].launches;
    if (total_ms) *total_ms = g_prof[index].ms;
    return g_prof_lost ? SKV_ERR_INTERNAL : SKV_OK;  // dropped samples: the totals are incomplete
  });
}

}  // extern "C"
