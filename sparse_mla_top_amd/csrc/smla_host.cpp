// smla_host.cpp -- the C ABI of libsparse_mla.so: argument validation, the
// wave-aware split selector, workspace carving and kernel launches.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "../../include/sparse_mla.h"
#include "smla_cache_ops.h"
#include "smla_internal.h"
#include "smla_validate.h"

using namespace smla;

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxBatch = 1 << 20;     // keeps B * q_len * 512 and the grids far below 2^31
constexpr int kMaxQLen = 4;            // query tokens per request
std::atomic<int> g_cu_count[kMaxDevices];   // 0 = not queried yet

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) { *cus = c; return SMLA_OK; }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    return SMLA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return SMLA_OK;
}

int check_shape(const smla_shape* s) {
  if (!s) return SMLA_ERR_INVALID_ARG;
  if (s->batch < 0 || s->max_pages_per_req < 1 || s->pool_pages < 1) return SMLA_ERR_INVALID_ARG;
  if (s->kv_format != SMLA_KV_BF16 && s->kv_format != SMLA_KV_FP8_E4M3_B128) return SMLA_ERR_INVALID_ARG;
  if (s->num_heads != SMLA_NUM_HEADS || s->d_qk != SMLA_D_QK || s->d_v != SMLA_D_V ||
      s->topk != SMLA_TOPK || s->page_size != SMLA_PAGE_SIZE)
    return SMLA_ERR_UNSUPPORTED_SHAPE;
  // slot = page * 64 + row must fit in int64 and the pool in the address space
  const int64_t rb = s->kv_format == SMLA_KV_BF16 ? kRowBytesBf16 : kRowBytesFp8;
  if (s->pool_pages > INT64_MAX / (kPage * rb)) return SMLA_ERR_INVALID_ARG;
  if (s->q_len < 0) return SMLA_ERR_INVALID_ARG;
  if (s->q_len > kMaxQLen) return SMLA_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)s->batch * (s->q_len > 0 ? s->q_len : 1) > kMaxBatch) return SMLA_ERR_INVALID_ARG;
  return SMLA_OK;
}

// Query tokens per request (0 reads as 1) and query sets (request, token).
int q_len_of(const smla_shape* s) { return s->q_len > 0 ? s->q_len : 1; }
int query_sets(const smla_shape* s) { return s->batch * q_len_of(s); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout (nsplit > 1), per query set (request, query token), Q sets
// in all: a fixed head of 64 KiB of uint32 arrival counters [Q][head group][2]
// (tickets, finished partial writes; room for kMaxMergeSets sets) and a
// 256-byte block holding the status word, then fp32 partial outputs
// [Q, nsplit, 64, 512] and fp32 partial lse [Q, nsplit, 64], each region at a
// 256-byte boundary.  The head sits at the same place for every shape and
// plan, and partial writes never reach it, so a workspace reused across batch
// sizes and split counts finds the counters at zero (each call that merges
// in-kernel resets its own).  The status word is non-zero once a merge has
// given up waiting (its counters may then be off); only smla_workspace_init
// clears it.
constexpr int kMaxMergeSets = 4096;
constexpr size_t kCountersOnly = (size_t)kMaxMergeSets * kHeadGroups * 2 * sizeof(uint32_t);
constexpr size_t kCounterBytes = kCountersOnly + 256;   // counters + status block
static_assert(kCounterBytes % 256 == 0, "counter head keeps the partials 256-byte aligned");
size_t ws_part_o_bytes(int B, int nsplit) { return align256((size_t)B * nsplit * kHeads * kDv * sizeof(float)); }
size_t ws_part_lse_bytes(int B, int nsplit) { return align256((size_t)B * nsplit * kHeads * sizeof(float)); }
size_t workspace_for(int B, int nsplit) {
  if (nsplit <= 1 || B == 0) return 0;
  return kCounterBytes + ws_part_o_bytes(B, nsplit) + ws_part_lse_bytes(B, nsplit);
}

// Estimated time (us) of one call with `nsplit` splits on `cus` compute units
// and the given merge placement.  One workgroup is resident per CU (its LDS
// tiles take most of the 160 KiB), so the B * q_len * 2 * nsplit workgroups
// (two head groups per query token) run in ceil(B*q_len*2*nsplit / cus) dispatch rounds, each as
// long as the longest split (chunk tiles of 32 tokens).  A round starts with
// every resident workgroup fetching its first tiles and its Q at once, a
// burst whose size grows with the grid.  Splitting adds the merge: in the
// kernel, one workgroup per request reads every partial (bounded by one CU's
// memory parallelism), or every split reads its share after a rendezvous; as a
// separate launch, a launch gap plus a short, device-wide read.  The constants
// are fitted to MI355X timings on cold caches (B = 1..96 with one and two
// query tokens, every split count and every merge placement), chosen so that
// the pick is the measured best or within a few per cent of it at every batch
// size.
double est_time_us(int B, int q_len, int nsplit, int chunk_tiles, int cus, int merge, int row_bytes) {
  const double t_start = 3.1863;          // launch, translation and first-gather latency per workgroup
  const double us_per_mb_burst = 0.0878;  // first tiles and Q of every resident workgroup
  const double t_tile = 0.7763;           // one 32-token tile for 32 heads on one CU
  const double t_per_split = 0.0539;      // per split of a request, within a round
  const double us_per_mb = 0.0915;        // gathered rows and per-split Q reads, device-wide
  const double t_fused0 = 4.9696, t_fused_split = 1.1186;    // in-kernel merge: one workgroup reads every partial
  const double t_sep0 = 5.9727, t_sep_split = 0.3295;        // combine launch: gap, lse, partial rounds
  const double t_spread0 = 6.8516, t_spread_split = 0.2097;  // every split merges a share after a rendezvous
  const double us_per_mb_part = 0.072;    // partial bytes written and read back (combine launch)
  const double mb = 1.0 / (1 << 20);
  const int grid = B * q_len * kHeadGroups * nsplit;
  const int rounds = (grid + cus - 1) / cus;
  const int first_tiles = chunk_tiles < 4 ? chunk_tiles : 4;
  const double burst_mb = mb * (double)(grid < cus ? grid : cus) *
                          ((double)first_tiles * kTile * row_bytes + (double)kHpw * kDqk * 2);
  double t = rounds * (t_start + us_per_mb_burst * burst_mb + chunk_tiles * t_tile + t_per_split * nsplit) +
             us_per_mb * mb * (double)B * ((double)kTopk * row_bytes + (double)q_len * nsplit * kHeads * kDqk * 2);
  if (nsplit > 1) {
    if (merge == SMLA_MERGE_IN_KERNEL)
      t += t_fused0 + t_fused_split * nsplit;
    else if (merge == SMLA_MERGE_SPREAD)
      t += t_spread0 + t_spread_split * nsplit;
    else
      t += t_sep0 + t_sep_split * nsplit + us_per_mb_part * mb * 2.0 * B * q_len * nsplit * kHeads * kDv * 4.0;
  }
  return t;
}

}  // namespace

extern "C" {

int smla_row_bytes(int kv_format) {
  if (kv_format == SMLA_KV_BF16) return kRowBytesBf16;
  if (kv_format == SMLA_KV_FP8_E4M3_B128) return kRowBytesFp8;
  return -1;
}

int smla_version(void) { return 103; }

const char* smla_strerror(int code) {
  switch (code) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_INVALID_ARG: return "invalid argument";
    case SMLA_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (need 64 heads, d_qk 576, d_v 512, topk 512, page 64, q_len <= 4)";
    case SMLA_ERR_WORKSPACE: return "workspace missing or too small";
    case SMLA_ERR_PLAN: return "plan override outside the supported values";
    case SMLA_ERR_HIP: return "HIP runtime error";
    case SMLA_ERR_INDEX: return "a top-k index or page id outside its range (validate mode)";
    case SMLA_ERR_MERGE: return "a split merge gave up waiting; the workspace needs smla_workspace_init (validate mode)";
    default: return "unknown error";
  }
}

// Host-only plan selection for a device with `num_cus` compute units.
int smla_plan_for_cus(const smla_shape* shape, const smla_plan* ov, int num_cus, smla_plan* out,
                      size_t* workspace_bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!out || !workspace_bytes || num_cus < 1) return SMLA_ERR_INVALID_ARG;
  smla_plan p = {0, kTile, kHpw, 1, SMLA_MERGE_AUTO};
  if (ov) {
    if (ov->nsplit < 0 || ov->nsplit > kTiles) return SMLA_ERR_PLAN;
    if (ov->tile_tokens != 0 && ov->tile_tokens != kTile) return SMLA_ERR_PLAN;
    if (ov->heads_per_wg != 0 && ov->heads_per_wg != kHpw) return SMLA_ERR_PLAN;
    if (ov->wg_per_cu < 0 || ov->wg_per_cu > 1) return SMLA_ERR_PLAN;
    if (ov->merge < SMLA_MERGE_AUTO || ov->merge > SMLA_MERGE_SPREAD) return SMLA_ERR_PLAN;
    p.nsplit = ov->nsplit;
    p.merge = ov->merge;
  }
  const int B = shape->batch;
  const int slots = num_cus * p.wg_per_cu;
  // a forced split count is normalised to whole tiles with no empty split
  int forced = 0;
  if (p.nsplit != 0) {
    const int c = (kTiles + p.nsplit - 1) / p.nsplit;
    forced = (kTiles + c - 1) / c;
  }
  double best = INFINITY;
  int best_ns = 1, best_merge = SMLA_MERGE_SEPARATE;
  for (int ns = 1; ns <= kTiles; ++ns) {
    const int chunk = (kTiles + ns - 1) / ns;
    if ((kTiles + chunk - 1) / chunk != ns) continue;   // only split counts with no empty split
    if (forced != 0 && ns != forced) continue;
    for (int m = SMLA_MERGE_IN_KERNEL; m <= SMLA_MERGE_SPREAD; ++m) {
      if (p.merge != SMLA_MERGE_AUTO && m != p.merge) continue;
      if ((m == SMLA_MERGE_IN_KERNEL || m == SMLA_MERGE_SPREAD) && ns > 1 && query_sets(shape) > kMaxMergeSets)
        continue;
      // the spread merge waits for every split of a request, so all of the
      // launch's workgroups must be resident at once; chosen automatically
      // only while the grid leaves half the CUs free (a margin for CUs that
      // other work on the device may hold), forced up to every CU
      if (m == SMLA_MERGE_SPREAD && ns > 1 &&
          (int64_t)query_sets(shape) * kHeadGroups * ns > (p.merge == SMLA_MERGE_SPREAD ? slots : slots / 2))
        continue;
      const double t = est_time_us(B > 0 ? B : 1, q_len_of(shape), ns, chunk, slots, m, smla_row_bytes(shape->kv_format));
      if (t < best - 1e-9) { best = t; best_ns = ns; best_merge = m; }
    }
  }
  if (!std::isfinite(best)) return SMLA_ERR_PLAN;   // a forced merge placement this shape cannot take
  p.nsplit = best_ns;
  p.merge = p.nsplit > 1 ? best_merge : SMLA_MERGE_AUTO;
  *out = p;
  *workspace_bytes = workspace_for(query_sets(shape), p.nsplit);
  return SMLA_OK;
}

int smla_plan_for(const smla_shape* shape, const smla_plan* ov, smla_plan* out, size_t* workspace_bytes) {
  int rc = check_shape(shape);
  if (rc) return rc;
  int cus = 0;
  rc = device_cus(&cus);
  if (rc) return rc;
  return smla_plan_for_cus(shape, ov, cus, out, workspace_bytes);
}

// Polls a merging workgroup makes before it gives up.  The environment
// variable SMLA_MERGE_SPIN_LIMIT (read at every call) lowers it, so tests can
// drive the give-up path with every kernel still running to completion.
static int merge_spin_limit() {
  const char* v = std::getenv("SMLA_MERGE_SPIN_LIMIT");
  if (!v || !*v) return kMergeSpinLimit;
  const long n = std::strtol(v, nullptr, 10);
  return n < 0 ? 0 : (n > kMergeSpinLimit ? kMergeSpinLimit : (int)n);
}

static bool validate_mode() {
  const char* v = std::getenv("SMLA_VALIDATE");
  return v && v[0] == '1';
}

// Validate mode (environment SMLA_VALIDATE=1, read at every call): before any
// launch, check the top-k indices and page ids and fail with SMLA_ERR_INDEX
// where the kernels would mask a slot for a reason other than a -1 entry.
// It adds a check kernel and a wait on the stream, so it is for tests and
// debugging, not for graph capture.
static int check_indices(const int32_t* page_table, const int32_t* topk_idx, const int32_t* ctx_len,
                         const smla_shape* shape, void* stream) {
  if (!validate_mode() || shape->batch == 0) return SMLA_OK;
  unsigned bad = 0;
  if (launch_validate(page_table, topk_idx, ctx_len, shape->batch, shape->max_pages_per_req, shape->pool_pages,
                      (hipStream_t)stream, &bad) != hipSuccess)
    return SMLA_ERR_HIP;
  return bad ? SMLA_ERR_INDEX : SMLA_OK;
}

// Validated launch description shared by the decode entry points.
struct Prepared {
  SplitArgs split;
  CombineArgs combine;
  int B = 0;
  int Q = 0;          // query sets (request, query token)
  int nsplit = 1;
  int merge = SMLA_MERGE_AUTO;
  int fmt = 0;
};

static int prepare(const void* q, const void* kv_pool, const int32_t* page_table, const int32_t* topk_idx,
                   const int32_t* ctx_len, float scale, void* out, float* lse, const smla_shape* shape,
                   const smla_plan* plan_or_null, void* workspace, size_t workspace_bytes, Prepared* pr) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !kv_pool || !page_table || !topk_idx || !ctx_len || !out || !lse) return SMLA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return SMLA_ERR_INVALID_ARG;
  const int B = shape->batch;
  const int Q = query_sets(shape);
  smla_plan plan;
  size_t need = 0;
  rc = smla_plan_for(shape, plan_or_null, &plan, &need);
  if (rc) return rc;
  if (need > 0 && (!workspace || workspace_bytes < need)) return SMLA_ERR_WORKSPACE;
  if ((need > 0 && ((uintptr_t)workspace & 15)) || ((uintptr_t)q & 15) || ((uintptr_t)kv_pool & 15) ||
      ((uintptr_t)out & 7))
    return SMLA_ERR_INVALID_ARG;
  SplitArgs& a = pr->split;
  a.q = (const uint16_t*)q;
  a.pool = (const uint8_t*)kv_pool;
  a.page_table = page_table;
  a.topk_idx = topk_idx;
  a.ctx_len = ctx_len;
  a.pool_pages = shape->pool_pages;
  a.max_pages = shape->max_pages_per_req;
  a.q_len = q_len_of(shape);
  a.nsplit = plan.nsplit;
  a.chunk_tiles = (kTiles + plan.nsplit - 1) / plan.nsplit;
  a.scale_log2 = scale * kLog2e;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_lse = nullptr;
  a.counters = nullptr;
  a.status = nullptr;
  a.spin_limit = merge_spin_limit();
  a.spread = plan.merge == SMLA_MERGE_SPREAD ? 1 : 0;
  if (plan.nsplit > 1) {
    a.counters = (uint32_t*)workspace;
    a.status = (uint32_t*)((uint8_t*)workspace + kCountersOnly);
    a.part_o = (float*)((uint8_t*)workspace + kCounterBytes);
    a.part_lse = (float*)((uint8_t*)workspace + kCounterBytes + ws_part_o_bytes(Q, plan.nsplit));
  }
  CombineArgs& c = pr->combine;
  c.part_o = a.part_o;
  c.part_lse = a.part_lse;
  c.nsplit = plan.nsplit;
  c.out = (uint16_t*)out;
  c.lse = lse;
  pr->B = B;
  pr->Q = Q;
  pr->nsplit = plan.nsplit;
  pr->merge = plan.merge;
  pr->fmt = shape->kv_format;
  return SMLA_OK;
}

int sparse_mla_decode(const void* q, const void* kv_pool, const int32_t* page_table,
                      const int32_t* topk_idx, const int32_t* ctx_len, float scale, void* out,
                      float* lse, const smla_shape* shape, const smla_plan* plan_or_null,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return smla::decode_with_workspace(q, kv_pool, page_table, topk_idx, ctx_len, scale, out, lse, shape, plan_or_null,
                                     workspace, workspace_bytes, stream);
}

}  // extern "C"

size_t smla::workspace_counter_bytes() { return kCounterBytes; }

// The body of sparse_mla_decode, shared with the entry point that brings its
// own workspace (smla_noalloc.hip).
int smla::decode_with_workspace(const void* q, const void* kv_pool, const int32_t* page_table,
                                const int32_t* topk_idx, const int32_t* ctx_len, float scale, void* out,
                                float* lse, const smla_shape* shape, const smla_plan* plan_or_null,
                                void* workspace, size_t workspace_bytes, void* stream) {
  Prepared pr;
  int rc = prepare(q, kv_pool, page_table, topk_idx, ctx_len, scale, out, lse, shape, plan_or_null,
                   workspace, workspace_bytes, &pr);
  if (rc || pr.B == 0) return rc;
  rc = check_indices(page_table, topk_idx, ctx_len, shape, stream);
  if (rc) return rc;
  if (pr.nsplit > 1 && pr.merge == SMLA_MERGE_SEPARATE) {
    pr.split.counters = nullptr;       // partials only; the combine launch merges them
    if (launch_split(pr.split, pr.fmt, pr.Q * kHeadGroups * pr.nsplit, (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_combine(pr.combine, pr.Q, (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
    return SMLA_OK;
  }
  // one launch: the last split of each request merges the partials (or
  // every split a share of them)
  if (launch_split(pr.split, pr.fmt, pr.Q * kHeadGroups * pr.nsplit, (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
  // validate mode: wait, and report a merge that gave up (the workspace status word)
  if (pr.nsplit > 1 && validate_mode()) {
    uint32_t st = 0;
    if (hipMemcpyAsync(&st, pr.split.status, sizeof st, hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
        hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
      return SMLA_ERR_HIP;
    if (st) return SMLA_ERR_MERGE;
  }
  return SMLA_OK;
}

extern "C" {

int smla_decode_split(const void* q, const void* kv_pool, const int32_t* page_table,
                      const int32_t* topk_idx, const int32_t* ctx_len, float scale, void* out,
                      float* lse, const smla_shape* shape, const smla_plan* plan_or_null,
                      void* workspace, size_t workspace_bytes, void* stream) {
  Prepared pr;
  int rc = prepare(q, kv_pool, page_table, topk_idx, ctx_len, scale, out, lse, shape, plan_or_null,
                   workspace, workspace_bytes, &pr);
  if (rc || pr.B == 0) return rc;
  rc = check_indices(page_table, topk_idx, ctx_len, shape, stream);
  if (rc) return rc;
  pr.split.counters = nullptr;          // partials only; smla_decode_combine merges them
  if (launch_split(pr.split, pr.fmt, pr.Q * kHeadGroups * pr.nsplit, (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

int smla_decode_combine(const smla_shape* shape, const smla_plan* plan_or_null, const void* workspace,
                        size_t workspace_bytes, void* out, float* lse, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!out || !lse) return SMLA_ERR_INVALID_ARG;
  smla_plan plan;
  size_t need = 0;
  rc = smla_plan_for(shape, plan_or_null, &plan, &need);
  if (rc) return rc;
  if (shape->batch == 0 || plan.nsplit == 1) return SMLA_OK;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15)) return SMLA_ERR_WORKSPACE;
  if ((uintptr_t)out & 7) return SMLA_ERR_INVALID_ARG;
  CombineArgs c;
  c.part_o = (const float*)((const uint8_t*)workspace + kCounterBytes);
  c.part_lse = (const float*)((const uint8_t*)workspace + kCounterBytes + ws_part_o_bytes(query_sets(shape), plan.nsplit));
  c.nsplit = plan.nsplit;
  c.out = (uint16_t*)out;
  c.lse = lse;
  if (launch_combine(c, query_sets(shape), (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

int smla_kv_append(const float* latent, const float* rope, const int32_t* req, const int32_t* pos,
                   const int32_t* page_table, void* kv_pool, int32_t n_tokens, const smla_shape* shape,
                   void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (n_tokens < 0) return SMLA_ERR_INVALID_ARG;
  if (n_tokens == 0) return SMLA_OK;
  if (!latent || !rope || !req || !pos || !page_table || !kv_pool) return SMLA_ERR_INVALID_ARG;
  if (((uintptr_t)latent & 15) || ((uintptr_t)rope & 15) || ((uintptr_t)kv_pool & 15)) return SMLA_ERR_INVALID_ARG;
  AppendArgs a;
  a.latent = latent;
  a.rope = rope;
  a.req = req;
  a.pos = pos;
  a.page_table = page_table;
  a.pool = (uint8_t*)kv_pool;
  a.pool_pages = shape->pool_pages;
  a.batch = shape->batch;
  a.max_pages = shape->max_pages_per_req;
  a.n = n_tokens;
  if (launch_append(a, shape->kv_format, (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

int smla_indexer_topk(const void* q_idx, const float* head_w, const void* key_pool, const int32_t* page_table,
                      const int32_t* ctx_len, float* scores, int32_t* topk_idx, const smla_shape* shape,
                      void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (shape->batch == 0) return SMLA_OK;
  if (!q_idx || !head_w || !key_pool || !page_table || !ctx_len || !scores || !topk_idx) return SMLA_ERR_INVALID_ARG;
  if (((uintptr_t)q_idx & 15) || ((uintptr_t)key_pool & 15)) return SMLA_ERR_INVALID_ARG;
  if ((int64_t)shape->max_pages_per_req * kPage > INT32_MAX / 2) return SMLA_ERR_INVALID_ARG;
  IndexerArgs a;
  a.q = (const uint16_t*)q_idx;
  a.w = head_w;
  a.keys = (const uint8_t*)key_pool;
  a.page_table = page_table;
  a.ctx_len = ctx_len;
  a.scores = scores;
  a.topk = topk_idx;
  a.pool_pages = shape->pool_pages;
  a.max_pages = shape->max_pages_per_req;
  if (launch_indexer(a, shape->batch, (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

int smla_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || ((uintptr_t)workspace & 3)) return workspace_bytes == 0 ? SMLA_OK : SMLA_ERR_INVALID_ARG;
  if (launch_zero((uint32_t*)workspace, workspace_bytes / 4, (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

int smla_gather_rows(const void* kv_pool, const int32_t* page_table, const int32_t* topk_idx,
                     const int32_t* ctx_len, const smla_shape* shape, void* rows, int64_t* slots,
                     void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!kv_pool || !page_table || !topk_idx || !ctx_len || !rows || !slots) return SMLA_ERR_INVALID_ARG;
  if (((uintptr_t)kv_pool & 15) || ((uintptr_t)rows & 15)) return SMLA_ERR_INVALID_ARG;
  if (shape->batch == 0) return SMLA_OK;
  rc = check_indices(page_table, topk_idx, ctx_len, shape, stream);
  if (rc) return rc;
  GatherArgs g;
  g.pool = (const uint8_t*)kv_pool;
  g.page_table = page_table;
  g.topk_idx = topk_idx;
  g.ctx_len = ctx_len;
  g.pool_pages = shape->pool_pages;
  g.max_pages = shape->max_pages_per_req;
  g.rows = (uint8_t*)rows;
  g.slots = slots;
  if (launch_gather(g, shape->kv_format, shape->batch, (hipStream_t)stream) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

}  // extern "C"
