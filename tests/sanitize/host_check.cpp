// host_check.cpp -- drives the library's host code (smla_host.cpp) on the CPU
// under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The kernel launchers and the four HIP runtime calls the host code makes are
// replaced here by stubs.  "Device" buffers are host allocations of exactly the
// size the C ABI documents, and each launcher stub touches the first and last
// element of every buffer the real kernel reads or writes, at the extents the
// kernel derives from its arguments (grid, query sets, split count).  A layout
// or size mistake in the host code (a workspace region that runs past the
// documented size, a counter block overlapping the partials, a grid that does
// not match the buffers) then shows as a sanitizer report or a failed check.
// Exit status 0 means every check passed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/sparse_mla.h"
#include "../../sparse_mla_top_amd/csrc/smla_cache_ops.h"
#include "../../sparse_mla_top_amd/csrc/smla_internal.h"
#include "../../sparse_mla_top_amd/csrc/smla_validate.h"

namespace {

int g_failures = 0;
#define CHECK(cond)                                                                   \
  do {                                                                                \
    if (!(cond)) {                                                                    \
      std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #cond);         \
      ++g_failures;                                                                   \
    }                                                                                 \
  } while (0)

// What the next launch is expected to see (set by the driver before each call).
struct Expect {
  int B = 0, q_len = 1, nsplit = 1, max_pages = 1, fmt = 0;
  int64_t pool_pages = 1;
  const uint8_t* ws = nullptr;   // workspace and its size as the caller passed them
  size_t ws_bytes = 0;
  int spin_limit = -1;           // expected SplitArgs::spin_limit (-1: not checked)
};
Expect g_ex;
int g_split_launches = 0, g_combine_launches = 0, g_zero_launches = 0;
unsigned g_validate_bad = 0;

volatile uint8_t g_sink;
template <class T> void touch_read(const T* p, int64_t n) {
  if (n <= 0) return;
  g_sink = *reinterpret_cast<const volatile uint8_t*>(p);
  g_sink = *reinterpret_cast<const volatile uint8_t*>(reinterpret_cast<const uint8_t*>(p + n) - 1);
}
template <class T> void touch_write(T* p, int64_t n) {
  if (n <= 0) return;
  std::memset(static_cast<void*>(p), 0, sizeof(T));
  std::memset(static_cast<void*>(p + n - 1), 0, sizeof(T));
}
bool inside_ws(const void* p, size_t bytes) {
  const uint8_t* b = static_cast<const uint8_t*>(p);
  return b >= g_ex.ws && b + bytes <= g_ex.ws + g_ex.ws_bytes;
}
int row_bytes(int fmt) { return smla_row_bytes(fmt); }

}  // namespace

// ---------------------------------------------------------------- HIP stubs
extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

// ------------------------------------------------------------ launch stubs
namespace smla {

hipError_t launch_split(const SplitArgs& a, int fmt, int nblocks, hipStream_t) {
  ++g_split_launches;
  const int Q = g_ex.B * g_ex.q_len;
  CHECK(fmt == g_ex.fmt);
  CHECK(a.q_len == g_ex.q_len);
  CHECK(a.nsplit == g_ex.nsplit);
  CHECK(nblocks == Q * kHeadGroups * a.nsplit);
  CHECK(a.chunk_tiles >= 1 && (a.nsplit - 1) * a.chunk_tiles < kTiles && a.nsplit * a.chunk_tiles >= kTiles);
  CHECK(a.max_pages == g_ex.max_pages && a.pool_pages == g_ex.pool_pages);
  CHECK(std::isfinite(a.scale_log2));
  if (g_ex.spin_limit >= 0) CHECK(a.spin_limit == g_ex.spin_limit);
  CHECK(a.spin_limit >= 0 && a.spin_limit <= kMergeSpinLimit);
  touch_read(a.q, (int64_t)Q * kHeads * kDqk);
  touch_read(a.pool, g_ex.pool_pages * kPage * row_bytes(fmt));
  touch_read(a.page_table, (int64_t)g_ex.B * g_ex.max_pages);
  touch_read(a.topk_idx, (int64_t)g_ex.B * kTopk);
  touch_read(a.ctx_len, g_ex.B);
  const bool fused = a.nsplit > 1 && a.counters != nullptr;
  CHECK(a.spread == 0 || a.spread == 1);
  if (a.spread && fused) CHECK(nblocks <= 256);   // every split waits for the others: one resident round
  if (a.nsplit == 1 || fused) {
    touch_write(a.out, (int64_t)Q * kHeads * kDv);
    touch_write(a.lse, (int64_t)Q * kHeads);
  }
  if (a.nsplit > 1) {
    CHECK(a.part_o && a.part_lse);
    const size_t po = (size_t)Q * a.nsplit * kHeads * kDv * sizeof(float);
    const size_t pl = (size_t)Q * a.nsplit * kHeads * sizeof(float);
    CHECK(inside_ws(a.part_o, po) && inside_ws(a.part_lse, pl));
    CHECK((const uint8_t*)a.part_o + po <= (const uint8_t*)a.part_lse);   // regions do not overlap
    CHECK(((uintptr_t)a.part_o & 255) == 0 && ((uintptr_t)a.part_lse & 255) == 0);
    touch_write(a.part_o, (int64_t)Q * a.nsplit * kHeads * kDv);
    touch_write(a.part_lse, (int64_t)Q * a.nsplit * kHeads);
    if (fused) {
      // counters [Q][head group][2], then the status word, all before the partials
      const size_t cb = (size_t)Q * kHeadGroups * 2 * sizeof(uint32_t);
      CHECK(inside_ws(a.counters, cb) && inside_ws(a.status, sizeof(uint32_t)));
      CHECK((const uint8_t*)a.counters + cb <= (const uint8_t*)a.status);
      CHECK((const uint8_t*)a.status + sizeof(uint32_t) <= (const uint8_t*)a.part_o);
      touch_write(a.counters, (int64_t)Q * kHeadGroups * 2);
    }
  } else {
    CHECK(!a.part_o && !a.part_lse && !a.counters);
  }
  return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& c, int Qn, hipStream_t) {
  ++g_combine_launches;
  CHECK(Qn == g_ex.B * g_ex.q_len && c.nsplit == g_ex.nsplit && c.nsplit > 1);
  CHECK(inside_ws(c.part_o, (size_t)Qn * c.nsplit * kHeads * kDv * 4));
  CHECK(inside_ws(c.part_lse, (size_t)Qn * c.nsplit * kHeads * 4));
  touch_read(c.part_o, (int64_t)Qn * c.nsplit * kHeads * kDv);
  touch_read(c.part_lse, (int64_t)Qn * c.nsplit * kHeads);
  touch_write(c.out, (int64_t)Qn * kHeads * kDv);
  touch_write(c.lse, (int64_t)Qn * kHeads);
  return hipSuccess;
}

hipError_t launch_gather(const GatherArgs& g, int fmt, int B, hipStream_t) {
  CHECK(B == g_ex.B && fmt == g_ex.fmt);
  touch_read(g.pool, g.pool_pages * kPage * row_bytes(fmt));
  touch_read(g.page_table, (int64_t)B * g.max_pages);
  touch_read(g.topk_idx, (int64_t)B * kTopk);
  touch_read(g.ctx_len, B);
  touch_write(g.rows, (int64_t)B * kTopk * row_bytes(fmt));
  touch_write(g.slots, (int64_t)B * kTopk);
  return hipSuccess;
}

hipError_t launch_zero(uint32_t* p, size_t n, hipStream_t) {
  ++g_zero_launches;
  for (size_t i = 0; i < n; ++i) p[i] = 0u;
  return hipSuccess;
}

hipError_t launch_validate(const int32_t* page_table, const int32_t* topk_idx, const int32_t* ctx_len, int batch,
                           int max_pages, int64_t, hipStream_t, unsigned* bad) {
  touch_read(page_table, (int64_t)batch * max_pages);
  touch_read(topk_idx, (int64_t)batch * kTopk);
  touch_read(ctx_len, batch);
  *bad = g_validate_bad;
  return hipSuccess;
}

hipError_t launch_append(const AppendArgs& a, int fmt, hipStream_t) {
  touch_read(a.latent, (int64_t)a.n * kDl);
  touch_read(a.rope, (int64_t)a.n * 64);
  touch_read(a.req, a.n);
  touch_read(a.pos, a.n);
  touch_read(a.page_table, (int64_t)a.batch * a.max_pages);
  touch_write(a.pool, a.pool_pages * kPage * row_bytes(fmt));
  return hipSuccess;
}

hipError_t launch_indexer(const IndexerArgs& a, int B, hipStream_t) {
  touch_read(a.q, (int64_t)B * kIdxHeads * kIdxDim);
  touch_read(a.w, (int64_t)B * kIdxHeads);
  touch_read(a.keys, a.pool_pages * kPage * kIdxDim * 2);
  touch_read(a.page_table, (int64_t)B * a.max_pages);
  touch_read(a.ctx_len, B);
  touch_write(a.scores, (int64_t)B * a.max_pages * kPage);
  touch_write(a.topk, (int64_t)B * kIdxTopk);
  return hipSuccess;
}

}  // namespace smla

// ------------------------------------------------------------------ driver
namespace {
using namespace smla;

smla_shape shape_of(int B, int fmt, int max_pages, int64_t pool_pages, int q_len) {
  smla_shape s;
  s.batch = B;
  s.num_heads = SMLA_NUM_HEADS;
  s.d_qk = SMLA_D_QK;
  s.d_v = SMLA_D_V;
  s.topk = SMLA_TOPK;
  s.page_size = SMLA_PAGE_SIZE;
  s.kv_format = fmt;
  s.max_pages_per_req = max_pages;
  s.pool_pages = pool_pages;
  s.q_len = q_len;
  return s;
}

// A "device" buffer of exactly n elements, 256-byte aligned, in its own
// allocation (so ASan reports any access past element n-1).
template <class T> struct Buf {
  T* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t count) : n(count) {
    void* v = nullptr;
    if (posix_memalign(&v, 256, count ? count * sizeof(T) : 1) != 0) std::abort();
    p = static_cast<T*>(v);
  }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  T* data() { return p; }
};

// The buffers of one decode call, at the sizes the C ABI documents.
struct Bufs {
  Buf<uint16_t> q;
  Buf<uint8_t> pool;
  Buf<int32_t> page_table, topk, ctx;
  Buf<uint16_t> out;
  Buf<float> lse;
  Bufs(int B, int q_len, int fmt, int max_pages, int64_t pool_pages)
      : q((size_t)B * q_len * kHeads * kDqk),
        pool((size_t)pool_pages * kPage * smla_row_bytes(fmt)),
        page_table((size_t)B * max_pages),
        topk((size_t)B * kTopk),
        ctx((size_t)B),
        out((size_t)B * q_len * kHeads * kDv),
        lse((size_t)B * q_len * kHeads) {}
};

int decode_case(int B, int q_len, int fmt, const smla_plan* plan, bool separate_stages = false) {
  const int max_pages = 40;
  const int64_t pool_pages = 64;
  smla_shape s = shape_of(B, fmt, max_pages, pool_pages, q_len);
  smla_plan p;
  size_t need = 0;
  int rc = smla_plan_for(&s, plan, &p, &need);
  if (rc) return rc;
  Bufs b(B, q_len > 0 ? q_len : 1, fmt, max_pages, pool_pages);
  Buf<uint8_t> wsb(need);          // the workspace: exactly `need` bytes
  uint8_t* ws = wsb.data();
  g_ex.B = B;
  g_ex.q_len = q_len > 0 ? q_len : 1;
  g_ex.nsplit = p.nsplit;
  g_ex.max_pages = max_pages;
  g_ex.pool_pages = pool_pages;
  g_ex.fmt = fmt;
  g_ex.ws = ws;
  g_ex.ws_bytes = need;
  if (separate_stages) {
    rc = smla_decode_split(b.q.data(), b.pool.data(), b.page_table.data(), b.topk.data(), b.ctx.data(), 0.07f,
                           b.out.data(), b.lse.data(), &s, plan, need ? ws : nullptr, need, nullptr);
    if (rc) return rc;
    return smla_decode_combine(&s, plan, need ? ws : nullptr, need, b.out.data(), b.lse.data(), nullptr);
  }
  return sparse_mla_decode(b.q.data(), b.pool.data(), b.page_table.data(), b.topk.data(), b.ctx.data(), 0.07f,
                           b.out.data(), b.lse.data(), &s, plan, need ? ws : nullptr, need, nullptr);
}

void test_plans_and_decode() {
  const int batches[] = {0, 1, 2, 3, 7, 16, 33, 64, 80, 96, 300, 2048, 4097};
  for (int fmt : {SMLA_KV_BF16, SMLA_KV_FP8_E4M3_B128})
    for (int B : batches)
      for (int q_len : {0, 1, 2, 4}) {
        if ((int64_t)B * (q_len ? q_len : 1) > 5000) continue;
        CHECK(decode_case(B, q_len, fmt, nullptr) == SMLA_OK);
        for (int ns = 1; ns <= 16; ++ns)
          for (int m = SMLA_MERGE_AUTO; m <= SMLA_MERGE_SPREAD; ++m) {
            // the full grid up to B = 33; larger batches (partials of GBs) at
            // a few split counts and one query token
            if (B > 33 && (q_len > 1 || (ns > 4 && ns != 16) || (B > 96 && ns > 2))) continue;
            smla_plan pl = {ns, 0, 0, 0, m};
            const int rc = decode_case(B, q_len, fmt, &pl);
            const int Q = B * (q_len ? q_len : 1);
            const int chunk = (kTiles + ns - 1) / ns, ns_eff = (kTiles + chunk - 1) / chunk;
            // the spread merge only for grids resident at once (256 CUs here)
            const bool over = ns > 1 && (((m == SMLA_MERGE_IN_KERNEL || m == SMLA_MERGE_SPREAD) && Q > 4096) ||
                                         (m == SMLA_MERGE_SPREAD && Q * kHeadGroups * ns_eff > 256));
            CHECK(rc == (over ? SMLA_ERR_PLAN : SMLA_OK));
            if (m == SMLA_MERGE_AUTO && ns > 1 && B > 0 && B <= 96) CHECK(decode_case(B, q_len, fmt, &pl, true) == SMLA_OK);
          }
      }
}

void test_argument_errors() {
  const int B = 4, fmt = SMLA_KV_FP8_E4M3_B128;
  smla_shape s = shape_of(B, fmt, 40, 64, 1);
  Bufs b(B, 1, fmt, 40, 64);
  smla_plan p;
  size_t need = 0;
  smla_plan four = {4, 0, 0, 0, SMLA_MERGE_IN_KERNEL};
  CHECK(smla_plan_for(&s, &four, &p, &need) == SMLA_OK && need > 0);
  Buf<uint8_t> ws(need);
  std::memset(ws.p, 0, need);
  g_ex = Expect{};
  g_ex.B = B;
  g_ex.nsplit = 4;
  g_ex.max_pages = 40;
  g_ex.pool_pages = 64;
  g_ex.fmt = fmt;
  g_ex.ws = ws.p;
  g_ex.ws_bytes = need;
  auto call = [&](const void* q, const void* pool, void* out, float scale, void* w, size_t wb, const smla_shape* sh,
                  const smla_plan* pl) {
    return sparse_mla_decode(q, pool, b.page_table.data(), b.topk.data(), b.ctx.data(), scale, out, b.lse.data(), sh,
                             pl, w, wb, nullptr);
  };
  const int before = g_split_launches;
  CHECK(call(b.q.data(), b.pool.data(), b.out.data(), 0.1f, ws.p, need, &s, &four) == SMLA_OK);
  CHECK(g_split_launches == before + 1);
  CHECK(call(b.q.data(), b.pool.data(), b.out.data(), 0.1f, ws.p, need - 1, &s, &four) == SMLA_ERR_WORKSPACE);
  CHECK(call(b.q.data(), b.pool.data(), b.out.data(), 0.1f, nullptr, 0, &s, &four) == SMLA_ERR_WORKSPACE);
  CHECK(call(b.q.data(), b.pool.data(), b.out.data(), NAN, ws.p, need, &s, &four) == SMLA_ERR_INVALID_ARG);
  CHECK(call(b.q.data(), b.pool.data(), b.out.data(), INFINITY, ws.p, need, &s, &four) == SMLA_ERR_INVALID_ARG);
  CHECK(call(nullptr, b.pool.data(), b.out.data(), 0.1f, ws.p, need, &s, &four) == SMLA_ERR_INVALID_ARG);
  CHECK(call((const uint8_t*)b.q.data() + 2, b.pool.data(), b.out.data(), 0.1f, ws.p, need, &s, &four) ==
        SMLA_ERR_INVALID_ARG);
  CHECK(call(b.q.data(), b.pool.data() + 8, b.out.data(), 0.1f, ws.p, need, &s, &four) == SMLA_ERR_INVALID_ARG);
  CHECK(call(b.q.data(), b.pool.data(), (uint8_t*)b.out.data() + 2, 0.1f, ws.p, need, &s, &four) ==
        SMLA_ERR_INVALID_ARG);
  CHECK(call(b.q.data(), b.pool.data(), b.out.data(), 0.1f, ws.p + 8, need - 8, &s, &four) != SMLA_OK);
  CHECK(call(b.q.data(), b.pool.data(), b.out.data(), 0.1f, ws.p, need, nullptr, &four) == SMLA_ERR_INVALID_ARG);
  CHECK(g_split_launches == before + 1);   // no launch on any error

  // shapes
  smla_shape bad = s;
  bad.kv_format = 7;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_INVALID_ARG);
  bad = s;
  bad.num_heads = 128;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_UNSUPPORTED_SHAPE);
  bad = s;
  bad.topk = 2048;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_UNSUPPORTED_SHAPE);
  bad = s;
  bad.batch = -1;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_INVALID_ARG);
  bad = s;
  bad.max_pages_per_req = 0;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_INVALID_ARG);
  bad = s;
  bad.pool_pages = INT64_MAX / 2;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_INVALID_ARG);
  bad = s;
  bad.q_len = 5;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_UNSUPPORTED_SHAPE);
  bad = s;
  bad.q_len = -1;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_INVALID_ARG);
  bad = s;
  bad.batch = (1 << 20) + 1;
  CHECK(smla_plan_for_cus(&bad, nullptr, 256, &p, &need) == SMLA_ERR_INVALID_ARG);
  bad = s;
  bad.batch = 1 << 20;   // the largest batch: the workspace size must not overflow
  for (int ns = 1; ns <= 16; ++ns) {
    smla_plan pl = {ns, 0, 0, 0, SMLA_MERGE_SEPARATE};
    CHECK(smla_plan_for_cus(&bad, &pl, 256, &p, &need) == SMLA_OK);
    if (p.nsplit > 1) CHECK(need > (size_t)(1 << 20) * p.nsplit * kHeads * kDv * 4);
  }
  CHECK(smla_plan_for_cus(&s, nullptr, 0, &p, &need) == SMLA_ERR_INVALID_ARG);
  CHECK(smla_plan_for_cus(&s, nullptr, 256, nullptr, &need) == SMLA_ERR_INVALID_ARG);
  for (smla_plan bp : {smla_plan{17, 0, 0, 0, 0}, smla_plan{-1, 0, 0, 0, 0}, smla_plan{0, 16, 0, 0, 0},
                       smla_plan{0, 0, 64, 0, 0}, smla_plan{0, 0, 0, 2, 0}, smla_plan{0, 0, 0, 0, 4},
                       smla_plan{0, 0, 0, 0, -1}})
    CHECK(smla_plan_for_cus(&s, &bp, 256, &p, &need) == SMLA_ERR_PLAN);
  // every CU count gives a plan within bounds
  for (int cus = 1; cus <= 1024; cus += 37)
    for (int Bx : {1, 5, 80, 96, 4096}) {
      smla_shape sx = shape_of(Bx, fmt, 40, 64, 1);
      CHECK(smla_plan_for_cus(&sx, nullptr, cus, &p, &need) == SMLA_OK);
      CHECK(p.nsplit >= 1 && p.nsplit <= 16);
    }
}

void test_validate_and_status() {
  const int B = 3, fmt = SMLA_KV_BF16;
  smla_shape s = shape_of(B, fmt, 40, 64, 1);
  Bufs b(B, 1, fmt, 40, 64);
  smla_plan p;
  size_t need = 0;
  smla_plan fused = {4, 0, 0, 0, SMLA_MERGE_IN_KERNEL};
  CHECK(smla_plan_for(&s, &fused, &p, &need) == SMLA_OK);
  Buf<uint8_t> ws(need);
  std::memset(ws.p, 0, need);
  g_ex = Expect{};
  g_ex.B = B;
  g_ex.nsplit = 4;
  g_ex.max_pages = 40;
  g_ex.pool_pages = 64;
  g_ex.fmt = fmt;
  g_ex.ws = ws.p;
  g_ex.ws_bytes = need;
  auto call = [&]() {
    return sparse_mla_decode(b.q.data(), b.pool.data(), b.page_table.data(), b.topk.data(), b.ctx.data(), 0.1f,
                             b.out.data(), b.lse.data(), &s, &fused, ws.p, need, nullptr);
  };
  setenv("SMLA_VALIDATE", "1", 1);
  g_validate_bad = 1;
  CHECK(call() == SMLA_ERR_INDEX);
  g_validate_bad = 0;
  CHECK(call() == SMLA_OK);
  // a merge that gave up: the status word after the counters is set
  const size_t counters = smla::workspace_counter_bytes() - 256;
  std::memset(ws.p + counters, 0xff, 4);
  CHECK(call() == SMLA_ERR_MERGE);
  CHECK(smla_workspace_init(ws.p, need, nullptr) == SMLA_OK);
  CHECK(call() == SMLA_OK);
  unsetenv("SMLA_VALIDATE");
  std::memset(ws.p + counters, 0xff, 4);
  CHECK(call() == SMLA_OK);   // outside validate mode the word is not read back
  CHECK(smla_workspace_init(ws.p, need, nullptr) == SMLA_OK);
  CHECK(smla_workspace_init(ws.p + 1, need - 1, nullptr) == SMLA_ERR_INVALID_ARG);
  CHECK(smla_workspace_init(nullptr, 0, nullptr) == SMLA_OK);
  // the spin limit knob: clamped to [0, kMergeSpinLimit], garbage reads as 0
  struct { const char* v; int want; } knobs[] = {{"0", 0}, {"7", 7}, {"-5", 0}, {"99999999999", kMergeSpinLimit},
                                                 {"abc", 0}, {"", kMergeSpinLimit}};
  for (auto& k : knobs) {
    setenv("SMLA_MERGE_SPIN_LIMIT", k.v, 1);
    g_ex.spin_limit = k.want;
    CHECK(call() == SMLA_OK);
  }
  unsetenv("SMLA_MERGE_SPIN_LIMIT");
  g_ex.spin_limit = kMergeSpinLimit;
  CHECK(call() == SMLA_OK);
  g_ex.spin_limit = -1;
}

void test_other_entry_points() {
  const int B = 5, mp = 12;
  const int64_t pp = 30;
  for (int fmt : {SMLA_KV_BF16, SMLA_KV_FP8_E4M3_B128}) {
    smla_shape s = shape_of(B, fmt, mp, pp, 1);
    Bufs b(B, 1, fmt, mp, pp);
    g_ex = Expect{};
    g_ex.B = B;
    g_ex.fmt = fmt;
    Buf<uint8_t> rows((size_t)B * kTopk * smla_row_bytes(fmt));
    Buf<int64_t> slots((size_t)B * kTopk);
    CHECK(smla_gather_rows(b.pool.data(), b.page_table.data(), b.topk.data(), b.ctx.data(), &s, rows.data(),
                           slots.data(), nullptr) == SMLA_OK);
    CHECK(smla_gather_rows(nullptr, b.page_table.data(), b.topk.data(), b.ctx.data(), &s, rows.data(),
                           slots.data(), nullptr) == SMLA_ERR_INVALID_ARG);
    const int n = 9;
    Buf<float> lat((size_t)n * kDl), rope((size_t)n * 64);
    Buf<int32_t> req(n), pos(n);
    CHECK(smla_kv_append(lat.data(), rope.data(), req.data(), pos.data(), b.page_table.data(), b.pool.data(), n, &s,
                         nullptr) == SMLA_OK);
    CHECK(smla_kv_append(lat.data(), rope.data(), req.data(), pos.data(), b.page_table.data(), b.pool.data(), -1, &s,
                         nullptr) == SMLA_ERR_INVALID_ARG);
    CHECK(smla_kv_append(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, &s, nullptr) == SMLA_OK);
  }
  smla_shape s = shape_of(B, SMLA_KV_BF16, mp, pp, 1);
  Buf<uint16_t> qi((size_t)B * 64 * 128), keys((size_t)pp * kPage * 128);
  Buf<float> w((size_t)B * 64), scores((size_t)B * mp * kPage);
  Buf<int32_t> pt((size_t)B * mp), ctx(B), topk((size_t)B * 512);
  CHECK(smla_indexer_topk(qi.data(), w.data(), keys.data(), pt.data(), ctx.data(), scores.data(), topk.data(), &s,
                          nullptr) == SMLA_OK);
  CHECK(smla_indexer_topk(qi.data(), nullptr, keys.data(), pt.data(), ctx.data(), scores.data(), topk.data(), &s,
                          nullptr) == SMLA_ERR_INVALID_ARG);
  for (int code = -10; code <= 1; ++code) CHECK(smla_strerror(code) != nullptr && smla_strerror(code)[0] != 0);
  CHECK(smla_row_bytes(SMLA_KV_BF16) == 1152 && smla_row_bytes(SMLA_KV_FP8_E4M3_B128) == 656 && smla_row_bytes(9) == -1);
  CHECK(smla_version() > 0);
}

}  // namespace

int main() {
  test_plans_and_decode();
  test_argument_errors();
  test_validate_and_status();
  test_other_entry_points();
  std::printf("host_check: %d split launches, %d combine launches, %d zero fills, %d failures\n", g_split_launches,
              g_combine_launches, g_zero_launches, g_failures);
  return g_failures == 0 ? 0 : 1;
}
