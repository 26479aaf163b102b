// smla_indexer.hip -- gfx950 kernels of the top-k indexer: score every context
// position of each request and select the 512 highest-scoring ones (the
// topk_idx that the decode kernels consume).
//
// The pages name the indexer (its launches per decode step: "Inside the Decode
// Performance Investigation", sections "The Setup" and "Task 2") but give no
// formula; this follows the published lightning indexer of DeepSeek's sparse
// attention, restated:
//     I[s] = sum_j w[j] * max(0, <q[j], k_s>)      (64 heads j, 128 dims)
// over positions s < ctx_len whose page is valid, k_s the bf16 key row of s in
// its own paged cache (same page table as the latent cache); the selection is
// the 512 largest I (equal scores: smaller s first), in that order, then -1.
//
//   score kernel  : one wave per 1024 positions; key rows stream from HBM
//                   into a per-wave LDS ring four tiles ahead and feed bf16
//                   16x16x32 MFMAs against Q held in registers; the
//                   ReLU-weighted head sum is a 16-lane DPP reduction.
//                   HBM-bound: 256 B read and 4 B written per position.
//   select kernel : one 1024-thread workgroup per request; the range of the
//                   valid scores' order-preserving keys is cut into 4096 bins
//                   (again inside the bin holding the 512th, as needed) until at
//                   most 4096 candidates remain, which are sorted in LDS by
//                   score, then position.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "smla_cache_ops.h"

namespace smla {

namespace {

typedef __bf16 ibf16x8 __attribute__((ext_vector_type(8)));
typedef float if32x4 __attribute__((ext_vector_type(4)));

constexpr int kScWaves = 4;                        // score kernel: 4 waves per workgroup
constexpr int kScRing = 4;                         // key tiles in flight per wave
constexpr int kScPagesPerWave = 16;                // 1024 positions per wave
constexpr int kScPosPerWave = kScPagesPerWave * kPage;
constexpr int kScPosPerWg = kScPosPerWave * kScWaves;
constexpr int kTileBytes = 16 * kIdxDim * 2;       // 16 key rows
constexpr int kSelThreads = 1024;                  // select kernel
constexpr int kSelVec = 4;                         // select: 16-byte score loads per thread per batch
constexpr int kMaxPageWords = 4096;                // page-validity bitmask in LDS: up to 131072 pages
static_assert(kScPagesPerWave <= 64, "page ids are held one per lane");

// Source of key rows that must not be read (invalid page, past the context).
__device__ __attribute__((aligned(16))) uint8_t g_zero_key[kIdxDim * 2];

__device__ __forceinline__ bool page_ok(const IndexerArgs& a, int b, int s, int* page) {
  if (s >= a.ctx_len[b]) return false;
  const int lp = s / kPage;
  if (lp >= a.max_pages) return false;
  const int pg = a.page_table[(int64_t)b * a.max_pages + lp];
  *page = pg;
  return pg >= 0 && (int64_t)pg < a.pool_pages;
}

// One direct-to-LDS load: 16 bytes per lane from `src` to LDS address
// lds + 16 * lane.  Inline asm, so the compiler neither orders it against
// every LDS access nor waits for it: completion is tracked with wait_vm.
// AFTER_READS first waits for this wave's outstanding LDS reads, for a load
// that overwrites a slot just read.
template <bool AFTER_READS>
__device__ __forceinline__ void lds_load16(const void* src, uint32_t lds) {
  if constexpr (AFTER_READS)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "m0", "memory");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "m0", "memory");
}
// s_waitcnt vmcnt(N); also a compiler barrier for the LDS reads that follow.
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// Wait for a tile when `after` (0 .. K) later tiles, 4 loads each, may stay in
// flight: vector memory loads complete in issue order.
template <int K> __device__ __forceinline__ void wait_tile(int after) {
  if constexpr (K == 0) {
    wait_vm<0>();
  } else {
    if (after >= K) wait_vm<4 * K>();
    else wait_tile<K - 1>(after);
  }
}

// Sum over the 16 lanes of each DPP row (lanes 16r .. 16r+15), all lanes
// receiving the total: pairs of lanes (xor 1, xor 2 within quads), then the
// mirrored quad in each half-row, then the mirrored half.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  return v;
}

// grid: x = block of 4096 positions, y = request b.  Wave v takes the 16 pages
// from position 4096 blockIdx.x + 1024 v, as 64 MFMA tiles of 16 positions.
// Each tile's 4 KB of key rows goes straight to a slot of the wave's own LDS
// ring (kScRing slots, no other wave touches them), kScRing tiles ahead of the
// one being scored.
__global__ __launch_bounds__(64 * kScWaves) void indexer_score_kernel(IndexerArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kScWaves * kScRing * kTileBytes];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s_wave = blockIdx.x * kScPosPerWg + kScPosPerWave * wave;
  const int ctx = a.ctx_len[b];
  const int npos = min(ctx, a.max_pages * kPage);  // positions the row of scores holds
  if (s_wave >= npos) return;
  const int g = lane >> 4, c16 = lane & 15;
  const int ntile = min(kScPosPerWave / 16, (npos - s_wave + 15) / 16);

  // lane j < 16: physical page of the wave's page j, -1 when invalid
  int pgv = -1;
  {
    const int lp = s_wave / kPage + lane;
    if (lane < kScPagesPerWave && lp < a.max_pages) {
      const int pg = a.page_table[(int64_t)b * a.max_pages + lp];
      pgv = pg >= 0 && (int64_t)pg < a.pool_pages ? pg : -1;
    }
  }
  // Q as the MFMA B operand: head block hb (16 heads), k-step ks (32 dims):
  // lane holds q[16 hb + c16][32 ks + 8 g .. + 7]
  const uint16_t* qb = a.q + (int64_t)b * kIdxHeads * kIdxDim;
  ibf16x8 qv[4][4];
  float wv[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    wv[hb] = a.w[(int64_t)b * kIdxHeads + 16 * hb + c16];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qv[hb][ks] = *reinterpret_cast<const ibf16x8*>(qb + (16 * hb + c16) * kIdxDim + 32 * ks + 8 * g);
  }

  // tile: 16 key rows, 4 KB contiguous within a page.  Load j reads rows
  // 4j .. 4j+3 as one contiguous KB: lane L takes row r = 4j + L / 16, 16-byte
  // chunk (L % 16) ^ r, so that in LDS row r holds its chunk c at
  // slot + 256 r + 16 (c ^ r); the swizzle keeps the MFMA operand reads below
  // (16 rows, one chunk each) on distinct banks.
  uint8_t* const mine = ring + wave * kScRing * kTileBytes;
  const uint32_t mine_lds = (uint32_t)(uintptr_t)mine;
  auto issue = [&](int tile, auto after_reads) {
    const int page = __builtin_amdgcn_readlane(pgv, tile >> 2);
    const uint32_t dst = mine_lds + (tile % kScRing) * kTileBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * j + (lane >> 4);
      const int s = s_wave + 16 * tile + r;
      const int chunk = (lane & 15) ^ r;
      const uint8_t* src = page >= 0 && s < ctx
                               ? a.keys + ((int64_t)page * kPage + (s & (kPage - 1))) * (kIdxDim * 2) + 16 * chunk
                               : g_zero_key + 16 * chunk;
      if (j == 0) lds_load16<decltype(after_reads)::value>(src, dst);
      else lds_load16<false>(src, dst + 1024 * j);
    }
  };
  const int npre = min(kScRing, ntile);
  for (int i = 0; i < npre; ++i) issue(i, std::false_type{});

  float keep = 0.f;                                // this lane's score in the current page
#pragma unroll 1
  for (int tile = 0; tile < ntile; ++tile) {
    // tiles issued after this one: their 4 loads each may stay in flight
    wait_tile<kScRing - 1>(min(kScRing - 1, ntile - 1 - tile));
    const uint8_t* slot = mine + (tile % kScRing) * kTileBytes;
    ibf16x8 kv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kv[ks] = *reinterpret_cast<const ibf16x8*>(slot + 256 * c16 + 16 * ((4 * ks + g) ^ c16));
    // A operand, k-step ks: lane (c16, g) holds key[16 tile + c16][32 ks + 8 g .. + 7]
    // S[16 positions][16 heads] per head block; lane (c16, g) holds positions 4g..4g+3 of head c16
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      if32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[ks], qv[hb][ks], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] += wv[hb] * fmaxf(acc[i], 0.f);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) part[i] = row16_sum(part[i]);   // over the 16 heads of the block
    // lane (c16, g) keeps position 16 (c16 / 4) + 4 g + c16 % 4 of the page: from tile c16 / 4
    const int tt = tile & 3;
    if ((c16 >> 2) == tt) {
      const int i = c16 & 3;
      keep = i == 0 ? part[0] : i == 1 ? part[1] : i == 2 ? part[2] : part[3];
    }
    if (tt == 3 || tile == ntile - 1) {
      const int sp = s_wave + 64 * (tile >> 2) + 16 * (c16 >> 2) + 4 * g + (c16 & 3);
      const bool pv = __builtin_amdgcn_readlane(pgv, tile >> 2) >= 0;
      if ((c16 >> 2) <= tt && sp < npos) a.scores[(int64_t)b * a.max_pages * kPage + sp] = pv ? keep : -INFINITY;
    }
    if (tile + kScRing < ntile) issue(tile + kScRing, std::true_type{});
  }
}

// Order-preserving 32-bit key of an fp32 score (larger score -> larger key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive prefix sum of one int per thread (kSelThreads threads);
// returns this thread's prefix and writes the block total to *total.
__device__ __forceinline__ int block_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int tw = wave_tot[w];
    before += w < wave ? tw : 0;
    all += tw;
  }
  __syncthreads();                                 // wave_tot is reused by the next scan
  *total = all;
  return before + incl - v;
}

// Wave-level reductions (all lanes receive the result).
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, 64));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Selection for one request (one 1024-thread workgroup).  The k-th largest key
// is bracketed, not computed: the range [min, max] of the valid keys is cut into
// at most 4096 equal bins, the bin holding the 512th largest is kept and cut
// again, until the keys at or above the kept bin number at most kCand.  Those
// candidates (every key above the bin, every key in it) go to LDS as
// (key << 32 | ~position) and a bitonic sort orders them: score descending,
// then position ascending.  The first 512 are the selection.  Only a single key
// value repeated more than kCand - 512 times at the threshold defeats the
// bracketing; then an ordered pass over positions takes the keys above it and
// the lowest positions holding it.
constexpr int kCand = 4096;
constexpr int kSampleMin = 32768;        // contexts from this many positions start from a sample
constexpr int kSampleLines = 256;        // 128-byte lines sampled: 8192 keys
constexpr int kSampleTarget = 1500;      // keys expected above the estimated bound

__global__ __launch_bounds__(kSelThreads) void indexer_select_kernel(IndexerArgs a) {
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int npos = max(0, min(a.ctx_len[b], a.max_pages * kPage));
  const float* sc = a.scores + (int64_t)b * a.max_pages * kPage;
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t validw[kMaxPageWords];       // bit p: page p of this request is valid
  __shared__ uint64_t cand[kCand];
  __shared__ uint32_t red_lo[kSelThreads / 64], red_hi[kSelThreads / 64];
  __shared__ int wave_tot[kSelThreads / 64];
  __shared__ uint32_t bin_s, above_s;
  __shared__ int ncand_s;

  // page validity, from one coalesced pass over the request's page-table row
  const int npages = (npos + kPage - 1) / kPage;
  const bool bitmask = npages <= 32 * kMaxPageWords;
  if (bitmask) {
    for (int i = t; i < (npages + 31) / 32; i += kSelThreads) validw[i] = 0;
    __syncthreads();
    for (int p = t; p < npages; p += kSelThreads) {
      const int pg = a.page_table[(int64_t)b * a.max_pages + p];
      if (pg >= 0 && (int64_t)pg < a.pool_pages) atomicOr(&validw[p >> 5], 1u << (p & 31));
    }
  }
  if (t == 0) ncand_s = 0;
  __syncthreads();
  // s0 is a multiple of 4: the four positions share one page
  auto page_valid = [&, npos](int s0) __attribute__((always_inline)) -> bool {
    if (bitmask) return (validw[s0 >> 11] >> ((s0 >> 6) & 31)) & 1u;
    int pg;
    return page_ok(a, b, s0, &pg);
  };
  // visit every position in batches of 4 kSelVec per thread (kSelVec 16-byte
  // loads per thread in flight); f(s, key, ok) is called by every lane, ok
  // false for positions that are out of range or on an invalid page
  auto for_positions = [&, npos](auto&& f) __attribute__((always_inline)) {
    for (int base = 0; base < npos; base += 4 * kSelVec * kSelThreads) {
      float4 v[kSelVec];
#pragma unroll
      for (int u = 0; u < kSelVec; ++u) {
        const int s0 = base + 4 * (t + u * kSelThreads);
        if (s0 + 3 < npos) {
          v[u] = *reinterpret_cast<const float4*>(sc + s0);
        } else {
          v[u].x = s0 < npos ? sc[s0] : 0.f;
          v[u].y = s0 + 1 < npos ? sc[s0 + 1] : 0.f;
          v[u].z = s0 + 2 < npos ? sc[s0 + 2] : 0.f;
          v[u].w = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kSelVec; ++u) {
        const int s0 = base + 4 * (t + u * kSelThreads);
        const bool pv = s0 < npos && page_valid(s0);
        const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) f(s0 + i, order_key(vv[i]), pv && s0 + i < npos);
      }
    }
  };

  // Block reductions: min and max of a key, sum of a count (all threads get them).
  auto block_range = [&, npos](uint32_t& klo, uint32_t& khi, int& cnt) __attribute__((always_inline)) {
    klo = wave_min(klo);
    khi = wave_max(khi);
    cnt = wave_sum(cnt);
    if (lane == 0) {
      red_lo[wave] = klo;
      red_hi[wave] = khi;
      wave_tot[wave] = cnt;
    }
    __syncthreads();
    klo = 0xffffffffu;
    khi = 0;
    cnt = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
      klo = min(klo, red_lo[w]);
      khi = max(khi, red_hi[w]);
      cnt += wave_tot[w];
    }
    __syncthreads();
  };
  // Over hist[0..4096), the bin d holding the want-th largest entry (counting
  // from the top bin down, want <= total); *above = entries in bins above d.
  // Thread t owns bins 4 (1023 - t) .. + 3; a prefix scan counts the bins above.
  auto crossing_bin = [&, npos](uint32_t want, uint32_t* above) __attribute__((always_inline)) -> uint32_t {
    const int r = kSelThreads - 1 - t;
    const uint32_t hv[4] = {hist[4 * r], hist[4 * r + 1], hist[4 * r + 2], hist[4 * r + 3]};
    int tot;
    uint32_t acc = (uint32_t)block_scan((int)(hv[0] + hv[1] + hv[2] + hv[3]), wave_tot, &tot);
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (acc < want && acc + hv[j] >= want) {
        bin_s = 4 * r + j;
        above_s = acc;
      }
      acc += hv[j];
    }
    __syncthreads();
    const uint32_t d = bin_s;
    *above = above_s;
    __syncthreads();
    return d;
  };
  auto bin_shift = [](uint32_t range) __attribute__((always_inline)) { return range < 4096u ? 0 : (32 - __clz(range)) - 12; };
  // Append every valid key >= lo to cand (wave by wave: ballot, one atomic);
  // ncand_s counts them all, only the first kCand are stored.
  auto collect = [&, npos](uint32_t lo) __attribute__((always_inline)) {
    for_positions([&](int s, uint32_t k, bool ok) __attribute__((always_inline)) {
      const bool take = ok && k >= lo;
      const uint64_t m = __ballot(take);
      if (m) {
        const int leader = __ffsll((unsigned long long)m) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(&ncand_s, __popcll(m));
        base = __shfl(base, leader, 64);
        const int off = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (take && base + off < kCand) cand[base + off] = ((uint64_t)k << 32) | (uint32_t)~(uint32_t)s;
      }
    });
    __syncthreads();
  };

  // Sort cand[0..P) descending (P a power of two, 512 .. kCand).  Thread t
  // holds entries t + 1024 m; stages whose partner lies within 64 entries pair
  // lanes of one wave and run in registers (lane shuffles, no barrier); the
  // wider stages exchange through LDS with a barrier each.
  auto sort_desc = [&, npos](int P) __attribute__((always_inline)) {
    const int per = P > kSelThreads ? P / kSelThreads : 1;
    const bool holds = t < P;                      // whole waves: P is a multiple of 64
    uint64_t x[kCand / kSelThreads];
    auto in_regs = [&](int size, int stride) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < kCand / kSelThreads; ++m) {
        if (m < per) {
          const int i = t + kSelThreads * m;
          const uint32_t lo32 = (uint32_t)__shfl_xor((int)(uint32_t)x[m], stride, 64);
          const uint32_t hi32 = (uint32_t)__shfl_xor((int)(uint32_t)(x[m] >> 32), stride, 64);
          const uint64_t y = ((uint64_t)hi32 << 32) | lo32;
          const bool keep_max = ((i & stride) == 0) == ((i & size) == 0);
          x[m] = keep_max ? (x[m] > y ? x[m] : y) : (x[m] < y ? x[m] : y);
        }
      }
    };
    auto load = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < kCand / kSelThreads; ++m)
        if (m < per) x[m] = cand[t + kSelThreads * m];
    };
    auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < kCand / kSelThreads; ++m)
        if (m < per) cand[t + kSelThreads * m] = x[m];
    };
    if (holds) {
      load();
      for (int size = 2; size <= 64; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) in_regs(size, stride);
      store();
    }
    __syncthreads();
    for (int size = 128; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride >= 64; stride >>= 1) {
        for (int q = t; q < P / 2; q += kSelThreads) {
          const int i = 2 * q - (q & (stride - 1));
          const int j = i + stride;
          const bool desc = (i & size) == 0;
          const uint64_t a0 = cand[i], a1 = cand[j];
          if ((a0 < a1) == desc) {
            cand[i] = a1;
            cand[j] = a0;
          }
        }
        __syncthreads();
      }
      if (holds) {
        load();
        for (int stride = 32; stride > 0; stride >>= 1) in_regs(size, stride);
        store();
      }
      __syncthreads();
    }
  };

  // Estimate from a sample: kSampleLines evenly spaced 128-byte lines of scores
  // (8 threads per line, 8 keys per thread).  A lower bound that about
  // kSampleTarget valid keys clear is read off their histogram; one pass then
  // collects every key above it.  With at least kIdxTopk and at most kCand
  // candidates the selection is among them (every other key is smaller); else
  // the exact path below runs.
  bool cand_ok = false;
  if (npos >= kSampleMin) {
    const int nlines = npos / 32;
    uint32_t sk[8];
    uint32_t slo = 0xffffffffu, shi = 0;
    int nsv = 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int line = r * (kSelThreads / 8) + (t >> 3);
      const int s0 = (int)((int64_t)line * nlines / kSampleLines) * 32 + 4 * (t & 7);   // s0 + 3 < npos
      const float4 v = *reinterpret_cast<const float4*>(sc + s0);
      const bool pv = page_valid(s0);
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t k = order_key(vv[i]);
        sk[4 * r + i] = pv ? k : 0u;
        if (pv) {
          slo = min(slo, k);
          shi = max(shi, k);
          ++nsv;
        }
      }
    }
    block_range(slo, shi, nsv);
    const uint32_t want = (uint32_t)max(1, (int)((int64_t)kSampleTarget * 8 * kSelThreads / npos));
    if ((uint32_t)nsv >= want) {
      const int sh = bin_shift(shi - slo);
      for (int i = t; i < 4096; i += kSelThreads) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (sk[i] >= slo && sk[i] != 0u) atomicAdd(&hist[(sk[i] - slo) >> sh], 1u);
      __syncthreads();
      uint32_t above;
      const uint32_t d = crossing_bin(want, &above);
      collect(slo + (d << sh));
      const int n = ncand_s;
      cand_ok = n >= kIdxTopk && n <= kCand;
      __syncthreads();
      if (!cand_ok && t == 0) ncand_s = 0;
      __syncthreads();
    }
  }

  int nsel = 0;
  uint32_t lo = 0, remaining = kIdxTopk;
  if (!cand_ok) {
    // exact path: range and count of the valid keys
    uint32_t klo = 0xffffffffu, khi = 0;
    int nvalid = 0;
    for_positions([&](int, uint32_t k, bool ok) __attribute__((always_inline)) {
      if (ok) {
        klo = min(klo, k);
        khi = max(khi, k);
        ++nvalid;
      }
    });
    block_range(klo, khi, nvalid);
    // bracket the threshold: keys in [lo, hi], `remaining` of them still to take
    uint32_t hi = khi, incnt = (uint32_t)nvalid;
    lo = nvalid <= kIdxTopk ? 0 : klo;             // at most kIdxTopk: every valid position is selected
    while (nvalid > kIdxTopk && kIdxTopk - remaining + incnt > (uint32_t)kCand && hi > lo) {
      const int sh = bin_shift(hi - lo);
      for (int i = t; i < 4096; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for_positions([&](int, uint32_t k, bool ok) __attribute__((always_inline)) {
        if (ok && k >= lo && k <= hi) atomicAdd(&hist[(k - lo) >> sh], 1u);
      });
      __syncthreads();
      uint32_t above;
      const uint32_t d = crossing_bin(remaining, &above);
      remaining -= above;
      incnt = hist[d];
      lo = lo + (d << sh);
      hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + ((1ull << sh) - 1));
      __syncthreads();
    }
    if (nvalid <= kIdxTopk || kIdxTopk - remaining + incnt <= (uint32_t)kCand) {
      collect(lo);                                 // at most kCand keys
      cand_ok = true;
    }
  }
  if (cand_ok) {
    const int n = min(ncand_s, kCand);
    nsel = min(n, kIdxTopk);
    int P = kIdxTopk;
    while (P < n) P <<= 1;
    for (int i = n + t; i < P; i += kSelThreads) cand[i] = 0ull;   // sorts last
    __syncthreads();
    sort_desc(P);
  } else {
    // one key T = lo = hi repeated too often: the keys above T, then the lowest
    // `remaining` positions holding T.  Thread t walks positions
    // [t L, (t + 1) L) twice: counting, then (after prefix sums over threads,
    // i.e. over positions) writing.
    const uint32_t T = lo;
    const int L = (npos + kSelThreads - 1) / kSelThreads;
    const int s_lo = min(npos, t * L), s_hi = min(npos, s_lo + L);
    int ngt = 0, neq = 0;
    for (int s = s_lo; s < s_hi; ++s) {
      if (!page_valid(s & ~3)) continue;
      const uint32_t k = order_key(sc[s]);
      ngt += k > T ? 1 : 0;
      neq += k == T ? 1 : 0;
    }
    int gt_tot, eq_tot;
    int gt_at = block_scan(ngt, wave_tot, &gt_tot);
    int eq_at = block_scan(neq, wave_tot, &eq_tot);
    for (int s = s_lo; s < s_hi; ++s) {
      if (!page_valid(s & ~3)) continue;
      const uint32_t k = order_key(sc[s]);
      const uint64_t e = ((uint64_t)k << 32) | (uint32_t)~(uint32_t)s;
      if (k > T) {
        if (gt_at < kIdxTopk) cand[gt_at] = e;
        ++gt_at;
      } else if (k == T) {
        if (eq_at < (int)remaining && gt_tot + eq_at < kIdxTopk) cand[gt_tot + eq_at] = e;
        ++eq_at;
      }
    }
    nsel = min(kIdxTopk, gt_tot + min(eq_tot, (int)remaining));
    __syncthreads();
    for (int i = nsel + t; i < kIdxTopk; i += kSelThreads) cand[i] = 0ull;
    __syncthreads();
    sort_desc(kIdxTopk);
  }
  for (int j = t; j < kIdxTopk; j += kSelThreads)
    a.topk[(int64_t)b * kIdxTopk + j] = j < nsel ? (int32_t)~(uint32_t)(cand[j] & 0xffffffffull) : -1;
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, int B, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  {
    const int64_t npos = (int64_t)a.max_pages * kPage;
    const dim3 grid((unsigned)((npos + kScPosPerWg - 1) / kScPosPerWg), B);
    hipLaunchKernelGGL(indexer_score_kernel, grid, dim3(64 * kScWaves), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(indexer_select_kernel, dim3(B), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smla
