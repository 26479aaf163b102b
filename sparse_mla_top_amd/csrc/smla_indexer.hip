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
//   score kernel  : one wave per 64 positions; key rows stream from HBM straight
//                   into bf16 16x16x32 MFMAs against Q held in registers, and the
//                   ReLU-weighted head sum is a 16-lane butterfly.  HBM-bound:
//                   256 B read and 4 B written per position.
//   select kernel : one 1024-thread workgroup per request; a three-pass radix
//                   select (12 + 12 + 8 bits) on order-preserving keys finds the
//                   512th score exactly, one ordered pass collects the winners
//                   (ties by position), and a bitonic sort orders them.
#include <hip/hip_runtime.h>

#include "smla_internal.h"

namespace smla {

namespace {

typedef __bf16 ibf16x8 __attribute__((ext_vector_type(8)));
typedef float if32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdxWaves = 4;                       // score kernel: 4 waves x 64 positions
constexpr int kIdxPosPerWg = 64 * kIdxWaves;
constexpr int kSelThreads = 1024;                  // select kernel

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

// grid: x = block of 256 positions, y = request b; wave v takes positions
// 256 blockIdx.x + 64 v .. + 63, as four 16-position MFMA tiles.
__global__ __launch_bounds__(64 * kIdxWaves) void indexer_score_kernel(IndexerArgs a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s_wave = blockIdx.x * kIdxPosPerWg + 64 * wave;
  const int npos = min(a.ctx_len[b], a.max_pages * kPage);   // positions the row of scores holds
  if (s_wave >= npos) return;
  const int g = lane >> 4, c16 = lane & 15;

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

#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    // K as the MFMA A operand: lane holds key[s = s_wave + 16 pb + c16][32 ks + 8 g .. + 7]
    const int s = s_wave + 16 * pb + c16;
    int page = 0;
    const bool ok = page_ok(a, b, s, &page);
    const uint8_t* krow = ok ? a.keys + ((int64_t)page * kPage + (s & (kPage - 1))) * (kIdxDim * 2) : g_zero_key;
    ibf16x8 kv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kv[ks] = *reinterpret_cast<const ibf16x8*>(krow + 2 * (32 * ks + 8 * g));
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
    // sum over the 16 heads of each block: the 16 lanes of one row group
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] += __shfl_xor(part[i], m, 16);
    // lane (c16 = i, g) writes position 16 pb + 4 g + i
    if (c16 < 4) {
      const int sp = s_wave + 16 * pb + 4 * g + c16;
      int pg = 0;
      float v = part[0];
      v = c16 == 1 ? part[1] : v;
      v = c16 == 2 ? part[2] : v;
      v = c16 == 3 ? part[3] : v;
      if (sp < npos) a.scores[(int64_t)b * a.max_pages * kPage + sp] = page_ok(a, b, sp, &pg) ? v : -INFINITY;
    }
  }
}

// Order-preserving 32-bit key of an fp32 score (larger score -> larger key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive prefix sum of one 0/1 flag per thread (1024 threads);
// returns this thread's prefix and writes the block total to *total.
__device__ __forceinline__ int block_scan(bool flag, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __builtin_amdgcn_ballot_w64(flag);
  const int in_wave = __builtin_popcountll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[wave] = __builtin_popcountll(m);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int t = wave_tot[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();                                 // wave_tot is reused by the next scan
  *total = all;
  return before + in_wave;
}

__global__ __launch_bounds__(kSelThreads) void indexer_select_kernel(IndexerArgs a) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int npos = min(a.ctx_len[b], a.max_pages * kPage);
  const float* sc = a.scores + (int64_t)b * a.max_pages * kPage;
  __shared__ uint32_t hist[4096];
  __shared__ int wave_tot[kSelThreads / 64];
  __shared__ uint64_t sel[kIdxTopk];
  __shared__ uint32_t prefix_s, remaining_s;
  __shared__ int cnt_s;

  // radix select of the kIdxTopk-th largest key among valid positions
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = kIdxTopk;
  int nvalid = 0;
  const int shifts[3] = {20, 8, 0}, widths[3] = {12, 12, 8};
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass], nb = 1 << widths[pass];
    for (int i = t; i < nb; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    int cnt = 0;
    for (int s = t; s < npos; s += kSelThreads) {
      int pg;
      if (!page_ok(a, b, s, &pg)) continue;
      const uint32_t k = order_key(sc[s]);
      ++cnt;
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    if (pass == 0) {
      // total valid positions (each thread's count, summed through LDS)
      if (t == 0) cnt_s = 0;
      __syncthreads();
      atomicAdd(&cnt_s, cnt);
      __syncthreads();
      nvalid = cnt_s;
      if (nvalid <= kIdxTopk) break;               // every valid position is selected
    }
    if (t == 0) {
      // from the top bin down, find the one holding the remaining-th largest key
      uint32_t above = 0;
      int d = nb - 1;
      for (; d > 0; --d) {
        if (above + hist[d] >= remaining) break;
        above += hist[d];
      }
      prefix_s = prefix | ((uint32_t)d << sh);
      remaining_s = remaining - above;
    }
    __syncthreads();
    prefix = prefix_s;
    remaining = remaining_s;
    mask |= (uint32_t)(nb - 1) << sh;
    __syncthreads();
  }
  const bool all_valid = nvalid <= kIdxTopk;
  const uint32_t T = prefix;                       // exact key of the kIdxTopk-th largest score

  // collect, in position order: keys above T, and the first `remaining` keys equal to T
  int taken_eq = 0, nsel = 0;
  for (int base = 0; base < npos; base += kSelThreads) {
    const int s = base + t;
    int pg;
    const bool v = s < npos && page_ok(a, b, s, &pg);
    const uint32_t k = v ? order_key(sc[s]) : 0u;
    const bool gt = v && (all_valid || k > T);
    const bool eq = v && !all_valid && k == T;
    int eq_tot;
    const int eq_rank = taken_eq + block_scan(eq, wave_tot, &eq_tot);
    const bool take = gt || (eq && eq_rank < (int)remaining);
    int sel_tot;
    const int slot = nsel + block_scan(take, wave_tot, &sel_tot);
    if (take && slot < kIdxTopk) sel[slot] = ((uint64_t)k << 32) | (uint32_t)~(uint32_t)s;
    taken_eq += eq_tot;
    nsel += sel_tot;
  }
  nsel = min(nsel, kIdxTopk);
  for (int i = nsel + t; i < kIdxTopk; i += kSelThreads) sel[i] = 0ull;   // sorts last
  __syncthreads();

  // bitonic sort, descending: score descending, then position ascending
  for (int size = 2; size <= kIdxTopk; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (t < kIdxTopk / 2) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const uint64_t x = sel[i], y = sel[j];
        if ((x < y) == desc) {
          sel[i] = y;
          sel[j] = x;
        }
      }
      __syncthreads();
    }
  for (int j = t; j < kIdxTopk; j += kSelThreads)
    a.topk[(int64_t)b * kIdxTopk + j] = j < nsel ? (int32_t)~(uint32_t)(sel[j] & 0xffffffffull) : -1;
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, int B, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  {
    const int64_t npos = (int64_t)a.max_pages * kPage;
    const dim3 grid((unsigned)((npos + kIdxPosPerWg - 1) / kIdxPosPerWg), B);
    hipLaunchKernelGGL(indexer_score_kernel, grid, dim3(64 * kIdxWaves), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(indexer_select_kernel, dim3(B), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smla
