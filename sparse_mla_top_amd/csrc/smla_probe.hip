// smla_probe.hip -- smla_read_rows: reads cache rows and discards them, to
// measure how fast this device moves the rows the decode reads when nothing
// else is done with them (no translation, no Q, no arithmetic).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/sparse_mla.h"

namespace {

constexpr int kProbeThreads = 1024;   // 16 waves
constexpr int kProbeDepth = 8;        // loads in flight per lane: 128 KB per compute unit
constexpr int kProbeMaxGroup = 4096;  // rows per group: their offsets are staged in LDS
constexpr int kProbeLds = 96 * 1024;  // more than half the CU's LDS: one workgroup per CU

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Group g reads the rows of slots[g * per_group .. + per_group) (those below
// n_slots; slots outside [0, pool_rows) count as rows of zeros) in 16-byte
// pieces, and leaves one checksum word per thread: the XOR of the 4 words of
// every piece it read (thread t reads pieces t, t + 1024, ... of the group's
// rows laid end to end).  The rows' byte offsets are staged in LDS first, then
// every lane keeps kProbeDepth loads in flight, issuing the next as each
// completes.  Addresses are clamped rather than guarded (a piece past the end,
// or of a skipped row, reads row 0 and is masked out), so the waits count the
// loads in flight exactly.
__global__ __launch_bounds__(kProbeThreads) void read_rows_kernel(const uint8_t* __restrict__ pool,
                                                                  const int64_t* __restrict__ slots,
                                                                  int64_t n_slots, int64_t pool_rows, int per_group,
                                                                  int row_bytes, uint32_t* __restrict__ sink) {
  extern __shared__ int64_t off_s[];   // byte offset of each row of the group, -1 when skipped
  const int64_t first = (int64_t)blockIdx.x * per_group;
  const int64_t last = first + per_group < n_slots ? first + per_group : n_slots;
  const int n = last > first ? (int)(last - first) : 0;
  for (int r = threadIdx.x; r < n; r += kProbeThreads) {
    const int64_t slot = slots[first + r];
    off_s[r] = slot >= 0 && slot < pool_rows ? slot * row_bytes : -1;
  }
  __syncthreads();
  const int chunks = row_bytes / 16;
  const int total = n * chunks;
  const int mine = total > (int)threadIdx.x ? (total - (int)threadIdx.x + kProbeThreads - 1) / kProbeThreads : 0;
  // address of this thread's j-th piece, and whether it counts
  auto piece = [&](int j, uint32_t& keep) {
    const int c = (int)threadIdx.x + j * kProbeThreads;
    const int cc = c < total ? c : 0;
    const int r = cc / chunks, ch = cc - r * chunks;
    const int64_t o = total > 0 ? off_s[r] : -1;
    keep = c < total && o >= 0 ? ~0u : 0u;
    return reinterpret_cast<const u32x4*>(pool + (o >= 0 ? o : 0) + 16 * ch);
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 v[kProbeDepth];
  uint32_t keep[kProbeDepth], knext[kProbeDepth];
  const u32x4* next[kProbeDepth];
#pragma unroll
  for (int d = 0; d < kProbeDepth; ++d) v[d] = __builtin_nontemporal_load(piece(d, keep[d]));
#pragma unroll
  for (int d = 0; d < kProbeDepth; ++d) next[d] = piece(kProbeDepth + d, knext[d]);
  // loads carry the non-temporal hint, as the decode's row loads do.
  // each step consumes the oldest load and issues the next into its slot; the
  // addresses of the following round are computed (LDS reads) while the
  // round's loads are in flight
  for (int j = 0; j < mine; j += kProbeDepth) {
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) {
      acc ^= v[d] & keep[d];
      v[d] = __builtin_nontemporal_load(next[d]);
      keep[d] = knext[d];
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) next[d] = piece(j + 2 * kProbeDepth + d, knext[d]);
  }
  sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

std::mutex g_attr_mu;
bool g_attr_set[64];

}  // namespace

extern "C" {

int smla_read_rows(const void* kv_pool, int64_t pool_rows, const int64_t* slots, int64_t n_slots, int32_t per_group,
                   int32_t row_bytes, int32_t n_groups, uint32_t* sink, void* stream) {
  // (a pool of at least one row: skipped pieces read its first bytes)
  if (!kv_pool || !slots || !sink || pool_rows < 1 || n_slots < 0 || per_group <= 0 || n_groups < 0)
    return SMLA_ERR_INVALID_ARG;
  if (row_bytes != smla_row_bytes(SMLA_KV_FP8_E4M3_B128) && row_bytes != smla_row_bytes(SMLA_KV_BF16))
    return SMLA_ERR_INVALID_ARG;
  if (((uintptr_t)kv_pool & 15) || ((uintptr_t)slots & 7) || ((uintptr_t)sink & 3)) return SMLA_ERR_INVALID_ARG;
  if ((int64_t)n_groups * per_group < n_slots) return SMLA_ERR_INVALID_ARG;   // every slot belongs to a group
  if (per_group > kProbeMaxGroup) return SMLA_ERR_INVALID_ARG;
  if (n_groups == 0) return SMLA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SMLA_ERR_HIP;
  {
    std::lock_guard<std::mutex> lock(g_attr_mu);
    if (!g_attr_set[dev]) {
      if (hipFuncSetAttribute((const void*)read_rows_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kProbeLds) !=
          hipSuccess)
        return SMLA_ERR_HIP;
      g_attr_set[dev] = true;
    }
  }
  hipLaunchKernelGGL(read_rows_kernel, dim3(n_groups), dim3(kProbeThreads), kProbeLds, (hipStream_t)stream,
                     (const uint8_t*)kv_pool, slots, n_slots, pool_rows, per_group, row_bytes, sink);
  return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_HIP;
}

}  // extern "C"
