// smla_validate.hip -- validate mode: a check of the top-k indices and page
// ids before a decode call.  The decode itself never fails on them: an index
// outside [0, ctx_len), a logical page past the page-table row or a page id
// outside the pool masks its slot.  Validate mode reports such inputs instead
// (SMLA_ERR_INDEX), for tests and debugging; -1 is the one mask marker it
// accepts.
#include "smla_validate.h"

#include "smla_internal.h"

namespace smla {

namespace {

__device__ unsigned g_bad_index;   // set by validate_kernel; zeroed before each check

__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ page_table,
                                                       const int32_t* __restrict__ topk_idx,
                                                       const int32_t* __restrict__ ctx_len, int batch, int max_pages,
                                                       int64_t pool_pages) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)batch * kTopk) return;
  const int b = (int)(t / kTopk);
  const int i = topk_idx[t];
  if (i == -1) return;
  bool bad = i < 0 || i >= ctx_len[b];
  if (!bad) {
    const int lp = i / kPage;
    bad = lp >= max_pages;
    if (!bad) {
      const int pg = page_table[(int64_t)b * max_pages + lp];
      bad = pg < 0 || (int64_t)pg >= pool_pages;
    }
  }
  if (bad) atomicOr(&g_bad_index, 1u);
}

const unsigned kZero = 0;

}  // namespace

hipError_t launch_validate(const int32_t* page_table, const int32_t* topk_idx, const int32_t* ctx_len, int batch,
                           int max_pages, int64_t pool_pages, hipStream_t stream, unsigned* bad) {
  *bad = 0;
  if (batch <= 0) return hipSuccess;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_bad_index), &kZero, sizeof(unsigned), 0,
                                        hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)batch * kTopk;
  validate_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(page_table, topk_idx, ctx_len, batch, max_pages,
                                                                     pool_pages);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned flag = 0;
  e = hipMemcpyFromSymbolAsync(&flag, HIP_SYMBOL(g_bad_index), sizeof(unsigned), 0, hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  *bad = flag ? 1u : 0u;
  return hipSuccess;
}

}  // namespace smla
