// smla_noalloc.hip -- sparse_mla_decode_noalloc: the decode with its workspace
// in a device array the library holds, for callers that cannot allocate.
#include <hip/hip_runtime.h>

#include <mutex>

#include "smla_internal.h"

namespace {

constexpr size_t kScratchBytes = SMLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The workspace of sparse_mla_decode_noalloc.  Each GPU that loads the library
// holds its own copy until the process ends.  Host code never passes this name
// to a kernel (on the host it is only a stand-in for the symbol): it uses the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device; null until set up

// The address of this device's `scratch`, set up on the first call on the
// device: the symbol's address is looked up with the device current, and the
// arrival counters at its start (which the in-kernel merge needs at zero and
// leaves at zero) are cleared with a fill kernel on `stream`.
int scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SMLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SMLA_ERR_HIP;
    if (smla::launch_zero(static_cast<uint32_t*>(p), smla::workspace_counter_bytes() / sizeof(uint32_t), stream) !=
        hipSuccess)
      return SMLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SMLA_OK;
}

}  // namespace

extern "C" int sparse_mla_decode_noalloc(const void* q, const void* kv_pool, const int32_t* page_table,
                                         const int32_t* topk_idx, const int32_t* ctx_len, float scale, void* out,
                                         float* lse, const smla_shape* shape, const smla_plan* plan_or_null,
                                         void* stream) {
  smla_plan plan;
  size_t need = 0;
  int rc = smla_plan_for(shape, plan_or_null, &plan, &need);   // validates the shape and plan
  if (rc) return rc;
  if (need > kScratchBytes) return SMLA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    rc = scratch_of_current_device(static_cast<hipStream_t>(stream), &ws);
    if (rc) return rc;
  }
  return smla::decode_with_workspace(q, kv_pool, page_table, topk_idx, ctx_len, scale, out, lse, shape,
                                     plan_or_null, ws, need > 0 ? kScratchBytes : 0, stream);
}
