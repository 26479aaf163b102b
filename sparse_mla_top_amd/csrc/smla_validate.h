// smla_validate.h -- the index check of validate mode (host side).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace smla {

// Check every top-k entry of `batch` requests: an entry other than -1 is bad
// when it lies outside [0, ctx_len[b]), its logical page is >= max_pages, or
// its page id is outside [0, pool_pages).  Runs on `stream` and waits for it;
// *bad receives 1 if any entry is bad, else 0.
hipError_t launch_validate(const int32_t* page_table, const int32_t* topk_idx, const int32_t* ctx_len, int batch,
                           int max_pages, int64_t pool_pages, hipStream_t stream, unsigned* bad);

}  // namespace smla
