// smla_internal.h -- constants and kernel argument blocks shared by the host
// launcher code and the kernels of libsparse_mla.so (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparse_mla.h"

namespace smla {

constexpr int kHeads = 64;
constexpr int kHpw = 32;        // query heads per split-kernel workgroup
constexpr int kHeadGroups = kHeads / kHpw;
constexpr int kDqk = 576;
constexpr int kDl = 512;        // latent dims
constexpr int kDv = 512;
constexpr int kTopk = 512;
constexpr int kPage = 64;
constexpr int kTile = 32;       // tokens per pipeline tile
constexpr int kTiles = kTopk / kTile;
constexpr int kQkWaves = 4;     // split kernel: 4 QK waves (16 heads x 16-token half each),
constexpr int kPvWaves = 4;     // 4 PV waves (128 latent dims each)
constexpr int kLdWaves = 4;     // and 4 loader waves that issue the row loads
constexpr int kWaves = kQkWaves + kPvWaves + kLdWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kFmtBf16 = 0;
constexpr int kFmtFp8 = 1;
constexpr int kRowBytesBf16 = 2 * kDqk;                  // 1152
constexpr int kRowBytesFp8 = kDl + 16 + 2 * 64;          // 656
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr int kMergeSpinLimit = 1 << 22;   // polls before a merging workgroup gives up

struct SplitArgs {
  const uint16_t* q;           // bf16 [B][q_len][64][576]
  const uint8_t* pool;
  const int32_t* page_table;   // [B][max_pages]
  const int32_t* topk_idx;     // [B][512]
  const int32_t* ctx_len;      // [B]
  int64_t pool_pages;
  int max_pages;
  int q_len;                   // query tokens per request (sharing its selection)
  int nsplit;                  // splits per request
  int chunk_tiles;             // tiles per split (last split may hold fewer)
  float scale_log2;            // softmax scale * log2(e)
  // per (request, query token) = "query set" qs = b * q_len + t:
  float* part_o;               // [qs][nsplit][64][512] normalised partial outputs
  float* part_lse;             // [qs][nsplit][64] natural-log lse of each split
  uint16_t* out;               // bf16 [qs][64][512] (written directly when nsplit == 1)
  float* lse;                  // [qs][64]
  uint32_t* counters;          // [qs][head group][2] tickets / finished writes; non-null: the last split merges
  uint32_t* status;            // workspace status word (non-zero: a merge gave up waiting; see sparse_mla.h)
  int spin_limit;              // polls before a merging workgroup gives up
  int spread;                  // with counters: every split merges a share (all splits resident at once)
};

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  int nsplit;
  uint16_t* out;
  float* lse;
};

struct GatherArgs {
  const uint8_t* pool;
  const int32_t* page_table;
  const int32_t* topk_idx;
  const int32_t* ctx_len;
  int64_t pool_pages;
  int max_pages;
  uint8_t* rows;
  int64_t* slots;
};

hipError_t launch_split(const SplitArgs& a, int fmt, int nblocks, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int B, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, int fmt, int B, hipStream_t stream);
hipError_t launch_zero(uint32_t* p, size_t n, hipStream_t stream);

// sparse_mla_decode with a given workspace (defined in smla_host.cpp; the C
// entry points sparse_mla_decode and sparse_mla_decode_noalloc call it).
int decode_with_workspace(const void* q, const void* kv_pool, const int32_t* page_table, const int32_t* topk_idx,
                          const int32_t* ctx_len, float scale, void* out, float* lse, const smla_shape* shape,
                          const smla_plan* plan_or_null, void* workspace, size_t workspace_bytes, void* stream);
// Bytes of the fixed counter head at the start of every workspace.
size_t workspace_counter_bytes();

}  // namespace smla
