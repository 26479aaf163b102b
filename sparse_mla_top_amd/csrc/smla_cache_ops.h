// smla_cache_ops.h -- argument blocks and launchers of the kernels around the
// decode: the cache producer (smla_append.hip) and the top-k indexer
// (smla_indexer.hip).  Shared by those kernels and the host code; not part of
// the C ABI.
#pragma once
#include "smla_internal.h"

namespace smla {

struct AppendArgs {
  const float* latent;         // fp32 [n][512]
  const float* rope;           // fp32 [n][64]
  const int32_t* req;          // [n] request of each new token
  const int32_t* pos;          // [n] its logical position
  const int32_t* page_table;   // [batch][max_pages]
  uint8_t* pool;               // rows written here
  int64_t pool_pages;
  int batch;
  int max_pages;
  int n;
};

constexpr int kIdxHeads = 64;   // indexer heads
constexpr int kIdxDim = 128;    // indexer head dim (bf16 key rows of 256 B)
constexpr int kIdxTopk = 512;

struct IndexerArgs {
  const uint16_t* q;           // bf16 [B][64][128]
  const float* w;              // [B][64] head weights
  const uint8_t* keys;         // bf16 key rows [pool_pages * 64][128]
  const int32_t* page_table;   // [B][max_pages]
  const int32_t* ctx_len;      // [B]
  float* scores;               // [B][max_pages * 64]
  int32_t* topk;               // [B][512]
  int64_t pool_pages;
  int max_pages;
};

hipError_t launch_append(const AppendArgs& a, int fmt, hipStream_t stream);
hipError_t launch_indexer(const IndexerArgs& a, int B, hipStream_t stream);

}  // namespace smla
