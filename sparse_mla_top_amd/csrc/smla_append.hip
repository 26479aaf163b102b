// smla_append.hip -- gfx950 kernel of the cache producer: quantise new tokens'
// latent and rope values and write their rows into the paged cache that the
// decode kernels read.
//
// The pages name the FP8 latent cache the decode gathers from and a hand-fused
// epilogue that would produce it ("Inside the Decode Performance Investigation",
// sections "Task 1" and "Task 3"); the row format is the one the decode reads:
//   fp8:  512 e4m3 codes | 4 fp32 scales (block j: dims 128j..128j+127) | 64 bf16 rope
//   bf16: 512 bf16 latent | 64 bf16 rope
// Per 128-dim block, scale = amax / 448 (1 for an all-zero block) and
// code = e4m3(x / scale), nearest with ties to even, saturated at +-448; bf16
// values are rounded to nearest, ties to even.  The work is pure data movement
// (2.3 KB read, 656 B written per fp8 row), so the kernel is laid out for
// coalescing: one wave per token, every lane moving 8 consecutive latent values.
#include <hip/hip_runtime.h>

#include "smla_cache_ops.h"

namespace smla {

namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kAppendWaves = 4;   // tokens per 256-thread workgroup

// Max over the 16 lanes of one 16-lane row (lanes 16j .. 16j+15).
__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 16));
  return v;
}

template <int FMT>
__global__ __launch_bounds__(64 * kAppendWaves) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kAppendWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.n) return;
  // destination slot; an out-of-range request, position or page skips the token
  const int b = a.req[t], p = a.pos[t];
  if (b < 0 || b >= a.batch || p < 0 || p / kPage >= a.max_pages) return;
  const int page = a.page_table[(int64_t)b * a.max_pages + p / kPage];
  if (page < 0 || (int64_t)page >= a.pool_pages) return;
  constexpr int kRow = FMT == kFmtFp8 ? kRowBytesFp8 : kRowBytesBf16;
  uint8_t* const row = a.pool + ((int64_t)page * kPage + (p & (kPage - 1))) * kRow;

  // lane: latent dims 8 lane .. 8 lane + 7
  const float4* src = reinterpret_cast<const float4*>(a.latent + (int64_t)t * kDl) + 2 * lane;
  const float4 u = src[0], w = src[1];
  float x[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
  if constexpr (FMT == kFmtFp8) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = row16_max(amax);                       // block lane / 16
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    int lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fminf(fmaxf(x[i] / scale, -448.0f), 448.0f);   // saturate
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
    *reinterpret_cast<uint2*>(row + 8 * lane) = make_uint2((uint32_t)lo, (uint32_t)hi);
    if ((lane & 15) == 0) *reinterpret_cast<float*>(row + kDl + 4 * (lane >> 4)) = scale;
  } else {
    bf16x8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)x[i];
    *reinterpret_cast<bf16x8_t*>(row + 16 * lane) = v;
  }
  // rope: lanes 0..15 take 4 values each
  if (lane < 16) {
    const float4 r = reinterpret_cast<const float4*>(a.rope + (int64_t)t * 64)[lane];
    bf16x4_t v = {(__bf16)r.x, (__bf16)r.y, (__bf16)r.z, (__bf16)r.w};
    constexpr int kRopeOff = FMT == kFmtFp8 ? kDl + 16 : 2 * kDl;
    *reinterpret_cast<bf16x4_t*>(row + kRopeOff + 8 * lane) = v;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int fmt, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const dim3 grid((a.n + kAppendWaves - 1) / kAppendWaves), block(64 * kAppendWaves);
  if (fmt == kFmtFp8)
    hipLaunchKernelGGL(append_kernel<kFmtFp8>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<kFmtBf16>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace smla
