// smla_kernels.hip -- gfx950 kernels of the sparse-MLA decode path.
//
//   split kernel   : per (request, top-k split): translate top-k indices to cache
//                    slots, gather the selected rows into LDS with direct-to-LDS
//                    loads, QK^T and PV on bf16 MFMA, online softmax, and write a
//                    normalised partial (O, lse) -- or the final output when the
//                    request is not split.
//   combine kernel : log-sum-exp merge of the partials of each (request, head).
//   gather kernel  : the translation + gather stage alone (test hook).
//
// The split-K structure and the online-softmax merge follow "The 64-Block
// Barrier" (section "The Split-K Prescription") and "The Commit That Rewrote
// the Bottleneck" (section "The Levers"); the tiling below is designed for
// CDNA4 (64-wide waves, 16x16x32 bf16 MFMA, 160 KiB LDS, LDS transpose reads).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

// Source of masked rows: reading zeros keeps every MFMA operand finite.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kRowBytesBf16];

template <int FMT> struct RowFmt;
template <> struct RowFmt<kFmtFp8> {
  static constexpr int kRow = kRowBytesFp8;   // 512 e4m3 | 16 B scales | 128 B rope
  static constexpr int kNbuf = 6;             // 6 x 20,992 B of LDS tiles
};
template <> struct RowFmt<kFmtBf16> {
  static constexpr int kRow = kRowBytesBf16;  // 576 bf16
  static constexpr int kNbuf = 3;             // 3 x 36,864 B
};

// ----------------------------------------------------------------------------
// Index translation (shared by the decode and gather kernels).
// Slot of top-k entry j of request b, or -1 when masked.
__device__ __forceinline__ int64_t translate(const int32_t* __restrict__ page_table,
                                             const int32_t* __restrict__ topk_idx,
                                             int ctx, int b, int j, int max_pages,
                                             int64_t pool_pages) {
  const int i = topk_idx[(int64_t)b * kTopk + j];
  if (i < 0 || i >= ctx) return -1;
  const int lp = i >> 6;
  if (lp >= max_pages) return -1;
  const int page = page_table[(int64_t)b * max_pages + lp];
  if (page < 0 || (int64_t)page >= pool_pages) return -1;
  return (int64_t)page * kPage + (i & (kPage - 1));
}

// Issue the direct-to-LDS loads of one tile (kTile rows).  Row r of the tile
// lands at lds + r * kRow; its 16-byte chunk c comes from the row's slot, or
// from the zero row when the slot is masked.  Wave w issues instructions
// w, w+4, ... of the tile; the count per wave is DmaCount<FMT>::of(w).
template <int FMT>
__device__ __forceinline__ void issue_tile(const uint8_t* __restrict__ pool,
                                           const int64_t LDS_AS* slot_s, int tok0,
                                           uint8_t LDS_AS* lds, int wave, int lane) {
  constexpr int kRow = RowFmt<FMT>::kRow;
  constexpr int kChunksRow = kRow / 16;
  constexpr int kChunks = kTile * kChunksRow;
  constexpr int kInstr = (kChunks + 63) / 64;
  // Re-derive the lane id here so the address arithmetic below is recomputed
  // per tile instead of being hoisted out of the tile loop (and spilled).
  int lane_v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(lane_v) : "v"(lane));
#pragma unroll
  for (int j = 0; j < kInstr; ++j) {
    if ((j & 3) != wave) continue;
    const int c = j * 64 + lane_v;
    if (c < kChunks) {
      const int r = c / kChunksRow;
      const int off = (c - r * kChunksRow) * 16;
      const int64_t slot = slot_s[tok0 + r];
      const uint8_t* src = slot >= 0 ? pool + slot * kRow + off : g_zero_row + off;
      __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)(lds + j * 64 * 16), 16, 0, 0);
    }
  }
}

template <int FMT> struct DmaCount {
  static constexpr int kChunks = kTile * (RowFmt<FMT>::kRow / 16);
  static constexpr int kInstr = (kChunks + 63) / 64;
  __device__ static constexpr int of(int wave) { return (kInstr - wave + 3) / 4; }
};

// s_waitcnt vmcnt(n) with the other counters left unconstrained (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  // n is a multiple of a per-wave DMA count; cover 0..63.
  switch (n) {
#define SMLA_W(k) case k: wait_vmcnt<k>(); break;
    SMLA_W(0) SMLA_W(1) SMLA_W(2) SMLA_W(3) SMLA_W(4) SMLA_W(5) SMLA_W(6) SMLA_W(7)
    SMLA_W(8) SMLA_W(9) SMLA_W(10) SMLA_W(11) SMLA_W(12) SMLA_W(13) SMLA_W(14) SMLA_W(15)
    SMLA_W(16) SMLA_W(17) SMLA_W(18) SMLA_W(19) SMLA_W(20) SMLA_W(21) SMLA_W(22) SMLA_W(23)
    SMLA_W(24) SMLA_W(25) SMLA_W(26) SMLA_W(27) SMLA_W(28) SMLA_W(29) SMLA_W(30) SMLA_W(31)
    SMLA_W(32) SMLA_W(33) SMLA_W(34) SMLA_W(35) SMLA_W(36) SMLA_W(37) SMLA_W(38) SMLA_W(39)
    SMLA_W(40) SMLA_W(41) SMLA_W(42) SMLA_W(43) SMLA_W(44) SMLA_W(45) SMLA_W(46) SMLA_W(47)
    SMLA_W(48) SMLA_W(49) SMLA_W(50) SMLA_W(51) SMLA_W(52) SMLA_W(53) SMLA_W(54) SMLA_W(55)
    SMLA_W(56) SMLA_W(57) SMLA_W(58) SMLA_W(59) SMLA_W(60) SMLA_W(61) SMLA_W(62) SMLA_W(63)
#undef SMLA_W
    default: wait_vmcnt<0>(); break;
  }
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint64_t v) {
  // e4m3fn -> bf16 is exact; the hardware conversion with unit scale.
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ float wave_max16(float v) {
  // max over lanes l, l^16, l^32, l^48 (the four row groups of an MFMA tile)
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Workgroup barrier that orders LDS only.  __syncthreads() would also wait for
// every outstanding global load, including the prefetched tiles in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Workgroup -> (request, split), keeping the splits of one request on one XCD:
// consecutive workgroup ids are dispatched round-robin over the 8 XCDs, so the
// id is decomposed as (xcd = id % 8, k = id / 8) and each XCD takes a
// contiguous range of work items.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int x = id & 7, k = id >> 3;
  const int q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + k;
}

// ----------------------------------------------------------------------------
// Split kernel.  256 threads = 4 waves; wave w owns heads 16w..16w+15 of the
// request and walks all tiles of the workgroup's top-k chunk.
//
// Per 32-token tile, per wave:
//   S^T[32 tok][16 heads] = K[32][576] . Q^T   (2 x 18 MFMA 16x16x32 bf16)
//     K operand: lane (token l%16, group g) holds dims 32c+8g..+7 of its row,
//     fp8 codes converted exactly to bf16; fp8 block scales multiply the fp32
//     partial of each 128-dim block.
//   online softmax in the log2 domain, per head (lane column l%16).
//   O^T[512 d][16 heads] += V^T[512][32 tok] . P^T   (32 MFMA 16x16x32 bf16)
//     V^T operand: one ds_read_tr8_b64 (fp8) / two ds_read_tr16_b64 (bf16)
//     gives lane (d l%16, group g) the 8 tokens of its k-slots; fp8 block
//     scales are folded into P (one bf16 P operand per 128-dim block).
// k-slot i of lane group g maps to token tok(g,i) = (i<4) ? 4g+i : 16+4g+i-4,
// which is exactly where the S^T accumulators of the two 16-token halves hold
// them, so P never leaves registers.
template <int FMT>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(SplitArgs a) {
  constexpr int kRow = RowFmt<FMT>::kRow;
  constexpr int kNbuf = RowFmt<FMT>::kNbuf;
  constexpr int kTileBytes = kTile * kRow;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[kNbuf * kTileBytes];
  __shared__ int64_t slot_s[kTopk];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4;          // row group of MFMA layouts
  const int c16 = lane & 15;        // column within a 16-wide MFMA tile

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int b = w / a.nsplit;
  const int s = w - b * a.nsplit;
  const int tile0 = s * a.chunk_tiles;
  if (tile0 >= kTopk / kTile) return;   // empty split (host never launches one)
  const int ntiles = min(a.chunk_tiles, kTopk / kTile - tile0);
  const int ntok = ntiles * kTile;
  const int ctx = a.ctx_len[b];

  // 1. index translation for the whole chunk
  for (int t = threadIdx.x; t < ntok; t += kThreads)
    slot_s[t] = translate(a.page_table, a.topk_idx, ctx, b, tile0 * kTile + t, a.max_pages,
                          a.pool_pages);

  // 2. Q^T fragment of this wave's 16 heads: 18 chunks of 32 dims, 8 per lane
  const int head = wave * 16 + c16;
  const uint16_t* qrow = a.q + ((int64_t)b * kHeads + head) * kDqk;
  bf16x8 qf[18];
#pragma unroll
  for (int c = 0; c < 18; ++c)
    qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c + 8 * g);

  lds_barrier();

  // 3. prefetch the first tiles
  const int npre = min(kNbuf, ntiles);
  for (int tt = 0; tt < npre; ++tt)
    issue_tile<FMT>(a.pool, (const int64_t LDS_AS*)slot_s, tt * kTile,
                    (uint8_t LDS_AS*)(tiles + tt * kTileBytes), wave, lane);

  const int dma_per_tile = DmaCount<FMT>::of(wave);

  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max (log2 domain), per head = lane column
  float l_run = 0.f;         // this lane's share of the running sum

  for (int tt = 0; tt < ntiles; ++tt) {
    const int issued = min(ntiles, kNbuf + tt);
    wait_vmcnt_rt((issued - tt - 1) * dma_per_tile);
    lds_barrier();

    const uint8_t* tb = tiles + (tt % kNbuf) * kTileBytes;
    const int tok_base = tt * kTile;

    // ---- scores S^T for the two 16-token halves
    f32x4 sacc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* krow = tb + (16 * m + c16) * kRow;
      f32x4 sm = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FMT == kFmtFp8) {
        float4 scl[4];     // block scales of tokens 16m + 4g + i
#pragma unroll
        for (int i = 0; i < 4; ++i)
          scl[i] = *reinterpret_cast<const float4*>(tb + (16 * m + 4 * g + i) * kRow + kDl);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const int c = blk * 4 + c4;
            const uint64_t raw = *reinterpret_cast<const uint64_t*>(krow + 32 * c + 8 * g);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(raw), qf[c], acc, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) sm[i] += acc[i] * (&scl[i].x)[blk];
        }
#pragma unroll
        for (int c = 16; c < 18; ++c) {
          const bf16x8 kr = *reinterpret_cast<const bf16x8*>(krow + kDl + 16 + 2 * (32 * (c - 16) + 8 * g));
          sm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, qf[c], sm, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 18; ++c) {
          const bf16x8 kr = *reinterpret_cast<const bf16x8*>(krow + 2 * (32 * c + 8 * g));
          sm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, qf[c], sm, 0, 0, 0);
        }
      }
      sacc[m] = sm;
    }

    // ---- online softmax (log2 domain); masked slots score -inf
    float p[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tok_base + 16 * m + 4 * g + i;
        const float v = slot_s[t] >= 0 ? sacc[m][i] * a.scale_log2 : -INFINITY;
        p[4 * m + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = wave_max16(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);   // 0 while nothing seen, 1 if max unchanged
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = exp2f(p[i] - m_use);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] *= alpha;
    }

    // ---- P^T operands (fp8: one per 128-dim block with its scales folded in)
    constexpr int kNP = (FMT == kFmtFp8) ? 4 : 1;
    bf16x8 pb[kNP];
    if constexpr (FMT == kFmtFp8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 sv = *reinterpret_cast<const float4*>(
            tb + (16 * (i >> 2) + 4 * g + (i & 3)) * kRow + kDl);
        pb[0][i] = (__bf16)(p[i] * sv.x);
        pb[1][i] = (__bf16)(p[i] * sv.y);
        pb[2][i] = (__bf16)(p[i] * sv.z);
        pb[3][i] = (__bf16)(p[i] * sv.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[0][i] = (__bf16)p[i];
    }

    // ---- O^T += V^T P^T over the 32 d-tiles
    if constexpr (FMT == kFmtFp8) {
      // source lane (2k + half) of a group supplies 8 bytes of token tok(g,k)
      const int kk = c16 >> 1, half = c16 & 1;
      const int tok = (kk < 4) ? (4 * g + kk) : (16 + 4 * g + kk - 4);
      const uint8_t* vsrc = tb + tok * kRow + 8 * half;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 LDS_AS*)(vsrc + 16 * dt));
        const uint64_t r64 = (uint64_t)(uint32_t)raw[0] | ((uint64_t)(uint32_t)raw[1] << 32);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(r64), pb[dt >> 3], o[dt], 0, 0, 0);
      }
    } else {
      // source lane (4k + q) of a group supplies 4 elements of token tok(g,k) / tok(g,4+k)
      const int kk = c16 >> 2, qd = c16 & 3;
      const uint8_t* v0 = tb + (4 * g + kk) * kRow + 8 * qd;
      const uint8_t* v1 = tb + (16 + 4 * g + kk) * kRow + 8 * qd;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(v0 + 32 * dt));
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(v1 + 32 * dt));
        // whole-vector bit casts: element-wise short -> __bf16 casts of this
        // result were mis-lowered (the upper dword was dropped)
        const i32x2 a0 = __builtin_bit_cast(i32x2, r0);
        const i32x2 a1 = __builtin_bit_cast(i32x2, r1);
        const i32x4 packed = {a0[0], a0[1], a1[0], a1[1]};
        const bf16x8 va = __builtin_bit_cast(bf16x8, packed);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[0], o[dt], 0, 0, 0);
      }
    }

    // ---- refill this buffer with tile tt + kNbuf
    if (tt + kNbuf < ntiles) {
      lds_barrier();
      issue_tile<FMT>(a.pool, (const int64_t LDS_AS*)slot_s, (tt + kNbuf) * kTile,
                      (uint8_t LDS_AS*)(tiles + (tt % kNbuf) * kTileBytes), wave, lane);
    }
  }

  // ---- finish: normalise and write
  const float L = wave_sum16(l_run);
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const float lse_v = L > 0.f ? (m_run + log2f(L)) * kLn2 : -INFINITY;
  // lane holds O^T[d = 16dt + 4g + i][head]
  if (a.nsplit == 1) {
    uint16_t* orow = a.out + ((int64_t)b * kHeads + head) * kDv;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[dt][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[dt][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[dt][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = make_uint2(lo, hi);
    }
    if (g == 0) a.lse[(int64_t)b * kHeads + head] = lse_v;
  } else {
    float* prow = a.part_o + (((int64_t)b * a.nsplit + s) * kHeads + head) * kDv;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *reinterpret_cast<float4*>(prow + 16 * dt + 4 * g) =
          make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (g == 0) a.part_lse[((int64_t)b * a.nsplit + s) * kHeads + head] = lse_v;
  }
}

// ----------------------------------------------------------------------------
// Combine: out[b,h,:] = sum_s w_s O_s / sum_s w_s with w_s = exp(lse_s - M),
// lse = M + ln sum_s w_s; all splits empty -> out 0, lse -inf.
// One 128-thread block per (request, head); thread t owns dims 4t..4t+3.
__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
  const int bh = blockIdx.x;                 // b * 64 + h
  const int b = bh >> 6, h = bh & 63;
  const float* lse_s = a.part_lse + (int64_t)b * a.nsplit * kHeads + h;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, lse_s[s * kHeads]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      const float ls = lse_s[s * kHeads];
      if (ls == -INFINITY) continue;
      const float wgt = __expf(ls - M);
      wsum += wgt;
      const float4 v = *reinterpret_cast<const float4*>(
          a.part_o + (((int64_t)b * a.nsplit + s) * kHeads + h) * kDv + 4 * threadIdx.x);
      acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  uint16_t* orow = a.out + ((int64_t)b * kHeads + h) * kDv + 4 * threadIdx.x;
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc.x * inv) | ((uint32_t)f32_to_bf16_rne(acc.y * inv) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc.z * inv) | ((uint32_t)f32_to_bf16_rne(acc.w * inv) << 16);
  *reinterpret_cast<uint2*>(orow) = make_uint2(lo, hi);
  if (threadIdx.x == 0) a.lse[(int64_t)b * kHeads + h] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
}

// ----------------------------------------------------------------------------
// Gather hook: one 64-thread block per (request, top-k slot).
template <int FMT>
__global__ __launch_bounds__(64) void gather_kernel(GatherArgs a) {
  constexpr int kRow = RowFmt<FMT>::kRow;
  const int j = blockIdx.x & (kTopk - 1);
  const int b = blockIdx.x >> 9;
  const int64_t slot = translate(a.page_table, a.topk_idx, a.ctx_len[b], b, j, a.max_pages, a.pool_pages);
  if (threadIdx.x == 0) a.slots[(int64_t)b * kTopk + j] = slot;
  uint8_t* dst = a.rows + ((int64_t)b * kTopk + j) * kRow;
  const uint8_t* src = slot >= 0 ? a.pool + slot * kRow : g_zero_row;
  for (int c = threadIdx.x; c < kRow / 16; c += 64)
    *reinterpret_cast<uint4*>(dst + 16 * c) = *reinterpret_cast<const uint4*>(src + 16 * c);
}

// ----------------------------------------------------------------------------
// Launchers (host side).
hipError_t launch_split(const SplitArgs& a, int fmt, int nblocks, hipStream_t stream) {
  if (fmt == kFmtFp8)
    hipLaunchKernelGGL(split_kernel<kFmtFp8>, dim3(nblocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(split_kernel<kFmtBf16>, dim3(nblocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(B * kHeads), dim3(128), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, int fmt, int B, hipStream_t stream) {
  if (fmt == kFmtFp8)
    hipLaunchKernelGGL(gather_kernel<kFmtFp8>, dim3(B * kTopk), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(gather_kernel<kFmtBf16>, dim3(B * kTopk), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smla
