// smla_kernels.hip -- gfx950 kernels of the sparse-MLA decode path.
//
//   split kernel   : per (request, head group of 32, top-k split): translate
//                    top-k indices to cache slots, gather the selected rows into
//                    LDS (register-staged loads), QK^T on fp8 MFMA (cache codes
//                    against Q as fp8 hi + lo; bf16 MFMA for the rope and for
//                    bf16 rows), online softmax, PV on bf16 MFMA, and write a
//                    normalised partial (O, lse) -- or the final output when the
//                    request is not split; optionally the splits merge in the
//                    same launch (the last split to finish, or every split a
//                    share once all have written).
//   combine kernel : log-sum-exp merge of the partials of each (request, head).
//   gather kernel  : the translation + gather stage alone (test hook).
//
// The split-K structure and the online-softmax merge follow "The 64-Block
// Barrier" (section "The Split-K Prescription") and "The Commit That Rewrote
// the Bottleneck" (section "The Levers"); the tiling below is designed for
// CDNA4 (64-wide waves, 16x16x128 fp8 and 32x32x16 bf16 MFMA, 160 KiB LDS, LDS
// transpose reads).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

// Source of masked rows: reading zeros keeps every MFMA operand finite.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kRowBytesBf16];

typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kPRow = 24;        // bf16 per P^T row in LDS (16 tokens + 8 pad: 48-byte rows, so the
                                 // 16-byte reads of 16 consecutive lanes hit distinct banks)

template <int FMT> struct RowFmt;
template <> struct RowFmt<kFmtFp8> {
  static constexpr int kRow = kRowBytesFp8;   // 512 e4m3 | 16 B scales | 128 B rope
  static constexpr int kNbuf = 4;             // 4 x 20,992 B of LDS tiles
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

// One direct-to-LDS load: 16 bytes per lane from `src` to LDS address
// lds_base + 16 * lane.  Written as inline asm on purpose: the compiler treats
// its builtin form as an LDS store that may alias every later LDS read and
// then waits for all outstanding loads (including prefetched tiles) before
// each read.  Completion is tracked explicitly with s_waitcnt vmcnt plus a
// workgroup barrier before any wave reads the tile.  No "memory" clobber:
// the asm is volatile (kept in order with barriers and other asm), and
// leaving ordinary loads free to move lets the row addresses of a whole tile
// be read from LDS before the first load is issued.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))   // wave-uniform
      : "m0");
}

// Layout of a tile (kTile = 32 rows of kRow bytes) in LDS: the rows packed
// one after another, exactly as they sit in a cache row, so slot s (16 bytes)
// holds chunk s % kChunksRow of row s / kChunksRow.  Each direct-to-LDS
// instruction fills 64 consecutive slots, so its 64 lanes read one to three
// rows' contiguous bytes: few cache lines per instruction, which is what sets
// the gather rate of a compute unit (a layout where one instruction touched
// 16 rows x 64 bytes gathered 2.4x slower on L2 hits).  The operand reads of
// the QK and PV waves run at nearly the rate of a contiguous layout on this
// row stride (656 = 164 dwords: the 16 rows a 16-lane group reads fall on
// distinct bank quads).
template <int FMT> struct TileLayout {
  static constexpr int kChunksRow = RowFmt<FMT>::kRow / 16;   // 41 (fp8) or 72 (bf16)
  static constexpr int kSlots = kTile * kChunksRow;
  static constexpr int kInstr = (kSlots + 63) / 64;           // 21 (fp8; the last one half full) or 36
  __device__ static constexpr uint32_t off(int row, int chunk) {   // byte offset in the tile
    return (uint32_t)(row * RowFmt<FMT>::kRow + 16 * chunk);
  }
};

// Issue the direct-to-LDS loads of one tile.  Instruction j fills slots
// 64j .. 64j + 63: lane l reads chunk (64j + l) % kChunksRow of row
// (64j + l) / kChunksRow from that row's address (the zero row when the slot
// is masked; bit 0 of the stored address marks that).  With NW issuing
// waves, wave v (0 .. NW-1) takes instructions v, v + NW, ...; its count per
// tile is DmaCount<FMT, NW>::of(v).
// TileSrc holds the wave's per-lane source addresses of one tile, read from
// LDS a tile ahead of the loads (lanes past the last slot hold 0 and issue
// nothing).
template <int FMT, int NW> struct DmaCount {
  static constexpr int kInstr = TileLayout<FMT>::kInstr;
  // issuing wave v (0 .. NW-1) takes instructions v, v + NW, ...
  __host__ __device__ static constexpr int of(int v) { return (kInstr - v + NW - 1) / NW; }
  // waves 0 .. kRichWaves-1 issue of(0) loads per tile, the rest of(NW - 1)
  static constexpr int kRichWaves = (kInstr % NW == 0) ? NW : kInstr % NW;
  static constexpr int kPerWave = of(0);
  static constexpr int kPoor = of(NW - 1);
  __device__ static constexpr int per(int v) { return v < kRichWaves ? kPerWave : kPoor; }
};

template <int FMT, int NW> struct TileSrc {
  uint64_t a[DmaCount<FMT, NW>::kPerWave];   // source of this lane's 16 bytes in instruction v + NW q
};
template <int FMT, int NW>
__device__ __forceinline__ TileSrc<FMT, NW> tile_src(const uint64_t LDS_AS* rowaddr_s, int tok0, int v, int lane) {
  using TL = TileLayout<FMT>;
  TileSrc<FMT, NW> s;
#pragma unroll
  for (int q = 0; q < DmaCount<FMT, NW>::kPerWave; ++q) {
    const int slot = 64 * (v + NW * q) + lane;
    const int row = slot / TL::kChunksRow, chunk = slot - row * TL::kChunksRow;
    s.a[q] = slot < TL::kSlots ? (rowaddr_s[tok0 + row] & ~1ull) + 16 * chunk : 0;
  }
  return s;
}
template <int FMT, int NW>
__device__ __forceinline__ void issue_tile(const TileSrc<FMT, NW>& s, uint8_t LDS_AS* lds, int v, int lane) {
  using TL = TileLayout<FMT>;
#pragma unroll
  for (int q = 0; q < DmaCount<FMT, NW>::kPerWave; ++q) {
    const int j = v + NW * q;
    if (j < TL::kInstr && 64 * j + lane < TL::kSlots)   // the last fp8 instruction fills 32 slots
      dma16((const void*)(uintptr_t)s.a[q], (uint32_t)(uintptr_t)(lds + j * 64 * 16));
  }
}

// Raw V^T operand of one PV MFMA as read from LDS: 8 fp8 codes or 8 bf16.
template <int FMT> struct VRaw { typedef i32x2 type; };
template <> struct VRaw<kFmtBf16> { typedef i32x4 type; };

// s_waitcnt vmcnt(n) with the other counters left unconstrained (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt vmcnt(n) for a wave-uniform n in 0 .. N (the immediate is
// chosen by a chain of scalar compares).
template <int N> __device__ __forceinline__ void wait_vmcnt_le(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) wait_vmcnt<N>();
    else wait_vmcnt_le<N - 1>(n);
  }
}

// Wait until at most `tiles_after` tiles' worth of this wave's loads are
// outstanding (loads complete in issue order), i.e. every earlier tile landed.
template <int PER_TILE>
__device__ __forceinline__ void wait_tiles(int tiles_after) {
  static_assert(3 * PER_TILE < 64, "vmcnt range");
  if (tiles_after >= 3) wait_vmcnt<3 * PER_TILE>();
  else if (tiles_after == 2) wait_vmcnt<2 * PER_TILE>();
  else if (tiles_after == 1) wait_vmcnt<PER_TILE>();
  else wait_vmcnt<0>();
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

// Reductions over lanes l, l^16, l^32, l^48 (the four row groups of a
// 16-wide MFMA tile) with the VALU lane-swap instructions, no LDS round trip.
// v_permlane16_swap_b32 a, b exchanges the odd 16-lane rows of a with the even
// rows of b; with a = b = x it leaves {x[l], x[l^16]} across the pair (a, b)
// in every lane.  v_permlane32_swap_b32 does the same across 32-lane halves.
// Inline asm because the builtin's lowering assumes only the first operand
// changes; s_nop padding covers the VALU-write to permlane-read hazard.
__device__ __forceinline__ void lane_swap16(float v, float& a, float& b) {
  unsigned x = __builtin_bit_cast(unsigned, v), y = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}
__device__ __forceinline__ void lane_swap32(float v, float& a, float& b) {
  unsigned x = __builtin_bit_cast(unsigned, v), y = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float xor16_max(float v) { float a, b; lane_swap16(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float xor32_max(float v) { float a, b; lane_swap32(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float xor16_sum(float v) { float a, b; lane_swap16(v, a, b); return a + b; }
__device__ __forceinline__ float xor32_sum(float v) { float a, b; lane_swap32(v, a, b); return a + b; }
__device__ __forceinline__ float wave_max16(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float wave_sum16(float v) { return xor32_sum(xor16_sum(v)); }

// Workgroup barrier that orders LDS only.  __syncthreads() would also wait for
// every outstanding global load, including the prefetched tiles in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier that orders nothing of this wave's own memory accesses
// (only the compiler's view of them): for a wave that has written no LDS
// since the last barrier, whose LDS reads may then stay in flight across it.
__device__ __forceinline__ void arrive_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Partial results travel between workgroups of one launch that may sit on
// different XCDs, whose L2 caches are not kept coherent with each other.
// Stores and loads carrying device scope (sc1) are made coherent by the
// hardware on their own, so no device-scope fence is needed: such a fence
// writes back or invalidates a whole L2.  Buffer accesses are used so each
// wave moves whole 1 KB runs (write-through at dword or 32-byte granularity
// would flood the memory system with partial-line writes).
constexpr int kSc1 = 16;                     // cache-policy bit: device scope
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The spread merge: a (query set, head group) partial is 64 runs of 1 KB;
// partials are loaded up to 8 splits at a time.
constexpr int kRunsPerGroup = 4 * 4 * 4;
constexpr int kSpreadBatch = 8;
// Wait until every global store this wave issued has completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Layout of one (request, split) partial output, 64 x 512 fp32 = 128 KB, in
// 128 runs of 1 KB.  Run c = ((vb * 4 + db) * 4 + jj) * 2 + hb holds, at
// float4 slot lane = l32 + 32 kg, dims 128vb + 32db + 8jj + 4kg + 0..3 of head
// 32hb + l32: exactly what lane `lane` of the PV wave owning latent slice vb
// keeps in registers 4jj..4jj+3 of accumulator [db][hb].
__device__ __forceinline__ uint32_t part_run_offset(int vb, int db, int jj, int hb, int lane) {
  return ((((vb * 4 + db) * 4 + jj) * 2 + hb) * 256 + lane * 4) * 4;     // bytes
}
constexpr uint32_t kPartBytes = kHeads * kDv * 4;
// Polls of the finished-writes counter before a merging workgroup gives up
// (never reached when every split runs: they are all past their compute).
// The launch passes the limit (SplitArgs::spin_limit, at most kMergeSpinLimit):
// tests force the give-up path with a limit of 0.

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
// Log-sum-exp merge of the nsplit partials of request b by one 512-thread
// workgroup: out = sum_s w_s O_s / sum_s w_s with w_s = exp(lse_s - M),
// M = max_s lse_s, lse = M + ln sum_s w_s; all splits empty -> out 0, lse -inf.
// Thread t owns head t/8 and dims 64(t%8) .. +63.
// Softmax weights of the nsplit partials of one head, written to
// wt[sp * stride] (normalised: they sum to 1), and the merged lse:
//   w_s = exp(lse_s - M) / sum_r exp(lse_r - M),  M = max_s lse_s,
//   lse = M + ln sum_r exp(lse_r - M);  every split empty -> w = 0, lse = -inf.
// Both merge paths call this, so they round identically.
template <class LseOf>
__device__ __forceinline__ float split_weights(int nsplit, LseOf lse_of, float* wt, int stride = kHeads) {
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, lse_of(sp));
  float wsum = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float e = M == -INFINITY ? 0.f : __expf(lse_of(sp) - M);
    wt[sp * stride] = e;
    wsum += e;
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  for (int sp = 0; sp < nsplit; ++sp) wt[sp * stride] *= inv;
  return wsum > 0.f ? M + __logf(wsum) : -INFINITY;
}

__device__ __forceinline__ f32x4 load_run(const float* part_o, int64_t block, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r = buffer_of(part_o + block * (kHeads * kDv), kPartBytes);
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1);
}

// The fused merge of (request b, head group hb) by its last split `own`
// (512 threads).  Its own partial is in LDS (`own_part`, at the offsets it has
// in a workspace block) with its lse in own_lse[h]; the other nsplit - 1
// partials and lses are in the workspace.  Same weights and the same
// split-ordered accumulation as the combine kernel; the lse loads and the
// first partial loads go out together, and each round loads four partials
// other than the own one: one memory round trip when nsplit <= 5.
__device__ __forceinline__ void merge_fused(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                            int nsplit, int b, int hb, int own, const uint8_t* own_part,
                                            const float* own_lse, uint16_t* __restrict__ out, float* __restrict__ lse,
                                            float* wt) {
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, l32 = lane & 31, kg = lane >> 5;
  // waves 0..7 each merge the 16 runs (vb, db0 .. db0 + 1, *); the others only
  // take part in the barriers
  const bool mw = wave < 8;
  const int vb = mw ? wave >> 1 : 0, db0 = 2 * (wave & 1);
  const int nother = nsplit - 1;
  auto other = [&](int k) { return k < own ? k : k + 1; };    // k-th split other than own, ascending
  const float* ls = part_lse + (int64_t)b * nsplit * kHeads + kHpw * hb;

  // lse of every split for the group's 32 heads (one per thread), issued first
  const int sp_l = t >> 5, h_l = t & (kHpw - 1);
  const float lv = sp_l < nsplit ? (sp_l == own ? own_lse[h_l] : load_agent(ls + sp_l * kHeads + h_l)) : 0.f;
  constexpr int kRound = 2;   // partials loaded per round (2 x 32 registers in flight)
  f32x4 v[kRound][2][4];
  auto issue = [&](int k0) {
#pragma unroll
    for (int u = 0; u < kRound; ++u)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[u][i][j] = mw && k0 + u < nother ? load_run(part_o, (int64_t)b * nsplit + other(k0 + u),
                                                        part_run_offset(vb, db0 + i, j, hb, lane))
                                             : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  issue(0);
  if (sp_l < nsplit) wt[t] = lv;
  lds_barrier();
  if (t < kHpw)   // in place, column t
    lse[(int64_t)b * kHeads + kHpw * hb + t] =
        split_weights(nsplit, [&](int sp) { return wt[sp * kHpw + t]; }, wt + t, kHpw);
  lds_barrier();
  if (!mw) return;   // no barrier follows

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto add = [&](int sp, auto&& val) {
    const float w = wt[sp * kHpw + l32];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += w * val(i, j);
  };
  auto own_val = [&](int i, int j) {
    return *reinterpret_cast<const f32x4*>(own_part + part_run_offset(vb, db0 + i, j, hb, lane));
  };
  bool own_done = false;
  for (int k0 = 0; k0 < nother; k0 += kRound) {
    if (k0 > 0) issue(k0);
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      if (k0 + u >= nother) break;
      const int sp = other(k0 + u);
      if (!own_done && own < sp) {
        add(own, own_val);
        own_done = true;
      }
      add(sp, [&](int i, int j) { return v[u][i][j]; });
    }
  }
  if (!own_done) add(own, own_val);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 x = acc[i][j];
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
      uint16_t* orow = out + ((int64_t)b * kHeads + kHpw * hb + l32) * kDv + 128 * vb + 32 * (db0 + i) + 8 * j + 4 * kg;
      *reinterpret_cast<uint2*>(orow) = make_uint2(lo, hi);
    }
}

// The spread merge of (query set vr, head group hg): split `own` of nsplit
// merges runs [64 own / nsplit, 64 (own + 1) / nsplit) of the group's 64
// partial runs (8 dims x 32 heads each) once every split has written its
// partial; the 12 waves take the share's runs in turn.  Same weights and the
// same split-ordered accumulation as the combine kernel, so the bits agree.
// Split 0 writes the merged lse.  A split whose wait gave up (`failed`) writes
// NaN into its share of out and into the group's lse.
__device__ __forceinline__ void merge_spread(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                             int nsplit, int vr, int hg, int own, bool failed,
                                             uint16_t* __restrict__ out, float* __restrict__ lse, float* wt) {
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, l32 = lane & 31, kg = lane >> 5;
  const float* ls = part_lse + (int64_t)vr * nsplit * kHeads + kHpw * hg;
  const int r0 = (kRunsPerGroup * own) / nsplit, r1 = (kRunsPerGroup * (own + 1)) / nsplit;
  // first run of this wave: its loads go out with the lse loads
  const int rw = r0 + wave;
  f32x4 v[kSpreadBatch];
  auto issue = [&](int r, int sp0) {
    const int vb = r >> 4, db = (r >> 2) & 3, jj = r & 3;
#pragma unroll
    for (int u = 0; u < kSpreadBatch; ++u)
      v[u] = r < r1 && sp0 + u < nsplit
                 ? load_run(part_o, (int64_t)vr * nsplit + sp0 + u, part_run_offset(vb, db, jj, hg, lane))
                 : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  issue(rw, 0);
  const float lv = t < nsplit * kHpw ? load_agent(ls + (t >> 5) * kHeads + (t & (kHpw - 1))) : 0.f;
  if (t < nsplit * kHpw) wt[t] = lv;
  lds_barrier();
  if (t < kHpw) {   // in place, column t
    const float l = split_weights(nsplit, [&](int sp) { return wt[sp * kHpw + t]; }, wt + t, kHpw);
    if (failed) lse[(int64_t)vr * kHeads + kHpw * hg + t] = __builtin_nanf("");
    else if (own == 0) lse[(int64_t)vr * kHeads + kHpw * hg + t] = l;
  }
  lds_barrier();
  for (int r = rw; r < r1; r += kWaves) {
    if (r != rw) issue(r, 0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < nsplit; sp0 += kSpreadBatch) {
      if (sp0 > 0) issue(r, sp0);
#pragma unroll
      for (int u = 0; u < kSpreadBatch; ++u) {
        if (sp0 + u >= nsplit) break;
        acc += wt[(sp0 + u) * kHpw + l32] * v[u];
      }
    }
    const int vb = r >> 4, db = (r >> 2) & 3, jj = r & 3;
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    uint16_t* orow = out + ((int64_t)vr * kHeads + kHpw * hg + l32) * kDv + 128 * vb + 32 * db + 8 * jj + 4 * kg;
    *reinterpret_cast<uint2*>(orow) = failed ? make_uint2(0x7fc07fc0u, 0x7fc07fc0u) : make_uint2(lo, hi);
  }
}

// The row loads of one split on one loader wave: NT tiles, N 16-byte loads
// per lane and tile (instructions v, v + 4, ... of each tile, as DmaCount
// deals them to 4 waves), staged in registers and written to LDS buffer
// t % NBUF just before the barrier that publishes tile t.  Tile t sits in
// register slot t % S from its load to its write, which frees the slot for
// tile t + S (S = 3 for fp8 rows, 2 for the larger bf16 rows).  Everything is
// unrolled on the compile-time tile count, so the compiler's waits before
// each write count exactly the loads issued after it (loads complete in issue
// order) and the next S - 1 tiles stay in flight.
// Lanes past the tile's last slot (the last fp8 instruction is half full)
// repeat that slot: same source, same bytes, same LDS address.
// Barrier k of the loop follows the write of tile k + 1 (PIPE: the QK waves
// read a tile ahead; tile 0 also before barrier 0) or tile k; NT + 1 barriers
// in all, as every other wave takes.
template <int FMT, int N, int NT, bool PIPE>
__device__ __forceinline__ void load_rows(const uint64_t LDS_AS* rowaddr_s, uint8_t LDS_AS* tiles, int v, int lane) {
  using TL = TileLayout<FMT>;
  constexpr int kNbufR = RowFmt<FMT>::kNbuf;
  constexpr int kTileBytes = kTile * RowFmt<FMT>::kRow;
  constexpr int S = FMT == kFmtFp8 ? 3 : 1;
  u32x4 reg[S][N];
  uint32_t dst[N];   // byte offset of this lane's 16 bytes of instruction q in a tile
#pragma unroll
  for (int q = 0; q < N; ++q) dst[q] = 16u * (uint32_t)min(64 * (v + 4 * q) + lane, TL::kSlots - 1);
  auto load = [&](int t, u32x4 (&d)[N]) {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const int slot = (int)(dst[q] >> 4);
      const int row = slot / TL::kChunksRow, chunk = slot - row * TL::kChunksRow;
      const uint64_t src = (rowaddr_s[t * kTile + row] & ~1ull) + 16 * chunk;
      // non-temporal: each row passes through this CU once (B=80: 0.3-0.5 us faster than plain loads)
      d[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 GLOBAL_AS*>(static_cast<uintptr_t>(src)));
    }
  };
  auto write = [&](int t, const u32x4 (&d)[N]) {
    uint8_t LDS_AS* base = tiles + (t % kNbufR) * kTileBytes;
#pragma unroll
    for (int q = 0; q < N; ++q) *reinterpret_cast<u32x4 LDS_AS*>(base + dst[q]) = d[q];
  };
  // Tiles 0 and 1 go out first; the rest of the first S only after tile 0 is
  // written, so the first write does not queue behind their issue (which
  // stalls while the compute unit's memory path is full).
  constexpr int kPre = NT < (S < 2 ? S : 2) ? NT : (S < 2 ? S : 2);
#pragma unroll
  for (int t = 0; t < kPre; ++t) load(t, reg[t]);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    write(t, reg[t % S]);
    if (t == 0) {
#pragma unroll
      for (int u = kPre; u < (NT < S ? NT : S); ++u) load(u, reg[u]);
    }
    if (t + S < NT) load(t + S, reg[t % S]);
    if (!PIPE || t > 0) lds_barrier();
  }
  // the barriers left: k = NT - 1 and NT (PIPE), or k = NT
  if (PIPE) lds_barrier();
  lds_barrier();
}

// load_rows for loader wave v (0 .. 3) of a split of NT tiles.
template <int FMT, bool PIPE, int NT>
__device__ __forceinline__ void load_rows_nt(const uint64_t LDS_AS* rowaddr_s, uint8_t LDS_AS* tiles, int v, int lane) {
  using Ld = DmaCount<FMT, kLdWaves>;
  if (v < Ld::kRichWaves) load_rows<FMT, Ld::kPerWave, NT, PIPE>(rowaddr_s, tiles, v, lane);
  else load_rows<FMT, Ld::kPoor, NT, PIPE>(rowaddr_s, tiles, v, lane);
}

// ----------------------------------------------------------------------------
// Split kernel.  768 threads = 12 waves, one workgroup per (request, head
// group of 32 heads, split), in three roles; wave w runs on SIMD w % 4:
//
//   QK waves 0..3 own heads 16(w&1)..+15 of the group and token half w>>1 of
//     every 32-token tile: S^T[16 tok][16 heads].
//     fp8 rows: per 128-dim scale block one 16x16x128 fp8 MFMA on the cache
//     codes as stored, against Q * 2^e_h split into fp8 hi + lo parts (e_h the
//     per-head power of two that puts max|q| in (224, 448]); hi + lo
//     reproduces Q * 2^e_h except where the residual falls below the e4m3
//     normal range, which rounds it to the 2^-9 subnormal step (error <= 2^-10
//     scaled, < 4.4e-6 of the head's max |q|).  The block scale multiplies the
//     fp32 block partial; the 64 rope dims use 16x16x32 bf16 MFMA.  bf16 rows:
//     18 bf16 MFMA.  In both operands k-slot g of a block covers dims
//     32g..32g+31, so the products pair the same dims.
//     Online softmax in the log2 domain per head (lane column) and half; the
//     running max is only raised when a tile's max exceeds it by more than
//     2^8, so the output is rarely rescaled (p stays <= 2^8), and the tile's
//     max is reduced across lanes only when some lane's own scores do.  P^T goes to LDS,
//     one bf16 copy per scale block with that block's scales folded in.
//   PV waves 4..7 own latent dims 128v..128v+127 (scale block v = w-4) for
//     the group's 32 heads: O^T[32 d][32 heads] += V^T[32 d][16 tok] .
//     P^T[16 tok][32 heads] per token half, with V^T from ds_read_tr8_b64
//     (fp8, converted exactly to bf16) or ds_read_tr16_b64 (bf16).
//   Loader waves 8..11 move the rows (load_rows).  PV and loader waves first
//     translate the split's top-k indices, one token per thread.
//
// Iteration k of the shared loop: QK waves finish tile k and start tile k+1
// while PV waves accumulate tile k-1; one workgroup barrier per iteration.
// Rows sit in a ring of kNbuf LDS tile buffers, written by the loader waves.
// k-slot i of lane group g holds token tok(g,i) = (i<4) ? 4g+i : 16+4g+i-4,
// which is where the S^T accumulators of the two halves hold them.
template <int FMT>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(SplitArgs a) {
  constexpr int kRow = RowFmt<FMT>::kRow;
  constexpr int kNbuf = RowFmt<FMT>::kNbuf;
  using TL = TileLayout<FMT>;
  constexpr int kTileBytes = kTile * kRow;
  // One LDS block: the tile ring, then P^T.  A merging workgroup reuses its
  // first 128 KB for its own partial output.
  constexpr int kRingBytes = kNbuf * kTileBytes;
  constexpr int kQBytes = kHpw * kDqk * 2;
  constexpr int kQOff = kRingBytes - kQBytes;      // Q staging: the end of the ring
  // P^T copies: one per 128-dim scale block (fp8 rows: P times that block's
  // scale) or a single one (bf16 rows)
  constexpr int kPCopies = FMT == kFmtFp8 ? 4 : 1;
  constexpr int kPBytes = 2 * kPCopies * 2 * kHpw * kPRow * 2;
  constexpr int kSmem = kRingBytes + kPBytes > (int)kPartBytes ? kRingBytes + kPBytes : (int)kPartBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  uint8_t* const tiles = smem;
  __shared__ uint64_t rowaddr_s[kTopk];            // row address | 1 when masked
  __shared__ __attribute__((aligned(16))) float bias_s[kTopk];   // score bias of each slot: 0 valid, -inf masked
  // P^T in bf16, already multiplied by the token's scale of the copy's block:
  // [buffer][copy][16-token half][head][token]
  __bf16 (*const p_s)[kPCopies][2][kHpw][kPRow] =
      reinterpret_cast<__bf16 (*)[kPCopies][2][kHpw][kPRow]>(smem + kRingBytes);
  __shared__ float alpha_s[2][2][kHpw];            // [buffer][half][head]
  __shared__ float mh_s[2][kHpw], lh_s[2][kHpw];   // per half: running max (log2) and sum
  __shared__ int last_s;
  __shared__ int poison_s;                         // the workspace status word was set before this call
  __shared__ float lsev_s[kHpw];                   // this split's lse per head
  __shared__ int fail_s;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4;          // row group of MFMA layouts
  const int c16 = lane & 15;        // column within a 16-wide MFMA tile
  const bool qk_role = wave < kQkWaves;

  // work item -> (request, split, query token, head group).  The q_len query
  // tokens of a request share its selected rows; all 2 * q_len workgroups of
  // one (request, split) are neighbours, so they run on one XCD and all but
  // the first gather the rows from that XCD's L2.  `vr` = (request, query
  // token) indexes everything per query (Q, out, lse, partials, counters);
  // `b` indexes the selection (indices, page table, context length).
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = w & 1;
  const int tq = (w >> 1) % a.q_len;
  const int bs = (w >> 1) / a.q_len;
  const int b = bs / a.nsplit;
  const int s = bs - b * a.nsplit;
  const int vr = b * a.q_len + tq;
  const int tile0 = s * a.chunk_tiles;
  if (tile0 >= kTiles) return;   // empty split (the host never launches one)
  const int ntiles = min(a.chunk_tiles, kTiles - tile0);
  // the loader waves are specialised on these counts (the host only forms
  // splits of 16 / nsplit tiles rounded up, nsplit in 1, 2, 3, 4, 6, 8, 16);
  // any other count leaves the whole workgroup before its first barrier
  if (ntiles != 16 && ntiles != 8 && ntiles != 6 && ntiles != 4 && ntiles != 3 && ntiles != 2 && ntiles != 1)
    return;
  const int ntok = ntiles * kTile;
  const int ctx = a.ctx_len[b];
  const bool fused = a.nsplit > 1 && a.counters != nullptr;   // merge in this launch
  uint32_t* const ctr = fused ? a.counters + 2 * (2 * vr + hg) : nullptr;   // tickets, finished writes

  // ---- 1. QK waves: wave q scores heads 16(q&1) .. +15 of the group against
  // token half q>>1 of every tile (lane column = head)
  const int hq = wave & 1, mh = (wave >> 1) & 1;
  const int hloc = 16 * hq + c16;                          // head within the group
  const int head = kHpw * hg + hloc;                       // head of the request
  // ---- 2. Q and index translation.  The QK waves request their heads' raw
  // Q at once, while the other eight waves translate (one token per thread),
  // so Q streams in during the two dependent index loads instead of sharing
  // the compute unit's memory path with the first tiles.
  if (!qk_role) {
    const int t = threadIdx.x - 64 * kQkWaves;      // token 0 .. 511
    bool valid = false;
    if (t < ntok) {
      const int64_t slot = translate(a.page_table, a.topk_idx, ctx, b, tile0 * kTile + t, a.max_pages,
                                     a.pool_pages);
      valid = slot >= 0;
      rowaddr_s[t] = valid ? (uint64_t)(uintptr_t)(a.pool + slot * kRow)
                           : ((uint64_t)(uintptr_t)g_zero_row | 1ull);
      bias_s[t] = valid ? 0.f : -INFINITY;
    }
    lds_barrier();   // the QK waves take the same barrier in their own branch below
  }
  static_assert(64 * (kPvWaves + kLdWaves) >= kTopk, "the translating waves cover every top-k slot");

  // ---- 3. row loads.  The loader waves alone move the rows: plain global
  // loads into registers, kLdSlots tiles ahead, each tile written to its LDS
  // buffer with ds_write just before the barrier that publishes it.  (A
  // direct-to-LDS load, while the memory path is busy, stalls the LDS reads of
  // the other waves of the compute unit; a register-staged tile costs the LDS
  // one short burst of writes.)  In iteration k the QK waves start tile k+1
  // and finish tile k, and the PV waves accumulate tile k-1 and read the V
  // operands of tile k, so tile k+2 is written during iteration k into the
  // buffer of tile k-2, whose last reads completed before barrier k.  Without
  // the QK look-ahead (bf16 rows: a ring of 3 buffers) tile k+1 is written
  // during iteration k into the buffer of tile k-2.
  const bool ld_role = wave >= kQkWaves + kPvWaves;
  const int lw = ld_role ? wave - kQkWaves - kPvWaves : 0;  // loader 0 .. 3
  constexpr bool kPipe = kNbuf >= 4;

  if (qk_role) {
    // ---------------------------------------------------------------- QK role
    // Q of the group's 32 heads: 36,864 contiguous bytes, brought into the
    // end of the tile ring (written with a tile only after the first loop
    // barrier, by when Q has been read) with contiguous 1 KB direct-to-LDS
    // loads, then read in the MFMA layout.  Loading it straight into the
    // layout would touch ~32 cache lines per instruction, and the two token
    // halves would load the same heads twice.
    {
      static_assert(kQBytes % 1024 == 0 && kQOff % 1024 == 0 && kQOff >= (kPipe ? 2 : 1) * kTileBytes,
                    "Q lies in the buffers written only after the first loop barrier");
      const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + ((int64_t)vr * kHeads + kHpw * hg) * kDqk);
      uint8_t* qlds = tiles + kQOff;
#pragma unroll
      for (int j = wave; j < kQBytes / 1024; j += kQkWaves)
        dma16(qsrc + 1024 * j + 16 * lane, (uint32_t)(uintptr_t)(qlds + 1024 * j));
      wait_vmcnt<0>();
    }
    lds_barrier();   // the translation barrier (the other waves take it in their branch above); Q has landed
    bf16x8 qraw[18];
    {
      const uint8_t* qrow = tiles + kQOff + hloc * (kDqk * 2);
      if constexpr (FMT == kFmtFp8) {
        // latent: 32 dims per lane group per block (4 x 8), rope: 8 dims per chunk
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            qraw[4 * blk + j] = *reinterpret_cast<const bf16x8*>(qrow + 2 * (128 * blk + 32 * g + 8 * j));
      } else {
#pragma unroll
        for (int c = 0; c < 16; ++c)
          qraw[c] = *reinterpret_cast<const bf16x8*>(qrow + 2 * (32 * c + 8 * g));
      }
#pragma unroll
      for (int c = 16; c < 18; ++c)
        qraw[c] = *reinterpret_cast<const bf16x8*>(qrow + 2 * (32 * c + 8 * g));
    }
    i32x8 qhi[FMT == kFmtFp8 ? 4 : 1], qlo[FMT == kFmtFp8 ? 4 : 1];
    bf16x8 qb[18];
    float qscale = 1.0f;           // 2^-e_h, folded into the softmax scale
    if constexpr (FMT == kFmtFp8) {
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qraw[c][e]));
      amax = wave_max16(amax);
      // e_h: largest power of two with amax * 2^e_h <= 448 (the e4m3 maximum)
      int ex = 0;
      if (amax > 0.f) {
        const int E = __builtin_amdgcn_frexp_expf(amax);          // amax = m * 2^E, m in [0.5,1)
        const float mnt = __builtin_amdgcn_frexp_mantf(amax);
        ex = (mnt <= 0.875f) ? 9 - E : 8 - E;
        ex = max(-120, min(120, ex));
      }
      const float up = __builtin_ldexpf(1.0f, ex);
      qscale = __builtin_ldexpf(1.0f, -ex);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float x[4], hf[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (float)qraw[4 * blk + j][4 * h2 + e] * up;
            int hv = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
            hv = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hv, true);
            hf[0] = __builtin_amdgcn_cvt_f32_fp8(hv, 0);
            hf[1] = __builtin_amdgcn_cvt_f32_fp8(hv, 1);
            hf[2] = __builtin_amdgcn_cvt_f32_fp8(hv, 2);
            hf[3] = __builtin_amdgcn_cvt_f32_fp8(hv, 3);
            int lv = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - hf[0], x[1] - hf[1], 0, false);
            lv = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - hf[2], x[3] - hf[3], lv, true);
            qhi[blk][2 * j + h2] = hv;
            qlo[blk][2 * j + h2] = lv;
          }
#pragma unroll
      for (int c = 16; c < 18; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[c][e] = (__bf16)((float)qraw[c][e] * up);   // exact: power of two
    } else {
#pragma unroll
      for (int c = 0; c < 18; ++c) qb[c] = qraw[c];
    }
    const float sc_log2 = a.scale_log2 * qscale;
    float m_run = -INFINITY;        // running max (log2 domain) of this head over this token half
    float l_run = 0.f;              // this lane's share of the running sum
    const int row = 16 * mh + c16;  // tile row this lane's K operand comes from

    // Scores are software-pipelined (fp8 rows): in iteration k the softmax
    // of tile k runs on raw scores whose MFMAs were issued in iteration k-1,
    // while the K operands of tile k+1 are read from LDS; the MFMAs of tile
    // k+1 follow and run into the barrier.  The block scales of tile k are
    // read ahead of tile k+1's K operands, so the softmax waits for them only.
    // Raw holds one tile's accumulators before the fp8 block scales.
    struct Raw {
      f32x4 acc[FMT == kFmtFp8 ? 4 : 1];   // [scale block] (fp8 rows only)
      f32x4 sm;                             // rope part (fp8 rows) or the whole score (bf16 rows)
    };
    struct KOps {                           // K operands of one tile (fp8 rows)
      i32x8 ka[4];                          // codes 128blk + 32g .. +31
      const uint8_t* tb;                    // the tile (its rope dims are read at the MFMAs)
    };
    auto read_k = [&](int kt, KOps& o) {
      const uint8_t* tb = tiles + (kt % kNbuf) * kTileBytes;
      // codes 128blk + 32g .. +31 = chunks 8blk + 2g, +1
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const i32x4 k0 = *reinterpret_cast<const i32x4*>(tb + TL::off(row, 8 * blk + 2 * g));
        const i32x4 k1 = *reinterpret_cast<const i32x4*>(tb + TL::off(row, 8 * blk + 2 * g + 1));
        o.ka[blk] = i32x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      }
      o.tb = tb;
    };
    auto mfma_scores = [&](const KOps& o, Raw& r) {
      // independent MFMA chains: hi of every block, rope, then lo.  The rope
      // dims 32c + 8g .. +7 (byte 528 + 2 (32c + 8g): chunk 33 + 4c + g) are
      // read here, their latency under the hi MFMAs, so they take no
      // registers across the softmax.
      bf16x8 kr[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) kr[c] = *reinterpret_cast<const bf16x8*>(o.tb + TL::off(row, 33 + 4 * c + g));
      f32x4 sm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
        r.acc[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.ka[blk], qhi[blk], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                     0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 2; ++c) sm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[c], qb[16 + c], sm, 0, 0, 0);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
        r.acc[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o.ka[blk], qlo[blk], r.acc[blk], 0, 0, 0, 0, 0, 0);
      r.sm = sm;
    };
    auto issue_scores = [&](int kt, Raw& r) {
      if constexpr (FMT == kFmtBf16) {
        const uint8_t* tb = tiles + (kt % kNbuf) * kTileBytes;
        f32x4 sm = {0.f, 0.f, 0.f, 0.f};
        // k-slot group g of 32-dim step c: dims 32c + 8g .. +7 = chunk 4c + g
#pragma unroll
        for (int c = 0; c < 18; ++c)
          sm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(tb + TL::off(row, 4 * c + g)),
                                                      qb[c], sm, 0, 0, 0);
        r.sm = sm;
      } else {
        KOps o;
        read_k(kt, o);
        mfma_scores(o, r);
      }
    };
    // block scales of this lane's tokens 16mh + 4g + i (fp8 rows)
    auto read_scales = [&](int kt, float4 (&sv)[4]) {
      const uint8_t* tb = tiles + (kt % kNbuf) * kTileBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = *reinterpret_cast<const float4*>(tb + TL::off(16 * mh + 4 * g + i, kDl / 16));
    };
    // softmax of tile kt from its raw scores; P^T and alpha to LDS
    auto finish_tile = [&](int kt, const Raw& r, const float4 (&sv)[4], const float4& bias) {
      f32x4 sacc = r.sm;
      if constexpr (FMT == kFmtFp8) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sacc[i] += r.acc[0][i] * sv[i].x + r.acc[1][i] * sv[i].y + r.acc[2][i] * sv[i].z + r.acc[3][i] * sv[i].w;
      }
      // online softmax (log2 domain) over this half; masked slots score -inf
      float p[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = __builtin_fmaf(sacc[i], sc_log2, (&bias.x)[i]);   // -inf when masked
        p[i] = v;
        tmax = fmaxf(tmax, v);
      }
      float m_cur = m_run;
      float alpha = 1.0f;
      // the head's max over its 16 tokens passes m_cur + 8 exactly when one of
      // its four lanes' own maxima does: reduce across lanes only then
      if (__builtin_amdgcn_ballot_w64(tmax > m_cur + 8.0f)) {
        tmax = wave_max16(tmax);
        const float m_new = (tmax > m_cur + 8.0f) ? tmax : m_cur;
        alpha = __builtin_amdgcn_exp2f(m_cur - m_new);   // 0 when nothing was seen before
        m_cur = m_new;
      }
      const float m_use = (m_cur == -INFINITY) ? 0.f : m_cur;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(p[i] - m_use);
        psum += p[i];
      }
      m_run = m_cur;
      l_run = l_run * alpha + psum;
      // P^T row of this head and half, tokens 4g .. 4g+3, one bf16 copy per
      // scale block with the block's scale folded in (the PV operand as is)
      const int pb = kt & 1;
#pragma unroll
      for (int cp = 0; cp < kPCopies; ++cp) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (__bf16)(FMT == kFmtFp8 ? p[i] * (&sv[i].x)[cp] : p[i]);
        *reinterpret_cast<bf16x4*>(&p_s[pb][cp][mh][hloc][4 * g]) = v;
      }
      if (g == 0) alpha_s[pb][mh][hloc] = alpha;
    };
    // Iteration k finishes tile k (raw scores in `cur`) and starts tile k+1
    // (into `nxt`), between barriers k and k+1.
    auto body = [&](int k, Raw& cur, Raw& nxt) {
      if constexpr (kPipe) {   // (the bf16 ring runs the unpipelined loop below)
        if (k == 0) {
          lds_barrier();
          issue_scores(0, cur);
        }
        float4 sv[4];
        read_scales(k, sv);
        const float4 bias = *reinterpret_cast<const float4*>(&bias_s[k * kTile + 16 * mh + 4 * g]);
        // The K reads and MFMAs of tile k+1 are unconditional so the compiler
        // can count the LDS reads in flight and let the softmax wait for the
        // scales alone; after the last tile they read a stale buffer and the
        // result is dropped.
        KOps ko;
        read_k(k + 1, ko);
        __builtin_amdgcn_sched_barrier(0);   // every read goes out before the softmax waits
        finish_tile(k, cur, sv, bias);
        mfma_scores(ko, nxt);
        lds_barrier();
      }
    };
    Raw ra;   // one buffer: tile k's raw scores are consumed before tile k+1's MFMAs overwrite them
    if constexpr (kPipe) {
      // unrolled by two
#pragma clang loop unroll(disable)
      for (int k = 0; k < ntiles; k += 2) {
        body(k, ra, ra);
        if (k + 1 < ntiles) body(k + 1, ra, ra);
      }
    } else {
#pragma clang loop unroll(disable)
      for (int k = 0; k <= ntiles; ++k) {
        lds_barrier();
        if (k == ntiles) break;
        Raw r;
        issue_scores(k, r);
        float4 sv[4];
        if constexpr (FMT == kFmtFp8) read_scales(k, sv);
        finish_tile(k, r, sv, *reinterpret_cast<const float4*>(&bias_s[k * kTile + 16 * mh + 4 * g]));
      }
    }

    // This split's scores are done (only the PV waves' last tile is left,
    // which waits on nothing): take the arrival ticket of this (request, head
    // group) now, so its latency overlaps that tile.  The holder of the last
    // ticket merges.
    if (fused && threadIdx.x == 0) {
      last_s = !a.spread && __hip_atomic_fetch_add(&ctr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                                (uint32_t)(a.nsplit - 1);
      poison_s = __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    }
    // this half's max and sum of each head for the PV waves
    const float L = wave_sum16(l_run);
    if (g == 0) {
      mh_s[mh][hloc] = m_run;
      lh_s[mh][hloc] = L;
    }
    lds_barrier();
  } else if (ld_role) {
    // ------------------------------------------------------------ loader role
    const uint64_t LDS_AS* ra = (const uint64_t LDS_AS*)rowaddr_s;
    uint8_t LDS_AS* tl = (uint8_t LDS_AS*)smem;
    // a split holds 16 / nsplit tiles rounded up, or the remainder: one of these
    switch (ntiles) {
      case 16: load_rows_nt<FMT, kPipe, 16>(ra, tl, lw, lane); break;
      case 8: load_rows_nt<FMT, kPipe, 8>(ra, tl, lw, lane); break;
      case 6: load_rows_nt<FMT, kPipe, 6>(ra, tl, lw, lane); break;
      case 4: load_rows_nt<FMT, kPipe, 4>(ra, tl, lw, lane); break;
      case 3: load_rows_nt<FMT, kPipe, 3>(ra, tl, lw, lane); break;
      case 2: load_rows_nt<FMT, kPipe, 2>(ra, tl, lw, lane); break;
      default: load_rows_nt<FMT, kPipe, 1>(ra, tl, lw, lane); break;
    }
    lds_barrier();                    // the QK waves publish each half's max and sum
  } else {
    // ---------------------------------------------------------------- PV role
    // 32x32x16 bf16 MFMA: O^T[32 d][32 heads] += V^T[32 d][16 tok] . P^T[16 tok][32 heads],
    // one accumulator per 16-token half (each half has its own running max).
    // Operand lane layout (both): row/col = lane % 32, k = 8 * (lane / 32) + i,
    // so k-slot (lane/32, i) of half kh is token 16kh + 8(lane/32) + i.
    const int vb = wave - kQkWaves;   // scale block / 128-dim slice of the latent
    const int l32 = lane & 31, kg = lane >> 5;
    f32x16 o[4][2];                   // [32-dim block of the slice][token half]
    // zero from an asm statement, so the compiler cannot hoist the zeroing
    // above the role branch and keep 128 registers live through the QK path
    float zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) o[i][j] = zero;

    // V^T operands of the tile accumulated next, as read from LDS: they are
    // read one iteration ahead (tile k at the end of iteration k, after the
    // MFMAs of tile k-1), so their latency hides under the MFMAs and the
    // barrier.  Tile k is published by the barrier of iteration k - 1 (k when
    // unpipelined) and its buffer is reloaded only in iteration k + 2.
    typename VRaw<FMT>::type vnext[2][4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int db = 0; db < 4; ++db) vnext[kh][db] = {};
    auto read_v = [&](int kt) {
      const uint8_t* tb = tiles + (kt % kNbuf) * kTileBytes;
      const int gg = lane >> 4;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          if constexpr (FMT == kFmtFp8) {
            // 16-lane group gg reads tokens 16kh + 8(gg>>1) + 0..7 x dims
            // 32db + 16(gg&1) + 0..15; source lane (2r + half) supplies 8 bytes of row r
            const int r = c16 >> 1, half = c16 & 1;
            const uint8_t* src = tb + TL::off(16 * kh + 8 * (gg >> 1) + r, 8 * vb + 2 * db + (gg & 1)) + 8 * half;
            vnext[kh][db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 LDS_AS*)src);
          } else {
            // two 4-row reads per group: rows 16kh + 8(gg>>1) + 0..3 and + 4..7;
            // source lane (4r + q) supplies 4 elements of row r
            const int r = c16 >> 2, q = c16 & 3;
            // dims 128vb + 32db + 16(gg&1) + 4q .. +3: chunk 16vb + 4db + 2(gg&1) + q/2, byte 8(q&1)
            const int row = 16 * kh + 8 * (gg >> 1) + r, chunk = 16 * vb + 4 * db + 2 * (gg & 1) + (q >> 1);
            const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(tb + TL::off(row, chunk) + 8 * (q & 1)));
            const i16x4 r1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(tb + TL::off(row + 4, chunk) + 8 * (q & 1)));
            // whole-vector bit casts: element-wise short -> __bf16 casts of this
            // result were mis-lowered (the upper dword was dropped)
            const i32x2 a0 = __builtin_bit_cast(i32x2, r0);
            const i32x2 a1 = __builtin_bit_cast(i32x2, r1);
            vnext[kh][db] = i32x4{a0[0], a0[1], a1[0], a1[1]};
          }
        }
    };

    // Iteration 0 has no P yet: it is a warm-up pass through the same loop
    // code on zero operands and an unwritten P buffer (loading the
    // instructions into the cache while the QK waves score tile 0); its
    // accumulators are reset.
#pragma clang loop unroll(disable)
    for (int k = 0; k <= ntiles; ++k) {
      arrive_barrier();
      const bool dry = k == 0;
      const int kt = dry ? 0 : k - 1;   // tile accumulated in this iteration
      const int pb = dry ? 1 : kt & 1;
      // P^T operands per half: 8 tokens 16kh + 8kg + i of head l32, from this
      // slice's copy (the block scale is already in)
      constexpr int kPCopies = FMT == kFmtFp8 ? 4 : 1;
      const int cp = kPCopies == 4 ? vb : 0;
      bf16x8 pv[2];
      float al[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        pv[kh] = *reinterpret_cast<const bf16x8*>(&p_s[pb][cp][kh][l32][8 * kg]);
        al[kh] = alpha_s[pb][kh][l32];
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        if (__builtin_amdgcn_ballot_w64(al[kh] != 1.0f)) {
#pragma unroll
          for (int db = 0; db < 4; ++db) o[db][kh] *= al[kh];
        }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          bf16x8 va;
          if constexpr (FMT == kFmtFp8) {
            const i32x2 raw = vnext[kh][db];
            va = fp8x8_to_bf16((uint64_t)(uint32_t)raw[0] | ((uint64_t)(uint32_t)raw[1] << 32));
          } else {
            va = __builtin_bit_cast(bf16x8, vnext[kh][db]);
          }
          o[db][kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pv[kh], o[db][kh], 0, 0, 0);
        }
      }
      if (dry) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) o[i][j] = f32x16{};
      }
      // V^T of tile k, read one iteration ahead: the reads' latency runs under
      // the barrier and the next P reads.
      if (k < ntiles) read_v(k);
    }

    lds_barrier();                    // QK waves have published each half's max and sum
    // combine the two halves of head l32:
    //   M = max(m0, m1), L = l0 2^(m0-M) + l1 2^(m1-M), out = (O0 2^(m0-M) + O1 2^(m1-M)) / L
    float f[2];
    float lse_v;
    {
      const float m0 = mh_s[0][l32], m1 = mh_s[1][l32];
      const float M = fmaxf(m0, m1);
      const float e0 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
      const float e1 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
      const float Lh = lh_s[0][l32] * e0 + lh_s[1][l32] * e1;
      const float inv = Lh > 0.f ? 1.0f / Lh : 0.f;
      f[0] = e0 * inv;
      f[1] = e1 * inv;
      lse_v = Lh > 0.f ? (M + __builtin_amdgcn_logf(Lh)) * kLn2 : -INFINITY;
    }
    const int ghead = kHpw * hg + l32;
    if (vb == 0 && kg == 0) {
      lsev_s[l32] = lse_v;
      if (a.nsplit == 1) a.lse[(int64_t)vr * kHeads + ghead] = lse_v;
      else if (!(fused && last_s)) store_agent(a.part_lse + ((int64_t)vr * a.nsplit + s) * kHeads + ghead, lse_v);
    }
    // register j of o[db][*] holds O^T[d = 128vb + 32db + 8(j/4) + 4kg + j%4][head l32]
    f32x16 res[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) res[db] = o[db][0] * f[0] + o[db][1] * f[1];
    if (a.nsplit == 1) {
      // this wave's 32 heads x 128 dims go through LDS (the ring is free now),
      // so each store writes 1 KB of whole rows: 4 heads x 256 bytes
      constexpr int kStRow = 128 * 2 + 16;   // bytes per head row, padded off the bank period
      uint8_t* stg = smem + vb * (kHpw * kStRow);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(res[db][4 * jj]) | ((uint32_t)f32_to_bf16_rne(res[db][4 * jj + 1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(res[db][4 * jj + 2]) | ((uint32_t)f32_to_bf16_rne(res[db][4 * jj + 3]) << 16);
          *reinterpret_cast<uint2*>(stg + l32 * kStRow + 2 * (32 * db + 8 * jj + 4 * kg)) = make_uint2(lo, hi);
        }
      uint16_t* obase = a.out + ((int64_t)vr * kHeads + kHpw * hg) * kDv + 128 * vb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = lane + 64 * i, h = c >> 4, pc = c & 15;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + h * kStRow + 16 * pc);
        // non-temporal: nothing in this launch reads the output back
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + (int64_t)h * kDv + 8 * pc));
      }
    } else if (!fused || !last_s) {
      const __amdgpu_buffer_rsrc_t r = buffer_of(a.part_o + ((int64_t)vr * a.nsplit + s) * (kHeads * kDv), kPartBytes);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 v = {res[db][4 * jj], res[db][4 * jj + 1], res[db][4 * jj + 2], res[db][4 * jj + 3]};
          const uint32_t off = part_run_offset(vb, db, jj, hg, lane);
          if (fused)   // read back in this launch, possibly on another XCD
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kSc1);
          else         // read by the combine launch
            __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
        }
    } else {
      // last split of this (request, head group): its own partial goes to
      // LDS, at the offsets it has in a workspace block
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(smem + part_run_offset(vb, db, jj, hg, lane)) =
              f32x4{res[db][4 * jj], res[db][4 * jj + 1], res[db][4 * jj + 2], res[db][4 * jj + 3]};
    }
  }

  // ---- fused merge
  if (!fused) return;
  if (poison_s) {
    // An earlier merge on this workspace gave up and left its counters off, so
    // no split can tell whether it is the last: lse is NaN (out is left as
    // is) until smla_workspace_init clears the workspace.
    if (threadIdx.x < kHpw) a.lse[(int64_t)vr * kHeads + kHpw * hg + threadIdx.x] = __builtin_nanf("");
    return;
  }
  if (a.spread) {
    // Every split merges a share once all have written: count this split's
    // arrival, wait (bounded) for the others, then count it as done waiting.
    // The split that finds every other done resets both counters: by then no
    // split is still polling.  (All splits of the launch are resident at
    // once: the host forms this plan only for grids of at most one
    // workgroup per compute unit.)
    wait_stores();
    lds_barrier();
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(&ctr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool done = false;
      for (int it = 0; it < a.spin_limit && !done; ++it) {
        done = __hip_atomic_load(&ctr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)a.nsplit;
        if (!done) __builtin_amdgcn_s_sleep(2);
      }
      if (!done) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(&ctr[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          (uint32_t)(a.nsplit - 1)) {
        __hip_atomic_store(&ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      fail_s = done ? 0 : 1;
    }
    lds_barrier();
    merge_spread(a.part_o, a.part_lse, a.nsplit, vr, hg, s, fail_s != 0, a.out, a.lse,
                 reinterpret_cast<float*>(rowaddr_s));
    return;
  }
  if (!last_s) {
    wait_stores();                       // this wave's partial stores have completed ...
    lds_barrier();                       // ... and so have every other wave's
    if (threadIdx.x == 0) __hip_atomic_fetch_add(&ctr[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // Last ticket: wait until the splits with earlier tickets (all resident and
  // past their compute) have finished writing, then merge with all 8 waves,
  // this split's own partial and lse read from LDS.
  if (threadIdx.x == 0) {
    bool done = false;
    for (int it = 0; it < a.spin_limit && !done; ++it) {
      done = __hip_atomic_load(&ctr[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)(a.nsplit - 1);
      if (!done) __builtin_amdgcn_s_sleep(2);
    }
    if (done) {
      ctr[0] = 0u;                       // both counters back to zero for the next call
      ctr[1] = 0u;
    } else {
      // gave up: the counters stay as they are (a straggler may still add to
      // them) and the status word marks the workspace for later calls
      __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    fail_s = done ? 0 : 1;
  }
  lds_barrier();
  merge_fused(a.part_o, a.part_lse, a.nsplit, vr, hg, s, smem, lsev_s, a.out, a.lse,
              reinterpret_cast<float*>(rowaddr_s));
  if (fail_s && threadIdx.x < kHpw) a.lse[(int64_t)vr * kHeads + kHpw * hg + threadIdx.x] = __builtin_nanf("");
}

// ----------------------------------------------------------------------------
// Combine as a launch of its own, spread over the device: one single-wave
// workgroup per (query set, latent slice vb, 32-head block hb, 32-dim block
// db), which merges the four runs (vb, db, jj, hb), so a query set's partials
// are read through 32 compute units.  Every split's runs are requested before
// the weights are known, up to kCombineBatch splits at once.  Weights come from
// split_weights and the runs are accumulated in split order, exactly as the
// fused merge does, so both give identical bits.
constexpr int kCombineThreads = 64;
constexpr int kCombineBatch = 8;
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  __shared__ float wt[16 * 32];
  const int b = blockIdx.x >> 5, vb = (blockIdx.x >> 3) & 3, hb = (blockIdx.x >> 2) & 1, db = blockIdx.x & 3;
  const int lane = threadIdx.x, l32 = lane & 31, kg = lane >> 5;
  const int ns = a.nsplit;
  const float* ls = a.part_lse + (int64_t)b * ns * kHeads + 32 * hb;
  // the lse loads (at most 8 per lane) and the first batch of runs go out
  // together: the weights are computed while the runs are in flight
  float lv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = lane + u * kCombineThreads;
    lv[u] = i < ns * 32 ? load_agent(ls + (i >> 5) * kHeads + (i & 31)) : 0.f;
  }
  f32x4 v[kCombineBatch][4];
  auto issue = [&](int sp) {
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[u][j] = sp + u < ns ? load_run(a.part_o, (int64_t)b * ns + sp + u, part_run_offset(vb, db, j, hb, lane))
                              : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  issue(0);
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (lane + u * kCombineThreads < ns * 32) wt[lane + u * kCombineThreads] = lv[u];
  __syncthreads();
  if (lane < 32) {   // in place, column lane: the lse of head 32hb + lane
    const float l = split_weights(ns, [&](int sp) { return wt[sp * 32 + lane]; }, wt + lane, 32);
    if (vb == 0 && db == 0) a.lse[(int64_t)b * kHeads + 32 * hb + lane] = l;
  }
  __syncthreads();
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < ns; sp += kCombineBatch) {
    if (sp > 0) issue(sp);
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (sp + u >= ns) break;
      const float w = wt[(sp + u) * 32 + l32];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += w * v[u][j];
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 x = acc[j];
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
    uint16_t* orow = a.out + ((int64_t)b * kHeads + 32 * hb + l32) * kDv + 128 * vb + 32 * db + 8 * j + 4 * kg;
    *reinterpret_cast<uint2*>(orow) = make_uint2(lo, hi);
  }
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
// Fill kernel that zeroes a counter array (used instead of a memset so that a
// captured graph holds only kernel nodes).
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
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
  hipLaunchKernelGGL(combine_kernel, dim3(B * 32), dim3(kCombineThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_zero(uint32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
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
