/*
 * sparse_mla.h -- C ABI of libsparse_mla.so: sparse-MLA decode attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (DeepSeek-V4-Flash decode attention as the pages describe it):
 * each request has 64 query heads; an indexer has selected up to 512 token
 * positions ("index_topk = 512") of a paged latent KV cache; every head
 * attends over those selected rows only ("Inside the Decode Performance
 * Investigation ...", section "The Setup"; "The 64-Block Barrier ...",
 * section "The Smoking Gun": gather, matrix-vector multiply, accumulation over
 * the 512 top-k tokens).  The work is split across the top-k dimension and the
 * partial results are merged with an online-softmax (log-sum-exp) combine
 * ("The 64-Block Barrier", section "The Split-K Prescription"; "The Commit That
 * Rewrote the Bottleneck", section "The Levers").
 *
 * Definition computed (per request b, head h), with x_t the dequantised
 * 576-dim cache row of selected token t (512 latent + 64 rope) and v_t its
 * 512 latent dims:
 *     s_t = scale * <q[b,h,:], x_t>
 *     out[b,h,:] = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m),   m = max_t s_t
 *     lse[b,h]   = ln sum_t exp(s_t)           (natural log of scaled scores)
 *     no selected token: out = 0, lse = -inf.
 *
 * Several query tokens per request (q_len = 2..4, e.g. the draft tokens of a
 * multi-token verify step) share the request's selection: every (query token,
 * head) row attends over the same selected rows, which are gathered once per
 * request and split.  The pages trace the split-K structure back to a verify
 * attention kernel ("The 64-Block Barrier", section "The Smoking Gun") and
 * name multi-token (MTP) verification ("Inside the Decode Performance
 * Investigation", section "Task 3") without defining how draft tokens'
 * selections relate; sharing one selection is the reading taken here.  With
 * q_len > 1, q, out and lse gain a query-token dimension after the request.
 *
 * Memory conventions (all pointers are caller-owned):
 *   - Device pointers are marked [device]; they must be valid on the current
 *     HIP device.  Host pointers are marked [host].
 *   - All arrays are dense, row-major, without padding.
 *   - Nothing is allocated per call.  Calls are asynchronous and ordered on
 *     `stream` (a hipStream_t; NULL = the default stream); on success the host
 *     does not wait for the GPU.  Inputs are only read.
 *   - Errors are detected before any launch and leave every output untouched.
 *     No C++ exception crosses this interface.
 *   - The library keeps no per-call state; concurrent calls on different
 *     streams are safe when their output and workspace buffers are disjoint.
 *   - Out-of-range top-k indices and page ids are not errors: their slots are
 *     masked.  Validate mode (environment SMLA_VALIDATE=1, read at every call)
 *     is for tests and debugging.  sparse_mla_decode, smla_decode_split and
 *     smla_gather_rows then first run a check kernel and wait for it on
 *     `stream`.  They return SMLA_ERR_INDEX, launching nothing else, when an
 *     entry other than -1 would be masked.  Calls in validate mode share one
 *     device flag: they must not overlap, and cannot be graph-captured.
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed problem constants (the pages: 64 query heads, index_topk = 512). */
#define SMLA_NUM_HEADS 64
#define SMLA_D_QK 576       /* 512 latent + 64 rope                        */
#define SMLA_D_V 512        /* values are the latent dims                  */
#define SMLA_TOPK 512
#define SMLA_PAGE_SIZE 64   /* tokens per cache page                       */

/* Cache row formats.  The pool is a flat array of rows; physical page p
 * holds rows p*64 .. p*64+63 (slot = page*64 + row). */
typedef enum {
    SMLA_KV_BF16 = 0,          /* 576 bf16: latent d0..d511, rope r0..r63 (1152 B)          */
    SMLA_KV_FP8_E4M3_B128 = 1  /* 512 OCP e4m3fn codes | 4 fp32 scales (scale j covers
                                  dims 128j..128j+127, little-endian) | 64 bf16 rope (656 B) */
} smla_kv_format;

/* Return codes. */
#define SMLA_OK 0
#define SMLA_ERR_INVALID_ARG (-1)       /* null pointer, negative size, bad enum           */
#define SMLA_ERR_UNSUPPORTED_SHAPE (-2) /* heads != 64, d != 576/512, topk != 512, page != 64, q_len > 4 */
#define SMLA_ERR_WORKSPACE (-3)         /* workspace NULL or smaller than smla_plan_for says */
#define SMLA_ERR_PLAN (-4)              /* an override plan outside the supported values    */
#define SMLA_ERR_HIP (-5)               /* a HIP runtime call failed                        */
#define SMLA_ERR_INDEX (-6)             /* validate mode only: a top-k index other than -1  */
                                        /* outside [0, ctx_len), past the page-table row,   */
                                        /* or on a page id outside [0, pool_pages)          */
#define SMLA_ERR_MERGE (-7)             /* validate mode only: an in-kernel split merge gave */
                                        /* up waiting (workspace status word set; see       */
                                        /* sparse_mla_decode): smla_workspace_init needed   */

typedef struct {
    int32_t batch;             /* B >= 0 requests                                   */
    int32_t num_heads;         /* must be 64                                        */
    int32_t d_qk;              /* must be 576                                       */
    int32_t d_v;               /* must be 512                                       */
    int32_t topk;              /* must be 512                                       */
    int32_t page_size;         /* must be 64                                        */
    int32_t max_pages_per_req; /* >= 1: row stride of page_table                    */
    int32_t kv_format;         /* smla_kv_format                                    */
    int64_t pool_pages;        /* >= 1: pages in kv_pool                            */
    int32_t q_len;             /* query tokens per request, 1..4 (0 reads as 1)     */
} smla_shape;

/* Where the split partials are merged (smla_plan.merge). */
#define SMLA_MERGE_AUTO 0      /* in a plan passed in: let the selector choose; in a plan
                                  returned: nothing to merge (nsplit = 1)                  */
#define SMLA_MERGE_IN_KERNEL 1 /* the last split of each request to finish merges them, in
                                  the same launch; only for batch * q_len <= 4096 (a plan
                                  forcing it beyond that returns SMLA_ERR_PLAN)            */
#define SMLA_MERGE_SEPARATE 2  /* a second launch: the combine kernel                      */
#define SMLA_MERGE_SPREAD 3    /* the same launch: once every split of a request has written
                                  its partial, each merges an equal share of the dims; only
                                  when every workgroup of the launch is resident at once
                                  (batch * q_len * 2 * nsplit <= compute units; the selector
                                  picks it itself only up to half of them) and for
                                  batch * q_len <= 4096 (a plan forcing it otherwise returns
                                  SMLA_ERR_PLAN)                                           */

/* Launch plan.  Zero fields mean "choose automatically". */
typedef struct {
    int32_t nsplit;       /* top-k splits per request (1..16); 1 = no partials, no merge  */
    int32_t tile_tokens;  /* tokens per pipeline tile (only 32 is supported)              */
    int32_t heads_per_wg; /* query heads per workgroup (only 32 is supported: two head  */
                          /* groups per request gather the same rows)                  */
    int32_t wg_per_cu;    /* resident workgroups per compute unit assumed by the selector */
    int32_t merge;        /* SMLA_MERGE_*                                                 */
} smla_plan;

/*
 * smla_plan_for -- choose the launch plan for `shape` on the current device and
 * report the workspace the decode call needs.
 *   shape            [host] problem description (validated as in sparse_mla_decode)
 *   override_or_null [host] non-zero fields force those plan values (tests, sweeps)
 *   out              [host] receives the complete plan
 *   workspace_bytes  [host] receives the bytes sparse_mla_decode needs (0 if nsplit = 1)
 * The plan depends only on the shape and the device, never on tensor contents,
 * so a call sequence can be captured into a HIP graph.
 * The split count follows the pages' lever of choosing NSPLIT so the grid fills
 * whole dispatch rounds ("Inside the Decode Performance Investigation",
 * section "Task 1"; "The Commit That Rewrote the Bottleneck", section "The
 * Levers"), with this device's compute-unit count.
 */
int smla_plan_for(const smla_shape* shape, const smla_plan* override_or_null, smla_plan* out,
                  size_t* workspace_bytes);

/*
 * smla_plan_for_cus -- smla_plan_for for a device with `num_cus` compute units,
 * without touching the GPU (host-only; used by tests and planning tools).
 */
int smla_plan_for_cus(const smla_shape* shape, const smla_plan* override_or_null, int num_cus,
                      smla_plan* out, size_t* workspace_bytes);

/*
 * sparse_mla_decode -- the attention defined at the top of this header.
 *   q          [device] bf16 [B, q_len, 64, 576]
 *   kv_pool    [device] u8   [pool_pages * 64 * row_bytes]  (row format = shape->kv_format)
 *   page_table [device] i32  [B, max_pages_per_req]: logical page -> physical page
 *   topk_idx   [device] i32  [B, 512]: logical token positions.  A slot is masked
 *                              (contributes nothing) when its index is outside
 *                              [0, ctx_len[b]), when index/64 >= max_pages_per_req, or
 *                              when its page id is outside [0, pool_pages).  Duplicate
 *                              indices count once per slot.
 *   ctx_len    [device] i32  [B]
 *   scale      softmax scale applied to <q, x> (e.g. 1/sqrt(576))
 *   out        [device] bf16 [B, q_len, 64, 512]  (round-to-nearest-even from fp32)
 *   lse        [device] fp32 [B, q_len, 64]
 *   shape      [host]   problem description
 *   plan_or_null [host] NULL = automatic plan; else as for smla_plan_for's override
 *   workspace  [device] scratch of at least the size smla_plan_for reports
 *                        (may be NULL when that size is 0).  Its first 64 KiB +
 *                        256 B hold the arrival counters of the merges in the
 *                        same launch and a status word, at the same place for
 *                        every shape and plan; the split partials follow.  It must be zero-filled
 *                        once before its first use (smla_workspace_init); every
 *                        successful call leaves the counters at zero again, so one
 *                        workspace serves calls of any batch size and split count
 *                        that fit in it.  Calls that share a workspace must not
 *                        overlap in time.
 *                        The in-kernel merge waits a bounded time for the other
 *                        splits of its request (they are resident and past their
 *                        compute, so the bound is only reached when something
 *                        went wrong).  If it gives up, it sets the status word,
 *                        leaves the counters as they are, still merges what the
 *                        partials hold and writes NaN into lse for that request's
 *                        heads.  A spread merge (SMLA_MERGE_SPREAD) that gives up
 *                        sets the same word and writes NaN into lse and into the
 *                        share of out it merges.  While the status word is set
 *                        every call that merges in the kernel (either form) on the
 *                        workspace writes NaN into lse and leaves out as it was.  A NaN lse therefore
 *                        means: call smla_workspace_init before the workspace's
 *                        next use.  In validate mode the call waits and returns
 *                        SMLA_ERR_MERGE when the status word is set.  (The
 *                        environment variable SMLA_MERGE_SPIN_LIMIT, read at every
 *                        call, lowers the bound: tests use it to drive this path.)
 *   stream     hipStream_t (NULL = default stream)
 * With nsplit = 1 the work is one kernel launch.  Otherwise each (request,
 * split) workgroup writes its partial result and the partials are merged by
 * the log-sum-exp combine of "The 64-Block Barrier", section "The Split-K
 * Prescription": by the last split of each request to finish, in the same
 * launch (SMLA_MERGE_IN_KERNEL); by every split, each merging a share of the
 * dims once all have written, in the same launch (SMLA_MERGE_SPREAD); or by the
 * combine kernel launched right after on the same stream (SMLA_MERGE_SEPARATE),
 * as the plan says.
 * Returns SMLA_OK or a negative SMLA_ERR_* code.
 */
int sparse_mla_decode(const void* q, const void* kv_pool, const int32_t* page_table,
                      const int32_t* topk_idx, const int32_t* ctx_len, float scale, void* out,
                      float* lse, const smla_shape* shape, const smla_plan* plan_or_null,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparse_mla_decode_noalloc -- sparse_mla_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, plans, kernels and results
 * (bit for bit) as sparse_mla_decode, without the workspace arguments: the
 * workspace is a device array that the library holds,
 * SMLA_NOALLOC_SCRATCH_BYTES per GPU, from the library's load on that GPU
 * until the process ends.  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library routine.
 *   - Returns SMLA_ERR_WORKSPACE, launching nothing, when the plan needs more
 *     workspace than that (smla_plan_for's workspace_bytes; each split
 *     partial takes 128 KiB + 256 B per (request, query token, split), plus
 *     the 64 KiB counter head), e.g. B * q_len * nsplit above ~250.
 *   - The first call on a GPU that needs the array looks up its device
 *     address and zeroes its counter head and status word with a fill kernel
 *     on `stream`.  A merge that gave up (see sparse_mla_decode) leaves that
 *     GPU's array marked for the rest of the process: lse then comes out NaN
 *     on every in-kernel merge.
 *   - Every call on one GPU uses that GPU's one array, and a call leaves it
 *     holding its partials: calls that overlap in time on one GPU (different
 *     streams or threads) race and must be serialised by the caller.
 * Returns as sparse_mla_decode does.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int sparse_mla_decode_noalloc(const void* q, const void* kv_pool, const int32_t* page_table,
                              const int32_t* topk_idx, const int32_t* ctx_len, float scale, void* out,
                              float* lse, const smla_shape* shape, const smla_plan* plan_or_null, void* stream);

/*
 * smla_decode_split / smla_decode_combine -- the two stages of
 * sparse_mla_decode as separate calls (a split kernel per (request, top-k
 * split), then the log-sum-exp combine kernel), for callers that schedule or
 * time the stages themselves ("Inside the Decode Performance Investigation",
 * sections "Task 1" and "Task 2": one split and one combine kernel per layer).
 *   smla_decode_split takes exactly the arguments of sparse_mla_decode.  With
 *   nsplit = 1 it writes out/lse itself; otherwise it fills the workspace with
 *   per-split partials (for each (request, query token, split) a 128 KB block
 *   holding the 64 x 512 fp32 output normalised by that split's own softmax
 *   denominator, in an internal element order that only smla_decode_combine
 *   reads; then fp32 [B * q_len, nsplit, 64] lse at the next 256-byte
 *   boundary) and leaves out/lse and the arrival counters alone.
 *   smla_decode_combine merges those partials into out/lse; the same shape and
 *   plan must be passed, and it does nothing when the plan has nsplit = 1.
 * Both return as sparse_mla_decode does.
 */
int smla_decode_split(const void* q, const void* kv_pool, const int32_t* page_table,
                      const int32_t* topk_idx, const int32_t* ctx_len, float scale, void* out,
                      float* lse, const smla_shape* shape, const smla_plan* plan_or_null,
                      void* workspace, size_t workspace_bytes, void* stream);
int smla_decode_combine(const smla_shape* shape, const smla_plan* plan_or_null, const void* workspace,
                        size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * smla_gather_rows -- test hook: the index translation and row gather stage of
 * the decode, on its own ("Inside the Decode Performance Investigation",
 * section "Task 1": scattered FP8 page gathers).
 *   kv_pool, page_table, topk_idx, ctx_len, shape: as for sparse_mla_decode
 *   rows  [device] u8  [B, 512, row_bytes]: the selected rows' bytes, zeros when masked
 *   slots [device] i64 [B, 512]: physical slot (page*64 + row), -1 when masked
 * Uses the same device functions as the decode kernel.  Returns as above.
 */
int smla_gather_rows(const void* kv_pool, const int32_t* page_table, const int32_t* topk_idx,
                     const int32_t* ctx_len, const smla_shape* shape, void* rows, int64_t* slots,
                     void* stream);

/*
 * smla_read_rows -- measurement aid: reads cache rows and discards them, so the
 * rate at which this device can move the rows the decode reads can be measured
 * with nothing else done to them (the pages judge the decode against the memory
 * bandwidth it reaches on scattered FP8 row gathers: "Inside the Decode
 * Performance Investigation", section "Task 1").
 *   kv_pool   [device] u8 pool of pool_rows >= 1 rows of row_bytes bytes, 16-byte aligned
 *   slots     [device] i64 [n_slots]: row indices (as smla_gather_rows returns);
 *             -1 and indices outside [0, pool_rows) are skipped
 *   per_group, n_groups: workgroup g (one per compute unit) reads the rows of
 *             slots[g * per_group .. + per_group); per_group <= 4096,
 *             n_groups * per_group >= n_slots
 *   row_bytes 656 or 1152
 *   sink      [device] u32 [n_groups * 1024]: per thread, the XOR of the four
 *             words of every 16-byte piece it read (thread t of group g reads
 *             pieces t, t + 1024, ... of the group's rows laid end to end)
 * Asynchronous on `stream`; returns SMLA_OK, SMLA_ERR_INVALID_ARG or SMLA_ERR_HIP.
 */
int smla_read_rows(const void* kv_pool, int64_t pool_rows, const int64_t* slots, int64_t n_slots,
                   int32_t per_group, int32_t row_bytes, int32_t n_groups, uint32_t* sink, void* stream);

/*
 * smla_kv_append -- the cache producer: quantise n_tokens new tokens' rows and
 * write them into the paged cache in the row format this library reads (the
 * pages name the FP8 latent cache the decode gathers from, "Inside the Decode
 * Performance Investigation", section "Task 1", and a hand-fused epilogue that
 * would produce it, section "Task 3").
 *   latent     [device] fp32 [n_tokens, 512], 16-byte aligned
 *   rope       [device] fp32 [n_tokens, 64], 16-byte aligned
 *   req        [device] i32  [n_tokens]: request of each token, in [0, shape->batch)
 *   pos        [device] i32  [n_tokens]: its logical position in that request
 *   page_table [device] i32  [B, max_pages_per_req], as for sparse_mla_decode
 *   kv_pool    [device] u8   pool; row page_table[req][pos / 64] * 64 + pos % 64 is written
 *   shape      [host]   batch, max_pages_per_req, pool_pages and kv_format are used
 * Row contents: fp8 format -- per 128-dim block j, scale_j = amax / 448 in fp32
 * (1.0 for an all-zero block) and code = e4m3fn(x / scale_j), nearest with ties
 * to even, saturated at +-448; then the 4 scales (fp32 little-endian) and the
 * rope values as bf16.  bf16 format -- latent then rope as bf16.  bf16 values
 * are rounded to nearest, ties to even.  A token whose request, position or page
 * is out of range is skipped; two tokens with one destination leave either row.
 * Only the destination rows are written.  Returns as sparse_mla_decode does.
 */
int smla_kv_append(const float* latent, const float* rope, const int32_t* req, const int32_t* pos,
                   const int32_t* page_table, void* kv_pool, int32_t n_tokens, const smla_shape* shape,
                   void* stream);

/*
 * smla_indexer_topk -- the top-k indexer: produce the topk_idx that
 * sparse_mla_decode reads.  The pages name the indexer ("Inside the Decode
 * Performance Investigation", sections "The Setup" and "Task 2") without a
 * formula; this computes the published lightning indexer of DeepSeek's sparse
 * attention: for request b and every position s < ctx_len[b] whose page is
 * valid (as for sparse_mla_decode),
 *     score[b][s] = sum_j head_w[b][j] * max(0, <q_idx[b][j], k_s>)   (j < 64 heads)
 * with k_s the bf16 key row of s, and selects the 512 valid positions of largest
 * score (equal scores: smaller s first), in that order, then -1 padding.
 *   q_idx      [device] bf16 [B, 64, 128], 16-byte aligned
 *   head_w     [device] fp32 [B, 64]
 *   key_pool   [device] bf16 [pool_pages * 64, 128]: one 256-B key row per slot,
 *                        16-byte aligned, paged by `page_table` like kv_pool
 *   page_table [device] i32  [B, max_pages_per_req]; ctx_len [device] i32 [B]
 *   scores     [device] fp32 [B, max_pages_per_req * 64]: written with each valid
 *                        position's fp32 score (-inf where its page is invalid;
 *                        positions >= ctx_len untouched); the selection is made on
 *                        these values
 *   topk_idx   [device] i32  [B, 512]
 *   shape      [host]   batch, max_pages_per_req and pool_pages are used
 * Two launches on `stream` (scores, then one selecting workgroup per request).
 * Returns as sparse_mla_decode does.
 */
int smla_indexer_topk(const void* q_idx, const float* head_w, const void* key_pool, const int32_t* page_table,
                      const int32_t* ctx_len, float* scores, int32_t* topk_idx, const smla_shape* shape,
                      void* stream);

/*
 * smla_workspace_init -- zero a workspace (its arrival counters and status
 * word) on `stream` with a fill kernel, before its first use by
 * sparse_mla_decode, after a call that did not complete, or after a merge gave
 * up waiting (NaN lse, or SMLA_ERR_MERGE in validate mode).
 * workspace [device], 4-byte aligned.
 */
int smla_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Bytes per cache row for a format (1152, 656), or -1. */
int smla_row_bytes(int kv_format);

/* Static description of an error code (never NULL). */
const char* smla_strerror(int code);

/* Library version: major * 10000 + minor * 100 + patch. */
int smla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
