/*
 * lbattn.h -- document-masked varlen attention for MI355X (gfx950), C ABI.
 *
 * What the library computes
 * -------------------------
 * Packed documents attend only inside themselves, so a pack's attention work
 * grows with the sum of squared document lengths rather than the square of
 * the pack length ("03 · 长文负载均衡" (llm-infra-atlas), section 1.1, the
 * W_attn formula; "数据并行负载均衡" (LoongForge), section 1).  The library
 * runs three operations on one GPU:
 *
 *   lb_varlen_attn_fwd  full forward over a packed sequence (cu_seqlens), with
 *                       a per-document causal mask or a shared-question mask
 *                       ("03 · 长文负载均衡", section 1.2);
 *   lb_block_attn_fwd   one ring step of a context-parallel rank: its query
 *                       shard against one key/value chunk, with global
 *                       positions and document ids carried per token, returning
 *                       out and log-sum-exp ("03 · 长文负载均衡", sections 3.2
 *                       and 4.2; "长序列训练与上下文并行", Ring Attention);
 *   lb_lse_merge        the online-softmax rescale-and-sum that folds two such
 *                       partial results ("03 · 长文负载均衡", section 3.2, DCP).
 *
 * Inside each forward call, a planning kernel cuts the queries into tiles,
 * keeps only the key spans that hold visible pairs (DCP's computation blocks,
 * section 3.2; MagiAttention's full/causal slices, section 4.4), bills each
 * tile its exact visible-pair count (Libra TAP, section 3.2), and orders tiles
 * longest first by an estimate of their time (VRSP, section 2.1; "数据并行负载均衡",
 * sections 4.2 and 4.4: LPT on a fitted load model).  A
 * persistent attention kernel then pulls (tile, key/value head) items from
 * that queue, so the next free compute unit always takes the largest
 * remaining item.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers, owned by the caller.  The
 *    library never allocates or frees memory.
 *  - Layout is THD (token-major): q [T][H][d], k and v [T][H_kv][d]; rows are
 *    contiguous, no padding between heads or tokens.  bf16 means IEEE
 *    bfloat16 stored in 16 bits.
 *  - Softmax scale is 1/sqrt(d).  lse is the natural log of the sum of
 *    exp(scaled logits) over the visible keys.  Query head h uses key/value
 *    head h / (H / H_kv).
 *  - Every compute call is asynchronous on `stream` (0 = the null stream) and
 *    returns before the GPU work finishes.  Host-checkable errors return
 *    before anything is enqueued.  Problems only the device can see (e.g. a
 *    decreasing cu_seqlens) set an error word in the workspace, make the
 *    attention kernel do nothing, and are read back with lb_read_device_error.
 *  - Supported shapes: d in {64, 128}; H % H_kv == 0 with H / H_kv in
 *    {1, 2, 4, 8}.  Other shapes return LB_EUNSUPPORTED.
 *  - Alignment: q, k, v, kv_chunk, out and out_* must be 16-byte aligned;
 *    the workspace must be 256-byte aligned.
 *  - No exception crosses this boundary; nothing here keeps state between
 *    calls except a per-device cache of the compute-unit count.
 */
#ifndef LBATTN_H
#define LBATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LB_OK = 0,
  LB_EINVAL = 1,        /* null pointer, negative size, bad mask kind, H % H_kv != 0 */
  LB_EUNSUPPORTED = 2,  /* shape outside what the kernels implement */
  LB_EWORKSPACE = 3,    /* workspace too small or misaligned */
  LB_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} lb_status;

typedef enum {
  LB_MASK_CAUSAL_DOC = 0,       /* key j visible to query i iff same segment and j <= i */
  LB_MASK_SHARED_QUESTION = 1   /* segment 0 is a question, the rest are answers: an answer
                                   sees the whole question and itself causally, never another
                                   answer; the question sees itself causally */
} lb_mask_kind;

/* Device error word values (lb_read_device_error). */
enum {
  LB_DEVERR_NONE = 0,
  LB_DEVERR_CU_SEQLENS = 1,   /* cu_seqlens[0] != 0, decreasing, or cu_seqlens[n_seg] != total_tokens */
  LB_DEVERR_CAPACITY = 2,     /* more fragments or tiles than the workspace holds */
  LB_DEVERR_SPANS = 4,        /* a query run meets more than LB_MAX_SPANS key runs of its document */
  LB_DEVERR_PLAN = 8,         /* lb_attn_run's shapes differ from those the workspace's plan was made for */
  LB_DEVERR_SLICES = 16       /* a slice list out of range, unsorted, overlapping, or of an unknown kind */
};

#define LB_MAX_SPANS 4
#define LB_MAX_PLAN_STEPS 16 /* block steps one lb_plan_block_steps call can plan */
#define LB_BLOCK_KEYS 64 /* keys per block the attention kernel steps through */
#define LB_NO_LOWER_BOUND (1 << 30) /* k_lo of a span whose keys have no lower bound */

/*
 * One tile of the plan, as lb_read_plan returns it, in queue order: ordering cost
 * descending, ties in natural order (fragment order, then tile order), except in the
 * LB_ORDER_DOCUMENTS order of lb_plan_varlen_ordered, the default of the varlen forward
 * (lb_plan_varlen, lb_varlen_attn_fwd), described there.  The cost of the varlen forward's
 * plans is the fitted time estimate of lb_plan_varlen_weighted; that of every other plan is
 * `blocks`.  A tile's
 * time is set mostly by the key blocks it sweeps, a short tile costing
 * as much as a full one ("03 · 长文负载均衡", section 3.3: a query block shorter than
 * one tile is billed as a whole tile), and items go out longest first ("数据并行负载
 * 均衡", section 4.4, LPT on estimated cost).  Costs are sorted on 15 bits: each is
 * divided by the least power of two that brings the plan's largest cost to 32767 or
 * below, rounding up, so the order is exact while no cost exceeds 32767 (a block count
 * does only for a document of over two million tokens) and a tile with work always
 * precedes every tile without.
 */
typedef struct {
  int32_t q_start;               /* first query row (index into the call's query rows) */
  int32_t q_len;                 /* rows in the tile (<= lb_tile_rows) */
  int32_t q_pos0;                /* mask position of the first row; row r has q_pos0 + r */
  int32_t n_spans;               /* key spans that hold visible pairs, 0..LB_MAX_SPANS */
  int64_t cost;                  /* exact visible (query, key) pairs of the tile, one head */
  int32_t k_start[LB_MAX_SPANS]; /* first key row of each span */
  int32_t k_len[LB_MAX_SPANS];   /* keys kept: those the tile's last row can see */
  int32_t k_pos0[LB_MAX_SPANS];  /* mask position of the span's first key */
  int32_t k_lo[LB_MAX_SPANS];    /* lower bound: key j of the span is visible to a row at position p
                                    only if k_lo + j >= p (LB_NO_LOWER_BOUND: no such bound) */
  int32_t blocks;                /* sum over spans of ceil(k_len / LB_BLOCK_KEYS): the order key,
                                    or its main term in the varlen forward's fitted estimate */
  int32_t reserved;              /* 0 in a plan; in a ring workspace the tile's step (lb_plan_ring), or
                                    in a fused ring span s's step in bits 4s..4s+3 (lb_plan_ring_fused) */
} lb_plan_tile;

/* One persistent workgroup's record (lb_read_worker_timing). */
typedef struct {
  uint32_t hw_id;        /* raw HW_ID register of the workgroup's first wave */
  uint32_t xcc_id;       /* raw XCC_ID register (accelerator complex die) */
  uint64_t t_start;      /* 100 MHz device clock when the workgroup started */
  uint64_t t_end;        /* ... and when it found the queue empty */
  int64_t pairs;         /* visible pairs x heads of the items it ran */
  int32_t items;         /* items it ran */
  int32_t blocks;        /* key blocks its items swept (query blocks, for the backward's key tiles) */
} lb_worker_record;

/* Query rows per tile for this head configuration (256 / (H / H_kv)); -1 if unsupported. */
int32_t lb_tile_rows(int32_t heads, int32_t kv_heads, int32_t d);

/*
 * Workspace bytes for calls of up to `max_tokens` query tokens (and, on the
 * block path, key/value tokens) and up to `max_segments` segments (varlen) or
 * runs of equal document id and consecutive position on either side (block).
 * Returns 0 for invalid or unsupported arguments.  The workspace holds the
 * plan and the per-workgroup records of the last call; it needs no clearing.
 */
size_t lb_workspace_bytes(int32_t max_tokens, int32_t max_segments, int32_t heads, int32_t kv_heads);

/*
 * Varlen forward.
 *   q          bf16 [total_tokens][heads][d]
 *   k, v       bf16 [total_tokens][kv_heads][d]
 *   cu_seqlens int32 [n_seg + 1], device; cu_seqlens[0] = 0, non-decreasing,
 *              cu_seqlens[n_seg] = total_tokens (checked on the device)
 *   mask_kind  lb_mask_kind
 *   out        bf16 [total_tokens][heads][d] (written for every row)
 *   lse        fp32 [heads][total_tokens]
 *   workspace  >= lb_workspace_bytes(total_tokens, n_seg, heads, kv_heads)
 * Every query sees at least itself, so every row gets a finite lse.
 */
lb_status lb_varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                             int32_t n_seg, int32_t total_tokens, int32_t heads, int32_t kv_heads,
                             int32_t d, int32_t mask_kind, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * lb_varlen_attn_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same plan and the same
 * kernels, with the plan kept in the library's own scratch array instead of a workspace.
 *   q, k, v, cu_seqlens, n_seg, total_tokens, heads, kv_heads, d, mask_kind, out, lse:
 *              as lb_varlen_attn_fwd (caller-owned device memory)
 * The scratch array is LB_NOALLOC_SCRATCH_BYTES of device memory per GPU, held from the
 * first call on that GPU until the process ends; the call allocates nothing (no hipMalloc,
 * no hipFree).  A plan needing more than that (lb_workspace_bytes(total_tokens, n_seg,
 * heads, kv_heads) > LB_NOALLOC_SCRATCH_BYTES) returns LB_EWORKSPACE before anything is
 * enqueued; every other host-side error is that of lb_varlen_attn_fwd.  Every call on one
 * GPU shares that GPU's array, so calls that overlap in time on one GPU (two streams, two
 * threads) race and must be serialised by the caller.  The device error word
 * (LB_DEVERR_*) lives in the array and cannot be read back: a malformed cu_seqlens makes
 * the call compute nothing, as in lb_varlen_attn_fwd; callers that need the diagnosis use
 * lb_varlen_attn_fwd with a workspace.
 */
#define LB_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
lb_status lb_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                     int32_t n_seg, int32_t total_tokens, int32_t heads, int32_t kv_heads,
                                     int32_t d, int32_t mask_kind, void* out, float* lse, hipStream_t stream);

/*
 * Block attention of one context-parallel step.
 *   q_shard    bf16 [n_q][heads][d]
 *   kv_chunk   bf16 [2][n_kv][kv_heads][d]: all of K, then all of V
 *   q_pos, kv_pos  int32 global positions of each token
 *   q_doc, kv_doc  int32 document ids of each token
 *   shared_doc LB_NO_SHARED_DOC, or the document id of a prefix every other document
 *              shares (the shared-question mask of "03 · 长文负载均衡", section 1.2, on
 *              the block path): each row of another document also sees every key of it
 *   out        fp32 [n_q][heads][d]; rows with no visible key are not written
 *   lse        fp32 [heads][n_q]; -inf for rows with no visible key
 *   workspace  >= lb_workspace_bytes(max(n_q, n_kv), max_runs, heads, kv_heads),
 *              max_runs bounding the runs of equal doc id and consecutive
 *              position on either side (exceeding it: LB_DEVERR_CAPACITY)
 * Key j is visible to query i iff q_doc[i] == kv_doc[j] and kv_pos[j] <= q_pos[i], or
 * kv_doc[j] == shared_doc != q_doc[i].  A query run meets at most LB_MAX_SPANS key runs
 * (its own document's and the shared document's together; beyond: LB_DEVERR_SPANS).
 * shared_doc < -1: LB_EINVAL.
 */
#define LB_NO_SHARED_DOC (-1)
lb_status lb_block_attn_fwd(const void* q_shard, int32_t n_q, const void* kv_chunk, int32_t n_kv,
                            const int32_t* q_pos, const int32_t* kv_pos, const int32_t* q_doc,
                            const int32_t* kv_doc, int32_t heads, int32_t kv_heads, int32_t d,
                            int32_t shared_doc, float* out, float* lse, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * The two halves of the forward calls.  lb_plan_varlen queues the tiles in the
 * LB_ORDER_DOCUMENTS order of lb_plan_varlen_ordered below, on the fitted time estimate that
 * lb_plan_varlen_weighted describes.  lb_varlen_attn_fwd is lb_plan_varlen followed by
 * lb_attn_run (bf16 out); lb_block_attn_fwd is lb_plan_block followed by lb_attn_run (fp32
 * out).  Split, a plan can serve several attention launches -- every layer of a model sees
 * the same cu_seqlens -- and each half can be timed on its own.  The plan stays valid in
 * the workspace until the next lb_plan_* call on it; the work queue rewinds itself at the
 * end of every lb_attn_run, so runs on one stream may repeat without re-planning.  Runs
 * that overlap in time on one workspace race.
 *
 * lb_attn_run's n_q, n_kv, heads and kv_heads must equal those of the plan; otherwise the
 * device sets LB_DEVERR_PLAN and writes nothing.  k and v are separate [n_kv][kv_heads][d]
 * bf16 arrays here (for the block path: kv_chunk and kv_chunk + n_kv*kv_heads*d).
 */
lb_status lb_plan_varlen(const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens, int32_t heads,
                         int32_t kv_heads, int32_t d, int32_t mask_kind, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * lb_plan_varlen with the caller's weights for the time estimate that orders the queue
 * ("数据并行负载均衡", section 4.2: a load model fitted to measured step times; section
 * 4.4: LPT on that estimate).  A tile's ordering cost is
 *     block_weight * blocks + pair_weight * (heads / kv_heads) * cost
 * with `blocks` and `cost` (visible pairs of one head) as in lb_plan_tile; the per-item
 * constant of a fitted model is left out, since it shifts every item alike.  Tiles,
 * spans and the workspace layout are those of lb_plan_varlen; only the queue order can
 * differ, and lb_attn_run runs the plan as any other.  The order is LPT on the estimate
 * (LB_ORDER_LPT of lb_plan_varlen_ordered); lb_plan_varlen uses the same estimate with
 * LB_LPT_FIT_BLOCK_WEIGHT and LB_LPT_FIT_PAIR_WEIGHT, grouped by document
 * (LB_ORDER_DOCUMENTS).  block_weight = 1, pair_weight = 0 orders by key blocks alone.
 *   block_weight  1 .. LB_LPT_BLOCK_WEIGHT_MAX (a tile with work never costs 0)
 *   pair_weight   0 .. LB_LPT_PAIR_WEIGHT_MAX
 * Weights out of range: LB_EINVAL; every other argument and error as lb_plan_varlen.
 * LB_LPT_FIT_BLOCK_WEIGHT : LB_LPT_FIT_PAIR_WEIGHT is the ratio fitted to this library's
 * attention kernel on MI355X by least squares over its workgroups' busy times on six
 * workloads: 1.37 us per key block, 3.3e-5 us per query-head pair.
 */
#define LB_LPT_BLOCK_WEIGHT_MAX ((1u << 24) - 1)
#define LB_LPT_PAIR_WEIGHT_MAX ((1u << 16) - 1)
#define LB_LPT_FIT_BLOCK_WEIGHT 41515u
#define LB_LPT_FIT_PAIR_WEIGHT 1u
lb_status lb_plan_varlen_weighted(const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens,
                                  int32_t heads, int32_t kv_heads, int32_t d, int32_t mask_kind,
                                  uint32_t block_weight, uint32_t pair_weight, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * lb_plan_varlen_weighted with a choice of queue order.
 *   LB_ORDER_LPT        the tiles by their estimate, largest first, ties in natural order
 *                       (lb_plan_varlen_weighted).
 *   LB_ORDER_DOCUMENTS  the fragments (one per segment of cu_seqlens) by the largest estimate
 *                       among their tiles, largest first, ties later fragment first; each
 *                       fragment's tiles together, from its last tile back to its first; the
 *                       tiles without key spans last, in descending natural order.  The
 *                       estimates are the 15-bit scaled ones of the LPT order.  This is LPT
 *                       applied to documents: the long documents' items go out first and
 *                       the short ones' at the end, as in LB_ORDER_LPT, but the items in
 *                       flight together mostly belong to one document and share its keys and
 *                       values in L2 (on the 32K long-tail pack of 30 documents, 0.48 GB
 *                       read past L2 per launch instead of 0.94, against 0.40 GB that every
 *                       order must read).  Plans of more than 4096 fragments or more than
 *                       16384 tiles are ordered as LB_ORDER_LPT.  Within a causal
 *                       document a later tile never sees fewer keys, so its tiles also go out
 *                       largest first, up to a shorter last tile.
 * order not one of these: LB_EINVAL; weights and every other argument as
 * lb_plan_varlen_weighted.  lb_plan_varlen is this call with LB_LPT_FIT_BLOCK_WEIGHT,
 * LB_LPT_FIT_PAIR_WEIGHT and LB_ORDER_DOCUMENTS.  Every order writes the same bits.
 */
#define LB_ORDER_LPT 0
#define LB_ORDER_DOCUMENTS 1
lb_status lb_plan_varlen_ordered(const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens,
                                 int32_t heads, int32_t kv_heads, int32_t d, int32_t mask_kind,
                                 uint32_t block_weight, uint32_t pair_weight, int32_t order, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

lb_status lb_plan_block(const int32_t* q_pos, const int32_t* q_doc, int32_t n_q, const int32_t* kv_pos,
                        const int32_t* kv_doc, int32_t n_kv, int32_t heads, int32_t kv_heads, int32_t d,
                        int32_t shared_doc, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Plans n_steps block steps of one query shard in one launch, one workgroup per step:
 * step s plans the shard (q_pos, q_doc, n_q) against kv_pos[s], kv_doc[s] (n_kv[s]
 * tokens) into workspaces[s] (workspace_bytes[s]), exactly as lb_plan_block would.  A
 * ring step's key/value positions and document ids follow from the packing alone, so a
 * rank can plan every step before the chunks arrive ("长序列训练与上下文并行", Ring
 * Attention: each step attends the chunk received from the previous rank; "03 ·
 * 长文负载均衡", section 4.2: the zigzag chunk assignment).
 *   kv_pos, kv_doc, n_kv, workspaces, workspace_bytes: host arrays of n_steps entries
 *   (the pointers in them are device pointers);  1 <= n_steps <= LB_MAX_PLAN_STEPS.
 * Every step is checked as lb_plan_block checks it before anything is launched; the
 * first failing step's status is returned and nothing runs.  Workspaces must be
 * distinct.
 */
lb_status lb_plan_block_steps(const int32_t* q_pos, const int32_t* q_doc, int32_t n_q,
                              const int32_t* const* kv_pos, const int32_t* const* kv_doc, const int32_t* n_kv,
                              int32_t n_steps, int32_t heads, int32_t kv_heads, int32_t d, int32_t shared_doc,
                              void* const* workspaces, const size_t* workspace_bytes, hipStream_t stream);

/*
 * One rank's ring in one attention launch.  A rank's ring runs one block step per chunk
 * it receives ("长序列训练与上下文并行", Ring Attention), and each step is a persistent
 * launch whose end waits for its largest items: a light step leaves most compute units
 * idle.  Merging the steps' plans gives one longest-first queue over the work of every
 * step ("数据并行负载均衡", section 4.4: LPT over all items; "03 · 长文负载均衡", section
 * 3.2: only blocks with visible pairs become work), and one launch runs it, each step's
 * partial (out, lse) into its own buffers as lb_attn_run would write it, bit for bit.  The
 * partials are then merged in step order (lb_lse_merge_parts, or lb_lse_merge step after step).
 *
 * lb_ring_workspace_bytes: bytes of a ring workspace for n_steps steps, each within the
 *   bounds given to lb_workspace_bytes (0 if out of range).
 * lb_plan_ring: merges the plans in workspaces[0..n_steps) (made by lb_plan_block or
 *   lb_plan_block_steps for the same query shard of n_q tokens, step s against n_kv[s]
 *   key/value tokens; host arrays holding device pointers) into ring_workspace (256-byte
 *   aligned, distinct from the step workspaces).  The tiles are copied in queue order:
 *   key blocks descending, then step, then the step's own order; each tile's `reserved`
 *   field holds its step; the steps' empty tiles follow.  A step plan that is not a
 *   forward block plan for these shapes sets LB_DEVERR_PLAN in the ring's error word, a
 *   step's own error bits pass on, more work tiles than 16384 (or than the workspace
 *   holds) set LB_DEVERR_CAPACITY; the ring then runs nothing.  Plan the ring again
 *   after any of its steps is planned again.  lb_read_plan, lb_read_device_error and
 *   lb_read_worker_timing read a ring workspace too.
 * lb_ring_attn_run: runs the ring's items.  q: bf16 [n_q][heads][d]; k[s], v[s]: bf16
 *   [n_kv[s]][kv_heads][d]; out[s]: fp32 [n_q][heads][d]; lse[s]: fp32 [heads][n_q]; all
 *   host arrays of n_steps device pointers, out and lse distinct per step.  Rows with no
 *   visible key in step s get lse[s] = -inf and out[s] unwritten, as lb_attn_run.  A ring
 *   made for other shapes or other n_kv sets LB_DEVERR_PLAN and runs nothing.  Argument
 *   errors return LB_EINVAL / LB_EUNSUPPORTED / LB_EWORKSPACE before anything is enqueued.
 */
size_t lb_ring_workspace_bytes(int32_t n_steps, int32_t max_tokens, int32_t max_segments, int32_t heads,
                               int32_t kv_heads);

lb_status lb_plan_ring(void* const* workspaces, const size_t* workspace_bytes, const int32_t* n_kv,
                       int32_t n_steps, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d,
                       void* ring_workspace, size_t ring_workspace_bytes, hipStream_t stream);

lb_status lb_ring_attn_run(const void* q, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d, int32_t n_steps,
                           const void* const* k, const void* const* v, const int32_t* n_kv, float* const* out,
                           float* const* lse, void* ring_workspace, size_t ring_workspace_bytes,
                           hipStream_t stream);

/*
 * One rank's ring fused per query tile.  The steps' plans of one query shard cut it into the
 * same tiles (the tiling depends on the query side only), so tile x of every step can run as
 * one item: its rows against the key spans of every step, in one online softmax, which is the
 * rescale-and-sum of the steps' partials ("03 · 长文负载均衡", section 3.2, DCP) taken inside the
 * tile rather than by merges after the launch.  The ring then writes no partials and needs no
 * merge; the queue holds one item per query tile and kv head, longest first ("数据并行负载均衡",
 * section 4.4).  The result equals the merged partials to the rounding of the bf16 softmax weights
 * (each path rounds them against its own running maximum), not bit for bit.
 *
 * lb_plan_ring_fused: as lb_plan_ring (same arguments and workspace), but tile x of the ring
 *   gathers tile x of every step: spans in step order (at most LB_MAX_SPANS in all; span s's
 *   step in bits 4s..4s+3 of `reserved`), pairs and key blocks summed.  Queue order: key
 *   blocks descending (above 32767 as 32767), ties in query order, tiles without spans last
 *   in query order.  Sets LB_DEVERR_SPANS when a tile would hold more spans (use lb_plan_ring
 *   then), LB_DEVERR_PLAN when a step plan is not a forward block plan for these shapes or the
 *   steps tile the queries differently, LB_DEVERR_CAPACITY above 4096 tiles or the workspace's
 *   capacity; the ring then runs nothing.
 * lb_ring_attn_run_fused: runs a fused ring.  q, k, v, n_kv as lb_ring_attn_run; out: fp32
 *   [n_q][heads][d], lse: fp32 [heads][n_q], device pointers: the merged result over every
 *   step.  Rows with no visible key in any step get lse = -inf and out unwritten.  A ring that
 *   is not a fused ring for these shapes sets LB_DEVERR_PLAN and runs nothing.  Argument
 *   errors return LB_EINVAL / LB_EUNSUPPORTED / LB_EWORKSPACE before anything is enqueued.
 */
lb_status lb_plan_ring_fused(void* const* workspaces, const size_t* workspace_bytes, const int32_t* n_kv,
                             int32_t n_steps, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d,
                             void* ring_workspace, size_t ring_workspace_bytes, hipStream_t stream);

lb_status lb_ring_attn_run_fused(const void* q, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d,
                                 int32_t n_steps, const void* const* k, const void* const* v, const int32_t* n_kv,
                                 float* out, float* lse, void* ring_workspace, size_t ring_workspace_bytes,
                                 hipStream_t stream);

/*
 * The backward of one rank's ring (the steps of lb_block_attn_bwd for n_steps key/value
 * chunks of one query shard), with every step's dK/dV items in one launch.  A dK/dV
 * launch ends with its longest key tiles (a tile near the start of a long document sweeps
 * every later query row of it), so one launch per step pays that tail once per step; one
 * longest-first queue over the key tiles of all steps ("数据并行负载均衡", section 4.4; the
 * partial key/value gradients of each step go back to the chunk's owner, "03 · 长文负载均衡",
 * section 4.4) runs the long tiles of all steps side by side.
 *   Shared by all steps: q_shard, n_q, dout, lse, dvec, q_pos, q_doc, heads, kv_heads, d,
 *   shared_doc and dq, as lb_block_attn_bwd takes them (dq fp32 [n_q][heads][d] is added to,
 *   step after step in index order).
 *   Per step s (host arrays of n_steps entries holding device pointers): kv_chunks[s] bf16
 *   [2][n_kv[s]][kv_heads][d], kv_pos[s], kv_doc[s], dkv[s] fp32 [2][n_kv[s]][kv_heads][d]
 *   (written: that chunk's partial dk, dv; zero where no row sees a key), workspaces[s] of
 *   workspace_bytes[s] (as lb_block_attn_bwd sizes it).  1 <= n_steps <= LB_MAX_PLAN_STEPS / 2,
 *   n_kv[s] >= 1; workspaces and dkv buffers distinct.
 *   ring_workspace: 256-byte aligned, lb_ring_workspace_bytes(n_steps, ...) bytes or more
 *   for the largest side; it receives the merged key-tile queue and the dK/dV launch's
 *   worker records.
 * Launches: one planning launch (both plans of every step), the merge of the key-tile
 * plans, one dQ launch per step, one dK/dV launch.  Device errors as lb_block_attn_bwd,
 * the dK/dV side's in ring_workspace.  Argument errors return before anything is enqueued.
 */
lb_status lb_block_attn_bwd_ring(const void* q_shard, int32_t n_q, const void* dout, const float* lse,
                                 const float* dvec, const int32_t* q_pos, const int32_t* q_doc, int32_t heads,
                                 int32_t kv_heads, int32_t d, int32_t shared_doc, int32_t n_steps,
                                 const void* const* kv_chunks, const int32_t* n_kv, const int32_t* const* kv_pos,
                                 const int32_t* const* kv_doc, float* dq, float* const* dkv,
                                 void* const* workspaces, const size_t* workspace_bytes, void* ring_workspace,
                                 size_t ring_workspace_bytes, hipStream_t stream);

/*
 * lb_block_attn_bwd_ring with the dQ side fused as the forward's fused ring is
 * (lb_plan_ring_fused): the steps' query-tile plans are fused into q_ring_workspace (256-byte
 * aligned, distinct from the other workspaces; sized by lb_ring_workspace_bytes), and one dQ
 * launch runs each query tile against the keys and values of every step, adding the tile
 * rows' whole dq into dq once.  dq, dkv and the other arguments as lb_block_attn_bwd_ring;
 * dk, dv have its bits, dq agrees with it to fp32 rounding (one sum over every step's key
 * blocks instead of a sum per step added into dq).  A query tile meeting more than
 * LB_MAX_SPANS key runs over all steps sets LB_DEVERR_SPANS in q_ring_workspace's error
 * word and the dQ launch then adds nothing (use lb_block_attn_bwd_ring then).  Argument
 * errors return before anything is enqueued.
 */
lb_status lb_block_attn_bwd_ring_fused(const void* q_shard, int32_t n_q, const void* dout, const float* lse,
                                       const float* dvec, const int32_t* q_pos, const int32_t* q_doc, int32_t heads,
                                       int32_t kv_heads, int32_t d, int32_t shared_doc, int32_t n_steps,
                                       const void* const* kv_chunks, const int32_t* n_kv,
                                       const int32_t* const* kv_pos, const int32_t* const* kv_doc, float* dq,
                                       float* const* dkv, void* const* workspaces, const size_t* workspace_bytes,
                                       void* ring_workspace, size_t ring_workspace_bytes, void* q_ring_workspace,
                                       size_t q_ring_workspace_bytes, hipStream_t stream);

lb_status lb_attn_run(const void* q, const void* k, const void* v, int32_t n_q, int32_t n_kv, int32_t heads,
                      int32_t kv_heads, int32_t d, int32_t out_f32, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* lb_attn_run for plans whose spans bound their visible keys from below as well (slice
   lists with INV-CAUSAL or BI-CAUSAL slices); it runs any plan, a little slower than
   lb_attn_run on plans without such bounds. */
lb_status lb_attn_run_lower(const void* q, const void* k, const void* v, int32_t n_q, int32_t n_kv, int32_t heads,
                            int32_t kv_heads, int32_t d, int32_t out_f32, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * In-place merge a <- merge(a, b) of two partials over disjoint key sets:
 *   M = max(lse_a, lse_b), w_x = exp(lse_x - M),
 *   lse_a = M + ln(w_a + w_b),  out_a = (w_a out_a + w_b out_b) / (w_a + w_b).
 * Where lse_b = -inf, row a is left untouched and out_b is not read; where
 * lse_a = -inf, out_a and lse_a are replaced by b's.
 *   out_a, out_b  fp32 [n_rows][heads][d];  lse_a, lse_b  fp32 [heads][n_rows]
 */
lb_status lb_lse_merge(float* out_a, float* lse_a, const float* out_b, const float* lse_b,
                       int32_t n_rows, int32_t heads, int32_t d, hipStream_t stream);

/*
 * The merges of a ring's partials in one pass: parts 1 .. n_parts - 1 merged into part 0 in
 * index order, each as lb_lse_merge would merge it, with the same bits as n_parts - 1 calls
 * of lb_lse_merge in sequence ("长序列训练与上下文并行", Ring Attention: the step results are
 * folded into the running one in step order).  A row is read from a partial only where
 * that partial has a visible key (lse != -inf) and written once; part 0's row is not read
 * where the first merge that touches the row keeps no share of it.
 *   out, lse  host arrays of n_parts device pointers, each as lb_lse_merge's out_a, lse_a
 *             (fp32 [n_rows][heads][d], [heads][n_rows]); distinct; out[0], lse[0] written
 *   2 <= n_parts <= LB_MAX_PLAN_STEPS; d a multiple of 4, at most 1024 (else LB_EUNSUPPORTED)
 * Argument errors return LB_EINVAL before anything is enqueued.
 */
lb_status lb_lse_merge_parts(float* const* out, float* const* lse, int32_t n_parts, int32_t n_rows, int32_t heads,
                             int32_t d, hipStream_t stream);

/*
 * ---- Backward -------------------------------------------------------------------
 * Gradients of the forwards above from their saved lse ("03 · 长文负载均衡", section 4.4:
 * MagiAttention reduces each block's partial key/value gradients back to the rank that
 * owns the keys; section 5: key/value gradients kept with their states).  With
 * P = exp(scale <q_i, k_j> - lse_i) on visible pairs and D_i = <dout_i, out_i>:
 *   dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (<dout_i, v_j> - D_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 * key/value gradients summed over the query heads of their kv group.  Rows whose lse
 * is -inf get no gradient.  The same masks and head mapping as the forward.
 */

/* Bytes of workspace lb_varlen_attn_bwd needs for packs up to max_tokens tokens and
   max_segments segments: two plans (query tiles for dq, key tiles for dk/dv) and the
   row values D ([heads][tokens] fp32).  0 when the head counts are unsupported. */
size_t lb_bwd_workspace_bytes(int32_t max_tokens, int32_t max_segments, int32_t heads, int32_t kv_heads);

/* Byte offset, inside a backward workspace, of its key-tile plan (the query-tile plan sits
   at offset 0), for lb_read_plan and lb_read_device_error on either half.  block_path = 0:
   lb_varlen_attn_bwd with total_tokens = n_q and n_seg segments; 1: lb_block_attn_bwd with
   this workspace size.  0 when the arguments are invalid. */
size_t lb_bwd_key_plan_offset(int32_t block_path, int32_t n_q, int32_t n_kv, int32_t n_seg, int32_t heads,
                              int32_t kv_heads, size_t workspace_bytes);

/*
 * D[h][i] = sum_d out[i][h][d] * dout[i][h][d] (fp32), the row values of the backward.
 *   out   bf16 [n_rows][heads][d] (out_f32 = 0) or fp32 (out_f32 = 1: a ring rank's merged
 *         block output);  dout bf16 [n_rows][heads][d];  dvec fp32 [heads][n_rows] (written).
 */
lb_status lb_attn_bwd_rowdot(const void* out, int32_t out_f32, const void* dout, int32_t n_rows, int32_t heads,
                             int32_t d, float* dvec, hipStream_t stream);

/*
 * Backward of lb_varlen_attn_fwd (same cu_seqlens, masks and shapes).
 *   q, k, v   the forward's inputs;  out, lse  its outputs (bf16 [T][heads][d], fp32 [heads][T]);
 *   dout      bf16 [T][heads][d];
 *   dq        bf16 [T][heads][d] (written);  dk, dv  bf16 [T][kv_heads][d] (written).
 * Launches one planning kernel (both plans), the D pass, the dq kernel and the dk/dv
 * kernel on `stream`.  Both plans queue their tiles in the LB_ORDER_DOCUMENTS order (see
 * lb_plan_varlen_ordered) of key blocks alone: the items of one document run side by side
 * and share its keys (dq) or its query rows (dk/dv) in L2.
 * workspace: lb_bwd_workspace_bytes(total_tokens, n_seg, ...) bytes,
 * 256-byte aligned, caller-owned; a plan error sets the device error word of its half
 * (read with lb_read_device_error on the workspace: the query-tile plan sits at its start).
 */
lb_status lb_varlen_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens,
                             int32_t heads, int32_t kv_heads, int32_t d, int32_t mask_kind, void* dq, void* dk,
                             void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One ring step of the backward of lb_block_attn_fwd: the query shard's dq contribution
 * and the key/value chunk's partial dk, dv (to be summed over the ranks that attended to
 * the chunk, at the rank that owns it).
 *   q_shard   bf16 [n_q][heads][d];  kv_chunk  bf16 [2][n_kv][kv_heads][d] (K then V);
 *   dout      bf16 [n_q][heads][d];
 *   lse, dvec fp32 [heads][n_q]: the whole row's lse after every step's merge, and
 *             D = <dout, out> of the merged out (lb_attn_bwd_rowdot with out_f32 = 1);
 *   q_pos, kv_pos, q_doc, kv_doc, shared_doc: as lb_block_attn_fwd;
 *   dq        fp32 [n_q][heads][d]: this step's contribution is ADDED (zero it before the
 *             first step; rows with no visible key in this step are left as they are);
 *   dkv       fp32 [2][n_kv][kv_heads][d]: this step's dk then dv, WRITTEN (every key).
 * workspace: split in two halves (query-tile and key-tile plans), each sized like an
 * lb_plan_block workspace; LB_EWORKSPACE when a half holds less than one run.
 */
lb_status lb_block_attn_bwd(const void* q_shard, int32_t n_q, const void* kv_chunk, int32_t n_kv, const void* dout,
                            const float* lse, const float* dvec, const int32_t* q_pos, const int32_t* kv_pos,
                            const int32_t* q_doc, const int32_t* kv_doc, int32_t heads, int32_t kv_heads, int32_t d,
                            int32_t shared_doc, float* dq, float* dkv, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * ---- Slice-list masks -------------------------------------------------------------
 * "03 · 长文负载均衡", section 4.4 (MagiAttention): a mask written as rectangles of
 * query rows x keys, each of one type; the mask is their union.  FULL: every pair of the
 * rectangle.  CAUSAL (aligned at the bottom-right corner): row r of the rectangle
 * (0-based) sees its keys 0 .. r + k_len - q_len.  Varlen causal, shared-question,
 * block-causal (frames that see their document up to their own end) and prefix masks
 * are all such lists.
 * The list is sorted by q_start; slices with the same (q_start, q_len) form one query
 * range and must cover disjoint key ranges (at most LB_MAX_SPANS of them); different
 * query ranges must not overlap.  A violation sets LB_DEVERR_SLICES (more than
 * LB_MAX_SPANS slices on one range: LB_DEVERR_SPANS) and nothing runs.
 */
typedef struct {
  int32_t q_start, q_len;  /* query rows [q_start, q_start + q_len), q_len >= 1 */
  int32_t k_start, k_len;  /* keys [k_start, k_start + k_len), k_len >= 1 */
  int32_t kind;            /* LB_SLICE_FULL, _CAUSAL, _INV_CAUSAL or _BI_CAUSAL */
} lb_mask_slice;

/* INV-CAUSAL is aligned at the top-left corner: row r sees keys r .. k_len - 1.
   BI-CAUSAL is CAUSAL and INV-CAUSAL at once (a band): keys r .. r + k_len - q_len; a causal
   sliding window is a list of such bands. */
enum { LB_SLICE_FULL = 0, LB_SLICE_CAUSAL = 1, LB_SLICE_INV_CAUSAL = 2, LB_SLICE_BI_CAUSAL = 3 };

/* The plan of a slice list: slices is a DEVICE array of n_slices entries; queries
   [0, n_q), keys [0, n_kv).  Workspace: lb_workspace_bytes(n_q, 2 * n_slices + 1, heads,
   kv_heads) bytes (a fragment per query range and one per run of rows no slice covers: those
   rows get lse = -inf from the run and their out is not written).  Run it with lb_attn_run (k, v of n_kv rows; out bf16 or fp32) when every slice is
   FULL or CAUSAL, with lb_attn_run_lower when some are INV-CAUSAL or BI-CAUSAL (lb_attn_run
   refuses such a plan: LB_DEVERR_PLAN). */
lb_status lb_plan_slices(const lb_mask_slice* slices, int32_t n_slices, int32_t n_q, int32_t n_kv, int32_t heads,
                         int32_t kv_heads, int32_t d, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward under a slice-list mask: q bf16 [n_q][heads][d], k, v bf16 [n_kv][kv_heads][d];
   out bf16 [n_q][heads][d], lse fp32 [heads][n_q].  lse is -inf on rows no slice covers
   (their out is not written) and on rows that see no key. */
lb_status lb_slices_attn_fwd(const void* q, const void* k, const void* v, const lb_mask_slice* slices,
                             int32_t n_slices, int32_t n_q, int32_t n_kv, int32_t heads, int32_t kv_heads, int32_t d,
                             void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* lb_status_string(lb_status s);

/* Synchronises `stream`, then copies the device error word of the last call that used
   `workspace` into *host_err (LB_DEVERR_* bits). */
lb_status lb_read_device_error(const void* workspace, size_t workspace_bytes, int32_t* host_err,
                               hipStream_t stream);

/* Synchronises `stream`, then copies the last call's plan: *n_tiles tiles in the order the
   persistent kernel hands them out (longest first; ties in natural order).  At most
   max_tiles are copied; *n_tiles is the full count. */
lb_status lb_read_plan(const void* workspace, size_t workspace_bytes, lb_plan_tile* host_tiles,
                       int32_t max_tiles, int32_t* n_tiles, hipStream_t stream);

/* Synchronises `stream`, then copies one record per persistent workgroup of the last
   attention launch (at most max_records; *n_records is the launch's count). */
lb_status lb_read_worker_timing(const void* workspace, size_t workspace_bytes,
                                lb_worker_record* host_records, int32_t max_records,
                                int32_t* n_records, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LBATTN_H */
