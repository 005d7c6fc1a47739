// Internal definitions shared by the host library (api.cpp) and the gfx950
// kernels: workspace layout, the plan's device records, launcher entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/lbattn.h"

namespace lb {

// Persistent attention kernel geometry: 8 waves of 64 lanes per workgroup, each
// wave owning 32 query rows of one head; a tile serves G = H / H_kv heads, so it
// holds 32 * 8 / G query rows.  Keys stream through LDS in blocks of 64.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBlockN = LB_BLOCK_KEYS;

// Planning kernel: one workgroup sorts the tile keys in LDS.
constexpr int kPlanThreads = 1024;
constexpr int kSortCap = 32768;     // tiles per plan (32-bit sort keys, 128 KB of LDS)
constexpr int kRingSortCap = 16384; // work tiles one ring merge takes (two int arrays in LDS)
constexpr int kFusedTileCap = 4096;  // query tiles one fused ring takes (its sort keys in LDS)
constexpr int kMaxWorkers = 2048;   // persistent workgroups per launch
constexpr int kXcds = 8;            // accelerator complex dies (XCDs) of an MI355X, one L2 each

inline __host__ __device__ int tile_rows_for_group(int group) { return kRowsPerWave * kWaves / group; }

// Workspace header, at offset 0.  Written by the planning kernel, read by the
// attention kernel and by the host read-back calls.
struct WsHeader {
  int32_t err;          // LB_DEVERR_* bits
  int32_t n_frags;      // query fragments
  int32_t n_tiles;
  int32_t n_items;      // (n_tiles - n_empty) * kv_heads queued items (0 after an error)
  int32_t n_queues;     // work queues: one per XCD when kv_heads is a multiple of kXcds, else 1
  int32_t n_kvruns;
  int32_t tile_rows;
  int32_t n_workers;    // persistent workgroups of the last attention launch
  int64_t off_frags, off_kvruns, off_tiles, off_order, off_workers;
  int32_t cap_frags, cap_tiles;
  int64_t total_pairs;  // sum of tile costs (one head)
  int32_t plan_n_q, plan_n_kv, plan_kv_heads, plan_heads;  // shapes the plan was made for
  int32_t done;         // attention workgroups that found every queue empty
  uint32_t magic;       // kPlanMagic once a plan has been written
  int32_t per_queue;    // items per queue
  int32_t n_empty;      // tiles with no key span: the last n_empty of the order, kept out of the queues
  int32_t transposed;   // 1: tiles are key blocks and spans are query runs (the backward's dK/dV plan)
  int32_t has_lower;    // 1: some span has a lower bound (needs the bounded attention kernel)
  int32_t queue_head[8];  // next item of each queue
  // ring workspaces only (magic kRingMagic): the steps merged, and each step's key/value count
  int32_t ring_steps;
  int32_t ring_n_kv[LB_MAX_PLAN_STEPS];
  // 1: a fused ring, one tile per query tile with the spans of every step (each span's step in
  // 4 bits of the tile's `reserved`, span s at bits 4s..4s+3); the steps' results are one
  int32_t ring_fused;
  int64_t off_ntiles;  // plan workspaces: the tiles in natural (query) order
};

constexpr uint32_t kPlanMagic = 0x4C424154u;
// A ring workspace: the work tiles of several block steps in one longest-first order, copied
// from the steps' plans with the step index in each tile's `reserved` field, then the steps'
// empty tiles; header and worker records laid out as in a plan workspace.
constexpr uint32_t kRingMagic = 0x4C42524Eu;
constexpr int64_t kWorkersOffset = 256;  // worker records sit right after the header
static_assert(sizeof(WsHeader) <= 256, "header must fit its slot");

// A query fragment with its key spans before per-tile clipping.
struct Frag {
  int32_t q_start, q_len, q_pos0, n_spans;
  int32_t k_start[LB_MAX_SPANS], k_len[LB_MAX_SPANS], k_pos0[LB_MAX_SPANS], k_lo[LB_MAX_SPANS];
};
static_assert(sizeof(Frag) == 80, "");

// A key/value run (block path): equal document id, consecutive positions.
struct KvRun {
  int32_t start, len, pos0, doc;
};

static_assert(sizeof(lb_plan_tile) == 96, "lb_plan_tile layout");
static_assert(offsetof(lb_plan_tile, k_lo) == offsetof(lb_plan_tile, k_start) + 12 * LB_MAX_SPANS,
              "span fields are contiguous: k_start, k_len, k_pos0, k_lo");
static_assert(sizeof(lb_worker_record) == 40, "lb_worker_record layout");

// Plan workspace regions.  `tiles` holds the tiles in queue order (longest first), so the
// kernels that run a plan read tile i of the queue without an indirection; `order` is the
// identity, kept for readers written against a separate order; `ntiles` is the planner's
// own natural-order copy, from which the queue order is gathered.
struct WsLayout {
  int64_t off_frags, off_ftile, off_kvruns, off_tiles, off_order, off_ntiles, off_workers, total;
  int32_t cap_frags, cap_tiles;
};

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

inline WsLayout ws_layout(int64_t cap_frags, int64_t cap_tiles) {
  WsLayout L{};
  int64_t o = kWorkersOffset;
  L.off_workers = o; o = align256(o + kMaxWorkers * (int64_t)sizeof(lb_worker_record));
  L.off_frags = o;   o = align256(o + cap_frags * (int64_t)sizeof(Frag));
  L.off_ftile = o;   o = align256(o + (cap_frags + 1) * (int64_t)sizeof(int32_t));
  L.off_kvruns = o;  o = align256(o + cap_frags * (int64_t)sizeof(KvRun));
  L.off_tiles = o;   o = align256(o + cap_tiles * (int64_t)sizeof(lb_plan_tile));
  L.off_order = o;   o = align256(o + cap_tiles * (int64_t)sizeof(int32_t));
  L.off_ntiles = o;  o = align256(o + cap_tiles * (int64_t)sizeof(lb_plan_tile));
  L.total = o;
  L.cap_frags = (int32_t)cap_frags;
  L.cap_tiles = (int32_t)cap_tiles;
  return L;
}

enum PlanMode { kPlanCausalDoc = 0, kPlanSharedQuestion = 1, kPlanBlock = 2, kPlanSlices = 3 };

// Key position offset of a FULL slice's span: below every query position, so that every
// key is visible (the planner's pair count stays in 64-bit range).
constexpr int32_t kFullSpanPos = -(1 << 30);
// The transposed counterpart: a query run at this position sees every key of the tile.
constexpr int32_t kFullRowsPos = 1 << 30;

struct PlanArgs {
  int32_t mode;
  int32_t transposed;  // plan key tiles with the query spans that see them
  const int32_t* cu_seqlens;
  int32_t n_seg, total_tokens;
  const int32_t *q_pos, *q_doc, *kv_pos, *kv_doc;
  int32_t shared_doc;  // block path: the document every other document's rows see in full; -1: none
  const lb_mask_slice* slices;
  int32_t n_slices;
  int32_t n_q, n_kv;
  int32_t tile_rows, heads, kv_heads;
  // LPT ordering cost of a tile: block_weight * key blocks + pair_weight * G * visible pairs
  uint32_t block_weight = 1;  // 1 .. LB_LPT_BLOCK_WEIGHT_MAX
  uint32_t pair_weight = 0;   // 0 .. LB_LPT_PAIR_WEIGHT_MAX
  int32_t order = LB_ORDER_LPT;  // LB_ORDER_DOCUMENTS: fragments longest first, each one's tiles last first
  char* ws;
  WsLayout L;
};

// Several block-step plans in one launch, one workgroup per step.
constexpr int kMaxPlanSteps = LB_MAX_PLAN_STEPS;
struct PlanBatch {
  PlanArgs step[kMaxPlanSteps];
};

// Ring workspace layout: header, worker records, then the merged tiles.
constexpr int64_t kRingTilesOffset = (kWorkersOffset + kMaxWorkers * (int64_t)sizeof(lb_worker_record) + 255) &
                                     ~int64_t(255);

// Merge of several block steps' plans into one ring workspace (one workgroup).
struct RingMergeArgs {
  const char* step_ws[kMaxPlanSteps];
  int64_t step_ws_bytes[kMaxPlanSteps];
  int32_t n_kv[kMaxPlanSteps];
  int32_t n_steps;
  int32_t n_q, heads, kv_heads;
  char* ring;
  int32_t ring_cap;    // tiles the ring workspace holds
  int32_t transposed;  // the steps' plans are key-tile plans (the backward's dK/dV side)
};

// Per-step operands of a ring attention launch (indexed by a tile's step).
struct RingSteps {
  const void* k[kMaxPlanSteps];
  const void* v[kMaxPlanSteps];
  float* out[kMaxPlanSteps];
  float* lse[kMaxPlanSteps];
  int32_t n_kv[kMaxPlanSteps];
  int32_t n_steps;
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int32_t n_q, n_kv;
  int32_t heads, kv_heads, group;
  float scale_log2;  // softmax scale * log2(e)
  char* ws;
  int64_t ws_bytes;
};

struct MergeArgs {
  float* out_a;
  float* lse_a;
  const float* out_b;
  const float* lse_b;
  int32_t n_rows, heads, d;
};

// Partials 1 .. n_parts - 1 merged into partial 0 (written), in one pass.
struct MergePartsArgs {
  float* out[kMaxPlanSteps];
  float* lse[kMaxPlanSteps];
  int32_t n_parts, n_rows, heads, d;
};

// Backward kernels.  dQ: the forward's query tiles and wave layout (8 waves, each 32
// rows of one head).  dK/dV: key tiles of 128 keys, 4 groups of 32 keys, each owned by a
// pair of waves that loops over all G heads; query rows stream in stages of 32, one head
// at a time.
constexpr int kBwdKeyGroups = 4;
inline __host__ __device__ int bwd_q_rows(int group) { return tile_rows_for_group(group); }
inline __host__ __device__ int bwd_k_rows(int) { return 32 * kBwdKeyGroups; }

struct BwdArgs {
  const void* q;     // bf16 [n_q][heads][d]
  const void* k;     // bf16 [n_kv][kv_heads][d]
  const void* v;
  const void* dout;  // bf16 [n_q][heads][d]
  const float* lse;  // [heads][n_q], natural log, whole-row values
  const float* dvec; // [heads][n_q], D = <dout, out>
  void* dq;          // bf16 [n_q][heads][d], or fp32 accumulated (out_f32)
  void* dk;          // bf16 [n_kv][kv_heads][d], or fp32 (out_f32)
  void* dv;
  int32_t n_q, n_kv;
  int32_t heads, kv_heads, group;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  char* ws;          // the plan this kernel reads (query tiles for dQ, key tiles for dK/dV)
  int64_t ws_bytes;
};

// Launchers, one per translation unit; each returns the launch's hipError_t.
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_plan_steps(const PlanBatch& b, int n_steps, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int d, bool out_f32, bool lower, int n_workers, hipStream_t s);
hipError_t launch_ring_merge(const RingMergeArgs& m, hipStream_t s);
hipError_t launch_ring_fuse(const RingMergeArgs& m, hipStream_t s);
hipError_t launch_ring_attention(const AttnArgs& a, const RingSteps& r, int d, int n_workers, bool fused,
                                 hipStream_t s);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_lse_merge_parts(const MergePartsArgs& a, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s);
hipError_t launch_bwd_rowdot(const void* out, bool out_f32, const void* dout, int n_rows, int heads, int d,
                             float* dvec, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool out_f32, int n_workers, hipStream_t s);
hipError_t launch_bwd_dkv(const BwdArgs& a, int d, bool out_f32, int n_workers, hipStream_t s);

// Per-step operands of a ring dK/dV launch (indexed by a key tile's step).
struct RingBwdSteps {
  const void* k[kMaxPlanSteps];
  const void* v[kMaxPlanSteps];
  float* dk[kMaxPlanSteps];
  float* dv[kMaxPlanSteps];
  int32_t n_kv[kMaxPlanSteps];
  int32_t n_steps;
};
hipError_t launch_bwd_dkv_ring(const BwdArgs& a, const RingBwdSteps& r, int d, int n_workers, hipStream_t s);
hipError_t launch_bwd_dq_fused(const BwdArgs& a, const RingBwdSteps& r, int d, int n_workers, hipStream_t s);

}  // namespace lb
