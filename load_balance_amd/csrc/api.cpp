// Host side of the C ABI declared in include/lbattn.h: argument checks,
// workspace carving, launch configuration and read-back helpers.  Every
// check that the host can make happens before anything is enqueued.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "lbattn_internal.h"

using namespace lb;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_workers[kMaxDevices];  // persistent workgroups per device (0 = unknown)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool group_supported(int32_t heads, int32_t kv_heads) {
  if (heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0) return false;
  const int g = heads / kv_heads;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Persistent grid size: resident workgroups of the attention kernel on the current device.
lb_status persistent_workers(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LB_EHIP;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_workers[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *out = cached;
      return LB_OK;
    }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return LB_EHIP;
  // one 512-thread workgroup per compute unit: 71.7 KB of LDS and ~2 waves per SIMD of registers
  const int n = std::min(cus, kMaxWorkers);
  if (dev >= 0 && dev < kMaxDevices) g_workers[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return LB_OK;
}

lb_status check_heads(int32_t heads, int32_t kv_heads, int32_t d) {
  if (heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0) return LB_EINVAL;
  if (!group_supported(heads, kv_heads) || (d != 64 && d != 128)) return LB_EUNSUPPORTED;
  return LB_OK;
}

// Checks of the attention half; nothing is enqueued.
lb_status check_run(const void* q, const void* k, const void* v, int32_t n_q, int32_t n_kv, int32_t heads,
                    int32_t kv_heads, int32_t d, void* out, float* lse, void* workspace, size_t workspace_bytes) {
  if (n_q < 0 || n_kv < 0) return LB_EINVAL;
  if (!q || !out || !lse || !workspace) return LB_EINVAL;
  if (n_kv > 0 && (!k || !v)) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4)) return LB_EINVAL;
  if (n_kv > 0 && (!aligned(k, 16) || !aligned(v, 16))) return LB_EINVAL;
  if (!aligned(workspace, 256)) return LB_EWORKSPACE;
  if ((int64_t)workspace_bytes < ws_layout(1, 1).total) return LB_EWORKSPACE;
  return LB_OK;
}

lb_status launch_run(const void* q, const void* k, const void* v, int32_t n_q, int32_t n_kv, int32_t heads,
                     int32_t kv_heads, int32_t d, bool out_f32, void* out, float* lse, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, bool lower = false) {
  int workers = 0;
  lb_status st = persistent_workers(&workers);
  if (st != LB_OK) return st;
  AttnArgs at{};
  at.q = q;
  at.k = n_kv > 0 ? k : q;
  at.v = n_kv > 0 ? v : q;
  at.out = out;
  at.lse = lse;
  at.n_q = n_q;
  at.n_kv = n_kv;
  at.heads = heads;
  at.kv_heads = kv_heads;
  at.group = heads / kv_heads;
  at.scale_log2 = (float)(1.0 / std::sqrt((double)d) * 1.4426950408889634);
  at.ws = static_cast<char*>(workspace);
  at.ws_bytes = (int64_t)workspace_bytes;
  return launch_attention(at, d, out_f32, lower, workers, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

// Checks and layout of a varlen plan; *L receives the layout when LB_OK.
lb_status prepare_plan_varlen(const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens, int32_t heads,
                              int32_t kv_heads, int32_t d, int32_t mask_kind, void* workspace,
                              size_t workspace_bytes, WsLayout* L) {
  if (!cu_seqlens || !workspace) return LB_EINVAL;
  if (n_seg < 1 || total_tokens < 0) return LB_EINVAL;
  if (mask_kind != LB_MASK_CAUSAL_DOC && mask_kind != LB_MASK_SHARED_QUESTION) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  if (!aligned(cu_seqlens, 4)) return LB_EINVAL;
  if (!aligned(workspace, 256)) return LB_EWORKSPACE;
  const int bm = tile_rows_for_group(heads / kv_heads);
  const int64_t tiles = ceil_div(total_tokens, bm) + n_seg;
  if (tiles > kSortCap) return LB_EUNSUPPORTED;
  *L = ws_layout(n_seg, tiles);
  if ((int64_t)workspace_bytes < L->total) return LB_EWORKSPACE;
  return LB_OK;
}

lb_status launch_plan_varlen(const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens, int32_t heads,
                             int32_t kv_heads, int32_t mask_kind, void* workspace, const WsLayout& L,
                             hipStream_t stream, uint32_t block_weight = LB_LPT_FIT_BLOCK_WEIGHT,
                             uint32_t pair_weight = LB_LPT_FIT_PAIR_WEIGHT, int32_t order = LB_ORDER_DOCUMENTS) {
  PlanArgs p{};
  p.block_weight = block_weight;
  p.pair_weight = pair_weight;
  p.order = order;
  p.mode = mask_kind == LB_MASK_CAUSAL_DOC ? kPlanCausalDoc : kPlanSharedQuestion;
  p.cu_seqlens = cu_seqlens;
  p.n_seg = n_seg;
  p.total_tokens = total_tokens;
  p.tile_rows = tile_rows_for_group(heads / kv_heads);
  p.heads = heads;
  p.kv_heads = kv_heads;
  p.ws = static_cast<char*>(workspace);
  p.L = L;
  return launch_plan(p, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

lb_status prepare_plan_block(const int32_t* q_pos, const int32_t* q_doc, int32_t n_q, const int32_t* kv_pos,
                             const int32_t* kv_doc, int32_t n_kv, int32_t heads, int32_t kv_heads, int32_t d,
                             void* workspace, size_t workspace_bytes, WsLayout* L) {
  if (n_q < 0 || n_kv < 0) return LB_EINVAL;
  if (!q_pos || !q_doc || !workspace) return LB_EINVAL;
  if (n_kv > 0 && (!kv_pos || !kv_doc)) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  if (!aligned(q_pos, 4) || !aligned(q_doc, 4)) return LB_EINVAL;
  if (n_kv > 0 && (!aligned(kv_pos, 4) || !aligned(kv_doc, 4))) return LB_EINVAL;
  if (!aligned(workspace, 256)) return LB_EWORKSPACE;
  const int bm = tile_rows_for_group(heads / kv_heads);
  // Runs are unknown to the host: take the largest run capacity the workspace holds.
  const int64_t max_runs = std::max<int64_t>(1, std::max(n_q, n_kv));
  auto layout_for = [&](int64_t f) { return ws_layout(f, std::min<int64_t>(kSortCap, ceil_div(n_q, bm) + f)); };
  if ((int64_t)workspace_bytes < layout_for(1).total) return LB_EWORKSPACE;
  int64_t lo = 1, hi = max_runs;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (layout_for(mid).total <= (int64_t)workspace_bytes) lo = mid; else hi = mid - 1;
  }
  *L = layout_for(lo);
  return LB_OK;
}

PlanArgs block_plan_args(const int32_t* q_pos, const int32_t* q_doc, int32_t n_q, const int32_t* kv_pos,
                         const int32_t* kv_doc, int32_t n_kv, int32_t heads, int32_t kv_heads, int32_t shared_doc,
                         void* workspace, const WsLayout& L) {
  PlanArgs p{};
  p.mode = kPlanBlock;
  p.q_pos = q_pos; p.q_doc = q_doc; p.kv_pos = kv_pos; p.kv_doc = kv_doc;
  p.shared_doc = shared_doc;
  p.n_q = n_q;
  p.n_kv = n_kv;
  p.tile_rows = tile_rows_for_group(heads / kv_heads);
  p.heads = heads;
  p.kv_heads = kv_heads;
  p.ws = static_cast<char*>(workspace);
  p.L = L;
  return p;
}

lb_status launch_plan_block(const int32_t* q_pos, const int32_t* q_doc, int32_t n_q, const int32_t* kv_pos,
                            const int32_t* kv_doc, int32_t n_kv, int32_t heads, int32_t kv_heads, int32_t shared_doc,
                            void* workspace, const WsLayout& L, hipStream_t stream) {
  const PlanArgs p =
      block_plan_args(q_pos, q_doc, n_q, kv_pos, kv_doc, n_kv, heads, kv_heads, shared_doc, workspace, L);
  return launch_plan(p, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

// ---- backward: two plans (query tiles for dQ, key tiles for dK/dV) in one workspace ----
struct BwdLayout {
  WsLayout q, k;        // each relative to its own region
  int64_t off_k;        // start of the key-tile plan's region
  int64_t off_dvec;     // D = <dout, out>, [heads][tokens] fp32 (varlen only)
  int64_t total;
};

BwdLayout bwd_layout_varlen(int64_t tokens, int64_t segments, int32_t heads, int32_t kv_heads) {
  const int G = heads / kv_heads;
  BwdLayout B{};
  B.q = ws_layout(segments, std::min<int64_t>(kSortCap + 1, ceil_div(tokens, bwd_q_rows(G)) + segments));
  B.k = ws_layout(segments, std::min<int64_t>(kSortCap + 1, ceil_div(tokens, bwd_k_rows(G)) + segments));
  B.off_k = B.q.total;
  B.off_dvec = B.off_k + B.k.total;
  B.total = align256(B.off_dvec + (int64_t)heads * tokens * 4);
  return B;
}

// Block path: the workspace is split in two halves, each holding as many runs as fit.
lb_status bwd_layout_block(int32_t n_q, int32_t n_kv, int32_t heads, int32_t kv_heads, size_t bytes,
                           BwdLayout* B) {
  const int G = heads / kv_heads;
  const int64_t half = ((int64_t)bytes / 2) & ~int64_t(255);
  const int64_t max_runs = std::max<int64_t>(1, std::max(n_q, n_kv));
  auto fit = [&](int64_t side_tokens, int bm, WsLayout* L) {
    auto layout_for = [&](int64_t f) { return ws_layout(f, std::min<int64_t>(kSortCap, ceil_div(side_tokens, bm) + f)); };
    if (layout_for(1).total > half) return false;
    int64_t lo = 1, hi = max_runs;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (layout_for(mid).total <= half) lo = mid; else hi = mid - 1;
    }
    *L = layout_for(lo);
    return true;
  };
  if (!fit(n_q, bwd_q_rows(G), &B->q) || !fit(n_kv, bwd_k_rows(G), &B->k)) return LB_EWORKSPACE;
  B->off_k = half;
  B->off_dvec = 2 * half;
  B->total = 2 * half;
  return LB_OK;
}

BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* dout, const float* lse, const float* dvec,
                 void* dq, void* dk, void* dv, int32_t n_q, int32_t n_kv, int32_t heads, int32_t kv_heads,
                 int32_t d) {
  BwdArgs b{};
  b.q = q; b.k = k; b.v = v; b.dout = dout; b.lse = lse; b.dvec = dvec;
  b.dq = dq; b.dk = dk; b.dv = dv;
  b.n_q = n_q; b.n_kv = n_kv;
  b.heads = heads; b.kv_heads = kv_heads; b.group = heads / kv_heads;
  b.scale = (float)(1.0 / std::sqrt((double)d));
  b.scale_log2 = (float)(1.0 / std::sqrt((double)d) * 1.4426950408889634);
  return b;
}

// Checks and layout of a slice-list plan; *L receives the layout when LB_OK.
lb_status prepare_plan_slices(const lb_mask_slice* slices, int32_t n_slices, int32_t n_q, int32_t n_kv, int32_t heads,
                              int32_t kv_heads, int32_t d, void* workspace, size_t workspace_bytes, WsLayout* L) {
  if (!slices || !workspace || n_slices < 1 || n_q < 0 || n_kv < 0) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  if (!aligned(slices, 4)) return LB_EINVAL;
  if (!aligned(workspace, 256)) return LB_EWORKSPACE;
  // fragments: one per query range, and one per run of rows no slice covers
  const int64_t frags = 2 * (int64_t)n_slices + 1;
  const int64_t tiles = ceil_div(n_q, tile_rows_for_group(heads / kv_heads)) + frags;
  if (tiles > kSortCap) return LB_EUNSUPPORTED;
  *L = ws_layout(frags, tiles);
  if ((int64_t)workspace_bytes < L->total) return LB_EWORKSPACE;
  return LB_OK;
}

lb_status launch_plan_slices(const lb_mask_slice* slices, int32_t n_slices, int32_t n_q, int32_t n_kv, int32_t heads,
                             int32_t kv_heads, void* workspace, const WsLayout& L, hipStream_t stream) {
  PlanArgs p{};
  p.mode = kPlanSlices;
  p.slices = slices;
  p.n_slices = n_slices;
  p.n_q = n_q;
  p.n_kv = n_kv;
  p.tile_rows = tile_rows_for_group(heads / kv_heads);
  p.heads = heads;
  p.kv_heads = kv_heads;
  p.ws = static_cast<char*>(workspace);
  p.L = L;
  return launch_plan(p, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

bool read_header(const void* ws, size_t bytes, WsHeader* h, hipStream_t s) {
  if (!ws || bytes < sizeof(WsHeader)) return false;
  if (hipStreamSynchronize(s) != hipSuccess) return false;
  return hipMemcpy(h, ws, sizeof(WsHeader), hipMemcpyDeviceToHost) == hipSuccess;
}

}  // namespace

extern "C" {

int32_t lb_tile_rows(int32_t heads, int32_t kv_heads, int32_t d) {
  if (!group_supported(heads, kv_heads) || (d != 64 && d != 128)) return -1;
  return tile_rows_for_group(heads / kv_heads);
}

size_t lb_workspace_bytes(int32_t max_tokens, int32_t max_segments, int32_t heads, int32_t kv_heads) {
  if (max_tokens < 0 || max_segments < 1 || !group_supported(heads, kv_heads)) return 0;
  const int bm = tile_rows_for_group(heads / kv_heads);
  const int64_t tiles = std::min<int64_t>(kSortCap, ceil_div(max_tokens, bm) + max_segments);
  return (size_t)ws_layout(max_segments, tiles).total;
}

lb_status lb_plan_varlen(const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens, int32_t heads,
                         int32_t kv_heads, int32_t d, int32_t mask_kind, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  WsLayout L;
  lb_status st = prepare_plan_varlen(cu_seqlens, n_seg, total_tokens, heads, kv_heads, d, mask_kind, workspace,
                                     workspace_bytes, &L);
  if (st != LB_OK) return st;
  return launch_plan_varlen(cu_seqlens, n_seg, total_tokens, heads, kv_heads, mask_kind, workspace, L, stream);
}

lb_status lb_plan_varlen_weighted(const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens,
                                  int32_t heads, int32_t kv_heads, int32_t d, int32_t mask_kind,
                                  uint32_t block_weight, uint32_t pair_weight, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (block_weight < 1 || block_weight > LB_LPT_BLOCK_WEIGHT_MAX || pair_weight > LB_LPT_PAIR_WEIGHT_MAX)
    return LB_EINVAL;
  WsLayout L;
  lb_status st = prepare_plan_varlen(cu_seqlens, n_seg, total_tokens, heads, kv_heads, d, mask_kind, workspace,
                                     workspace_bytes, &L);
  if (st != LB_OK) return st;
  return launch_plan_varlen(cu_seqlens, n_seg, total_tokens, heads, kv_heads, mask_kind, workspace, L, stream,
                            block_weight, pair_weight, LB_ORDER_LPT);
}

lb_status lb_plan_varlen_ordered(const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens, int32_t heads,
                                 int32_t kv_heads, int32_t d, int32_t mask_kind, uint32_t block_weight,
                                 uint32_t pair_weight, int32_t order, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (block_weight < 1 || block_weight > LB_LPT_BLOCK_WEIGHT_MAX || pair_weight > LB_LPT_PAIR_WEIGHT_MAX)
    return LB_EINVAL;
  if (order != LB_ORDER_LPT && order != LB_ORDER_DOCUMENTS) return LB_EINVAL;
  WsLayout L;
  lb_status st = prepare_plan_varlen(cu_seqlens, n_seg, total_tokens, heads, kv_heads, d, mask_kind, workspace,
                                     workspace_bytes, &L);
  if (st != LB_OK) return st;
  return launch_plan_varlen(cu_seqlens, n_seg, total_tokens, heads, kv_heads, mask_kind, workspace, L, stream,
                            block_weight, pair_weight, order);
}

lb_status lb_plan_block(const int32_t* q_pos, const int32_t* q_doc, int32_t n_q, const int32_t* kv_pos,
                        const int32_t* kv_doc, int32_t n_kv, int32_t heads, int32_t kv_heads, int32_t d,
                        int32_t shared_doc, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (shared_doc < -1) return LB_EINVAL;
  WsLayout L;
  lb_status st = prepare_plan_block(q_pos, q_doc, n_q, kv_pos, kv_doc, n_kv, heads, kv_heads, d, workspace,
                                    workspace_bytes, &L);
  if (st != LB_OK) return st;
  return launch_plan_block(q_pos, q_doc, n_q, kv_pos, kv_doc, n_kv, heads, kv_heads, shared_doc, workspace, L,
                           stream);
}

lb_status lb_plan_block_steps(const int32_t* q_pos, const int32_t* q_doc, int32_t n_q,
                              const int32_t* const* kv_pos, const int32_t* const* kv_doc, const int32_t* n_kv,
                              int32_t n_steps, int32_t heads, int32_t kv_heads, int32_t d, int32_t shared_doc,
                              void* const* workspaces, const size_t* workspace_bytes, hipStream_t stream) {
  if (n_steps < 1 || n_steps > kMaxPlanSteps || shared_doc < -1) return LB_EINVAL;
  if (!kv_pos || !kv_doc || !n_kv || !workspaces || !workspace_bytes) return LB_EINVAL;
  PlanBatch b{};
  for (int s = 0; s < n_steps; ++s) {
    for (int r = 0; r < s; ++r)
      if (workspaces[r] == workspaces[s]) return LB_EINVAL;
    WsLayout L;
    lb_status st = prepare_plan_block(q_pos, q_doc, n_q, kv_pos[s], kv_doc[s], n_kv[s], heads, kv_heads, d,
                                      workspaces[s], workspace_bytes[s], &L);
    if (st != LB_OK) return st;
    b.step[s] = block_plan_args(q_pos, q_doc, n_q, kv_pos[s], kv_doc[s], n_kv[s], heads, kv_heads, shared_doc,
                                workspaces[s], L);
  }
  return launch_plan_steps(b, n_steps, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

size_t lb_ring_workspace_bytes(int32_t n_steps, int32_t max_tokens, int32_t max_segments, int32_t heads,
                               int32_t kv_heads) {
  if (n_steps < 1 || n_steps > kMaxPlanSteps || max_tokens < 0 || max_segments < 1 ||
      !group_supported(heads, kv_heads))
    return 0;
  const int bm = tile_rows_for_group(heads / kv_heads);
  const int64_t tiles = (int64_t)n_steps * std::min<int64_t>(kSortCap, ceil_div(max_tokens, bm) + max_segments);
  return (size_t)align256(kRingTilesOffset + tiles * (int64_t)sizeof(lb_plan_tile));
}

namespace {
lb_status ring_merge_args(void* const* workspaces, const size_t* workspace_bytes, const int32_t* n_kv,
                          int32_t n_steps, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d,
                          void* ring_workspace, size_t ring_workspace_bytes, RingMergeArgs* out) {
  if (n_steps < 1 || n_steps > kMaxPlanSteps || n_q < 0) return LB_EINVAL;
  if (!workspaces || !workspace_bytes || !n_kv || !ring_workspace) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  if (!aligned(ring_workspace, 256)) return LB_EWORKSPACE;
  const int64_t cap = ((int64_t)ring_workspace_bytes - kRingTilesOffset) / (int64_t)sizeof(lb_plan_tile);
  if (cap < 1) return LB_EWORKSPACE;
  RingMergeArgs m{};
  for (int s = 0; s < n_steps; ++s) {
    if (!workspaces[s] || n_kv[s] < 0) return LB_EINVAL;
    if (!aligned(workspaces[s], 256) || workspace_bytes[s] < sizeof(WsHeader)) return LB_EWORKSPACE;
    if (workspaces[s] == ring_workspace) return LB_EINVAL;
    m.step_ws[s] = static_cast<const char*>(workspaces[s]);
    m.step_ws_bytes[s] = (int64_t)workspace_bytes[s];
    m.n_kv[s] = n_kv[s];
  }
  m.n_steps = n_steps;
  m.n_q = n_q;
  m.heads = heads;
  m.kv_heads = kv_heads;
  m.ring = static_cast<char*>(ring_workspace);
  m.ring_cap = (int32_t)std::min<int64_t>(cap, INT32_MAX);
  m.transposed = 0;
  *out = m;
  return LB_OK;
}
}  // namespace

lb_status lb_plan_ring(void* const* workspaces, const size_t* workspace_bytes, const int32_t* n_kv,
                       int32_t n_steps, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d,
                       void* ring_workspace, size_t ring_workspace_bytes, hipStream_t stream) {
  RingMergeArgs m{};
  const lb_status st = ring_merge_args(workspaces, workspace_bytes, n_kv, n_steps, n_q, heads, kv_heads, d,
                                       ring_workspace, ring_workspace_bytes, &m);
  if (st != LB_OK) return st;
  return launch_ring_merge(m, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

lb_status lb_plan_ring_fused(void* const* workspaces, const size_t* workspace_bytes, const int32_t* n_kv,
                             int32_t n_steps, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d,
                             void* ring_workspace, size_t ring_workspace_bytes, hipStream_t stream) {
  RingMergeArgs m{};
  const lb_status st = ring_merge_args(workspaces, workspace_bytes, n_kv, n_steps, n_q, heads, kv_heads, d,
                                       ring_workspace, ring_workspace_bytes, &m);
  if (st != LB_OK) return st;
  return launch_ring_fuse(m, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

namespace {
// fused: one result (out[0], lse[0]) for every step instead of a partial per step
lb_status ring_attn_run(const void* q, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d, int32_t n_steps,
                        const void* const* k, const void* const* v, const int32_t* n_kv, float* const* out,
                        float* const* lse, void* ring_workspace, size_t ring_workspace_bytes, bool fused,
                        hipStream_t stream) {
  if (n_steps < 1 || n_steps > kMaxPlanSteps || n_q < 0) return LB_EINVAL;
  if (!q || !k || !v || !n_kv || !out || !lse || !ring_workspace) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  if (!aligned(q, 16)) return LB_EINVAL;
  if (!aligned(ring_workspace, 256)) return LB_EWORKSPACE;
  if ((int64_t)ring_workspace_bytes < kRingTilesOffset) return LB_EWORKSPACE;
  RingSteps r{};
  const int n_out = fused ? 1 : n_steps;
  for (int s = 0; s < n_out; ++s) {
    if (!out[s] || !lse[s]) return LB_EINVAL;
    if (!aligned(out[s], 16) || !aligned(lse[s], 4)) return LB_EINVAL;
    for (int o = 0; o < s; ++o)
      if (out[o] == out[s] || lse[o] == lse[s]) return LB_EINVAL;  // each step writes its own partial
  }
  for (int s = 0; s < n_steps; ++s) {
    if (n_kv[s] < 0) return LB_EINVAL;
    if (n_kv[s] > 0 && (!k[s] || !v[s] || !aligned(k[s], 16) || !aligned(v[s], 16))) return LB_EINVAL;
    r.k[s] = n_kv[s] > 0 ? k[s] : q;
    r.v[s] = n_kv[s] > 0 ? v[s] : q;
    r.out[s] = out[fused ? 0 : s];
    r.lse[s] = lse[fused ? 0 : s];
    r.n_kv[s] = n_kv[s];
  }
  r.n_steps = n_steps;
  if (n_q == 0) return LB_OK;
  int workers = 0;
  st = persistent_workers(&workers);
  if (st != LB_OK) return st;
  AttnArgs at{};
  at.q = q;
  at.k = q;
  at.v = q;
  at.out = out[0];
  at.lse = lse[0];
  at.n_q = n_q;
  at.n_kv = 0;
  at.heads = heads;
  at.kv_heads = kv_heads;
  at.group = heads / kv_heads;
  at.scale_log2 = (float)(1.0 / std::sqrt((double)d) * 1.4426950408889634);
  at.ws = static_cast<char*>(ring_workspace);
  at.ws_bytes = (int64_t)ring_workspace_bytes;
  return launch_ring_attention(at, r, d, workers, fused, stream) == hipSuccess ? LB_OK : LB_EHIP;
}
}  // namespace

lb_status lb_ring_attn_run(const void* q, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d, int32_t n_steps,
                           const void* const* k, const void* const* v, const int32_t* n_kv, float* const* out,
                           float* const* lse, void* ring_workspace, size_t ring_workspace_bytes,
                           hipStream_t stream) {
  return ring_attn_run(q, n_q, heads, kv_heads, d, n_steps, k, v, n_kv, out, lse, ring_workspace,
                       ring_workspace_bytes, false, stream);
}

lb_status lb_ring_attn_run_fused(const void* q, int32_t n_q, int32_t heads, int32_t kv_heads, int32_t d,
                                 int32_t n_steps, const void* const* k, const void* const* v, const int32_t* n_kv,
                                 float* out, float* lse, void* ring_workspace, size_t ring_workspace_bytes,
                                 hipStream_t stream) {
  float* const outs[1] = {out};
  float* const lses[1] = {lse};
  return ring_attn_run(q, n_q, heads, kv_heads, d, n_steps, k, v, n_kv, outs, lses, ring_workspace,
                       ring_workspace_bytes, true, stream);
}

lb_status lb_attn_run(const void* q, const void* k, const void* v, int32_t n_q, int32_t n_kv, int32_t heads,
                      int32_t kv_heads, int32_t d, int32_t out_f32, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  lb_status st = check_run(q, k, v, n_q, n_kv, heads, kv_heads, d, out, lse, workspace, workspace_bytes);
  if (st != LB_OK) return st;
  if (n_q == 0) return LB_OK;
  return launch_run(q, k, v, n_q, n_kv, heads, kv_heads, d, out_f32 != 0, out, lse, workspace, workspace_bytes,
                    stream);
}

lb_status lb_attn_run_lower(const void* q, const void* k, const void* v, int32_t n_q, int32_t n_kv, int32_t heads,
                            int32_t kv_heads, int32_t d, int32_t out_f32, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  lb_status st = check_run(q, k, v, n_q, n_kv, heads, kv_heads, d, out, lse, workspace, workspace_bytes);
  if (st != LB_OK) return st;
  if (n_q == 0) return LB_OK;
  return launch_run(q, k, v, n_q, n_kv, heads, kv_heads, d, out_f32 != 0, out, lse, workspace, workspace_bytes,
                    stream, true);
}

lb_status lb_varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                             int32_t n_seg, int32_t total_tokens, int32_t heads, int32_t kv_heads,
                             int32_t d, int32_t mask_kind, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!k || !v) return LB_EINVAL;
  lb_status st = check_run(q, k, v, total_tokens, total_tokens, heads, kv_heads, d, out, lse, workspace,
                           workspace_bytes);
  if (st != LB_OK) return st;
  WsLayout L;
  st = prepare_plan_varlen(cu_seqlens, n_seg, total_tokens, heads, kv_heads, d, mask_kind, workspace,
                           workspace_bytes, &L);
  if (st != LB_OK) return st;
  if (total_tokens == 0) return LB_OK;
  st = launch_plan_varlen(cu_seqlens, n_seg, total_tokens, heads, kv_heads, mask_kind, workspace, L, stream);
  if (st != LB_OK) return st;
  return launch_run(q, k, v, total_tokens, total_tokens, heads, kv_heads, d, false, out, lse, workspace,
                    workspace_bytes, stream);
}

// The plan workspace of lb_varlen_attn_fwd_noalloc.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address (one per GPU, each GPU holding its own
// copy) is looked up once per device and only that address is handed to kernels.
static __device__ __align__(256) char scratch[LB_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's scratch address; looked up on the first call made on that device.
lb_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LB_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return LB_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LB_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LB_OK;
}
}  // namespace

lb_status lb_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                     int32_t n_seg, int32_t total_tokens, int32_t heads, int32_t kv_heads,
                                     int32_t d, int32_t mask_kind, void* out, float* lse, hipStream_t stream) {
  if (n_seg < 1 || total_tokens < 0) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  // the plan this call needs, against the array's fixed size, before touching the device
  const int bm = tile_rows_for_group(heads / kv_heads);
  const int64_t tiles = ceil_div(total_tokens, bm) + n_seg;
  if (tiles > kSortCap) return LB_EUNSUPPORTED;
  if (ws_layout(n_seg, tiles).total > (int64_t)LB_NOALLOC_SCRATCH_BYTES) return LB_EWORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != LB_OK) return st;
  return lb_varlen_attn_fwd(q, k, v, cu_seqlens, n_seg, total_tokens, heads, kv_heads, d, mask_kind, out, lse, ws,
                            LB_NOALLOC_SCRATCH_BYTES, stream);
}

lb_status lb_block_attn_fwd(const void* q_shard, int32_t n_q, const void* kv_chunk, int32_t n_kv,
                            const int32_t* q_pos, const int32_t* kv_pos, const int32_t* q_doc,
                            const int32_t* kv_doc, int32_t heads, int32_t kv_heads, int32_t d,
                            int32_t shared_doc, float* out, float* lse, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  const __bf16* kbase = static_cast<const __bf16*>(kv_chunk);
  const __bf16* vbase = kbase ? kbase + (int64_t)n_kv * kv_heads * d : nullptr;
  if (n_kv < 0 || kv_heads <= 0 || d <= 0 || shared_doc < -1) return LB_EINVAL;
  lb_status st = check_run(q_shard, kbase, vbase, n_q, n_kv, heads, kv_heads, d, out, lse, workspace,
                           workspace_bytes);
  if (st != LB_OK) return st;
  WsLayout L;
  st = prepare_plan_block(q_pos, q_doc, n_q, kv_pos, kv_doc, n_kv, heads, kv_heads, d, workspace, workspace_bytes,
                          &L);
  if (st != LB_OK) return st;
  if (n_q == 0) return LB_OK;
  st = launch_plan_block(q_pos, q_doc, n_q, kv_pos, kv_doc, n_kv, heads, kv_heads, shared_doc, workspace, L,
                         stream);
  if (st != LB_OK) return st;
  return launch_run(q_shard, kbase, vbase, n_q, n_kv, heads, kv_heads, d, true, out, lse, workspace,
                    workspace_bytes, stream);
}

lb_status lb_lse_merge(float* out_a, float* lse_a, const float* out_b, const float* lse_b, int32_t n_rows,
                       int32_t heads, int32_t d, hipStream_t stream) {
  if (!out_a || !lse_a || !out_b || !lse_b) return LB_EINVAL;
  if (n_rows < 0 || heads <= 0 || d <= 0) return LB_EINVAL;
  if (d % 4 != 0 || d > 1024) return LB_EUNSUPPORTED;
  if (!aligned(out_a, 16) || !aligned(out_b, 16) || !aligned(lse_a, 4) || !aligned(lse_b, 4)) return LB_EINVAL;
  if (n_rows == 0) return LB_OK;
  MergeArgs m{out_a, lse_a, out_b, lse_b, n_rows, heads, d};
  return launch_lse_merge(m, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

lb_status lb_lse_merge_parts(float* const* out, float* const* lse, int32_t n_parts, int32_t n_rows, int32_t heads,
                             int32_t d, hipStream_t stream) {
  if (!out || !lse || n_parts < 2 || n_parts > kMaxPlanSteps) return LB_EINVAL;
  if (n_rows < 0 || heads <= 0 || d <= 0) return LB_EINVAL;
  if (d % 4 != 0 || d > 1024) return LB_EUNSUPPORTED;
  MergePartsArgs m{};
  for (int i = 0; i < n_parts; ++i) {
    if (!out[i] || !lse[i] || !aligned(out[i], 16) || !aligned(lse[i], 4)) return LB_EINVAL;
    for (int o = 0; o < i; ++o)
      if (out[o] == out[i] || lse[o] == lse[i]) return LB_EINVAL;
    m.out[i] = out[i];
    m.lse[i] = lse[i];
  }
  m.n_parts = n_parts;
  m.n_rows = n_rows;
  m.heads = heads;
  m.d = d;
  if (n_rows == 0) return LB_OK;
  return launch_lse_merge_parts(m, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

lb_status lb_plan_slices(const lb_mask_slice* slices, int32_t n_slices, int32_t n_q, int32_t n_kv, int32_t heads,
                         int32_t kv_heads, int32_t d, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  WsLayout L;
  lb_status st = prepare_plan_slices(slices, n_slices, n_q, n_kv, heads, kv_heads, d, workspace, workspace_bytes, &L);
  if (st != LB_OK) return st;
  return launch_plan_slices(slices, n_slices, n_q, n_kv, heads, kv_heads, workspace, L, stream);
}

lb_status lb_slices_attn_fwd(const void* q, const void* k, const void* v, const lb_mask_slice* slices,
                             int32_t n_slices, int32_t n_q, int32_t n_kv, int32_t heads, int32_t kv_heads, int32_t d,
                             void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!k || !v) return LB_EINVAL;
  lb_status st = check_run(q, k, v, n_q, n_kv, heads, kv_heads, d, out, lse, workspace, workspace_bytes);
  if (st != LB_OK) return st;
  WsLayout L;
  st = prepare_plan_slices(slices, n_slices, n_q, n_kv, heads, kv_heads, d, workspace, workspace_bytes, &L);
  if (st != LB_OK) return st;
  if (n_q == 0) return LB_OK;
  // rows no slice covers are the plan's tiles without a key span: the attention launch sets
  // their lse to -inf
  st = launch_plan_slices(slices, n_slices, n_q, n_kv, heads, kv_heads, workspace, L, stream);
  if (st != LB_OK) return st;
  return launch_run(q, k, v, n_q, n_kv, heads, kv_heads, d, false, out, lse, workspace, workspace_bytes, stream,
                    true);
}

size_t lb_bwd_workspace_bytes(int32_t max_tokens, int32_t max_segments, int32_t heads, int32_t kv_heads) {
  if (max_tokens < 0 || max_segments < 1 || !group_supported(heads, kv_heads)) return 0;
  return (size_t)bwd_layout_varlen(max_tokens, max_segments, heads, kv_heads).total;
}

size_t lb_bwd_key_plan_offset(int32_t block_path, int32_t n_q, int32_t n_kv, int32_t n_seg, int32_t heads,
                              int32_t kv_heads, size_t workspace_bytes) {
  if (!group_supported(heads, kv_heads) || n_q < 0 || n_kv < 0) return 0;
  if (block_path) {
    BwdLayout B;
    return bwd_layout_block(n_q, n_kv, heads, kv_heads, workspace_bytes, &B) == LB_OK ? (size_t)B.off_k : 0;
  }
  if (n_seg < 1) return 0;
  return (size_t)bwd_layout_varlen(n_q, n_seg, heads, kv_heads).off_k;
}

lb_status lb_attn_bwd_rowdot(const void* out, int32_t out_f32, const void* dout, int32_t n_rows, int32_t heads,
                             int32_t d, float* dvec, hipStream_t stream) {
  if (!out || !dout || !dvec || n_rows < 0 || heads <= 0) return LB_EINVAL;
  if (d != 64 && d != 128) return LB_EUNSUPPORTED;
  if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(dvec, 4)) return LB_EINVAL;
  if (n_rows == 0) return LB_OK;
  return launch_bwd_rowdot(out, out_f32 != 0, dout, n_rows, heads, d, dvec, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

lb_status lb_varlen_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, const int32_t* cu_seqlens, int32_t n_seg, int32_t total_tokens,
                             int32_t heads, int32_t kv_heads, int32_t d, int32_t mask_kind, void* dq, void* dk,
                             void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !dout || !lse || !cu_seqlens || !dq || !dk || !dv || !workspace) return LB_EINVAL;
  if (n_seg < 1 || total_tokens < 0) return LB_EINVAL;
  if (mask_kind != LB_MASK_CAUSAL_DOC && mask_kind != LB_MASK_SHARED_QUESTION) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  for (const void* p : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned(p, 16)) return LB_EINVAL;
  if (!aligned(lse, 4) || !aligned(cu_seqlens, 4)) return LB_EINVAL;
  if (!aligned(workspace, 256)) return LB_EWORKSPACE;
  const BwdLayout B = bwd_layout_varlen(total_tokens, n_seg, heads, kv_heads);
  if (B.q.cap_tiles > kSortCap || B.k.cap_tiles > kSortCap) return LB_EUNSUPPORTED;
  if ((int64_t)workspace_bytes < B.total) return LB_EWORKSPACE;
  if (total_tokens == 0) return LB_OK;
  char* ws = static_cast<char*>(workspace);
  float* dvec = reinterpret_cast<float*>(ws + B.off_dvec);
  PlanBatch pb{};
  for (int side = 0; side < 2; ++side) {
    PlanArgs& p = pb.step[side];
    p.mode = mask_kind == LB_MASK_CAUSAL_DOC ? kPlanCausalDoc : kPlanSharedQuestion;
    p.transposed = side;
    p.order = LB_ORDER_DOCUMENTS;  // a document's items share its rows (dK/dV) or keys (dQ) in L2
    p.cu_seqlens = cu_seqlens;
    p.n_seg = n_seg;
    p.total_tokens = total_tokens;
    p.tile_rows = side == 0 ? bwd_q_rows(heads / kv_heads) : bwd_k_rows(heads / kv_heads);
    p.heads = heads;
    p.kv_heads = kv_heads;
    p.ws = ws + (side == 0 ? 0 : B.off_k);
    p.L = side == 0 ? B.q : B.k;
  }
  if (launch_plan_steps(pb, 2, stream) != hipSuccess) return LB_EHIP;
  if (launch_bwd_rowdot(out, false, dout, total_tokens, heads, d, dvec, stream) != hipSuccess) return LB_EHIP;
  int workers = 0;
  st = persistent_workers(&workers);
  if (st != LB_OK) return st;
  BwdArgs b = bwd_args(q, k, v, dout, lse, dvec, dq, dk, dv, total_tokens, total_tokens, heads, kv_heads, d);
  b.ws = ws;
  b.ws_bytes = B.q.total;
  if (launch_bwd_dq(b, d, false, workers, stream) != hipSuccess) return LB_EHIP;
  b.ws = ws + B.off_k;
  b.ws_bytes = B.k.total;
  return launch_bwd_dkv(b, d, false, workers, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

lb_status lb_block_attn_bwd(const void* q_shard, int32_t n_q, const void* kv_chunk, int32_t n_kv, const void* dout,
                            const float* lse, const float* dvec, const int32_t* q_pos, const int32_t* kv_pos,
                            const int32_t* q_doc, const int32_t* kv_doc, int32_t heads, int32_t kv_heads, int32_t d,
                            int32_t shared_doc, float* dq, float* dkv, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  if (n_q < 0 || n_kv < 0 || shared_doc < -1) return LB_EINVAL;
  if (!q_shard || !dout || !lse || !dvec || !q_pos || !q_doc || !dq || !workspace) return LB_EINVAL;
  if (n_kv > 0 && (!kv_chunk || !kv_pos || !kv_doc || !dkv)) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  if (!aligned(q_shard, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(lse, 4) || !aligned(dvec, 4))
    return LB_EINVAL;
  if (n_kv > 0 && (!aligned(kv_chunk, 16) || !aligned(dkv, 16))) return LB_EINVAL;
  if (!aligned(q_pos, 4) || !aligned(q_doc, 4) || (n_kv > 0 && (!aligned(kv_pos, 4) || !aligned(kv_doc, 4))))
    return LB_EINVAL;
  if (!aligned(workspace, 256)) return LB_EWORKSPACE;
  BwdLayout B;
  st = bwd_layout_block(n_q, n_kv, heads, kv_heads, workspace_bytes, &B);
  if (st != LB_OK) return st;
  if (n_q == 0 || n_kv == 0) return LB_OK;
  char* ws = static_cast<char*>(workspace);
  const __bf16* kbase = static_cast<const __bf16*>(kv_chunk);
  const __bf16* vbase = kbase + (int64_t)n_kv * kv_heads * d;
  PlanBatch pb{};
  for (int side = 0; side < 2; ++side) {
    pb.step[side] = block_plan_args(q_pos, q_doc, n_q, kv_pos, kv_doc, n_kv, heads, kv_heads, shared_doc,
                                    ws + (side == 0 ? 0 : B.off_k), side == 0 ? B.q : B.k);
    pb.step[side].transposed = side;
    pb.step[side].tile_rows = side == 0 ? bwd_q_rows(heads / kv_heads) : bwd_k_rows(heads / kv_heads);
  }
  if (launch_plan_steps(pb, 2, stream) != hipSuccess) return LB_EHIP;
  int workers = 0;
  st = persistent_workers(&workers);
  if (st != LB_OK) return st;
  float* dk = dkv;
  float* dv = dkv + (int64_t)n_kv * kv_heads * d;
  BwdArgs b = bwd_args(q_shard, kbase, vbase, dout, lse, dvec, dq, dk, dv, n_q, n_kv, heads, kv_heads, d);
  b.ws = ws;
  b.ws_bytes = B.off_k;
  if (launch_bwd_dq(b, d, true, workers, stream) != hipSuccess) return LB_EHIP;
  b.ws = ws + B.off_k;
  b.ws_bytes = (int64_t)workspace_bytes - B.off_k;
  return launch_bwd_dkv(b, d, true, workers, stream) == hipSuccess ? LB_OK : LB_EHIP;
}

namespace {
// q_ring: null for one dQ launch per step, else the workspace the steps' query-tile plans are
// fused into for one dQ launch over every step
lb_status bwd_ring(const void* q_shard, int32_t n_q, const void* dout, const float* lse, const float* dvec,
                   const int32_t* q_pos, const int32_t* q_doc, int32_t heads, int32_t kv_heads, int32_t d,
                   int32_t shared_doc, int32_t n_steps, const void* const* kv_chunks, const int32_t* n_kv,
                   const int32_t* const* kv_pos, const int32_t* const* kv_doc, float* dq, float* const* dkv,
                   void* const* workspaces, const size_t* workspace_bytes, void* ring_workspace,
                   size_t ring_workspace_bytes, void* q_ring, size_t q_ring_bytes, hipStream_t stream) {
  if (n_q < 0 || shared_doc < -1 || n_steps < 1 || 2 * n_steps > kMaxPlanSteps) return LB_EINVAL;
  if (!q_shard || !dout || !lse || !dvec || !q_pos || !q_doc || !dq || !ring_workspace) return LB_EINVAL;
  if (!kv_chunks || !n_kv || !kv_pos || !kv_doc || !dkv || !workspaces || !workspace_bytes) return LB_EINVAL;
  lb_status st = check_heads(heads, kv_heads, d);
  if (st != LB_OK) return st;
  if (!aligned(q_shard, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(lse, 4) || !aligned(dvec, 4) ||
      !aligned(q_pos, 4) || !aligned(q_doc, 4))
    return LB_EINVAL;
  if (!aligned(ring_workspace, 256)) return LB_EWORKSPACE;
  const int64_t cap = ((int64_t)ring_workspace_bytes - kRingTilesOffset) / (int64_t)sizeof(lb_plan_tile);
  if (cap < 1) return LB_EWORKSPACE;
  const int64_t q_cap = q_ring ? ((int64_t)q_ring_bytes - kRingTilesOffset) / (int64_t)sizeof(lb_plan_tile) : 0;
  if (q_ring && (!aligned(q_ring, 256) || q_cap < 1)) return LB_EWORKSPACE;
  if (q_ring && q_ring == ring_workspace) return LB_EINVAL;
  BwdLayout B[kMaxPlanSteps];
  for (int s = 0; s < n_steps; ++s) {
    if (n_kv[s] < 1 || !kv_chunks[s] || !kv_pos[s] || !kv_doc[s] || !dkv[s] || !workspaces[s]) return LB_EINVAL;
    if (!aligned(kv_chunks[s], 16) || !aligned(dkv[s], 16) || !aligned(kv_pos[s], 4) || !aligned(kv_doc[s], 4))
      return LB_EINVAL;
    for (int o = 0; o < s; ++o)
      if (workspaces[o] == workspaces[s] || dkv[o] == dkv[s]) return LB_EINVAL;
    if (workspaces[s] == ring_workspace || (q_ring && workspaces[s] == q_ring)) return LB_EINVAL;
    if (!aligned(workspaces[s], 256)) return LB_EWORKSPACE;
    st = bwd_layout_block(n_q, n_kv[s], heads, kv_heads, workspace_bytes[s], &B[s]);
    if (st != LB_OK) return st;
  }
  if (n_q == 0) return LB_OK;
  // every step's two plans in one launch, then the key-tile plans merged into one queue
  PlanBatch pb{};
  for (int s = 0; s < n_steps; ++s) {
    char* ws = static_cast<char*>(workspaces[s]);
    for (int side = 0; side < 2; ++side) {
      PlanArgs& p = pb.step[2 * s + side];
      p = block_plan_args(q_pos, q_doc, n_q, kv_pos[s], kv_doc[s], n_kv[s], heads, kv_heads, shared_doc,
                          ws + (side == 0 ? 0 : B[s].off_k), side == 0 ? B[s].q : B[s].k);
      p.transposed = side;
      p.tile_rows = side == 0 ? bwd_q_rows(heads / kv_heads) : bwd_k_rows(heads / kv_heads);
    }
  }
  if (launch_plan_steps(pb, 2 * n_steps, stream) != hipSuccess) return LB_EHIP;
  RingMergeArgs m{};
  for (int s = 0; s < n_steps; ++s) {
    m.step_ws[s] = static_cast<const char*>(workspaces[s]) + B[s].off_k;
    m.step_ws_bytes[s] = (int64_t)workspace_bytes[s] - B[s].off_k;
    m.n_kv[s] = n_kv[s];
  }
  m.n_steps = n_steps;
  m.n_q = n_q;
  m.heads = heads;
  m.kv_heads = kv_heads;
  m.ring = static_cast<char*>(ring_workspace);
  m.ring_cap = (int32_t)std::min<int64_t>(cap, INT32_MAX);
  m.transposed = 1;
  if (launch_ring_merge(m, stream) != hipSuccess) return LB_EHIP;
  if (q_ring) {  // the query-tile plans fused: one tile per query tile with every step's spans
    RingMergeArgs mq = m;
    for (int s = 0; s < n_steps; ++s) {
      mq.step_ws[s] = static_cast<const char*>(workspaces[s]);
      mq.step_ws_bytes[s] = B[s].off_k;
    }
    mq.ring = static_cast<char*>(q_ring);
    mq.ring_cap = (int32_t)std::min<int64_t>(q_cap, INT32_MAX);
    mq.transposed = 0;
    if (launch_ring_fuse(mq, stream) != hipSuccess) return LB_EHIP;
  }
  int workers = 0;
  st = persistent_workers(&workers);
  if (st != LB_OK) return st;
  // dq: the steps in order, each adding into the one fp32 buffer
  RingBwdSteps r{};
  for (int s = 0; s < n_steps; ++s) {
    const __bf16* kbase = static_cast<const __bf16*>(kv_chunks[s]);
    const __bf16* vbase = kbase + (int64_t)n_kv[s] * kv_heads * d;
    float* dk = dkv[s];
    float* dv = dkv[s] + (int64_t)n_kv[s] * kv_heads * d;
    BwdArgs b = bwd_args(q_shard, kbase, vbase, dout, lse, dvec, dq, dk, dv, n_q, n_kv[s], heads, kv_heads, d);
    b.ws = static_cast<char*>(workspaces[s]);
    b.ws_bytes = B[s].off_k;
    if (!q_ring && launch_bwd_dq(b, d, true, workers, stream) != hipSuccess) return LB_EHIP;
    r.k[s] = kbase;
    r.v[s] = vbase;
    r.dk[s] = dk;
    r.dv[s] = dv;
    r.n_kv[s] = n_kv[s];
  }
  r.n_steps = n_steps;
  if (q_ring) {  // dq: one launch, each query tile against every step's keys and values
    BwdArgs bq = bwd_args(q_shard, q_shard, q_shard, dout, lse, dvec, dq, r.dk[0], r.dv[0], n_q, 0, heads, kv_heads, d);
    bq.ws = static_cast<char*>(q_ring);
    bq.ws_bytes = (int64_t)q_ring_bytes;
    if (launch_bwd_dq_fused(bq, r, d, workers, stream) != hipSuccess) return LB_EHIP;
  }
  // dk, dv: every step's key tiles in one launch, each step's gradients into its own buffer
  BwdArgs b = bwd_args(q_shard, q_shard, q_shard, dout, lse, dvec, dq, r.dk[0], r.dv[0], n_q, 0, heads, kv_heads, d);
  b.ws = static_cast<char*>(ring_workspace);
  b.ws_bytes = (int64_t)ring_workspace_bytes;
  return launch_bwd_dkv_ring(b, r, d, workers, stream) == hipSuccess ? LB_OK : LB_EHIP;
}
}  // namespace

lb_status lb_block_attn_bwd_ring(const void* q_shard, int32_t n_q, const void* dout, const float* lse,
                                 const float* dvec, const int32_t* q_pos, const int32_t* q_doc, int32_t heads,
                                 int32_t kv_heads, int32_t d, int32_t shared_doc, int32_t n_steps,
                                 const void* const* kv_chunks, const int32_t* n_kv, const int32_t* const* kv_pos,
                                 const int32_t* const* kv_doc, float* dq, float* const* dkv,
                                 void* const* workspaces, const size_t* workspace_bytes, void* ring_workspace,
                                 size_t ring_workspace_bytes, hipStream_t stream) {
  return bwd_ring(q_shard, n_q, dout, lse, dvec, q_pos, q_doc, heads, kv_heads, d, shared_doc, n_steps, kv_chunks,
                  n_kv, kv_pos, kv_doc, dq, dkv, workspaces, workspace_bytes, ring_workspace, ring_workspace_bytes,
                  nullptr, 0, stream);
}

lb_status lb_block_attn_bwd_ring_fused(const void* q_shard, int32_t n_q, const void* dout, const float* lse,
                                       const float* dvec, const int32_t* q_pos, const int32_t* q_doc, int32_t heads,
                                       int32_t kv_heads, int32_t d, int32_t shared_doc, int32_t n_steps,
                                       const void* const* kv_chunks, const int32_t* n_kv,
                                       const int32_t* const* kv_pos, const int32_t* const* kv_doc, float* dq,
                                       float* const* dkv, void* const* workspaces, const size_t* workspace_bytes,
                                       void* ring_workspace, size_t ring_workspace_bytes, void* q_ring_workspace,
                                       size_t q_ring_workspace_bytes, hipStream_t stream) {
  if (!q_ring_workspace) return LB_EINVAL;
  return bwd_ring(q_shard, n_q, dout, lse, dvec, q_pos, q_doc, heads, kv_heads, d, shared_doc, n_steps, kv_chunks,
                  n_kv, kv_pos, kv_doc, dq, dkv, workspaces, workspace_bytes, ring_workspace, ring_workspace_bytes,
                  q_ring_workspace, q_ring_workspace_bytes, stream);
}

const char* lb_status_string(lb_status s) {
  switch (s) {
    case LB_OK: return "ok";
    case LB_EINVAL: return "invalid argument";
    case LB_EUNSUPPORTED: return "unsupported shape";
    case LB_EWORKSPACE: return "workspace too small or misaligned";
    case LB_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

lb_status lb_read_device_error(const void* workspace, size_t workspace_bytes, int32_t* host_err,
                               hipStream_t stream) {
  if (!host_err) return LB_EINVAL;
  WsHeader h;
  if (!workspace || workspace_bytes < sizeof(WsHeader)) return LB_EWORKSPACE;
  if (!read_header(workspace, workspace_bytes, &h, stream)) return LB_EHIP;
  *host_err = h.err;
  return LB_OK;
}

lb_status lb_read_plan(const void* workspace, size_t workspace_bytes, lb_plan_tile* host_tiles,
                       int32_t max_tiles, int32_t* n_tiles, hipStream_t stream) {
  if (!n_tiles || (max_tiles > 0 && !host_tiles) || max_tiles < 0) return LB_EINVAL;
  WsHeader h;
  if (!workspace || workspace_bytes < sizeof(WsHeader)) return LB_EWORKSPACE;
  if (!read_header(workspace, workspace_bytes, &h, stream)) return LB_EHIP;
  *n_tiles = h.n_tiles;
  const int n = std::min(h.n_tiles, max_tiles);
  if (n <= 0) return LB_OK;
  if (h.off_order + (int64_t)h.n_tiles * 4 > (int64_t)workspace_bytes ||
      h.off_tiles + (int64_t)h.n_tiles * (int64_t)sizeof(lb_plan_tile) > (int64_t)workspace_bytes)
    return LB_EWORKSPACE;
  std::vector<int32_t> order(h.n_tiles);
  std::vector<lb_plan_tile> nat(h.n_tiles);
  const char* base = static_cast<const char*>(workspace);
  if (hipMemcpy(nat.data(), base + h.off_tiles, nat.size() * sizeof(lb_plan_tile), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return LB_EHIP;
  if (h.magic == kRingMagic) {  // a ring workspace stores its tiles in queue order
    for (int i = 0; i < h.n_tiles; ++i) order[i] = i;
  } else if (hipMemcpy(order.data(), base + h.off_order, order.size() * 4, hipMemcpyDeviceToHost) != hipSuccess) {
    return LB_EHIP;
  }
  for (int i = 0; i < n; ++i) {
    const int32_t j = order[i];
    if (j < 0 || j >= h.n_tiles) return LB_EHIP;
    host_tiles[i] = nat[j];
  }
  return LB_OK;
}

lb_status lb_read_worker_timing(const void* workspace, size_t workspace_bytes, lb_worker_record* host_records,
                                int32_t max_records, int32_t* n_records, hipStream_t stream) {
  if (!n_records || (max_records > 0 && !host_records) || max_records < 0) return LB_EINVAL;
  WsHeader h;
  if (!workspace || workspace_bytes < sizeof(WsHeader)) return LB_EWORKSPACE;
  if (!read_header(workspace, workspace_bytes, &h, stream)) return LB_EHIP;
  *n_records = h.n_workers;
  const int n = std::min(h.n_workers, max_records);
  if (n <= 0) return LB_OK;
  if (h.off_workers + (int64_t)n * (int64_t)sizeof(lb_worker_record) > (int64_t)workspace_bytes)
    return LB_EWORKSPACE;
  if (hipMemcpy(host_records, static_cast<const char*>(workspace) + h.off_workers,
                n * sizeof(lb_worker_record), hipMemcpyDeviceToHost) != hipSuccess)
    return LB_EHIP;
  return LB_OK;
}

}  // extern "C"
