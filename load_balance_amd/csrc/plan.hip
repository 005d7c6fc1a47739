// Planning kernel: turns cu_seqlens (or per-token positions and document ids)
// into the longest-first queue of attention tiles.
//
// Only (query tile, key span) pairs holding visible pairs become work
// ("03 · 长文负载均衡", section 3.2: DCP generates computation blocks only for
// block pairs whose mask is not all zero), masks are described as rectangles
// of full or causal kind (section 4.4, MagiAttention's AttnSlice), each tile
// carries its exact number of visible (query, key) pairs (section 3.2, Libra
// TAP), and tiles are handed out largest first (section 2.1, VRSP's LPT
// placement; "数据并行负载均衡", section 4.4, LPT on estimated cost).  The
// estimate that orders them is a linear cost wb * blocks + wp * G * pairs: blocks
// is the number of 64-key blocks a tile sweeps (the attention kernel spends the
// same time on a block whatever share of it is visible, and a tile of few rows as
// long as a full one; section 3.3: a query block shorter than one tile is billed
// as a whole tile), pairs its visible (query, key) pairs, G the query heads one
// item serves.  The caller picks the weights (section 4.2 of the same page: a
// load model fitted to measured times); wb = 1, wp = 0 orders by blocks alone.
//
// One workgroup of 1024 threads does everything: the metadata is a few
// thousand integers, far below what a multi-workgroup launch would pay off.
//   1. fragments: one per segment (varlen) or per run of equal document id and
//      consecutive position (block path); spans = keys the fragment may see.
//   2. tiles: each fragment cut into `tile_rows` rows from its start; spans
//      clipped to what the tile's last row sees; pairs in closed form, blocks.
//   3. order: sort of (cost descending, natural index) keys in LDS; or, with
//      LB_ORDER_DOCUMENTS, of (the fragment's largest cost descending, natural index
//      descending) keys: the fragments longest first, each one's tiles from its last row
//      back, so that the items in flight at one time share their fragment's keys and values
//      in L2 (the order the tiles of one fragment run in decides only which reads hit).
// The plan lands in the caller's workspace; the attention kernel reads it.
#include "lbattn_internal.h"

namespace lb {
namespace {

constexpr int NT = kPlanThreads;
// Sort keys are 32 bits: (kCostMax - q) above kIndexBits bits of natural index, so that
// ascending keys are costs descending, ties in natural order.  q is the tile's cost divided
// by 2^shift and rounded up, shift the least that brings the plan's largest cost to
// kCostMax or below: with costs up to kCostMax the order is exact, and a tile with work
// never ties with an empty one (cost 0).
constexpr int kIndexBits = 17;
constexpr uint32_t kIndexMask = (1u << kIndexBits) - 1;
constexpr uint32_t kCostMax = (1u << (32 - kIndexBits)) - 1;
static_assert(kSortCap <= (int)kIndexMask + 1, "a tile index must fit the key");

constexpr int kPlanWaves = NT / 64;

constexpr int kRunRounds = 4;
// LB_ORDER_DOCUMENTS applies to plans of at most kGroupCap fragments and kSortCap / 2 tiles
// (the fragment maxima sit in their own LDS array; the bitonic sort's keys then stay clear of
// the tile table it reads fragments from); larger plans are ordered as LB_ORDER_LPT.
constexpr int kGroupCap = 4096;

struct PlanShared {
  uint32_t keys[kSortCap];
  uint32_t group_q[kGroupCap];  // LB_ORDER_DOCUMENTS: each fragment's largest scaled cost
  int32_t wave_sum[kPlanWaves];
  int32_t run_sum[kRunRounds][kPlanWaves];
  int32_t err;
  int32_t n_empty;
  int32_t has_lower;
  unsigned long long pairs;
  unsigned long long max_cost;
};

// Exclusive prefix sum of one value per thread across the workgroup (thread order),
// with the workgroup total in *total: a shuffle scan inside each wave, then the wave
// totals through LDS.  Two barriers.
__device__ __forceinline__ int block_excl_scan(int v, PlanShared& sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int x = __shfl_up(incl, off);
    if (lane >= off) incl += x;
  }
  if (lane == 63) sh.wave_sum[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    const int c = sh.wave_sum[i];
    base += i < w ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Sum over integers y < x of clamp(y, 0, L).
__device__ __forceinline__ int64_t clamp_prefix(int64_t x, int64_t L) {
  const int64_t m = x - 1;
  if (m <= 0) return 0;
  if (m <= L) return m * (m + 1) / 2;
  return L * (L + 1) / 2 + (m - L) * L;
}

// Visible pairs between n consecutive query positions p0.. and one span
// (keys at positions kp0 .. kp0 + L - 1, key visible iff its position <= the query's).
__device__ __forceinline__ int64_t span_pairs(int64_t p0, int64_t n, int64_t kp0, int64_t L) {
  const int64_t a = p0 - kp0 + 1;  // keys the first row sees, before clamping
  return clamp_prefix(a + n, L) - clamp_prefix(a, L);
}

// Marks run starts of (pos, doc) and writes their indices, in order, to starts[]; returns
// the count.  A super-round covers kRunRounds rounds of 4 * NT consecutive tokens; thread t
// takes tokens 4t .. 4t+3 of each round, one 16-byte load per array when aligned (lanes
// reading 16 bytes apart in separate 4-byte loads run several times slower through the
// vector cache).  The offsets come from lane ballots (bit counts below the lane) and one
// exchange of wave totals through LDS.
__device__ __forceinline__ int find_runs(const int32_t* pos, const int32_t* doc, int n, int cap, int32_t* starts,
                         int stride_ints, PlanShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool vec = ((reinterpret_cast<uintptr_t>(pos) | reinterpret_cast<uintptr_t>(doc)) & 15) == 0;
  int total = 0;
  for (int sbase = 0; sbase < n; sbase += kRunRounds * 4 * NT) {
    // tokens i0 - 1 .. i0 + 3 of each round: i0 .. i0 + 3 in one 16-byte load where the
    // pointers allow it and the round is whole; i0 - 1 from the next lower lane, lane 0
    // loading its own
    int pp[kRunRounds][5], dd[kRunRounds][5];
#pragma unroll
    for (int r = 0; r < kRunRounds; ++r) {
      const int i0 = sbase + r * 4 * NT + 4 * tid;
      if (vec && i0 + 3 < n) {
        const int4 p4 = *reinterpret_cast<const int4*>(pos + i0);
        const int4 d4 = *reinterpret_cast<const int4*>(doc + i0);
        pp[r][1] = p4.x; pp[r][2] = p4.y; pp[r][3] = p4.z; pp[r][4] = p4.w;
        dd[r][1] = d4.x; dd[r][2] = d4.y; dd[r][3] = d4.z; dd[r][4] = d4.w;
      } else {
#pragma unroll
        for (int e = 1; e < 5; ++e) {
          const int i = i0 + e - 1;
          pp[r][e] = i < n ? pos[i] : 0;
          dd[r][e] = i < n ? doc[i] : 0;
        }
      }
      const bool own = lane == 0 && i0 > 0 && i0 <= n;
      const int p_own = own ? pos[i0 - 1] : 0, d_own = own ? doc[i0 - 1] : 0;
      const int p_up = __shfl_up(pp[r][4], 1), d_up = __shfl_up(dd[r][4], 1);
      pp[r][0] = lane == 0 ? p_own : p_up;
      dd[r][0] = lane == 0 ? d_own : d_up;
    }
    uint32_t mask[kRunRounds];
    int below[kRunRounds];  // run starts in lower lanes of this wave, per round
#pragma unroll
    for (int r = 0; r < kRunRounds; ++r) {
      const int i0 = sbase + r * 4 * NT + 4 * tid;
      mask[r] = 0;
      below[r] = 0;
      int wave_total = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        const bool st = i < n && (i == 0 || dd[r][e + 1] != dd[r][e] || pp[r][e + 1] != pp[r][e] + 1);
        mask[r] |= (uint32_t)st << e;
        const uint64_t b = __ballot(st);
        below[r] += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        wave_total += __popcll(b);
      }
      if (lane == 0) sh.run_sum[r][w] = wave_total;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRunRounds; ++r) {
      const int i0 = sbase + r * 4 * NT + 4 * tid;
      int before = 0, all = 0;
#pragma unroll
      for (int x = 0; x < kPlanWaves; ++x) {
        const int c = sh.run_sum[r][x];
        before += x < w ? c : 0;
        all += c;
      }
      int idx = total + before + below[r];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (mask[r] >> e & 1) {
          if (idx < cap) starts[(int64_t)idx * stride_ints] = i0 + e;
          ++idx;
        }
      total += all;
    }
    __syncthreads();  // run_sum is rewritten by the next super-round or the next call
  }
  if (total > cap) {
    if (tid == 0) sh.err |= LB_DEVERR_CAPACITY;
    total = 0;
  }
  __syncthreads();
  return total;
}

// One bitonic phase k over sh.keys[0, n_pad): the stages whose partner distance j is 64
// or more go through LDS with a workgroup barrier each; the remaining stages (j < 64) pair
// lanes of one wave and run in registers with lane shuffles.
__device__ __forceinline__ void bitonic_phase(PlanShared& sh, int n_pad, int k, int j_first) {
  const int tid = threadIdx.x;
  int j = j_first;
  for (; j >= 64; j >>= 1) {
    for (int i = tid; i < n_pad; i += NT) {
      const int p = i ^ j;
      if (p > i) {
        const uint32_t x = sh.keys[i], y = sh.keys[p];
        const bool ascending = (i & k) == 0;
        if ((x > y) == ascending) {
          sh.keys[i] = y;
          sh.keys[p] = x;
        }
      }
    }
    __syncthreads();
  }
  if (j == 0) return;
  // every thread of the workgroup runs the shuffles (padding lanes carry the largest key)
  for (int base = 0; base < max(n_pad, NT); base += NT) {
    const int i = base + tid;
    uint32_t x = i < n_pad ? sh.keys[i] : ~uint32_t(0);
    for (int kk = (j_first >= 64 ? k : 2); kk <= k; kk <<= 1) {
      for (int jj = (kk == k ? j : kk >> 1); jj > 0; jj >>= 1) {
        const uint32_t y = __shfl_xor(x, jj);
        const bool ascending = (i & kk) == 0;
        const bool lower = (i & jj) == 0;
        x = (lower == ascending) ? (x < y ? x : y) : (x < y ? y : x);
      }
    }
    if (i < n_pad) sh.keys[i] = x;
  }
  __syncthreads();
}

// LDS staging inside the sort buffer, used before the sort needs it: key/value runs in the
// first quarter, a copy of the fragments (when they fit) in the second, each fragment's
// first tile index in the second half.
constexpr int kSortBytes = kSortCap * (int)sizeof(uint32_t);
constexpr int kLdsRuns = kSortBytes / 4 / (int)sizeof(KvRun);
constexpr int kLdsFrags = kSortBytes / 4 / (int)sizeof(Frag);
constexpr int kLdsFtile = kSortBytes / 2 / (int)sizeof(int32_t);
constexpr int kMaxTilesPerThread = kSortCap / NT;
constexpr int kRankSortMax = 2048;  // tiles ranked directly; larger plans take the bitonic sort
static_assert(kRankSortMax % NT == 0 && kRankSortMax <= kSortCap, "");

// Sum and maximum of a 64-bit value over the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += shfl_xor_u64(v, m);
  return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = max(v, shfl_xor_u64(v, m));
  return v;
}

__device__ __forceinline__ void plan_body(const PlanArgs& a, PlanShared& sh) {
  const int tid = threadIdx.x;
  char* ws = a.ws;
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  Frag* frags = reinterpret_cast<Frag*>(ws + a.L.off_frags);
  KvRun* kvr = reinterpret_cast<KvRun*>(ws + a.L.off_kvruns);
  lb_plan_tile* tiles = reinterpret_cast<lb_plan_tile*>(ws + a.L.off_tiles);
  lb_plan_tile* ntiles = reinterpret_cast<lb_plan_tile*>(ws + a.L.off_ntiles);
  int32_t* order = reinterpret_cast<int32_t*>(ws + a.L.off_order);
  KvRun* lds_runs = reinterpret_cast<KvRun*>(&sh.keys[0]);
  Frag* lds_frags = reinterpret_cast<Frag*>(&sh.keys[kSortCap / 4]);
  int32_t* lds_ftile = reinterpret_cast<int32_t*>(&sh.keys[kSortCap / 2]);

  if (tid == 0) {
    sh.err = 0;
    sh.pairs = 0;
    sh.max_cost = 0;
    sh.n_empty = 0;
    sh.has_lower = 0;
  }
  __syncthreads();

  // ---- 1. fragments and their spans -------------------------------------------------
  int n_frags = 0, n_kvruns = 0;
  if (a.mode == kPlanCausalDoc || a.mode == kPlanSharedQuestion) {
    const int32_t* cu = a.cu_seqlens;
    for (int i = tid; i <= a.n_seg; i += NT) {
      const int c = cu[i];
      bool bad = (i == 0 && c != 0) || (i > 0 && c < cu[i - 1]) || (i == a.n_seg && c != a.total_tokens);
      if (bad) atomicOr(&sh.err, LB_DEVERR_CU_SEQLENS);
    }
    __syncthreads();
    n_frags = a.n_seg;
    if (sh.err == 0) {
      const int Q = cu[1] - cu[0];
      for (int s = tid; s < n_frags; s += NT) {
        Frag f{};
#pragma unroll
        for (int o = 0; o < LB_MAX_SPANS; ++o) f.k_lo[o] = LB_NO_LOWER_BOUND;
        f.q_start = cu[s];
        f.q_len = cu[s + 1] - cu[s];
        if (a.mode == kPlanCausalDoc) {
          f.q_pos0 = 0;
          f.n_spans = 1;
          f.k_start[0] = f.q_start; f.k_len[0] = f.q_len; f.k_pos0[0] = 0;
        } else if (a.transposed && s == 0) {
          // the question's keys, seen by the question's later rows and by every answer row:
          // one span over the rest of the pack, positions = row index (an answer row's
          // index is at least Q, past every question key)
          f.q_pos0 = 0;
          f.n_spans = 1;
          f.k_start[0] = cu[0]; f.k_len[0] = a.total_tokens - cu[0]; f.k_pos0[0] = 0;
        } else if (a.transposed) {  // an answer's keys, seen by its own rows only
          f.q_pos0 = Q;
          f.n_spans = 1;
          f.k_start[0] = f.q_start; f.k_len[0] = f.q_len; f.k_pos0[0] = Q;
        } else if (s == 0) {  // the question: causal on itself
          f.q_pos0 = 0;
          f.n_spans = 1;
          f.k_start[0] = cu[0]; f.k_len[0] = Q; f.k_pos0[0] = 0;
        } else {  // an answer: positions continue after the question
          f.q_pos0 = Q;
          const int own = Q > 0 ? 1 : 0;  // slot of the answer's own span, after the question's
          if (Q > 0) { f.k_start[0] = cu[0]; f.k_len[0] = Q; f.k_pos0[0] = 0; }
          f.k_start[own] = f.q_start; f.k_len[own] = f.q_len; f.k_pos0[own] = Q;
          f.n_spans = own + 1;
        }
        frags[s] = f;
        if (n_frags <= kLdsFrags) lds_frags[s] = f;
      }
    }
  } else if (a.mode == kPlanSlices) {
    // one fragment per query range: slice s opens one when its range differs from s - 1's.
    // Rows no slice covers (before a range, between two, after the last) make a fragment
    // with no key span, so that their lse is -inf like any row that sees no key.
    const lb_mask_slice* sl = a.slices;
    int running = 0;
    for (int base = 0; base < a.n_slices; base += NT) {
      const int s = base + tid;
      bool opens = false, gap = false;
      int gap_start = 0;
      if (s < a.n_slices) {
        const lb_mask_slice x = sl[s];
        bool bad = x.q_len < 1 || x.k_len < 1 || x.q_start < 0 || x.k_start < 0 || x.q_start > a.n_q - x.q_len ||
                   x.k_start > a.n_kv - x.k_len || x.kind < LB_SLICE_FULL || x.kind > LB_SLICE_BI_CAUSAL;
        opens = s == 0 || sl[s - 1].q_start != x.q_start || sl[s - 1].q_len != x.q_len;
        if (s > 0 && opens && sl[s - 1].q_start + sl[s - 1].q_len > x.q_start) bad = true;  // unsorted or overlapping
        if (!opens && sl[s - 1].k_start + sl[s - 1].k_len > x.k_start) bad = true;  // key ranges must ascend, disjoint
        if (bad) atomicOr(&sh.err, LB_DEVERR_SLICES);
        gap_start = s == 0 ? 0 : sl[s - 1].q_start + sl[s - 1].q_len;
        gap = opens && !bad && x.q_start > gap_start;
      }
      int total;
      const int off = block_excl_scan((opens ? 1 : 0) + (gap ? 1 : 0), sh, &total);
      if (gap && running + off < a.L.cap_frags) {
        Frag g{};
#pragma unroll
        for (int o = 0; o < LB_MAX_SPANS; ++o) g.k_lo[o] = LB_NO_LOWER_BOUND;
        g.q_start = gap_start;
        g.q_len = sl[s].q_start - gap_start;
        frags[running + off] = g;
        if (running + off < kLdsFrags) lds_frags[running + off] = g;
      }
      if (opens && running + off + (gap ? 1 : 0) < a.L.cap_frags) {
        // the fragment's spans: this slice and the following ones on the same range
        const lb_mask_slice x = sl[s];
        Frag f{};
#pragma unroll
        for (int o = 0; o < LB_MAX_SPANS; ++o) f.k_lo[o] = LB_NO_LOWER_BOUND;
        f.q_start = x.q_start;
        f.q_len = x.q_len;
        f.q_pos0 = 0;
        int ns = 0;
        for (int j = s; j < a.n_slices; ++j) {
          const lb_mask_slice y = sl[j];
          if (y.q_start != x.q_start || y.q_len != x.q_len) break;
          if (ns == LB_MAX_SPANS) { atomicOr(&sh.err, LB_DEVERR_SPANS); break; }
          // upper bound (bottom-right diagonal) for CAUSAL and BI-CAUSAL, lower bound (top-left
          // diagonal: key j of the slice from row j on) for INV-CAUSAL and BI-CAUSAL
          const bool upper = y.kind == LB_SLICE_CAUSAL || y.kind == LB_SLICE_BI_CAUSAL;
          const bool lower = y.kind == LB_SLICE_INV_CAUSAL || y.kind == LB_SLICE_BI_CAUSAL;
          const int pos0 = upper ? y.q_len - y.k_len : kFullSpanPos;
          const int lo = lower ? 0 : LB_NO_LOWER_BOUND;
          if (lower) sh.has_lower = 1;
#pragma unroll
          for (int o = 0; o < LB_MAX_SPANS; ++o)
            if (o == ns) { f.k_start[o] = y.k_start; f.k_len[o] = y.k_len; f.k_pos0[o] = pos0; f.k_lo[o] = lo; }
          ++ns;
        }
        f.n_spans = ns;
        const int at = running + off + (gap ? 1 : 0);
        frags[at] = f;
        if (at < kLdsFrags) lds_frags[at] = f;
      }
      running += total;
    }
    // the rows after the last range
    const int end = a.n_slices > 0 ? sl[a.n_slices - 1].q_start + sl[a.n_slices - 1].q_len : 0;
    if (end < a.n_q) {
      if (tid == 0 && running < a.L.cap_frags) {
        Frag g{};
#pragma unroll
        for (int o = 0; o < LB_MAX_SPANS; ++o) g.k_lo[o] = LB_NO_LOWER_BOUND;
        g.q_start = end;
        g.q_len = a.n_q - end;
        frags[running] = g;
        if (running < kLdsFrags) lds_frags[running] = g;
      }
      ++running;
    }
    n_frags = running;
    if (n_frags > a.L.cap_frags && tid == 0) sh.err |= LB_DEVERR_CAPACITY;
  } else {  // block path: runs of equal doc id and consecutive position
    // Transposed, the tile side is the keys and the spans are query runs: the same search
    // with the two sides swapped and the visibility test turned around.
    const int32_t* t_pos = a.transposed ? a.kv_pos : a.q_pos;
    const int32_t* t_doc = a.transposed ? a.kv_doc : a.q_doc;
    const int32_t* s_pos = a.transposed ? a.q_pos : a.kv_pos;
    const int32_t* s_doc = a.transposed ? a.q_doc : a.kv_doc;
    const int n_t = a.transposed ? a.n_kv : a.n_q, n_s = a.transposed ? a.n_q : a.n_kv;
    n_frags = find_runs(t_pos, t_doc, n_t, a.L.cap_frags, &frags[0].q_start, sizeof(Frag) / 4, sh);
    n_kvruns = find_runs(s_pos, s_doc, n_s, min(a.L.cap_frags, kLdsRuns), &kvr[0].start, sizeof(KvRun) / 4, sh);
    if (sh.err == 0) {
      // complete the key/value runs, in LDS for the span search below
      for (int r = tid; r < n_kvruns; r += NT) {
        const int s = kvr[r].start;
        const int e = r + 1 < n_kvruns ? kvr[r + 1].start : n_s;
        lds_runs[r] = KvRun{s, e - s, s_pos[s], s_doc[s]};
      }
      __syncthreads();
      for (int r = tid; r < n_frags; r += NT) {
        const int s = frags[r].q_start;
        const int e = r + 1 < n_frags ? frags[r + 1].q_start : n_t;
        Frag f{};
#pragma unroll
        for (int o = 0; o < LB_MAX_SPANS; ++o) f.k_lo[o] = LB_NO_LOWER_BOUND;
        f.q_start = s;
        f.q_len = e - s;
        f.q_pos0 = t_pos[s];
        const int doc = t_doc[s];
        const int last_pos = f.q_pos0 + f.q_len - 1;
        int ns = 0;
        int full_end = -1;  // end of the last span in the buffer when that span is FULL, else -1
        for (int j = 0; j < n_kvruns; ++j) {
          const KvRun kr = lds_runs[j];
          // The shared document's keys are seen in full by every other document's rows
          // (the shared-question mask): as a FULL span (keys far below every row) or,
          // transposed, a query run far above every key.
          const int key_doc = a.transposed ? doc : kr.doc, row_doc = a.transposed ? kr.doc : doc;
          const bool shared = a.shared_doc >= 0 && key_doc == a.shared_doc && row_doc != a.shared_doc;
          // other document, or no pair: keys wholly after the query run (forward), or
          // queries wholly before the key run (transposed)
          if (!shared &&
              (kr.doc != doc || (a.transposed ? kr.pos0 + kr.len - 1 < f.q_pos0 : kr.pos0 > last_pos)))
            continue;
          if (shared && full_end == kr.start) {
            // a FULL run right after a FULL span in the buffer extends it: positions play no
            // part in a FULL span, so one span covers both (a document cut into several
            // chunks per rank stays one span)
#pragma unroll
            for (int o = 0; o < LB_MAX_SPANS; ++o)
              if (o == ns - 1) f.k_len[o] += kr.len;
            full_end += kr.len;
            continue;
          }
          if (ns == LB_MAX_SPANS) { atomicOr(&sh.err, LB_DEVERR_SPANS); break; }
          const int pos0 = shared ? (a.transposed ? kFullRowsPos : kFullSpanPos) : kr.pos0;
#pragma unroll
          for (int o = 0; o < LB_MAX_SPANS; ++o)  // slot ns, selected so the fields stay in registers
            if (o == ns) { f.k_start[o] = kr.start; f.k_len[o] = kr.len; f.k_pos0[o] = pos0; }
          ++ns;
          full_end = shared ? kr.start + kr.len : -1;
        }
        f.n_spans = ns;
        frags[r] = f;
        if (n_frags <= kLdsFrags) lds_frags[r] = f;
      }
    }
  }
  if (n_frags + 1 > kLdsFtile && tid == 0) sh.err |= LB_DEVERR_CAPACITY;
  __syncthreads();

  // ---- 2. tiles in natural order ---------------------------------------------------
  const int bm = a.tile_rows;
  int n_tiles = 0;
  if (sh.err == 0) {
    int running = 0;
    for (int base = 0; base < n_frags; base += NT) {
      const int f = base + tid;
      const int qlen = f < n_frags ? (n_frags <= kLdsFrags ? lds_frags[f].q_len : frags[f].q_len) : 0;
      const int cnt = (qlen + bm - 1) / bm;
      int total;
      const int off = block_excl_scan(cnt, sh, &total);
      if (f < n_frags) lds_ftile[f] = running + off;
      running += total;
    }
    n_tiles = running;
    if (tid == 0) lds_ftile[n_frags] = n_tiles;
    if (n_tiles > a.L.cap_tiles) {
      if (tid == 0) sh.err |= LB_DEVERR_CAPACITY;
    }
  }
  // LB_ORDER_DOCUMENTS: each fragment's largest ordering cost, kept while the tiles are cut in
  // the LDS that held phase 1's key/value runs (the first quarter of the sort buffer)
  const bool by_doc = a.order == LB_ORDER_DOCUMENTS && n_frags <= kGroupCap && n_tiles <= kSortCap / 2;
  unsigned long long* frag_cost = reinterpret_cast<unsigned long long*>(&sh.keys[0]);
  static_assert(kGroupCap * sizeof(unsigned long long) <= kSortCap / 4 * sizeof(uint32_t), "");
  if (by_doc)
    for (int i = tid; i < n_frags; i += NT) frag_cost[i] = 0;
  __syncthreads();
  // ordering cost of a tile; the weights are below 2^24 and 2^16, so with blocks below 2^25,
  // G <= 8 and pairs below 2^39 (256 rows by 2^31 keys) a cost stays below 2^59
  const unsigned long long wp = (unsigned long long)a.pair_weight * (unsigned)(a.heads / a.kv_heads);
  auto cost_of = [&](int blocks, int64_t pairs) -> unsigned long long {
    return (unsigned long long)a.block_weight * (unsigned)blocks + wp * (unsigned long long)pairs;
  };
  // the order terms of this thread's first tiles, kept for the rank sort's keys
  constexpr int kMine = kRankSortMax / NT;
  int mine_blocks[kMine] = {};
  int64_t mine_pairs[kMine] = {};
  if (sh.err == 0) {
    unsigned long long my_pairs = 0, my_max = 0;
#pragma unroll
    for (int k = 0; k < kMaxTilesPerThread; ++k) {
      const int t = tid + k * NT;
      if (t >= n_tiles) break;
      int lo = 0, hi = n_frags - 1;  // last fragment whose first tile <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (lds_ftile[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const Frag f = n_frags <= kLdsFrags ? lds_frags[lo] : frags[lo];
      const int kt = t - lds_ftile[lo];
      lb_plan_tile T{};
#pragma unroll
      for (int o = 0; o < LB_MAX_SPANS; ++o) T.k_lo[o] = LB_NO_LOWER_BOUND;
      T.q_start = f.q_start + kt * bm;
      T.q_len = min(bm, f.q_len - kt * bm);
      T.q_pos0 = f.q_pos0 + kt * bm;
      const int last = T.q_pos0 + T.q_len - 1;
      int ns = 0, blocks = 0;
      int64_t cost = 0;
#pragma unroll
      for (int sp = 0; sp < LB_MAX_SPANS; ++sp) {
        if (sp >= f.n_spans) break;
        // forward: keys below the lower bound of the tile's first row dropped, then keys up
        // to the tile's last row kept; transposed: query rows from the tile's first key on
        // (c rows of the span see none of the tile's keys)
        const int lo0 = f.k_lo[sp];
        const int c = a.transposed ? max(0, T.q_pos0 - f.k_pos0[sp])
                                   : (lo0 == LB_NO_LOWER_BOUND ? 0 : min(f.k_len[sp], max(0, T.q_pos0 - lo0)));
        const int keep = a.transposed ? f.k_len[sp] - c : min(f.k_len[sp] - c, last - (f.k_pos0[sp] + c) + 1);
        if (keep <= 0) continue;
        const int s_start = f.k_start[sp] + c, s_pos0 = f.k_pos0[sp] + c;
        const int s_lo = lo0 == LB_NO_LOWER_BOUND ? lo0 : lo0 + c;
#pragma unroll
        for (int o = 0; o <= sp; ++o)  // slot ns <= sp, selected so T stays in registers
          if (o == ns) { T.k_start[o] = s_start; T.k_len[o] = keep; T.k_pos0[o] = s_pos0; T.k_lo[o] = s_lo; }
        // visible pairs: a key at position x and a query at position y with x <= y; the
        // count is the same whichever side is the tile.  A lower bound removes, for each row
        // at position y, the keys j with s_lo + j < y: sum over rows of clamp(y - s_lo, 0, keep).
        int64_t pairs = a.transposed ? span_pairs(s_pos0, keep, T.q_pos0, T.q_len)
                                     : span_pairs(T.q_pos0, T.q_len, s_pos0, keep);
        // (when s_pos0 > s_lo + 1 the band is empty for every row)
        if (s_lo != LB_NO_LOWER_BOUND)
          pairs = s_pos0 > s_lo + 1 ? 0
                                    : pairs - (clamp_prefix((int64_t)T.q_pos0 - s_lo + T.q_len, keep) -
                                               clamp_prefix((int64_t)T.q_pos0 - s_lo, keep));
        cost += pairs;
        blocks += (keep + kBlockN - 1) / kBlockN;
        ++ns;
      }
      T.n_spans = ns;
      T.cost = cost;
      T.blocks = blocks;
      ntiles[t] = T;
      if (ns == 0) atomicAdd(&sh.n_empty, 1);  // no blocks: sorts to the end of the order
      my_pairs += (unsigned long long)cost;
      my_max = max(my_max, cost_of(blocks, cost));
      if (by_doc && blocks > 0) atomicMax(&frag_cost[lo], cost_of(blocks, cost));
      if (k < kMine) {
        mine_blocks[k] = blocks;
        mine_pairs[k] = cost;
      }
    }
    // one LDS atomic per wave: 1024 lanes updating one LDS word one after another would
    // take longer than everything else in this phase
    my_pairs = wave_sum_u64(my_pairs);
    my_max = wave_max_u64(my_max);
    if ((tid & 63) == 0) {
      atomicAdd(&sh.pairs, my_pairs);
      atomicMax(&sh.max_cost, my_max);
    }
  }
  __syncthreads();  // the staging areas are dead from here on; the sort buffer takes over

  // sort keys: (kCostMax - q) << kIndexBits | natural index, q the rounded-up scaled cost;
  // ascending keys are costs descending with ties in natural order, and every key is unique.
  // A tile's cost is recomputed from its blocks and pairs: kept in registers for the rank
  // sort's (at most two per thread), read back from the tile's record for the bitonic sort
  // (a cost for each of up to 32 tiles per thread would not stay in registers).
  int shift = 0;
  while (((sh.max_cost + (1ull << shift) - 1) >> shift) > kCostMax) ++shift;
  const unsigned long long round = (1ull << shift) - 1;
  auto scaled = [&](int blocks, int64_t pairs) -> uint32_t {
    return (uint32_t)((cost_of(blocks, pairs) + round) >> shift);
  };
  // the fragment of tile t (tiles are numbered fragment after fragment)
  auto frag_of = [&](int t) -> int {
    int lo = 0, hi = n_frags - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (lds_ftile[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  // the fragments' largest costs scaled as the tiles' are (scaling is monotone: the scaled
  // maximum is the maximum of the scaled costs); 0 for a fragment without a tile with blocks
  if (by_doc && sh.err == 0)
    for (int i = tid; i < n_frags; i += NT) {
      const unsigned long long c = frag_cost[i];
      sh.group_q[i] = c > 0 ? (uint32_t)((c + round) >> shift) : 0u;
    }
  __syncthreads();
  // LB_ORDER_LPT: (kCostMax - q) << kIndexBits | t, q the tile's scaled cost: costs descending,
  // ties in natural order.  LB_ORDER_DOCUMENTS: q the largest of the tile's fragment (0 for a
  // tile without spans, so that those still come last) and the index reversed: fragments
  // longest first, ties and the tiles within a fragment in descending natural order.
  auto key_of = [&](int t, int blocks, int64_t pairs) -> uint32_t {
    if (by_doc) {
      const uint32_t q = blocks > 0 ? sh.group_q[frag_of(t)] : 0u;
      return ((kCostMax - q) << kIndexBits) | (kIndexMask - (uint32_t)t);
    }
    return ((kCostMax - scaled(blocks, pairs)) << kIndexBits) | (uint32_t)t;
  };

  // ---- 3. longest-first order of the unique keys; tiles copied to their queue positions --
  // The documents order of a plan whose tiles all have spans needs no sort of the tiles: the
  // fragments are ranked by their keys ((kCostMax - group q) << kIndexBits | reversed
  // fragment index, the order the tiles' keys give them), a prefix sum over the fragments in
  // that order gives each one's first queue position, and a tile's place is its fragment's
  // first position plus the tiles of the fragment after it.  The fragment keys, ranks and
  // positions use the first quarter of the sort buffer (free since the fragment maxima were
  // scaled); the fragments' first tiles stay in lds_ftile.
  const bool direct = by_doc && sh.n_empty == 0 && n_frags <= kRankSortMax;
  if (sh.err == 0 && n_tiles > 0 && direct) {
    uint32_t* fkey = &sh.keys[0];                // fragment keys, then first queue positions
    int32_t* fpos = reinterpret_cast<int32_t*>(&sh.keys[kRankSortMax]);  // tiles per rank, scanned
    constexpr int kFrag = kRankSortMax / NT;
    const int nf4 = (n_frags + 3) & ~3;
    for (int f = tid; f < nf4; f += NT)
      fkey[f] = f < n_frags ? ((kCostMax - sh.group_q[f]) << kIndexBits) | (kIndexMask - (uint32_t)f) : ~0u;
    __syncthreads();
    int frank[kFrag];
    const uint4* fkey4 = reinterpret_cast<const uint4*>(fkey);
#pragma unroll
    for (int k = 0; k < kFrag; ++k) {
      const int f = tid + k * NT;
      frank[k] = 0;
      if (f < n_frags) {
        const uint32_t mine = fkey[f];
        for (int i = 0; i < nf4 / 4; ++i) {
          const uint4 v = fkey4[i];
          frank[k] += (v.x < mine ? 1 : 0) + (v.y < mine ? 1 : 0) + (v.z < mine ? 1 : 0) + (v.w < mine ? 1 : 0);
        }
        fpos[frank[k]] = lds_ftile[f + 1] - lds_ftile[f];
      }
    }
    __syncthreads();
    // exclusive prefix sum of the tile counts in fragment order
    int running = 0;
    for (int base = 0; base < n_frags; base += NT) {
      const int r = base + tid;
      const int cnt = r < n_frags ? fpos[r] : 0;
      int total;
      const int off = block_excl_scan(cnt, sh, &total);
      if (r < n_frags) fpos[r] = running + off;
      running += total;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kFrag; ++k) {
      const int f = tid + k * NT;
      if (f < n_frags) fkey[f] = (uint32_t)fpos[frank[k]];
    }
    __syncthreads();
    for (int t = tid; t < n_tiles; t += NT) {
      const int f = frag_of(t);
      const int q = (int)fkey[f] + (lds_ftile[f + 1] - 1 - t);
      tiles[q] = ntiles[t];
      order[q] = q;
    }
  } else if (sh.err == 0 && n_tiles > 0 && n_tiles <= kRankSortMax) {
    // Up to kRankSortMax tiles, every thread ranks its own keys against all of them (the keys
    // are unique, so the ranks are a permutation): n^2 / threads broadcast reads from LDS,
    // four keys per read, and one barrier, against the bitonic network's 55 barrier-separated
    // passes at 1024 keys.
    uint32_t my_key[kMine];
#pragma unroll
    for (int k = 0; k < kMine; ++k) {
      const int t = tid + k * NT;
      my_key[k] = ~0u;
      if (t < n_tiles) {
        my_key[k] = key_of(t, mine_blocks[k], mine_pairs[k]);
        sh.keys[t] = my_key[k];
      }
    }
    const int n4 = (n_tiles + 3) & ~3;
    if (tid < n4 - n_tiles) sh.keys[n_tiles + tid] = ~0u;  // above every key: never counted
    __syncthreads();
    int rank[kMine] = {};
    const uint4* keys4 = reinterpret_cast<const uint4*>(sh.keys);
#pragma unroll
    for (int k = 0; k < kMine; ++k) {
      if (k * NT >= n_tiles) break;  // no thread holds a k-th tile
#pragma unroll 4
      for (int i = 0; i < n4 / 4; ++i) {
        const uint4 v = keys4[i];
        rank[k] += (v.x < my_key[k] ? 1 : 0) + (v.y < my_key[k] ? 1 : 0) + (v.z < my_key[k] ? 1 : 0) +
                   (v.w < my_key[k] ? 1 : 0);
      }
    }
#pragma unroll
    for (int k = 0; k < kMine; ++k) {
      if (tid + k * NT >= n_tiles) break;
      tiles[rank[k]] = ntiles[tid + k * NT];  // this thread's own tile, written by it in phase 2
      order[rank[k]] = rank[k];
    }
  } else if (sh.err == 0 && n_tiles > 0) {
    // bitonic sort of the keys in LDS
    int n_pad = 1;
    while (n_pad < n_tiles) n_pad <<= 1;
    for (int i = tid; i < n_pad; i += NT)
      sh.keys[i] = i < n_tiles ? key_of(i, ntiles[i].blocks, ntiles[i].cost) : ~0u;
    __syncthreads();
    // phases k = 2 .. min(n_pad, 64) pair lanes of one wave only: all in registers at once
    bitonic_phase(sh, n_pad, min(n_pad, 64), min(n_pad, 64) >> 1);
    for (int k = 128; k <= n_pad; k <<= 1) bitonic_phase(sh, n_pad, k, k >> 1);
    for (int i = tid; i < n_tiles; i += NT) {
      const uint32_t idx = sh.keys[i] & kIndexMask;
      tiles[i] = ntiles[by_doc ? kIndexMask - idx : idx];
      order[i] = i;
    }
  }
  __syncthreads();

  if (tid == 0) {
    const bool ok = sh.err == 0;
    // one queue per XCD when the kv heads split evenly over them: queue x serves kv heads
    // x, x + 8, ... so that an XCD's L2 holds the keys and values of its own heads
    const int nq = a.kv_heads % kXcds == 0 ? kXcds : 1;
    hdr->err = sh.err;
    hdr->n_frags = ok ? n_frags : 0;
    hdr->n_tiles = ok ? n_tiles : 0;
    const int n_work = ok ? n_tiles - sh.n_empty : 0;
    hdr->n_items = n_work * a.kv_heads;
    hdr->n_empty = ok ? sh.n_empty : 0;
    hdr->n_queues = nq;
    hdr->per_queue = n_work * a.kv_heads / nq;
    for (int q = 0; q < kXcds; ++q) hdr->queue_head[q] = 0;
    hdr->n_kvruns = n_kvruns;
    hdr->tile_rows = bm;
    hdr->n_workers = 0;
    hdr->off_frags = a.L.off_frags;
    hdr->off_kvruns = a.L.off_kvruns;
    hdr->off_tiles = a.L.off_tiles;
    hdr->off_order = a.L.off_order;
    hdr->off_ntiles = a.L.off_ntiles;
    hdr->off_workers = a.L.off_workers;
    hdr->cap_frags = a.L.cap_frags;
    hdr->cap_tiles = a.L.cap_tiles;
    hdr->total_pairs = ok ? (int64_t)sh.pairs : 0;
    hdr->transposed = a.transposed;
    hdr->has_lower = ok ? sh.has_lower : 0;
    const bool pair_sides = a.mode == kPlanBlock || a.mode == kPlanSlices;
    hdr->plan_n_q = pair_sides ? a.n_q : a.total_tokens;
    hdr->plan_n_kv = pair_sides ? a.n_kv : a.total_tokens;
    hdr->plan_kv_heads = a.kv_heads;
    hdr->plan_heads = a.heads;
    hdr->ring_fused = 0;
    hdr->done = 0;
    hdr->magic = kPlanMagic;
  }
}

__global__ __launch_bounds__(NT) void plan_kernel(PlanArgs a) {
  __shared__ PlanShared sh;
  plan_body(a, sh);
}

// Independent plans of several block steps: workgroup s plans step s into its own
// workspace.  The steps differ only in their key/value metadata, which a ring step
// knows before the chunk's data arrive.
__global__ __launch_bounds__(NT) void plan_steps_kernel(PlanBatch b) {
  __shared__ PlanShared sh;
  const PlanArgs a = b.step[blockIdx.x];
  plan_body(a, sh);
}

// ---- the ring: several steps' plans merged into one longest-first queue ----------------
// The work tiles of all steps, ordered by key blocks (descending), then step, then their
// place in the step's own order: the same longest-first rule over the union, so that one
// persistent launch can run every step with no tail per step.  Each step's plan is already
// sorted, so a tile's place in the union is its place in its own step plus, for every other
// step, the number of that step's tiles that go before it (a binary search in LDS).  The
// tiles are copied in that order, each with its step in `reserved`, and the steps' empty
// tiles follow.
__device__ __forceinline__ int count_before(const int32_t* blk, int n, int b, bool ties_before) {
  // blk[0..n) is descending: entries > b (and == b when ties_before) come first
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int x = blk[mid];
    if (x > b || (ties_before && x == b)) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ void copy_tile(lb_plan_tile* dst, const lb_plan_tile* src, int step) {
  static_assert(sizeof(lb_plan_tile) % 16 == 0, "");
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(lb_plan_tile) / 16); ++i) d4[i] = s4[i];
  dst->reserved = step;
}

__global__ __launch_bounds__(NT) void ring_merge_kernel(RingMergeArgs m) {
  __shared__ int32_t blk[kRingSortCap];  // key blocks of the work tiles, step after step
  __shared__ int32_t src[kRingSortCap];  // their index in the step's tile array
  __shared__ int32_t base[kMaxPlanSteps + 1], ebase[kMaxPlanSteps + 1];
  __shared__ const lb_plan_tile* tiles_of[kMaxPlanSteps];
  __shared__ const int32_t* order_of[kMaxPlanSteps];
  __shared__ int32_t ntiles_of[kMaxPlanSteps];
  __shared__ int32_t err;       // written by thread 0 before the first barrier only
  __shared__ int32_t err_tiles;  // bad order entries found by the copy loops
  __shared__ int64_t pairs;
  const int tid = threadIdx.x;
  const int n_steps = m.n_steps;
  WsHeader* rh = reinterpret_cast<WsHeader*>(m.ring);
  lb_plan_tile* out = reinterpret_cast<lb_plan_tile*>(m.ring + kRingTilesOffset);

  // one thread per step reads that step's header, so the steps' header loads overlap
  __shared__ int32_t work_of[kMaxPlanSteps], empty_of[kMaxPlanSteps], err_of[kMaxPlanSteps];
  __shared__ int64_t pairs_of[kMaxPlanSteps];
  if (tid < n_steps) {
    const int s = tid;
    const WsHeader* h = reinterpret_cast<const WsHeader*>(m.step_ws[s]);
    const int64_t nt = h->n_tiles, ne = h->n_empty;
    // a step's plan must be a block plan of the ring's kind made for these shapes, and lie inside
    // its workspace; its own error bits pass on
    const bool bad = h->magic != kPlanMagic || h->transposed != m.transposed || h->has_lower != 0 ||
                     h->plan_n_q != m.n_q || h->plan_n_kv != m.n_kv[s] || h->plan_heads != m.heads ||
                     h->plan_kv_heads != m.kv_heads || nt < 0 || ne < 0 || ne > nt ||
                     h->off_tiles < kWorkersOffset || h->off_order < kWorkersOffset ||
                     h->off_tiles + nt * (int64_t)sizeof(lb_plan_tile) > m.step_ws_bytes[s] ||
                     h->off_order + nt * 4 > m.step_ws_bytes[s];
    err_of[s] = bad ? LB_DEVERR_PLAN : h->err;
    work_of[s] = bad ? 0 : (int)(nt - ne);
    empty_of[s] = bad ? 0 : (int)ne;
    tiles_of[s] = reinterpret_cast<const lb_plan_tile*>(m.step_ws[s] + (bad ? 0 : h->off_tiles));
    order_of[s] = reinterpret_cast<const int32_t*>(m.step_ws[s] + (bad ? 0 : h->off_order));
    ntiles_of[s] = bad ? 0 : (int)nt;
    pairs_of[s] = bad ? 0 : h->total_pairs;
  }
  __syncthreads();
  if (tid == 0) {
    int e = 0;
    int64_t p = 0;
    base[0] = ebase[0] = 0;
    for (int s = 0; s < n_steps; ++s) {
      e |= err_of[s];
      base[s + 1] = base[s] + work_of[s];
      ebase[s + 1] = ebase[s] + empty_of[s];
      p += pairs_of[s];
    }
    if (base[n_steps] > kRingSortCap || (int64_t)base[n_steps] + ebase[n_steps] > m.ring_cap) e |= LB_DEVERR_CAPACITY;
    err = e;
    err_tiles = 0;
    pairs = p;
  }
  __syncthreads();
  const int M = base[n_steps], E = ebase[n_steps];
  const bool steps_ok = err == 0;  // the same for every thread: err is not written again
  if (steps_ok) {
    for (int j = tid; j < M; j += NT) {
      int s = 0;
      while (j >= base[s + 1]) ++s;
      int t = order_of[s][j - base[s]];
      if (t < 0 || t >= ntiles_of[s]) {  // an order entry outside the step's tiles: refuse the ring
        atomicOr(&err_tiles, LB_DEVERR_PLAN);
        t = 0;
      }
      src[j] = t;
      blk[j] = tiles_of[s][t].blocks;
    }
  }
  __syncthreads();
  // (no barrier below depends on err_tiles: a thread that sees it set late only copies
  // tiles of a ring that is refused anyway)
  if (steps_ok && err_tiles == 0) {
    for (int j = tid; j < M; j += NT) {
      int s = 0;
      while (j >= base[s + 1]) ++s;
      const int b = blk[j];
      int rank = j - base[s];
      for (int o = 0; o < n_steps; ++o)
        if (o != s) rank += count_before(blk + base[o], base[o + 1] - base[o], b, o < s);
      copy_tile(&out[rank], &tiles_of[s][src[j]], s);
    }
    for (int j = tid; j < E; j += NT) {
      int s = 0;
      while (j >= ebase[s + 1]) ++s;
      const int t = order_of[s][ntiles_of[s] - (ebase[s + 1] - ebase[s]) + (j - ebase[s])];
      if (t >= 0 && t < ntiles_of[s]) copy_tile(&out[M + j], &tiles_of[s][t], s);
      else atomicOr(&err_tiles, LB_DEVERR_PLAN);
    }
  }
  __syncthreads();
  if (tid == 0) {
    err |= err_tiles;
    const bool ok = err == 0;
    const int nq = m.kv_heads % kXcds == 0 ? kXcds : 1;
    rh->err = err;
    rh->n_frags = 0;
    rh->n_kvruns = 0;
    rh->n_tiles = ok ? M + E : 0;
    rh->n_empty = ok ? E : 0;
    rh->n_items = ok ? M * m.kv_heads : 0;
    rh->n_queues = nq;
    rh->per_queue = (ok ? M * m.kv_heads : 0) / nq;
    for (int q = 0; q < kXcds; ++q) rh->queue_head[q] = 0;
    rh->tile_rows = 0;
    rh->n_workers = 0;
    rh->off_frags = rh->off_kvruns = 0;
    rh->off_tiles = rh->off_order = kRingTilesOffset;  // queue order is storage order
    rh->off_workers = kWorkersOffset;
    rh->cap_frags = 0;
    rh->cap_tiles = m.ring_cap;
    rh->total_pairs = ok ? pairs : 0;
    rh->transposed = m.transposed;
    rh->has_lower = 0;
    rh->plan_n_q = m.n_q;
    rh->plan_n_kv = 0;
    rh->plan_heads = m.heads;
    rh->plan_kv_heads = m.kv_heads;
    rh->ring_steps = n_steps;
    for (int s = 0; s < kMaxPlanSteps; ++s) rh->ring_n_kv[s] = s < n_steps ? m.n_kv[s] : 0;
    rh->ring_fused = 0;
    rh->off_ntiles = 0;
    rh->done = 0;
    rh->magic = kRingMagic;
  }
}

// ---- a fused ring: one tile per query tile, with the key spans of every step ---------------
// The steps' plans cut the query shard into the same tiles (the tiling depends on the query
// side only), so query tile x of the fused ring gathers tile x of every step, read from the
// natural-order copy each plan keeps: its spans in step order, each span's step in 4 bits of
// `reserved` (span s at bits 4s..4s+3), its pairs and key blocks summed.  One attention item
// then runs the rows against the keys of every step with one online softmax and writes what
// the steps' partials would have merged to (the rescale-and-sum of the partials, taken inside
// the tile).  Queue order: key blocks descending (above 32767 as 32767), ties in natural order,
// the tiles without spans last in natural order -- the unique 32-bit keys (32767 - blocks) << 17
// | x, ranked against each other in LDS.  A tile with more than LB_MAX_SPANS spans refuses the
// ring (LB_DEVERR_SPANS), as do more than kFusedTileCap tiles (LB_DEVERR_CAPACITY).
__device__ __forceinline__ void fused_tile(const lb_plan_tile* const* nt_of, int n_steps, int x, lb_plan_tile* F,
                                           bool* same_rows, int* n_spans) {
  const lb_plan_tile* t0 = &nt_of[0][x];
  F->q_start = t0->q_start;
  F->q_len = t0->q_len;
  F->q_pos0 = t0->q_pos0;
#pragma unroll
  for (int o = 0; o < LB_MAX_SPANS; ++o) {
    F->k_start[o] = 0;
    F->k_len[o] = 0;
    F->k_pos0[o] = 0;
    F->k_lo[o] = LB_NO_LOWER_BOUND;
  }
  int ns = 0, blocks = 0;
  int64_t cost = 0;
  uint32_t steps = 0;
  bool same = true;
  for (int s = 0; s < n_steps; ++s) {
    const lb_plan_tile* t = &nt_of[s][x];
    same = same && t->q_start == F->q_start && t->q_len == F->q_len && t->q_pos0 == F->q_pos0;
    const int tn = min(max(t->n_spans, 0), LB_MAX_SPANS);
    // span slots chosen by comparison, not by a computed index: the tile stays in registers
#pragma unroll
    for (int sp = 0; sp < LB_MAX_SPANS; ++sp) {
      if (sp >= tn) break;
#pragma unroll
      for (int o = 0; o < LB_MAX_SPANS; ++o)
        if (o == ns) {
          F->k_start[o] = t->k_start[sp];
          F->k_len[o] = t->k_len[sp];
          F->k_pos0[o] = t->k_pos0[sp];
        }
      if (ns < LB_MAX_SPANS) steps |= (uint32_t)s << (4 * ns);
      ++ns;
    }
    cost += t->cost;
    blocks += t->blocks;
  }
  F->n_spans = min(ns, LB_MAX_SPANS);
  F->cost = cost;
  F->blocks = blocks;
  F->reserved = (int32_t)steps;
  *same_rows = same;
  *n_spans = ns;
}

__global__ __launch_bounds__(NT) void ring_fuse_kernel(RingMergeArgs m) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[kFusedTileCap];
  __shared__ const lb_plan_tile* nt_of[kMaxPlanSteps];
  __shared__ int32_t n_of[kMaxPlanSteps], err_of[kMaxPlanSteps];
  __shared__ int64_t pairs_of[kMaxPlanSteps];
  __shared__ int32_t err;        // written by thread 0 before the second barrier only
  __shared__ int32_t err_tiles;  // found while the tiles are gathered
  __shared__ int32_t n_empty;
  const int tid = threadIdx.x;
  const int n_steps = m.n_steps;
  WsHeader* rh = reinterpret_cast<WsHeader*>(m.ring);
  lb_plan_tile* out = reinterpret_cast<lb_plan_tile*>(m.ring + kRingTilesOffset);
  if (tid < n_steps) {
    const int s = tid;
    const WsHeader* h = reinterpret_cast<const WsHeader*>(m.step_ws[s]);
    const int64_t nt = h->n_tiles;
    // a step's plan must be a forward block plan made for these shapes, with its natural-order
    // tiles inside its workspace; its own error bits pass on
    const bool bad = h->magic != kPlanMagic || h->transposed != 0 || h->has_lower != 0 ||
                     h->plan_n_q != m.n_q || h->plan_n_kv != m.n_kv[s] || h->plan_heads != m.heads ||
                     h->plan_kv_heads != m.kv_heads || nt < 0 || h->off_ntiles < kWorkersOffset ||
                     h->off_ntiles + nt * (int64_t)sizeof(lb_plan_tile) > m.step_ws_bytes[s];
    err_of[s] = bad ? LB_DEVERR_PLAN : h->err;
    n_of[s] = bad ? 0 : (int)nt;
    nt_of[s] = reinterpret_cast<const lb_plan_tile*>(m.step_ws[s] + (bad ? 0 : h->off_ntiles));
    pairs_of[s] = bad ? 0 : h->total_pairs;
  }
  if (tid == 0) {
    err_tiles = 0;
    n_empty = 0;
  }
  __syncthreads();
  if (tid == 0) {
    int e = 0;
    for (int s = 0; s < n_steps; ++s) e |= err_of[s] | (n_of[s] != n_of[0] ? LB_DEVERR_PLAN : 0);
    if (n_of[0] > kFusedTileCap || n_of[0] > m.ring_cap) e |= LB_DEVERR_CAPACITY;
    err = e;
  }
  __syncthreads();
  const int N = err == 0 ? n_of[0] : 0;
  // pass 1: every tile's key (and its checks)
  for (int x = tid; x < N; x += NT) {
    lb_plan_tile F;
    bool same;
    int ns;
    fused_tile(nt_of, n_steps, x, &F, &same, &ns);
    if (!same) atomicOr(&err_tiles, LB_DEVERR_PLAN);
    if (ns > LB_MAX_SPANS) atomicOr(&err_tiles, LB_DEVERR_SPANS);
    if (F.blocks <= 0) atomicAdd(&n_empty, 1);
    keys[x] = (uint32_t)(32767 - min(max(F.blocks, 0), 32767)) << 17 | (uint32_t)x;
  }
  const int n4 = (N + 3) & ~3;
  if (tid < n4 - N) keys[N + tid] = ~0u;  // above every key: never counted
  __syncthreads();
  // pass 2: each tile's rank among the keys (unique, so the ranks are a permutation), and the
  // tile written at it
  if (err_tiles == 0) {
    const uint4* keys4 = reinterpret_cast<const uint4*>(keys);
    for (int x = tid; x < N; x += NT) {
      const uint32_t k = keys[x];
      int rank = 0;
      for (int i = 0; i < n4 / 4; ++i) {
        const uint4 v = keys4[i];
        rank += (v.x < k ? 1 : 0) + (v.y < k ? 1 : 0) + (v.z < k ? 1 : 0) + (v.w < k ? 1 : 0);
      }
      lb_plan_tile F;
      bool same;
      int ns;
      fused_tile(nt_of, n_steps, x, &F, &same, &ns);
      out[rank] = F;
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int e = err | err_tiles;
    const bool ok = e == 0;
    int64_t p = 0;
    for (int s = 0; s < n_steps; ++s) p += pairs_of[s];
    const int nq = m.kv_heads % kXcds == 0 ? kXcds : 1;
    const int n_work = ok ? N - n_empty : 0;
    rh->err = e;
    rh->n_frags = 0;
    rh->n_kvruns = 0;
    rh->n_tiles = ok ? N : 0;
    rh->n_empty = ok ? n_empty : 0;
    rh->n_items = n_work * m.kv_heads;
    rh->n_queues = nq;
    rh->per_queue = n_work * m.kv_heads / nq;
    for (int q = 0; q < kXcds; ++q) rh->queue_head[q] = 0;
    rh->tile_rows = 0;
    rh->n_workers = 0;
    rh->off_frags = rh->off_kvruns = 0;
    rh->off_tiles = rh->off_order = kRingTilesOffset;  // queue order is storage order
    rh->off_workers = kWorkersOffset;
    rh->off_ntiles = 0;
    rh->cap_frags = 0;
    rh->cap_tiles = m.ring_cap;
    rh->total_pairs = ok ? p : 0;
    rh->transposed = 0;
    rh->has_lower = 0;
    rh->plan_n_q = m.n_q;
    rh->plan_n_kv = 0;
    rh->plan_heads = m.heads;
    rh->plan_kv_heads = m.kv_heads;
    rh->ring_steps = n_steps;
    for (int s = 0; s < kMaxPlanSteps; ++s) rh->ring_n_kv[s] = s < n_steps ? m.n_kv[s] : 0;
    rh->ring_fused = 1;
    rh->done = 0;
    rh->magic = kRingMagic;
  }
}

}  // namespace

hipError_t launch_ring_merge(const RingMergeArgs& m, hipStream_t s) {
  hipLaunchKernelGGL(ring_merge_kernel, dim3(1), dim3(NT), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_ring_fuse(const RingMergeArgs& m, hipStream_t s) {
  hipLaunchKernelGGL(ring_fuse_kernel, dim3(1), dim3(NT), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_plan_steps(const PlanBatch& b, int n_steps, hipStream_t s) {
  hipLaunchKernelGGL(plan_steps_kernel, dim3(n_steps), dim3(NT), 0, s, b);
  return hipGetLastError();
}

}  // namespace lb
