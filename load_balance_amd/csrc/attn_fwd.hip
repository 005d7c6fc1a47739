// Persistent masked attention forward for gfx950 (MI355X).
//
// Work items are (tile, key/value head) pairs taken from the longest-first
// queue the planning kernel wrote: every workgroup loops "pop the next item,
// run it", so an idle compute unit always takes the largest remaining item --
// LPT list scheduling ("03 · 长文负载均衡", section 2.1, VRSP's LPT placement;
// "数据并行负载均衡", section 4.4, the greedy first phase), done at run time
// rather than from a static assignment because equal FLOPs do not take equal
// time on every device (same page, section 2.1: 256 identical GPUs differ by
// about 7%).
//
// Per item the workgroup runs blocked attention with online softmax (the
// FlashAttention prerequisite of "长序列训练与上下文并行"): key/value blocks of
// 64 tokens go through LDS; each of the 8 waves owns 32 query rows of one of
// the G = H/H_kv query heads that share the key/value head, so one K/V load
// serves G heads.  Both products run on bf16 MFMA (v_mfma_f32_32x32x16_bf16)
// with fp32 accumulation, in transposed form so that no register transpose is
// needed:
//   S^T[key][q] = K . Q^T    A = K rows from LDS, B = Q held in registers
//   O^T[d][q]  += V^T . P^T  A = V read transposed from LDS, B = P^T straight from S^T
// K and V blocks reach LDS by direct global -> LDS copies, two blocks ahead, into a
// 4-slot ring of swizzled row tiles; V^T fragments come from gfx950's LDS transpose load.
// A lane of the 32x32 accumulator owns one query column (q = lane % 32), so
// row max / row sum are per-lane loops plus one exchange with lane ^ 32, and
// the rescale of O is a per-lane scalar.  Exponentials use exp2 with the
// softmax scale folded into one FMA.  The running maximum is only moved when
// it grows by more than 2^8 in the exp2 domain, which keeps every exp2 <= 256
// (safe in fp32/bf16) and skips almost all rescales of O.
//
// Masking is decided per (wave, key block): blocks entirely above the wave's
// diagonal are skipped, blocks entirely visible take the mask-free path, only
// diagonal and ragged blocks evaluate "key position <= query position" per
// element.
#include "lbattn_internal.h"
#include "lds_staging.h"

namespace lb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BN = kBlockN;
constexpr int kStages = 4;  // LDS ring: the lagging waves read block j-1, block j+1 has landed, j+2 lands
constexpr int kPairBits = 40;  // a workgroup's pairs stay below 2^40; its key blocks below 2^23
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kLn2 = 0.69314718055994530942f;

template <int D>
struct Lds {
  static constexpr int kBytes = BN * D * 2;  // a K block (64 swizzled rows); the V block follows
  static constexpr int stage = 2 * kBytes;
  static constexpr int copiesPerStage = 2 * TileCopier<D, BN>::kCopies;
};

// Output staging for the epilogue: each wave's rows, row-major, in 1/8 of the ring's stages
// 1 .. kStages-1 (stage 0 receives the next item's first key block meanwhile), in as many
// passes (32, 16 or 8 rows each) as that space requires.
template <int D, bool OUT_F32>
struct EpilogueLds {
  static constexpr int kRowBytes = D * (OUT_F32 ? 4 : 2);
  static constexpr int kStride = kRowBytes + 16;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBase = Lds<D>::stage;
  static constexpr int kSpace = ((kStages - 1) * Lds<D>::stage / kWaves) & ~15;
  static constexpr int kRows = 32 * kStride <= kSpace ? 32 : 16 * kStride <= kSpace ? 16 : 8;
  static constexpr int kPasses = 32 / kRows;
  static constexpr int kWaveBytes = kSpace;
  static_assert(kRows * kStride <= kSpace, "epilogue staging does not fit in the ring");
  static_assert(64 % kChunks == 0 && kRows % (64 / kChunks) == 0, "whole rows per store step");
};

__device__ __forceinline__ uint64_t device_clock() { return __builtin_amdgcn_s_memrealtime(); }

// The two halves of a wave hold the same query rows (lanes r and r + 32): the value of the
// lane 32 apart through v_permlane32_swap, a VALU exchange, rather than an LDS permute.  The
// swap leaves the partner's value in its first result on the upper half and in its second on
// the lower half.  (Combined directly, as op(first, second), the compiler folds the two
// results of a swap of one value into one.)
__device__ __forceinline__ float partner_lane(float x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_bit_cast(float, (lane & 32) ? r[0] : r[1]);
}

// Workgroup barrier that orders LDS only.  The waves of a workgroup share nothing through
// global memory here, and __syncthreads() would also wait for every outstanding global
// store (the previous item's output) to complete.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_getreg immediates: (size - 1) << 11 | offset << 6 | register id.
__device__ __forceinline__ uint32_t hw_id_reg() { return __builtin_amdgcn_s_getreg((31 << 11) | 4); }
__device__ __forceinline__ uint32_t xcc_id_reg() { return __builtin_amdgcn_s_getreg((15 << 11) | 20); }

// Raw buffer resource word 3 for gfx9-family dword loads (no format conversion).


// Uniform description of one key block: which span, which block of it.
struct KvBlock {
  int key0;   // first key of the block, relative to its span
  int len;    // keys of the span (already clipped to the tile's last row)
  int pos0;   // mask position of the span's first key
  int start;  // first key row of the span
  int lo0;    // lower bound: key j of the span is visible to a row at position p only if lo0 + j >= p
};

// LOWER: spans may carry a lower bound on their visible keys (INV-CAUSAL and BI-CAUSAL
// slices).  Without it the kernel refuses such plans: the bound costs scalar registers in
// the key loop, so the common instance goes without.
// RING: the workspace is a ring workspace, several block steps' tiles in one longest-first
// queue; a tile's step (its `reserved` field) selects the keys, values and outputs of that
// step in r.  One launch then runs every step of a rank's ring, each step's partial into its
// own buffers, with no tail per step.
// FUSED (with RING): a fused ring, one tile per query tile with the key spans of every step (span
// s's step in bits 4s..4s+3 of the tile's `reserved`); an item runs its rows against the keys of
// every step in one online softmax and writes the merged result to the first step's buffers.
template <int D, bool OUT_F32, bool LOWER, bool RING, bool FUSED = false>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs a, RingSteps r) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * Lds<D>::stage];
  // s_item[p]: the item after the one whose descriptor is in s_tile[p] (written by thread 0
  // when that item starts, read by every wave in its epilogue).  Two entries, so that thread
  // 0 can write the next one while a slower wave still reads the last one, and the epilogue
  // needs no closing barrier.
  __shared__ int s_item[2];
  // The descriptors of the item being run and of the next one, copied from the plan by wave 0
  // with direct global-to-LDS loads while the previous item runs, so that no wave waits on a
  // global round trip for a descriptor between items.
  __shared__ __attribute__((aligned(16))) lb_plan_tile s_tile[2];
  // Thread 0's bookkeeping (queue state, counts for the worker record) lives in LDS, so that
  // it holds no register through the key loop.
  __shared__ struct {
    uint64_t t_start;
    int64_t pairs;  // visible pairs in the low kPairBits, key blocks swept above them
    int items;
    int queue;      // the queue this workgroup pops from
    int dry;        // every queue found empty
  } s_pop;

  // LDS addresses of the ring and of the descriptor slots, for the direct copies
  const uint32_t ring_lds = lds_addr(smem), tile_lds = lds_addr(s_tile);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  // Waves 0-3 and 4-7 share the four SIMDs pairwise.  The second group runs half a key
  // block behind the first (softmax and PV of block j-1, then QK^T of block j), so on every
  // SIMD one wave feeds the matrix cores while the other runs the exponentials.
  const bool lagging = wave >= 4;

  WsHeader* hdr = reinterpret_cast<WsHeader*>(a.ws);
  // A missing plan, or one made for other shapes or another workspace size, could index
  // outside this launch's buffers: then run nothing and flag it.
  const int64_t n_tiles_hdr = hdr->n_tiles;
  bool mismatch = hdr->magic != (RING ? kRingMagic : kPlanMagic) || hdr->transposed != 0 ||
                  (!LOWER && hdr->has_lower != 0) ||
                        hdr->plan_n_q != a.n_q ||
                        hdr->plan_n_kv != a.n_kv ||
                        hdr->plan_kv_heads != a.kv_heads || hdr->plan_heads != a.heads ||
                        hdr->n_empty < 0 || hdr->n_empty > n_tiles_hdr ||
                        hdr->n_items != (n_tiles_hdr - hdr->n_empty) * a.kv_heads || n_tiles_hdr < 0 ||
                        (hdr->n_queues != 1 && hdr->n_queues != kXcds) || a.kv_heads % hdr->n_queues != 0 ||
                        (int64_t)hdr->per_queue * hdr->n_queues != hdr->n_items ||
                        hdr->off_tiles < kWorkersOffset || hdr->off_order < kWorkersOffset ||
                        hdr->off_tiles + n_tiles_hdr * (int64_t)sizeof(lb_plan_tile) > a.ws_bytes ||
                        hdr->off_order + n_tiles_hdr * 4 > a.ws_bytes;
  if constexpr (RING) {
    // the ring was merged from plans made for these steps' key/value counts
    mismatch = mismatch || r.n_steps < 1 || r.n_steps > kMaxPlanSteps || hdr->ring_steps != r.n_steps ||
               hdr->ring_fused != (FUSED ? 1 : 0);
#pragma unroll
    for (int s = 0; s < kMaxPlanSteps; ++s)
      if (s < r.n_steps && hdr->ring_n_kv[s] != r.n_kv[s]) mismatch = true;
  }
  const int n_items = mismatch ? 0 : hdr->n_items;
  // plans and rings both store their tiles in queue order: tile i of the queue is tiles[i]
  const lb_plan_tile* tiles = reinterpret_cast<const lb_plan_tile*>(a.ws + (mismatch ? 0 : hdr->off_tiles));
  if (mismatch && blockIdx.x == 0 && tid == 0) atomicOr(&hdr->err, LB_DEVERR_PLAN);
  auto tile_at = [&](int64_t i) -> const lb_plan_tile* { return &tiles[i]; };
  // a ring tile's step (a fused ring tile: its first span's), kept inside the launch's step table
  auto step_of = [&](const lb_plan_tile* T) -> int {
    const int v = __builtin_amdgcn_readfirstlane(T->reserved);
    return min(max(FUSED ? (v & 15) : v, 0), r.n_steps - 1);
  };

  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q);
  const char* Kb = reinterpret_cast<const char*>(a.k);
  const char* Vb = reinterpret_cast<const char*>(a.v);
  const int row_bytes = a.kv_heads * D * 2;  // one token's K (or V) across all kv heads
  TileCopier<D, BN> copier;  // this wave's share of a K or V block's copy
  copier.init(row_bytes, wave, lane);
  TrOffsets<D> vt_off;  // lane offsets of the V^T fragments in a value block
  vt_off.init(lane);

  const int G = a.group;
  const int head_in_group = wave % G;
  const int wr0 = (wave / G) * kRowsPerWave;  // first tile row of this wave
  const float c = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  if (tid == 0) {
    s_pop.t_start = device_clock();
    s_pop.pairs = 0;
    s_pop.items = 0;
  }


  // Tiles with no key span only set lse = -inf on their rows: a grid-stride pass before the
  // queues, without barriers or LDS.
  {
    const int n_empty = mismatch ? 0 : hdr->n_empty;
    for (int e = blockIdx.x; e < n_empty; e += gridDim.x) {
      const lb_plan_tile* T = tile_at(n_tiles_hdr - n_empty + e);
      const int q_start = T->q_start, q_len = T->q_len;
      float* lse_e = a.lse;
      if constexpr (RING) lse_e = r.lse[FUSED ? 0 : step_of(T)];
      for (int idx = tid; idx < q_len * a.heads; idx += kThreads)
        lse_e[(int64_t)(idx / q_len) * a.n_q + q_start + idx % q_len] = -__builtin_inff();
    }
  }

  // Work queues: with one queue per XCD, a workgroup serves its own XCD's queue (kv heads
  // q, q + 8, ...) so the XCD's L2 keeps those heads' keys and values, and steals from the
  // other queues, in turn, once its own is empty.
  const int n_queues = mismatch ? 1 : hdr->n_queues;
  const int per_queue = mismatch ? 0 : hdr->per_queue;
  const int heads_per_queue = a.kv_heads / n_queues;
  if (tid == 0) {
    s_pop.queue = (int)(xcc_id_reg() % (uint32_t)n_queues);
    s_pop.dry = n_items == 0;
  }

  // Thread 0: completes a pop whose atomicAdd on the current queue returned k.  A dry queue
  // sends it on to the next queue in rotation that still holds items, judged from one read
  // of every queue head (another workgroup may still empty that queue first).
  auto finish_pop = [&](int k) -> int {
    int queue = s_pop.queue, item = -1;
    bool queues_dry = s_pop.dry != 0;
    while (!queues_dry) {
      if (k < per_queue) {
        item = queue * per_queue + k;
        break;
      }
      int heads[kXcds];
#pragma unroll
      for (int q = 0; q < kXcds; ++q)
        heads[q] = q < n_queues ? __atomic_load_n(&hdr->queue_head[q], __ATOMIC_RELAXED) : per_queue;
      int next = -1;
      for (int step = 1; step < n_queues; ++step) {
        const int q = (queue + step) % n_queues;
        if (heads[q] < per_queue) { next = q; break; }
      }
      if (next < 0) { queues_dry = true; break; }
      queue = next;
      k = atomicAdd(&hdr->queue_head[queue], 1);
    }
    s_pop.queue = queue;
    s_pop.dry = queues_dry;
    return item;
  };
  // thread 0: the first step of a pop, or -1 with the queues dry
  auto start_pop = [&]() -> int { return s_pop.dry ? -1 : atomicAdd(&hdr->queue_head[s_pop.queue], 1); };
  if (tid == 0) {
    const int k = start_pop();
    s_item[1] = k < 0 ? -1 : finish_pop(k);  // as if an item in slot 1 had run before
  }
  lds_barrier();
  int qitem = __builtin_amdgcn_readfirstlane(s_item[1]);

  // The loads an item starts with, issued before it starts so that their latency hides
  // behind the previous item's end: this wave's Q fragment (B operand of S^T = K Q^T; lane
  // holds Q[q = l32][d = kk*16 + hh*8 .. +8], zeros past the tile's end) and the first key
  // block, copied into ring slot 0.
  bf16x8 qreg[D / 16];
  auto issue_q = [&](int item, const lb_plan_tile* T) {
    const int q_of = item / max(per_queue, 1), k_in = item - q_of * per_queue;
    const int g = q_of + n_queues * (k_in % heads_per_queue);
    const int q_start = __builtin_amdgcn_readfirstlane(T->q_start);
    const int q_len = __builtin_amdgcn_readfirstlane(T->q_len);
    const int n_spans = __builtin_amdgcn_readfirstlane(T->n_spans);
    // one buffer over this wave's rows of the tile: no branches (a branch around a load
    // makes the compiler wait for every load before it), zeros past the tile's end
    const int head = __builtin_amdgcn_readfirstlane(g * G + head_in_group);
    const int w0 = __builtin_amdgcn_readfirstlane(wr0);
    const int q_row_bytes = a.heads * D * 2;
    const int rows = n_spans > 0 ? min(max(q_len - w0, 0), kRowsPerWave) : 0;
    const uint64_t q_off = ((uint64_t)(q_start + w0) * a.heads + head) * D * 2;
    const uint64_t q_off_u = (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)q_off) |
                             ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(q_off >> 32)) << 32);
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<const char*>(Q) + q_off_u), (short)0,
                                          __builtin_amdgcn_readfirstlane(rows * q_row_bytes), kBufferFlags);
    const int voff = l32 * q_row_bytes + hh * 16;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qreg[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, voff + kk * 32, 0, 0));
  };
  auto issue_block0 = [&](int item, const lb_plan_tile* T) {
    const int q_of = item / max(per_queue, 1), k_in = item - q_of * per_queue;
    const int g = q_of + n_queues * (k_in % heads_per_queue);
    const int n_spans = __builtin_amdgcn_readfirstlane(T->n_spans);
    const char* Kx = Kb;
    const char* Vx = Vb;
    if constexpr (RING) {
      const int st = step_of(T);
      Kx = reinterpret_cast<const char*>(r.k[st]);
      Vx = reinterpret_cast<const char*>(r.v[st]);
    }
    const int k_start0 = __builtin_amdgcn_readfirstlane(T->k_start[0]);
    const int k_len0 = __builtin_amdgcn_readfirstlane(T->k_len[0]);
    if (n_spans > 0) {
      const uint32_t lds = ring_lds;  // block 0 goes to slot 0 (kept out of the epilogue staging)
      const int valid = __builtin_amdgcn_readfirstlane(min(k_len0, BN));
      copier.issue(Kx, row_bytes, k_start0, valid, g, lds);
      copier.issue(Vx, row_bytes, k_start0, valid, g, lds + Lds<D>::kBytes);
    }
  };
  // Wave 0 copies an item's 96-byte descriptor into an LDS slot (lanes 0-5, 16 bytes each);
  // the copy lands asynchronously and is waited for before the barrier that precedes its use.
  auto fetch_tile = [&](int item, lb_plan_tile* slot) {
    // through a buffer over the queue's tiles: the tile's offset in a scalar register, each
    // lane's 16-byte piece in a 32-bit vector offset (no 64-bit address per lane)
    const int q_of = item / max(per_queue, 1), k_in = item - q_of * per_queue;
    const int t_off = __builtin_amdgcn_readfirstlane((k_in / heads_per_queue) * (int)sizeof(lb_plan_tile));
    const i32x4 rt = buffer_rsrc(reinterpret_cast<const char*>(tiles) + t_off,
                                 (int)sizeof(lb_plan_tile));
    if (wave == 0 && lane < (int)(sizeof(lb_plan_tile) / 16))
      copy16_to_lds(rt, tile_lds + (uint32_t)((char*)slot - (char*)s_tile), lane * 16);
  };
  auto wait_tile = [&]() {
    if (wave == 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the descriptor copy has landed
  };
  int slot = 0;  // s_tile[slot] holds the descriptor of the item being run
  // Items are popped one ahead of the one whose loads go out: thread 0 issues the atomic in
  // an item's epilogue and completes the pop at the next item's start, so the round trip
  // sits on no wave's path.  s_item[slot] then holds the item after the one being run.
  int k_after = -1;  // thread 0: that atomic's result, or -1 with the queues dry
  if (qitem >= 0) {
    fetch_tile(qitem, &s_tile[0]);
    wait_tile();
    lds_barrier();
    issue_q(qitem, &s_tile[0]);
    issue_block0(qitem, &s_tile[0]);
    if (tid == 0) k_after = start_pop();
  }

  while (qitem >= 0) {

    // item k of queue q: tile order[k / heads_per_queue], kv head q + n_queues * (k % heads_per_queue)
    const int q_of = qitem / max(per_queue, 1), k_in = qitem - q_of * per_queue;
    const int g = q_of + n_queues * (k_in % heads_per_queue);
    const lb_plan_tile* T = &s_tile[slot];  // this item's descriptor, in LDS
    const char* Kit = Kb;
    const char* Vit = Vb;
    int step = 0;              // the step whose buffers the item writes
    uint32_t span_steps = 0;   // FUSED: span s's step in bits 4s..4s+3
    if constexpr (RING) {
      const int st0 = step_of(T);
      Kit = reinterpret_cast<const char*>(r.k[st0]);
      Vit = reinterpret_cast<const char*>(r.v[st0]);
      if constexpr (FUSED) span_steps = __builtin_amdgcn_readfirstlane((uint32_t)T->reserved);
      else step = st0;
    }
    // tile fields, read once and kept wave-uniform
    const int q_start = __builtin_amdgcn_readfirstlane(T->q_start);
    const int q_len = __builtin_amdgcn_readfirstlane(T->q_len);
    const int q_pos0 = __builtin_amdgcn_readfirstlane(T->q_pos0);
    const int n_spans = __builtin_amdgcn_readfirstlane(T->n_spans);
    // Span fields ride in the lanes of one register: lanes 0-3 k_start, 4-7 k_len, 8-11 k_pos0,
    // 12-15 k_lo; a wave reads them back with v_readlane only when it steps into a new span.
    const int span_v = lane < (LOWER ? 4 : 3) * LB_MAX_SPANS ? (&T->k_start[0])[lane] : 0;
    int n_kv_tiles = 0;
#pragma unroll
    for (int s = 0; s < LB_MAX_SPANS; ++s)
      if (s < n_spans) n_kv_tiles += (__builtin_amdgcn_readlane(span_v, LB_MAX_SPANS + s) + BN - 1) / BN;
    if (tid == 0) {
      ++s_pop.items;
      s_pop.pairs += T->cost * G + (static_cast<int64_t>(n_kv_tiles) << kPairBits);
      s_item[slot] = k_after < 0 ? -1 : finish_pop(k_after);
    }
    // the next item's descriptor goes to the other slot while this item runs (thread 0 has
    // just popped it; lane 0 of wave 0 is thread 0)
    if (wave == 0) {
      const int nxt_item = __builtin_amdgcn_readfirstlane(s_item[slot]);
      if (nxt_item >= 0) fetch_tile(nxt_item, &s_tile[slot ^ 1]);
    }
    auto span_of = [&](int s) {
      KvBlock b;
      b.key0 = 0;
      b.start = __builtin_amdgcn_readlane(span_v, s);
      b.len = __builtin_amdgcn_readlane(span_v, LB_MAX_SPANS + s);
      b.pos0 = __builtin_amdgcn_readlane(span_v, 2 * LB_MAX_SPANS + s);
      b.lo0 = LOWER ? __builtin_amdgcn_readlane(span_v, 3 * LB_MAX_SPANS + s) : LB_NO_LOWER_BOUND;
      return b;
    };

    const int head = g * G + head_in_group;
    const int my_row = wr0 + l32;                 // tile row owned by this lane
    const bool wave_rows = wr0 < q_len;           // this wave has at least one real row
    const int wave_last = min(wr0 + kRowsPerWave, q_len) - 1;
    const int64_t grow = (int64_t)q_start + my_row;
    const int qpos = q_pos0 + my_row;


    f32x16 acc_o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc_o[i] = f32x16{};
    float m_used = -__builtin_inff();
    float l_part = 0.f;
    f32x16 acc_s[2];

    // does key block b have any visible pair for this wave's real rows?
    // (and, under a lower bound, does the block's last key reach down to the wave's first row?)
    auto live = [&](const KvBlock& b) {
      return wave_rows && b.pos0 + b.key0 <= q_pos0 + wave_last && (!LOWER || b.lo0 + b.key0 + BN - 1 >= q_pos0 + wr0);
    };

    auto qk = [&](const char* ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        acc_s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 kf = row_frag<D>(ks, kb * 32 + l32, 2 * kk + hh);
          acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[kk], acc_s[kb], 0, 0, 0);
        }
      }
    };

    // mask (diagonal / ragged blocks only), online softmax, O^T += V^T P^T
    auto softmax_pv = [&](const KvBlock& b, const char* vs) {
      const bool full = b.key0 + BN <= b.len && b.pos0 + b.key0 + BN - 1 <= q_pos0 + wr0 &&
                        (!LOWER || b.lo0 + b.key0 >= q_pos0 + wave_last);
      if (!full) {
        // key k of the block is visible iff k < lim (span end, and position <= this row's)
        // and, under a lower bound, k >= lim_lo
        const int lim = min(b.len, qpos - b.pos0 + 1) - b.key0 - hh * 4;
        if constexpr (LOWER) {
          const int lim_lo = qpos - b.lo0 - b.key0 - hh * 4;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int k = kb * 32 + (i / 4) * 8 + (i % 4);
              if (!(k < lim && k >= lim_lo)) acc_s[kb][i] = -__builtin_inff();
            }
        } else {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (!(kb * 32 + (i / 4) * 8 + (i % 4) < lim)) acc_s[kb][i] = -__builtin_inff();
        }
      }
      // row max as a tree of 3-input maxima (depth 4, not a chain of 16).  The NaN-propagating
      // maximum maps to gfx950's v_maximum3_f32 as it is; fmaxf would first quiet its inputs.
      auto mx2 = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
      float t[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int e = 3 * i;
        t[i] = mx2(mx2(acc_s[e / 16][e % 16], acc_s[(e + 1) / 16][(e + 1) % 16]), acc_s[(e + 2) / 16][(e + 2) % 16]);
      }
      t[10] = mx2(acc_s[1][14], acc_s[1][15]);
      const float u0 = mx2(mx2(t[0], t[1]), t[2]), u1 = mx2(mx2(t[3], t[4]), t[5]);
      const float u2 = mx2(mx2(t[6], t[7]), t[8]), u3 = mx2(t[9], t[10]);
      const float m_own = mx2(mx2(u0, u1), mx2(u2, u3));
      const float mx = mx2(m_own, partner_lane(m_own, lane));
      const float m_tile = mx * c;
      const bool need = m_tile > m_used + kRescaleThreshold;  // false when the row saw nothing
      if (__any(need)) {
        const float m_new = need ? m_tile : m_used;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_used - m_new) : 1.0f;
        m_used = m_new;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
      }
      const float m_sub = m_used == -__builtin_inff() ? 0.0f : m_used;
      // P^T in bf16, chunk ks16 = keys ks16*16 .. +16 of the block (S^T rows acc_s[ks16 / 2],
      // elements (ks16 % 2) * 8 ..): pairs [p0, p1) of its four
      bf16x8 pf[4];
      float lsum[2] = {0.0f, 0.0f};  // this block's row sum, in two chains
      auto exp_pairs = [&](int ks16, int p0, int p1) {
        const int kb = ks16 / 2, cc = ks16 % 2;
#pragma unroll
        for (int p = p0; p < p1; ++p) {
          const int j = 2 * p;
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[kb][cc * 8 + j], c, -m_sub));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[kb][cc * 8 + j + 1], c, -m_sub));
          const bf16x2 pp = {(__bf16)e0, (__bf16)e1};
          // the row sum takes exactly the bf16 weights that enter the PV product
          lsum[ks16 & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum[ks16 & 1], false);
          pf[ks16][j] = pp[0];
          pf[ks16][j + 1] = pp[1];
        }
      };
      constexpr int kDb = D / 32;             // 32-wide d blocks of O^T
      constexpr int kPairsPerMfma = 4 / kDb;  // exponential pairs of the next chunk per MFMA
      auto read_v = [&](int ks16, bf16x8* dst) {
#pragma unroll
        for (int db = 0; db < kDb; ++db)
          dst[db] = tr_frag_at<D>(vs, vt_off, ks16 * 16, db);
      };
      // An explicit pipeline, fenced so that the scheduler keeps it whatever surrounds the
      // loop: the MFMAs of chunk ks run with the exponentials of chunk ks + 1 between them,
      // while the V^T fragments of chunk ks + 2 are read.
      bf16x8 vf[2][kDb];
      read_v(0, vf[0]);
      __builtin_amdgcn_sched_barrier(0);
      exp_pairs(0, 0, 4);
      read_v(1, vf[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < kDb; ++db) {
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks & 1][db], pf[ks], acc_o[db], 0, 0, 0);
          if (ks + 1 < 4) exp_pairs(ks + 1, db * kPairsPerMfma, (db + 1) * kPairsPerMfma);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (ks + 2 < 4) read_v(ks + 2, vf[ks & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      l_part += lsum[0] + lsum[1];
    };

    // Block 0 was copied into slot 0 during the previous epilogue, with this wave's Q
    // fragment: both are waited for here, before any copy of this item goes out (a wait for
    // the fragment inside the loop would also wait for every copy in flight).  Block b goes
    // to slot b % kStages; at block `it` the copy of block it + 2 goes out (blocks 1 and 2 at
    // block 0, once the key loop's first barrier has ended every wave's epilogue staging).
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    int cur_s = 0;
    KvBlock cur = span_of(0);
    int iss_s = 0;  // the next block to copy in
    KvBlock iss = cur;
    auto advance = [&](KvBlock& b, int& s) {
      b.key0 += BN;
      if (b.key0 >= b.len) {
        ++s;
        if (s < n_spans) b = span_of(s);
      }
    };
    advance(iss, iss_s);
    auto issue_block = [&](int slot_i) {
      const uint32_t lds = ring_lds + slot_i * Lds<D>::stage;
      const int k0 = __builtin_amdgcn_readfirstlane(iss.start + iss.key0);
      const int valid = __builtin_amdgcn_readfirstlane(min(iss.len - iss.key0, BN));
      const char* Kx = Kit;
      const char* Vx = Vit;
      if constexpr (FUSED) {  // the keys and values of the step the span belongs to
        const int st = min((int)(span_steps >> (4 * iss_s)) & 15, r.n_steps - 1);
        Kx = reinterpret_cast<const char*>(r.k[st]);
        Vx = reinterpret_cast<const char*>(r.v[st]);
      }
      copier.issue(Kx, row_bytes, k0, valid, g, lds);
      copier.issue(Vx, row_bytes, k0, valid, g, lds + Lds<D>::kBytes);
      advance(iss, iss_s);
    };
    KvBlock prev{0, 0, 0, 0, LB_NO_LOWER_BOUND};
    bool prev_live = false;

    for (int it = 0; it < n_kv_tiles; ++it) {
      // this wave's copies of block `it` have landed once at most those of block it + 1 are in
      // flight; the barrier publishes every wave's, and frees slot it + 2 (block it - 2)
      if (it > 0 && it + 1 < n_kv_tiles) wait_stage(1, Lds<D>::copiesPerStage);
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      if (it == 0) {
        if (1 < n_kv_tiles) issue_block(1);
        if (2 < n_kv_tiles) issue_block(2);
      } else if (it + 2 < n_kv_tiles) {
        issue_block((it + 2) % kStages);
      }
      const char* stage = smem + (it % kStages) * Lds<D>::stage;
      const char* prev_stage = smem + ((it + kStages - 1) % kStages) * Lds<D>::stage;
      const bool cur_live = live(cur);
      if (!lagging) {
        if (cur_live) {
          qk(stage);
          softmax_pv(cur, stage + Lds<D>::kBytes);
        }
      } else {
        if (prev_live) softmax_pv(prev, prev_stage + Lds<D>::kBytes);
        if (cur_live) qk(stage);
      }
      prev = cur;
      prev_live = cur_live;
      advance(cur, cur_s);
    }
    if (lagging && prev_live)
      softmax_pv(prev, smem + ((n_kv_tiles + kStages - 1) % kStages) * Lds<D>::stage + Lds<D>::kBytes);
    // This wave's Q fragment for the next item goes out before the epilogue barrier (the
    // leading waves, done with their last block, otherwise wait there for the lagging ones):
    // the next item's number (s_item) and descriptor are published by the key loop's
    // barriers once it has two or more blocks (the descriptor copy is older than block 1's,
    // which the second barrier waits for), by a barrier of their own otherwise.
    if (n_kv_tiles < 2) {
      wait_tile();
      lds_barrier();
    }
    {
      const int nxt = __builtin_amdgcn_readfirstlane(s_item[slot]);
      if (nxt >= 0) issue_q(nxt, &s_tile[slot ^ 1]);
    }

    // ---- epilogue: out = O / l, lse = ln(sum exp) ----
    // Every wave is done with the LDS ring after this barrier (the next item's descriptor has
    // been published above): the next item's first block goes out first, then thread 0's
    // atomic for the item after it.  (No wait for wave 0's copies here: it would also wait for
    // its Q fragment, just issued.)
    lds_barrier();
    const int next_item = __builtin_amdgcn_readfirstlane(s_item[slot]);
    if (next_item >= 0) {
      issue_block0(next_item, &s_tile[slot ^ 1]);
      if (tid == 0) k_after = start_pop();
    }
    const float l_tot = l_part + partner_lane(l_part, lane);
    const bool row_real = wave_rows && my_row < q_len;
    const bool empty = !(l_tot > 0.0f);
    // rows written: bit r for tile row wr0 + r (lanes r and r + 32 hold the same row)
    const uint32_t wmask = (uint32_t)__ballot(row_real && !empty);
    const float inv = empty ? 0.0f : 1.0f / l_tot;
    // Lanes own query rows, so direct stores would put 32 rows, heads * D apart, into every
    // store instruction.  Each wave stages its rows row-major in its own slice of the ring
    // and stores them 16 contiguous bytes per lane.
    using Epi = EpilogueLds<D, OUT_F32>;
    // lane-only addresses stay here rather than being hoisted out of the item loop, where
    // they would hold registers through the whole key loop
    int t_e = tid;
    asm volatile("" : "+v"(t_e));
    const int lane_e = t_e & 63, l32_e = t_e & 31;
    char* ebuf = smem + Epi::kBase + (t_e >> 6) * Epi::kWaveBytes;
#pragma unroll
    for (int pass = 0; pass < Epi::kPasses; ++pass) {
      const int r_lo = pass * Epi::kRows;
      if (pass > 0) __builtin_amdgcn_wave_barrier();
      if (l32_e >= r_lo && l32_e < r_lo + Epi::kRows) {
        char* rowp = ebuf + (l32_e - r_lo) * Epi::kStride;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d0 = db * 32 + r * 8 + hh * 4;
            if constexpr (OUT_F32) {
              f32x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = acc_o[db][r * 4 + e] * inv;
              *reinterpret_cast<f32x4*>(rowp + d0 * 4) = o;
            } else {
              bf16x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc_o[db][r * 4 + e] * inv);
              *reinterpret_cast<bf16x4*>(rowp + d0 * 2) = o;
            }
          }
      }
      float* lse_out = a.lse;
      if constexpr (RING) lse_out = r.lse[step];
      if (pass == 0 && row_real && hh == 0)
        lse_out[(int64_t)head * a.n_q + grow] = empty ? -__builtin_inff() : (m_used + __builtin_log2f(l_tot)) * kLn2;
      // LDS instructions of one wave complete in order: the reads below see the writes above.
      // One step of 64 lanes covers kRowsPerStep whole rows.
      constexpr int kRowsPerStep = 64 / Epi::kChunks;
      const int row0 = lane_e / Epi::kChunks, ch = lane_e % Epi::kChunks;
      const char* src = ebuf + row0 * Epi::kStride + ch * 16;
      char* out_base = reinterpret_cast<char*>(a.out);
      if constexpr (RING) out_base = reinterpret_cast<char*>(r.out[step]);
      char* dst = out_base +
                  (((int64_t)q_start + wr0 + r_lo + row0) * a.heads + head) * Epi::kRowBytes + ch * 16;
      const int64_t dst_step = (int64_t)kRowsPerStep * a.heads * Epi::kRowBytes;
#pragma unroll
      for (int j = 0; j < Epi::kRows / kRowsPerStep; ++j) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(src + j * kRowsPerStep * Epi::kStride);
        if (wmask >> (r_lo + row0 + j * kRowsPerStep) & 1) *reinterpret_cast<u32x4*>(dst + j * dst_step) = x;
      }
    }
    // No barrier here: the next item's prologue writes only stage 0 of the ring (kept out of
    // the staging), s_item[slot ^ 1] and s_tile[slot] (read by no wave after the epilogue's
    // first barrier); the key loop's first barrier then orders the staging reads above
    // before the loader writes stages 1 and 2.
    qitem = next_item;
    slot ^= 1;
  }

  if (tid == 0) {
    lb_worker_record rec;
    rec.hw_id = hw_id_reg();
    rec.xcc_id = xcc_id_reg();
    rec.t_start = s_pop.t_start;
    rec.t_end = device_clock();
    rec.pairs = s_pop.pairs & ((int64_t{1} << kPairBits) - 1);
    rec.items = s_pop.items;
    rec.blocks = static_cast<int32_t>(s_pop.pairs >> kPairBits);
    lb_worker_record* recs = reinterpret_cast<lb_worker_record*>(a.ws + kWorkersOffset);
    recs[blockIdx.x] = rec;
    if (blockIdx.x == 0) hdr->n_workers = gridDim.x;
    // The last workgroup out rewinds the queue: every workgroup has made its final pop
    // before counting itself done, so no pop can follow the reset.
    __threadfence();
    if (atomicAdd(&hdr->done, 1) == (int)gridDim.x - 1) {
      for (int q = 0; q < kXcds; ++q) atomicExch(&hdr->queue_head[q], 0);
      atomicExch(&hdr->done, 0);
    }
  }
}

}  // namespace

template <int D, bool OUT_F32>
static void launch_d(const AttnArgs& a, bool lower, int n_workers, hipStream_t s) {
  const RingSteps none{};
  if (lower) hipLaunchKernelGGL((attn_kernel<D, OUT_F32, true, false>), dim3(n_workers), dim3(kThreads), 0, s, a, none);
  else hipLaunchKernelGGL((attn_kernel<D, OUT_F32, false, false>), dim3(n_workers), dim3(kThreads), 0, s, a, none);
}

hipError_t launch_attention(const AttnArgs& a, int d, bool out_f32, bool lower, int n_workers, hipStream_t s) {
  if (d == 128) {
    if (out_f32) launch_d<128, true>(a, lower, n_workers, s); else launch_d<128, false>(a, lower, n_workers, s);
  } else {
    if (out_f32) launch_d<64, true>(a, lower, n_workers, s); else launch_d<64, false>(a, lower, n_workers, s);
  }
  return hipGetLastError();
}

hipError_t launch_ring_attention(const AttnArgs& a, const RingSteps& r, int d, int n_workers, bool fused,
                                 hipStream_t s) {
  if (d == 128) {
    if (fused) hipLaunchKernelGGL((attn_kernel<128, true, false, true, true>), dim3(n_workers), dim3(kThreads), 0, s, a, r);
    else hipLaunchKernelGGL((attn_kernel<128, true, false, true>), dim3(n_workers), dim3(kThreads), 0, s, a, r);
  } else {
    if (fused) hipLaunchKernelGGL((attn_kernel<64, true, false, true, true>), dim3(n_workers), dim3(kThreads), 0, s, a, r);
    else hipLaunchKernelGGL((attn_kernel<64, true, false, true>), dim3(n_workers), dim3(kThreads), 0, s, a, r);
  }
  return hipGetLastError();
}

}  // namespace lb
