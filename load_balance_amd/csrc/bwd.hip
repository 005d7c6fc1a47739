// Backward of the masked attention for gfx950 (MI355X): dQ, dK, dV from the
// forward's saved log-sum-exp.
//
// The context-parallel systems of "03 · 长文负载均衡" train, so their attention
// blocks carry gradients: section 4.4 (MagiAttention) reduces the partial key/value
// gradients of every block back to the rank that owns the keys, and section 5 keeps
// key/value gradients with their states.  The gradient itself is the plain one of
// softmax attention, with P = exp(s - lse) rebuilt from the saved lse:
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Two persistent kernels share the forward's queue machinery and plan format:
//   * dQ, query-stationary, over the forward's query tiles and wave layout (8 waves,
//     two per SIMD, each 32 rows of one head): per 64-key block, S^T = K Q^T and
//     dP^T = V dO^T (K and V rows from LDS, Q and dO held in registers), then
//     dQ^T += K^T dS^T with K^T read transposed from the same LDS rows.
//   * dK/dV, key-stationary, over key tiles whose spans are the query rows that see
//     them (the transposed plan), in producer/consumer wave pairs: per block of 32
//     query rows and head, the producer computes S = Q K^T and dP = dO V^T (Q and dO
//     rows from LDS, K and V held in registers) and from them P and dS; the consumer
//     accumulates dV^T += dO^T P and dK^T += Q^T dS a block later.  The heads of a kv
//     group add into the same accumulators, so no reduction over heads follows.
// Both stream their row tiles through LDS rings filled by direct global->LDS copies;
// the transposed operands come from gfx950's LDS transpose load.
#include "lbattn_internal.h"
#include "lds_staging.h"

namespace lb {
namespace {

// compile-time flag for code written once for the masked and the mask-free path: a block
// fully visible to the wave takes the path without a compare per element
template <bool B>
struct Masked {
  static constexpr bool value = B;
};


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = kBlockN;  // keys per block of the dQ kernel
constexpr int kDqWaves = 8;
constexpr int kDqThreads = kDqWaves * 64;
constexpr int kQB = 32;      // query rows per stage of the dK/dV kernel (one MFMA block)

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint64_t device_clock() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t hw_id_reg() { return __builtin_amdgcn_s_getreg((31 << 11) | 4); }
__device__ __forceinline__ uint32_t xcc_id_reg() { return __builtin_amdgcn_s_getreg((15 << 11) | 20); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


// ------------------------------------------------------------------------------------
// The plan and its queues (same format and protocol as the forward's)
// ------------------------------------------------------------------------------------
// RING: the workspace is a ring workspace (several steps' tiles in one queue, stored in
// queue order, each tile's step in its `reserved` word).
template <bool RING>
struct QueuesT {
  WsHeader* hdr;
  const lb_plan_tile* tiles;
  const int32_t* order;
  int n_items, n_queues, per_queue, heads_per_queue, queue;
  int64_t n_tiles;
  int n_empty;
  bool dry;  // thread 0's view

  // fused: the ring must be a fused ring (lb_plan_ring_fused), else an unfused one
  __device__ void open(const BwdArgs& a, int transposed, const RingBwdSteps* r = nullptr, bool fused = false) {
    hdr = reinterpret_cast<WsHeader*>(a.ws);
    const int64_t nt = hdr->n_tiles;
    bool bad = hdr->magic != (RING ? kRingMagic : kPlanMagic) || hdr->transposed != transposed ||
               hdr->plan_n_q != a.n_q ||
                     hdr->plan_n_kv != a.n_kv || hdr->plan_kv_heads != a.kv_heads || hdr->plan_heads != a.heads ||
                     hdr->n_empty < 0 || hdr->n_empty > nt || hdr->n_items != (nt - hdr->n_empty) * a.kv_heads ||
                     nt < 0 || (hdr->n_queues != 1 && hdr->n_queues != kXcds) || a.kv_heads % hdr->n_queues != 0 ||
                     (int64_t)hdr->per_queue * hdr->n_queues != hdr->n_items || hdr->off_tiles < kWorkersOffset ||
                     hdr->off_order < kWorkersOffset ||
                     hdr->off_tiles + nt * (int64_t)sizeof(lb_plan_tile) > a.ws_bytes ||
                     hdr->off_order + nt * 4 > a.ws_bytes;
    if constexpr (RING) {
      // the ring was merged from plans made for these steps' key/value counts
      bad = bad || r->n_steps < 1 || r->n_steps > kMaxPlanSteps || hdr->ring_steps != r->n_steps ||
            hdr->ring_fused != (fused ? 1 : 0);
      for (int s = 0; s < kMaxPlanSteps; ++s)
        if (s < r->n_steps && hdr->ring_n_kv[s] != r->n_kv[s]) bad = true;
    }
    if (bad && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&hdr->err, LB_DEVERR_PLAN);
    n_items = bad ? 0 : hdr->n_items;
    n_tiles = bad ? 0 : nt;
    n_empty = bad ? 0 : hdr->n_empty;
    tiles = reinterpret_cast<const lb_plan_tile*>(a.ws + (bad ? 0 : hdr->off_tiles));
    order = reinterpret_cast<const int32_t*>(a.ws + (bad ? 0 : hdr->off_order));
    n_queues = bad ? 1 : hdr->n_queues;
    per_queue = bad ? 0 : hdr->per_queue;
    heads_per_queue = a.kv_heads / n_queues;
    queue = (int)(xcc_id_reg() % (uint32_t)n_queues);
    dry = n_items == 0;
  }

  // Thread 0: the next item (global index), or -1 when every queue is empty.
  __device__ int pop() {
    while (!dry) {
      const int k = atomicAdd(&hdr->queue_head[queue], 1);
      if (k < per_queue) return queue * per_queue + k;
      int next = -1;
      for (int step = 1; step < n_queues; ++step) {
        const int q = (queue + step) % n_queues;
        if (__atomic_load_n(&hdr->queue_head[q], __ATOMIC_RELAXED) < per_queue) { next = q; break; }
      }
      if (next < 0) dry = true; else queue = next;
    }
    return -1;
  }

  // item k of queue q: tile order[k / heads_per_queue], kv head q + n_queues * (k % heads_per_queue)
  __device__ void decode(int item, const lb_plan_tile** T, int* g) const {
    // the header fields come through vector loads: state that the results are uniform
    const int q_of = item / max(per_queue, 1), k_in = item - q_of * per_queue;
    *g = __builtin_amdgcn_readfirstlane(q_of + n_queues * (k_in % heads_per_queue));
    *T = tile_at(k_in / heads_per_queue);
  }

  // the tile at queue position i: through the plan's order, or (ring) stored in queue order
  __device__ const lb_plan_tile* tile_at(int64_t i) const {
    if constexpr (RING) return &tiles[i];
    else return &tiles[__builtin_amdgcn_readfirstlane(order[i])];
  }

  // The last workgroup out rewinds the queues (every pop has happened before it counts itself).
  __device__ void close(const BwdArgs& a, uint64_t t_start, int items, int64_t pairs, int blocks) {
    if (threadIdx.x != 0) return;
    lb_worker_record rec;
    rec.hw_id = hw_id_reg();
    rec.xcc_id = xcc_id_reg();
    rec.t_start = t_start;
    rec.t_end = device_clock();
    rec.pairs = pairs;
    rec.items = items;
    rec.blocks = blocks;
    reinterpret_cast<lb_worker_record*>(a.ws + kWorkersOffset)[blockIdx.x] = rec;
    if (blockIdx.x == 0) hdr->n_workers = gridDim.x;
    __threadfence();
    if (atomicAdd(&hdr->done, 1) == (int)gridDim.x - 1) {
      for (int q = 0; q < kXcds; ++q) atomicExch(&hdr->queue_head[q], 0);
      atomicExch(&hdr->done, 0);
    }
  }
};

using Queues = QueuesT<false>;

struct Span {
  int start, len, pos0;
};

__device__ __forceinline__ Span span_of(const lb_plan_tile* T, int s) {
  return Span{__builtin_amdgcn_readfirstlane(T->k_start[s]), __builtin_amdgcn_readfirstlane(T->k_len[s]),
              __builtin_amdgcn_readfirstlane(T->k_pos0[s])};
}

// Writes one wave's 32 rows, staged row-major in LDS (`rows` rows valid, from lane-owned
// rows), to a [row][heads][D] tensor: bf16, fp32, or fp32 added to what is there.
template <int D, int MODE>  // MODE 0: bf16 store, 1: fp32 store, 2: fp32 accumulate
__device__ __forceinline__ void store_rows(const char* stage, int stride, char* dst_row0, int64_t dst_row_step,
                                           int rows, int lane) {
  constexpr int kRowBytes = D * (MODE == 0 ? 2 : 4);
  constexpr int kChunks = kRowBytes / 16;
  constexpr int kRowsPerStep = 64 / kChunks;
  const int r0 = lane / kChunks, ch = lane % kChunks;
#pragma unroll
  for (int j = 0; j < 32 / kRowsPerStep; ++j) {
    const int r = r0 + j * kRowsPerStep;
    if (r < rows) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * stride + ch * 16);
      u32x4* dst = reinterpret_cast<u32x4*>(dst_row0 + r * dst_row_step + ch * 16);
      if constexpr (MODE == 2) {
        const f32x4 old = __builtin_bit_cast(f32x4, *dst);
        *dst = __builtin_bit_cast(u32x4, old + __builtin_bit_cast(f32x4, x));
      } else {
        *dst = x;
      }
    }
  }
}

// Stages a 32-column accumulator set (acc[db] holds X^T[d = db*32 + ...][col = lane % 32])
// as 32 rows of D values, row-major: row = lane % 32, scaled by `mul`.
template <int D, bool F32>
__device__ __forceinline__ void stage_rows(char* stage, int stride, const f32x16* acc, float mul, int lane,
                                           int r_lo = 0, int n_rows = 32) {
  const int l32 = lane & 31, hh = lane >> 5;
  if (l32 < r_lo || l32 >= r_lo + n_rows) return;
  char* rowp = stage + (l32 - r_lo) * stride;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d0 = db * 32 + r * 8 + hh * 4;
      if constexpr (F32) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[db][r * 4 + e] * mul;
        *reinterpret_cast<f32x4*>(rowp + d0 * 4) = o;
      } else {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[db][r * 4 + e] * mul);
        *reinterpret_cast<bf16x4*>(rowp + d0 * 2) = o;
      }
    }
}

// ------------------------------------------------------------------------------------
// D = rowsum(dO * O)
// ------------------------------------------------------------------------------------
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void rowdot_kernel(const void* out, const void* dout, int n_rows, int heads,
                                                     float* dvec) {
  constexpr int kLanes = D / 8;  // lanes per (row, head): 8 elements each
  const int64_t rec = ((int64_t)blockIdx.x * 256 + threadIdx.x) / kLanes;
  const int part = threadIdx.x % kLanes;
  const bool ok = rec < (int64_t)n_rows * heads;
  float s = 0.f;
  if (ok) {
    const int64_t base = rec * D + part * 8;
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(dout) + base);
    if constexpr (OUT_F32) {
      const f32x4 o0 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(out) + base);
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(out) + base + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s += o0[e] * (float)g[e] + o1[e] * (float)g[e + 4];
    } else {
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(out) + base);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)o[e] * (float)g[e];
    }
  }
#pragma unroll
  for (int off = kLanes / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (ok && part == 0) {
    const int64_t row = rec / heads, h = rec % heads;
    dvec[h * n_rows + row] = s;
  }
}

// Walks a tile's spans in blocks of `step` rows, `reps` passes per block (heads).  The
// cursor carries the spans still ahead of it, read once per item into uniform registers and
// shifted forward, never indexed: the loop that walks them then issues no memory read (a
// vector or scratch read there would wait for every copy in flight).
struct SpanCursor {
  int off, rep, left;  // left: spans after the current one
  Span sp, n1, n2, n3;
  bool down;           // each span's blocks from its last to its first
  __device__ __forceinline__ static int last_block(int len, int step) { return (len - 1) / step * step; }
  __device__ __forceinline__ void start(const lb_plan_tile* T, int step, bool descending = false) {
    static_assert(LB_MAX_SPANS == 4, "the cursor holds up to four spans");
    rep = 0;
    down = descending;
    left = __builtin_amdgcn_readfirstlane(T->n_spans) - 1;
    sp = span_of(T, 0);
    n1 = span_of(T, 1);
    n2 = span_of(T, 2);
    n3 = span_of(T, 3);
    off = down ? last_block(sp.len, step) : 0;
  }
  // blocks of `step` rows over all spans (the span count is at least 1)
  __device__ __forceinline__ int blocks(int step) const {
    return (sp.len + step - 1) / step + (left >= 1 ? (n1.len + step - 1) / step : 0) +
           (left >= 2 ? (n2.len + step - 1) / step : 0) + (left >= 3 ? (n3.len + step - 1) / step : 0);
  }
  __device__ __forceinline__ void next(int step, int reps) {
    if (++rep == reps) {
      rep = 0;
      off += down ? -step : step;
      if ((down ? off < 0 : off >= sp.len) && left > 0) {
        --left;
        sp = n1;
        n1 = n2;
        n2 = n3;
        off = down ? last_block(sp.len, step) : 0;
      }
    }
  }
};

// ------------------------------------------------------------------------------------
// dQ: query-stationary
// ------------------------------------------------------------------------------------
constexpr int kDqStages = 4;  // LDS ring depth of the dQ kernel

template <int D>
struct DqLds {
  static constexpr int tileBytes = BN * D * 2;  // 64 keys of K or V
  static constexpr int stage = 2 * tileBytes;   // K, V
  static constexpr int copiesPerStage = 2 * TileCopier<D, BN>::kCopies;
  static constexpr int ring = kDqStages * stage;
  static_assert(BN == 64, "a stage is one 64-row tile per tensor");
};

// FUSED: the workspace is a fused ring (lb_plan_ring_fused over the steps' query-tile plans):
// each tile holds the key spans of every step, span s's step in bits 4s..4s+3 of `reserved`,
// whose keys and values r gives; one item adds the tile rows' whole dq over every step.
template <int D, int HPW, bool OUT_F32, bool FUSED = false>
__global__ __launch_bounds__(kDqThreads, 1) void bwd_dq_kernel(BwdArgs a, RingBwdSteps r) {
  using L = DqLds<D>;
  __shared__ __attribute__((aligned(1024))) char smem[L::ring];
  __shared__ int s_item;
  const uint32_t ring_lds = lds_addr(smem);  // the ring's LDS address, for the copies

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int G = a.group;
  const int HG = G / HPW, RG = kDqWaves / HG;
  const int rg = wave % RG, hgi = wave / RG;
  const int wr0 = rg * 32;
  const float c = a.scale_log2;
  const int64_t row_bytes = (int64_t)a.kv_heads * D * 2;
  const __bf16* Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* dO = reinterpret_cast<const __bf16*>(a.dout);

  QueuesT<FUSED> qs;
  qs.open(a, 0, &r, FUSED);
  uint64_t t_start = tid == 0 ? device_clock() : 0;
  int my_items = 0, my_blocks = 0;
  int64_t my_pairs = 0;

  if (tid == 0) s_item = qs.pop();
  lds_barrier();
  int item = __builtin_amdgcn_readfirstlane(s_item);
  while (item >= 0) {
    const lb_plan_tile* T;
    int g;
    qs.decode(item, &T, &g);
    const int q_start = __builtin_amdgcn_readfirstlane(T->q_start);
    const int q_len = __builtin_amdgcn_readfirstlane(T->q_len);
    const int q_pos0 = __builtin_amdgcn_readfirstlane(T->q_pos0);
    // FUSED: the step of every span, and the tile's span count (the copy cursor's span index
    // is n_spans - 1 - left)
    const uint32_t span_steps = FUSED ? __builtin_amdgcn_readfirstlane((uint32_t)T->reserved) : 0u;
    const int n_spans_t = __builtin_amdgcn_readfirstlane(T->n_spans);
    SpanCursor cur;  // the key block being computed
    cur.start(T, BN);
    const int n_blocks = cur.blocks(BN);
    if (tid == 0) {
      my_blocks += n_blocks;
      ++my_items;
      my_pairs += T->cost * G;
    }
    const int my_row = wr0 + l32;
    const bool row_real = my_row < q_len;
    const bool wave_rows = wr0 < q_len;
    const int wave_last = min(wr0 + 32, q_len) - 1;
    const int qpos = q_pos0 + my_row;
    const int64_t grow = (int64_t)q_start + my_row;

    bf16x8 qreg[HPW][D / 16], doreg[HPW][D / 16];
    float lse2[HPW], dvv[HPW];
    f32x16 acc[HPW][D / 32];
#pragma unroll
    for (int e = 0; e < HPW; ++e) {
      const int head = g * G + hgi * HPW + e;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 xq = u32x4{0, 0, 0, 0}, xd = u32x4{0, 0, 0, 0};
        if (row_real) {
          const int64_t off = (grow * a.heads + head) * D + kk * 16 + hh * 8;
          xq = *reinterpret_cast<const u32x4*>(Q + off);
          xd = *reinterpret_cast<const u32x4*>(dO + off);
        }
        qreg[e][kk] = __builtin_bit_cast(bf16x8, xq);
        doreg[e][kk] = __builtin_bit_cast(bf16x8, xd);
      }
      const float l = row_real ? a.lse[(int64_t)head * a.n_q + grow] : -__builtin_inff();
      // a row that sees nothing (or no row): every weight is 0
      lse2[e] = l == -__builtin_inff() ? __builtin_inff() : l * 1.4426950408889634f;
      dvv[e] = row_real ? a.dvec[(int64_t)head * a.n_q + grow] : 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[e][db] = f32x16{};
    }

    // the rows' operands are in registers before any copy goes out: a wait for them inside the
    // loop would also wait for every copy in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    SpanCursor nxt = cur;  // the next key block to copy in
    auto issue = [&](int slot) {
      const int k0 = __builtin_amdgcn_readfirstlane(nxt.sp.start + nxt.off);
      const int valid = __builtin_amdgcn_readfirstlane(max(0, min(nxt.sp.len - nxt.off, BN)));
      const uint32_t lds = ring_lds + slot * L::stage;
      const void* kx = a.k;
      const void* vx = a.v;
      if constexpr (FUSED) {  // the keys and values of the step the span belongs to
        const int idx = min(max(n_spans_t - 1 - nxt.left, 0), LB_MAX_SPANS - 1);
        const int st = min((int)(span_steps >> (4 * idx)) & 15, r.n_steps - 1);
        kx = r.k[st];
        vx = r.v[st];
      }
      TileCopier<D, BN>::issue_now(kx, row_bytes, k0, valid, g, lds, wave, lane);
      TileCopier<D, BN>::issue_now(vx, row_bytes, k0, valid, g, lds + L::tileBytes, wave, lane);
      nxt.next(BN, 1);
    };
#pragma unroll
    for (int k = 0; k < kDqStages - 1; ++k)
      if (k < n_blocks) issue(k);
    for (int it = 0; it < n_blocks; ++it) {
      // as in the dK/dV kernel: this wave's copies of block `it` have landed, the barrier
      // publishes every wave's and frees the slot the next copy goes to
      static_assert(kDqStages == 4, "wait_stage covers two younger stages");
      wait_stage(min(kDqStages - 2, n_blocks - 1 - it), L::copiesPerStage);
      lds_barrier();
      if (it + kDqStages - 1 < n_blocks) issue((it + kDqStages - 1) % kDqStages);
      const char* ks = smem + (it % kDqStages) * L::stage;
      const char* vs = ks + L::tileBytes;
      const Span cs = cur.sp;
      const int key0 = cur.off;
      const bool live = wave_rows && cs.pos0 + key0 <= q_pos0 + wave_last;
      if (live) {
        // visible iff the key's position <= the row's, and the key lies in its span
        const bool full = key0 + BN <= cs.len && cs.pos0 + key0 + BN - 1 <= q_pos0 + wr0;
        const int lim = min(cs.len, qpos - cs.pos0 + 1) - key0 - hh * 4;
        // head by head: the operand fragments are read again for the second head rather
        // than holding two heads' S^T and dP^T at once
#pragma unroll
        for (int e = 0; e < HPW; ++e) {
          // keeps the compiler from merging the two heads' identical LDS reads into one
          // set of 48 live fragments
          if (e > 0) asm volatile("" ::: "memory");
          f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              const bf16x8 kf = row_frag<D>(ks, kb * 32 + l32, 2 * kk + hh);
              const bf16x8 vf = row_frag<D>(vs, kb * 32 + l32, 2 * kk + hh);
              s[kb] = mfma(kf, qreg[e][kk], s[kb]);
              dp[kb] = mfma(vf, doreg[e][kk], dp[kb]);
            }
          bf16x8 dsf[4];
          auto make_ds = [&](auto masked) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                  const int i = cc * 8 + j;
                  const bool vis = !decltype(masked)::value || (kb * 32 + (i / 4) * 8 + (i % 4) < lim);
                  const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, -lse2[e])) : 0.f;
                  dsf[kb * 2 + cc][j] = (__bf16)(p * (dp[kb][i] - dvv[e]));
                }
          };
          if (full) make_ds(Masked<false>{});
          else make_ds(Masked<true>{});
#pragma unroll
          for (int ks16 = 0; ks16 < 4; ++ks16)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
              acc[e][db] = mfma(tr_frag<D>(ks, ks16 * 16, db, lane), dsf[ks16], acc[e][db]);
        }
      }
      cur.next(BN, 1);
    }

    // epilogue: dQ = scale * dQ^T, staged row-major per wave, head by head (fp32 rows in two
    // passes of 16 where 32 rows of every wave do not fit in the ring)
    lds_barrier();
    constexpr int kEpiStride = OUT_F32 ? D * 4 + 16 : D * 2 + 16;
    constexpr int kPassRows = kDqWaves * 32 * kEpiStride <= L::ring ? 32 : 16;
    static_assert(kDqWaves * kPassRows * kEpiStride <= L::ring, "epilogue staging must fit in the ring");
    char* ebuf = smem + wave * kPassRows * kEpiStride;
    const int64_t row_step = (int64_t)a.heads * D * (OUT_F32 ? 4 : 2);
#pragma unroll
    for (int e = 0; e < HPW; ++e) {
      const int head = g * G + hgi * HPW + e;
#pragma unroll
      for (int r_lo = 0; r_lo < 32; r_lo += kPassRows) {
        __builtin_amdgcn_wave_barrier();
        stage_rows<D, OUT_F32>(ebuf, kEpiStride, acc[e], a.scale, lane, r_lo, kPassRows);
        __builtin_amdgcn_wave_barrier();
        char* dst = reinterpret_cast<char*>(a.dq) +
                    (((int64_t)q_start + wr0 + r_lo) * a.heads + head) * D * (OUT_F32 ? 4 : 2);
        const int rows = max(0, min(kPassRows, q_len - wr0 - r_lo));
        store_rows<D, OUT_F32 ? 2 : 0>(ebuf, kEpiStride, dst, row_step, rows, lane);
      }
    }
    lds_barrier();
    if (tid == 0) s_item = qs.pop();
    lds_barrier();
    item = __builtin_amdgcn_readfirstlane(s_item);
  }
  qs.close(a, t_start, my_items, my_pairs, my_blocks);
}

// ------------------------------------------------------------------------------------
// dK, dV: key-stationary, producer and consumer waves
// ------------------------------------------------------------------------------------
// A tile of 128 keys; 8 waves, two per SIMD, in pairs that own 32 keys each.  The producer of
// a pair (waves 0-3) holds its keys' K and V and, per block of 32 query rows of one head,
// computes S = Q K^T and dP = dO V^T, then P = exp(S - lse) and dS = P (dP - D), which it
// leaves in LDS as bf16 in the layout of an MFMA B operand.  The consumer (waves 4-7) takes
// them one block later and accumulates both dV^T = sum dO^T P and dK^T = sum Q^T dS.  Each
// block costs both waves of a SIMD the same 16 MFMAs.  The heads of the kv group add into the
// same accumulators, so no reduction over heads or waves follows.
//
// Query rows stream in stages of 32 rows of one head through a ring of kKvStages LDS slots:
// at stage i the producers read slot i, the consumers slot i - 1, and the copy of stage i + 2
// goes into slot i + 2 (the consumers left it at stage i - 1).  A stage holds the 32 Q rows and
// 32 dO rows (swizzled row tiles) and the rows' raw lse and D; P and dS go through two slots
// of their own.
constexpr int kKvWaves = 8;
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kKeyGroups = kBwdKeyGroups;  // 32 keys each: 128 keys per tile
constexpr int kKvStages = 4;   // LDS ring depth

template <int D>
struct KvLds {
  static constexpr int tileBytes = kQB * D * 2;              // 32 rows of one tensor
  static constexpr int stage = 2 * tileBytes + 2 * kQB * 4;  // Q, dO; raw lse, D
  static constexpr int ring = kKvStages * stage;
  static constexpr int xBytes = 2048;                    // one B operand block: 64 lanes x 2 x 16 bytes
  static constexpr int xSlot = kKeyGroups * 2 * xBytes;  // P and dS of every key group
  static constexpr int total = ring + 2 * xSlot;
  static constexpr int epiStride = D * 4 + 16;
  static_assert(kKeyGroups * 32 * epiStride <= total, "epilogue staging must fit in the kernel's LDS");
};

// A wave's share of a stage's copies: waves 0-3 copy the Q tile, waves 4-7 the dO tile (a
// 32-row tile is 8 or 4 pieces of 1 KB, one or two per wave of the half), and every wave 8 rows
// of lse (even waves) or D (odd waves).  Every wave issues the same count, kPerStage, so that
// the vmcnt waits are uniform.  Rows past the span's end read as zeros, and so do their lse and
// D.  The lane offsets are computed once.
template <int D>
struct StageCopier {
  using L = KvLds<D>;
  static constexpr int kChunks = D / 8, kRowsPerCopy = 1024 / (D * 2), kCopies = D / 64;
  static constexpr int kPerStage = kCopies + 1;
  static_assert(kCopies * 4 * 1024 == L::tileBytes, "four waves per tile");
  int voff[kCopies], voff_v;  // lane byte offsets from the tile's (the vector's) first row
  uint32_t loff, loff_v;      // the wave's pieces within a stage (wave-uniform)
  int t, w;                   // the wave's tensor (0: Q, 1: dO); its index

  __device__ __forceinline__ void init(int64_t row_step, int wave, int lane) {
    w = __builtin_amdgcn_readfirstlane(wave);
    t = w >> 2;
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int row = ((w & 3) * kCopies + j) * kRowsPerCopy + lane / kChunks;
      const int chunk = (lane % kChunks) ^ swz<D>(row);  // lane writes slot lane % kChunks of its row
      voff[j] = row * (int)row_step + chunk * 16;
    }
    loff = __builtin_amdgcn_readfirstlane(t * L::tileBytes + (w & 3) * kCopies * 1024);
    voff_v = ((w >> 1) * 8 + lane) * 4;
    loff_v = __builtin_amdgcn_readfirstlane(2 * L::tileBytes + (w & 1) * kQB * 4 + (w >> 1) * 32);
  }
  // the stage at cursor `c` (32 rows of head g * G + c.rep from row sp.start + off) to LDS
  // address `lds`
  __device__ __forceinline__ void issue(const BwdArgs& a, uint32_t lds, const SpanCursor& c, int g, int lane) const {
    const int head = __builtin_amdgcn_readfirstlane(g * a.group + c.rep);
    const int r0 = __builtin_amdgcn_readfirstlane(c.sp.start + c.off);
    const int valid = __builtin_amdgcn_readfirstlane(max(0, min(c.sp.len - c.off, kQB)));
    const int64_t row_step = (int64_t)a.heads * D * 2;
    const char* base = reinterpret_cast<const char*>(t == 0 ? a.q : a.dout) + (int64_t)r0 * row_step +
                       (int64_t)head * D * 2;
    const i32x4 rs = buffer_rsrc(base, valid * (int)row_step);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) copy16_to_lds(rs, lds + loff + j * 1024, voff[j]);
    const float* vec = (w & 1) ? a.dvec : a.lse;
    const i32x4 rv = buffer_rsrc(vec + (int64_t)head * a.n_q + r0, valid * 4);
    if (lane < 8) copy4_to_lds(rv, lds + loff_v, voff_v);
  }
};

// RING: a ring workspace of several steps' key tiles; a tile's step selects the keys, values
// and gradient outputs of that step in r (one launch for every step of a rank's ring).
// Requires a finite lse for every row of a span (a row that sees a key of the tile has one).
template <int D, bool OUT_F32, bool RING>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkv_kernel(BwdArgs a, RingBwdSteps r) {
  using L = KvLds<D>;
  __shared__ __attribute__((aligned(1024))) char smem[L::total];
  __shared__ int s_item;
  char* xbuf = smem + L::ring;
  const uint32_t ring_lds = lds_addr(smem);  // the ring's LDS address, for the copies
  StageCopier<D> copier;
  copier.init((int64_t)a.heads * D * 2, threadIdx.x >> 6, threadIdx.x & 63);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int G = a.group;
  const int kg = wave % kKeyGroups;
  const bool producer = wave < kKeyGroups;
  const float c = a.scale_log2;
  constexpr float kNegLog2e = -1.4426950408889634f;
  const __bf16* Kb = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* Vb = reinterpret_cast<const __bf16*>(a.v);
  // a ring tile's step, kept inside the launch's step table
  auto step_of = [&](const lb_plan_tile* T) -> int {
    return min(max(__builtin_amdgcn_readfirstlane(T->reserved), 0), r.n_steps - 1);
  };

  QueuesT<RING> qs;
  qs.open(a, 1, &r);
  uint64_t t_start = tid == 0 ? device_clock() : 0;
  int my_items = 0, my_blocks = 0;
  int64_t my_pairs = 0;

  // key tiles no query row sees: zero gradients, a grid-stride pass before the queues
  for (int e = blockIdx.x; e < qs.n_empty; e += gridDim.x) {
    const lb_plan_tile* T = qs.tile_at(qs.n_tiles - qs.n_empty + e);
    const int k_start = T->q_start, k_len = T->q_len;
    const int per_row = a.kv_heads * D;
    void* dk_e = a.dk;
    void* dv_e = a.dv;
    if constexpr (RING) {
      const int st = step_of(T);
      dk_e = r.dk[st];
      dv_e = r.dv[st];
    }
    for (int idx = tid; idx < k_len * per_row; idx += kKvThreads) {
      const int64_t o = (int64_t)k_start * per_row + idx;
      if constexpr (OUT_F32) {
        reinterpret_cast<float*>(dk_e)[o] = 0.f;
        reinterpret_cast<float*>(dv_e)[o] = 0.f;
      } else {
        reinterpret_cast<__bf16*>(dk_e)[o] = (__bf16)0.f;
        reinterpret_cast<__bf16*>(dv_e)[o] = (__bf16)0.f;
      }
    }
  }

  if (tid == 0) s_item = qs.pop();
  lds_barrier();
  int item = __builtin_amdgcn_readfirstlane(s_item);
  while (item >= 0) {
    const lb_plan_tile* T;
    int g;
    qs.decode(item, &T, &g);
    const int k_start = __builtin_amdgcn_readfirstlane(T->q_start);  // the tile's keys
    const int k_len = __builtin_amdgcn_readfirstlane(T->q_len);
    const int k_pos0 = __builtin_amdgcn_readfirstlane(T->q_pos0);
    // Each span's query rows stream from its last block to its first: the key tiles of one
    // document all end at the document's last row, so tiles that run at the same time read
    // the same rows at about the same time and share them in L2.
    SpanCursor cur;  // the block the producers compute
    cur.start(T, kQB, true);
    if (tid == 0) {
      ++my_items;
      my_pairs += T->cost * G;
    }
    const __bf16* K = Kb;
    const __bf16* V = Vb;
    int step = 0;
    if constexpr (RING) {
      step = step_of(T);
      K = reinterpret_cast<const __bf16*>(r.k[step]);
      V = reinterpret_cast<const __bf16*>(r.v[step]);
    }
    const int my_key = kg * 32 + l32;
    const bool key_real = my_key < k_len;
    const int kpos = k_pos0 + my_key;
    const int pair_key_first = k_pos0 + kg * 32;                       // position of the pair's first key
    const int pair_key_last = k_pos0 + min(kg * 32 + 32, k_len) - 1;  // and of its last
    const bool pair_keys = kg * 32 < k_len;
    // A block of `rows` rows from position pos0 has a visible pair with the pair's keys iff its
    // last row is at or after their first key.
    auto live_block = [&](int rows, int pos0) { return pair_keys && rows > 0 && pos0 + rows - 1 >= pair_key_first; };

    const int n_stages = cur.blocks(kQB) * G;
    if (tid == 0) my_blocks += cur.blocks(64) * G;  // recorded in the plan's 64-row query blocks
    SpanCursor nxt = cur;  // the next stage to copy in
    // Both roles run the same barrier sequence: one per stage, then two in the epilogue.  The
    // roles are separate code paths, so that the producer's K and V and the consumer's
    // accumulators can share registers.
    // Copies go out only once the wave's own loads are in registers: a wait for those inside
    // the loop would also wait for every copy in flight.
    auto start_copies = [&]() {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (k < n_stages) {
          copier.issue(a, ring_lds + k * L::stage, nxt, g, lane);
          nxt.next(kQB, G);
        }
    };
    // Stage `it`: this wave's copies of it have landed once at most those of stage it + 1 are
    // in flight; the barrier publishes every wave's copies and the P, dS of block it - 1, and
    // frees slot it + 2 (stage it - 2) and the P, dS slot of block it - 2.
    auto stage_sync = [&](int it) {
      if (it + 1 < n_stages) wait_stage(1, StageCopier<D>::kPerStage);
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      if (it + 2 < n_stages) {
        copier.issue(a, ring_lds + ((it + 2) % kKvStages) * L::stage, nxt, g, lane);
        nxt.next(kQB, G);
      }
    };

    if (producer) {
      // stationary operands: the pair's keys' K and V as B fragments
      bf16x8 kfr[D / 16], vfr[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 xk = u32x4{0, 0, 0, 0}, xv = u32x4{0, 0, 0, 0};
        if (key_real) {
          const int64_t off = ((int64_t)(k_start + my_key) * a.kv_heads + g) * D + kk * 16 + hh * 8;
          xk = *reinterpret_cast<const u32x4*>(K + off);
          xv = *reinterpret_cast<const u32x4*>(V + off);
        }
        kfr[kk] = __builtin_bit_cast(bf16x8, xk);
        vfr[kk] = __builtin_bit_cast(bf16x8, xv);
      }
      start_copies();
      for (int it = 0; it <= n_stages; ++it) {
        stage_sync(it);
        const int rows = min(kQB, cur.sp.len - cur.off);
        const int row_pos0 = cur.sp.pos0 + cur.off;  // position of the block's first row
        if (it < n_stages && live_block(rows, row_pos0)) {
          const char* h = smem + (it % kKvStages) * L::stage;
          const char* qtile = h;
          const char* dotile = h + L::tileBytes;
          const float* lsep = reinterpret_cast<const float*>(h + 2 * L::tileBytes);
          const float* dvp = lsep + kQB;
          char* xw = xbuf + (it & 1) * L::xSlot + kg * 2 * L::xBytes;
          // rows of this lane's accumulators: 8 i4 + 4 hh + j of the block; keys: column l32
          // all operand reads first (their latency overlaps), then the S and dP chains interleaved
          bf16x8 fq[D / 16], fd[D / 16];
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            fq[kk] = row_frag<D>(qtile, l32, 2 * kk + hh);
            fd[kk] = row_frag<D>(dotile, l32, 2 * kk + hh);
          }
          __builtin_amdgcn_sched_barrier(0);
          f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            s = mfma(fq[kk], kfr[kk], s);
            dp = mfma(fd[kk], vfr[kk], dp);
          }
          bf16x8 pf[2], dsf[2];
          // the lane's key sees row 8 i4 + 4 hh + j iff that row's position is at least the
          // key's: compared as kdist <= 8 i4 + j, against constants
          const int kdist = kpos - row_pos0 - 4 * hh;
          auto make = [&](auto masked) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const f32x4 lv = *reinterpret_cast<const f32x4*>(lsep + 8 * i4 + 4 * hh);
              const f32x4 dv = *reinterpret_cast<const f32x4*>(dvp + 8 * i4 + 4 * hh);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int i = i4 * 4 + j;
                const bool vis = !decltype(masked)::value || kdist <= 8 * i4 + j;
                const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, lv[j] * kNegLog2e)) : 0.f;
                pf[i / 8][i % 8] = (__bf16)p;
                dsf[i / 8][i % 8] = (__bf16)(p * (dp[i] - dv[j]));
              }
            }
          };
          if (row_pos0 >= pair_key_last) make(Masked<false>{});
          else make(Masked<true>{});
          *reinterpret_cast<bf16x8*>(xw + lane * 16) = pf[0];
          *reinterpret_cast<bf16x8*>(xw + 1024 + lane * 16) = pf[1];
          *reinterpret_cast<bf16x8*>(xw + L::xBytes + lane * 16) = dsf[0];
          *reinterpret_cast<bf16x8*>(xw + L::xBytes + 1024 + lane * 16) = dsf[1];
        }
        if (it < n_stages) cur.next(kQB, G);
      }
      lds_barrier();  // the consumers stage dK
      lds_barrier();  // the consumers stage dV
    } else {
      f32x16 acck[D / 32], accv[D / 32];  // dK^T and dV^T of the pair's keys
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acck[db] = accv[db] = f32x16{};
      start_copies();
      for (int it = 0; it <= n_stages; ++it) {
        stage_sync(it);
        if (it == 0) continue;
        // block it - 1, at cur
        const int rows = min(kQB, cur.sp.len - cur.off);
        const int row_pos0 = cur.sp.pos0 + cur.off;
        if (live_block(rows, row_pos0)) {
          const char* h = smem + ((it - 1) % kKvStages) * L::stage;
          const char* qtile = h;
          const char* dotile = h + L::tileBytes;
          const char* xr = xbuf + ((it - 1) & 1) * L::xSlot + kg * 2 * L::xBytes;
          const bf16x8 p0 = *reinterpret_cast<const bf16x8*>(xr + lane * 16);
          const bf16x8 p1 = *reinterpret_cast<const bf16x8*>(xr + 1024 + lane * 16);
          const bf16x8 d0 = *reinterpret_cast<const bf16x8*>(xr + L::xBytes + lane * 16);
          const bf16x8 d1 = *reinterpret_cast<const bf16x8*>(xr + L::xBytes + 1024 + lane * 16);
          // every operand read goes out before the first product: the reads' latency then
          // overlaps, and each product waits only for its own operands
          bf16x8 fv[2][D / 32], fk[2][D / 32];
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            fv[0][db] = tr_frag<D>(dotile, 0, db, lane);
            fv[1][db] = tr_frag<D>(dotile, 16, db, lane);
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            fk[0][db] = tr_frag<D>(qtile, 0, db, lane);
            fk[1][db] = tr_frag<D>(qtile, 16, db, lane);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            accv[db] = mfma(fv[0][db], p0, accv[db]);
            accv[db] = mfma(fv[1][db], p1, accv[db]);
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            acck[db] = mfma(fk[0][db], d0, acck[db]);
            acck[db] = mfma(fk[1][db], d1, acck[db]);
          }
        }
        cur.next(kQB, G);
      }
      // epilogue: dK = scale * dK^T, then dV = dV^T, staged in LDS
      const int rows = max(0, min(32, k_len - kg * 32));
      const int64_t elt = OUT_F32 ? 4 : 2;
      const int64_t row_step = (int64_t)a.kv_heads * D * elt;
      const int64_t first = (((int64_t)k_start + kg * 32) * a.kv_heads + g) * D * elt;
      char* ebuf = smem + kg * 32 * L::epiStride;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        lds_barrier();
        void* grad = t == 0 ? a.dk : a.dv;
        if constexpr (RING) grad = t == 0 ? r.dk[step] : r.dv[step];
        stage_rows<D, OUT_F32>(ebuf, L::epiStride, t == 0 ? acck : accv, t == 0 ? a.scale : 1.0f, lane);
        __builtin_amdgcn_wave_barrier();
        store_rows<D, OUT_F32 ? 1 : 0>(ebuf, L::epiStride, reinterpret_cast<char*>(grad) + first, row_step, rows,
                                       lane);
      }
    }
    lds_barrier();
    if (tid == 0) s_item = qs.pop();
    lds_barrier();
    item = __builtin_amdgcn_readfirstlane(s_item);
  }
  qs.close(a, t_start, my_items, my_pairs, my_blocks);
}

}  // namespace

hipError_t launch_bwd_rowdot(const void* out, bool out_f32, const void* dout, int n_rows, int heads, int d,
                             float* dvec, hipStream_t s) {
  const int64_t lanes = (int64_t)n_rows * heads * (d / 8);
  const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
  if (d == 128) {
    if (out_f32) hipLaunchKernelGGL((rowdot_kernel<128, true>), grid, block, 0, s, out, dout, n_rows, heads, dvec);
    else hipLaunchKernelGGL((rowdot_kernel<128, false>), grid, block, 0, s, out, dout, n_rows, heads, dvec);
  } else {
    if (out_f32) hipLaunchKernelGGL((rowdot_kernel<64, true>), grid, block, 0, s, out, dout, n_rows, heads, dvec);
    else hipLaunchKernelGGL((rowdot_kernel<64, false>), grid, block, 0, s, out, dout, n_rows, heads, dvec);
  }
  return hipGetLastError();
}

template <int D, bool F32>
static void dq_launch(const BwdArgs& a, int workers, hipStream_t s) {
  const RingBwdSteps none{};
  hipLaunchKernelGGL((bwd_dq_kernel<D, 1, F32>), dim3(workers), dim3(kDqThreads), 0, s, a, none);
}

hipError_t launch_bwd_dq_fused(const BwdArgs& a, const RingBwdSteps& r, int d, int n_workers, hipStream_t s) {
  if (d == 128) hipLaunchKernelGGL((bwd_dq_kernel<128, 1, true, true>), dim3(n_workers), dim3(kDqThreads), 0, s, a, r);
  else hipLaunchKernelGGL((bwd_dq_kernel<64, 1, true, true>), dim3(n_workers), dim3(kDqThreads), 0, s, a, r);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, bool out_f32, int n_workers, hipStream_t s) {
  if (d == 128) {
    if (out_f32) dq_launch<128, true>(a, n_workers, s); else dq_launch<128, false>(a, n_workers, s);
  } else {
    if (out_f32) dq_launch<64, true>(a, n_workers, s); else dq_launch<64, false>(a, n_workers, s);
  }
  return hipGetLastError();
}

template <int D, bool F32>
static void dkv_launch(const BwdArgs& a, int workers, hipStream_t s) {
  const RingBwdSteps none{};
  hipLaunchKernelGGL((bwd_dkv_kernel<D, F32, false>), dim3(workers), dim3(kKvThreads), 0, s, a, none);
}

hipError_t launch_bwd_dkv(const BwdArgs& a, int d, bool out_f32, int n_workers, hipStream_t s) {
  if (d == 128) {
    if (out_f32) dkv_launch<128, true>(a, n_workers, s); else dkv_launch<128, false>(a, n_workers, s);
  } else {
    if (out_f32) dkv_launch<64, true>(a, n_workers, s); else dkv_launch<64, false>(a, n_workers, s);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkv_ring(const BwdArgs& a, const RingBwdSteps& r, int d, int n_workers, hipStream_t s) {
  if (d == 128)
    hipLaunchKernelGGL((bwd_dkv_kernel<128, true, true>), dim3(n_workers), dim3(kKvThreads), 0, s, a, r);
  else
    hipLaunchKernelGGL((bwd_dkv_kernel<64, true, true>), dim3(n_workers), dim3(kKvThreads), 0, s, a, r);
  return hipGetLastError();
}

}  // namespace lb
