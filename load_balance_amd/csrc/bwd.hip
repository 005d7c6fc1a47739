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
//     dQ^T += K^T dS^T with K^T from LDS.
//   * dK/dV, key-stationary, over key tiles whose spans are the query rows that see
//     them (the transposed plan): per block of 32 query rows and head,
//     S = Q K^T and dP = dO V^T (Q and dO rows from LDS, K and V held in
//     registers), then dV^T += dO^T P and dK^T += Q^T dS.  The heads of a kv group
//     add into the same accumulators, so no reduction over heads follows.
// The dK/dV kernel's waves run alone on their SIMDs (4 waves per workgroup) and may
// hold 512 registers: two stationary operand sets and two accumulators stay live.
// Transposed operands (K^T, Q^T, dO^T) are written to LDS by the loader with the
// index permutation that lets the other MFMA operand come straight from an
// accumulator (the forward's V^T layout).
#include "lbattn_internal.h"

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
constexpr int kQB = 64;      // query rows per stage of the dK/dV kernel (two MFMA blocks of 32)
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ int vt_pos(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

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

// Two bf16 values of one 16-byte chunk pair, interleaved for a transposed row: the
// words for elements 2m and 2m + 1 of two consecutive source rows.
__device__ __forceinline__ uint32_t pair_lo(uint32_t x0, uint32_t x1) { return (x0 & 0xFFFFu) | (x1 << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t x0, uint32_t x1) { return (x0 >> 16) | (x1 & 0xFFFF0000u); }

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

  __device__ void open(const BwdArgs& a, int transposed, const RingBwdSteps* r = nullptr) {
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
      bad = bad || r->n_steps < 1 || r->n_steps > kMaxPlanSteps || hdr->ring_steps != r->n_steps;
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

// ------------------------------------------------------------------------------------
// dQ: query-stationary
// ------------------------------------------------------------------------------------
template <int D>
struct DqLds {
  static constexpr int kStride = D * 2 + 16;  // K or V row
  static constexpr int tStride = BN * 2 + 16; // K^T row (one d, the block's keys)
  static constexpr int rowsBytes = BN * kStride;
  static constexpr int tBytes = D * tStride;
  static constexpr int stage = 2 * rowsBytes + tBytes;  // K rows, V rows, K^T
  static constexpr int kUnits = (BN / 2) * (D / 8);     // (key pair, 16-byte chunk) units of K
  static constexpr int kPerThread = (kUnits + kDqThreads - 1) / kDqThreads;  // the last one partial at d = 64
  static constexpr int vChunks = BN * (D / 8);
  static constexpr int vPerThread = vChunks / kDqThreads;
  static constexpr int epiStride = D * 4 + 16;
};

template <int D>
struct DqLoader {
  using L = DqLds<D>;
  u32x4 kr[L::kPerThread][2];
  u32x4 vr[L::vPerThread];

  __device__ __forceinline__ void load(const char* K, const char* V, int k0, int valid, int row_bytes, int g,
                                       int tid) {
    const int64_t base = (int64_t)k0 * row_bytes + (int64_t)g * D * 2;
    const int nbytes = min(valid, BN) * row_bytes;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), (short)0, nbytes,
                                                                        kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), (short)0, nbytes,
                                                                        kBufferFlags);
#pragma unroll
    for (int e = 0; e < L::kPerThread; ++e) {
      const int u = tid + e * kDqThreads, p = u % (BN / 2), ch = u / (BN / 2);
      if (L::kUnits % kDqThreads == 0 || u < L::kUnits) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
          kr[e][x] = __builtin_amdgcn_raw_buffer_load_b128(rk, (2 * p + x) * row_bytes + ch * 16, 0, 0);
      }
    }
#pragma unroll
    for (int e = 0; e < L::vPerThread; ++e) {
      const int c = tid + e * kDqThreads, row = c / (D / 8), ch = c % (D / 8);
      vr[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, row * row_bytes + ch * 16, 0, 0);
    }
  }

  __device__ __forceinline__ void store(char* stage, int tid) {
    char* ks = stage;
    char* vs = stage + L::rowsBytes;
    char* kt = stage + 2 * L::rowsBytes;
#pragma unroll
    for (int e = 0; e < L::kPerThread; ++e) {
      const int u = tid + e * kDqThreads, p = u % (BN / 2), ch = u / (BN / 2);
      if (!(L::kUnits % kDqThreads == 0 || u < L::kUnits)) continue;
#pragma unroll
      for (int x = 0; x < 2; ++x) *reinterpret_cast<u32x4*>(ks + (2 * p + x) * L::kStride + ch * 16) = kr[e][x];
      const int col = vt_pos(2 * p) * 2;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        *reinterpret_cast<uint32_t*>(kt + (ch * 8 + 2 * m) * L::tStride + col) = pair_lo(kr[e][0][m], kr[e][1][m]);
        *reinterpret_cast<uint32_t*>(kt + (ch * 8 + 2 * m + 1) * L::tStride + col) = pair_hi(kr[e][0][m], kr[e][1][m]);
      }
    }
#pragma unroll
    for (int e = 0; e < L::vPerThread; ++e) {
      const int c = tid + e * kDqThreads, row = c / (D / 8), ch = c % (D / 8);
      *reinterpret_cast<u32x4*>(vs + row * L::kStride + ch * 16) = vr[e];
    }
  }
};

template <int D, int HPW, bool OUT_F32>
__global__ __launch_bounds__(kDqThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using L = DqLds<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::stage];
  __shared__ int s_item;
  static_assert(kDqWaves * 32 * (D * 2 + 16) <= 2 * L::stage, "epilogue staging must fit in the ring");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int G = a.group;
  const int HG = G / HPW, RG = kDqWaves / HG;
  const int rg = wave % RG, hgi = wave / RG;
  const int wr0 = rg * 32;
  const float c = a.scale_log2;
  const int row_bytes = a.kv_heads * D * 2;
  const char* Kb = reinterpret_cast<const char*>(a.k);
  const char* Vb = reinterpret_cast<const char*>(a.v);
  const __bf16* Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* dO = reinterpret_cast<const __bf16*>(a.dout);

  Queues qs;
  qs.open(a, 0);
  uint64_t t_start = tid == 0 ? device_clock() : 0;
  int my_items = 0, my_blocks = 0;
  int64_t my_pairs = 0;
  DqLoader<D> ld;

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
    const int n_spans = __builtin_amdgcn_readfirstlane(T->n_spans);
    int n_blocks = 0;
    for (int s = 0; s < n_spans; ++s) n_blocks += (span_of(T, s).len + BN - 1) / BN;
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

    int cur_s = 0;
    Span cur = span_of(T, 0);
    int key0 = 0;
    if (n_blocks > 0) {
      ld.load(Kb, Vb, cur.start, cur.len, row_bytes, g, tid);
      ld.store(smem, tid);
    }
    for (int it = 0; it < n_blocks; ++it) {
      lds_barrier();
      // the block after this one
      Span nxt = cur;
      int nkey0 = key0 + BN, nx_s = cur_s;
      if (nkey0 >= cur.len) {
        ++nx_s;
        nkey0 = 0;
        if (nx_s < n_spans) nxt = span_of(T, nx_s);
      }
      const bool has_next = it + 1 < n_blocks;
      if (has_next) ld.load(Kb, Vb, nxt.start + nkey0, nxt.len - nkey0, row_bytes, g, tid);
      const char* stage = smem + (it & 1) * L::stage;
      const char* ks = stage;
      const char* vs = stage + L::rowsBytes;
      const char* kt = stage + 2 * L::rowsBytes;
      const bool live = wave_rows && cur.pos0 + key0 <= q_pos0 + wave_last;
      if (live) {
        // visible iff the key's position <= the row's, and the key lies in its span
        const bool full = key0 + BN <= cur.len && cur.pos0 + key0 + BN - 1 <= q_pos0 + wr0;
        const int lim = min(cur.len, qpos - cur.pos0 + 1) - key0 - hh * 4;
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
              const bf16x8 kf =
                  *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + l32) * L::kStride + (kk * 16 + hh * 8) * 2);
              const bf16x8 vf =
                  *reinterpret_cast<const bf16x8*>(vs + (kb * 32 + l32) * L::kStride + (kk * 16 + hh * 8) * 2);
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
            for (int db = 0; db < D / 32; ++db) {
              const bf16x8 tf =
                  *reinterpret_cast<const bf16x8*>(kt + (db * 32 + l32) * L::tStride + (ks16 * 16 + hh * 8) * 2);
              acc[e][db] = mfma(tf, dsf[ks16], acc[e][db]);
            }
        }
      }
      if (has_next) ld.store(smem + ((it + 1) & 1) * L::stage, tid);
      cur = nxt;
      cur_s = nx_s;
      key0 = nkey0;
    }

    // epilogue: dQ = scale * dQ^T, staged row-major per wave, head by head (fp32 rows in two
    // passes of 16 where 32 rows of every wave do not fit in the ring)
    lds_barrier();
    constexpr int kEpiStride = OUT_F32 ? D * 4 + 16 : D * 2 + 16;
    constexpr int kPassRows = kDqWaves * 32 * kEpiStride <= 2 * L::stage ? 32 : 16;
    static_assert(kDqWaves * kPassRows * kEpiStride <= 2 * L::stage, "epilogue staging must fit in the ring");
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
        char* dst = reinterpret_cast<char*>(a.dq) + (((int64_t)q_start + wr0 + r_lo) * a.heads + head) * D * (OUT_F32 ? 4 : 2);
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
// dK, dV: key-stationary, waves split by role
// ------------------------------------------------------------------------------------
// A tile of 128 keys; 8 waves, two per SIMD.  Waves 0-3 (one per 32 keys) hold K and V and
// accumulate dK^T = sum Q^T dS (S and dP recomputed); waves 4-7 hold K and accumulate
// dV^T = sum dO^T P (S recomputed).  Each runs every head of the kv group, so no reduction
// over heads or waves follows, and each fits in 256 registers.  Query rows stream in
// stages of 64 (two MFMA blocks of 32), one head per stage, through a ring of kKvStages
// LDS stages that both roles read, kKvStages - 1 of them in flight.
//
// A stage holds the 64 Q rows and 64 dO rows row-major, copied from global memory straight
// into LDS by the buffer loads' LDS mode (no registers, no stores), and the rows' raw lse
// and D.  The row-major tiles serve both products: S = Q K^T and dP = dO V^T read row
// fragments, and dK^T += Q^T dS and dV^T += dO^T P read the transposed fragments with
// gfx950's LDS transpose load (ds_read_b64_tr_b16), which hands each lane one d column of
// 4 rows.  Each row's 16-byte chunks are stored XOR-permuted by the row (swz) so that both
// kinds of read hit 64 distinct banks per pass.
constexpr int kKvWaves = 8;
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kKeyGroups = 4;  // 32 keys each: 128 keys per tile
constexpr int kKvStages = 4;   // LDS ring depth

template <int D>
struct KvLds {
  static constexpr int rowBytes = D * 2;              // one Q or dO row, unpadded
  static constexpr int chunks = D / 8;                 // 16-byte chunks per row
  static constexpr int tileBytes = kQB * rowBytes;     // 64 rows of one tensor
  static constexpr int stage = 2 * tileBytes + 2 * kQB * 4;  // Q, dO; raw lse, D
  static constexpr int rowsPerDma = 1024 / rowBytes;   // rows one wave's 16-byte-per-lane copy covers
  static constexpr int dmaPerTensor = kQB / rowsPerDma / kKvWaves;  // copies per wave per tensor
  static constexpr int dmaPerStage = 2 * dmaPerTensor + 1;          // + one for lse or D
  static constexpr int ring = kKvStages * stage;
  static constexpr int epiStride = D * 4 + 16;
  static constexpr int epiRows = kKvWaves * 32 * epiStride <= ring ? 32 : 16;  // rows per epilogue pass
  static_assert(kQB % (rowsPerDma * kKvWaves) == 0, "the copies must divide evenly over the waves");
  static_assert(kKvWaves * epiRows * epiStride <= ring, "epilogue staging must fit in the ring");
};

// The chunk permutation of row r (r mod 16 decides it).  Row reads: 16 lanes read one
// logical chunk of 16 consecutive rows, which land on 16 distinct chunk slots (d = 128) or on
// 8 slots in each bank half (d = 64: two rows per 256 bytes).  Transpose reads: 32 lanes read
// four logical chunks (a 64-byte run) of 4 consecutive rows, which land on 4 disjoint runs.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }  // s_waitcnt vmcnt(n) only

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + nbytes): reads past the end return zeros.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p), __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFF)),
               __builtin_amdgcn_readfirstlane(nbytes), kBufferFlags};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (int)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// Copies global -> LDS without registers: lane i's 16 (or 4) bytes at voffset land at
// lds + 16 i (or 4 i).  Written as inline assembly on purpose: the compiler, seeing the
// builtin's LDS write, would wait for every copy in flight before each LDS read of the loop;
// the kernel waits for its copies itself (vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, uint32_t lds, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(i32x4 rsrc, uint32_t lds, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// The stages of one key tile: for each span, each 64 rows, each head of the group.  The
// cursor carries the spans still ahead of it, read once per item into uniform registers and
// shifted forward, never indexed: the loop that walks them then issues no memory read (a
// vector or scratch read there would wait for every copy in flight).
struct StageCursor {
  int off, hs, left;  // left: spans after the current one
  Span sp, n1, n2, n3;
  __device__ __forceinline__ void start(const lb_plan_tile* T) {
    static_assert(LB_MAX_SPANS == 4, "the cursor holds up to four spans");
    off = hs = 0;
    left = __builtin_amdgcn_readfirstlane(T->n_spans) - 1;
    sp = span_of(T, 0);
    n1 = span_of(T, 1);
    n2 = span_of(T, 2);
    n3 = span_of(T, 3);
  }
  __device__ __forceinline__ void next(int G) {
    if (++hs == G) {
      hs = 0;
      off += kQB;
      if (off >= sp.len && left > 0) {
        off = 0;
        --left;
        sp = n1;
        n1 = n2;
        n2 = n3;
      }
    }
  }
};

// Copies stage `c` (64 rows of one head from row sp.start + off) into `buf`: every wave issues
// dmaPerStage copies (the same count in every wave, so that vmcnt waits are uniform).  Rows
// past the span's end read as zeros (the buffer range ends there), and so do their lse and D.
template <int D>
__device__ __forceinline__ void issue_stage(const BwdArgs& a, char* buf, const StageCursor& c, int g, int wave,
                                            int lane) {
  using L = KvLds<D>;
  const int head = __builtin_amdgcn_readfirstlane(g * a.group + c.hs);
  const int r0 = __builtin_amdgcn_readfirstlane(c.sp.start + c.off);
  const int valid = __builtin_amdgcn_readfirstlane(max(0, min(c.sp.len - c.off, kQB)));
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const int row_step = a.heads * D * 2;
  const uint32_t lds = lds_addr(buf);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const char* base = reinterpret_cast<const char*>(t == 0 ? a.q : a.dout) + (int64_t)r0 * row_step +
                       (int64_t)head * D * 2;
    const i32x4 rs = buffer_rsrc(base, valid * row_step);
#pragma unroll
    for (int j = 0; j < L::dmaPerTensor; ++j) {
      const int blk = w * L::dmaPerTensor + j;  // the 1 KB piece of the tile
      const int row = blk * L::rowsPerDma + lane / L::chunks;
      const int chunk = (lane % L::chunks) ^ swz<D>(row);  // lane writes slot lane % chunks of its row
      copy16_to_lds(rs, lds + t * L::tileBytes + blk * 1024, row * row_step + chunk * 16);
    }
  }
  // lse (even waves) or D (odd waves), 16 rows per wave, 4 bytes per lane
  const float* vec = (w & 1) ? a.dvec : a.lse;
  const int q16 = w >> 1;
  const i32x4 rv = buffer_rsrc(vec + (int64_t)head * a.n_q + r0, valid * 4);
  if (lane < 16) copy4_to_lds(rv, lds + 2 * L::tileBytes + (w & 1) * kQB * 4 + q16 * 64, (q16 * 16 + lane) * 4);
}

// RING: a ring workspace of several steps' key tiles; a tile's step selects the keys, values
// and gradient outputs of that step in r (one launch for every step of a rank's ring).
// Requires a finite lse for every row of a span (a row that sees a key of the tile has one).
template <int D, bool OUT_F32, bool RING>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkv_kernel(BwdArgs a, RingBwdSteps r) {
  using L = KvLds<D>;
  __shared__ __attribute__((aligned(1024))) char smem[L::ring];
  __shared__ int s_item;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int G = a.group;
  const int kg = wave % kKeyGroups;
  const bool dk_role = wave < kKeyGroups;  // else the dV role
  const float c = a.scale_log2;
  constexpr float kNegLog2e = -1.4426950408889634f;
  const __bf16* Kb = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* Vb = reinterpret_cast<const __bf16*>(a.v);
  // a ring tile's step, kept inside the launch's step table
  auto step_of = [&](const lb_plan_tile* T) -> int {
    return min(max(__builtin_amdgcn_readfirstlane(T->reserved), 0), r.n_steps - 1);
  };

  // Per-lane LDS offsets inside a tile.  Row fragment kk (A operand of S or dP): row l32 of
  // the 32-row block, logical chunk 2 kk + hh.  Transposed fragment (A operand of dK^T or
  // dV^T), half q of column block db: the lane's 16-lane group supplies 4 rows x 16 columns,
  // this lane's address being row 8 q + 4 hh + (lane % 16) / 4 of the 16-row block and
  // columns 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4) .. + 3.
  const int sw_r = swz<D>(l32);
  const int lg = lane & 15, gq = (lane >> 4) & 1;
  auto row_frag = [&](const char* tile, int sb, int kk) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(tile + (sb * 32 + l32) * L::rowBytes + (((2 * kk + hh) ^ sw_r) << 4));
  };
  auto tr_frag = [&](const char* tile, int sb, int ks, int db) -> bf16x8 {
    bf16x4 h[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = sb * 32 + ks * 16 + 8 * q + 4 * hh + (lg >> 2);
      const int col = db * 32 + 16 * gq + 4 * (lg & 3);
      const char* p = tile + row * L::rowBytes + (((col >> 3) ^ swz<D>(row)) << 4) + (col & 7) * 2;
      h[q] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
    }
    return __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
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
    StageCursor cur;  // the stage being computed
    cur.start(T);
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
    const int wave_key_last = k_pos0 + min(kg * 32 + 32, k_len) - 1;  // position of the wave's last key
    const bool wave_keys = kg * 32 < k_len;

    // stationary operands: the wave's 32 keys as B fragments (K for both roles, V for dK)
    bf16x8 kfr[D / 16], vfr[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 xk = u32x4{0, 0, 0, 0}, xv = u32x4{0, 0, 0, 0};
      if (key_real) {
        const int64_t off = ((int64_t)(k_start + my_key) * a.kv_heads + g) * D + kk * 16 + hh * 8;
        xk = *reinterpret_cast<const u32x4*>(K + off);
        if (dk_role) xv = *reinterpret_cast<const u32x4*>(V + off);
      }
      kfr[kk] = __builtin_bit_cast(bf16x8, xk);
      vfr[kk] = __builtin_bit_cast(bf16x8, xv);
    }
    f32x16 acc[D / 32];  // dK^T or dV^T of the wave's keys
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    const int n_stages =
        ((cur.sp.len + kQB - 1) / kQB + (cur.left >= 1 ? (cur.n1.len + kQB - 1) / kQB : 0) +
         (cur.left >= 2 ? (cur.n2.len + kQB - 1) / kQB : 0) + (cur.left >= 3 ? (cur.n3.len + kQB - 1) / kQB : 0)) *
        G;
    if (tid == 0) my_blocks += n_stages;
    StageCursor nxt = cur;  // the next stage to copy in
#pragma unroll
    for (int k = 0; k < kKvStages - 1; ++k)
      if (k < n_stages) {
        issue_stage<D>(a, smem + k * L::stage, nxt, g, wave, lane);
        nxt.next(G);
      }
    for (int it = 0; it < n_stages; ++it) {
      // this wave's copies of stage `it` have landed once at most the younger stages' are
      // outstanding; the barrier then makes every wave's copies visible, and tells that every
      // wave is done with the slot the next copy goes to
      const int younger = min(kKvStages - 2, n_stages - 1 - it);
      if (younger >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * L::dmaPerStage));
      else if (younger == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(L::dmaPerStage));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      static_assert(kKvStages == 4, "the waits above cover two younger stages");
      lds_barrier();
      if (it + kKvStages - 1 < n_stages) {
        issue_stage<D>(a, smem + ((it + kKvStages - 1) % kKvStages) * L::stage, nxt, g, wave, lane);
        nxt.next(G);
      }

      const char* h = smem + (it % kKvStages) * L::stage;
      const char* qtile = h;
      const char* dotile = h + L::tileBytes;
      const float* lsep = reinterpret_cast<const float*>(h + 2 * L::tileBytes);
      const float* dvp = lsep + kQB;
      const int rows_valid = min(kQB, cur.sp.len - cur.off);
      const int row_pos0 = cur.sp.pos0 + cur.off;  // position of the stage's first row
#pragma unroll
      for (int sb = 0; sb < kQB / 32; ++sb) {
        const int sb_rows = min(32, rows_valid - sb * 32);
        const int sb_pos0 = row_pos0 + sb * 32;
        // any visible pair: the sub-block's last row at or after the wave's first key
        const bool live = wave_keys && sb_rows > 0 && sb_pos0 + sb_rows - 1 >= k_pos0 + kg * 32;
        if (!live) continue;
        // rows of this lane's accumulator: 8i + 4hh + j of the sub-block; keys: column l32
        const bool full = sb_pos0 >= wave_key_last;
        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) s = mfma(row_frag(qtile, sb, kk), kfr[kk], s);
        if (dk_role) {
          f32x16 dp = f32x16{};
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) dp = mfma(row_frag(dotile, sb, kk), vfr[kk], dp);
          bf16x8 dsf[2];
          auto make_ds = [&](auto masked) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const f32x4 lv = *reinterpret_cast<const f32x4*>(lsep + sb * 32 + 8 * i4 + 4 * hh);
              const f32x4 dv = *reinterpret_cast<const f32x4*>(dvp + sb * 32 + 8 * i4 + 4 * hh);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int i = i4 * 4 + j;
                const bool vis = !decltype(masked)::value || kpos <= sb_pos0 + 8 * i4 + 4 * hh + j;
                const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, lv[j] * kNegLog2e)) : 0.f;
                dsf[i / 8][i % 8] = (__bf16)(p * (dp[i] - dv[j]));
              }
            }
          };
          if (full) make_ds(Masked<false>{});
          else make_ds(Masked<true>{});
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[db] = mfma(tr_frag(qtile, sb, ks, db), dsf[ks], acc[db]);
        } else {
          bf16x8 pf[2];
          auto make_p = [&](auto masked) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const f32x4 lv = *reinterpret_cast<const f32x4*>(lsep + sb * 32 + 8 * i4 + 4 * hh);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int i = i4 * 4 + j;
                const bool vis = !decltype(masked)::value || kpos <= sb_pos0 + 8 * i4 + 4 * hh + j;
                pf[i / 8][i % 8] =
                    (__bf16)(vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, lv[j] * kNegLog2e)) : 0.f);
              }
            }
          };
          if (full) make_p(Masked<false>{});
          else make_p(Masked<true>{});
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[db] = mfma(tr_frag(dotile, sb, ks, db), pf[ks], acc[db]);
        }
      }
      cur.next(G);
    }

    // epilogue: dK = scale * dK^T, dV = dV^T, each role its own tensor, staged in the ring
    lds_barrier();
    {
      char* ebuf = smem + wave * L::epiRows * L::epiStride;
      const int rows = max(0, min(32, k_len - kg * 32));
      const int64_t elt = OUT_F32 ? 4 : 2;
      const int64_t row_step = (int64_t)a.kv_heads * D * elt;
      const int64_t first = (((int64_t)k_start + kg * 32) * a.kv_heads + g) * D * elt;
      void* grad = dk_role ? a.dk : a.dv;
      if constexpr (RING) grad = dk_role ? r.dk[step] : r.dv[step];
#pragma unroll
      for (int r_lo = 0; r_lo < 32; r_lo += L::epiRows) {
        __builtin_amdgcn_wave_barrier();
        stage_rows<D, OUT_F32>(ebuf, L::epiStride, acc, dk_role ? a.scale : 1.0f, lane, r_lo, L::epiRows);
        __builtin_amdgcn_wave_barrier();
        store_rows<D, OUT_F32 ? 1 : 0>(ebuf, L::epiStride, reinterpret_cast<char*>(grad) + first + r_lo * row_step,
                                       row_step, max(0, min(L::epiRows, rows - r_lo)), lane);
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
  hipLaunchKernelGGL((bwd_dq_kernel<D, 1, F32>), dim3(workers), dim3(kDqThreads), 0, s, a);
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
