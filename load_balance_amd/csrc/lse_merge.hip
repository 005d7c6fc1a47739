// In-place log-sum-exp merge of two partial attention results over disjoint key
// sets: the online-softmax rescale-and-sum that folds the blocks contributing
// to one output ("03 · 长文负载均衡", section 3.2, DCP; "长序列训练与上下文并行",
// Ring Attention: each ring step's local result is merged into the running one).
//
// HBM-bound elementwise work.  One workgroup of 4 waves takes 64 consecutive rows of
// one head: it reads their 64 lse_b values in one coalesced load, and only the rows with
// a visible key in the second partial (a ballot) move data.  Wave 0 computes the rows'
// weights into an LDS table (compacted by the ballot) and writes the merged lse; after
// one barrier the four waves share the rows' 16-byte pieces, each loading its whole
// share before storing any.  A ring step that touches few rows of the shard costs little
// more than reading lse_b, and a row group's data moves in one round trip per wave.
#include <algorithm>

#include "lbattn_internal.h"

namespace lb {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;
constexpr int kBatch = 8;  // units per lane loaded before any is stored

// One merge step of a row whose second partial has a visible key (lb != -inf): the weights
// of the two partials (wa = 0: the first is not read) and the merged lse.  The pairwise merge
// and the merge of several partials share this definition and merge_vec, so that merging
// several partials in one pass gives the bits of the pairwise merges in sequence.
struct MergeStep {
  float wa, wb, lse;
};
__device__ __forceinline__ MergeStep merge_step(float la, float lb) {
  MergeStep r{0.0f, 1.0f, lb};
  if (la != -__builtin_inff()) {
    const float m = fmaxf(la, lb);
    const float ea = __expf(la - m), eb = __expf(lb - m);
    const float inv = 1.0f / (ea + eb);
    r.wa = ea * inv;
    r.wb = eb * inv;
    r.lse = m + __logf(ea + eb);
  }
  return r;
}
__device__ __forceinline__ f32x4 merge_vec(f32x4 x, f32x4 y, float wa, float wb) {
  return wa == 0.0f ? y : x * wa + y * wb;
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  // the taken rows of the group, compacted, and their two weights
  __shared__ int s_row[64];
  __shared__ float s_wa[64], s_wb[64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t groups = ((int64_t)a.n_rows + 63) / 64;  // row groups per head
  const int64_t n_tasks = groups * a.heads;
  const int chunks = a.d / 4;  // 16-byte pieces of one (row, head) vector
  for (int64_t task = blockIdx.x; task < n_tasks; task += gridDim.x) {
    // task-major over heads: neighbouring workgroups read neighbouring lse entries
    const int head = (int)(task / groups);
    const int64_t row0 = (task % groups) * 64;
    const int64_t row = row0 + lane;
    const bool in = row < a.n_rows;
    const int64_t li = (int64_t)head * a.n_rows + row;
    const float lb = in ? a.lse_b[li] : -__builtin_inff();
    const bool take = lb != -__builtin_inff();
    const uint64_t mask = __ballot(take);  // the same in every wave: the same 64 rows
    if (mask == 0) continue;
    if (w == 0 && take) {
      // this lane's row: weights of the two partials (wa = 0: out_a is not read) and the merged lse
      const MergeStep st = merge_step(a.lse_a[li], lb);
      a.lse_a[li] = st.lse;
      const int slot = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      s_row[slot] = lane;
      s_wa[slot] = st.wa;
      s_wb[slot] = st.wb;
    }
    __syncthreads();
    // Units (taken row, 16-byte piece) are spread over the workgroup's lanes; each lane loads
    // a batch of units before it stores any (a store to out_a could alias a later load, so
    // the compiler would not hoist loads across it), keeping 2 x kBatch loads in flight.
    const int units = __popcll(mask) * chunks;
    for (int u0 = w * 64; u0 < units; u0 += kBatch * kMergeThreads) {
      f32x4 x[kBatch], y[kBatch];
      float ca[kBatch], cb[kBatch];
      f32x4* dst[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int u = u0 + j * kMergeThreads + lane;
        const bool ok = u < units;
        const int k = ok ? u / chunks : 0, c = ok ? u - k * chunks : 0;
        const int64_t rh = (row0 + s_row[k]) * a.heads + head;
        ca[j] = ok ? s_wa[k] : -1.0f;  // -1: no unit
        cb[j] = s_wb[k];
        dst[j] = reinterpret_cast<f32x4*>(a.out_a + rh * a.d) + c;
        // out_b is read once and never again: a non-temporal load keeps it from displacing
        // out_a's lines, which are written back right after
        y[j] = ok ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.out_b + rh * a.d) + c) : f32x4{};
        // out_a is not read where lse_a = -inf (ca = 0): the first partial never wrote that row
        x[j] = ca[j] > 0.0f ? *dst[j] : f32x4{};
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (ca[j] >= 0.0f) *dst[j] = merge_vec(x[j], y[j], ca[j], cb[j]);
    }
    __syncthreads();  // the table is read by every wave before the next group's wave 0 writes it
  }
}

// Several partials over disjoint key sets merged into the first, parts 1, 2, ... in order, in
// one pass: per row the weights of each merge step in turn (merge_step), then each 16-byte
// piece of the row read once from every partial that has a visible key there, folded in the
// same order (merge_vec), and written once.  The same bits as n - 1 pairwise merges in
// sequence; a row of the first partial is read only where the first step that touches the
// row keeps a share of it.  Same task layout as merge_kernel.
constexpr int kPartBatch = 4;  // units per lane in flight
__global__ __launch_bounds__(kMergeThreads) void merge_parts_kernel(MergePartsArgs a) {
  __shared__ int s_row[64];
  __shared__ uint32_t s_parts[64];  // bit i - 1: part i has a visible key in the row
  __shared__ float s_wa[kMaxPlanSteps][64], s_wb[kMaxPlanSteps][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t groups = ((int64_t)a.n_rows + 63) / 64;
  const int64_t n_tasks = groups * a.heads;
  const int chunks = a.d / 4;
  const int n = a.n_parts;
  for (int64_t task = blockIdx.x; task < n_tasks; task += gridDim.x) {
    const int head = (int)(task / groups);
    const int64_t row0 = (task % groups) * 64;
    const int64_t row = row0 + lane;
    const bool in = row < a.n_rows;
    const int64_t li = (int64_t)head * a.n_rows + row;
    uint32_t parts = 0;
    for (int i = 1; i < n; ++i)
      if (in && a.lse[i][li] != -__builtin_inff()) parts |= 1u << (i - 1);
    const uint64_t mask = __ballot(parts != 0);
    if (mask == 0) continue;
    if (w == 0 && parts != 0) {
      const int slot = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      float la = a.lse[0][li];
      for (int i = 1; i < n; ++i) {
        if (!(parts >> (i - 1) & 1)) continue;
        const MergeStep st = merge_step(la, a.lse[i][li]);
        s_wa[i - 1][slot] = st.wa;
        s_wb[i - 1][slot] = st.wb;
        la = st.lse;
      }
      a.lse[0][li] = la;
      s_row[slot] = lane;
      s_parts[slot] = parts;
    }
    __syncthreads();
    const int units = __popcll(mask) * chunks;
    for (int u0 = w * 64; u0 < units; u0 += kPartBatch * kMergeThreads) {
      f32x4 o[kPartBatch];
      uint32_t pj[kPartBatch];
      int kj[kPartBatch];
      int64_t off[kPartBatch];  // the piece's offset in floats, the same in every partial
#pragma unroll
      for (int j = 0; j < kPartBatch; ++j) {
        const int u = u0 + j * kMergeThreads + lane;
        const bool ok = u < units;
        const int k = ok ? u / chunks : 0, c = ok ? u - k * chunks : 0;
        kj[j] = k;
        pj[j] = ok ? s_parts[k] : 0u;
        off[j] = ((row0 + s_row[k]) * a.heads + head) * a.d + 4 * c;
        // the first partial's piece, where the first step that touches the row keeps a share of it
        const int first = pj[j] ? __builtin_ctz(pj[j]) : 0;
        o[j] = pj[j] && s_wa[first][k] > 0.0f ? *reinterpret_cast<const f32x4*>(a.out[0] + off[j]) : f32x4{};
      }
      for (int i = 1; i < n; ++i) {
        f32x4 y[kPartBatch];
#pragma unroll
        for (int j = 0; j < kPartBatch; ++j)
          y[j] = (pj[j] >> (i - 1) & 1)
                     ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.out[i] + off[j]))
                     : f32x4{};
#pragma unroll
        for (int j = 0; j < kPartBatch; ++j)
          if (pj[j] >> (i - 1) & 1) o[j] = merge_vec(o[j], y[j], s_wa[i - 1][kj[j]], s_wb[i - 1][kj[j]]);
      }
#pragma unroll
      for (int j = 0; j < kPartBatch; ++j)
        if (pj[j]) *reinterpret_cast<f32x4*>(a.out[0] + off[j]) = o[j];
    }
    __syncthreads();  // the tables are read by every wave before the next group's wave 0 writes them
  }
}

}  // namespace

hipError_t launch_lse_merge_parts(const MergePartsArgs& a, hipStream_t s) {
  const int64_t tasks = ((int64_t)a.n_rows + 63) / 64 * a.heads;
  const int64_t blocks = std::min<int64_t>(tasks, 16384);
  hipLaunchKernelGGL(merge_parts_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t tasks = ((int64_t)a.n_rows + 63) / 64 * a.heads;
  const int64_t blocks = std::min<int64_t>(tasks, 16384);
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void fill_f32_kernel(float* p, int64_t n, float value) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = value;
}
}  // namespace

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s) {
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

}  // namespace lb
