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
      const float la = a.lse_a[li];
      float wa = 0.0f, wb = 1.0f, lse = lb;
      if (la != -__builtin_inff()) {
        const float m = fmaxf(la, lb);
        const float ea = __expf(la - m), eb = __expf(lb - m);
        const float inv = 1.0f / (ea + eb);
        wa = ea * inv;
        wb = eb * inv;
        lse = m + __logf(ea + eb);
      }
      a.lse_a[li] = lse;
      const int slot = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      s_row[slot] = lane;
      s_wa[slot] = wa;
      s_wb[slot] = wb;
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
        if (ca[j] >= 0.0f) *dst[j] = ca[j] == 0.0f ? y[j] : x[j] * ca[j] + y[j] * cb[j];
    }
    __syncthreads();  // the table is read by every wave before the next group's wave 0 writes it
  }
}

}  // namespace

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
