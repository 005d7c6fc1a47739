// In-place log-sum-exp merge of two partial attention results over disjoint key
// sets: the online-softmax rescale-and-sum that folds the blocks contributing
// to one output ("03 · 长文负载均衡", section 3.2, DCP; "长序列训练与上下文并行",
// Ring Attention: each ring step's local result is merged into the running one).
//
// HBM-bound elementwise work: d/4 lanes own one (row, head), each moving 16
// bytes of out_a and out_b.  Rows whose lse_b is -inf (no visible key in the
// second partial) read nothing beyond their two lse values.
#include "lbattn_internal.h"

namespace lb {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lanes_per_row = a.d / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rh = gid / lanes_per_row;  // row * heads + head
  const int part = (int)(gid % lanes_per_row);
  if (rh >= (int64_t)a.n_rows * a.heads) return;
  const int64_t row = rh / a.heads;
  const int head = (int)(rh % a.heads);
  const int64_t li = (int64_t)head * a.n_rows + row;
  const float lb = a.lse_b[li];
  if (lb == -__builtin_inff()) return;
  const float la = a.lse_a[li];
  f32x4* oa = reinterpret_cast<f32x4*>(a.out_a + rh * a.d) + part;
  const f32x4 ob = reinterpret_cast<const f32x4*>(a.out_b + rh * a.d)[part];
  if (la == -__builtin_inff()) {
    *oa = ob;
    if (part == 0) a.lse_a[li] = lb;
    return;
  }
  const float m = fmaxf(la, lb);
  const float wa = __expf(la - m), wb = __expf(lb - m);
  const float inv = 1.0f / (wa + wb);
  const f32x4 x = *oa;
  *oa = (x * wa + ob * wb) * inv;
  if (part == 0) a.lse_a[li] = m + __logf(wa + wb);
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t threads = (int64_t)a.n_rows * a.heads * (a.d / 4);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lb
