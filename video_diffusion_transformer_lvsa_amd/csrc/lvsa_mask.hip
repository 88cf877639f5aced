// LVSA frame mask: A(t) = G_s ∪ W(t).
//
// "LVSA: Training-Free Sparse Attention for Long Video Diffusion", §2
// "Methodology", core mechanism: rotating global anchors G_s (shifted by the
// denoising step s modulo T_per, every frame an anchor exactly once per
// T_per steps) plus a local window of W frames around the query frame that
// is widened where it overlaps anchors, so that |A(t)| stays at the budget C.
//
// Anchors are f ≡ s (mod T_per). The window is the nearest-first prefix of
// the frames ordered by (|f - t|, f); such a prefix is always one run
// [lo, hi] around t, grown one frame at a time (the earlier frame on a
// tie). One thread per query frame grows [lo, hi] from W frames until the
// union reaches min(C, T) frames, then writes the members in ascending order.
#include "internal.h"

namespace lvsa {
namespace {

__global__ void lvsa_mask_kernel(int T, int C, int window, int T_per, int step, int32_t* __restrict__ kv_idx,
                                 int32_t* __restrict__ kv_cnt, int cap) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int off = step % T_per;
  const int n_anchor = off < T ? (T - 1 - off) / T_per + 1 : 0;
  const int target = C < T ? C : T;
  const int base_k = window < T ? window : T;

  int lo = t, hi = t, k = 1;
  int count = n_anchor + ((t % T_per) == off ? 0 : 1);
  while (k < T && (k < base_k || count < target)) {
    // next frame in nearest-first order: lo-1 if it is not farther than hi+1
    int f;
    if (lo > 0 && (hi + 1 >= T || (t - (lo - 1)) <= (hi + 1 - t))) {
      f = --lo;
    } else {
      f = ++hi;
    }
    if ((f % T_per) != off) ++count;
    ++k;
  }

  int32_t* row = kv_idx + (size_t)t * cap;
  int nout = 0;
  for (int f = 0; f < T && nout < cap; ++f) {
    if ((f % T_per) == off || (f >= lo && f <= hi)) row[nout++] = f;
  }
  kv_cnt[t] = nout;
  for (int i = nout; i < cap; ++i) row[i] = -1;
}

}  // namespace

hipError_t launch_lvsa_mask(int T, int C, int window, int T_per, int step, int32_t* kv_idx, int32_t* kv_cnt,
                            int cap, hipStream_t s) {
  const int threads = 64;
  dim3 grid((T + threads - 1) / threads), block(threads);
  hipLaunchKernelGGL(lvsa_mask_kernel, grid, block, 0, s, T, C, window, T_per, step, kv_idx, kv_cnt, cap);
  return hipGetLastError();
}

}  // namespace lvsa
