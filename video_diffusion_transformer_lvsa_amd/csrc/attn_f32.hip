// Block-sparse / dense softmax attention forward for fp32 inputs (VALU).
//
// Same operation and key-list semantics as the bf16 matrix-core kernel
// ("LVSA: Training-Free Sparse Attention for Long Video Diffusion", §1 and
// §2 complexity; Draft Attention article, block-sparse execution), computed
// in fp32 throughout: one thread per query row, K/V tiles of 32 rows staged
// in LDS and read as broadcasts, exact-order online softmax per tile. This
// path serves small fp32 problems; it is not tuned for throughput.
#include "internal.h"

namespace lvsa {
namespace {

constexpr int kRows = kBM_F32;  // query rows per workgroup (one per thread)
constexpr int kBN = 32;         // keys per tile

__device__ __forceinline__ int block_lim_f(const AttnArgs& a, int b) {
  if (b < 0 || b >= a.nkb) return 0;
  int lim = a.block_k;
  if (a.block_valid) {
    int bv = a.block_valid[b];
    lim = bv < 0 ? 0 : (bv < lim ? bv : lim);
  }
  int rem = a.n - b * a.block_k;
  return rem < lim ? rem : lim;
}

__device__ __forceinline__ int key_phys(const AttnArgs& a, const int32_t* list, int cnt, int L, int vj) {
  if (vj >= L) return -1;
  if (a.dense) return vj;
  int slot = vj / a.block_k;
  int off = vj - slot * a.block_k;
  if (slot >= cnt) return -1;
  int blk = list[slot];
  if (blk < 0 || blk >= a.nkb) return -1;
  return off < block_lim_f(a, blk) ? blk * a.block_k + off : -1;
}

template <int D>
__global__ __launch_bounds__(kRows) void bsa_fwd_f32_kernel(AttnArgs a) {
  __shared__ float Kt[kBN][D];
  __shared__ float Vt[kBN][D];
  __shared__ int kok[kBN];

  const int tid = threadIdx.x;
  const int logical = blockIdx.x;
  const int qt = logical % a.tiles_per_qb;
  const int rest = logical / a.tiles_per_qb;
  const int qb = rest % a.nqb;
  const int h = rest / a.nqb;

  const int blk_lo = qb * a.block_q;
  const int blk_end = min(blk_lo + a.block_q, a.n);
  int qlim = a.block_q;
  if (a.block_valid) {
    int bv = a.block_valid[qb];
    qlim = bv < 0 ? 0 : (bv < qlim ? bv : qlim);
  }
  const int qend = min(blk_lo + qlim, blk_end);
  const int row_lo = blk_lo + qt * kRows;
  const int qrow = row_lo + tid;
  const bool q_in_blk = qrow < blk_end;
  const bool q_valid = qrow < qend;

  const size_t head_off = (size_t)h * (size_t)a.n * D;
  const float* Qh = (const float*)a.q + head_off;
  const float* Kh = (const float*)a.k + head_off;
  const float* Vh = (const float*)a.v + head_off;
  float* Oh = a.o + head_off;

  const int32_t* list = nullptr;
  int cnt = 0, L = a.n;
  if (!a.dense) {
    const int hm = a.mask_heads > 1 ? h : 0;
    const int base = hm * a.nqb + qb;
    cnt = a.kv_cnt[base];
    cnt = cnt < 0 ? 0 : (cnt > a.max_kv ? a.max_kv : cnt);
    list = a.kv_idx + (size_t)base * a.max_kv;
    L = cnt * a.block_k;
  }
  if (row_lo >= qend) L = 0;

  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = q_valid ? Qh[(size_t)qrow * D + c] : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int vt0 = 0; vt0 < L; vt0 += kBN) {
    __syncthreads();
    for (int e = tid; e < kBN * D; e += kRows) {
      const int r = e / D, c = e % D;
      const int p = key_phys(a, list, cnt, L, vt0 + r);
      Kt[r][c] = p >= 0 ? Kh[(size_t)p * D + c] : 0.f;
      Vt[r][c] = p >= 0 ? Vh[(size_t)p * D + c] : 0.f;
      if (c == 0) kok[r] = p >= 0;
    }
    __syncthreads();
    float s[kBN];
    float mx = -INFINITY;
    for (int j = 0; j < kBN; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = __builtin_fmaf(q[c], Kt[j][c], acc);
      s[j] = kok[j] ? acc * a.scale : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
    for (int j = 0; j < kBN; ++j) {
      const float p = expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, Vt[j][c], o[c]);
    }
    m = m_new;
  }

  if (q_in_blk) {
    const float inv = (q_valid && l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) Oh[(size_t)qrow * D + c] = o[c] * inv;
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, int d, hipStream_t s) {
  if (a.total_tiles == 0) return hipSuccess;
  dim3 grid(a.total_tiles), block(kRows);
  if (d == 128)
    hipLaunchKernelGGL((bsa_fwd_f32_kernel<128>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((bsa_fwd_f32_kernel<64>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace lvsa
