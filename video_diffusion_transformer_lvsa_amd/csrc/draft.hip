// Draft Attention mask builder, token reorder and row gather.
//
// Source: "科学家提出视频扩散模型加速方法，在H100实现一倍以上端到端加速"
// (163.com article on Draft Attention): latent tokens are viewed as a
// [t, h, w] video; Q and K are average-pooled over pool_h x pool_w tiles
// into a low-resolution draft attention map; the draft map gives a sparse
// mask keeping the important connections; with pool_h * pool_w = block_size
// one map entry is one block of the block-sparse kernel; a reorder gathers
// each block's tokens into one contiguous run so the kernel reads them as a
// unit.
//
// The pooled means and the map use a fixed fp32 evaluation order (sequential
// sums from +0.0, one correctly rounded division, separate multiply and add)
// so that any two implementations of the same order agree bit for bit; this
// file is compiled without floating-point contraction.
#include "internal.h"

#pragma clang fp contract(off)

namespace lvsa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Reorder tables: perm (slot -> token or -1), inv_perm (token -> slot),
// block_valid (valid tokens per block, which fill its first slots).
// ---------------------------------------------------------------------------
__global__ void draft_perm_kernel(DraftGeom g, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                  int32_t* __restrict__ block_valid) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= g.n_pad) return;
  const int b = p / g.bs, slot = p - b * g.bs;
  const int t = b / (g.nbh * g.nbw);
  const int rb = b - t * (g.nbh * g.nbw);
  const int hb = rb / g.nbw, wb = rb - hb * g.nbw;
  const int vh = min(g.ph, g.H - hb * g.ph);
  const int vw = min(g.pw, g.W - wb * g.pw);
  const int nv = vh * vw;
  if (slot == 0) block_valid[b] = nv;
  if (slot < nv) {
    const int hi = slot / vw, wi = slot - hi * vw;
    const int tok = (t * g.H + hb * g.ph + hi) * g.W + wb * g.pw + wi;
    perm[p] = tok;
    inv_perm[tok] = p;
  } else {
    perm[p] = -1;
  }
}

// ---------------------------------------------------------------------------
// Pool (Q, K) + reorder (Q, K, V). One group of LPR lanes owns one
// (tensor, head, block); each lane owns CH consecutive channels and walks
// the block's slots in order, so every channel's sum is a sequential fold.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack(const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(v[i] << 16);
    x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void draft_pool_gather_kernel(DraftGeom g, int heads, int d,
                                                                const void* __restrict__ q,
                                                                const void* __restrict__ k,
                                                                const void* __restrict__ v, float* __restrict__ qbar,
                                                                float* __restrict__ kbar, float* __restrict__ kbarT,
                                                                void* __restrict__ q_perm, void* __restrict__ k_perm,
                                                                void* __restrict__ v_perm) {
  constexpr int CH = BF16 ? 8 : 4;  // channels per 16-byte chunk
  const int LPR = d / CH;           // lanes per row
  const int gpb = blockDim.x / LPR; // groups per workgroup
  const int which = blockIdx.y;     // 0 = Q, 1 = K, 2 = V
  const int grp = blockIdx.x * gpb + threadIdx.x / LPR;
  const int lane = threadIdx.x % LPR;
  if (grp >= heads * g.nb) return;
  const int h = grp / g.nb, b = grp - h * g.nb;

  const void* src = which == 0 ? q : (which == 1 ? k : v);
  void* dst = which == 0 ? q_perm : (which == 1 ? k_perm : v_perm);
  float* bar = which == 0 ? qbar : (which == 1 ? kbar : nullptr);

  const int t = b / (g.nbh * g.nbw);
  const int rb = b - t * (g.nbh * g.nbw);
  const int hb = rb / g.nbw, wb = rb - hb * g.nbw;
  const int vh = min(g.ph, g.H - hb * g.ph);
  const int vw = min(g.pw, g.W - wb * g.pw);
  const int nv = vh * vw;

  const u32x4* S = (const u32x4*)src + (size_t)h * g.n * LPR;
  u32x4* Dd = dst ? (u32x4*)dst + ((size_t)h * g.n_pad + (size_t)b * g.bs) * LPR : nullptr;

  float acc[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) acc[i] = 0.f;

  const int tok0 = (t * g.H + hb * g.ph) * g.W + wb * g.pw;
#pragma unroll 4
  for (int slot = 0; slot < nv; ++slot) {
    const int hi = slot / vw, wi = slot - hi * vw;
    const int tok = tok0 + hi * g.W + wi;
    const u32x4 x = S[(size_t)tok * LPR + lane];
    if (Dd) Dd[(size_t)slot * LPR + lane] = x;
    if (bar) {
      if (BF16) {
        float f[8];
        unpack(x, f);
#pragma unroll
        for (int i = 0; i < CH; ++i) acc[i] = __fadd_rn(acc[i], f[i]);
      } else {
#pragma unroll
        for (int i = 0; i < CH; ++i) acc[i] = __fadd_rn(acc[i], __uint_as_float(x[i]));
      }
    }
  }
  if (Dd) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int slot = nv; slot < g.bs; ++slot) Dd[(size_t)slot * LPR + lane] = z;
  }
  if (bar) {
    const float cnt = (float)nv;
    float* out = bar + ((size_t)h * g.nb + b) * d + lane * CH;
#pragma unroll
    for (int i = 0; i < CH; ++i) out[i] = __fdiv_rn(acc[i], cnt);
    if (which == 1) {  // K̄ᵀ [heads, d, nb] for coalesced reads by the map kernel
      float* outT = kbarT + (size_t)h * d * g.nb + (size_t)(lane * CH) * g.nb + b;
#pragma unroll
      for (int i = 0; i < CH; ++i) outT[(size_t)i * g.nb] = __fdiv_rn(acc[i], cnt);
    }
  }
}

// ---------------------------------------------------------------------------
// Draft map + top-k. One workgroup owns R query-block rows of one head.
//  1. s[r][j] = fold_c fl(acc + fl(q̄[r][c] * k̄[j][c])) for every KV block j;
//     thread t owns columns t, t + 256, ... and reads k̄ from its transposed
//     copy, so a wave's loads are contiguous, while the R query values of a
//     channel are one LDS broadcast. Each score is stored in LDS as an
//     order-preserving unsigned code (-0 folded into +0).
//  2. One wave per row selects the k largest codes, ties to the lower block
//     index: a 32-step bisection finds the k-th largest code tau; the row
//     keeps every code > tau and the first (k - #{> tau}) codes == tau in
//     index order, written out in ascending index order with ballots.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned int order_code(float s) {
  unsigned int bits = __float_as_uint(s);
  if (bits == 0x80000000u) bits = 0u;
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((unsigned int)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((unsigned int)mask, 0u));
}

template <int R>
__global__ __launch_bounds__(256) void draft_select_kernel(const float* __restrict__ qbar,
                                                           const float* __restrict__ kbarT, int heads, int nb, int d,
                                                           int topk, int32_t* __restrict__ kv_idx,
                                                           int32_t* __restrict__ kv_cnt) {
  extern __shared__ unsigned int codes[];  // [R][nb64]
  __shared__ float qsT[128 * R];           // [d][R]; d <= 128 (checked on the host)

  const int tid = threadIdx.x;
  const int nb64 = (nb + 63) & ~63;
  const int rows_per_head = (nb + R - 1) / R;
  const int h = blockIdx.x / rows_per_head;
  const int i0 = (blockIdx.x - h * rows_per_head) * R;
  const int nr = min(R, nb - i0);

  for (int e = tid; e < R * d; e += blockDim.x) {
    const int c = e / R, r = e - c * R;
    qsT[e] = r < nr ? qbar[((size_t)h * nb + i0 + r) * d + c] : 0.f;
  }
  __syncthreads();

  const float* kh = kbarT + (size_t)h * d * nb;
  const int ngroups = (nb + 255) / 256;
  for (int m0 = 0; m0 < ngroups; m0 += 4) {
    float acc[4][R];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[m][r] = 0.f;
#pragma unroll 4
    for (int c = 0; c < d; ++c) {
      float qv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) qv[r] = qsT[c * R + r];
      const float* kc = kh + (size_t)c * nb;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int j = tid + 256 * (m0 + m);
        const float kv = j < nb ? kc[j] : 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = __fadd_rn(acc[m][r], __fmul_rn(qv[r], kv));
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int j = tid + 256 * (m0 + m);
      if (j < nb64) {
#pragma unroll
        for (int r = 0; r < R; ++r) codes[r * nb64 + j] = j < nb ? order_code(acc[m][r]) : 0u;
      }
    }
  }
  __syncthreads();

  const int w = tid >> 6, lane = tid & 63;
  const int nch = nb64 >> 6;
  for (int r = w; r < nr; r += (int)(blockDim.x >> 6)) {
    const unsigned int* row = codes + r * nb64;
    unsigned int tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned int cand = tau | (1u << bit);
      int cnt = 0;
      for (int m = 0; m < nch; ++m) {
        const int j = 64 * m + lane;
        cnt += __popcll(__ballot(j < nb && row[j] >= cand));
      }
      if (cnt >= topk) tau = cand;
    }
    int greater = 0;
    for (int m = 0; m < nch; ++m) {
      const int j = 64 * m + lane;
      greater += __popcll(__ballot(j < nb && row[j] > tau));
    }
    const int need_eq = topk - greater;
    int32_t* out = kv_idx + ((size_t)h * nb + i0 + r) * topk;
    int eq_seen = 0, base = 0;
    for (int m = 0; m < nch; ++m) {
      const int j = 64 * m + lane;
      const bool valid = j < nb;
      const unsigned int a = row[j];
      const bool eq = valid && a == tau;
      const unsigned long long eqm = __ballot(eq);
      const bool take = valid && (a > tau || (eq && eq_seen + lanes_below(eqm) < need_eq));
      const unsigned long long tm = __ballot(take);
      if (take) out[base + lanes_below(tm)] = j;
      eq_seen += __popcll(eqm);
      base += __popcll(tm);
    }
    if (lane == 0) kv_cnt[(size_t)h * nb + i0 + r] = topk;
  }
}

__global__ void draft_scores_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar, int nb_q,
                                    int nb_k, int d, float* __restrict__ scores) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y;
  const int h = blockIdx.z;
  if (j >= nb_k) return;
  const float* qr = qbar + ((size_t)h * nb_q + i) * d;
  const float* kr = kbar + ((size_t)h * nb_k + j) * d;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = __fadd_rn(acc, __fmul_rn(qr[c], kr[c]));
  scores[((size_t)h * nb_q + i) * nb_k + j] = acc;
}

// ---------------------------------------------------------------------------
// Row gather with zero fill: one 16-byte chunk per thread, grid-stride.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void token_permute_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int heads, int n_src, int n_dst, int cpr,
                                                            const int32_t* __restrict__ map) {
  const size_t total = (size_t)heads * n_dst * cpr;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const size_t row = e / cpr;
    const int ch = (int)(e - row * cpr);
    const int h = (int)(row / n_dst);
    const int i = (int)(row - (size_t)h * n_dst);
    const int s = map[i];
    u32x4 x = {0u, 0u, 0u, 0u};
    if (s >= 0 && s < n_src) x = src[((size_t)h * n_src + s) * cpr + ch];
    dst[e] = x;
  }
}

}  // namespace

hipError_t launch_draft_perm(const DraftGeom& g, int32_t* perm, int32_t* inv_perm, int32_t* block_valid,
                             hipStream_t s) {
  dim3 grid((g.n_pad + 255) / 256), block(256);
  hipLaunchKernelGGL(draft_perm_kernel, grid, block, 0, s, g, perm, inv_perm, block_valid);
  return hipGetLastError();
}

hipError_t launch_draft_pool_gather(const DraftGeom& g, int heads, int d, int dt, const void* q, const void* k,
                                    const void* v, float* qbar, float* kbar, float* kbarT, void* q_perm,
                                    void* k_perm, void* v_perm, hipStream_t s) {
  const int ch = dt == 1 ? 8 : 4;
  const int lpr = d / ch;
  const int gpb = 256 / lpr;
  const int groups = heads * g.nb;
  dim3 grid((groups + gpb - 1) / gpb, v_perm ? 3 : 2), block(256);
  if (dt == 1)
    hipLaunchKernelGGL(draft_pool_gather_kernel<true>, grid, block, 0, s, g, heads, d, q, k, v, qbar, kbar, kbarT,
                       q_perm, k_perm, v_perm);
  else
    hipLaunchKernelGGL(draft_pool_gather_kernel<false>, grid, block, 0, s, g, heads, d, q, k, v, qbar, kbar, kbarT,
                       q_perm, k_perm, v_perm);
  return hipGetLastError();
}

hipError_t launch_draft_select(const float* qbar, const float* kbarT, int heads, int nb, int d, int topk,
                               int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s) {
  // Rows per workgroup so that the score codes take at most 32 KB of LDS.
  const int nb64 = (nb + 63) & ~63;
  const int R = nb64 <= 1024 ? 8 : (nb64 <= 2048 ? 4 : 2);
  const size_t shm = (size_t)R * nb64 * sizeof(unsigned int);
  dim3 grid(heads * ((nb + R - 1) / R)), block(256);
  if (R == 8)
    hipLaunchKernelGGL(draft_select_kernel<8>, grid, block, shm, s, qbar, kbarT, heads, nb, d, topk, kv_idx, kv_cnt);
  else if (R == 4)
    hipLaunchKernelGGL(draft_select_kernel<4>, grid, block, shm, s, qbar, kbarT, heads, nb, d, topk, kv_idx, kv_cnt);
  else
    hipLaunchKernelGGL(draft_select_kernel<2>, grid, block, shm, s, qbar, kbarT, heads, nb, d, topk, kv_idx, kv_cnt);
  return hipGetLastError();
}

hipError_t launch_draft_scores(const float* qbar, const float* kbar, int heads, int nb_q, int nb_k, int d,
                               float* scores, hipStream_t s) {
  dim3 grid((nb_k + 127) / 128, nb_q, heads), block(128);
  hipLaunchKernelGGL(draft_scores_kernel, grid, block, 0, s, qbar, kbar, nb_q, nb_k, d, scores);
  return hipGetLastError();
}

hipError_t launch_token_permute(const void* src, void* dst, int esize, int heads, int n_src, int n_dst, int d,
                                const int32_t* map, hipStream_t s) {
  const int cpr = d * esize / 16;
  const size_t total = (size_t)heads * n_dst * cpr;
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(token_permute_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst,
                     heads, n_src, n_dst, cpr, map);
  return hipGetLastError();
}

}  // namespace lvsa
