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
                                                                float* __restrict__ kbar, void* __restrict__ q_perm,
                                                                void* __restrict__ k_perm, void* __restrict__ v_perm) {
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
  }
}

// ---------------------------------------------------------------------------
// Draft map + top-k. One workgroup owns R query-block rows of one head:
//  1. s[r][j] = fold_c fl(acc + fl(q̄[r][c] * k̄[j][c])) for every KV block j;
//  2. each score becomes a 64-bit key (descending score, then ascending j;
//     -0 canonicalised to +0) and each row is bitonic-sorted in LDS;
//  3. the first k keys mark their blocks; a workgroup scan writes the marked
//     block ids in ascending order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long score_key(float s, int j) {
  unsigned int bits = __float_as_uint(s);
  if (bits == 0x80000000u) bits = 0u;
  const unsigned int asc = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  return ((unsigned long long)(~asc) << 32) | (unsigned int)j;
}

__global__ __launch_bounds__(256) void draft_select_kernel(const float* __restrict__ qbar,
                                                           const float* __restrict__ kbar, int heads, int nb, int d,
                                                           int topk, int nbp, int R, int32_t* __restrict__ kv_idx,
                                                           int32_t* __restrict__ kv_cnt) {
  extern __shared__ unsigned long long smem[];
  unsigned long long* keys = smem;                      // [R][nbp]
  float* qs = (float*)(keys + (size_t)R * nbp);         // [R][d]
  unsigned char* sel = (unsigned char*)(qs + R * d);    // [R][nbp]
  __shared__ int scan[256];

  const int tid = threadIdx.x;
  const int rows_per_head = (nb + R - 1) / R;
  const int h = blockIdx.x / rows_per_head;
  const int i0 = (blockIdx.x - h * rows_per_head) * R;
  const int nr = min(R, nb - i0);

  for (int e = tid; e < R * d; e += blockDim.x) {
    const int r = e / d;
    qs[e] = r < nr ? qbar[((size_t)h * nb + i0 + r) * d + (e - r * d)] : 0.f;
  }
  __syncthreads();

  const float* kh = kbar + (size_t)h * nb * d;
  for (int j = tid; j < nbp; j += blockDim.x) {
    if (j < nb) {
      float acc[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = 0.f;
      const float4* kr = (const float4*)(kh + (size_t)j * d);
      for (int c4 = 0; c4 < d / 4; ++c4) {
        const float4 kv = kr[c4];
        const float kc[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (r < R) acc[r] = __fadd_rn(acc[r], __fmul_rn(qs[r * d + 4 * c4 + u], kc[u]));
        }
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r < R) keys[(size_t)r * nbp + j] = score_key(acc[r], j);
    } else {
      for (int r = 0; r < R; ++r) keys[(size_t)r * nbp + j] = ~0ull;
    }
  }
  __syncthreads();

  // Ascending bitonic sort of each row.
  const int half_n = nbp >> 1;
  for (int kk = 2; kk <= nbp; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int e = tid; e < R * half_n; e += blockDim.x) {
        const int r = e / half_n, ip = e - r * half_n;
        const int i = (ip / jj) * 2 * jj + (ip % jj);
        const int p = i + jj;
        unsigned long long* row = keys + (size_t)r * nbp;
        const unsigned long long x = row[i], y = row[p];
        const bool up = (i & kk) == 0;
        if ((x > y) == up) {
          row[i] = y;
          row[p] = x;
        }
      }
      __syncthreads();
    }
  }

  for (int e = tid; e < R * nbp; e += blockDim.x) sel[e] = 0;
  __syncthreads();
  for (int e = tid; e < R * topk; e += blockDim.x) {
    const int r = e / topk, i = e - r * topk;
    const unsigned int j = (unsigned int)(keys[(size_t)r * nbp + i] & 0xffffffffu);
    if (r < nr && j < (unsigned int)nb) sel[r * nbp + j] = 1;
  }
  __syncthreads();

  // Ascending compaction of the marked blocks, one row at a time.
  const int per = (nbp + blockDim.x - 1) / blockDim.x;
  for (int r = 0; r < nr; ++r) {
    const int j0 = tid * per;
    int c = 0;
    for (int u = 0; u < per; ++u)
      if (j0 + u < nb) c += sel[r * nbp + j0 + u];
    scan[tid] = c;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    int pos = scan[tid] - c;
    int32_t* out = kv_idx + ((size_t)h * nb + i0 + r) * topk;
    for (int u = 0; u < per; ++u) {
      const int j = j0 + u;
      if (j < nb && sel[r * nbp + j]) out[pos++] = j;
    }
    if (tid == 0) kv_cnt[(size_t)h * nb + i0 + r] = topk;
    __syncthreads();
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
                                    const void* v, float* qbar, float* kbar, void* q_perm, void* k_perm,
                                    void* v_perm, hipStream_t s) {
  const int ch = dt == 1 ? 8 : 4;
  const int lpr = d / ch;
  const int gpb = 256 / lpr;
  const int groups = heads * g.nb;
  dim3 grid((groups + gpb - 1) / gpb, v_perm ? 3 : 2), block(256);
  if (dt == 1)
    hipLaunchKernelGGL(draft_pool_gather_kernel<true>, grid, block, 0, s, g, heads, d, q, k, v, qbar, kbar, q_perm,
                       k_perm, v_perm);
  else
    hipLaunchKernelGGL(draft_pool_gather_kernel<false>, grid, block, 0, s, g, heads, d, q, k, v, qbar, kbar, q_perm,
                       k_perm, v_perm);
  return hipGetLastError();
}

hipError_t launch_draft_select(const float* qbar, const float* kbar, int heads, int nb, int d, int topk,
                               int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s) {
  int nbp = 1;
  while (nbp < nb) nbp <<= 1;
  int R = 4096 / nbp;
  R = R < 1 ? 1 : (R > 8 ? 8 : R);
  const size_t shm = (size_t)R * nbp * 8 + (size_t)R * d * 4 + (size_t)R * nbp;
  const int rows_per_head = (nb + R - 1) / R;
  dim3 grid(heads * rows_per_head), block(256);
  hipLaunchKernelGGL(draft_select_kernel, grid, block, shm, s, qbar, kbar, heads, nb, d, topk, nbp, R, kv_idx,
                     kv_cnt);
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
