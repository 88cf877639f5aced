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
// Pool (Q, K) + reorder (Q, K, V). One workgroup owns one (tensor, head,
// block). The block's rows are moved in stages of 4 rounds; in a round the
// 256 threads load 4 KB of rows as 16-byte chunks (rows of one pool-tile line
// are contiguous in the source) and store them to the block's slots in the
// reordered tensor, pads as zeros. For Q and K a stage is also staged in LDS,
// where lane c folds channel c over the stage's slots in slot order, so every
// channel's sum is one sequential fold across the whole block (or, with
// MAXP, its running maximum).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_local(int w, int G) {
  // Workgroup w runs on XCD w % 8: give each XCD a contiguous range of work
  // items so that neighbouring blocks share an L2 (and K-bar-transposed
  // columns merge there before they are written back).
  const int xcd = w & 7, idx = w >> 3, q8 = G >> 3, r8 = G & 7;
  return (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + idx;
}

template <bool BF16, bool MAXP>
__global__ __launch_bounds__(256) void draft_pool_gather_kernel(DraftGeom g, int heads, int d,
                                                                const void* __restrict__ q,
                                                                const void* __restrict__ k,
                                                                const void* __restrict__ v, float* __restrict__ qbar,
                                                                float* __restrict__ kbar, float* __restrict__ kbarT,
                                                                void* __restrict__ q_perm, void* __restrict__ k_perm,
                                                                void* __restrict__ v_perm) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int ROUNDS = 4;
  __shared__ u32x4 stage[ROUNDS * 256];  // 16 KB

  const int G = (v_perm ? 3 : 2) * heads * g.nb;
  const int L = xcd_local(blockIdx.x, G);
  const int which = L / (heads * g.nb);  // 0 = Q, 1 = K, 2 = V
  const int rem = L - which * heads * g.nb;
  const int h = rem / g.nb, b = rem - h * g.nb;

  const void* src = which == 0 ? q : (which == 1 ? k : v);
  void* dst = which == 0 ? q_perm : (which == 1 ? k_perm : v_perm);
  const bool pool = which < 2;

  const int t = b / (g.nbh * g.nbw);
  const int rb = b - t * (g.nbh * g.nbw);
  const int hb = rb / g.nbw, wb = rb - hb * g.nbw;
  const int vh = min(g.ph, g.H - hb * g.ph);
  const int vw = min(g.pw, g.W - wb * g.pw);
  const int nv = vh * vw;
  const int tok0 = (t * g.H + hb * g.ph) * g.W + wb * g.pw;

  const int rowc = d * ES / 16;          // 16-byte chunks per row
  const int rpr = 256 / rowc;            // rows per round
  const int tid = threadIdx.x;
  const int sub = tid / rowc, ch = tid - sub * rowc;
  const u32x4* S = (const u32x4*)src + (size_t)h * g.n * rowc;
  u32x4* Dd = dst ? (u32x4*)dst + ((size_t)h * g.n_pad + (size_t)b * g.bs) * rowc : nullptr;

  float acc = MAXP ? -INFINITY : 0.f;
  for (int s0 = 0; s0 < g.bs; s0 += ROUNDS * rpr) {
    u32x4 x[ROUNDS];
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int slot = s0 + i * rpr + sub;
      x[i] = u32x4{0u, 0u, 0u, 0u};
      if (slot < nv) {
        const int hi = slot / vw, wi = slot - hi * vw;
        x[i] = S[(size_t)(tok0 + hi * g.W + wi) * rowc + ch];
      }
    }
    if (Dd) {
#pragma unroll
      for (int i = 0; i < ROUNDS; ++i) {
        const int slot = s0 + i * rpr + sub;
        if (slot < g.bs) Dd[(size_t)slot * rowc + ch] = x[i];
      }
    }
    if (pool) {
#pragma unroll
      for (int i = 0; i < ROUNDS; ++i) stage[i * 256 + tid] = x[i];
      __syncthreads();
      if (tid < d) {
        const int n_here = min(ROUNDS * rpr, nv - s0);
        const unsigned char* base = (const unsigned char*)stage + tid * ES;
        for (int r = 0; r < n_here; ++r) {
          float xv;
          if (BF16)
            xv = __uint_as_float((unsigned int)*(const unsigned short*)(base + (size_t)r * d * ES) << 16);
          else
            xv = *(const float*)(base + (size_t)r * d * ES);
          acc = MAXP ? fmaxf(acc, xv) : __fadd_rn(acc, xv);
        }
      }
      __syncthreads();
    }
  }
  if (pool && tid < d) {
    const float mean = MAXP ? __fadd_rn(acc, 0.f) : __fdiv_rn(acc, (float)nv);
    (which == 0 ? qbar : kbar)[((size_t)h * g.nb + b) * d + tid] = mean;
    if (which == 1) kbarT[((size_t)h * d + tid) * g.nb + b] = mean;
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

  // A row's codes are read in groups of 16 per lane (code m of a group is
  // block 64 (g0 + m) + lane); a row of at most 1024 blocks stays in
  // registers for the whole selection, longer rows are re-read from LDS on
  // every pass. Pads hold code 0, which neither a bisection candidate (>= 1)
  // nor a "> tau" test counts; the final pass skips them explicitly.
  const int w = tid >> 6, lane = tid & 63;
  const int nch = nb64 >> 6;
  const bool resident = nch <= 16;
  for (int r = w; r < nr; r += (int)(blockDim.x >> 6)) {
    const unsigned int* row = codes + r * nb64;
    unsigned int a[16];
    auto load_group = [&](int g0) {
#pragma unroll
      for (int m = 0; m < 16; ++m) a[m] = g0 + m < nch ? row[64 * (g0 + m) + lane] : 0u;
    };
    if (resident) load_group(0);
    unsigned int tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned int cand = tau | (1u << bit);
      int cnt = 0;
      for (int g0 = 0; g0 < nch; g0 += 16) {
        if (!resident) load_group(g0);
#pragma unroll
        for (int m = 0; m < 16; ++m) cnt += __popcll(__ballot(a[m] >= cand));
      }
      if (cnt >= topk) tau = cand;
    }
    int greater = 0;
    for (int g0 = 0; g0 < nch; g0 += 16) {
      if (!resident) load_group(g0);
#pragma unroll
      for (int m = 0; m < 16; ++m) greater += __popcll(__ballot(a[m] > tau));
    }
    const int need_eq = topk - greater;
    int32_t* out = kv_idx + ((size_t)h * nb + i0 + r) * topk;
    int eq_seen = 0, base = 0;
    for (int g0 = 0; g0 < nch; g0 += 16) {
      if (!resident) load_group(g0);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int j = 64 * (g0 + m) + lane;
        const bool ok = j < nb;
        const bool eq = ok && a[m] == tau;
        const unsigned long long eqm = __ballot(eq);
        const bool take = ok && (a[m] > tau || (eq && eq_seen + lanes_below(eqm) < need_eq));
        const unsigned long long tm = __ballot(take);
        if (take) out[base + lanes_below(tm)] = j;
        eq_seen += __popcll(eqm);
        base += __popcll(tm);
      }
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
// Row gather with zero fill. A workgroup moves 1024 consecutive 16-byte
// chunks of one head's destination (4 per thread, 256 apart, so every load
// and store instruction of a wave touches 1 KB of consecutive bytes).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void token_permute_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int n_src, int n_dst, int cpr, int wg_per_head,
                                                            const int32_t* __restrict__ map) {
  const int h = blockIdx.x / wg_per_head;
  const int e0 = (blockIdx.x - h * wg_per_head) * 1024 + threadIdx.x;
  const int total = n_dst * cpr;
  const u32x4* S = src + (size_t)h * n_src * cpr;
  u32x4* D = dst + (size_t)h * n_dst * cpr;
  u32x4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + 256 * i;
    x[i] = u32x4{0u, 0u, 0u, 0u};
    if (e < total) {
      const int row = e / cpr, ch = e - row * cpr;
      const int s = map[row];
      if (s >= 0 && s < n_src) x[i] = S[(size_t)s * cpr + ch];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + 256 * i;
    if (e < total) D[e] = x[i];
  }
}

}  // namespace

hipError_t launch_draft_perm(const DraftGeom& g, int32_t* perm, int32_t* inv_perm, int32_t* block_valid,
                             hipStream_t s) {
  dim3 grid((g.n_pad + 255) / 256), block(256);
  hipLaunchKernelGGL(draft_perm_kernel, grid, block, 0, s, g, perm, inv_perm, block_valid);
  return hipGetLastError();
}

hipError_t launch_draft_pool_gather(const DraftGeom& g, int heads, int d, int dt, bool pool_max, const void* q, const void* k,
                                    const void* v, float* qbar, float* kbar, float* kbarT, void* q_perm,
                                    void* k_perm, void* v_perm, hipStream_t s) {
  const int items = (v_perm ? 3 : 2) * heads * g.nb;
  dim3 grid(items), block(256);
#define LVSA_POOL_LAUNCH(BF, MX)                                                                              \
  hipLaunchKernelGGL((draft_pool_gather_kernel<BF, MX>), grid, block, 0, s, g, heads, d, q, k, v, qbar, kbar, kbarT, \
                     q_perm, k_perm, v_perm)
  if (dt == 1 && pool_max) LVSA_POOL_LAUNCH(true, true);
  else if (dt == 1) LVSA_POOL_LAUNCH(true, false);
  else if (pool_max) LVSA_POOL_LAUNCH(false, true);
  else LVSA_POOL_LAUNCH(false, false);
#undef LVSA_POOL_LAUNCH
  return hipGetLastError();
}

hipError_t launch_draft_select(const float* qbar, const float* kbarT, int heads, int nb, int d, int topk,
                               int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s) {
  // Rows per workgroup so that the score codes take at most 32 KB of LDS.
  const int nb64 = (nb + 63) & ~63;
  const int R = nb64 <= 1024 ? 8 : (nb64 <= 2048 ? 4 : 2);  // R * nb64 <= 8192
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
  const long long per_head = ((long long)n_dst * cpr + 1023) / 1024;
  if ((long long)heads * per_head == 0) return hipSuccess;
  hipLaunchKernelGGL(token_permute_kernel, dim3((unsigned)(heads * per_head)), dim3(256), 0, s, (const u32x4*)src,
                     (u32x4*)dst, n_src, n_dst, cpr, (int)per_head, map);
  return hipGetLastError();
}

}  // namespace lvsa
