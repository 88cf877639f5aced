// Block-sparse / dense softmax attention forward, bf16 in, fp32 out, on the
// gfx950 matrix cores.
//
// What it computes ("LVSA: Training-Free Sparse Attention for Long Video
// Diffusion", §1 problem statement and §2 complexity; the Draft Attention
// article's block-sparse execution on reordered tokens): every query row
// attends to the rows of the KV blocks listed for its query block,
// O = softmax(scale * Q Kᵀ) V over those keys only.
//
// Design (one workgroup = 4 waves = 128 query rows; one wave = 32 rows):
//  * The KV list of a query block is walked as one "virtual" key sequence:
//    list slot i covers virtual rows [i*block_k, (i+1)*block_k). Tiles of
//    BN virtual rows are gathered row by row into LDS, so a frame list of
//    21 frames of 1560 tokens is 512 tiles of 64 with only the last one
//    ragged, whatever the frame size.
//  * Scores are formed transposed, Sᵀ = K Qᵀ, with v_mfma_f32_32x32x16_bf16:
//    the accumulator layout then gives each lane one query column and 16
//    keys per 32x32 block, so the row max/sum of the online softmax is
//    in-lane work plus one exchange between the two half-waves, and Pᵀ is
//    already in the B-operand layout of the second product Oᵀ += Vᵀ Pᵀ.
//  * Q stays in VGPRs for the whole key walk. K is staged row-major in LDS,
//    V is staged transposed (Vᵀ, keys contiguous) by an in-register 4x8
//    transpose at staging time; both use XOR swizzles instead of padding.
//    LDS is double-buffered: the global loads of tile i+1 are in flight
//    while tile i is computed, one barrier per tile.
//  * Probabilities are exp2(s*scale*log2e - m*scale*log2e), rounded to bf16
//    for the PV product; the row sum accumulates the same rounded values
//    (v_dot2_f32_bf16 against ones), so O is a convex combination of V rows
//    up to fp32 accumulation. The O rescale is skipped when no lane's max
//    moved.
//  * Workgroup ids are remapped so that consecutive query tiles (same head,
//    same query block, same key list) land on the same XCD and share its L2.
#include "internal.h"

namespace lvsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBM = kBM_BF16;

// Where the BN virtual key rows of one tile live. Uniform across the workgroup.
struct Tile {
  int vt0;         // first virtual row
  int off0;        // offset of vt0 inside its list slot
  int blk0, blk1;  // KV block of that slot and of the next slot (-1: none)
  int lim0, lim1;  // valid rows of those blocks
  int full;        // all BN rows are valid keys
};

__device__ __forceinline__ int block_lim(const AttnArgs& a, int b) {
  if (b < 0 || b >= a.nkb) return 0;
  int lim = a.block_k;
  if (a.block_valid) {
    int bv = a.block_valid[b];
    lim = bv < 0 ? 0 : (bv < lim ? bv : lim);
  }
  int rem = a.n - b * a.block_k;
  return rem < lim ? rem : lim;
}

__device__ __forceinline__ int list_entry(const AttnArgs& a, const int32_t* list, int cnt, int slot) {
  if (slot >= cnt) return -1;
  int b = list[slot];
  return (b < 0 || b >= a.nkb) ? -1 : b;
}

template <int BN>
__device__ __forceinline__ Tile make_tile(const AttnArgs& a, const int32_t* list, int cnt, int L, int it) {
  Tile t;
  t.vt0 = it * BN;
  t.off0 = 0;
  t.blk0 = t.blk1 = -1;
  t.lim0 = t.lim1 = 0;
  if (a.dense) {
    t.full = t.vt0 + BN <= L;
    return t;
  }
  if (a.block_k >= BN) {
    int slot = t.vt0 / a.block_k;
    t.off0 = t.vt0 - slot * a.block_k;
    t.blk0 = list_entry(a, list, cnt, slot);
    t.blk1 = list_entry(a, list, cnt, slot + 1);
    t.lim0 = block_lim(a, t.blk0);
    t.lim1 = block_lim(a, t.blk1);
    bool in_len = t.vt0 + BN <= L;
    if (t.off0 + BN <= a.block_k)
      t.full = in_len && (t.off0 + BN <= t.lim0);
    else
      t.full = in_len && (t.lim0 == a.block_k) && (t.off0 + BN - a.block_k <= t.lim1);
  } else {
    t.full = 0;
  }
  return t;
}

// Physical row (within the head) of virtual row vt0 + r, or -1 if that key is invalid.
template <int BN>
__device__ __forceinline__ int row_phys(const AttnArgs& a, const Tile& t, const int32_t* list, int cnt, int L, int r) {
  int vj = t.vt0 + r;
  if (vj >= L) return -1;
  if (a.dense) return vj;
  if (a.block_k >= BN) {
    int pos = t.off0 + r;
    bool second = pos >= a.block_k;
    int blk = second ? t.blk1 : t.blk0;
    int off = second ? pos - a.block_k : pos;
    int lim = second ? t.lim1 : t.lim0;
    return off < lim ? blk * a.block_k + off : -1;
  }
  int slot = vj / a.block_k;
  int off = vj - slot * a.block_k;
  int blk = list_entry(a, list, cnt, slot);
  return off < block_lim(a, blk) ? blk * a.block_k + off : -1;
}

__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

template <int D, int BN>
__global__ __launch_bounds__(kThreads, 2) void bsa_fwd_bf16_kernel(AttnArgs a) {
  constexpr int KSTEPS = D / 16;   // k-steps of Sᵀ = K Qᵀ
  constexpr int NKB = BN / 32;     // 32-key blocks per tile
  constexpr int PVSTEPS = BN / 16; // k-steps of Oᵀ += Vᵀ Pᵀ
  constexpr int NDB = D / 32;      // 32-row blocks of Oᵀ
  constexpr int CPR = D / 8;       // 16-byte chunks per K row
  constexpr int RPI = kThreads / CPR;  // K rows per load instruction
  constexpr int KJ = BN / RPI;     // K rows per thread
  static_assert(KJ == 4, "tile shape");
  static_assert((BN / 4) * (D / 8) == kThreads, "one 4x8 V unit per thread");

  __shared__ u32x4 Ks[2][BN * CPR];
  __shared__ u32x2 Vs[2][D * (BN / 4)];
  __shared__ unsigned int kval[2][BN / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // XCD-aware tile order: workgroup w runs on XCD w % 8; give each XCD a
  // contiguous range of logical tiles.
  const int G = a.total_tiles;
  const int w = blockIdx.x;
  const int xcd = w & 7, idx = w >> 3, q8 = G >> 3, r8 = G & 7;
  const int logical = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + idx;
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
  const int row_lo = blk_lo + qt * kBM;
  const int qrow = row_lo + wave * 32 + l32;
  const bool q_in_blk = qrow < blk_end && (qrow - blk_lo) < (qt + 1) * kBM;
  const bool q_valid = qrow < qend;

  const size_t head_off = (size_t)h * (size_t)a.n * D;
  const uint16_t* __restrict__ Qh = (const uint16_t*)a.q + head_off;
  const uint16_t* __restrict__ Kh = (const uint16_t*)a.k + head_off;
  const uint16_t* __restrict__ Vh = (const uint16_t*)a.v + head_off;
  float* __restrict__ Oh = a.o + head_off;

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
  if (row_lo >= qend) L = 0;  // no valid query in this tile: only zeros are written
  const int ntiles = (L + BN - 1) / BN;

  // Q as the B operand of Sᵀ = K Qᵀ: lane (query l32, half) holds d = 16*kk + 8*half .. +7.
  bf16x8 qreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (q_valid) v = *(const u32x4*)(Qh + qrow * D + 16 * kk + 8 * half);
    qreg[kk] = __builtin_bit_cast(bf16x8, v);
  }

  // Loader roles. K: thread = (row r0 + RPI*j, 16-byte chunk kc).
  const int kc = tid % CPR;
  const int kr0 = tid / CPR;
  // V: thread = 4 keys (4*vkg .. +3) x 8 channels (8*vdg .. +7); within a wave
  // 8 key groups x 8 channel groups, arranged so LDS writes are conflict-free.
  constexpr int NKGB = BN / 32;
  const int vkg = (lane & 7) + 8 * (wave % NKGB);
  const int vdg = 2 * (lane >> 4) + ((lane >> 3) & 1) + 8 * (wave / NKGB);

  u32x4 kreg[KJ], vreg[4];
  int kphys[KJ];

  auto load_tile = [&](const Tile& t) {
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      int p = row_phys<BN>(a, t, list, cnt, L, kr0 + RPI * j);
      kphys[j] = p;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (p >= 0) v = *(const u32x4*)(Kh + p * D + 8 * kc);
      kreg[j] = v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int p = row_phys<BN>(a, t, list, cnt, L, 4 * vkg + j);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (p >= 0) v = *(const u32x4*)(Vh + p * D + 8 * vdg);
      vreg[j] = v;
    }
  };

  auto store_tile = [&](int st) {
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      int r = kr0 + RPI * j;
      Ks[st][r * CPR + (kc ^ (r & 7))] = kreg[j];
    }
    // 4 keys x 8 channels -> 8 rows of Vᵀ, each 4 keys (8 bytes).
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      unsigned int e01 = (vreg[0][m] & 0xffffu) | (vreg[1][m] << 16);
      unsigned int e23 = (vreg[2][m] & 0xffffu) | (vreg[3][m] << 16);
      unsigned int o01 = (vreg[0][m] >> 16) | (vreg[1][m] & 0xffff0000u);
      unsigned int o23 = (vreg[2][m] >> 16) | (vreg[3][m] & 0xffff0000u);
      int d0 = 8 * vdg + 2 * m;
      int d1 = d0 + 1;
      Vs[st][d0 * (BN / 4) + (vkg ^ (d0 & 15))] = u32x2{e01, e23};
      Vs[st][d1 * (BN / 4) + (vkg ^ (d1 & 15))] = u32x2{o01, o23};
    }
    if (kc == 0) {
#pragma unroll
      for (int j = 0; j < KJ; ++j) ((unsigned char*)kval[st])[kr0 + RPI * j] = kphys[j] >= 0 ? 1 : 0;
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  Tile cur = make_tile<BN>(a, list, cnt, L, 0);
  if (ntiles > 0) {
    load_tile(cur);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    const bool more = it + 1 < ntiles;
    Tile nxt;
    if (more) {
      nxt = make_tile<BN>(a, list, cnt, L, it + 1);
      load_tile(nxt);
    }

    // Sᵀ = K Qᵀ for this tile: NKB accumulators of 32 keys x 32 queries.
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int r = kb * 32 + l32;
        const int ch = 2 * kk + half;
        bf16x8 A = __builtin_bit_cast(bf16x8, Ks[st][r * CPR + (ch ^ (r & 7))]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qreg[kk], s[kb], 0, 0, 0);
      }
    }

    // Mask invalid keys. Accumulator register r of block kb holds key
    // kb*32 + 8*(r/4) + 4*half + r%4 of the tile.
    if (!cur.full) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          unsigned int f4 = kval[st][(kb * 32 + 8 * g + 4 * half) >> 2];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (((f4 >> (8 * i)) & 0xffu) == 0u) s[kb][4 * g + i] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c);
    if (__ballot(alpha != 1.f) != 0ull) {
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    m_run = m_new;
    const float nm = -m_use * c;

    // Pᵀ in the B-operand layout of Oᵀ += Vᵀ Pᵀ: step kk takes registers
    // 8*(kk%2) .. +7 of block kk/2, i.e. keys 16*kk + 8*(j/4) + 4*half + j%4.
    bf16x8 pb[PVSTEPS];
#pragma unroll
    for (int kk = 0; kk < PVSTEPS; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + j], c, nm));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + j + 1], c, nm));
        bf16x2 p2 = {(__bf16)x0, (__bf16)x1};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_run, false);
        pb[kk][j] = p2[0];
        pb[kk][j + 1] = p2[1];
      }
    }

    // Oᵀ += Vᵀ Pᵀ. A operand: row d = 32*db + l32, keys of chunks 4*kk + half
    // and 4*kk + 2 + half (4 keys each).
#pragma unroll
    for (int kk = 0; kk < PVSTEPS; ++kk) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 32 + l32;
        const u32x2 lo = Vs[st][d * (BN / 4) + ((4 * kk + half) ^ (d & 15))];
        const u32x2 hi = Vs[st][d * (BN / 4) + ((4 * kk + 2 + half) ^ (d & 15))];
        const u32x4 A4 = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, A4), pb[kk], oacc[db], 0, 0, 0);
      }
    }

    if (more) {
      store_tile(st ^ 1);
      cur = nxt;
    }
    __syncthreads();
  }

  // Epilogue: combine the two half-waves' partial sums, normalise, store fp32.
  const float l_tot = l_run + other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_in_blk) {
    float* orow = Oh + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        float4 v;
        if (q_valid) {
          v = make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                          oacc[db][4 * g + 3] * inv);
        } else {
          v = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        *(float4*)(orow + d0) = v;
      }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int d, hipStream_t s) {
  if (a.total_tiles == 0) return hipSuccess;
  dim3 grid(a.total_tiles), block(kThreads);
  if (d == 128)
    hipLaunchKernelGGL((bsa_fwd_bf16_kernel<128, 64>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((bsa_fwd_bf16_kernel<64, 128>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace lvsa
