// Block-sparse / dense softmax attention forward with FP8 (OCP E4M3)
// operands on the gfx950 matrix cores (v_mfma_f32_32x32x64_f8f6f4), fp32
// accumulation and softmax, fp32 output.
//
// What it computes: the attention of "LVSA: Training-Free Sparse Attention
// for Long Video Diffusion" (§1 problem statement, §2 complexity) over the
// listed KV blocks -- LVSA frame lists, or the Draft Attention article's
// top-k blocks on the reordered tokens (with per-block valid counts) or on
// the raster [t, h, w] layout -- on per-head E4M3 codes of Q, K and V: with
// q = sq*Q8, k = sk*K8, v = sv*V8 (codes decoded exactly),
// O = softmax(scale * q kᵀ) v. The Draft Attention article names
// quantization as its next step.
//
// Design, as the bf16 kernel (32 query rows per wave, the KV list walked as
// one virtual key sequence in 64-key tiles, one barrier per tile, Sᵀ of tile
// i+1 on the matrix core while tile i's softmax runs) with these
// differences:
//  * a deeper pipeline: step i also runs the PV product of tile i-1 under
//    the softmax of tile i (the softmax is the longer part here), so K is
//    loaded two tiles ahead and V in the step before it is read;
//  * 4 or 8 waves per workgroup (128 or 256 query rows sharing each K/V
//    tile), chosen per launch;
//  * operands are bytes: a K tile is 64 rows x 128 B, a Vᵀ tile (V is given
//    transposed, [heads, d, ldv]) is 128 rows x 64 B, each 8 KB; both come
//    from global memory into LDS with LDS-destination buffer loads (16 B per
//    lane; 4 B per lane -- one group of 4 keys -- where a tile is not one
//    physical run). Keys are valid as a prefix of each group of 4 (n and
//    block_k are multiples of 4, pool rows hold whole groups), so a partial
//    tile masks its scores with one flag byte per key, and the other bytes
//    of a partly valid group are finite codes that meet probability 0;
//  * the 32x32x64 MFMA operand layout (checked on the GPU): lane l holds row
//    (A) or column (B) l mod 32 and k = 32*(l/32) .. +31, one byte each;
//    Sᵀ = K Qᵀ takes 2 k-steps over d = 128, Oᵀ += Vᵀ Pᵀ one k-step over
//    the 64 keys of a tile;
//  * probabilities are rounded to E4M3 (v_cvt_pk_fp8_f32, nearest even).
//    They are computed against a lagging reference (one of the row's
//    scores) with no row max; when a lane's probabilities of a tile sum to
//    more than 2^8 the wave moves the reference to the row max, rescales
//    and recomputes the tile, so every rounded probability is <= 2^8, inside
//    the E4M3 range;
//  * K rows sit in LDS in a permuted order, row r = 32kb + 8g + 4h + i
//    holding key 32h + 16kb + 4g + i, so that the Sᵀ accumulator of lane
//    (query, half h) holds exactly keys 32h .. 32h+31, in the byte order of
//    the PV product's B operand: the packed probabilities feed the matrix
//    core as they are, with no exchange between the half-waves;
//  * the row sum adds the unrounded fp32 probabilities.
#include <type_traits>

#include "attn_tiles.h"

namespace lvsa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ i32x8 lds_read32(const unsigned char* base, unsigned off0, unsigned off1) {
  const u32x4 a = *(const u32x4*)(base + off0);
  const u32x4 b = *(const u32x4*)(base + off1);
  i32x8 r;
  r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
  r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
  return r;
}

__device__ __forceinline__ unsigned int pack4_fp8(float a, float b, float c, float d) {
  // The first conversion fills bytes 0-1 and keeps bytes 2-3 of its third
  // operand, which the second conversion overwrites: any value serves, and
  // the bits of a (dead once its row sum is taken) need no extra register.
  unsigned int w = (unsigned int)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)__float_as_uint(a), false);
  w = (unsigned int)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
  return w;
}

// Tile key held by K row r of LDS: r = 32kb + 8g + 4h + i -> 32h + 16kb + 4g + i.
__device__ __forceinline__ int krow(int r) {
  return (((r >> 2) & 1) << 5) | (((r >> 5) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
}

// NW waves per workgroup, 32 query rows each, sharing every K/V tile.
template <int MODE, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bsa_fwd_fp8_kernel(AttnArgs a, const float* __restrict__ qsc,
                                                                      const float* __restrict__ ksc,
                                                                      const float* __restrict__ vsc) {
  constexpr int D = 128, BN = 64, NKB = 2, NDB = 4, BM = 32 * NW;
  constexpr int TILE = BN * D;  // 8 KB per K or Vᵀ tile
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char ks1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vs1[TILE];
  __shared__ unsigned int kval[4][BN / 4];  // per-key flags of tile i in slot i % 4
  auto kbuf = [&](int st) -> unsigned char* { return st == 0 ? ks0 : ks1; };
  auto vbuf = [&](int st) -> unsigned char* { return st == 0 ? vs0 : vs1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int G = a.total_tiles;
  const int w = blockIdx.x;
  const int xcd = w & 7, idx = w >> 3, q8 = G >> 3, r8 = G & 7;
  const int logical = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + idx;
  const int qt = logical % a.tiles_per_qb;
  const int rest = logical / a.tiles_per_qb;
  int qb = rest % a.nqb;
  const int h = rest / a.nqb;
  if (MODE == MODE_T2D) {
    // Raster Draft: consecutive workgroups (one XCD) take the same pool tile
    // of consecutive frames, whose top-k lists share more key blocks than
    // those of neighbouring tiles of one frame (measured: 1.2 % faster).
    const int per = a.nbh * a.nbw, nt = a.nqb / per;
    qb = (qb % nt) * per + qb / nt;
  }

  const int blk_lo = qb * a.block_q;
  const int blk_end = min(blk_lo + a.block_q, a.n);
  int qlim = a.block_q;
  if (MODE == MODE_LIST && a.block_valid) {
    const int bv = a.block_valid[qb];
    qlim = bv < 0 ? 0 : (bv < qlim ? bv : qlim);
  }
  const int qend = min(blk_lo + qlim, blk_end);
  const int row_lo = blk_lo + qt * BM;
  int qrow = row_lo + wave * 32 + l32;
  bool q_in_blk = qrow < blk_end;  // output row to write (0 for pad rows)
  bool q_valid = qrow < qend;      // query with keys
  bool no_queries = row_lo >= qend;
  if (MODE == MODE_T2D) {
    // Query block qb is a raster pool tile; slot s = (s / pw, s % pw).
    const BlkGeom gq = blk_geom(a, qb);
    const int slot = qt * BM + wave * 32 + l32;
    const int hi = slot >> a.lpw, wi = slot & (a.pw - 1);
    q_valid = slot < a.block_q && hi < gq.vh && wi < gq.vw;
    q_in_blk = q_valid;
    qrow = q_valid ? gq.tok + hi * a.gW + wi : 0;
    no_queries = ((qt * BM) >> a.lpw) >= gq.vh;
  }

  const size_t head_off = (size_t)h * (size_t)a.n * D;  // bytes: one byte per element
  const int head_bytes = a.n * D;
  const __amdgpu_buffer_rsrc_t Qr =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.q + head_off), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t Kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.k + head_off), (short)0, head_bytes, 0x00020000);
  const size_t vhead_off = (size_t)h * D * (size_t)a.ldv;  // Vᵀ rows have a.ldv bytes
  const __amdgpu_buffer_rsrc_t Vr = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.v + vhead_off),
                                                                      (short)0, D * a.ldv, 0x00020000);
  float* __restrict__ Oh = a.o + head_off;

  const int32_t* list = nullptr;
  int cnt = 0, L = a.n;
  if (MODE != MODE_DENSE) {
    const int hm = a.mask_heads > 1 ? h : 0;
    const int base = hm * a.nqb + qb;
    cnt = a.kv_cnt[base];
    cnt = cnt < 0 ? 0 : (cnt > a.max_kv ? a.max_kv : cnt);
    list = a.kv_idx + (size_t)base * a.max_kv;
    L = cnt * a.block_k;
  }
  if (no_queries) L = 0;
  const int ntiles = (L + BN - 1) / BN;

  // Qᵀ operand: lane (query l32, half) holds d = 64 s + 32 half .. +31.
  i32x8 qreg[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const unsigned off = q_valid ? (unsigned)(qrow * D + 64 * s + 32 * half) : kInvalid;
    const u32x4 lo = bload(Qr, off);
    const u32x4 hi = bload(Qr, q_valid ? off + 16u : kInvalid);
    qreg[s][0] = (int)lo[0]; qreg[s][1] = (int)lo[1]; qreg[s][2] = (int)lo[2]; qreg[s][3] = (int)lo[3];
    qreg[s][4] = (int)hi[0]; qreg[s][5] = (int)hi[1]; qreg[s][6] = (int)hi[2]; qreg[s][7] = (int)hi[3];
  }

  // LDS layouts. K: row r (key) is 128 B, chunk c (16 B) at c ^ ((r >> 1) & 7).
  // Vᵀ: row d is 64 B (keys), chunk c at c ^ ((d >> 2) & 3). Every 16-lane
  // group of a 128-bit read then covers 16 distinct 16-byte bank groups.
  // K loads: instruction j (< 8/NW) of wave `wave` fills the 1 KB chunk
  // c = NW*j + wave, LDS rows R = 8c + lane/8, LDS chunk lane%8, from tile
  // key krow(R).
  constexpr int KJ = 8 / NW, VJ = 8 / NW, VJ4 = 32 / NW;
  const int kr_l = lane >> 3, kc_l = lane & 7;
  // MODE_T2D (pw = 16): tile key k is token base0 + (k / 16) * W + k % 16.
  auto key_off = [&](int k) { return MODE == MODE_T2D ? (k >> 4) * a.gW + (k & 15) : k; };
  unsigned kdma[KJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int R = 8 * (NW * j + wave) + kr_l;
    kdma[j] = (unsigned)(key_off(krow(R)) * 128 + 16 * (kc_l ^ ((R >> 1) & 7)));
  }
  // Vᵀ loads (16 B): instruction j of wave `wave` fills the 1 KB chunk
  // c = NW*j + wave, rows d = 16c + lane/4, LDS chunk lane%4.
  const int vd_l = lane >> 2, vc_l = lane & 3;
  const unsigned vdma = (unsigned)(vd_l * a.ldv + key_off(16 * (vc_l ^ ((vd_l >> 2) & 3))));

  unsigned kra[2][2];  // [k-step][16-byte half of the 32-byte operand] for key row l32 (+32 kb)
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = 4 * s + 2 * half + u;
      kra[s][u] = (unsigned)(l32 * 128 + 16 * (c ^ ((l32 >> 1) & 7)));
    }
  unsigned vra[2];  // Vᵀ row d = 32 db + l32, keys 32 half .. +31
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = 2 * half + u;
    vra[u] = (unsigned)(l32 * 64 + 16 * (c ^ ((l32 >> 2) & 3)));
  }

  // All BN rows valid and physically consecutive from base0: one run, or two
  // runs of adjacent blocks (then base1 == base0); MODE_T2D: a full tile of
  // 16-wide pool rows (four runs of 16 tokens). The 16-byte V pieces of such
  // a tile start at multiples of 4 bytes (base0, W and a.ldv are), which the
  // LDS-destination loads accept.
  auto simple = [&](const TileD& t) {
    return MODE == MODE_T2D ? (t.full && a.pw == 16) : (t.full && (t.bnd >= BN || t.base1 == t.base0));
  };
  auto dma16 = [&](__amdgpu_buffer_rsrc_t r, unsigned char* dst, unsigned voff, unsigned soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
  };
  auto dma4 = [&](__amdgpu_buffer_rsrc_t r, unsigned char* dst, unsigned voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, voff, 0u, 0, 0);
  };
  // K of a tile, and (for a tile that is not full) one flag byte per key
  // into kval[slot]: byte k is key k of the tile.
  auto load_k = [&](const TileD& t, int st, int slot) {
    unsigned char* kb = kbuf(st);
    if (simple(t)) {
      const unsigned so = (unsigned)(t.base0 * D);
#pragma unroll
      for (int j = 0; j < KJ; ++j) dma16(Kr, kb + 1024 * (NW * j + wave), kdma[j], so);
    } else {
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        const int R = 8 * (NW * j + wave) + kr_l;
        const int p = tile_row<BN, MODE>(a, t, list, cnt, krow(R));
        const unsigned off = p >= 0 ? (unsigned)(p * 128 + 16 * (kc_l ^ ((R >> 1) & 7))) : kInvalid;
        dma16(Kr, kb + 1024 * (NW * j + wave), off, 0u);
        // The valid keys of a group of 4 are a prefix of it (runs and pool
        // rows hold whole groups); the other bytes of a partly valid group
        // of V are finite codes that meet probability 0.
        if (kc_l == 0) ((unsigned char*)kval[slot])[krow(R)] = p >= 0 ? 1 : 0;
      }
    }
  };
  auto load_v = [&](const TileD& t, int st) {
    unsigned char* vb = vbuf(st);
    if (simple(t)) {
      const unsigned so = (unsigned)t.base0;
#pragma unroll
      for (int j = 0; j < VJ; ++j)
        dma16(Vr, vb + 1024 * (NW * j + wave), vdma, so + (unsigned)(16 * (NW * j + wave)) * (unsigned)a.ldv);
    } else {
      // 4-byte pieces: instruction j fills the 256 B chunk c = NW*j + wave,
      // rows d = 4c + lane/16; LDS piece lane%16 of the row holds keys
      // 4q .. 4q+3 of the tile.
#pragma unroll
      for (int j = 0; j < VJ4; ++j) {
        const int d = 4 * (NW * j + wave) + (lane >> 4);
        const int p4 = lane & 15;
        const int q = 4 * ((p4 >> 2) ^ ((d >> 2) & 3)) + (p4 & 3);
        const int p = tile_row<BN, MODE>(a, t, list, cnt, 4 * q);
        dma4(Vr, vb + 256 * (NW * j + wave), p >= 0 ? (unsigned)(d * a.ldv + p) : kInvalid);
      }
    }
  };
  auto qk = [&](int st, f32x16 (&s)[NKB]) {
    const f32x16 zero = {};
    const unsigned char* kb = kbuf(st);
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2) {
        const i32x8 A = lds_read32(kb + kb2 * 4096, kra[ss][0], kra[ss][1]);
        s[kb2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, qreg[ss], ss == 0 ? zero : s[kb2], 0, 0, 0, 0,
                                                                   0, 0);
      }
    }
  };
  auto wait_dma = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mc = -INFINITY;
  float l_run = 0.f;
  // Kept a positive normal number: with tiny per-head scales the product
  // could underflow to 0, and a masked key's -inf score times 0 is NaN. At
  // that size every score is 0 to within fp32, so the result is unchanged.
  const float c = fmaxf(a.scale_log2 * qsc[h] * ksc[h], 1.17549435e-38f);

  // exp2(s*c - m) of a tile's scores in E4M3 as the Pᵀ operand: word
  // 4kb + g holds the scores cur[kb][4g .. 4g+3], keys 32*half + 16kb + 4g +
  // (0..3), so byte k of the operand is key 32*half + k. Returns the lane's
  // sum of the unrounded values.
  auto probs = [&](const f32x16 (&cur)[NKB], float m, i32x8& pB) {
    const float nm = (m == -INFINITY) ? 0.f : -m;
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[kb2][4 * g + t], c, nm));
        if (g & 1)
          t1 += (p[0] + p[1]) + (p[2] + p[3]);
        else
          t0 += (p[0] + p[1]) + (p[2] + p[3]);
        pB[4 * kb2 + g] = (int)pack4_fp8(p[0], p[1], p[2], p[3]);
      }
    return t0 + t1;
  };

  // Oᵀ += Vᵀ Pᵀ over one tile (Vᵀ in stage st).
  auto pv = [&](int st, const i32x8& pB) {
    const unsigned char* vb = vbuf(st);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const i32x8 A = lds_read32(vb + db * 2048, vra[0], vra[1]);
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, pB, oacc[db], 0, 0, 0, 0, 0, 0);
    }
  };

  // Pipeline over tiles i = 0, 1, ...: step i loads K of tile i+2 and Vᵀ of
  // tile i, runs Sᵀ of tile i+1 and PV of tile i-1 on the matrix core while
  // the softmax of tile i runs on the VALU, then waits for its loads and
  // meets the other waves at one barrier. K and Vᵀ of tile i sit in stage
  // i % 2, so step i reads only stage (i+1) % 2 and fills only stage i % 2.
  f32x16 s[NKB], sn[NKB];
  i32x8 pa, pz;
  TileStream ks;
  stream_init<BN, MODE>(ks, a, list, cnt, 0);
  TileD tq0, tq1;  // descriptors of tiles i and i+1
  if (ntiles > 0) {
    tq0 = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    tq1 = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    load_k(tq0, 0, 0);
    load_k(tq1, 1, 1);
  }
  wait_dma();
  __syncthreads();
  if (ntiles > 0) qk(0, s);
  __syncthreads();

  auto step = [&](auto with_pv, const int st, const int i, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB],
                  const i32x8& pprev, i32x8& pcur) {
    const TileD tk = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    load_k(tk, st, (i + 2) & 3);
    load_v(tq0, st);
    const int full_i = tq0.full;
    tq0 = tq1;
    tq1 = tk;

    if (!full_i) {
      const unsigned* fl = kval[i & 3];
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // score rows 32kb + 8g + 4h + u are keys 32h + 16kb + 4g + u
          const unsigned f4 = fl[8 * half + 4 * kb2 + g];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (((f4 >> (8 * u)) & 0xffu) == 0u) cur[kb2][4 * g + u] = -INFINITY;
        }
    }

    qk(st ^ 1, nxt);
    if constexpr (decltype(with_pv)::value) pv(st ^ 1, pprev);

    // Probabilities against the running reference mc, with no row max: a
    // lane whose probabilities of this tile sum to more than kSumFp8 (so one
    // of them may exceed 2^8), or whose row has no reference yet, sends the
    // wave through the exact path, which moves mc to the row max, rescales
    // and recomputes.
    float tl = probs(cur, mc, pcur);
    // Interleave the MFMAs (4 of Sᵀ, 4 of PV) with their LDS reads (kept
    // ahead) and the softmax VALU work, which depends on neither: six VALU
    // instructions after each MFMA, the rest after the last one (measured:
    // 1.6 % faster than twelve on LVSA lists, 0.5 % on Draft lists).
    if constexpr (decltype(with_pv)::value) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (g < 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
    }
    if (__ballot(!(tl <= kSumFp8) || mc == -INFINITY) != 0ull) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[kb2][r]);
      mx = half_max(mx) * c;
      const float mc_new = fmaxf(mc, mx);
      const float alpha = mc_new == mc ? 1.f : __builtin_amdgcn_exp2f(mc - mc_new);
      mc = mc_new;
      l_run *= alpha;
      // O holds tiles up to i-1 against the old reference.
#pragma unroll
      for (int u = 0; u < NDB; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[u][r] *= alpha;
      tl = probs(cur, mc, pcur);
    }
    l_run += tl;

    wait_dma();
    __syncthreads();
  };

  using no_pv = std::integral_constant<bool, false>;
  using with_pv = std::integral_constant<bool, true>;
  int it = 0;
  if (ntiles > 0) {
    step(no_pv{}, 0, 0, s, sn, pz, pa);
    it = 1;
  }
  for (; it + 1 < ntiles; it += 2) {
    step(with_pv{}, 1, it, sn, s, pa, pz);
    step(with_pv{}, 0, it + 1, s, sn, pz, pa);
  }
  bool last_in_pz = false;
  if (it < ntiles) {
    step(with_pv{}, 1, it, sn, s, pa, pz);
    last_in_pz = true;
  }
  // PV of the last tile (its Vᵀ in stage (ntiles-1) % 2).
  if (ntiles > 0) {
    if (last_in_pz)
      pv(1, pz);
    else
      pv(0, pa);
  }

  const float l_tot = half_sum(l_run);
  const float inv = l_tot > 0.f && q_valid ? vsc[h] / l_tot : 0.f;  // pad rows: 0
  if (q_in_blk) {
    float* orow = Oh + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        *(float4*)(orow + d0) = make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                            oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      }
  }
}

// Waves per workgroup. Eight waves (256 query rows) load each K/V tile once
// for twice the rows, but the two waves that share a SIMD then run in step;
// measured on MI355X: 6 % faster on dense 196560-token attention, slower on
// 1560-row query blocks, whose last 24 rows would hold a whole 256-row
// workgroup. So: eight waves when 256-row tiles leave no more idle rows in a
// query block than 128-row tiles do.
int fp8_waves(const AttnArgs& a) {
  if (a.tile2d) return 4;
  const int r = a.block_q % 256;
  return (r == 0 || r > 128) ? 8 : 4;
}

}  // namespace

hipError_t launch_draft_attn_fp8(const AttnArgs& a, const float* qs, const float* ks, const float* vs,
                                 hipStream_t s) {
  if (a.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((bsa_fwd_fp8_kernel<MODE_T2D, 4>), dim3(a.total_tiles), dim3(256), 0, s, a, qs, ks, vs);
  return hipGetLastError();
}

int fp8_rows_per_workgroup(const AttnArgs& a) { return 32 * fp8_waves(a); }

hipError_t launch_attn_fp8(const AttnArgs& a, const float* qs, const float* ks, const float* vs, hipStream_t s) {
  if (a.total_tiles == 0) return hipSuccess;
  const int nw = fp8_waves(a);
  dim3 grid(a.total_tiles), block(64 * nw);
  if (nw == 8) {
    if (a.dense)
      hipLaunchKernelGGL((bsa_fwd_fp8_kernel<MODE_DENSE, 8>), grid, block, 0, s, a, qs, ks, vs);
    else
      hipLaunchKernelGGL((bsa_fwd_fp8_kernel<MODE_LIST, 8>), grid, block, 0, s, a, qs, ks, vs);
  } else {
    if (a.dense)
      hipLaunchKernelGGL((bsa_fwd_fp8_kernel<MODE_DENSE, 4>), grid, block, 0, s, a, qs, ks, vs);
    else
      hipLaunchKernelGGL((bsa_fwd_fp8_kernel<MODE_LIST, 4>), grid, block, 0, s, a, qs, ks, vs);
  }
  return hipGetLastError();
}

}  // namespace lvsa
