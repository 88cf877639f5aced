// Block-sparse / dense softmax attention forward, bf16 in, fp32 out, on the
// gfx950 matrix cores.
//
// What it computes ("LVSA: Training-Free Sparse Attention for Long Video
// Diffusion", §1 problem statement and §2 complexity; the Draft Attention
// article's block-sparse execution on reordered tokens, or in place on the
// raster [t, h, w] layout where a block is a pool_h x pool_w tile): every
// query row attends to the rows of the KV blocks listed for its query block,
// O = softmax(scale * Q Kᵀ) V over those keys only.
//
// Design (one workgroup = 4 waves = 128 query rows, or for d = 128 lists and
// dense attention 8 waves = 256 rows; one wave = 32 rows):
//  * The KV list of a query block is walked as one "virtual" key sequence:
//    list slot i covers virtual rows [i*block_k, (i+1)*block_k). Tiles of
//    BN virtual rows are gathered row by row, so a frame list of 21 frames
//    of 1560 tokens is 512 tiles of 64 with only the last one ragged,
//    whatever the frame size. A row that is not a valid key gets a buffer
//    offset past the end of the buffer and reads as zero.
//  * Scores are formed transposed, Sᵀ = K Qᵀ, with v_mfma_f32_32x32x16_bf16:
//    the accumulator layout gives each lane one query column and 16 keys
//    per 32x32 block, so the row max/sum of the online softmax is in-lane
//    work plus one v_permlane32_swap between the half-waves, and Pᵀ is
//    already in the B-operand layout of the second product Oᵀ += Vᵀ Pᵀ.
//  * Q stays in VGPRs for the whole key walk.
//  * d = 128 (bsa_fwd_d128_kernel): K and V tiles go from global memory
//    straight into LDS with buffer loads that have an LDS destination; Vᵀ
//    operands are read from the row-major V tile with ds_read_b64_tr_b16.
//    d = 64 (bsa_fwd_bf16_kernel): rows are staged through VGPRs and V is
//    transposed in registers (4x8) before it is written to LDS. Both use
//    XOR swizzles instead of padding.
//  * Software pipeline, one barrier per tile: while the softmax of tile i
//    runs on the VALU, the MFMAs of Sᵀ for tile i+1 run on the matrix core
//    (K runs one tile ahead of V in LDS, two tiles ahead in global loads).
//    d = 128 fixes the instruction order inside a step with scheduling
//    group barriers, so each Sᵀ MFMA is followed by its share of the
//    softmax and the LDS reads run ahead of the MFMAs that use them.
//  * Probabilities are exp2(s*c - m), c = scale*log2(e), rounded to bf16
//    for the PV product; the row sum accumulates the same rounded values
//    (v_dot2_f32_bf16 against ones), so O is a convex combination of V rows
//    up to fp32 accumulation. The reference m is one of the row's scores
//    (times c) and lags the running max: d = 128 computes a tile's
//    probabilities against it without any row max, and only when a lane's
//    probabilities of the tile sum to more than 2^16 (so one of them may be
//    large) does the wave take the row max, move m to it, rescale O and
//    recompute the tile. Probabilities stay <= 2^16, far inside bf16 and
//    fp32 range. d = 64 moves m when the tile max exceeds it by more than
//    8 (in log2 units).
//  * Workgroup ids are remapped so that consecutive query tiles (same head,
//    same query block, same key list) land on the same XCD and share its L2,
//    which then serves most K/V re-reads (95-96 % hit rate on LVSA lists).
//  * For LVSA frames (1560 rows = 12 x 128 + 24) the host launches this
//    kernel over the full rows only, as six 256-row workgroups of eight
//    waves per frame (each K/V tile loaded into LDS serves 256 query rows,
//    half the L2-to-LDS bytes per FLOP of 128-row workgroups); the short
//    tails of four frames per workgroup run in attn_grp.hip (MODE_TAIL).
//    In an eight-wave workgroup the two waves of a SIMD meet at the same
//    barriers, so the upper four waves issue their Sᵀ MFMAs before their
//    softmax instead of interleaving them, and the lower four interleave
//    one VALU instruction per MFMA instead of four.
//  * MODE_T2D (raster Draft): query and key blocks are pool tiles of the
//    [t, h, w] grid; a 64-key tile is 64/pool_w pool rows, and a full tile of
//    16-wide rows loads as four runs of 16 consecutive tokens.
#include "attn_tiles.h"

namespace lvsa {
namespace {


template <int D, int BN, int MODE>
__global__ __launch_bounds__(kThreads, 2) void bsa_fwd_bf16_kernel(AttnArgs a) {
  constexpr int KSTEPS = D / 16;   // k-steps of Sᵀ = K Qᵀ
  constexpr int NKB = BN / 32;     // 32-key blocks per tile
  constexpr int PVSTEPS = BN / 16; // k-steps of Oᵀ += Vᵀ Pᵀ
  constexpr int NDB = D / 32;      // 32-row blocks of Oᵀ
  constexpr int CPR = D / 8;       // 16-byte chunks per K row
  constexpr int RPI = kThreads / CPR;  // K rows per load instruction
  constexpr int KJ = BN / RPI;     // K rows per thread
  constexpr int NKGB = BN / 32;    // 8-key-group blocks of the V loader
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
  const bool q_in_blk = qrow < blk_end;
  const bool q_valid = qrow < qend;

  const size_t head_off = (size_t)h * (size_t)a.n * D;
  const int head_bytes = a.n * D * 2;
  const __amdgpu_buffer_rsrc_t Qr =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.q + head_off), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t Kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.k + head_off), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t Vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.v + head_off), (short)0, head_bytes, 0x00020000);
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
  if (row_lo >= qend) L = 0;  // no valid query in this tile: only zeros are written
  const int ntiles = (L + BN - 1) / BN;

  // Q as the B operand of Sᵀ = K Qᵀ: lane (query l32, half) holds d = 16*kk + 8*half .. +7.
  bf16x8 qreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const unsigned off = q_valid ? (unsigned)((qrow * D + 16 * kk + 8 * half) * 2) : kInvalid;
    qreg[kk] = __builtin_bit_cast(bf16x8, bload(Qr, off));
  }

  // Loader roles. K: thread = (row kr0 + RPI*j, 16-byte chunk kc).
  const int kc = tid % CPR;
  const int kr0 = tid / CPR;
  // V: thread = 4 keys (4*vkg .. +3) x 8 channels (8*vdg .. +7); within a wave
  // 8 key groups x 8 channel groups, arranged so the LDS writes are conflict-free.
  const int vkg = (lane & 7) + 8 * (wave % NKGB);
  const int vdg = 2 * (lane >> 4) + ((lane >> 3) & 1) + 8 * (wave / NKGB);

  u32x4 kreg[KJ], vreg[4];
  unsigned vok = 0;

  // Per-thread byte offsets of the loader rows inside a tile whose rows are
  // one contiguous run (the common case); the run's start is a scalar offset.
  const unsigned kofs = (unsigned)((kr0 * D + 8 * kc) * 2);        // + j * RPI*D*2 for row j
  const unsigned vofs = (unsigned)((4 * vkg * D + 8 * vdg) * 2);   // + j * D*2 for row j

  // A tile is "simple" when all BN rows are valid keys of one block run.
  auto simple = [&](const TileD& t) { return t.full && t.bnd >= BN; };

  auto load_k = [&](const TileD& t) {
    if (simple(t)) {
      const unsigned so = (unsigned)(t.base0 * D * 2);
#pragma unroll
      for (int j = 0; j < KJ; ++j)
        kreg[j] = __builtin_amdgcn_raw_buffer_load_b128(Kr, kofs, so + (unsigned)(j * RPI * D * 2), 0);
    } else {
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        const int p = tile_row<BN, MODE>(a, t, list, cnt, kr0 + RPI * j);
        kreg[j] = bload(Kr, p >= 0 ? (unsigned)((p * D + 8 * kc) * 2) : kInvalid);
      }
    }
  };
  auto load_v = [&](const TileD& t) {
    if (simple(t)) {
      const unsigned so = (unsigned)(t.base0 * D * 2);
      vok = 0x01010101u;
#pragma unroll
      for (int j = 0; j < 4; ++j) vreg[j] = __builtin_amdgcn_raw_buffer_load_b128(Vr, vofs + j * D * 2, so, 0);
    } else {
      vok = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = tile_row<BN, MODE>(a, t, list, cnt, 4 * vkg + j);
        vok |= (p >= 0 ? 1u : 0u) << (8 * j);
        vreg[j] = bload(Vr, p >= 0 ? (unsigned)((p * D + 8 * vdg) * 2) : kInvalid);
      }
    }
  };
  // LDS swizzles (no padding). K: 16-byte chunk c of row r sits at chunk
  // c ^ (r & KSW). Vᵀ: 8-byte chunk c (4 keys) of row d sits at c ^ vsw(d).
  // Both keep 16 consecutive rows of a read (and of a write) on distinct banks
  // for 32 and for 64 four-byte banks.
  constexpr int KSW = CPR >= 16 ? 15 : CPR - 1;
  auto vsw = [](int d) { return BN == 64 ? ((d & 15) ^ ((d >> 4) & 1)) : (d & 31); };
  auto store_k = [&](int st) {
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int r = kr0 + RPI * j;
      Ks[st][r * CPR + (kc ^ (r & KSW))] = kreg[j];
    }
  };
  auto store_v = [&](int st) {
    // 4 keys x 8 channels -> 8 rows of Vᵀ, each 4 keys (8 bytes): byte
    // permutes pick the low (even channel) or high (odd channel) halves.
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const unsigned e01 = __builtin_amdgcn_perm(vreg[1][m], vreg[0][m], 0x05040100u);
      const unsigned e23 = __builtin_amdgcn_perm(vreg[3][m], vreg[2][m], 0x05040100u);
      const unsigned o01 = __builtin_amdgcn_perm(vreg[1][m], vreg[0][m], 0x07060302u);
      const unsigned o23 = __builtin_amdgcn_perm(vreg[3][m], vreg[2][m], 0x07060302u);
      const int d0 = 8 * vdg + 2 * m;
      const int d1 = d0 + 1;
      Vs[st][d0 * (BN / 4) + (vkg ^ vsw(d0))] = u32x2{e01, e23};
      Vs[st][d1 * (BN / 4) + (vkg ^ vsw(d1))] = u32x2{o01, o23};
    }
    if (vdg == 0) kval[st][vkg] = vok;  // validity bytes of keys 4*vkg .. +3
  };
  auto qk = [&](int st, f32x16 (&s)[NKB]) {
    const f32x16 zero = {};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int r = kb * 32 + l32;
        const int ch = 2 * kk + half;
        const bf16x8 A = __builtin_bit_cast(bf16x8, Ks[st][r * CPR + (ch ^ (r & KSW))]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qreg[kk], kk == 0 ? zero : s[kb], 0, 0, 0);
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mc = -INFINITY;  // reference max, already multiplied by c
  float l_run = 0.f;
  const float c = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  f32x16 s[NKB], sn[NKB];
  int full_cur = 1;
  TileStream ks;  // the K stream, two tiles ahead of the tile being reduced
  stream_init<BN, MODE>(ks, a, list, cnt, 0);
  TileD tprev;  // descriptor of the tile whose K was loaded last (V follows one step later)
  if (ntiles > 0) {
    const TileD t0 = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    const TileD t1 = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    load_k(t0);
    load_v(t0);
    store_k(0);
    store_v(0);
    load_k(t1);
    store_k(1);
    full_cur = t0.full;
    tprev = t1;
  }
  __syncthreads();
  if (ntiles > 0) qk(0, s);
  __syncthreads();

  // One pipeline step: tile `it` is in `cur` (raw scores) and `nxt` receives tile it+1.
  auto step = [&](int it, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB]) {
    const int st = it & 1;
    // Global loads: K two tiles ahead, V one tile ahead (past the end they read zeros).
    const TileD tk = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    const TileD tv = tprev;
    tprev = tk;
    load_k(tk);
    load_v(tv);

    // Mask the invalid keys of tile i. Accumulator register r of block kb
    // holds key kb*32 + 8*(r/4) + 4*half + r%4 of the tile.
    if (!full_cur) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const unsigned f4 = kval[st][(kb * 32 + 8 * g + 4 * half) >> 2];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (((f4 >> (8 * i)) & 0xffu) == 0u) cur[kb][4 * g + i] = -INFINITY;
        }
    }

    // Sᵀ of tile i+1 on the matrix core while the VALU does the softmax of tile i.
    qk(st ^ 1, nxt);

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[kb][r]);
    mx = half_max(mx) * c;
    const bool need = mx > mc + kRescale;
    const float mc_new = need ? mx : mc;
    const float alpha = need ? __builtin_amdgcn_exp2f(mc - mc_new) : 1.f;
    mc = mc_new;
    l_run *= alpha;
    const float nm = (mc == -INFINITY) ? 0.f : -mc;

    // Pᵀ in the B-operand layout of Oᵀ += Vᵀ Pᵀ: step kk takes registers
    // 8*(kk%2) .. +7 of block kk/2, i.e. keys 16*kk + 8*(j/4) + 4*half + j%4.
    bf16x8 pb[PVSTEPS];
#pragma unroll
    for (int kk = 0; kk < PVSTEPS; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[kk >> 1][8 * (kk & 1) + j], c, nm));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[kk >> 1][8 * (kk & 1) + j + 1], c, nm));
        const bf16x2 p2 = {(__bf16)x0, (__bf16)x1};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_run, false);
        pb[kk][j] = p2[0];
        pb[kk][j + 1] = p2[1];
      }
    }
    // The rescale test waits for the row sum so the branch cannot split the
    // block above (l_run == l_run is false only for NaN).
    if (__ballot(need && (l_run == l_run)) != 0ull) {
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }

    // Oᵀ += Vᵀ Pᵀ. A operand: row d = 32*db + l32, keys of chunks 4*kk + half
    // and 4*kk + 2 + half (4 keys each).
#pragma unroll
    for (int kk = 0; kk < PVSTEPS; ++kk) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 32 + l32;
        const u32x2 lo = Vs[st][d * (BN / 4) + ((4 * kk + half) ^ vsw(d))];
        const u32x2 hi = Vs[st][d * (BN / 4) + ((4 * kk + 2 + half) ^ vsw(d))];
        const u32x4 A4 = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, A4), pb[kk], oacc[db], 0, 0, 0);
      }
    }

    // K of tile i+2 replaces K of tile i (read last iteration); V of tile i+1
    // replaces V of tile i-1 (read last iteration).
    store_k(st);
    store_v(st ^ 1);
    full_cur = tv.full;
    __syncthreads();
  };

  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(it, s, sn);
    step(it + 1, sn, s);
  }
  if (it < ntiles) step(it, s, sn);

  // Epilogue: combine the two half-waves' partial sums, normalise, store fp32.
  const float l_tot = half_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_in_blk) {
    float* orow = Oh + (size_t)qrow * D;
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


// ---------------------------------------------------------------------------
// d = 128: K and V tiles go from HBM straight into LDS (buffer loads with an
// LDS destination, 16 bytes per lane), so no VGPRs hold staged rows and no
// instructions write LDS; the Vᵀ operand of the PV product is read from the
// row-major V tile with ds_read_b64_tr_b16. In a group of 16 lanes that
// instruction gives lane j element j%4 of the 8 bytes read by lanes
// 4m + j/4 (m = 0..3): when lane i reads keys kb + i/4, channels
// dbase + 4*(i%4) .. +3, lane j receives channel dbase + j of keys kb..kb+3,
// which is exactly four k-slots of the MFMA A operand.
// LDS rows are 256 bytes (16 chunks of 16 bytes); chunk c of row r is stored
// at c ^ (r & 15) for K and at c ^ gv(r & 3), gv = {0, 4, 10, 14}, for V:
// both keep every read conflict-free with 32 and with 64 banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int gv_swz(int x) { return 4 * x + 2 * (x >> 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// SKIP: waves whose 32 rows hold no valid query (pad slots of reordered
// blocks) skip the math but still take their share of the loads and every
// barrier. Only instantiated for launches with per-block valid counts: the
// extra branch splits the loop body and costs the list walk some overlap.
// NW: waves per workgroup (32 query rows each). Four waves run two
// workgroups per CU; eight waves run one, and each K/V tile loaded into LDS
// then serves 256 query rows instead of 128.
template <int MODE, bool SKIP, int NW = 4>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bsa_fwd_d128_kernel(AttnArgs a) {
  static_assert(NW == 4 || (NW == 8 && (MODE == MODE_LIST || MODE == MODE_DENSE)), "eight waves: list or dense");
  constexpr int D = 128, BN = 64, KSTEPS = 8, NKB = 2, PVSTEPS = 4, NDB = 4;
  constexpr int BM = 32 * NW;      // query rows per workgroup
  constexpr int NJ = BN / 4 / NW;  // DMA instructions per wave per K or V tile
  constexpr int TILE = BN * D * 2;  // 16 KB per K or V tile
  // Four separate LDS objects (K and V of two stages) so the compiler can see
  // that reading one stage does not wait for the loads filling the other.
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char ks1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vs1[TILE];
  __shared__ unsigned int kval[2][BN / 4];
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
  if (a.block_valid) {
    int bv = a.block_valid[qb];
    qlim = bv < 0 ? 0 : (bv < qlim ? bv : qlim);
  }
  const int qend = min(blk_lo + qlim, blk_end);
  const int row_lo = blk_lo + qt * BM;
  int qrow = row_lo + wave * 32 + l32;
  bool active = !SKIP || row_lo + wave * 32 < qend;
  bool q_in_blk = qrow < blk_end;
  bool q_valid = qrow < qend;
  bool no_queries = row_lo >= qend;
  if (MODE == MODE_T2D) {
    // Query block qb is a raster pool tile; slot s = (s / pw, s % pw).
    const BlkGeom gq = blk_geom(a, qb);
    const int s0 = qt * BM;
    const int slot = s0 + wave * 32 + l32;
    const int hi = slot >> a.lpw, wi = slot & (a.pw - 1);
    q_valid = slot < a.block_q && hi < gq.vh && wi < gq.vw;
    q_in_blk = q_valid;
    qrow = q_valid ? gq.tok + hi * a.gW + wi : 0;
    active = !SKIP || ((s0 + wave * 32) >> a.lpw) < gq.vh;
    no_queries = (s0 >> a.lpw) >= gq.vh;
  }

  const size_t head_off = (size_t)h * (size_t)a.n * D;
  const int head_bytes = a.n * D * 2;
  const __amdgpu_buffer_rsrc_t Qr =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.q + head_off), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t Kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.k + head_off), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t Vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.v + head_off), (short)0, head_bytes, 0x00020000);
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

  bf16x8 qreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const unsigned off = q_valid ? (unsigned)((qrow * D + 16 * kk + 8 * half) * 2) : kInvalid;
    qreg[kk] = __builtin_bit_cast(bf16x8, bload(Qr, off));
  }

  // DMA roles: instruction j of wave `wave` fills tile rows 4*NW*j + 4*wave
  // .. +3; lane writes row 4*NW*j + dR, LDS chunk dp.
  const int dR = 4 * wave + (lane >> 4);
  const int dp = lane & 15;
  const unsigned kdma = (unsigned)(dR * 256 + 16 * (dp ^ (dR & 15)));
  const unsigned vdma = (unsigned)(dR * 256 + 16 * (dp ^ gv_swz(dR & 3)));

  // LDS read addresses (bytes inside a stage). K: row kb*32 + l32, chunk 2kk + half.
  unsigned kra[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) kra[kk] = (unsigned)(l32 * 256 + 16 * ((2 * kk + half) ^ (l32 & 15)));
  // Vᵀ via transpose reads: lane (group g = lane/16, i = lane%16) reads keys
  // 16kk + 8s + 4*(g/2) + i/4, channels 32db + 16*(g%2) + 4*(i%4) .. +3.
  const int ti = lane & 15, tg = lane >> 4;
  unsigned vra[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    vra[db] = (unsigned)((4 * (tg >> 1) + (ti >> 2)) * 256 +
                         16 * ((4 * db + 2 * (tg & 1) + ((ti & 3) >> 1)) ^ gv_swz(ti >> 2)) + 8 * (ti & 1));

  // A tile whose 64 rows are valid and are 4 runs of 16 consecutive rows of
  // K/V (one run per DMA instruction) loads with one scalar offset per run.
  // All BN rows valid and physically consecutive from base0: one run, or two
  // runs of adjacent blocks (then base1 == base0).
  auto simple = [&](const TileD& t) {
    return MODE == MODE_T2D ? (t.full && a.pw == 16) : (t.full && (t.bnd >= BN || t.base1 == t.base0));
  };
  const unsigned run_bytes = MODE == MODE_T2D ? (unsigned)a.gW * D * 2 : 1024u * NW;
  auto dma = [&](__amdgpu_buffer_rsrc_t r, int st, int kind, int j, unsigned voff, unsigned soff) {
    unsigned char* dst = (kind == 0 ? kbuf(st) : vbuf(st)) + 1024 * NW * j + 1024 * wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
  };
  auto load_k = [&](const TileD& t, int st) {
    if (simple(t)) {
      const unsigned so = (unsigned)(t.base0 * D * 2);
#pragma unroll
      for (int j = 0; j < NJ; ++j) dma(Kr, st, 0, j, kdma, so + run_bytes * j);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int R = 4 * NW * j + dR;
        const int p = tile_row<BN, MODE>(a, t, list, cnt, R);
        dma(Kr, st, 0, j, p >= 0 ? (unsigned)(p * 256 + 16 * (dp ^ (R & 15))) : kInvalid, 0u);
      }
    }
  };
  auto load_v = [&](const TileD& t, int st) {
    if (simple(t)) {
      const unsigned so = (unsigned)(t.base0 * D * 2);
#pragma unroll
      for (int j = 0; j < NJ; ++j) dma(Vr, st, 1, j, vdma, so + run_bytes * j);
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int R = 4 * NW * j + dR;
        const int p = tile_row<BN, MODE>(a, t, list, cnt, R);
        dma(Vr, st, 1, j, p >= 0 ? (unsigned)(p * 256 + 16 * (dp ^ gv_swz(R & 3))) : kInvalid, 0u);
        if (dp == 0) ((unsigned char*)kval[st])[R] = p >= 0 ? 1 : 0;
      }
    }
  };
  auto qk = [&](int st, f32x16 (&s)[NKB]) {
    const f32x16 zero = {};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, *(const u32x4*)(kbuf(st) + kb * 8192 + kra[kk]));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qreg[kk], kk == 0 ? zero : s[kb], 0, 0, 0);
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
  const float c = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // exp2(s*c - m) of a tile's scores, rounded to bf16 into the B operand of
  // the PV product; returns the lane's sum of the rounded values.
  auto probs = [&](const f32x16 (&cur)[NKB], float m, bf16x8 (&pb)[PVSTEPS]) {
    const float nm = (m == -INFINITY) ? 0.f : -m;
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < PVSTEPS; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[kk >> 1][8 * (kk & 1) + j], c, nm));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[kk >> 1][8 * (kk & 1) + j + 1], c, nm));
        const bf16x2 p2 = {(__bf16)x0, (__bf16)x1};
        if (kk & 1)
          t1 = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, t1, false);
        else
          t0 = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, t0, false);
        pb[kk][j] = p2[0];
        pb[kk][j + 1] = p2[1];
      }
    }
    return t0 + t1;
  };

  f32x16 s[NKB], sn[NKB];
  int full_cur = 1;
  TileStream ks;
  stream_init<BN, MODE>(ks, a, list, cnt, 0);
  TileD tprev;
  if (ntiles > 0) {
    const TileD t0 = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    const TileD t1 = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    load_k(t0, 0);
    load_v(t0, 0);
    load_k(t1, 1);
    full_cur = t0.full;
    tprev = t1;
  }
  wait_dma();
  __syncthreads();
  if (ntiles > 0 && active) qk(0, s);
  __syncthreads();

  auto step = [&](const int st, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB]) {
    // K of tile i+2 into the stage of tile i (its K was read last step);
    // V of tile i+1 into the other stage (its V was read last step).
    const TileD tk = stream_tile<BN, MODE>(ks, a, L);
    stream_next<BN, MODE>(ks, a, list, cnt);
    const TileD tv = tprev;
    tprev = tk;
    load_k(tk, st);
    load_v(tv, st ^ 1);

    if (active) {
      if (!full_cur) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const unsigned f4 = kval[st][(kb * 32 + 8 * g + 4 * half) >> 2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (((f4 >> (8 * i)) & 0xffu) == 0u) cur[kb][4 * g + i] = -INFINITY;
          }
      }

      // Probabilities against the running reference mc, with no row max:
      // a lane whose probabilities of this tile sum to more than kSumBf16
      // (or whose row has no reference yet) sends the wave through the
      // exact path, which moves mc to the row max, rescales and recomputes.
      bf16x8 pb[PVSTEPS];
      float tl;
      if (NW == 8 && wave >= 4) {
        // Eight waves: waves w and w + 4 share a SIMD and meet at the same
        // barriers. The upper four issue their 16 Sᵀ MFMAs first and the
        // softmax after them, so their VALU work runs beside the PV MFMAs
        // of the lower four, whose softmax runs beside these MFMAs.
        qk(st ^ 1, nxt);
        tl = probs(cur, mc, pb);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < 13) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x402, 200, 0);
      } else {
        qk(st ^ 1, nxt);
        tl = probs(cur, mc, pb);
        // Interleave the 16 Sᵀ MFMAs with their K reads (kept three ahead) and
        // the softmax VALU work, which does not depend on them: a wave overlaps
        // its own VALU work with its MFMAs only where the two are interleaved.
        // Four VALU instructions per MFMA with four waves; the lower waves of
        // an eight-wave workgroup take one (measured: 1.2-1.5 % faster than
        // four; two and three in between, none or the upper waves' order
        // slower).
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < 13) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, NW == 8 ? 1 : 4, 0);
        }
      }
      if (__ballot(!(tl <= kSumBf16) || mc == -INFINITY) != 0ull) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[kb][r]);
        mx = half_max(mx) * c;
        const float mc_new = fmaxf(mc, mx);
        const float alpha = mc_new == mc ? 1.f : __builtin_amdgcn_exp2f(mc - mc_new);
        mc = mc_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        tl = probs(cur, mc, pb);
      }
      l_run += tl;

#pragma unroll
      for (int kk = 0; kk < PVSTEPS; ++kk) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          lds_u8* const vb = (lds_u8*)vbuf(st) + vra[db] + 16 * kk * 256;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * 256));
          const s16x4 both[2] = {lo, hi};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pb[kk], oacc[db], 0, 0, 0);
        }
      }
      // Vᵀ reads run eight (four MFMAs) ahead of the PV MFMAs.
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }

    }

    full_cur = tv.full;
    wait_dma();
    __syncthreads();
  };

  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(0, s, sn);
    step(1, sn, s);
  }
  if (it < ntiles) step(0, s, sn);

  const float l_tot = half_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (MODE == MODE_T2D) {
    // Recompute the output row from an opaque copy of the lane id rather
    // than keep it live through the key walk.
    int lid = l32;
    asm volatile("" : "+v"(lid));
    const BlkGeom gq = blk_geom(a, qb);
    const int slot = qt * BM + wave * 32 + lid;
    const int hi = slot >> a.lpw, wi = slot & (a.pw - 1);
    q_valid = slot < a.block_q && hi < gq.vh && wi < gq.vw;
    q_in_blk = q_valid;
    qrow = q_valid ? gq.tok + hi * a.gW + wi : 0;
  }
  if (q_in_blk) {
    float* orow = Oh + (size_t)qrow * D;
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

template <int D, int BN>
hipError_t launch_mode(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.total_tiles), block(kThreads);
  if (a.dense)
    hipLaunchKernelGGL((bsa_fwd_bf16_kernel<D, BN, MODE_DENSE>), grid, block, 0, s, a);
  else if (a.block_k >= BN)
    hipLaunchKernelGGL((bsa_fwd_bf16_kernel<D, BN, MODE_LIST>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((bsa_fwd_bf16_kernel<D, BN, MODE_SMALL>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_d128(const AttnArgs& a, int waves, hipStream_t s) {
  dim3 grid(a.total_tiles), block(kThreads);
  if (waves == 8) {
    if (a.dense)
      hipLaunchKernelGGL((bsa_fwd_d128_kernel<MODE_DENSE, false, 8>), grid, dim3(512), 0, s, a);
    else if (a.block_k >= 64 && !a.block_valid)
      hipLaunchKernelGGL((bsa_fwd_d128_kernel<MODE_LIST, false, 8>), grid, dim3(512), 0, s, a);
    else
      return hipErrorInvalidValue;
  } else if (a.dense)
    hipLaunchKernelGGL((bsa_fwd_d128_kernel<MODE_DENSE, false>), grid, block, 0, s, a);
  else if (a.block_k >= 64 && a.block_valid)
    hipLaunchKernelGGL((bsa_fwd_d128_kernel<MODE_LIST, true>), grid, block, 0, s, a);
  else if (a.block_k >= 64)
    hipLaunchKernelGGL((bsa_fwd_d128_kernel<MODE_LIST, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((bsa_fwd_d128_kernel<MODE_SMALL, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_draft_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((bsa_fwd_d128_kernel<MODE_T2D, false>), dim3(a.total_tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, int d, hipStream_t s, int waves) {
  if (a.total_tiles == 0) return hipSuccess;
  if (waves != 4 && (waves != 8 || d != 128)) return hipErrorInvalidValue;
  return d == 128 ? launch_d128(a, waves, s) : launch_mode<64, 128>(a, s);
}

}  // namespace lvsa
