// Block-sparse softmax attention forward with a compacted key walk, bf16 in,
// fp32 out, d = 128, on the gfx950 matrix cores: Draft Attention's block
// lists, and the short last tile of LVSA frames.
//
// What it computes: every query row of a query block attends to the valid
// keys of the KV blocks listed for it, O = softmax(scale * Q Kᵀ) V over those
// keys only. MODE_GRP and MODE_T2DG: Draft Attention's block-sparse execution
// (the article's block-size and reorder paragraphs) on the reordered tokens
// (blocks with per-block valid counts) or in place on the raster [t, h, w]
// layout where a block is a pool tile 16 tokens wide. MODE_TAIL: the rows of
// LVSA frames ("LVSA: Training-Free Sparse Attention for Long Video
// Diffusion", §2: a frame's queries attend to the frames of its attend set)
// past their last full 128-row tile (24 of the 1560 rows of a Wan frame);
// the full tiles are the work of bsa_fwd_d128_kernel. A workgroup takes the
// tails of four consecutive frames, one wave each, and walks the union of
// their lists once (the lists of neighbouring frames share most entries);
// each key carries the bits of the waves whose list holds it, and a wave
// masks the others. A frame's tail alone in a 128-row workgroup cost 6.5 %
// of the LVSA time for 1.5 % of the rows.
//
// Same algorithm, LDS layouts, operand layouts and software pipeline as
// bsa_fwd_d128_kernel (attn_bf16.hip, whose header describes them), with two
// differences:
//  * The key walk lists each block's valid rows only, as groups of up to 16
//    consecutive physical rows, and a 64-key tile is four consecutive groups
//    (attn_tiles.h, GTile), so the empty part of a partly valid edge block
//    costs no tile. One DMA instruction loads one group with a scalar base
//    offset. Both layouts produce the same groups in the same order, so the
//    reorder and raster paths agree bit for bit.
//  * The workgroup first turns its key list into an LDS table (first row or
//    token and valid extent per slot, all threads at once; lists of up to
//    kGrpMaxSlots slots), and the walk reads the entry of the next slot from
//    it one slot ahead. Reading the list and the block geometry with scalar
//    loads at every slot change, and once more over the whole list to size
//    the walk, left two dependent load latencies per slot in the step
//    (measured: 1.5 % slower on the reorder path, 3 % on the raster path).
//
// A kernel of its own so that the LVSA and dense launches keep their code:
// small changes of that kernel's instruction schedule were measured to lower
// its L2 hit rate on the 14B LVSA workload from 96 % to 46-58 % on most
// boxes, for reasons not found.
#include "attn_tiles.h"

namespace lvsa {
namespace {

__device__ __forceinline__ int gv_swz(int x) { return 4 * x + 2 * (x >> 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <int MODE, bool SKIP>
__global__ __launch_bounds__(kThreads, 2) void bsa_fwd_d128_grp_kernel(AttnArgs a) {
  constexpr int D = 128, BN = 64, KSTEPS = 8, NKB = 2, PVSTEPS = 4, NDB = 4;
  constexpr int TILE = BN * D * 2;  // 16 KB per K or V tile
  // Four separate LDS objects (K and V of two stages) so the compiler can see
  // that reading one stage does not wait for the loads filling the other.
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char ks1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vs1[TILE];
  __shared__ unsigned int kval[2][BN / 4];
  // The key list as a table of (first physical row or token, valid extent)
  // per slot, built once by all threads, so that the walk reads the next
  // slot from LDS instead of waiting on two dependent scalar loads.
  __shared__ int2 stab[kGrpMaxSlots];
  __shared__ int sgroups;
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
  static_assert(MODE == MODE_GRP || MODE == MODE_T2DG || MODE == MODE_TAIL, "compacted walk modes only");
  constexpr bool RASTER = MODE == MODE_T2DG;
  constexpr bool TAIL = MODE == MODE_TAIL;
  int qt, qb, h;
  if (TAIL) {
    // Workgroup = four consecutive query blocks of one head; wave w takes the
    // tail rows of block 4g + w.
    const int ng4 = (a.nqb + 3) >> 2;
    h = logical / ng4;
    qb = 4 * (logical - h * ng4) + wave;
    qt = 0;
  } else {
    qt = logical % a.tiles_per_qb;
    const int rest = logical / a.tiles_per_qb;
    qb = rest % a.nqb;
    h = rest / a.nqb;
  }
  if (RASTER) {
    // Raster Draft: consecutive workgroups (one XCD) take the same pool tile
    // of consecutive frames, whose top-k lists share more key blocks than
    // those of neighbouring tiles of one frame (measured: 1.2 % faster).
    const int per = a.nbh * a.nbw, nt = a.nqb / per;
    qb = (qb % nt) * per + qb / nt;
  }

  const int blk_lo = qb * a.block_q;
  const int blk_end = min(blk_lo + a.block_q, a.n);
  int qlim = a.block_q;
  if (!TAIL && a.block_valid) {
    int bv = a.block_valid[qb];
    qlim = bv < 0 ? 0 : (bv < qlim ? bv : qlim);
  }
  const int qend = min(blk_lo + qlim, blk_end);
  const int row_lo = blk_lo + qt * kBM;
  int qrow = row_lo + wave * 32 + l32;
  bool active = !SKIP || row_lo + wave * 32 < qend;
  bool q_in_blk = qrow < blk_end;
  bool q_valid = qrow < qend;
  bool no_queries = row_lo >= qend;
  if (RASTER) {
    // Query block qb is a raster pool tile; slot s = (s / pw, s % pw).
    const BlkGeom gq = blk_geom(a, qb);
    const int s0 = qt * kBM;
    const int slot = s0 + wave * 32 + l32;
    const int hi = slot >> a.lpw, wi = slot & (a.pw - 1);
    q_valid = slot < a.block_q && hi < gq.vh && wi < gq.vw;
    q_in_blk = q_valid;
    qrow = q_valid ? gq.tok + hi * a.gW + wi : 0;
    active = !SKIP || ((s0 + wave * 32) >> a.lpw) < gq.vh;
    no_queries = (s0 >> a.lpw) >= gq.vh;
  }
  if (TAIL) {
    // Rows past the block's last full 128-row tile (at most 32).
    const int tail_lo = (a.block_q >> 7) << 7;
    qrow = blk_lo + tail_lo + l32;
    q_valid = qb < a.nqb && l32 < a.block_q - tail_lo && qrow < a.n;
    q_in_blk = q_valid;
    active = qb < a.nqb;
    no_queries = false;
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

  const int mrow = (a.mask_heads > 1 ? h : 0) * a.nqb + qb;
  int cnt = 0;
  const int32_t* list = nullptr;
  if (!TAIL) {
    cnt = a.kv_cnt[mrow];
    cnt = cnt < 0 ? 0 : (cnt > a.max_kv ? a.max_kv : cnt);
    list = a.kv_idx + (size_t)mrow * a.max_kv;
  }
  // Slot table and the walk's length in groups. Slot info: MODE_GRP the
  // block's valid rows; MODE_T2DG valid columns | valid pool rows << 8
  // (columns <= 64); 0 for an invalid entry or an empty block.
  if (tid == 0) sgroups = 0;
  __syncthreads();
  if (TAIL) {
    // The union of the four lists as a multiset: the r-th occurrence of a
    // block in any list is one slot, wanted by every wave whose list holds
    // that block at least r + 1 times (info = valid rows | wave bits << 24).
    // Slots follow list 0 in its order, then what lists 1, 2, 3 add, in
    // theirs. Wave w reads list w, lane l its entries l and l + 64
    // (max_kv <= kTailMaxKv = 128: at most 512 slots, below the raw lists).
    int* const raw = reinterpret_cast<int*>(&stab[kGrpMaxSlots / 2]);  // [4][128]
    __shared__ int wcount[4][2];
    const int lj = tid >> 6, fj = (qb - wave) + lj;
    int cj = 0;
    if (fj < a.nqb) {
      cj = a.kv_cnt[(a.mask_heads > 1 ? h : 0) * a.nqb + fj];
      cj = cj < 0 ? 0 : (cj > a.max_kv ? a.max_kv : cj);
    }
    const int32_t* const lst = a.kv_idx + (size_t)((a.mask_heads > 1 ? h : 0) * a.nqb + fj) * a.max_kv;
    int bb[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int lp = lane + 64 * e;
      int b = -1;
      if (lp < cj) {
        b = lst[lp];
        b = (b < 0 || b >= a.nkb) ? -1 : b;
      }
      raw[128 * lj + lp] = b;
      bb[e] = b;
    }
    __syncthreads();
    bool own[2];
    int wbits[2];
    unsigned long long ob[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int lp = lane + 64 * e, b = bb[e];
      own[e] = false;
      wbits[e] = 0;
      if (b >= 0) {
        int r = 0;
        for (int pp = 0; pp < lp; ++pp) r += raw[128 * lj + pp] == b;
        own[e] = true;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          int c = 0;
          for (int pp = 0; pp < 128; ++pp) c += raw[128 * jj + pp] == b;
          if (c > r) {
            wbits[e] |= 1 << jj;
            if (jj < lj) own[e] = false;
          }
        }
      }
      ob[e] = __ballot(own[e]);
      if (lane == 0) wcount[lj][e] = __builtin_popcountll(ob[e]);
    }
    __syncthreads();
    int pos0 = 0;
    for (int jj = 0; jj < lj; ++jj) pos0 += wcount[jj][0] + wcount[jj][1];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (own[e]) {
        const int pos = pos0 + (e ? wcount[lj][0] : 0) + __builtin_popcountll(ob[e] & ((1ull << lane) - 1ull));
        const int lim = block_lim(a, bb[e]);
        stab[pos] = make_int2(bb[e] * a.block_k, lim > 0 ? (lim | (wbits[e] << 24)) : 0);
        if (lim > 0) atomicAdd(&sgroups, (lim + 15) >> 4);
      }
    }
    int total = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) total += wcount[jj][0] + wcount[jj][1];
    cnt = __builtin_amdgcn_readfirstlane(total);
  } else {
    int mine = 0;
    for (int sl = tid; sl < cnt; sl += kThreads) {
      const int b = list[sl];
      int base = 0, info = 0, ng = 0;
      if (b >= 0 && b < a.nkb) {
        if (MODE == MODE_GRP) {
          const int lim = block_lim(a, b);
          base = b * a.block_k;
          info = lim;
          ng = (lim + 15) >> 4;
        } else {
          const BlkGeom geo = blk_geom(a, b);
          base = geo.tok;
          info = geo.vw | (geo.vh << 8);
          ng = geo.vw > 0 ? geo.vh : 0;
        }
      }
      stab[sl] = make_int2(base, ng > 0 ? info : 0);
      mine += ng;
    }
    if (mine) atomicAdd(&sgroups, mine);
  }
  __syncthreads();
  const int L = no_queries ? 0 : 16 * __builtin_amdgcn_readfirstlane(sgroups);  // compacted key rows
  const int ntiles = (L + BN - 1) / BN;

  bf16x8 qreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const unsigned off = q_valid ? (unsigned)((qrow * D + 16 * kk + 8 * half) * 2) : kInvalid;
    qreg[kk] = __builtin_bit_cast(bf16x8, bload(Qr, off));
  }

  // DMA roles: instruction j of wave `wave` fills tile rows 16j + 4*wave .. +3;
  // lane writes row 16j + dR, LDS chunk dp.
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

  auto dma = [&](__amdgpu_buffer_rsrc_t r, int st, int kind, int j, unsigned voff, unsigned soff) {
    unsigned char* dst = (kind == 0 ? kbuf(st) : vbuf(st)) + 4096 * j + 1024 * wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
  };
  // Compacted walk: DMA instruction j fills group j (tile rows 16j .. 16j+15),
  // one scalar base per group; rows past a group's valid count read zeros.
  auto load_kg = [&](const GTile& t, int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma(Kr, st, 0, j, (t.full || dR < t.nv[j]) ? kdma : kInvalid, (unsigned)(t.base[j] * D * 2));
  };
  auto load_vg = [&](const GTile& t, int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = t.full || dR < t.nv[j];
      dma(Vr, st, 1, j, ok ? vdma : kInvalid, (unsigned)(t.base[j] * D * 2));
      // per-key flags of a masked tile: 1 for a valid key, or (MODE_TAIL) the
      // bits of the waves it belongs to
      if (!t.full && dp == 0) ((unsigned char*)kval[st])[16 * j + dR] = ok ? (TAIL ? t.wm[j] : 1) : 0;
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
  // The key walk: tile descriptors of the virtual sequence, or of the
  // compacted group sequence.
  // Group cursor: slot gslot (first row or token gbase, info ginfo, gng
  // groups), next group gg; the entry of slot gslot + 1 is read one slot ahead.
  auto slot_ng = [&](int info) {
    return MODE == MODE_GRP ? (info + 15) >> 4 : TAIL ? ((info & 0xFFFFFF) + 15) >> 4 : info >> 8;
  };
  auto rd_slot = [&](int sl) { return sl < cnt ? stab[sl] : make_int2(0, 0); };
  int gslot = 0, gg = 0, gng = 0, gbase = 0, ginfo = 0;
  int2 gpre = rd_slot(0);
  auto gadvance = [&]() {  // to the next slot with groups (gng = 0 past the end)
    do {
      gbase = __builtin_amdgcn_readfirstlane(gpre.x);
      ginfo = __builtin_amdgcn_readfirstlane(gpre.y);
      gng = slot_ng(ginfo);
      gpre = rd_slot(gslot + 1);
      ++gslot;
    } while (gng == 0 && gslot <= cnt);
    gg = 0;
  };
  gadvance();
  // MODE_TAIL: bits of the waves that have a frame
  const int tail_live = TAIL ? (1 << min(4, a.nqb - (qb - wave))) - 1 : 0;
  // Group j of the next tile is group g of the current slot.
  auto group = [&](GTile& t, int j, int g) {
    if (MODE == MODE_GRP) {
      t.base[j] = gbase + 16 * g;
      t.nv[j] = min(16, ginfo - 16 * g);
    } else if (TAIL) {
      t.base[j] = gbase + 16 * g;
      t.nv[j] = min(16, (ginfo & 0xFFFFFF) - 16 * g);
      t.wm[j] = (unsigned)ginfo >> 24;
    } else {
      t.base[j] = gbase + g * a.gW;
      t.nv[j] = min(16, ginfo & 255);
    }
  };
  auto next_tile = [&]() {
    GTile t;
    t.full = 1;
    if (gng - gg >= 4) {
      // All four groups from the current slot: no per-group slot test
      // (measured: Draft 1.6-1.9 % faster than the per-group walk alone).
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        group(t, j, gg + j);
        t.full &= (t.nv[j] == 16);
      }
      gg += 4;
      if (gg == gng) gadvance();
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (gng == 0) {
          t.base[j] = 0;
          t.nv[j] = 0;
          if (TAIL) t.wm[j] = 0;
        } else {
          group(t, j, gg);
          if (++gg == gng) gadvance();
        }
        t.full &= (t.nv[j] == 16);
      }
    }
    // MODE_TAIL: a tile needs the per-wave key masks unless every group is
    // wanted by every wave that has a frame
    if (TAIL) t.full = t.full && (t.wm[0] & t.wm[1] & t.wm[2] & t.wm[3]) == tail_live;
    return t;
  };
  GTile tprev;
  if (ntiles > 0) {
    const auto t0 = next_tile();
    const auto t1 = next_tile();
    load_kg(t0, 0);
    load_vg(t0, 0);
    load_kg(t1, 1);
    full_cur = t0.full;
    tprev = t1;
  }
  wait_dma();
  __syncthreads();
  if (ntiles > 0 && active) qk(0, s);
  __syncthreads();

  const unsigned wbit = TAIL ? (1u << wave) : 0xffu;  // key flag bits that make a key valid for this wave
  auto step = [&](const int st, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB]) {
    // K of tile i+2 into the stage of tile i (its K was read last step);
    // V of tile i+1 into the other stage (its V was read last step).
    const auto tk = next_tile();
    const auto tv = tprev;
    tprev = tk;
    load_kg(tk, st);
    load_vg(tv, st ^ 1);

    if (active) {
      if (!full_cur) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const unsigned f4 = kval[st][(kb * 32 + 8 * g + 4 * half) >> 2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (((f4 >> (8 * i)) & wbit) == 0u) cur[kb][4 * g + i] = -INFINITY;
          }
      }

      qk(st ^ 1, nxt);

      // Probabilities against the running reference mc, with no row max:
      // a lane whose probabilities of this tile sum to more than kSumBf16
      // (or whose row has no reference yet) sends the wave through the
      // exact path, which moves mc to the row max, rescales and recomputes.
      bf16x8 pb[PVSTEPS];
      float tl = probs(cur, mc, pb);
      // Interleave the 16 Sᵀ MFMAs with their K reads (kept three ahead) and
      // the softmax VALU work, which does not depend on them: a wave overlaps
      // its own VALU work with its MFMAs only where the two are interleaved.
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 13) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
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
  if (RASTER) {
    // Recompute the output row from an opaque copy of the lane id rather
    // than keep it live through the key walk.
    int lid = l32;
    asm volatile("" : "+v"(lid));
    const BlkGeom gq = blk_geom(a, qb);
    const int slot = qt * kBM + wave * 32 + lid;
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

}  // namespace

hipError_t launch_lvsa_tail_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((bsa_fwd_d128_grp_kernel<MODE_TAIL, true>), dim3(a.total_tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grp_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.total_tiles == 0) return hipSuccess;
  if (a.tile2d)
    hipLaunchKernelGGL((bsa_fwd_d128_grp_kernel<MODE_T2DG, false>), dim3(a.total_tiles), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bsa_fwd_d128_grp_kernel<MODE_GRP, true>), dim3(a.total_tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lvsa
