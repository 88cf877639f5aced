// Tile walk shared by the attention kernels: the virtual key sequence over a
// query block's KV list, tile descriptors, list and block-geometry reads,
// half-wave reductions and buffer loads. Included by the kernel sources only.
#pragma once

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
constexpr unsigned kInvalid = 0x80000000u;  // byte offset past every buffer: loads return 0
constexpr float kRescale = 8.0f;            // log2 headroom before the reference max moves
constexpr float kSumBf16 = 65536.0f;        // bf16 d = 128: largest lane sum of a tile's probabilities
constexpr float kSumFp8 = 256.0f;           // FP8: the same, so that every probability is <= 2^8 < 448

enum { MODE_DENSE = 0, MODE_LIST = 1, MODE_SMALL = 2, MODE_T2D = 3, MODE_GRP = 4, MODE_T2DG = 5, MODE_TAIL = 6 };

// Where the BN virtual key rows of one tile live. Uniform across the workgroup.
// Row r < bnd is physical row base0 + r, row r >= bnd is base1 + r; row r is
// a valid key iff r < rmax and (r < v0 or bnd <= r < v1).
// MODE_T2D (a tile of a raster pool tile): bnd = pw; row r is token
// base0 + (r / pw) * W + r % pw, valid iff r < rmax, r / pw < v0 and
// r % pw < v1.
struct TileD {
  int vt0;
  int base0, base1, bnd, v0, v1, rmax;
  int full;
};

// Index data is read through the constant address space: it is not written
// during the kernel, and uniform reads then become scalar loads.
typedef const __attribute__((address_space(4))) int32_t cint32;
__device__ __forceinline__ int32_t cload(const int32_t* p, int i) { return ((cint32*)p)[i]; }

__device__ __forceinline__ int block_lim(const AttnArgs& a, int b) {
  if (b < 0 || b >= a.nkb) return 0;
  int lim = a.block_k;
  if (a.block_valid) {
    int bv = cload(a.block_valid, b);
    lim = bv < 0 ? 0 : (bv < lim ? bv : lim);
  }
  int rem = a.n - b * a.block_k;
  return rem < lim ? rem : lim;
}

__device__ __forceinline__ int list_entry(const AttnArgs& a, const int32_t* list, int cnt, int slot) {
  if (slot < 0 || slot >= cnt) return -1;
  int b = cload(list, slot);
  return (b < 0 || b >= a.nkb) ? -1 : b;
}

// Raster pool tile b = (t, hb, wb): its first token and valid rows/columns
// (0, 0, 0 for b < 0).
struct BlkGeom {
  int tok, vh, vw;
};
// x / m for small x, m >= 1 (block indices: x < 4096): the float quotient is
// within one of the exact one, which a single correction step fixes.
__device__ __forceinline__ int div_small(int x, int m, float inv_m) {
  int q = (int)((float)x * inv_m);
  q -= (q * m > x);
  q += ((q + 1) * m <= x);
  return q;
}

__device__ __forceinline__ BlkGeom blk_geom(const AttnArgs& a, int b) {
  BlkGeom g = {0, 0, 0};
  if (b < 0) return g;
  const int per = a.nbh * a.nbw;
  const int t = div_small(b, per, a.inv_per), rb = b - t * per;
  const int hb = div_small(rb, a.nbw, a.inv_nbw), wb = rb - hb * a.nbw;
  g.tok = (t * a.gH + hb * a.ph) * a.gW + wb * a.pw;
  g.vh = min(a.ph, a.gH - hb * a.ph);
  g.vw = min(a.pw, a.gW - wb * a.pw);
  return g;
}

// Walks the tiles of one key list in order. Advancing by one tile costs a
// few scalar operations; only positioning at a start tile divides.
struct TileStream {
  int vt0;          // first virtual row of the current tile
  int slot, off;    // list slot of vt0 and the offset inside it
  int blk0, lim0;   // KV block of that slot and its valid rows
  int blk1, lim1;   // the same for the next slot
  int r0;           // MODE_T2D: first tile row of the current tile
  BlkGeom g0;       // MODE_T2D: geometry of blk0
};

template <int BN, int MODE>
__device__ __forceinline__ void stream_init(TileStream& ts, const AttnArgs& a, const int32_t* list, int cnt, int it) {
  ts.vt0 = it * BN;
  ts.slot = ts.off = 0;
  ts.blk0 = ts.blk1 = -1;
  ts.lim0 = ts.lim1 = 0;
  if (MODE == MODE_LIST || MODE == MODE_T2D) {
    ts.slot = ts.vt0 / a.block_k;
    ts.off = ts.vt0 - ts.slot * a.block_k;
    ts.blk0 = list_entry(a, list, cnt, ts.slot);
    ts.blk1 = list_entry(a, list, cnt, ts.slot + 1);
  }
  if (MODE == MODE_LIST) {
    ts.lim0 = block_lim(a, ts.blk0);
    ts.lim1 = block_lim(a, ts.blk1);
  }
  if (MODE == MODE_T2D) {
    ts.r0 = ts.off >> a.lpw;
    ts.g0 = blk_geom(a, ts.blk0);
  }
}

template <int BN, int MODE>
__device__ __forceinline__ void stream_next(TileStream& ts, const AttnArgs& a, const int32_t* list, int cnt) {
  ts.vt0 += BN;
  if (MODE == MODE_LIST) {
    ts.off += BN;
    if (ts.off >= a.block_k) {  // block_k >= BN: at most one slot per tile
      ts.off -= a.block_k;
      ts.slot += 1;
      ts.blk0 = ts.blk1;
      ts.lim0 = ts.lim1;
      ts.blk1 = list_entry(a, list, cnt, ts.slot + 1);
      ts.lim1 = block_lim(a, ts.blk1);
    }
  }
  if (MODE == MODE_T2D) {
    ts.off += BN;
    ts.r0 += a.rpt;
    if (ts.off >= a.block_k) {  // block_k is a multiple of BN: the tile starts the next slot
      ts.off = 0;
      ts.r0 = 0;
      ts.slot += 1;
      ts.blk0 = ts.blk1;
      ts.g0 = blk_geom(a, ts.blk0);
      ts.blk1 = list_entry(a, list, cnt, ts.slot + 1);
    }
  }
}

template <int BN, int MODE>
__device__ __forceinline__ TileD stream_tile(const TileStream& ts, const AttnArgs& a, int L) {
  TileD t;
  t.vt0 = ts.vt0;
  t.rmax = L - ts.vt0;
  if (MODE == MODE_DENSE) {
    t.base0 = t.base1 = ts.vt0;
    t.bnd = BN;
    t.v0 = t.rmax;
    t.v1 = 0;
    t.full = t.rmax >= BN;
  } else if (MODE == MODE_LIST) {
    t.bnd = a.block_k - ts.off;
    t.base0 = ts.blk0 * a.block_k + ts.off;
    t.base1 = ts.blk1 * a.block_k - t.bnd;
    t.v0 = min(t.bnd, ts.lim0 - ts.off);
    t.v1 = t.bnd + ts.lim1;
    t.full = t.rmax >= BN && t.v0 >= min(t.bnd, BN) && (t.bnd >= BN || t.v1 >= BN);
  } else if (MODE == MODE_T2D) {
    t.bnd = a.pw;
    t.base0 = ts.g0.tok + ts.r0 * a.gW;
    t.base1 = 0;
    t.v0 = max(0, min(a.rpt, ts.g0.vh - ts.r0));
    t.v1 = ts.g0.vw;
    t.full = t.rmax >= BN && t.v0 == a.rpt && t.v1 == a.pw;
  } else {
    t.base0 = t.base1 = t.bnd = t.v0 = t.v1 = 0;
    t.full = 0;
  }
  return t;
}

// ---------------------------------------------------------------------------
// Compacted key walk in 16-row groups (MODE_GRP: lists over blocks with
// per-block valid counts; MODE_T2DG: raster pool tiles 16 tokens wide). A
// listed block contributes its valid rows only, as groups of up to 16
// consecutive physical rows: MODE_GRP rows 16g .. 16g+15 of the block (the
// last group of a block may be short), MODE_T2DG pool row g (its valid
// columns). A 64-key tile is four consecutive groups, so the empty part of a
// partly valid block costs no tile. The order of the keys is the list order,
// then the row order inside a block: the reordered and the raster layout of
// the same pool tiles produce the same tiles.
// ---------------------------------------------------------------------------
struct GTile {
  int base[4];  // first physical row of group j
  int nv[4];    // valid rows of group j (0 .. 16)
  int wm[4];    // MODE_TAIL: bit w set if the keys of group j are keys of wave w
  int full;     // every group has 16 valid rows (MODE_TAIL: and is wanted by every wave)
};

// Physical row of tile row r, or -1 if r is not a valid key.
template <int BN, int MODE>
__device__ __forceinline__ int tile_row(const AttnArgs& a, const TileD& t, const int32_t* list, int cnt, int r) {
  if (MODE == MODE_SMALL) {
    const int vj = t.vt0 + r;
    if (r >= t.rmax) return -1;
    const int slot = vj / a.block_k;
    const int off = vj - slot * a.block_k;
    const int blk = list_entry(a, list, cnt, slot);
    return off < block_lim(a, blk) ? blk * a.block_k + off : -1;
  }
  if (MODE == MODE_T2D) {
    const int hi = r >> a.lpw, wi = r & (t.bnd - 1);
    const bool ok2 = (r < t.rmax) & (hi < t.v0) & (wi < t.v1);
    return ok2 ? t.base0 + hi * a.gW + wi : -1;
  }
  const bool ok = (r < t.rmax) & ((r < t.v0) | ((r >= t.bnd) & (r < t.v1)));
  const int p = (r < t.bnd ? t.base0 : t.base1) + r;
  return ok ? p : -1;
}

// Both half-waves end with f(x[l], x[l ^ 32]).
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

}  // namespace
}  // namespace lvsa
