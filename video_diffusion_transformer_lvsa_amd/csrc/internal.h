// Internal declarations shared by the host API (api.cpp) and the kernel
// translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lvsa {

// Arguments of one attention launch (block-sparse or dense). Pointers are
// device pointers; sizes were validated on the host.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  int heads;
  int n;             // tokens per head
  int block_q;       // query block size (rows)
  int block_k;       // KV block size (rows)
  int nqb;           // ceil(n / block_q)
  int nkb;           // ceil(n / block_k)
  int tiles_per_qb;  // ceil(block_q / BM) for the kernel's BM
  int total_tiles;   // heads * nqb * tiles_per_qb
  const int32_t* kv_idx;       // [mask_heads, nqb, max_kv] or NULL (dense)
  const int32_t* kv_cnt;       // [mask_heads, nqb] or NULL (dense)
  int max_kv;
  int mask_heads;
  const int32_t* block_valid;  // [nkb] or NULL
  float scale_log2;            // softmax scale * log2(e)
  float scale;                 // softmax scale
  int dense;                   // 1: every query sees all n keys
  // Blocks as pool_h x pool_w tiles of a [T, H, W] raster grid (draft_attn_fwd;
  // tile2d = 0 otherwise): block b = (t, hb, wb) in raster order, block_q =
  // block_k = ph*pw slots, slot s = (s / pw, s % pw) inside the tile.
  int tile2d;
  int gH, gW, ph, pw, nbh, nbw;
  int rpt;  // tile rows per 64-slot key tile (64 / pw)
  int lpw;  // log2(pw): pw divides 64
  float inv_per, inv_nbw;  // 1 / (nbh * nbw), 1 / nbw: block index -> (t, hb, wb)
  int ldv;                 // FP8 kernel: row pitch in bytes of the transposed V, [heads, d, ldv]
};

// Query rows per workgroup of the bf16 MFMA kernel and of the fp32 kernel.
constexpr int kBM_BF16 = 128;
constexpr int kBM_F32 = 64;

// waves = 8 (d = 128; dense, or lists without block_valid): 256 query rows
// per workgroup, so a.tiles_per_qb = ceil(block_q / 256).
hipError_t launch_attn_bf16(const AttnArgs& a, int d, hipStream_t s, int waves = 4);
// Draft attention on the raster layout (d = 128, bf16): a.tile2d = 1.
hipError_t launch_draft_attn_bf16(const AttnArgs& a, hipStream_t s);
// d = 128 bf16 attention with the compacted key walk: lists over blocks with
// per-block valid counts (block_k >= 64, a multiple of 16), or the raster
// layout with pools 16 tokens wide (a.tile2d = 1).
hipError_t launch_grp_bf16(const AttnArgs& a, hipStream_t s);
// Longest key list (max_kv) launch_grp_bf16 accepts: its workgroups hold the
// list as an LDS table of this many slots.
constexpr int kGrpMaxSlots = 1024;
// The last rows of each query block that do not fill a 128-row tile, for
// lists shared by consecutive blocks (LVSA frames): one workgroup takes the
// tails of four consecutive blocks, one wave each, and walks the union of
// their lists once, each wave keeping the keys of its own list. The caller
// launches the kernels above for the full tiles only (a.tiles_per_qb =
// block_q / 128). Needs block_q == block_k, block_q % 128 in 1 .. 32, no
// block_valid, max_kv <= kTailMaxKv; a.total_tiles = heads * ceil(nqb / 4).
constexpr int kTailMaxKv = 128;
hipError_t launch_lvsa_tail_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, int d, hipStream_t s);
// E4M3 codes (q, k row-major [heads, n, 128], v transposed [heads, 128, a.ldv])
// with per-head dequantization factors qs, ks, vs (device arrays).
hipError_t launch_attn_fp8(const AttnArgs& a, const float* qs, const float* ks, const float* vs, hipStream_t s);
// Query rows per workgroup of the FP8 kernel for these arguments.
int fp8_rows_per_workgroup(const AttnArgs& a);
// FP8 Draft attention on the raster layout (a.tile2d = 1).
hipError_t launch_draft_attn_fp8(const AttnArgs& a, const float* qs, const float* ks, const float* vs,
                                 hipStream_t s);

hipError_t launch_lvsa_mask(int T, int C, int window, int T_per, int step, int32_t* kv_idx, int32_t* kv_cnt,
                            int cap, hipStream_t s);

struct DraftGeom {
  int T, H, W;         // grid
  int ph, pw, bs;      // pool tile and block size
  int nbh, nbw, nb;    // blocks per column/row, total
  int n, n_pad;        // tokens, padded tokens
};

hipError_t launch_draft_perm(const DraftGeom& g, int32_t* perm, int32_t* inv_perm, int32_t* block_valid,
                             hipStream_t s);
// Pools q and k (dtype 0 = f32, 1 = bf16; mean, or maximum when pool_max)
// into qbar/kbar and, when the *_perm pointers are non-NULL, writes the
// reordered tensors.
hipError_t launch_draft_pool_gather(const DraftGeom& g, int heads, int d, int dt, bool pool_max, const void* q, const void* k,
                                    const void* v, float* qbar, float* kbar, float* kbarT, void* q_perm,
                                    void* k_perm, void* v_perm, hipStream_t s);
hipError_t launch_draft_select(const float* qbar, const float* kbarT, int heads, int nb, int d, int topk,
                               int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s);
hipError_t launch_draft_scores(const float* qbar, const float* kbar, int heads, int nb_q, int nb_k, int d,
                               float* scores, hipStream_t s);
// Per-head E4M3 codes of src ([heads, n, d], dtype 0 = f32, 1 = bf16) into dst
// ([heads, n, d], or [heads, d, ld] when transpose: d <= 128, ld a multiple of
// 16, >= n); scales[h] receives the dequantization factor.
hipError_t launch_quantize_fp8(const void* src, int dt, int heads, int n, int d, bool transpose, int ld,
                               uint8_t* dst, float* scales, hipStream_t s);
// Size of the library-owned device scratch (one copy per GPU, held until the
// process ends) that draft_mask_and_perm_noalloc uses as its workspace.
constexpr size_t kScratchBytes = (size_t)48 << 20;
// Address of the current device's scratch (looked up once per device).
hipError_t scratch_address(void** out);

hipError_t launch_token_permute(const void* src, void* dst, int esize, int heads, int n_src, int n_dst, int d,
                                const int32_t* map, hipStream_t s);

}  // namespace lvsa
