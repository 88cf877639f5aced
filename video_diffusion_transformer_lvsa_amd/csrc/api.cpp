// Host side of liblvsa.so: argument validation, error reporting and kernel
// dispatch for the C ABI declared in include/lvsa.h.
//
// Every entry point validates its arguments before touching the GPU and
// returns a negative lvsa_status with a thread-local message on failure; no
// C++ exception leaves this file.
#include "lvsa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_err() { g_err[0] = '\0'; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 1 = a gfx950 device is current, 0 = none.
std::mutex g_dev_mu;
int g_dev_ok[64];  // 0 unknown, 1 ok, -1 bad

int check_device() {
  int n = 0;
  const hipError_t ec = hipGetDeviceCount(&n);
  if (ec != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return fail(LVSA_EDEVICE, "no GPU visible to HIP (%s, %d devices)", hipGetErrorString(ec), n);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(LVSA_EDEVICE, "hipGetDevice failed");
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (dev >= 0 && dev < 64 && g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(LVSA_EDEVICE, "hipGetDeviceProperties failed");
    }
    g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (g_dev_ok[dev] < 0) return fail(LVSA_EDEVICE, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
  }
  if (dev >= 0 && dev < 64 && g_dev_ok[dev] < 0) return fail(LVSA_EDEVICE, "device %d is not gfx950", dev);
  return LVSA_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LVSA_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return LVSA_OK;
}

// |A(t)| for one query frame (same growth rule as the kernel).
int lvsa_set_size(int t, int T, int C, int window, int T_per, int step) {
  const int off = step % T_per;
  const int n_anchor = off < T ? (T - 1 - off) / T_per + 1 : 0;
  const int target = C < T ? C : T;
  const int base_k = window < T ? window : T;
  int lo = t, hi = t, k = 1;
  int count = n_anchor + ((t % T_per) == off ? 0 : 1);
  while (k < T && (k < base_k || count < target)) {
    int f;
    if (lo > 0 && (hi + 1 >= T || (t - (lo - 1)) <= (hi + 1 - t)))
      f = --lo;
    else
      f = ++hi;
    if ((f % T_per) != off) ++count;
    ++k;
  }
  return count;
}

constexpr int kMaxFrames = 1 << 16;

int check_lvsa_params(int T, int C, int window, int T_per, int step) {
  if (T < 1 || T > kMaxFrames) return fail(LVSA_EINVAL, "T=%d must be in [1, %d]", T, kMaxFrames);
  if (C < 1) return fail(LVSA_EINVAL, "C=%d must be >= 1", C);
  if (window < 1) return fail(LVSA_EINVAL, "window=%d must be >= 1", window);
  if (T_per < 1) return fail(LVSA_EINVAL, "T_per=%d must be >= 1", T_per);
  if (step < 0) return fail(LVSA_EINVAL, "step=%d must be >= 0", step);
  return LVSA_OK;
}

int geom(int T, int H, int W, int ph, int pw, lvsa::DraftGeom* g) {
  if (T < 1 || H < 1 || W < 1) return fail(LVSA_EINVAL, "grid %dx%dx%d must be positive", T, H, W);
  if (ph < 1 || pw < 1) return fail(LVSA_EINVAL, "pool %dx%d must be positive", ph, pw);
  const long long bs = (long long)ph * pw;
  if (bs > 1024) return fail(LVSA_EUNSUPPORTED, "block size pool_h*pool_w=%lld > 1024", bs);
  const long long nbh = (H + ph - 1) / ph, nbw = (W + pw - 1) / pw;
  const long long nb = (long long)T * nbh * nbw;
  const long long n = (long long)T * H * W;
  const long long n_pad = nb * bs;
  if (n_pad > (1ll << 30)) return fail(LVSA_EINVAL, "padded token count %lld too large", n_pad);
  g->T = T;
  g->H = H;
  g->W = W;
  g->ph = ph;
  g->pw = pw;
  g->bs = (int)bs;
  g->nbh = (int)nbh;
  g->nbw = (int)nbw;
  g->nb = (int)nb;
  g->n = (int)n;
  g->n_pad = (int)n_pad;
  return LVSA_OK;
}

int topk_for(double sparsity, int nb, int* k) {
  if (!(sparsity >= 0.0 && sparsity <= 1.0)) return fail(LVSA_EINVAL, "sparsity %g must be in [0, 1]", sparsity);
  volatile double x = (1.0 - sparsity) * (double)nb;  // two roundings, no contraction
  double kk = std::floor(x + 0.5);
  if (kk < 1) kk = 1;
  if (kk > nb) kk = nb;
  *k = (int)kk;
  return LVSA_OK;
}

int check_attn(const void* q, const void* k, const void* v, const float* o, int dt, int heads, int n, int d) {
  if (dt != LVSA_F32 && dt != LVSA_BF16) return fail(LVSA_EINVAL, "dtype %d unknown", dt);
  if (d != 64 && d != 128) return fail(LVSA_EUNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (heads < 0 || n < 0) return fail(LVSA_EINVAL, "heads=%d n=%d must be >= 0", heads, n);
  if ((long long)n * d >= (1ll << 30)) return fail(LVSA_EINVAL, "n*d=%lld exceeds 2^30", (long long)n * d);
  if (heads > 0 && n > 0) {
    if (!q || !k || !v || !o) return fail(LVSA_EINVAL, "q, k, v, o must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
      return fail(LVSA_EINVAL, "q, k, v, o must be 16-byte aligned");
  }
  return LVSA_OK;
}

int run_attn(lvsa::AttnArgs& a, int dt, int d, void* stream) {
  const int bm = dt == LVSA_BF16 ? lvsa::kBM_BF16 : lvsa::kBM_F32;
  a.tiles_per_qb = (a.block_q + bm - 1) / bm;
  // Block lists over blocks that end in a short tile (LVSA frames: 1560 rows
  // = 12 x 128 + 24): the full tiles in one launch, the short tails of four
  // consecutive blocks per workgroup in a second one.
  const int tail = a.block_q % lvsa::kBM_BF16;
  const bool split = dt == LVSA_BF16 && d == 128 && !a.dense && !a.block_valid && a.block_q == a.block_k &&
                     a.block_q > lvsa::kBM_BF16 && tail > 0 && tail <= 32 && a.max_kv <= lvsa::kTailMaxKv &&
                     a.block_k < (1 << 24);
  // Dense d = 128 bf16 attention, and blocks of an even number of full
  // 128-row tiles, run as 256-row workgroups of eight waves (each K/V tile in
  // LDS serves twice the query rows).
  const int waves = dt == LVSA_BF16 && d == 128 && (a.dense || (split && (a.block_q / lvsa::kBM_BF16) % 2 == 0)) ? 8 : 4;
  if (split)
    a.tiles_per_qb = a.block_q / (32 * waves);
  else if (waves == 8)
    a.tiles_per_qb = (a.block_q + 255) / 256;
  const long long total = (long long)a.heads * a.nqb * a.tiles_per_qb;
  if (total >= (1ll << 31)) return fail(LVSA_EINVAL, "too many query tiles (%lld)", total);
  a.total_tiles = (int)total;
  if (total == 0) return LVSA_OK;
  int rc = check_device();
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (split) {
    hipError_t e = lvsa::launch_attn_bf16(a, d, s, waves);
    if (e == hipSuccess) {
      lvsa::AttnArgs t = a;
      t.total_tiles = (int)((long long)a.heads * ((a.nqb + 3) / 4));
      e = lvsa::launch_lvsa_tail_bf16(t, s);
    }
    return launched(e, "attention launch");
  }
  // Block lists with per-block valid counts (Draft on reordered tokens) walk
  // only the valid rows of each block.
  const bool grp = dt == LVSA_BF16 && d == 128 && !a.dense && a.block_valid && a.block_q == a.block_k &&
                   a.block_k >= 64 && a.block_k % 16 == 0 && a.max_kv <= lvsa::kGrpMaxSlots;
  hipError_t e = grp ? lvsa::launch_grp_bf16(a, s)
                     : (dt == LVSA_BF16 ? lvsa::launch_attn_bf16(a, d, s, waves) : lvsa::launch_attn_f32(a, d, s));
  return launched(e, "attention launch");
}

int check_fp8_attn(const void* q8, const void* k8, const void* vt8, int ldv, const float* qs, const float* ks,
                   const float* vs, const float* o, int heads, int n, int d, float scale) {
  if (d != 128) return fail(LVSA_EUNSUPPORTED, "FP8 attention supports d = 128 (got %d)", d);
  if (heads < 0 || n < 0) return fail(LVSA_EINVAL, "heads=%d n=%d must be >= 0", heads, n);
  if (n % 4 != 0) return fail(LVSA_EUNSUPPORTED, "FP8 attention needs n a multiple of 4 (got %d)", n);
  if ((long long)n * d >= (1ll << 30)) return fail(LVSA_EINVAL, "n*d=%lld exceeds 2^30", (long long)n * d);
  if (ldv < n || ldv % 16 != 0) return fail(LVSA_EINVAL, "ldv=%d must be a multiple of 16 and >= n=%d", ldv, n);
  if ((long long)d * ldv >= (1ll << 31)) return fail(LVSA_EINVAL, "d*ldv exceeds 2^31");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(LVSA_EINVAL, "scale must be finite and positive");
  if (heads > 0 && n > 0) {
    if (!q8 || !k8 || !vt8 || !o || !qs || !ks || !vs)
      return fail(LVSA_EINVAL, "q8, k8, vt8, o and the scales must be non-NULL");
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(vt8) || !aligned16(o))
      return fail(LVSA_EINVAL, "q8, k8, vt8, o must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(qs) | reinterpret_cast<uintptr_t>(ks) | reinterpret_cast<uintptr_t>(vs)) & 3u)
      return fail(LVSA_EINVAL, "scales must be 4-byte aligned");
  }
  return LVSA_OK;
}

int run_fp8(lvsa::AttnArgs& a, const float* qs, const float* ks, const float* vs, void* stream) {
  const int bm = lvsa::fp8_rows_per_workgroup(a);
  a.tiles_per_qb = (a.block_q + bm - 1) / bm;
  const long long total = (long long)a.heads * a.nqb * a.tiles_per_qb;
  if (total >= (1ll << 31)) return fail(LVSA_EINVAL, "too many query tiles (%lld)", total);
  a.total_tiles = (int)total;
  if (total == 0) return LVSA_OK;
  int rc = check_device();
  if (rc) return rc;
  return launched(lvsa::launch_attn_fp8(a, qs, ks, vs, reinterpret_cast<hipStream_t>(stream)),
                  "FP8 attention launch");
}

}  // namespace

extern "C" {

const char* lvsa_last_error(void) { return g_err; }

const char* lvsa_version(void) { return "lvsa-mi355x 0.1 (gfx950)"; }

int lvsa_mask_capacity(int T, int C, int window, int T_per, int step) {
  clear_err();
  int rc = check_lvsa_params(T, C, window, T_per, step);
  if (rc) return rc;
  int cap = 1;
  for (int t = 0; t < T; ++t) {
    const int c = lvsa_set_size(t, T, C, window, T_per, step);
    if (c > cap) cap = c;
  }
  return cap;
}

int lvsa_mask(int T, int C, int window, int T_per, int step, int32_t* kv_idx, int32_t* kv_cnt, int cap,
              void* stream) {
  clear_err();
  int rc = check_lvsa_params(T, C, window, T_per, step);
  if (rc) return rc;
  if (!kv_idx || !kv_cnt) return fail(LVSA_EINVAL, "kv_idx and kv_cnt must be non-NULL");
  if (cap < 1) return fail(LVSA_EINVAL, "cap=%d must be >= 1", cap);
  const int need = lvsa_mask_capacity(T, C, window, T_per, step);
  if (need < 0) return need;
  if (cap < need) return fail(LVSA_ERANGE, "cap=%d < required %d", cap, need);
  rc = check_device();
  if (rc) return rc;
  return launched(lvsa::launch_lvsa_mask(T, C, window, T_per, step, kv_idx, kv_cnt, cap,
                                         reinterpret_cast<hipStream_t>(stream)),
                  "lvsa_mask launch");
}

int draft_grid_info(int T, int H, int grid_w, int pool_h, int pool_w, double sparsity, int* nb, int* n_pad,
                    int* block_size, int* k) {
  clear_err();
  lvsa::DraftGeom g;
  int rc = geom(T, H, grid_w, pool_h, pool_w, &g);
  if (rc) return rc;
  int kk = 0;
  rc = topk_for(sparsity, g.nb, &kk);
  if (rc) return rc;
  if (nb) *nb = g.nb;
  if (n_pad) *n_pad = g.n_pad;
  if (block_size) *block_size = g.bs;
  if (k) *k = kk;
  return LVSA_OK;
}

size_t draft_workspace_bytes(int heads, int T, int H, int grid_w, int d, int pool_h, int pool_w) {
  clear_err();
  lvsa::DraftGeom g;
  if (geom(T, H, grid_w, pool_h, pool_w, &g)) return 0;
  if (heads < 1 || d < 1) return 0;
  return 3 * (size_t)heads * g.nb * d * sizeof(float);
}

namespace {

// Shared by draft_mask_and_perm and its no-allocation variant: validation and
// the three launches. workspace == NULL means "use the library's scratch".
int draft_mask_impl(const void* q, const void* k, const void* v, int dt, int heads, int T, int H, int grid_w, int d,
                    int pool_h, int pool_w, double sparsity, int pool_mode, int32_t* kv_idx, int32_t* kv_cnt,
                    int32_t* perm, int32_t* inv_perm, int32_t* block_valid, void* q_perm, void* k_perm, void* v_perm,
                    void* workspace, size_t ws_bytes, bool own_scratch, void* stream) {
  if (dt != LVSA_F32 && dt != LVSA_BF16) return fail(LVSA_EINVAL, "dtype %d unknown", dt);
  if (d != 64 && d != 128) return fail(LVSA_EUNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (heads < 1) return fail(LVSA_EINVAL, "heads=%d must be >= 1", heads);
  if (pool_mode != LVSA_POOL_MEAN && pool_mode != LVSA_POOL_MAX) return fail(LVSA_EINVAL, "pool_mode %d unknown", pool_mode);
  lvsa::DraftGeom g;
  int rc = geom(T, H, grid_w, pool_h, pool_w, &g);
  if (rc) return rc;
  if (g.nb > 4096) return fail(LVSA_EUNSUPPORTED, "nb=%d > 4096 draft blocks", g.nb);
  if ((long long)g.n_pad * d >= (1ll << 31)) return fail(LVSA_EINVAL, "N_pad*d exceeds 2^31");
  int topk = 0;
  rc = topk_for(sparsity, g.nb, &topk);
  if (rc) return rc;
  if (!q || !k) return fail(LVSA_EINVAL, "q and k must be non-NULL");
  if (!kv_idx || !kv_cnt || !perm || !inv_perm || !block_valid)
    return fail(LVSA_EINVAL, "kv_idx, kv_cnt, perm, inv_perm, block_valid must be non-NULL");
  const int nperm = (q_perm != nullptr) + (k_perm != nullptr) + (v_perm != nullptr);
  if (nperm != 0 && nperm != 3) return fail(LVSA_EINVAL, "q_perm, k_perm, v_perm must be all NULL or all non-NULL");
  if (nperm == 3 && !v) return fail(LVSA_EINVAL, "v must be non-NULL when v_perm is given");
  if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || !aligned16(q_perm) || !aligned16(k_perm) ||
      !aligned16(v_perm) || !aligned16(workspace))
    return fail(LVSA_EINVAL, "tensors and workspace must be 16-byte aligned");
  const size_t need = 3 * (size_t)heads * g.nb * d * sizeof(float);
  if (own_scratch) {
    if (need > lvsa::kScratchBytes)
      return fail(LVSA_ENOMEM, "pooled Q, K need %zu bytes of scratch; the library holds %zu (heads*nb*d <= %zu)", need,
                  lvsa::kScratchBytes, lvsa::kScratchBytes / (3 * sizeof(float)));
  } else if (!workspace || ws_bytes < need) {
    return fail(LVSA_ENOMEM, "workspace %zu bytes < required %zu", ws_bytes, need);
  }
  rc = check_device();
  if (rc) return rc;
  if (own_scratch) {
    rc = launched(lvsa::scratch_address(&workspace), "scratch address lookup");
    if (rc) return rc;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* qbar = static_cast<float*>(workspace);
  float* kbar = qbar + (size_t)heads * g.nb * d;
  float* kbarT = kbar + (size_t)heads * g.nb * d;
  rc = launched(lvsa::launch_draft_perm(g, perm, inv_perm, block_valid, s), "draft perm launch");
  if (rc) return rc;
  rc = launched(lvsa::launch_draft_pool_gather(g, heads, d, dt, pool_mode == LVSA_POOL_MAX, q, k, v, qbar, kbar, kbarT,
                                               q_perm, k_perm, v_perm, s),
                "draft pool launch");
  if (rc) return rc;
  return launched(lvsa::launch_draft_select(qbar, kbarT, heads, g.nb, d, topk, kv_idx, kv_cnt, s),
                  "draft select launch");
}

}  // namespace

int draft_mask_and_perm(const void* q, const void* k, const void* v, int dt, int heads, int T, int H, int grid_w,
                        int d, int pool_h, int pool_w, double sparsity, int pool_mode, int32_t* kv_idx, int32_t* kv_cnt,
                        int32_t* perm, int32_t* inv_perm, int32_t* block_valid, void* q_perm, void* k_perm,
                        void* v_perm, void* workspace, size_t ws_bytes, void* stream) {
  clear_err();
  return draft_mask_impl(q, k, v, dt, heads, T, H, grid_w, d, pool_h, pool_w, sparsity, pool_mode, kv_idx, kv_cnt,
                         perm, inv_perm, block_valid, q_perm, k_perm, v_perm, workspace, ws_bytes, false, stream);
}

int draft_mask_and_perm_noalloc(const void* q, const void* k, const void* v, int dt, int heads, int T, int H,
                                int grid_w, int d, int pool_h, int pool_w, double sparsity, int pool_mode,
                                int32_t* kv_idx, int32_t* kv_cnt, int32_t* perm, int32_t* inv_perm,
                                int32_t* block_valid, void* q_perm, void* k_perm, void* v_perm, void* stream) {
  clear_err();
  return draft_mask_impl(q, k, v, dt, heads, T, H, grid_w, d, pool_h, pool_w, sparsity, pool_mode, kv_idx, kv_cnt,
                         perm, inv_perm, block_valid, q_perm, k_perm, v_perm, nullptr, 0, true, stream);
}

int draft_scores(const float* qbar, const float* kbar, int heads, int nb_q, int nb_k, int d, float* scores,
                 void* stream) {
  clear_err();
  if (heads < 0 || nb_q < 0 || nb_k < 0 || d < 1) return fail(LVSA_EINVAL, "bad sizes");
  if (nb_q > 65535 || heads > 65535) return fail(LVSA_EUNSUPPORTED, "nb_q and heads must be <= 65535");
  if ((long long)heads * nb_q * nb_k == 0) return LVSA_OK;
  if (!qbar || !kbar || !scores) return fail(LVSA_EINVAL, "qbar, kbar, scores must be non-NULL");
  if (!aligned16(qbar) || !aligned16(kbar) || !aligned16(scores)) return fail(LVSA_EINVAL, "pointers must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  return launched(lvsa::launch_draft_scores(qbar, kbar, heads, nb_q, nb_k, d, scores,
                                            reinterpret_cast<hipStream_t>(stream)),
                  "draft scores launch");
}

int token_permute(const void* src, void* dst, int dt, int heads, int n_src, int n_dst, int d,
                  const int32_t* dst_to_src, void* stream) {
  clear_err();
  if (dt != LVSA_F32 && dt != LVSA_BF16) return fail(LVSA_EINVAL, "dtype %d unknown", dt);
  const int esize = dt == LVSA_BF16 ? 2 : 4;
  if (heads < 0 || n_src < 0 || n_dst < 0 || d < 1) return fail(LVSA_EINVAL, "bad sizes");
  if ((d * esize) % 16 != 0 || d > 4096) return fail(LVSA_EUNSUPPORTED, "row of %d elements is not a multiple of 16 bytes", d);
  if ((long long)heads * n_dst == 0) return LVSA_OK;
  const long long cpr = (long long)d * esize / 16;
  if ((long long)n_src * cpr >= (1ll << 31) || (long long)n_dst * cpr >= (1ll << 31) ||
      (long long)heads * ((n_dst * cpr + 1023) / 1024) >= (1ll << 31))
    return fail(LVSA_EINVAL, "a head of %d or %d rows of %d elements exceeds 2^31 16-byte chunks", n_src, n_dst, d);
  if (!src || !dst || !dst_to_src) return fail(LVSA_EINVAL, "src, dst, dst_to_src must be non-NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(LVSA_EINVAL, "src and dst must be 16-byte aligned");
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  const size_t sb = (size_t)heads * n_src * d * esize, db = (size_t)heads * n_dst * d * esize;
  if (s0 < d0 + db && d0 < s0 + sb) return fail(LVSA_EINVAL, "src and dst overlap");
  int rc = check_device();
  if (rc) return rc;
  return launched(lvsa::launch_token_permute(src, dst, esize, heads, n_src, n_dst, d, dst_to_src,
                                             reinterpret_cast<hipStream_t>(stream)),
                  "token_permute launch");
}

int block_sparse_attn_fwd(const void* q, const void* k, const void* v, float* o, int dt, int heads, int n, int d,
                          int block_q, int block_k, const int32_t* kv_idx, const int32_t* kv_cnt, int max_kv,
                          int mask_heads, const int32_t* block_valid, float scale, void* stream) {
  clear_err();
  int rc = check_attn(q, k, v, o, dt, heads, n, d);
  if (rc) return rc;
  if (block_q < 1 || block_k < 1) return fail(LVSA_EINVAL, "block_q=%d block_k=%d must be >= 1", block_q, block_k);
  if (max_kv < 0) return fail(LVSA_EINVAL, "max_kv=%d must be >= 0", max_kv);
  if (mask_heads != 1 && mask_heads != heads) return fail(LVSA_EINVAL, "mask_heads=%d must be 1 or heads=%d", mask_heads, heads);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(LVSA_EINVAL, "scale must be finite and positive");
  if (block_valid && block_q != block_k) return fail(LVSA_EINVAL, "block_valid requires block_q == block_k");
  if (heads == 0 || n == 0) return LVSA_OK;
  if (!kv_cnt || (max_kv > 0 && !kv_idx)) return fail(LVSA_EINVAL, "kv_cnt (and kv_idx when max_kv > 0) must be non-NULL");
  const long long nqb = ((long long)n + block_q - 1) / block_q;
  const long long nkb = ((long long)n + block_k - 1) / block_k;
  if ((long long)nkb * block_k >= (1ll << 31) || (long long)max_kv * block_k >= (1ll << 31))
    return fail(LVSA_EINVAL, "key list spans more than 2^31 rows");
  lvsa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.heads = heads;
  a.n = n;
  a.block_q = block_q;
  a.block_k = block_k;
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.max_kv = max_kv;
  a.mask_heads = mask_heads;
  a.block_valid = block_valid;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dense = 0;
  return run_attn(a, dt, d, stream);
}

int draft_attn_fwd(const void* q, const void* k, const void* v, float* o, int dt, int heads, int T, int H,
                   int grid_w, int d, int pool_h, int pool_w, const int32_t* kv_idx, const int32_t* kv_cnt,
                   int max_kv, float scale, void* stream) {
  clear_err();
  lvsa::DraftGeom g;
  int rc = geom(T, H, grid_w, pool_h, pool_w, &g);
  if (rc) return rc;
  rc = check_attn(q, k, v, o, dt, heads, g.n, d);
  if (rc) return rc;
  if (dt != LVSA_BF16 || d != 128) return fail(LVSA_EUNSUPPORTED, "draft_attn_fwd supports bf16 with d = 128");
  if (g.bs % 64 != 0 || 64 % pool_w != 0)
    return fail(LVSA_EUNSUPPORTED, "pool %dx%d: pool_h*pool_w must be a multiple of 64 and pool_w must divide 64",
                pool_h, pool_w);
  if (max_kv < 0) return fail(LVSA_EINVAL, "max_kv=%d must be >= 0", max_kv);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(LVSA_EINVAL, "scale must be finite and positive");
  if (heads == 0) return LVSA_OK;
  if (!kv_cnt || (max_kv > 0 && !kv_idx)) return fail(LVSA_EINVAL, "kv_cnt (and kv_idx when max_kv > 0) must be non-NULL");
  if ((long long)max_kv * g.bs >= (1ll << 31)) return fail(LVSA_EINVAL, "key list spans more than 2^31 rows");
  lvsa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.heads = heads;
  a.n = g.n;
  a.block_q = g.bs;
  a.block_k = g.bs;
  a.nqb = g.nb;
  a.nkb = g.nb;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.max_kv = max_kv;
  a.mask_heads = heads;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.tile2d = 1;
  a.gH = H;
  a.gW = grid_w;
  a.ph = pool_h;
  a.pw = pool_w;
  a.nbh = g.nbh;
  a.nbw = g.nbw;
  a.rpt = 64 / pool_w;
  a.lpw = 0;
  while ((1 << a.lpw) < pool_w) ++a.lpw;
  a.inv_per = 1.0f / (float)(g.nbh * g.nbw);
  a.inv_nbw = 1.0f / (float)g.nbw;
  a.tiles_per_qb = (g.bs + lvsa::kBM_BF16 - 1) / lvsa::kBM_BF16;
  const long long total = (long long)heads * g.nb * a.tiles_per_qb;
  if (total >= (1ll << 31)) return fail(LVSA_EINVAL, "too many query tiles (%lld)", total);
  a.total_tiles = (int)total;
  rc = check_device();
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool grp = pool_w == 16 && max_kv <= lvsa::kGrpMaxSlots;
  return launched(grp ? lvsa::launch_grp_bf16(a, s) : lvsa::launch_draft_attn_bf16(a, s),
                  "draft attention launch");
}

int dense_attn_fwd(const void* q, const void* k, const void* v, float* o, int dt, int heads, int n, int d,
                   float scale, void* stream) {
  clear_err();
  int rc = check_attn(q, k, v, o, dt, heads, n, d);
  if (rc) return rc;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(LVSA_EINVAL, "scale must be finite and positive");
  if (heads == 0 || n == 0) return LVSA_OK;
  lvsa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.heads = heads;
  a.n = n;
  a.block_q = n;
  a.block_k = n;
  a.nqb = 1;
  a.nkb = 1;
  a.max_kv = 0;
  a.mask_heads = 1;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dense = 1;
  return run_attn(a, dt, d, stream);
}

int quantize_fp8_e4m3(const void* src, int dt, int heads, int n, int d, int transpose, int ld, uint8_t* dst,
                      float* scales, void* stream) {
  clear_err();
  if (dt != LVSA_F32 && dt != LVSA_BF16) return fail(LVSA_EINVAL, "dtype %d unknown", dt);
  if (d != 64 && d != 128) return fail(LVSA_EUNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (heads < 0 || n < 0) return fail(LVSA_EINVAL, "heads=%d n=%d must be >= 0", heads, n);
  if (heads > 65535) return fail(LVSA_EUNSUPPORTED, "heads=%d: at most 65535", heads);
  if ((long long)n * d >= (1ll << 30)) return fail(LVSA_EINVAL, "n*d=%lld exceeds 2^30", (long long)n * d);
  if (transpose != 0 && transpose != 1) return fail(LVSA_EINVAL, "transpose=%d must be 0 or 1", transpose);
  if (transpose) {
    if (ld < n || ld % 16 != 0) return fail(LVSA_EINVAL, "ld=%d must be a multiple of 16 and >= n=%d", ld, n);
    if ((long long)d * ld >= (1ll << 31)) return fail(LVSA_EINVAL, "d*ld exceeds 2^31");
  } else if (ld != 0) {
    return fail(LVSA_EINVAL, "ld=%d must be 0 when transpose = 0", ld);
  }
  if (heads == 0) return LVSA_OK;
  if (!scales || (n > 0 && (!src || !dst))) return fail(LVSA_EINVAL, "src, dst, scales must be non-NULL");
  if ((n > 0 && (!aligned16(src) || !aligned16(dst))) || (reinterpret_cast<uintptr_t>(scales) & 3u))
    return fail(LVSA_EINVAL, "src, dst must be 16-byte aligned and scales 4-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  return launched(lvsa::launch_quantize_fp8(src, dt, heads, n, d, transpose != 0, ld, dst, scales,
                                            reinterpret_cast<hipStream_t>(stream)),
                  "fp8 quantization launch");
}

int block_sparse_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, int ldv,
                              const float* q_scale, const float* k_scale, const float* v_scale, float* o, int heads,
                              int n, int d, int block_q, int block_k, const int32_t* kv_idx, const int32_t* kv_cnt,
                              int max_kv, int mask_heads, const int32_t* block_valid, float scale, void* stream) {
  clear_err();
  int rc = check_fp8_attn(q8, k8, vt8, ldv, q_scale, k_scale, v_scale, o, heads, n, d, scale);
  if (rc) return rc;
  if (block_q < 1 || block_k < 1) return fail(LVSA_EINVAL, "block_q=%d block_k=%d must be >= 1", block_q, block_k);
  if (block_k < 64 || block_k % 4 != 0)
    return fail(LVSA_EUNSUPPORTED, "block_k=%d: the FP8 kernel needs block_k >= 64 and a multiple of 4", block_k);
  if (max_kv < 0) return fail(LVSA_EINVAL, "max_kv=%d must be >= 0", max_kv);
  if (mask_heads != 1 && mask_heads != heads) return fail(LVSA_EINVAL, "mask_heads=%d must be 1 or heads=%d", mask_heads, heads);
  if (block_valid && block_q != block_k) return fail(LVSA_EINVAL, "block_valid requires block_q == block_k");
  if (heads == 0 || n == 0) return LVSA_OK;
  if (!kv_cnt || (max_kv > 0 && !kv_idx)) return fail(LVSA_EINVAL, "kv_cnt (and kv_idx when max_kv > 0) must be non-NULL");
  const long long nqb = ((long long)n + block_q - 1) / block_q;
  const long long nkb = ((long long)n + block_k - 1) / block_k;
  if ((long long)nkb * block_k >= (1ll << 31) || (long long)max_kv * block_k >= (1ll << 31))
    return fail(LVSA_EINVAL, "key list spans more than 2^31 rows");
  lvsa::AttnArgs a{};
  a.block_valid = block_valid;
  a.q = q8;
  a.k = k8;
  a.v = vt8;
  a.o = o;
  a.heads = heads;
  a.n = n;
  a.block_q = block_q;
  a.block_k = block_k;
  a.nqb = (int)nqb;
  a.nkb = (int)nkb;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.max_kv = max_kv;
  a.mask_heads = mask_heads;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.ldv = ldv;
  return run_fp8(a, q_scale, k_scale, v_scale, stream);
}

int dense_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, int ldv, const float* q_scale,
                       const float* k_scale, const float* v_scale, float* o, int heads, int n, int d, float scale,
                       void* stream) {
  clear_err();
  int rc = check_fp8_attn(q8, k8, vt8, ldv, q_scale, k_scale, v_scale, o, heads, n, d, scale);
  if (rc) return rc;
  if (heads == 0 || n == 0) return LVSA_OK;
  lvsa::AttnArgs a{};
  a.q = q8;
  a.k = k8;
  a.v = vt8;
  a.o = o;
  a.heads = heads;
  a.n = n;
  a.block_q = n;
  a.block_k = n;
  a.nqb = 1;
  a.nkb = 1;
  a.mask_heads = 1;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dense = 1;
  a.ldv = ldv;
  return run_fp8(a, q_scale, k_scale, v_scale, stream);
}

int draft_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, int ldv, const float* q_scale,
                       const float* k_scale, const float* v_scale, float* o, int heads, int T, int H, int grid_w,
                       int d, int pool_h, int pool_w, const int32_t* kv_idx, const int32_t* kv_cnt, int max_kv,
                       float scale, void* stream) {
  clear_err();
  lvsa::DraftGeom g;
  int rc = geom(T, H, grid_w, pool_h, pool_w, &g);
  if (rc) return rc;
  if (grid_w % 4 != 0) return fail(LVSA_EUNSUPPORTED, "FP8 Draft attention needs grid_w a multiple of 4 (got %d)", grid_w);
  rc = check_fp8_attn(q8, k8, vt8, ldv, q_scale, k_scale, v_scale, o, heads, g.n, d, scale);
  if (rc) return rc;
  if (g.bs % 64 != 0 || 64 % pool_w != 0 || pool_w < 4)
    return fail(LVSA_EUNSUPPORTED,
                "pool %dx%d: pool_h*pool_w must be a multiple of 64 and pool_w one of 4, 8, 16, 32, 64", pool_h,
                pool_w);
  if (max_kv < 0) return fail(LVSA_EINVAL, "max_kv=%d must be >= 0", max_kv);
  if (heads == 0) return LVSA_OK;
  if (!kv_cnt || (max_kv > 0 && !kv_idx)) return fail(LVSA_EINVAL, "kv_cnt (and kv_idx when max_kv > 0) must be non-NULL");
  if ((long long)max_kv * g.bs >= (1ll << 31)) return fail(LVSA_EINVAL, "key list spans more than 2^31 rows");
  lvsa::AttnArgs a{};
  a.q = q8;
  a.k = k8;
  a.v = vt8;
  a.o = o;
  a.heads = heads;
  a.n = g.n;
  a.block_q = g.bs;
  a.block_k = g.bs;
  a.nqb = g.nb;
  a.nkb = g.nb;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.max_kv = max_kv;
  a.mask_heads = heads;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.ldv = ldv;
  a.tile2d = 1;
  a.gH = H;
  a.gW = grid_w;
  a.ph = pool_h;
  a.pw = pool_w;
  a.nbh = g.nbh;
  a.nbw = g.nbw;
  a.rpt = 64 / pool_w;
  a.lpw = 0;
  while ((1 << a.lpw) < pool_w) ++a.lpw;
  a.inv_per = 1.0f / (float)(g.nbh * g.nbw);
  a.inv_nbw = 1.0f / (float)g.nbw;
  a.tiles_per_qb = (g.bs + lvsa::kBM_BF16 - 1) / lvsa::kBM_BF16;
  const long long total = (long long)heads * g.nb * a.tiles_per_qb;
  if (total >= (1ll << 31)) return fail(LVSA_EINVAL, "too many query tiles (%lld)", total);
  a.total_tiles = (int)total;
  rc = check_device();
  if (rc) return rc;
  return launched(lvsa::launch_draft_attn_fp8(a, q_scale, k_scale, v_scale, reinterpret_cast<hipStream_t>(stream)),
                  "FP8 Draft attention launch");
}

}  // extern "C"
