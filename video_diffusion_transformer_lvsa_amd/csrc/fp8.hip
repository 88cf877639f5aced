// Per-head FP8 (OCP E4M3) quantization of Q, K, V for the low-precision
// attention variant.
//
// The Draft Attention article (163.com) names quantization as the next step
// after its sparse mask; it fixes no format. Here: one scale per (tensor,
// head), scale = fl32(amax / 448) (1 when amax = 0), byte = E4M3 nearest to
// fl32(x / scale) with the quotient clamped to [-448, 448], ties to even
// (v_cvt_pk_fp8_f32 rounds to nearest even; it does not saturate, hence the
// clamp). V may be written transposed, [heads, d, ld] (ld >= n, a multiple of
// 16; bytes n .. ld-1 of a row are set to 0, so every byte of the operand is
// a finite code), which is the operand layout the attention's PV product reads.
#include "internal.h"

namespace lvsa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void fill_zero_kernel(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

__device__ __forceinline__ void load8(const void* src, size_t e, bool bf16, float (&x)[8]) {
  if (bf16) {
    const u32x4 v = *(const u32x4*)((const uint16_t*)src + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[i] << 16);
      x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
    const u32x4 a = *(const u32x4*)((const float*)src + e);
    const u32x4 b = *(const u32x4*)((const float*)src + e + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(a[i]);
      x[4 + i] = __uint_as_float(b[i]);
    }
  }
}

// amax[h] = max |x| over head h (as float bits: non-negative floats order as
// unsigned integers). Four 8-element loads in flight per thread, one atomic
// per workgroup. Grid: (blocks per head, heads).
template <bool BF16>
__global__ __launch_bounds__(256) void amax_kernel(const void* __restrict__ src, int per_head,
                                                   float* __restrict__ amax) {
  __shared__ float wmax[4];
  const int h = blockIdx.y;
  const size_t base = (size_t)h * per_head;
  const int stride = gridDim.x * 256 * 8;
  float m = 0.f;
  int e = (blockIdx.x * 256 + threadIdx.x) * 8;
  for (; e + 3 * stride < per_head; e += 4 * stride) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8(src, base + e + (size_t)u * stride, BF16, x[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[u][i]));
  }
  for (; e < per_head; e += stride) {
    float x[8];
    load8(src, base + e, BF16, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax((unsigned int*)&amax[h], __float_as_uint(m));
  }
}

__device__ __forceinline__ float head_scale(float amax) { return amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f; }

__device__ __forceinline__ unsigned int q4(const float* x, float s) {
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(__fdiv_rn(x[i], s), -448.f), 448.f);
  unsigned int w = 0u;
  w = (unsigned int)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], (int)w, false);
  w = (unsigned int)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)w, true);
  return w;
}

// Row-major codes, 16 elements per thread. Grid: (blocks per head, heads).
template <bool BF16>
__global__ __launch_bounds__(256) void quant_kernel(const void* __restrict__ src, int per_head,
                                                    const float* __restrict__ amax, uint8_t* __restrict__ dst) {
  const int h = blockIdx.y;
  const float s = head_scale(amax[h]);
  const size_t base = (size_t)h * per_head;
  for (int e = (blockIdx.x * 256 + threadIdx.x) * 16; e < per_head; e += gridDim.x * 256 * 16) {
    float x[16];
    load8(src, base + e, BF16, *(float(*)[8])x);
    load8(src, base + e + 8, BF16, *(float(*)[8])(x + 8));
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = q4(x + 4 * i, s);
    *(u32x4*)(dst + base + e) = w;
  }
}

// Transposed codes [heads, d, ld]: a workgroup quantizes 64 tokens x d
// channels through LDS. Grid: (ceil(n / 64), heads).
template <bool BF16>
__global__ __launch_bounds__(256) void quant_t_kernel(const void* __restrict__ src, int n, int d, int ld,
                                                      const float* __restrict__ amax, uint8_t* __restrict__ dst) {
  __shared__ uint8_t tile[128 * 64];  // [channel][token]
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  const float s = head_scale(amax[h]);
  const int cpr = d / 8;  // 8-channel chunks per token row
  for (int c = threadIdx.x; c < 64 * cpr; c += 256) {
    const int r = c / cpr, ch = (c - r * cpr) * 8;
    float x[8];
    if (t0 + r < n) {
      load8(src, ((size_t)h * n + t0 + r) * d + ch, BF16, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    const unsigned int w0 = q4(x, s), w1 = q4(x + 4, s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[(ch + i) * 64 + r] = (uint8_t)(w0 >> (8 * i));
      tile[(ch + 4 + i) * 64 + r] = (uint8_t)(w1 >> (8 * i));
    }
  }
  __syncthreads();
  const int full = min(64, n - t0);
  if (blockIdx.x == gridDim.x - 1) {  // row padding n .. ld-1
    const int padw = ld - n;
    for (int c = threadIdx.x; c < d * padw; c += 256) {
      const int ch = c / padw;
      dst[((size_t)h * d + ch) * ld + n + (c - ch * padw)] = 0;
    }
  }
  for (int c = threadIdx.x; c < d * 4; c += 256) {  // 16-byte pieces of each channel row
    const int ch = c >> 2, p = (c & 3) * 16;
    uint8_t* out = dst + ((size_t)h * d + ch) * ld + t0 + p;
    if (p + 16 <= full) {  // ld, t0 and p are multiples of 16
      *(u32x4*)out = *(const u32x4*)(tile + ch * 64 + p);
    } else {
      for (int i = 0; i < 16 && p + i < full; ++i) out[i] = tile[ch * 64 + p + i];
    }
  }
}

__global__ void scale_kernel(float* __restrict__ scales, int heads) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h < heads) scales[h] = head_scale(scales[h]);
}

}  // namespace

hipError_t launch_quantize_fp8(const void* src, int dt, int heads, int n, int d, bool transpose, int ld,
                               uint8_t* dst, float* scales, hipStream_t s) {
  const int per_head = n * d;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((heads + 255) / 256), dim3(256), 0, s, scales, heads);
  const int bph = max(1, min(512, (per_head + 256 * 64 - 1) / (256 * 64)));
  if (dt == 1)
    hipLaunchKernelGGL(amax_kernel<true>, dim3(bph, heads), dim3(256), 0, s, src, per_head, scales);
  else
    hipLaunchKernelGGL(amax_kernel<false>, dim3(bph, heads), dim3(256), 0, s, src, per_head, scales);
  if (n == 0) {
    // scales only
  } else if (transpose) {
    if (dt == 1)
      hipLaunchKernelGGL(quant_t_kernel<true>, dim3((n + 63) / 64, heads), dim3(256), 0, s, src, n, d, ld, scales,
                         dst);
    else
      hipLaunchKernelGGL(quant_t_kernel<false>, dim3((n + 63) / 64, heads), dim3(256), 0, s, src, n, d, ld, scales,
                         dst);
  } else {
    if (dt == 1)
      hipLaunchKernelGGL(quant_kernel<true>, dim3(bph * 4, heads), dim3(256), 0, s, src, per_head, scales, dst);
    else
      hipLaunchKernelGGL(quant_kernel<false>, dim3(bph * 4, heads), dim3(256), 0, s, src, per_head, scales, dst);
  }
  hipLaunchKernelGGL(scale_kernel, dim3((heads + 255) / 256), dim3(256), 0, s, scales, heads);
  return hipGetLastError();
}

}  // namespace lvsa
