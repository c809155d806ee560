// MXFP4 path: input quantisation kernels and the Direct-P forward.
//
// Quantisation follows the OCP MX v1.0 rule for FP4 (E2M1 elements, one E8M0
// power-of-two scale per 32 elements); "Hardware-Aware FP4 FlashAttention-4",
// section "1. Direct-P para Inferencia Directa" (Selección de Formato), uses
// MXFP4's power-of-two block scales for P and V.

#include "common.h"
#include "launch.h"

namespace attn {
namespace {

// Shared exponent of a block: floor(log2(amax)) - 2, clamped to [-127, 127];
// 0 for an all-zero block.  Read straight from the fp32 exponent field.
__device__ __forceinline__ int block_exponent(float amax) {
  if (amax == 0.f) return 0;
  const int field = (__float_as_int(amax) >> 23) & 0xFF;
  const int e = (field == 0 ? -127 : field - 127) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E2M1 magnitude code of y >= 0: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to
// the even code, saturating.  Midpoints alternate between rounding down (tie to
// an even code below) and up (even code above).
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  return (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
         (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) +
         (uint32_t)(y > 5.0f);
}

__device__ __forceinline__ uint32_t encode(float x, int e) {
  const uint32_t mag = e2m1_code(__builtin_ldexpf(fabsf(x), -e));
  return (x < 0.f && mag != 0u) ? (mag | 8u) : mag;
}

__global__ void quantize_rows_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
                                     uint8_t* __restrict__ scales, long long nblocks) {
  const long long blk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  const f32x4* src = (const f32x4*)(x + blk * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 t = src[i];
    v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = block_exponent(amax);
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) word |= encode(v[8 * w + n], e) << (4 * n);
    out[w] = word;
  }
  *(u32x4*)(codes + blk * 16) = out;
  scales[blk] = (uint8_t)(e + 127);
}

__global__ void quantize_cols_t_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
                                       uint8_t* __restrict__ scales, int rows, int cols,
                                       long long total) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int nrb = rows / 32;
  const int col = (int)(t % cols);
  const long long rest = t / cols;
  const int rb = (int)(rest % nrb);
  const long long b = rest / nrb;
  const float* src = x + (b * rows + (long long)rb * 32) * cols + col;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = src[(long long)i * cols];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int e = block_exponent(amax);
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) word |= encode(v[8 * w + n], e) << (4 * n);
    out[w] = word;
  }
  const long long crow = b * cols + col;  // row of the transposed output
  uint8_t* dst = codes + crow * (rows / 2) + rb * 16;
  // rows/2 may not keep 16-byte alignment for every row; store word by word
  uint32_t* d32 = (uint32_t*)dst;
  d32[0] = out[0]; d32[1] = out[1]; d32[2] = out[2]; d32[3] = out[3];
  scales[crow * nrb + rb] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_quantize_rows(const float* x, uint8_t* codes, uint8_t* scales, long long rows,
                                int cols, void* stream) {
  const long long nblocks = rows * (cols / 32);
  const int threads = 256;
  const long long grid = (nblocks + threads - 1) / threads;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)grid), dim3(threads), 0,
                     (hipStream_t)stream, x, codes, scales, nblocks);
  return hipGetLastError();
}

hipError_t launch_quantize_cols_t(const float* x, uint8_t* codes, uint8_t* scales, int batch,
                                  int rows, int cols, void* stream) {
  const long long total = (long long)batch * (rows / 32) * cols;
  const int threads = 256;
  const long long grid = (total + threads - 1) / threads;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize_cols_t_kernel, dim3((unsigned)grid), dim3(threads), 0,
                     (hipStream_t)stream, x, codes, scales, rows, cols, total);
  return hipGetLastError();
}

hipError_t launch_fwd_mxfp4(const Mxfp4Args& a) {
  (void)a;
  return hipErrorNotSupported;
}

}  // namespace attn
