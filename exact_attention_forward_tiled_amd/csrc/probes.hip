// Test-only probes (built into libattn_probes.so, never into libattn.so).
//
// Each probe runs one fixed-size wave (or a fixed grid for the rate probes)
// and writes raw per-lane results, so the tests can check on the host the
// register layouts the kernels rely on: MFMA operand / accumulator lane maps,
// the LDS transposing read, the half-wave swap, and the fp4 scaled MFMA.  All
// buffers are sized by the caller exactly as documented per function.

#include "common.h"

using namespace attn;

namespace {

// a, b: 64 lanes x 8 bf16 each; c: 64 lanes x 16 fp32.
__global__ void mfma_bf16_probe(const uint16_t* a, const uint16_t* b, float* c) {
  const int l = threadIdx.x;
  const bf16x8 av = as_bf16x8(*(const u32x4*)(a + 8 * l));
  const bf16x8 bv = as_bf16x8(*(const u32x4*)(b + 8 * l));
  f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, zero16(), 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) c[16 * l + i] = acc[i];
}

// out: 64 lanes x 4 u16.  LDS holds u16 values 0..1023 (value = element index);
// lane l reads the 8 bytes at element 4*l with the transposing read.
__global__ void tr16_probe(uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[1024];
  const int l = threadIdx.x;
  for (int i = l; i < 1024; i += 64) lds[i] = (uint16_t)i;
  __syncthreads();
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(lds + 4 * l));
#pragma unroll
  for (int i = 0; i < 4; ++i) out[4 * l + i] = (uint16_t)t[i];
}

// out: 64 lanes x 2 u32 (both results of the swap with x = lane id).
__global__ void permlane32_probe(uint32_t* out) {
  const uint32_t l = threadIdx.x;
  auto r = __builtin_amdgcn_permlane32_swap(l, l + 100u, false, false);
  out[2 * l] = r[0];
  out[2 * l + 1] = r[1];
}

// a, b: 64 lanes x 16 bytes of fp4 codes (32 per lane); sa, sb: 64 scale bytes;
// c: 64 lanes x 16 fp32.
__global__ void mfma_fp4_probe(const uint8_t* a, const uint8_t* b, const uint8_t* sa,
                               const uint8_t* sb, float* c) {
  const int l = threadIdx.x;
  const u32x4 a4 = *(const u32x4*)(a + 16 * l);
  const u32x4 b4 = *(const u32x4*)(b + 16 * l);
  i32x8 av = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
  i32x8 bv = {(int)b4[0], (int)b4[1], (int)b4[2], (int)b4[3], 0, 0, 0, 0};
  f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, zero16(), 4, 4, 0,
                                                                (int)sa[l], 0, (int)sb[l]);
#pragma unroll
  for (int i = 0; i < 16; ++i) c[16 * l + i] = acc[i];
}

// Throughput probe: every thread runs `iters` rounds of 8 independent chains.
// mode 0: v_exp_f32; 1: cubic exp2; 2: fma only.  out: one float per thread.
template <int MODE>
__global__ void rate_probe(float* out, int iters, float seed) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = seed * (float)(threadIdx.x + i) * 1e-6f - 1.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (MODE == 0) {
        x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.5f;
      } else if constexpr (MODE == 1) {
        float y = fmaxf(x[i], -126.0f);
        const float n = __builtin_floorf(y);
        const float f = y - n;
        const float p = __builtin_fmaf(f, __builtin_fmaf(f, __builtin_fmaf(f, 0.078f, 0.226f), 0.695f), 1.0f);
        x[i] = __int_as_float(__float_as_int(p) + ((int)n << 23)) - 1.5f;
      } else {
        x[i] = __builtin_fmaf(x[i], 0.999f, -0.5f);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int probe_mfma_bf16(const void* a, const void* b, float* c, void* stream) {
  hipLaunchKernelGGL(mfma_bf16_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint16_t*)a, (const uint16_t*)b, c);
  return (int)hipGetLastError();
}

int probe_tr16(void* out, void* stream) {
  hipLaunchKernelGGL(tr16_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (uint16_t*)out);
  return (int)hipGetLastError();
}

int probe_permlane32(void* out, void* stream) {
  hipLaunchKernelGGL(permlane32_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (uint32_t*)out);
  return (int)hipGetLastError();
}

int probe_mfma_fp4(const void* a, const void* b, const void* sa, const void* sb, float* c,
                   void* stream) {
  hipLaunchKernelGGL(mfma_fp4_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint8_t*)a, (const uint8_t*)b, (const uint8_t*)sa,
                     (const uint8_t*)sb, c);
  return (int)hipGetLastError();
}

// out must hold blocks * 256 floats.
int probe_rate(float* out, int blocks, int iters, int mode, void* stream) {
  if (blocks < 1 || iters < 1) return -1;
  if (mode == 0)
    hipLaunchKernelGGL(rate_probe<0>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 1.0f);
  else if (mode == 1)
    hipLaunchKernelGGL(rate_probe<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 1.0f);
  else
    hipLaunchKernelGGL(rate_probe<2>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 1.0f);
  return (int)hipGetLastError();
}

}  // extern "C"
