// Test-only probes (built into libattn_probes.so, never into libattn.so).
//
// Each probe runs one fixed-size wave (or a fixed grid for the rate probes)
// and writes raw per-lane results, so the tests can check on the host the
// register layouts the kernels rely on: MFMA operand / accumulator lane maps,
// the LDS transposing read, the half-wave swap, and the fp4 / fp8 scaled MFMA.  All
// buffers are sized by the caller exactly as documented per function.

#include "common.h"

using namespace attn;

namespace {

// One 512-thread workgroup per block, the attention kernels' shape: lane 0 of
// every wave records the HW_ID hardware register (SIMD id in bits 5:4, CU id in
// bits 11:8), out[block * 8 + wave].
__global__ void __launch_bounds__(512) wave_place_probe(uint32_t* out) {
  __shared__ uint32_t pad[16384];   // 64 KiB, as the attention kernels use
  const int wave = threadIdx.x >> 6;
  pad[threadIdx.x] = threadIdx.x;
  __syncthreads();
  const uint32_t id = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11)) + 0u * pad[threadIdx.x ^ 1];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 8 + wave] = id;
}

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
// Transposing LDS read probe: LDS word i (16 bits) holds i; lane l reads 8 bytes at word
// addr[l] (a multiple of 4, at most 1020) with ds_read_b64_tr_b16.  out: 64 lanes x 4 words.
__global__ void tr16_probe(const int* addr, uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[1024];
  const int l = threadIdx.x;
  for (int i = l; i < 1024; i += 64) lds[i] = (uint16_t)i;
  __syncthreads();
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const int a = addr[l] & 1020;   // in bounds whatever the caller passes
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(lds + a));
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


// MFMA issue-rate probe: 4 independent 32x32x16 bf16 accumulation chains per wave.
__global__ void mfma_rate_probe(float* out, int iters) {
  const int l = threadIdx.x & 63;
  u32x4 av = {(uint32_t)l, 1u, 2u, 3u}, bv = {3u, 2u, 1u, (uint32_t)l};
  const bf16x8 a = as_bf16x8(av), b = as_bf16x8(bv);
  f32x16 c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// MFMA / VALU co-issue probe: one block per CU (the 96 KiB LDS pad keeps a second one off),
// 256 threads (one wave per SIMD) or 512 (two).  Each wave runs `iters` rounds of 4
// v_mfma_f32_32x32x16_bf16 on 4 independent accumulators, each MFMA followed by V fp32 FMAs
// on 8 independent loop-carried chains.  The SIMD's cycles per (MFMA + V FMAs) over all its
// waves is the event-timed launch span times the clock, divided by its MFMAs.
// stats (2 x u64, summed atomically): shader-clock cycles and 100 MHz ticks of wave 0 of
// each block, whose ratio is the clock.
template <int V>
__global__ void __launch_bounds__(512) overlap_probe(float* __restrict__ out,
                                                     unsigned long long* __restrict__ stats,
                                                     int iters) {
  __shared__ float pad[24576];
  pad[threadIdx.x] = (float)threadIdx.x;
  const int l = threadIdx.x & 63;
  u32x4 av = {(uint32_t)l, 1u, 2u, 3u}, bv = {3u, 2u, 1u, (uint32_t)l};
  const bf16x8 a = as_bf16x8(av), b = as_bf16x8(bv);
  f32x16 c[4] = {zero16(), zero16(), zero16(), zero16()};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)(threadIdx.x + i) * 1e-3f;
  __syncthreads();
  const float y = 0.999f + 1e-9f * pad[threadIdx.x ^ 1], z = 1e-7f;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < V; ++v) x[v & 7] = __builtin_fmaf(x[v & 7], y, z);
    }
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) s += c[k][0] + c[k][15];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    atomicAdd(stats, c1 - c0);
    atomicAdd(stats + 1, r1 - r0);
  }
}

// Clock-under-load probe, in the attention kernels' shape: 512-thread blocks (8 waves, two
// per SIMD), one block per CU.  Each wave runs `iters` iterations of 8
// v_mfma_f32_32x32x16_bf16 on operands taken from random data (src: 2048 x 16 bytes):
//   MODE 0  operands cycle through 4 register-held pairs;
//   MODE 1  every A operand is read from LDS (ds_read_b128, 16 B per lane per MFMA, as the
//           attention kernel reads its K and V^T operands);
//   MODE 2  MODE 1 plus about 5 VALU instructions per MFMA (fma, exp, max, bf16 pack, add:
//           the softmax's share per MFMA).
// stats (2 x u64, summed atomically): shader-clock cycles and 100 MHz ticks over each
// block's lifetime (wave 0), whose ratio is the clock the block ran at.
template <int MODE>
__global__ void __launch_bounds__(512) power_probe(const u32x4* __restrict__ src,
                                                   float* __restrict__ out,
                                                   unsigned long long* __restrict__ stats,
                                                   int iters) {
  __shared__ u32x4 buf[2048];
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  for (int i = t; i < 2048; i += 512) buf[i] = src[i];
  __syncthreads();
  u32x4 a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a[k] = src[(64 * (w + k) + l) & 2047];
    b[k] = src[(64 * (w + k + 8) + l) & 2047];
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = zero16();
  float x = __uint_as_float(0x3f000000u | (src[l][0] & 0x7fffffu)), mx = 0.f, sum = 0.f;
  uint32_t pk = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const u32x4 av = MODE >= 1 ? buf[((it * 8 + u) * 64 + l) & 2047] : a[u & 3];
      acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(b[u & 3]),
                                                          acc[u & 3], 0, 0, 0);
      if constexpr (MODE == 2) {
        x = __builtin_fmaf(x, 0.999f, 0.0007f);
        const float e = __builtin_amdgcn_exp2f(-x);
        mx = fmaxf(mx, e);
        pk ^= pack_bf16x2(e, mx);
        sum += e;
      }
    }
  }
  float s = sum + mx + (float)(pk & 1u);
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i];
  out[blockIdx.x * 512 + t] = s;
  if (t == 0) {
    atomicAdd(stats, __builtin_amdgcn_s_memtime() - c0);
    atomicAdd(stats + 1, __builtin_amdgcn_s_memrealtime() - r0);
  }
}

// LDS access-pattern probe: one wave; lane l reads (WRITE = 0) or writes (WRITE = 1) the
// 16 bytes at byte offset addr[l] of a 32 KiB LDS buffer, `iters` times.  Run under the
// LDS bank-conflict counter, it gives the conflict cycles of one ds_read_b128 /
// ds_write_b128 with that lane-to-address map.  addr[l] must be a multiple of 16 below
// 32768 (the host checks).
template <int WRITE>
__global__ void __launch_bounds__(64) lds_pattern_probe(const uint32_t* __restrict__ addr,
                                                        float* __restrict__ out, int iters) {
  __shared__ u32x4 buf[2048];
  const int l = threadIdx.x;
  for (int i = l; i < 2048; i += 64) buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const uint32_t a = addr[l] >> 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
    if constexpr (WRITE) {
      buf[a] = u32x4{(uint32_t)it, (uint32_t)l, 0u, 0u};
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
      acc += buf[a];
      asm volatile("" ::"v"(acc));
    }
  }
  __syncthreads();
  out[l] = (float)(acc[0] + acc[1] + buf[l][0]);
}

// LDS read-rate probe: 256 threads, each wave reads 16 B (mode 0, ds_read_b128) or
// 8 B with the transposing read (mode 1) per lane per step from a 32 KiB buffer.
template <int MODE>
__global__ void lds_rate_probe(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) u32x4 buf[2048];
  const int t = threadIdx.x, l = t & 63;
  for (int i = t; i < 2048; i += blockDim.x) buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = ((it * 8 + u) * 64 + l) & 2047;
      if constexpr (MODE == 0) {
        acc += buf[idx];
      } else {
        typedef short i16x4 __attribute__((ext_vector_type(4)));
        i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)((uint16_t*)buf + idx * 4));
        acc[0] += (uint32_t)r[0]; acc[1] += (uint32_t)r[1];
        acc[2] += (uint32_t)r[2]; acc[3] += (uint32_t)r[3];
      }
    }
  }
  out[blockIdx.x * blockDim.x + t] = (float)(acc[0] + acc[1] + acc[2] + acc[3]);
}

// Direct-to-LDS load probe: one wave; lane l fetches the 16 bytes at global
// element 4*(63 - l) (u32 values = element index) with global_load_lds_dwordx4
// into a 1 KiB LDS block; the block is then copied out linearly.
// src: 256 u32; out: 256 u32.
__global__ void lds_dma_probe(const uint32_t* src, uint32_t* out) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[256];
  const int l = threadIdx.x;
  for (int i = l; i < 256; i += 64) lds[i] = 0xFFFFFFFFu;
  __syncthreads();
  __builtin_amdgcn_global_load_lds((const void*)(src + 4 * (63 - l)),
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int i = l; i < 256; i += 64) out[i] = lds[i];
}

// Rounding probe: lane i converts x[2i], x[2i+1] with the packed bf16 convert
// and accumulates their dot product with (1, 1) onto acc[i].
// x: 128 floats; acc: 64 floats; out: 64 x (u32 packed pair, f32 dot result).
__global__ void cvt_dot_probe(const float* x, const float* acc, uint32_t* out) {
  const int l = threadIdx.x;
  const uint32_t pk = pack_bf16x2(x[2 * l], x[2 * l + 1]);
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  const float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc[l], false);
  out[2 * l] = pk;
  out[2 * l + 1] = __float_as_uint(d);
}


// fp4 convert probe.  x: 64 lanes x 2 floats; scale: 64 floats; out: 64 lanes x 4 u32,
// out[4l + sel] = v_cvt_scalef32_pk_fp4_f32 of (x[2l], x[2l+1]) into byte `sel` of 0xFFFFFFFF.
__global__ void cvt_fp4_probe(const float* x, const float* scale, uint32_t* out) {
  const int l = threadIdx.x;
  const float a = x[2 * l], b = x[2 * l + 1], s = scale[l];
  out[4 * l + 0] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0xFFFFFFFFu, a, b, s, 0);
  out[4 * l + 1] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0xFFFFFFFFu, a, b, s, 1);
  out[4 * l + 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0xFFFFFFFFu, a, b, s, 2);
  out[4 * l + 3] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0xFFFFFFFFu, a, b, s, 3);
}

// fp4 decode probe.  src: 64 u32; scale: 64 floats; out: 64 lanes x 4 sels x 2 floats.
__global__ void dec_fp4_probe(const uint32_t* src, const float* scale, float* out) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const int l = threadIdx.x;
  const uint32_t v = src[l];
  const float s = scale[l];
  f2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, s, 0);
  f2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, s, 1);
  f2 d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, s, 2);
  f2 d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, s, 3);
  out[8 * l + 0] = d0[0]; out[8 * l + 1] = d0[1];
  out[8 * l + 2] = d1[0]; out[8 * l + 3] = d1[1];
  out[8 * l + 4] = d2[0]; out[8 * l + 5] = d2[1];
  out[8 * l + 6] = d3[0]; out[8 * l + 7] = d3[1];
}

// fp4 MFMA with 32-bit scale words and byte selection 2 for both operands.
// a, b: 64 lanes x 16 bytes; sa, sb: 64 u32; c: 64 lanes x 16 fp32.
__global__ void mfma_fp4_sel2_probe(const uint8_t* a, const uint8_t* b, const uint32_t* sa,
                                    const uint32_t* sb, float* c) {
  const int l = threadIdx.x;
  const u32x4 a4 = *(const u32x4*)(a + 16 * l);
  const u32x4 b4 = *(const u32x4*)(b + 16 * l);
  i32x8 av = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
  i32x8 bv = {(int)b4[0], (int)b4[1], (int)b4[2], (int)b4[3], 0, 0, 0, 0};
  f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, zero16(), 4, 4, 2,
                                                                (int)sa[l], 2, (int)sb[l]);
#pragma unroll
  for (int i = 0; i < 16; ++i) c[16 * l + i] = acc[i];
}

// fp8 (E4M3) scaled MFMA.  a, b: 64 lanes x 32 bytes of E4M3 codes; sa, sb: 64 scale
// bytes; c: 64 lanes x 16 fp32.
__global__ void mfma_fp8_probe(const uint8_t* a, const uint8_t* b, const uint8_t* sa,
                               const uint8_t* sb, float* c) {
  const int l = threadIdx.x;
  const u32x4 a0 = *(const u32x4*)(a + 32 * l), a1 = *(const u32x4*)(a + 32 * l + 16);
  const u32x4 b0 = *(const u32x4*)(b + 32 * l), b1 = *(const u32x4*)(b + 32 * l + 16);
  i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
              (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  i32x8 bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
              (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, zero16(), 0, 0, 0,
                                                                (int)sa[l], 0, (int)sb[l]);
#pragma unroll
  for (int i = 0; i < 16; ++i) c[16 * l + i] = acc[i];
}

// fp8 (E4M3) convert probe.  x: 64 lanes x 2 floats; out: 64 lanes x 2 u32,
// out[2l + sel] = v_cvt_scalef32_pk_fp8_f32 of (x[2l], x[2l+1]) with scale 1 into
// 16-bit half `sel` of 0xFFFFFFFF.
__global__ void cvt_fp8_probe(const float* x, uint32_t* out) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const int l = threadIdx.x;
  const float a = x[2 * l], b = x[2 * l + 1];
  const s16x2 ones = {-1, -1};
  out[2 * l + 0] = __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ones, a, b, 1.0f, false));
  out[2 * l + 1] = __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ones, a, b, 1.0f, true));
}

}  // namespace

extern "C" {

int probe_mfma_bf16(const void* a, const void* b, float* c, void* stream) {
  hipLaunchKernelGGL(mfma_bf16_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint16_t*)a, (const uint16_t*)b, c);
  return (int)hipGetLastError();
}

int probe_tr16(const void* addr, void* out, void* stream) {
  hipLaunchKernelGGL(tr16_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const int*)addr,
                     (uint16_t*)out);
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

// out must hold blocks * 256 floats.
int probe_mfma_rate(float* out, int blocks, int iters, void* stream) {
  if (blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mfma_rate_probe, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

// src: 2048 x 16 bytes of operand data; out: blocks * 512 floats; stats: 2 x u64.
int probe_power(const void* src, float* out, unsigned long long* stats, int blocks, int iters,
                int mode, void* stream) {
  if (blocks < 1 || iters < 1 || mode < 0 || mode > 2) return -1;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const u32x4*)src, out, stats, iters);
  };
  if (mode == 0) go(power_probe<0>);
  else if (mode == 1) go(power_probe<1>);
  else go(power_probe<2>);
  return (int)hipGetLastError();
}

// out: blocks * threads floats; stats: 2 x u64 (added to); threads 256 or 512; v in
// {0, 4, 8, 12, 16}.
int probe_overlap(float* out, unsigned long long* stats, int blocks, int threads, int iters,
                  int v, void* stream) {
  if (blocks < 1 || iters < 1 || (threads != 256 && threads != 512)) return -1;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream, out, stats,
                       iters);
  };
  switch (v) {
    case 0: go(overlap_probe<0>); break;
    case 4: go(overlap_probe<4>); break;
    case 8: go(overlap_probe<8>); break;
    case 12: go(overlap_probe<12>); break;
    case 16: go(overlap_probe<16>); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

// addr: 64 byte offsets (multiples of 16, below 32768); out: 64 floats.
int probe_lds_pattern(const void* addr, float* out, int iters, int write, void* stream) {
  if (iters < 1) return -1;
  if (write)
    hipLaunchKernelGGL(lds_pattern_probe<1>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const uint32_t*)addr, out, iters);
  else
    hipLaunchKernelGGL(lds_pattern_probe<0>, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const uint32_t*)addr, out, iters);
  return (int)hipGetLastError();
}

// out must hold blocks * 256 floats.
int probe_lds_rate(float* out, int blocks, int iters, int mode, void* stream) {
  if (blocks < 1 || iters < 1) return -1;
  if (mode == 0)
    hipLaunchKernelGGL(lds_rate_probe<0>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(lds_rate_probe<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

int probe_lds_dma(const void* src, void* out, void* stream) {
  hipLaunchKernelGGL(lds_dma_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint32_t*)src, (uint32_t*)out);
  return (int)hipGetLastError();
}

int probe_cvt_dot(const void* x, const void* acc, void* out, void* stream) {
  hipLaunchKernelGGL(cvt_dot_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const float*)x, (const float*)acc, (uint32_t*)out);
  return (int)hipGetLastError();
}

int probe_cvt_fp4(const void* x, const void* scale, void* out, void* stream) {
  hipLaunchKernelGGL(cvt_fp4_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const float*)x,
                     (const float*)scale, (uint32_t*)out);
  return (int)hipGetLastError();
}

int probe_dec_fp4(const void* src, const void* scale, void* out, void* stream) {
  hipLaunchKernelGGL(dec_fp4_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint32_t*)src, (const float*)scale, (float*)out);
  return (int)hipGetLastError();
}

int probe_mfma_fp4_sel2(const void* a, const void* b, const void* sa, const void* sb, float* c,
                        void* stream) {
  hipLaunchKernelGGL(mfma_fp4_sel2_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint8_t*)a, (const uint8_t*)b, (const uint32_t*)sa,
                     (const uint32_t*)sb, c);
  return (int)hipGetLastError();
}

// out must hold blocks * 8 uint32.
int probe_wave_place(void* out, int blocks, void* stream) {
  if (blocks < 1) return -1;
  hipLaunchKernelGGL(wave_place_probe, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                     (uint32_t*)out);
  return (int)hipGetLastError();
}

int probe_mfma_fp8(const void* a, const void* b, const void* sa, const void* sb, float* c,
                   void* stream) {
  hipLaunchKernelGGL(mfma_fp8_probe, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint8_t*)a, (const uint8_t*)b, (const uint8_t*)sa,
                     (const uint8_t*)sb, c);
  return (int)hipGetLastError();
}

int probe_cvt_fp8(const void* x, void* out, void* stream) {
  hipLaunchKernelGGL(cvt_fp8_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const float*)x,
                     (uint32_t*)out);
  return (int)hipGetLastError();
}

}  // extern "C"
