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


// ---------------------------------------------------------------------------
// Direct-P forward ("Hardware-Aware FP4 FlashAttention-4", section "1. Direct-P
// para Inferencia Directa").
//
// Work split, staging and the software pipeline follow the bf16 kernel: one
// workgroup = 8 waves x 32 query rows; 64-key tiles of K codes/scales and V^T
// codes/scales are staged through registers into double-buffered LDS; pipeline
// step j issues the PV product of tile j-1, the QK product of tile j+1 and the
// Direct-P mapping of tile j.  All three products run on
// v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and E8M0 block scales:
//   S^T  = K Q^T       A = K codes (32 keys x 64 d), B = Q codes (registers)
//   O^T += V^T P^T     A = V^T codes (32 d x 64 keys), B = P codes (registers)
//   L   += 1 P^T       A = all-ones codes: every accumulator row is the row sum
// The last one is the consistent normaliser of the page's "Normalización
// Consistente": the denominator is summed from exactly the rounded codes and
// block scales that the PV product consumes, by the same hardware.
//
// Direct-P (same section, "Mapeo Directo"): the log-scores t = s * scale * log2(e)
// go straight to E2M1 codes, one power-of-two scale per 32 keys, relative to an
// integer reference max m (moved only when a tile's max exceeds m + tau):
//   E    = floor(block max - m) - 2                 (block max in [4, 8) * 2^E)
//   code = RNE_E2M1(2^(t - m - E))                  (saturating at 6)
// The code is the E2M1 value nearest 2^x, i.e. x compared against the log2
// midpoints of the E2M1 grid; on gfx950 the cheapest exact form of that
// comparison is one v_exp_f32 and the hardware fp4 convert (two codes per
// instruction), which is what is issued.  Because m is an integer, the codes do
// not depend on which m the kernel held, and the rescale factors are exact
// powers of two.

constexpr int kMWaves = 8;
constexpr int kMRows = 32;
constexpr int kMBr = kMWaves * kMRows;   // 256 query rows per workgroup
constexpr int kMBc = 64;                 // keys per tile
constexpr int kMThreads = kMWaves * 64;
constexpr int kMD = 128;                 // head dimension of this path
constexpr int kCodeRow = kMD / 2;        // code bytes per Q/K row
constexpr int kScaleRow = kMD / 32;      // scale bytes per Q/K row

// Raw buffer descriptor over `bytes` bytes at `base`: loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mrsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// K row of the tile read by A-row m of 32-key MFMA block mb.  With this order the
// S^T accumulator of lane half h holds exactly keys 32h .. 32h+31 of the tile
// (register r of block mb: key 32h + 16mb + r), i.e. one whole P scale block.
__device__ __forceinline__ int krow(int mb, int m) {
  return 32 * ((m >> 2) & 1) + 16 * mb + 4 * (m >> 3) + (m & 3);
}
// 16-byte chunk swizzle of a K code row (64 B = 4 chunks): the 16 lanes the LDS
// serves together read 16 distinct bank groups.
__device__ __forceinline__ int kswz(int row) { return ((row >> 2) & 1) | (((row >> 5) & 1) << 1); }

__device__ __forceinline__ i32x8 fp4_operand(u32x4 v) {
  return i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
}

// max of two floats as one v_max_f32 (fmaxf on a lane swap's output or a loop-carried value
// adds a quieting max per operand; the operands are scores, integers or -inf)
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

struct MBuf {
  // code units: [0, 256) K, unit(row, c) = row*4 + (c ^ kswz(row));
  //             [256, 512) V^T, 256 + unit(col, h) = 256 + col*2 + (h ^ ((col>>3)&1))
  u32x4 code[2 * 256];
  // scale bytes: [0, 256) K, byte 4r + b = scale of d block b of key row r;
  //              [256, 512) V^T, byte 256 + 2c + h = scale of key block h of column c
  uint8_t scale[4 * kMBc + 2 * kMD];
};

struct MStage {
  u32x4 codes;     // tid < 256: K codes (row tid/4, chunk tid%4); else V^T codes (col, half)
  uint32_t sc;     // scale byte tid of the tile (MBuf::scale layout)
};

// Direct-P mapping of one 64-key tile for this lane (32 keys: its P scale block).
// Returns whether any row of the wave moved its reference max (then O and the
// row sum must be multiplied by alpha before the next PV product).
// BAND: the lane sees keys [klo, khi] only (a sliding window and / or its document;
// khi < N), which replaces the causal and ragged-tail tests.
template <bool CAUSAL, bool MASK, bool BAND>
__device__ __forceinline__ bool directp_tile(const f32x16 (&s)[2], u32x4& codes, uint32_t& sbyte,
                                             float& m, float& alpha, int kv0, int qi, int N,
                                             float c, float tau, int h, int klo, int khi) {
  const float NEG_INF = -__builtin_inff();
  auto visible = [&](int mb, int r) {
    const int key = kv0 + 32 * h + 16 * mb + r;
    // non-short-circuit in the band form: evaluated whole, no branch per element
    return BAND ? (key >= klo) & (key <= khi) : key < N && (!CAUSAL || key <= qi);
  };
  // block max over this lane's 32 scores: four independent chains
  float bq[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = (!MASK || visible(mb, r)) ? s[mb][r] : NEG_INF;
      bq[r & 3] = fmaxf(bq[r & 3], v);
    }
  const float bm = fmaxf(fmaxf(bq[0], bq[1]), fmaxf(bq[2], bq[3]));
  // this lane's block max (log2); without a mask every score, so the maximum, is finite
  const float Mb = (MASK && bm == NEG_INF) ? NEG_INF : bm * c;
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(Mb), __float_as_uint(Mb), false,
                                             false);
  const float mx = vmax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));   // tile row max

  const bool any = __ballot(mx > m + tau) != 0;
  const float m_up = vmax(m, __builtin_ceilf(mx));   // unconditional: the choice is a select
  const float m_new = any ? m_up : m;
  if constexpr (MASK) {
    alpha = (m_new == NEG_INF) ? 1.f
            : (m == NEG_INF ? 0.f : __builtin_ldexpf(1.f, (int)(m - m_new)));
  } else {
    // m_new is a finite integer; m is an integer or -inf, whose conversion saturates, so
    // alpha = 2^(m - m_new) is 0 on a row's first tile
    alpha = __builtin_ldexpf(1.f, (int)(m - m_new));
  }
  m = m_new;

  bool flush = MASK && ((Mb == NEG_INF) || (m_new == NEG_INF));
  float e = flush ? 0.f : __builtin_floorf(Mb - m_new) - 2.f;
  flush = flush || e < -127.f;
  e = flush ? 0.f : e;
  const float bias = flush ? __builtin_inff() : m_new + e;
  sbyte = (uint32_t)((int)e + 127);

#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float y[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int el = 8 * w + q;                // element index = key - 32h = 16mb + r
      const int mb = el >> 4, r = el & 15;
      float x = __builtin_fmaf(s[mb][r], c, -bias);
      if constexpr (MASK) x = visible(mb, r) ? x : NEG_INF;
      y[q] = __builtin_amdgcn_exp2f(x);
    }
    // the four converts write all four bytes, so the first one starts from the register's
    // old contents rather than a zeroed register
    uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes[w], y[0], y[1], 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[2], y[3], 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[4], y[5], 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y[6], y[7], 1.0f, 3);
    codes[w] = word;
  }
  return any;
}

template <bool CAUSAL, bool BAND>
__global__ __attribute__((amdgpu_flat_work_group_size(kMThreads, kMThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_mxfp4_kernel(const uint8_t* __restrict__ Q4, const uint8_t* __restrict__ QS,
                      const uint8_t* __restrict__ K4, const uint8_t* __restrict__ KS,
                      const uint8_t* __restrict__ VT4, const uint8_t* __restrict__ VTS,
                      float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int N,
                      int nqb, float c, float tau, uint32_t qsign, int window,
                      const int* __restrict__ doc_off, int n_docs,
                      unsigned long long* __restrict__ stats) {
  __shared__ MBuf buf[2];
  const float NEG_INF = -__builtin_inff();
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index through readfirstlane: the staging roles below (K codes: waves 0-3, V^T
  // codes: 4-7) are whole waves, so their selects are scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, h = lane >> 5;

  const int group = Hq / Hkv;
  // shader-clock and 100 MHz reference stamps, for the clock statistic
  const unsigned long long clk0 = __builtin_amdgcn_s_memtime();
  const unsigned long long ref0 = __builtin_amdgcn_s_memrealtime();
  const WorkItem wi = decode_workgroup(blockIdx.x, gridDim.x, Hkv, group, nqb, CAUSAL);
  const int b = wi.b, hkv = wi.hkv, g = wi.g;
  const int qb = CAUSAL ? (nqb - 1 - wi.qb_rank) : wi.qb_rank;
  const int hq = hkv * group + g;
  const int Q0 = qb * kMBr;
  const int q0 = Q0 + wave * kMRows;
  const int qi = q0 + n32;

  const size_t qhead = (size_t)(b * Hq + hq) * N;
  const size_t khead = (size_t)(b * Hkv + hkv) * N;
  const uint8_t* K4h = K4 + khead * kCodeRow;
  const uint8_t* KSh = KS + khead * kScaleRow;
  const uint8_t* VT4h = VT4 + khead * kCodeRow;       // [kMD][N/2] per head
  const uint8_t* VTSh = VTS + khead * kScaleRow;      // [kMD][N/32] per head
  const int nvb = N / 32;                             // V scale bytes per column
  const __amdgpu_buffer_rsrc_t rvt = mrsrc(VT4h, kMD * (N / 2));
  const __amdgpu_buffer_rsrc_t rvs = mrsrc(VTSh, kMD * nvb);

  // Q codes: lane holds d elements 64kc + 32h .. +31 of query qi (B operand of QK);
  // byte 2kc of qsc is the scale of that block.
  u32x4 qc[2];
  uint32_t qsc;
  {
    const int qr = min(qi, N - 1);
    const uint8_t* qrow = Q4 + (qhead + qr) * kCodeRow;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) qc[kc] = *(const u32x4*)(qrow + 32 * kc + 16 * h) ^ qsign;
    const uint8_t* srow = QS + (qhead + qr) * kScaleRow;
    qsc = ((uint32_t)srow[0] | ((uint32_t)srow[1] << 8) | ((uint32_t)srow[2] << 16) |
           ((uint32_t)srow[3] << 24)) >> (8 * h);
  }

  f32x16 acc[kMD / 32], lacc;
#pragma unroll
  for (int i = 0; i < kMD / 32; ++i) acc[i] = zero16();
  lacc = zero16();
  float m = NEG_INF;

  // BAND (the bf16 forward's rules): row i sees keys [lo(i), hi(i)], from a window W
  // (i - W < j, and j < i + W without the causal mask) and / or its document; both
  // bounds are non-decreasing in i, so a block's first and last rows bound its keys.
  // The document search reads only doc_off[0 .. n_docs] and keeps lo <= i <= hi.
  auto row_bounds = [&](int i, int& lo, int& hi) {
    lo = window ? max(0, i - window + 1) : 0;
    hi = CAUSAL ? i : (window ? min(N - 1, i + window - 1) : N - 1);
    if (n_docs > 0) {
      int a = 0, z = n_docs;
      while (z - a > 1) {
        const int mid = (a + z) >> 1;
        if (doc_off[mid] <= i) a = mid;
        else z = mid;
      }
      lo = max(lo, min(doc_off[a], i));
      hi = min(hi, max(doc_off[a + 1] - 1, i));
    }
  };
  int klo = 0, khi = 0, wg_lo_first = 0, wg_hi_first = 0, wg_lo_last = 0, wg_hi_last = 0;
  int w_lo = 0, w_hi = 0, unused = 0;
  if (BAND) {
    row_bounds(min(qi, N - 1), klo, khi);
    row_bounds(Q0, wg_lo_first, wg_hi_first);
    row_bounds(min(Q0 + kMBr - 1, N - 1), wg_lo_last, wg_hi_last);
    row_bounds(min(q0, N - 1), w_lo, unused);
    row_bounds(min(q0 + kMRows - 1, N - 1), unused, w_hi);
  }
  // tiles t0 .. t0 + n - 1 (local index j = tile - t0)
  const int t0 = BAND ? wg_lo_first / kMBc : 0;
  const int kv_end = BAND ? wg_hi_last + 1 : (CAUSAL ? min(N, Q0 + kMBr) : N);
  const int n = (kv_end + kMBc - 1) / kMBc - t0;
  const int wave_end = BAND ? w_hi + 1 : (CAUSAL ? min(N, q0 + kMRows) : N);
  const bool wave_live = q0 < N;

  // Stage t (read by pipeline step t from buffer t & 1) holds K tile t+1 and V tile t-1.
  // Every thread stages one code unit (K for waves 0-3, V^T for waves 4-7) and one scale
  // byte, choosing the source by wave-uniform selects, so a pipeline step has no branches
  // and is one scheduling region.  The loads are unconditional, with the tile index
  // clamped into [0, n) (in bounds), and so are the stores: a stage past the tiles lands
  // in a buffer half that no later product reads.
  const bool kpart = wave < 4;
  const int su = tid - 256, scol = su >> 1, shh = su & 1;        // V^T unit of waves 4-7
  const int code_slot = kpart ? (tid >> 2) * 4 + ((tid & 3) ^ kswz(tid >> 2))
                              : 256 + scol * 2 + (shh ^ ((scol >> 3) & 1));
  auto load_stage = [&](MStage& sg, int t) {
    const int kt = min(t + 1, n - 1), vt = max(min(t - 1, n - 1), 0);
    const int kk0 = (t0 + kt) * kMBc, vk0 = (t0 + vt) * kMBc;
    const __amdgpu_buffer_rsrc_t rk = mrsrc(K4h + (size_t)kk0 * kCodeRow, (N - kk0) * kCodeRow);
    sg.codes = __builtin_amdgcn_raw_buffer_load_b128(
        kpart ? rk : rvt,
        kpart ? (tid >> 2) * kCodeRow + (tid & 3) * 16 : scol * (N / 2) + vk0 / 2 + 16 * shh,
        0, 0);
    // a V key block past N gets a neutral scale; the load reads block 0 then (in range)
    const bool past = vk0 + 32 * shh >= N;
    const __amdgpu_buffer_rsrc_t rs =
        kpart ? mrsrc(KSh + (size_t)kk0 * kScaleRow, (N - kk0) * kScaleRow) : rvs;
    const int off = kpart ? tid : scol * nvb + (past ? 0 : vk0 / 32 + shh);
    const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
    sg.sc = (!kpart && past) ? 127u : byte;
  };
  auto store_stage = [&](const MStage& sg, int t) {
    MBuf& bb = buf[t & 1];
    bb.code[code_slot] = sg.codes;
    bb.scale[tid] = (uint8_t)sg.sc;
  };

  const int kr0 = krow(0, n32), kr1 = krow(1, n32);
  const uint32_t ONES = 0x22222222u;   // E2M1 code 2 (= 1.0) in every nibble

  // MFMAs of one pipeline step: PV + row sum of the previous tile (P codes pp,
  // P scale byte ep, V^T from bb), then QK of the next tile into sn (K from bb).
  auto mfmas = [&](const MBuf& bb, const u32x4& pp, uint32_t ep, bool pv, bool qk,
                   f32x16 (&sn)[2]) {
    if (pv) {
      const i32x8 bp = fp4_operand(pp);
#pragma unroll
      for (int cb = 0; cb < kMD / 32; ++cb) {
        const int col = 32 * cb + n32;
        const u32x4 va = bb.code[256 + col * 2 + (h ^ ((col >> 3) & 1))];
        const int vs = bb.scale[4 * kMBc + col * 2 + h];
        acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(va), bp, acc[cb], 4,
                                                                  4, 0, vs, 0, (int)ep);
      }
      lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fp4_operand(u32x4{ONES, ONES, ONES, ONES}), bp, lacc, 4, 4, 0, 127, 0, (int)ep);
    }
    if (qk) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = mb ? kr1 : kr0;
        const int ksc = (int)(*(const uint32_t*)(bb.scale + 4 * row) >> (8 * h));
        // d elements 0..63 (scale byte 0 of the shifted scale words), then 64..127 (byte 2)
        const u32x4 ka0 = bb.code[row * 4 + ((0 + h) ^ kswz(row))];
        const u32x4 ka1 = bb.code[row * 4 + ((2 + h) ^ kswz(row))];
        f32x16 a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fp4_operand(ka0), fp4_operand(qc[0]), zero16(), 4, 4, 0, ksc, 0, (int)qsc);
        a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(ka1), fp4_operand(qc[1]), a,
                                                            4, 4, 2, ksc, 2, (int)qsc);
        sn[mb] = a;
      }
    }
  };

  // ---- prologue: K tile 0 -> buffer 1; stage 0 -> buffer 0; stage 1 in registers ----
  MStage stg;
  {
    MStage s0;
    load_stage(s0, -1);            // K tile 0 (its V half is overwritten later)
    load_stage(stg, 0);
    store_stage(s0, 1);            // buffer 1: K tile 0 and its scales
    store_stage(stg, 0);           // buffer 0: K tile 1
    // no V tile precedes tile 0: zero codes and neutral scales, written by the same
    // threads (same slots) that stored this half just above
    if (!kpart) {
      buf[0].code[code_slot] = u32x4{0u, 0u, 0u, 0u};
      buf[0].scale[tid] = 127;
    }
  }
  load_stage(stg, 1);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  f32x16 s_cur[2], s_nxt[2];
  u32x4 p_prev = u32x4{0u, 0u, 0u, 0u}, p_cur;
  uint32_t e_prev = 127u, e_cur = 127u;
  mfmas(buf[1], p_prev, e_prev, false, true, s_cur);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  bool any_prev = false;
  float alpha_prev = 1.f;
  // unmasked tiles [lo_full, n_full): every row of the workgroup sees all their keys
  const int n_full = BAND ? (wg_hi_first + 1) / kMBc - t0 : (CAUSAL ? min(Q0, N) / kMBc : N / kMBc);
  const int lo_full = BAND ? min(n, (wg_lo_last + kMBc - 1) / kMBc - t0) : 0;
  // rescale decisions that fired; every step's decision passes through rescale() once
  unsigned n_fires = 0;
  auto rescale = [&]() {
    if (any_prev) {
#pragma unroll
      for (int i = 0; i < kMD / 32; ++i) acc[i] *= alpha_prev;
      lacc *= alpha_prev;
      ++n_fires;
    }
  };
  // Pipeline step j: PV and row sum of tile j-1 (pp, ep), QK of tile j+1 into sn,
  // Direct-P of tile j (sc -> pc, ec); then the staging of stage j+1 and the barrier.
  auto step = [&](int j, bool pv, bool qk, bool masked, f32x16 (&sc)[2], f32x16 (&sn)[2],
                  const u32x4& pp, uint32_t ep, u32x4& pc, uint32_t& ec) {
    rescale();
    mfmas(buf[j & 1], pp, ep, pv, qk, sn);
    float alpha;
    bool any;
    if (masked)
      any = directp_tile<CAUSAL, true, BAND>(sc, pc, ec, m, alpha, (t0 + j) * kMBc, qi, N, c,
                                             tau, h, klo, khi);
    else
      any = directp_tile<CAUSAL, false, BAND>(sc, pc, ec, m, alpha, (t0 + j) * kMBc, qi, N, c,
                                              tau, h, klo, khi);
    any_prev = any;
    alpha_prev = alpha;
    // the weights are done before the barrier: left alone, the compiler moves them into the
    // next step, beside that step's own weights and in front of the products that use them
    asm volatile("" ::"v"(pc), "v"(ec));
    store_stage(stg, j + 1);
    load_stage(stg, j + 2);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto advance = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) s_cur[i] = s_nxt[i];
    p_prev = p_cur;
    e_prev = e_cur;
  };

  // masked tiles: below lo_full (some row's lower edge, BAND) and from n_full on
  auto masked_at = [&](int jj) { return jj < lo_full || jj >= n_full; };
  // step 0 has no PV product (no tile before it)
  step(0, false, n > 1, masked_at(0), s_cur, s_nxt, p_prev, e_prev, p_cur, e_cur);
  advance();
  int j = 1;
  // masked steps below the band's lower edge
  for (; j < min(lo_full, n - 1); ++j) {
    step(j, true, true, true, s_cur, s_nxt, p_prev, e_prev, p_cur, e_cur);
    advance();
  }
  // unmasked steps with both products, two at a time with the S / P registers swapping
  // roles (no copies)
  for (; j + 1 < min(n_full, n - 1); j += 2) {
    step(j, true, true, false, s_cur, s_nxt, p_prev, e_prev, p_cur, e_cur);
    step(j + 1, true, true, false, s_nxt, s_cur, p_cur, e_cur, p_prev, e_prev);
  }
  for (; j < n - 1; ++j) {
    step(j, true, true, masked_at(j), s_cur, s_nxt, p_prev, e_prev, p_cur, e_cur);
    advance();
  }
  // the last step has no QK product (no tile after it)
  if (n > 1) {
    step(n - 1, true, false, masked_at(n - 1), s_cur, s_nxt, p_prev, e_prev, p_cur, e_cur);
    advance();
  }
  rescale();
  mfmas(buf[n & 1], p_prev, e_prev, true, false, s_nxt);

  // ---- epilogue: O = acc / l, LSE = ln2 * m + ln l ----
  const float l = lacc[0];
  if (qi < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* Orow = O + (qhead + qi) * kMD;
#pragma unroll
    for (int cb = 0; cb < kMD / 32; ++cb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 out = {acc[cb][4 * a4] * inv, acc[cb][4 * a4 + 1] * inv, acc[cb][4 * a4 + 2] * inv,
                     acc[cb][4 * a4 + 3] * inv};
        *(f32x4*)(Orow + cb * 32 + 8 * a4 + 4 * h) = out;
      }
    if (h == 0)
      LSE[qhead + qi] = l > 0.f ? (m + __builtin_log2f(l)) * kLn2 : -__builtin_inff();
  }
  // Statistics without per-step bookkeeping: the wave's visible tiles are the local
  // indices [j_lo, j_hi); the first always fires (the reference max starts at -inf) and
  // the rest are the counted steps; the other tiles hold no visible key and never fire.
  if (stats != nullptr && lane == 0 && wave_live) {
    const int j_hi = min(n, (wave_end + kMBc - 1) / kMBc - t0);
    const int j_lo = BAND ? max(0, w_lo / kMBc - t0) : 0;
    if (j_hi > j_lo) {
      atomicAdd(stats, (unsigned long long)(j_hi - j_lo - 1));
      atomicAdd(stats + 1, (unsigned long long)(n_fires - 1u));
    }
  }
  if (stats != nullptr && threadIdx.x == 0) {
    atomicAdd(stats + 2, __builtin_amdgcn_s_memtime() - clk0);
    atomicAdd(stats + 3, __builtin_amdgcn_s_memrealtime() - ref0);
  }
}

template <bool CAUSAL, bool BAND>
hipError_t launch_mxfp4(const MxArgs& a) {
  const int nqb = (a.N + kMBr - 1) / kMBr;
  const long long grid = (long long)a.B * a.Hq * nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_mxfp4_kernel<CAUSAL, BAND>), dim3((unsigned)grid), dim3(kMThreads), 0,
                     (hipStream_t)a.stream, a.qc, a.qs, a.kc, a.ks, a.vtc, a.vts, a.o, a.lse,
                     a.Hq, a.Hkv, a.N, nqb, a.c, a.tau, a.qsign, a.window, a.doc_offsets,
                     a.n_docs, a.stats);
  return hipGetLastError();
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

hipError_t launch_fwd_mxfp4(const MxArgs& a) {
  if (a.d != kMD) return hipErrorNotSupported;
  const bool band = a.window > 0 || a.n_docs > 0;
  if (a.causal) return band ? launch_mxfp4<true, true>(a) : launch_mxfp4<true, false>(a);
  return band ? launch_mxfp4<false, true>(a) : launch_mxfp4<false, false>(a);
}

}  // namespace attn
