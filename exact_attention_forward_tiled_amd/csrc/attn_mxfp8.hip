// MXFP8 path: input quantisation kernels and the FP8 forward.
//
// "Hardware-Aware FP4 FlashAttention-4", section "Resultados", sets its FP4 fast
// path beside an FP8 path ("NV/FP8", mean cosine about 0.990 against BF16), and
// its section "2. Causal Backward Cuantizado" keeps P and V in FP8; the aigc.bar
// page, section "从V1到V4", credits FlashAttention-3 with FP8 support.  On gfx950
// FP8 runs on the same scaled MFMA as FP4 (twice the bf16 rate), so the operands
// here are OCP MXFP8: E4M3 elements with one E8M0 power-of-two scale per 32
// elements (Q and K blocked along d, V along the keys), and the softmax weights
// are rounded to E4M3 with one power-of-two scale per 32 keys before the PV
// product.

#include "common.h"
#include "launch.h"

namespace attn {
namespace {

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Shared exponent of an MXFP8 block: floor(log2(amax)) - 8 (8 = exponent of the
// largest E4M3 binade), clamped to [-127, 127]; 0 for an all-zero block.
__device__ __forceinline__ int block_exponent8(float amax) {
  if (amax == 0.f) return 0;
  const int field = (__float_as_int(amax) >> 23) & 0xFF;
  const int e = (field == 0 ? -127 : field - 127) - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four E4M3 codes of x[0..3] / 2^e in one word (element i in byte i): rounded to
// nearest even by the hardware convert after clamping to +-448 (saturation); a
// value that rounds to magnitude 0 is stored as +0.
__device__ __forceinline__ uint32_t encode4(const float* x, int e) {
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = fminf(fmaxf(__builtin_ldexpf(x[i], -e), -448.f), 448.f);
  const s16x2 zero = {0, 0};
  const s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero, y[0], y[1], 1.0f, false);
  const uint32_t w = __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[2], y[3], 1.0f, true));
  // bytes 0x80 (negative zero) -> 0x00
  const uint32_t mag = w & 0x7F7F7F7Fu;
  const uint32_t nz = ((mag + 0x7F7F7F7Fu) | mag) & 0x80808080u;   // bit 7 set where mag != 0
  return w & (nz | 0x7F7F7F7Fu);
}

__device__ __forceinline__ void encode_block(const float (&v)[32], int e, u32x4 (&out)[2]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) out[w >> 2][w & 3] = encode4(&v[4 * w], e);
}

__global__ void quantize8_rows_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
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
  const int e = block_exponent8(amax);
  u32x4 out[2];
  encode_block(v, e, out);
  u32x4* dst = (u32x4*)(codes + blk * 32);
  dst[0] = out[0];
  dst[1] = out[1];
  scales[blk] = (uint8_t)(e + 127);
}

__global__ void quantize8_cols_t_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
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
  const int e = block_exponent8(amax);
  u32x4 out[2];
  encode_block(v, e, out);
  const long long crow = b * cols + col;   // row of the transposed output
  u32x4* dst = (u32x4*)(codes + crow * rows + (long long)rb * 32);   // 32-byte aligned
  dst[0] = out[0];
  dst[1] = out[1];
  scales[crow * nrb + rb] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------------------
// FP8 forward.
//
// Work split and staging are those of the MXFP4 forward: one workgroup = 8 waves x
// 32 query rows; 64-key tiles of K codes/scales and V^T codes/scales are staged
// through registers into double-buffered LDS.  Pipeline step j issues the QK
// product of tile j, then the PV product of tile j-1 (which covers the QK latency),
// then the weights of tile j: the scores live only within a step and the P codes
// pass from one step to the next in the same registers, so the loop needs no
// register copies and stays well inside the 256 registers a wave has here.  All three products run on v_mfma_scale_f32_32x32x64_f8f6f4
// with E4M3 operands (format 0) and E8M0 block scales:
//   S^T  = K Q^T       A = K codes (32 keys x 64 d), B = Q codes (registers)
//   O^T += V^T P^T     A = V^T codes (32 d x 64 keys), B = P codes (registers)
//   L   += 1 P^T       A = all-ones codes: every accumulator row is the row sum,
//                      taken from exactly the rounded weights PV consumes
// Operand layout of the E4M3 form of that MFMA (probed on the device): lane
// (i, h) of a 32-row operand holds 32 bytes in 8 registers; bytes 0-15 belong to
// k-block 0 (k 0..31) and bytes 16-31 to k-block 1 (k 32..63), each k-block made
// of the 16-byte halves of lanes (i, 0) and (i, 1); the scale byte of lane (i, b)
// scales k-block b of row i.  So each lane loads d (or keys) 16h .. 16h+15 and
// 32 + 16h .. 32 + 16h + 15 of a 64-wide k-chunk, and every MX block of 32
// consecutive elements is one k-block.
//
// Weights: the log-scores t = s * scale * log2(e) are taken relative to an integer
// reference max m (moved only when a tile's max exceeds m + tau), with one
// power-of-two scale per 32 keys:
//   E    = floor(block max - m) - 7                (block max in [128, 256) * 2^E)
//   code = RNE_E4M3(2^(t - m - E))                 (v_exp_f32, then the fp8 convert)
// The block maximum stays one binade below E4M3's largest, so nothing saturates.
// Because m is an integer the codes do not depend on which m the kernel held, and
// the rescale factors are exact powers of two.

constexpr int k8Waves = 8;
constexpr int k8Rows = 32;
constexpr int k8Br = k8Waves * k8Rows;   // 256 query rows per workgroup
constexpr int k8Bc = 64;                 // keys per tile
constexpr int k8Threads = k8Waves * 64;
constexpr int k8D = 128;                 // head dimension of this path
constexpr int k8CodeRow = k8D;           // code bytes per Q/K row
constexpr int k8ScaleRow = k8D / 32;     // scale bytes per Q/K row
constexpr int k8PExp = 7;                // P block exponent: floor(block max - m) - 7

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc8(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// K row of the tile read by A-row m of 32-key MFMA block mb: register r of the
// S^T accumulator block mb of lane half h then holds key 32mb + 16h + r, so each
// lane's P bytes 0-15 (mb = 0) and 16-31 (mb = 1) are exactly the keys the PV
// product's k-blocks 0 and 1 expect from it.
__device__ __forceinline__ int krow8(int mb, int m) {
  return 32 * mb + 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}
// LDS layouts.  A 16-byte ds_read_b128 serves 16 lanes at a time over 64 banks
// (256 bytes), so the 16 lanes must hit 16 distinct 16-byte slots of that window.
// Rows (K) and columns (V^T) are padded by one 16-byte chunk, so consecutive rows
// advance by 9 (K) or 5 (V^T) slots mod 16, both invertible: 16 rows whose
// positions differ mod 16 never collide, whichever chunk they read.  The chunk
// offset then simply adds to a per-lane row base (one address register per
// read stream, compile-time immediates for the rest).
constexpr int k8KStride = k8CodeRow + 16;    // 144 bytes per staged K row
constexpr int k8VStride = k8Bc + 16;         // 80 bytes per staged V^T column
// Position of K row r in LDS.  The 16 rows read together, krow8(mb, 0..15) =
// {0..7, 16..23} + 32mb (or {8..15, 24..31} + 32mb for the other 16 lanes), land
// on positions whose residues mod 16 are all distinct.
__device__ __forceinline__ int kpos8(int r) { return r ^ (((r >> 4) & 1) << 3); }

__device__ __forceinline__ i32x8 fp8_operand(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// max of two floats as one v_max_f32 (fmaxf on a lane swap's output or a loop-carried value
// adds a quieting max per operand; the operands are scores, integers or -inf)
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

struct F8Buf {
  uint8_t kcode[k8Bc * k8KStride];   // K row r at kpos8(r) * 144, 128 code bytes
  uint8_t vcode[k8D * k8VStride];    // V^T column c at c * 80, 64 code bytes (keys)
  // scale bytes: [0, 256) K, byte 4r + b = scale of d block b of key row r;
  // [256, 512) V^T, byte 256 + 2c + h = scale of key block h of column c
  uint8_t scale[4 * k8Bc + 2 * k8D];
};

__device__ __forceinline__ u32x4 lds16(const uint8_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void sts16(uint8_t* p, const u32x4& v) { *(u32x4*)p = v; }

struct F8Stage {
  u32x4 k;       // K codes: row tid/8, chunk tid%8
  u32x4 v;       // V^T codes: column tid/4, chunk tid%4
  uint32_t sc;   // scale byte tid of the tile (F8Buf::scale layout)
};

// Weights of one 64-key tile for this lane (32 keys: its P scale block).  Returns
// whether any row of the wave moved its reference max (then O and the row sum
// must be multiplied by alpha before the next PV product).
// BAND: the lane sees keys [klo, khi] only (a sliding window and / or its document; the
// bounds already hold the causal limit and N).
template <bool CAUSAL, bool MASK, bool BAND>
__device__ __forceinline__ bool fp8p_tile(const f32x16 (&s)[2], u32x4 (&codes)[2],
                                          uint32_t& sbyte, float& m, float& alpha, int kv0,
                                          int qi, int N, float c, float tau, int h, int klo,
                                          int khi) {
  const float NEG_INF = -__builtin_inff();
  auto visible = [&](int mb, int r) {
    const int key = kv0 + 32 * mb + 16 * h + r;
    return BAND ? (key >= klo) & (key <= khi) : key < N && (!CAUSAL || key <= qi);
  };
  // this lane's maxima over its 16 scores of each 32-key block (two chains each)
  float bq[2][2] = {{NEG_INF, NEG_INF}, {NEG_INF, NEG_INF}};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = (!MASK || visible(mb, r)) ? s[mb][r] : NEG_INF;
      bq[mb][r & 1] = fmaxf(bq[mb][r & 1], v);
    }
  float ml[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const float bm = fmaxf(bq[mb][0], bq[mb][1]);
    // log2 units; without a mask every score, so the maximum, is finite
    ml[mb] = (MASK && bm == NEG_INF) ? NEG_INF : bm * c;
  }
  // block b's 32 keys sit in lanes (n, 0) and (n, 1): the first swap leaves lane half h
  // with both halves' maxima of block h, the second hands both block maxima to every lane
  auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(ml[0]), __float_as_uint(ml[1]),
                                             false, false);
  const float own = vmax(__uint_as_float(s1[0]), __uint_as_float(s1[1]));   // block h max
  auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(own), __float_as_uint(own), false,
                                             false);
  const float B0 = __uint_as_float(s2[0]), B1 = __uint_as_float(s2[1]);
  const float mx = vmax(B0, B1);                              // tile row max

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

  // per block: E = floor(block max - m) - 7, or flushed (fully masked, or E < -127)
  float bias[2], eb[2];
  const float Bm[2] = {B0, B1};
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    bool flush = MASK && ((Bm[b] == NEG_INF) || (m_new == NEG_INF));
    float e = flush ? 0.f : __builtin_floorf(Bm[b] - m_new) - (float)k8PExp;
    flush = flush || e < -127.f;
    eb[b] = flush ? 0.f : e;
    bias[b] = flush ? __builtin_inff() : m_new + e;
  }
  sbyte = (uint32_t)((int)(h ? eb[1] : eb[0]) + 127);    // this lane scales block h

#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float y[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int el = 4 * w + q;                // byte index = 16mb + r
      const int mb = el >> 4, r = el & 15;
      float x = __builtin_fmaf(s[mb][r], c, -bias[mb]);
      if constexpr (MASK) x = visible(mb, r) ? x : NEG_INF;
      y[q] = __builtin_amdgcn_exp2f(x);
    }
    // the second convert overwrites the high half, so the first one starts from the
    // word's old contents rather than a zeroed register
    const s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
        __builtin_bit_cast(s16x2, codes[w >> 2][w & 3]), y[0], y[1], 1.0f, false);
    codes[w >> 2][w & 3] = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[2], y[3], 1.0f, true));
  }
  return any;
}

template <bool CAUSAL, bool BAND>
__global__ __attribute__((amdgpu_flat_work_group_size(k8Threads, k8Threads), amdgpu_waves_per_eu(2, 2)))
void fwd_mxfp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ QS,
                      const uint8_t* __restrict__ K8, const uint8_t* __restrict__ KS,
                      const uint8_t* __restrict__ VT8, const uint8_t* __restrict__ VTS,
                      float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int N,
                      int nqb, float c, float tau, uint32_t qsign, int window,
                      const int* __restrict__ doc_off, int n_docs,
                      unsigned long long* __restrict__ stats) {
  __shared__ F8Buf buf[2];
  const float NEG_INF = -__builtin_inff();
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index through readfirstlane: the scale staging roles are whole waves
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, h = lane >> 5;

  const int group = Hq / Hkv;
  const unsigned long long clk0 = __builtin_amdgcn_s_memtime();
  const unsigned long long ref0 = __builtin_amdgcn_s_memrealtime();
  const WorkItem wi = decode_workgroup(blockIdx.x, gridDim.x, Hkv, group, nqb, CAUSAL);
  const int b = wi.b, hkv = wi.hkv, g = wi.g;
  const int qb = CAUSAL ? (nqb - 1 - wi.qb_rank) : wi.qb_rank;
  const int hq = hkv * group + g;
  const int Q0 = qb * k8Br;
  const int q0 = Q0 + wave * k8Rows;
  const int qi = q0 + n32;

  const size_t qhead = (size_t)(b * Hq + hq) * N;
  const size_t khead = (size_t)(b * Hkv + hkv) * N;
  const uint8_t* K8h = K8 + khead * k8CodeRow;
  const uint8_t* KSh = KS + khead * k8ScaleRow;
  const uint8_t* VT8h = VT8 + khead * k8CodeRow;      // [k8D][N] per head
  const uint8_t* VTSh = VTS + khead * k8ScaleRow;     // [k8D][N/32] per head
  const int nvb = N / 32;                             // V scale bytes per column
  const __amdgpu_buffer_rsrc_t rvt = rsrc8(VT8h, k8D * N);
  const __amdgpu_buffer_rsrc_t rvs = rsrc8(VTSh, k8D * nvb);

  // Q codes: for each 64-wide d chunk kc the lane holds d 64kc + 16h .. +15 and
  // 64kc + 32 + 16h .. +15 of query qi (B operand of QK); byte 2kc of qsc is the scale
  // of d block 2kc + h, the k-block this lane scales.
  i32x8 qc[2];
  uint32_t qsc;
  {
    const int qr = min(qi, N - 1);
    const uint8_t* qrow = Q8 + (qhead + qr) * k8CodeRow;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x4 lo = *(const u32x4*)(qrow + 64 * kc + 16 * h) ^ qsign;
      const u32x4 hi = *(const u32x4*)(qrow + 64 * kc + 32 + 16 * h) ^ qsign;
      qc[kc] = fp8_operand(lo, hi);
    }
    const uint8_t* srow = QS + (qhead + qr) * k8ScaleRow;
    qsc = ((uint32_t)srow[0] | ((uint32_t)srow[1] << 8) | ((uint32_t)srow[2] << 16) |
           ((uint32_t)srow[3] << 24)) >> (8 * h);
  }

  f32x16 acc[k8D / 32], lacc;
#pragma unroll
  for (int i = 0; i < k8D / 32; ++i) acc[i] = zero16();
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
    row_bounds(min(Q0 + k8Br - 1, N - 1), wg_lo_last, wg_hi_last);
    row_bounds(min(q0, N - 1), w_lo, unused);
    row_bounds(min(q0 + k8Rows - 1, N - 1), unused, w_hi);
  }
  // tiles t0 .. t0 + n - 1 (local index j = tile - t0)
  const int t0 = BAND ? wg_lo_first / k8Bc : 0;
  const int kv_end = BAND ? wg_hi_last + 1 : (CAUSAL ? min(N, Q0 + k8Br) : N);
  const int n = (kv_end + k8Bc - 1) / k8Bc - t0;
  const int wave_end = BAND ? w_hi + 1 : (CAUSAL ? min(N, q0 + k8Rows) : N);
  const bool wave_live = q0 < N;

  const int krs = tid >> 3, kcs = tid & 7;     // K staging unit of this thread
  const int vcs = tid >> 2, vch = tid & 3;     // V^T staging unit of this thread

  // Stage t (read by pipeline step t from buffer t & 1) holds K tile t and V tile t-1.
  // Every thread stages one code unit of K, one of V^T and one scale byte; the loads are
  // unconditional, with the tile index clamped into [0, n) (in bounds), and so are the
  // stores: a stage past the tiles lands in a buffer half no later product reads.  The
  // scale's source (K or V^T) is a wave-uniform select, so the step has no branches.
  auto load_stage = [&](F8Stage& sg, int t) {
    const int kt = min(t, n - 1), vt = max(min(t - 1, n - 1), 0);
    const int kk0 = (t0 + kt) * k8Bc, vk0 = (t0 + vt) * k8Bc;
    const __amdgpu_buffer_rsrc_t rk = rsrc8(K8h + (size_t)kk0 * k8CodeRow, (N - kk0) * k8CodeRow);
    sg.k = __builtin_amdgcn_raw_buffer_load_b128(rk, krs * k8CodeRow + kcs * 16, 0, 0);
    // keys past N in the last tile read the next column's codes (finite; they meet zero
    // weights) or, past the head, zeros from the range check
    sg.v = __builtin_amdgcn_raw_buffer_load_b128(rvt, vcs * N + vk0 + 16 * vch, 0, 0);
    const bool kpart = wave < 4;                      // tid < 256: a K scale byte
    const int u = tid - 256, col = u >> 1, hb = u & 1;
    // a V key block past N gets a neutral scale; the load reads block 0 then (in range)
    const bool past = vk0 + 32 * hb >= N;
    const __amdgpu_buffer_rsrc_t rs =
        kpart ? rsrc8(KSh + (size_t)kk0 * k8ScaleRow, (N - kk0) * k8ScaleRow) : rvs;
    const int off = kpart ? tid : col * nvb + (past ? 0 : vk0 / 32 + hb);
    const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
    sg.sc = (!kpart && past) ? 127u : byte;
  };
  auto store_stage = [&](const F8Stage& sg, int t) {
    F8Buf& bb = buf[t & 1];
    sts16(bb.kcode + kpos8(krs) * k8KStride + 16 * kcs, sg.k);
    sts16(bb.vcode + vcs * k8VStride + 16 * vch, sg.v);
    bb.scale[tid] = (uint8_t)sg.sc;
  };

  // per-lane LDS byte offsets of the operand reads (chunk and column-block offsets
  // are compile-time immediates)
  const int kr0 = krow8(0, n32), kr1 = krow8(1, n32);
  const int ka0 = kpos8(kr0) * k8KStride + 16 * h, ka1 = kpos8(kr1) * k8KStride + 16 * h;
  const int va = n32 * k8VStride + 16 * h;
  const uint32_t ONES = 0x38383838u;           // E4M3 1.0 in every byte
  // the all-ones A operand of the row-sum product, built once: opaque to the compiler, so
  // it stays in its registers instead of being rebuilt before every product
  i32x8 ones8 = fp8_operand(u32x4{ONES, ONES, ONES, ONES}, u32x4{ONES, ONES, ONES, ONES});
  asm volatile("" : "+v"(ones8));

  // MFMAs of one pipeline step: QK of this step's tile into sn (K from bb), then PV and
  // row sum of the previous tile (P codes pp, P scale byte ep, V^T from bb).  The PV
  // products cover the latency of the QK results the weights wait for.
  auto mfmas = [&](const F8Buf& bb, const u32x4 (&pp)[2], uint32_t ep, bool pv, bool qk,
                   f32x16 (&sn)[2]) {
    if (qk) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = mb ? kr1 : kr0;
        const uint8_t* kp = bb.kcode + (mb ? ka1 : ka0);
        const int ksc = (int)(*(const uint32_t*)(bb.scale + 4 * row) >> (8 * h));
        // d elements 0..63 (scale byte 0 of the shifted scale words), then 64..127 (byte 2)
        const u32x4 a00 = lds16(kp), a01 = lds16(kp + 32);
        const u32x4 a10 = lds16(kp + 64), a11 = lds16(kp + 96);
        f32x16 a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fp8_operand(a00, a01), qc[0], zero16(), 0, 0, 0, ksc, 0, (int)qsc);
        a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp8_operand(a10, a11), qc[1], a, 0, 0,
                                                            2, ksc, 2, (int)qsc);
        sn[mb] = a;
      }
    }
    if (pv) {
      const i32x8 bp = fp8_operand(pp[0], pp[1]);
#pragma unroll
      for (int cb = 0; cb < k8D / 32; ++cb) {
        const int col = 32 * cb + n32;
        const uint8_t* vp = bb.vcode + va + 32 * cb * k8VStride;
        const u32x4 v0 = lds16(vp), v1 = lds16(vp + 32);
        const int vs = bb.scale[4 * k8Bc + col * 2 + h];
        acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp8_operand(v0, v1), bp,
                                                                  acc[cb], 0, 0, 0, vs, 0,
                                                                  (int)ep);
      }
      lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, bp, lacc, 0, 0, 0, 127, 0,
                                                             (int)ep);
    }
  };

  // ---- prologue: stage 0 (K tile 0; no V tile precedes it) -> buffer 0; stage 1 in
  //      registers ----
  F8Stage stg;
  load_stage(stg, 0);
  store_stage(stg, 0);
  // zero V codes and neutral V scales, written by the same threads that stored this half
  sts16(buf[0].vcode + vcs * k8VStride + 16 * vch, u32x4{0u, 0u, 0u, 0u});
  if (!(wave < 4)) buf[0].scale[tid] = 127;
  load_stage(stg, 1);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // P codes and scale of the latest tile: written by the weights of step j, read by the
  // PV product of step j + 1 before the weights of that step overwrite them
  u32x4 p[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  uint32_t ep = 127u;

  bool any_prev = false;
  float alpha_prev = 1.f;
  // unmasked tiles [lo_full, n_full): every row of the workgroup sees all their keys
  const int n_full = BAND ? (wg_hi_first + 1) / k8Bc - t0 : (CAUSAL ? min(Q0, N) / k8Bc : N / k8Bc);
  const int lo_full = BAND ? min(n, (wg_lo_last + k8Bc - 1) / k8Bc - t0) : 0;
  // rescale decisions that fired; every step's decision passes through rescale() once
  unsigned n_fires = 0;
  auto rescale = [&]() {
    if (any_prev) {
#pragma unroll
      for (int i = 0; i < k8D / 32; ++i) acc[i] *= alpha_prev;
      lacc *= alpha_prev;
      ++n_fires;
    }
  };
  // Pipeline step j: QK of tile j, PV and row sum of tile j-1, weights of tile j; then
  // the staging of stage j+1 and the barrier.  S lives only within the step.
  auto step = [&](int j, bool pv, bool masked) {
    rescale();
    f32x16 s[2];
    mfmas(buf[j & 1], p, ep, pv, true, s);
    float alpha;
    bool any;
    if (masked)
      any = fp8p_tile<CAUSAL, true, BAND>(s, p, ep, m, alpha, (t0 + j) * k8Bc, qi, N, c, tau, h,
                                          klo, khi);
    else
      any = fp8p_tile<CAUSAL, false, BAND>(s, p, ep, m, alpha, (t0 + j) * k8Bc, qi, N, c, tau,
                                           h, klo, khi);
    any_prev = any;
    alpha_prev = alpha;
    store_stage(stg, j + 1);
    load_stage(stg, j + 2);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // step 0 has no PV product (no tile before it); then the unmasked steps, then the
  // masked ones (causal diagonal, ragged tail)
  if constexpr (BAND) {
    // masked below lo_full (some row's lower edge) and from n_full on
    step(0, false, 0 < lo_full || 0 >= n_full);
    for (int j = 1; j < n; ++j) step(j, true, j < lo_full || j >= n_full);
  } else {
    step(0, false, 0 >= n_full);
    int j = 1;
    for (; j < min(n_full, n); ++j) step(j, true, false);
    for (; j < n; ++j) step(j, true, true);
  }
  // PV and row sum of the last tile (its V^T was staged by the last step into buffer n&1)
  rescale();
  {
    f32x16 unused[2];
    mfmas(buf[n & 1], p, ep, true, false, unused);
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * m + ln l ----
  const float l = lacc[0];
  if (qi < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* Orow = O + (qhead + qi) * k8D;
#pragma unroll
    for (int cb = 0; cb < k8D / 32; ++cb)
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
    const int j_hi = min(n, (wave_end + k8Bc - 1) / k8Bc - t0);
    const int j_lo = BAND ? max(0, w_lo / k8Bc - t0) : 0;
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
hipError_t launch_mxfp8(const MxArgs& a) {
  const int nqb = (a.N + k8Br - 1) / k8Br;
  const long long grid = (long long)a.B * a.Hq * nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_mxfp8_kernel<CAUSAL, BAND>), dim3((unsigned)grid), dim3(k8Threads), 0,
                     (hipStream_t)a.stream, a.qc, a.qs, a.kc, a.ks, a.vtc, a.vts, a.o, a.lse,
                     a.Hq, a.Hkv, a.N, nqb, a.c, a.tau, a.qsign, a.window, a.doc_offsets,
                     a.n_docs, a.stats);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize8_rows(const float* x, uint8_t* codes, uint8_t* scales, long long rows,
                                 int cols, void* stream) {
  const long long nblocks = rows * (cols / 32);
  const int threads = 256;
  const long long grid = (nblocks + threads - 1) / threads;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize8_rows_kernel, dim3((unsigned)grid), dim3(threads), 0,
                     (hipStream_t)stream, x, codes, scales, nblocks);
  return hipGetLastError();
}

hipError_t launch_quantize8_cols_t(const float* x, uint8_t* codes, uint8_t* scales, int batch,
                                   int rows, int cols, void* stream) {
  const long long total = (long long)batch * (rows / 32) * cols;
  const int threads = 256;
  const long long grid = (total + threads - 1) / threads;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize8_cols_t_kernel, dim3((unsigned)grid), dim3(threads), 0,
                     (hipStream_t)stream, x, codes, scales, rows, cols, total);
  return hipGetLastError();
}

hipError_t launch_fwd_mxfp8(const MxArgs& a) {
  if (a.d != k8D) return hipErrorNotSupported;
  const bool band = a.window > 0 || a.n_docs > 0;
  if (a.causal) return band ? launch_mxfp8<true, true>(a) : launch_mxfp8<true, false>(a);
  return band ? launch_mxfp8<false, true>(a) : launch_mxfp8<false, false>(a);
}

}  // namespace attn
