// bf16 fused attention forward for gfx950 (CDNA4).
//
// One workgroup = 4 waves = 128 query rows of one (batch, query head); each
// wave owns 32 query rows.  K/V are streamed through LDS in tiles of 64 keys
// (double buffered; the next tile's global loads are in flight while the
// current tile is computed), so the N x N score matrix never leaves
// registers ("FlashAttention-4发布：原生支持Blackwell…", section "从V1到V4",
// FlashAttention (2022) entry).  Both products run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//
//   S^T = K Q^T   A = K tile from LDS (rows permuted, see below), B = Q in VGPRs
//   O^T += V^T P^T  A = V^T tile from LDS, B = P straight from the S^T registers
//
// Computing the transposed score tile puts one query per lane (lane % 32) and
// 16 keys per 32-key block in that lane's registers, so the row max and row
// sum are in-lane plus one exchange with lane ^ 32, and the rescale factor is
// a per-lane scalar.  K rows are read in an order that swaps bits 2 and 3 of
// the row index; with it the 8 consecutive accumulator registers of a lane
// hold 8 consecutive keys, which is exactly the B-operand layout of the PV
// product, so P needs no shuffle between the two MFMAs.
//
// Online softmax with a rescale threshold ("FlashAttention-4 de NVIDIA…",
// section "La ventaja técnica"; aigc.bar page, section "FlashAttention-4：为
// Blackwell而生的性能猛兽", item 1): the running maximum m (log2 units) is
// only raised, and O and l only rescaled, when some row's tile maximum exceeds
// m + tau; otherwise the weights 2^(t - m) may reach 2^tau, which fp32
// accumulation absorbs.  The result is the same in exact arithmetic.
//
// The exponential is either the hardware v_exp_f32 or a VALU cubic
// ("FlashAttention-4 de NVIDIA…", section "La ventaja técnica": cubic
// polynomials on the FMA units instead of the special-function unit).

#include "common.h"
#include "exp2_poly.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBc = 64;                     // keys per K/V tile
constexpr int kThreads = kWaves * 64;
constexpr int kVtStride = kBc + 8;          // padded V^T row (elements): 144 B, conflict-free reads

__device__ __forceinline__ float exp2_poly(float x) {
  // 2^x = 2^n * p(f), n = floor(x), f = x - n; x clamped at -126 so the
  // exponent add cannot wrap (the result is then below 2^-125, i.e. ~0).
  x = fmaxf(x, -126.0f);
  const float n = __builtin_floorf(x);
  const float f = x - n;
  const float p = __builtin_fmaf(f, __builtin_fmaf(f, __builtin_fmaf(f, ATTN_EXP2_C3, ATTN_EXP2_C2),
                                                   ATTN_EXP2_C1), 1.0f);
  return __int_as_float(__float_as_int(p) + ((int)n << 23));
}

template <bool POLY>
__device__ __forceinline__ float exp2_sel(float x) {
  if constexpr (POLY) return exp2_poly(x);
  else return __builtin_amdgcn_exp2f(x);
}

// Row of the K tile read by MFMA row m of a 32-row block: bits 2 and 3 swapped.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D>
struct TileRegs {
  static constexpr int kChunks = kBc * D / 8;            // 16-byte chunks in a K tile
  static constexpr int kPerThread = kChunks / kThreads;  // K chunks per thread
  u32x4 k[kPerThread];
  u32x2 v[8];                                            // 8 keys x 4 columns of V
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* __restrict__ Kh,
                                          const uint16_t* __restrict__ Vh, int kv0, int N, int tid) {
  constexpr int NCH = D / 8;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kPerThread; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / NCH, ch = idx % NCH;
    const int key = kv0 + row;
    u32x4 z = {0u, 0u, 0u, 0u};
    r.k[i] = key < N ? *(const u32x4*)(Kh + (size_t)key * D + ch * 8) : z;
  }
  constexpr int CG = D / 4;  // 4-column groups per row
  if (tid < (kBc / 8) * CG) {
    const int cg = tid % CG, kg = tid / CG;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kv0 + kg * 8 + e;
      u32x2 z = {0u, 0u};
      r.v[e] = key < N ? *(const u32x2*)(Vh + (size_t)key * D + cg * 4) : z;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, u32x4* __restrict__ sk,
                                           u32x4* __restrict__ svt, int tid) {
  constexpr int NCH = D / 8;
  constexpr int SWZ = (NCH < 16 ? NCH : 16) - 1;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kPerThread; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / NCH, ch = idx % NCH;
    sk[row * NCH + (ch ^ (row & SWZ))] = r.k[i];
  }
  constexpr int CG = D / 4;
  if (tid < (kBc / 8) * CG) {
    const int cg = tid % CG, kg = tid / CG;
    // transpose 8 keys x 4 columns into 4 columns x 8 keys
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int w = c >> 1;
      u32x4 out;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = r.v[2 * p][w], b = r.v[2 * p + 1][w];
        out[p] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      }
      const int col = cg * 4 + c;
      svt[(col * kVtStride + kg * 8) / 8] = out;
    }
  }
}

template <int D, bool CAUSAL, bool POLY>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                     int Hq, int Hkv, int N, int nqb, float c, float tau, uint32_t qsign,
                     unsigned long long* __restrict__ stats) {
  constexpr int NCH = D / 8;
  constexpr int SWZ = (NCH < 16 ? NCH : 16) - 1;
  __shared__ u32x4 sk[2][kBc * D / 8];
  __shared__ u32x4 svt[2][D * kVtStride / 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = lane & 31, h = lane >> 5;

  // Workgroup -> (batch, kv head, query block, query head in the group).  Workgroups
  // are dealt round-robin to the 8 XCDs; renumber so each XCD gets a contiguous
  // range, in which the query heads of one kv head and neighbouring query blocks
  // sit together and share K/V tiles in that XCD's L2.  Causal: heaviest blocks first.
  const int G = gridDim.x, w = blockIdx.x;
  const int L = (G % 8 == 0) ? (w % 8) * (G / 8) + (w / 8) : w;
  const int group = Hq / Hkv;
  const int g = L % group;
  const int t1 = L / group;
  const int qb_rank = t1 % nqb;
  const int t2 = t1 / nqb;
  const int hkv = t2 % Hkv, b = t2 / Hkv;
  const int hq = hkv * group + g;
  const int qb = CAUSAL ? (nqb - 1 - qb_rank) : qb_rank;

  const int Q0 = qb * kBr;
  const int q0 = Q0 + wave * kRowsPerWave;
  const int qi = q0 + n32;
  const uint16_t* Qh = Q + ((size_t)(b * Hq + hq) * N) * D;
  const uint16_t* Kh = K + ((size_t)(b * Hkv + hkv) * N) * D;
  const uint16_t* Vh = V + ((size_t)(b * Hkv + hkv) * N) * D;

  // Q fragment: B operand of S^T = K Q^T, lane holds Q[qi][16t + 8h .. +7].
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    u32x4 z = {0u, 0u, 0u, 0u};
    u32x4 x = qi < N ? *(const u32x4*)(Qh + (size_t)qi * D + 16 * t + 8 * h) : z;
    x ^= qsign;
    qf[t] = as_bf16x8(x);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = zero16();
  float m_ref = -__builtin_inff();
  float lsum = 0.f;
  unsigned steps = 0, rescales = 0;
  bool first = true;

  const int kv_end = CAUSAL ? min(N, Q0 + kBr) : N;
  const int ntiles = (kv_end + kBc - 1) / kBc;

  TileRegs<D> regs;
  load_tile<D>(regs, Kh, Vh, 0, N, tid);
  store_tile<D>(regs, sk[0], svt[0], tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * kBc;
    if (j + 1 < ntiles) load_tile<D>(regs, Kh, Vh, kv0 + kBc, N, tid);

    const bool active = (!CAUSAL || kv0 <= q0 + kRowsPerWave - 1) && q0 < N;
    if (active) {
      const u32x4* kb = sk[j & 1];
      const u32x4* vb = svt[j & 1];

      // ---- S^T = K Q^T for 64 keys x 32 queries ----
      f32x16 s[2] = {zero16(), zero16()};
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int row = mb * 32 + perm_row(n32);
          const int ch = 2 * t + h;
          const bf16x8 a = as_bf16x8(kb[row * NCH + (ch ^ (row & SWZ))]);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[mb], 0, 0, 0);
        }
      }
      // register r of block mb holds key kv0 + 32*mb + 16*(r/8) + 8*h + r%8

      const bool masked = (CAUSAL && kv0 + kBc - 1 > q0) || (kv0 + kBc > N);
      unsigned long long valid = ~0ull;  // bit (mb*16 + r)
      if (masked) {
        valid = 0ull;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * mb + 16 * (r >> 3) + 8 * h + (r & 7);
            const bool ok = key < N && (!CAUSAL || key <= qi);
            if (ok) valid |= 1ull << (mb * 16 + r);
            else s[mb][r] = -__builtin_inff();
          }
      }

      float mx = -__builtin_inff();
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
      mx = max_across_halves(mx);
      const float mt = (mx == -__builtin_inff()) ? mx : mx * c;

      if (!first) ++steps;
      const bool need = mt > m_ref + tau;
      if (__ballot(need)) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = (m_new == -__builtin_inff()) ? 1.f : exp2_sel<POLY>(m_ref - m_new);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
        lsum *= alpha;
        m_ref = m_new;
        if (!first) ++rescales;
      }
      first = false;
      const float mu = (m_ref == -__builtin_inff()) ? 0.f : m_ref;

      // ---- P = 2^(t - m) as the bf16 B operand, one 16-key step per 8 registers ----
      bf16x8 p[4];
      float part = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int r = hf * 8 + e;
            float e0 = exp2_sel<POLY>(__builtin_fmaf(s[mb][r], c, -mu));
            float e1 = exp2_sel<POLY>(__builtin_fmaf(s[mb][r + 1], c, -mu));
            if (masked) {
              e0 = (valid >> (mb * 16 + r)) & 1 ? e0 : 0.f;
              e1 = (valid >> (mb * 16 + r + 1)) & 1 ? e1 : 0.f;
            }
            part += e0 + e1;
            pk[e / 2] = pack_bf16x2(e0, e1);
          }
          p[mb * 2 + hf] = as_bf16x8(pk);
        }
      lsum += part;

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int col = cb * 32 + n32;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a = as_bf16x8(vb[(col * kVtStride + 16 * ks + 8 * h) / 8]);
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[ks], acc[cb], 0, 0, 0);
        }
      }
    }

    if (j + 1 < ntiles) store_tile<D>(regs, sk[(j + 1) & 1], svt[(j + 1) & 1], tid);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) ----
  const float ltot = sum_across_halves(lsum);
  if (qi < N) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float* Orow = O + ((size_t)(b * Hq + hq) * N + qi) * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 out = {acc[cb][4 * a4] * inv, acc[cb][4 * a4 + 1] * inv, acc[cb][4 * a4 + 2] * inv,
                     acc[cb][4 * a4 + 3] * inv};
        *(f32x4*)(Orow + cb * 32 + 8 * a4 + 4 * h) = out;
      }
    if (h == 0)
      LSE[(size_t)(b * Hq + hq) * N + qi] =
          ltot > 0.f ? (m_ref + __builtin_log2f(ltot)) * kLn2 : -__builtin_inff();
  }
  if (stats != nullptr && lane == 0 && q0 < N) {
    atomicAdd(stats, (unsigned long long)steps);
    atomicAdd(stats + 1, (unsigned long long)rescales);
  }
}

template <int D, bool CAUSAL, bool POLY>
hipError_t launch_one(const FwdArgs& a) {
  const int nqb = (a.N + kBr - 1) / kBr;
  const long long grid = (long long)a.B * a.Hq * nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, POLY>), dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.o, a.lse, a.Hq, a.Hkv, a.N, nqb, a.c, a.tau, a.qsign,
                     a.stats);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  const bool poly = a.exp_mode == 1;
  if (a.d == 128) {
    if (a.causal) return poly ? launch_one<128, true, true>(a) : launch_one<128, true, false>(a);
    return poly ? launch_one<128, false, true>(a) : launch_one<128, false, false>(a);
  }
  if (a.causal) return poly ? launch_one<64, true, true>(a) : launch_one<64, true, false>(a);
  return poly ? launch_one<64, false, true>(a) : launch_one<64, false, false>(a);
}

}  // namespace attn
