// bf16 fused attention forward for gfx950 (CDNA4).
//
// Work split.  One workgroup = 8 waves = 256 query rows of one (batch, query
// head); each wave owns 32 query rows, so every SIMD runs two waves and the
// hardware interleaves one wave's softmax (VALU) with the other's matrix
// products (MFMA).  K/V are streamed through LDS in tiles of 128 keys, double
// buffered: while tile j is computed, tile j+1 is already in flight, so the
// N x N score matrix never leaves registers ("FlashAttention-4发布：原生支持
// Blackwell…", section "从V1到V4", FlashAttention (2022) entry).
//
// Products.  Both run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//   S^T  = K Q^T     A = K tile from LDS (rows permuted, see perm_row), B = Q in VGPRs
//   O^T += V^T P^T   A = V^T tile from LDS,                             B = P in VGPRs
// The transposed score tile puts one query per lane (lane % 32) and, per
// 32-key block, 16 keys in that lane's registers: the row max and row sum are
// in-lane plus one swap with lane ^ 32, and the rescale factor is a per-lane
// scalar.  Reading K rows with bits 2 and 3 of the row index swapped makes 8
// consecutive accumulator registers hold 8 consecutive keys, which is the
// B-operand layout of the PV product, so P goes from S to the next MFMA with
// no data movement.
//
// Staging.  K goes global -> LDS with direct 16-byte loads (no VGPRs), in an
// XOR-swizzled layout that makes the MFMA operand reads bank-conflict free.
// V is read with coalesced 4-byte loads, transposed in registers and written
// as V^T (the PV A operand needs 8 consecutive keys of one column per lane),
// again swizzled so both the writes and the reads are conflict free.
//
// Softmax.  Online, in log2 units, with a rescale threshold
// ("FlashAttention-4 de NVIDIA…", section "La ventaja técnica"; aigc.bar page,
// section "FlashAttention-4：为Blackwell而生的性能猛兽", item 1): the running max
// m is only raised, and O and l only rescaled, when some row's tile max exceeds
// m + tau; otherwise the weights 2^(t - m) may reach 2^tau, which fp32
// accumulation absorbs.  Exact in exact arithmetic.  The row sum is taken over
// the fp32 weights (before the bf16 rounding the PV operand needs), so the LSE
// carries no bf16 rounding noise.
//
// Exponential: hardware v_exp_f32, or a VALU cubic ("FlashAttention-4 de
// NVIDIA…", section "La ventaja técnica": cubic polynomials on the FMA units
// instead of the special-function unit), selectable for comparison.

#include "common.h"
#include "exp2_poly.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 8;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // 256 query rows per workgroup
constexpr int kBc = 128;                    // keys per K/V tile in LDS
constexpr int kSub = 64;                    // keys per compute step (online-softmax update)
constexpr int kThreads = kWaves * 64;

template <int D>
struct Geo {
  static constexpr int NCH = D / 8;                        // 16-byte chunks per K row
  static constexpr int KCH = kBc * NCH;                    // 16-byte chunks per K tile
  static constexpr int KDMA_PER_WAVE = KCH / 64 / kWaves;  // 1 KiB direct loads per wave
  static constexpr int VKC = kBc / 8;                      // 8-key chunks per tile
  static constexpr int VCH = D * VKC;                      // 16-byte chunks per V^T tile
  static constexpr int CP = D / 2;                         // column pairs of a V row
  static constexpr int KG_STRIDE = kThreads / CP;          // key groups covered per pass
  static constexpr int KG_PER_THREAD = (kBc / 8) / KG_STRIDE;
  static_assert(KCH % (64 * kWaves) == 0, "K tile must split into whole direct loads");
  static_assert(kBc % 64 == 0, "a direct load covers 64 rows of one chunk column");
  static_assert(KG_PER_THREAD >= 1 && (kBc / 8) % KG_STRIDE == 0, "V staging split");
};

// Raw buffer descriptor over `bytes` bytes at `base`: loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

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

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS layouts (16-byte units):
//   K tile   sk[c * kBc + r]   c = 16-byte chunk of the d axis, r = key row
//   V^T tile svt[kc * D + col] kc = group of 8 keys, col = d column
// In both, the 16 lanes that the LDS serves together read 16 consecutive units
// (bank-conflict free), and an operand's address is one per-lane base plus a
// compile-time offset.

// K tile -> LDS with direct 16-byte loads: each load fills one chunk column for
// 64 consecutive rows.  Rows past N come back as zeros (their scores are masked).
template <int D>
__device__ __forceinline__ void issue_k_tile(u32x4* sk, __amdgpu_buffer_rsrc_t rk, const int* koff,
                                             int wave) {
  using G = Geo<D>;
#pragma unroll
  for (int i = 0; i < G::KDMA_PER_WAVE; ++i) {
    const int g0 = (wave * G::KDMA_PER_WAVE + i) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rk, (__attribute__((address_space(3))) void*)(sk + g0), 16, koff[i], 0, 0, 0);
  }
}

// Per-lane byte offsets (within a K tile) of this wave's direct loads.
template <int D>
__device__ __forceinline__ void k_offsets(int* koff, int wave, int lane) {
  using G = Geo<D>;
#pragma unroll
  for (int i = 0; i < G::KDMA_PER_WAVE; ++i) {
    const int g0 = (wave * G::KDMA_PER_WAVE + i) * 64;
    const int c = g0 / kBc, r = g0 % kBc + lane;
    koff[i] = r * D * 2 + c * 16;
  }
}

template <int D>
struct VRegs {
  uint32_t w[Geo<D>::KG_PER_THREAD][8];
};

// V tile: thread (cp, kg) reads columns 2cp, 2cp+1 of keys 8kg .. 8kg+7 (each load
// instruction covers whole rows: coalesced).  Rows past N come back as zeros.
template <int D>
__device__ __forceinline__ void load_v_tile(VRegs<D>& r, __amdgpu_buffer_rsrc_t rv, int voff) {
  using G = Geo<D>;
#pragma unroll
  for (int kk = 0; kk < G::KG_PER_THREAD; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r.w[kk][e] = __builtin_amdgcn_raw_buffer_load_b32(
          rv, voff + (8 * kk * G::KG_STRIDE + e) * D * 2, 0, 0);
}

template <int D>
__device__ __forceinline__ void store_v_tile(const VRegs<D>& r, u32x4* svt, int tid) {
  using G = Geo<D>;
  const int cp = tid % G::CP, kgb = tid / G::CP;
#pragma unroll
  for (int kk = 0; kk < G::KG_PER_THREAD; ++kk) {
    const int kg = kgb + kk * G::KG_STRIDE;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4 out;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = r.w[kk][2 * p], b = r.w[kk][2 * p + 1];
        out[p] = cc ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      }
      svt[kg * D + 2 * cp + cc] = out;
    }
  }
}

struct RowState {
  float m;       // running max, log2 units (-inf before the first visible key)
  float l;       // this lane's partial row sum (keys of its half of each block)
  unsigned steps, rescales;
  bool first;
};

// One 64-key step (keys kv0 .. kv0+63, at key offset `sub` of the LDS tile) for
// this wave's 32 query rows.
template <int D, bool CAUSAL, bool POLY, bool MASK>
__device__ __forceinline__ void tile_step(const u32x4* __restrict__ kb,
                                          const u32x4* __restrict__ vb,
                                          const bf16x8 (&qf)[D / 16], f32x16 (&acc)[D / 32],
                                          RowState& st, int sub, int kv0, int qi, int N, float c,
                                          float tau, int n32, int h) {
  using G = Geo<D>;
  constexpr int MB = kSub / 32;  // 32-key blocks per step
  const float NEG_INF = -__builtin_inff();

  // ---- S^T = K Q^T ----
  f32x16 s[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) s[mb] = zero16();
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = sub + mb * 32 + perm_row(n32);
      const bf16x8 a = as_bf16x8(kb[(2 * t + h) * kBc + row]);
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[mb], 0, 0, 0);
    }
  }
  // register r of block mb holds key kv0 + 32*mb + 16*(r/8) + 8*h + r%8

  if constexpr (MASK) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * mb + 16 * (r >> 3) + 8 * h + (r & 7);
        const bool ok = key < N && (!CAUSAL || key <= qi);
        s[mb][r] = ok ? s[mb][r] : NEG_INF;
      }
  }

  float mx = NEG_INF;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
  mx = half_swap_max(mx);
  const float mt = (mx == NEG_INF) ? NEG_INF : mx * c;

  if (!st.first) ++st.steps;
  if (__ballot(mt > st.m + tau)) {
    const float m_new = fmaxf(st.m, mt);
    const float alpha = (m_new == NEG_INF) ? 1.f : exp2_sel<POLY>(st.m - m_new);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
    st.l *= alpha;
    st.m = m_new;
    if (!st.first) ++st.rescales;
  }
  st.first = false;
  const float mu = (st.m == NEG_INF) ? 0.f : st.m;

  // ---- P = 2^(t - m), packed as the bf16 B operand (one 16-key step per 8 registers) ----
  bf16x8 p[kSub / 16];
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float s0 = s[mb][hf * 8 + 2 * e], s1 = s[mb][hf * 8 + 2 * e + 1];
        float e0 = exp2_sel<POLY>(__builtin_fmaf(s0, c, -mu));
        float e1 = exp2_sel<POLY>(__builtin_fmaf(s1, c, -mu));
        if constexpr (MASK) {
          e0 = (s0 == NEG_INF) ? 0.f : e0;
          e1 = (s1 == NEG_INF) ? 0.f : e1;
        }
        pk[e] = pack_bf16x2(e0, e1);
        ls[e] += e0 + e1;
      }
      p[mb * 2 + hf] = as_bf16x8(pk);
    }
  st.l += (ls[0] + ls[1]) + (ls[2] + ls[3]);

  // ---- O^T += V^T P^T ----
#pragma unroll
  for (int ks = 0; ks < kSub / 16; ++ks) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int col = cb * 32 + n32;
      const int kc = sub / 8 + 2 * ks + h;
      const bf16x8 a = as_bf16x8(vb[kc * D + col]);
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[ks], acc[cb], 0, 0, 0);
    }
  }
}

template <int D, bool CAUSAL, bool POLY>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                     int Hq, int Hkv, int N, int nqb, float c, float tau, uint32_t qsign,
                     unsigned long long* __restrict__ stats) {
  using G = Geo<D>;
  __shared__ u32x4 sk[2][G::KCH];
  __shared__ u32x4 svt[2][G::VCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = lane & 31, h = lane >> 5;

  // Workgroup -> (batch, kv head, query block, query head in the group).  Workgroups
  // are dealt round-robin to the 8 XCDs; renumber so each XCD gets a contiguous
  // range, in which the query heads of one kv head and neighbouring query blocks
  // sit together and share K/V tiles in that XCD's L2.  Causal: heaviest blocks first.
  const int G_ = gridDim.x, w = blockIdx.x;
  const int L = (G_ % 8 == 0) ? (w % 8) * (G_ / 8) + (w / 8) : w;
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
  {
    const int qc = min(qi, N - 1);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      u32x4 x = *(const u32x4*)(Qh + (size_t)qc * D + 16 * t + 8 * h);
      x ^= qsign;
      qf[t] = as_bf16x8(x);
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = zero16();
  RowState st{-__builtin_inff(), 0.f, 0u, 0u, true};

  const int kv_end = CAUSAL ? min(N, Q0 + kBr) : N;
  const int ntiles = (kv_end + kBc - 1) / kBc;

  // Per-tile buffer descriptors: rows at or past N read as zeros.
  auto tile_rsrc = [&](const uint16_t* head, int kv0) {
    return make_rsrc(head + (size_t)kv0 * D, (N - kv0) * D * 2);
  };
  int koff[G::KDMA_PER_WAVE];
  k_offsets<D>(koff, wave, lane);
  const int voff = ((8 * (tid / G::CP)) * D + 2 * (tid % G::CP)) * 2;

  VRegs<D> vr;
  issue_k_tile<D>(sk[0], tile_rsrc(Kh, 0), koff, wave);
  load_v_tile<D>(vr, tile_rsrc(Vh, 0), voff);
  store_v_tile<D>(vr, svt[0], tid);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * kBc;
    const int nb = (j + 1) & 1;
    const bool more = j + 1 < ntiles;
    if (more) {
      issue_k_tile<D>(sk[nb], tile_rsrc(Kh, kv0 + kBc), koff, wave);
      load_v_tile<D>(vr, tile_rsrc(Vh, kv0 + kBc), voff);
    }

#pragma unroll
    for (int sub = 0; sub < kBc; sub += kSub) {
      const int ks0 = kv0 + sub;
      const bool active = (!CAUSAL || ks0 <= q0 + kRowsPerWave - 1) && q0 < N && ks0 < N;
      if (active) {
        const bool masked = (CAUSAL && ks0 + kSub - 1 > q0) || (ks0 + kSub > N);
        if (masked)
          tile_step<D, CAUSAL, POLY, true>(sk[j & 1], svt[j & 1], qf, acc, st, sub, ks0, qi, N,
                                           c, tau, n32, h);
        else
          tile_step<D, CAUSAL, POLY, false>(sk[j & 1], svt[j & 1], qf, acc, st, sub, ks0, qi, N,
                                            c, tau, n32, h);
      }
    }

    if (more) store_v_tile<D>(vr, svt[nb], tid);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) ----
  const float ltot = half_swap_sum(st.l);
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
          ltot > 0.f ? (st.m + __builtin_log2f(ltot)) * kLn2 : -__builtin_inff();
  }
  if (stats != nullptr && lane == 0 && q0 < N) {
    atomicAdd(stats, (unsigned long long)st.steps);
    atomicAdd(stats + 1, (unsigned long long)st.rescales);
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
