// bf16 fused attention forward for gfx950 (CDNA4).
//
// Work split.  One workgroup = 8 waves = 256 query rows of one (batch, query
// head); each wave owns 32 query rows.  K/V are streamed through LDS in tiles
// of 64 keys, so the N x N score matrix never leaves registers
// ("FlashAttention-4发布：原生支持Blackwell…", section "从V1到V4",
// FlashAttention (2022) entry).
//
// Ping-pong.  Waves 0-3 (group A) and 4-7 (group B) put one wave of each group
// on every SIMD.  Each wave alternates two phases per key tile:
//   VALU phase:  online softmax of the scores it holds (max, exp2, bf16 pack)
//   MFMA phase:  O^T += V^T P^T for this tile, then S^T = K Q^T for the next
// Group B runs one phase behind group A, and the workgroup barrier between
// phases keeps it there, so on every SIMD one wave's exponentials overlap the
// other wave's matrix products.  This is the CDNA form of overlapping the
// softmax stage with the tensor-core stage ("FlashAttention-4 de NVIDIA…",
// section "La ventaja técnica"; "Hardware-Aware FP4 FlashAttention-4",
// section "1. Direct-P…", two query tiles sharing K/V so that one tile's
// softmax overlaps the other's MMA).
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
// Staging.  K/V tiles are fetched from HBM/L2 into registers with coalesced
// buffer loads two phases before they are needed, then written to LDS.  K is
// stored row-major with the 16-byte chunks of each row XOR-permuted so that
// both the writes and the MFMA operand reads are bank-conflict free; V is
// transposed in registers and stored as V^T (the PV A operand needs 8
// consecutive keys of one column per lane).  Rows past N read as zeros
// through the buffer descriptor's range check and are masked.
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
constexpr int kBc = 64;                     // keys per K/V tile (one online-softmax step)
constexpr int kThreads = kWaves * 64;

template <int D>
struct Geo {
  static constexpr int NCH = D / 8;                        // 16-byte chunks per row
  static constexpr int KUNITS = kBc * NCH;                 // 16-byte units per K tile
  static constexpr int K_PER_THREAD = KUNITS / kThreads;   // K units staged per thread
  static constexpr int VUNITS = D * (kBc / 8);             // 16-byte units per V^T tile
  static constexpr int CP = D / 2;                         // column pairs of a V row
  static constexpr int V_THREADS = CP * (kBc / 8);         // threads that stage V
  static constexpr int SW_SHIFT = (NCH == 16) ? 0 : 1;     // chunk swizzle granularity
  static constexpr int ROW_BYTES = D * 2;
  static_assert(KUNITS % kThreads == 0, "K tile must split evenly over the workgroup");
  static_assert(V_THREADS <= kThreads, "V tile staging needs at most one thread per pair");
  static_assert(NCH == 8 || NCH == 16, "d = 64 or 128");
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

// Workgroup barrier for LDS hand-over only: this wave's LDS writes are
// complete before it arrives; outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- LDS layouts (16-byte units) ----
//   K tile   unit(row, c) = row * NCH + (c ^ sw(row)),  sw(row) = perm_row(row & 15) >> SW_SHIFT
//   V^T tile unit(kc, col) = kc * D + col              kc = group of 8 keys, col = d column
// In both, the 16 lanes that the LDS serves together touch 16 distinct bank
// groups for every MFMA operand read and every staging write.

template <int D>
struct Stage {
  u32x4 k[Geo<D>::K_PER_THREAD];   // K rows, 16-byte chunks, in global order
  uint32_t v[8];                   // V: one column pair for 8 consecutive keys
};

template <int D>
__device__ __forceinline__ void load_k(Stage<D>& s, __amdgpu_buffer_rsrc_t rk, int tid) {
  using G = Geo<D>;
#pragma unroll
  for (int i = 0; i < G::K_PER_THREAD; ++i) {
    const int g = tid + i * kThreads;
    s.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (g / G::NCH) * G::ROW_BYTES + (g % G::NCH) * 16,
                                                   0, 0);
  }
}

template <int D>
__device__ __forceinline__ void load_v(Stage<D>& s, __amdgpu_buffer_rsrc_t rv, int tid) {
  using G = Geo<D>;
  if (G::V_THREADS == kThreads || tid < G::V_THREADS) {
    const int cp = tid % G::CP, kg = tid / G::CP;
    const int base = (8 * kg * D + 2 * cp) * 2;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      s.v[e] = __builtin_amdgcn_raw_buffer_load_b32(rv, base + e * G::ROW_BYTES, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void store_k(const Stage<D>& s, u32x4* sk, int tid) {
  using G = Geo<D>;
#pragma unroll
  for (int i = 0; i < G::K_PER_THREAD; ++i) {
    const int g = tid + i * kThreads;
    const int row = g / G::NCH, c = g % G::NCH;
    sk[row * G::NCH + (c ^ (perm_row(row & 15) >> G::SW_SHIFT))] = s.k[i];
  }
}

template <int D>
__device__ __forceinline__ void store_v(const Stage<D>& s, u32x4* sv, int tid) {
  using G = Geo<D>;
  if (G::V_THREADS == kThreads || tid < G::V_THREADS) {
    const int cp = tid % G::CP, kg = tid / G::CP;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4 out;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = s.v[2 * p], b = s.v[2 * p + 1];
        out[p] = cc ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                    : __builtin_amdgcn_perm(b, a, 0x05040100u);
      }
      sv[kg * D + 2 * cp + cc] = out;
    }
  }
}

// ---- MFMA phase ----
//
// One phase issues up to 32 MFMAs: first O^T += V^T P^T for the current tile
// (D/32 accumulator blocks x 4 key steps of 16), then S^T = K Q^T for the next
// tile (2 key blocks of 32 x D/16 steps).  Every MFMA takes its A operand from
// LDS; the operands are read into a ring of registers kDepth MFMAs ahead of
// their use, and the issue order is pinned to "one MFMA, one LDS read", so the
// LDS latency hides behind the MFMAs already in the pipe.

constexpr int kDepth = 6;

template <int D, bool PV, bool QK>
__device__ __forceinline__ void mfma_phase(const u32x4* sv, const u32x4* sk, const bf16x8 (&p)[4],
                                           f32x16 (&acc)[D / 32], const bf16x8 (&qf)[D / 16],
                                           f32x16 (&s)[2], uint32_t vaddr, uint32_t kaddr) {
  using G = Geo<D>;
  constexpr int NPV = PV ? 4 * (D / 32) : 0;
  constexpr int NQK = QK ? 2 * (D / 16) : 0;
  constexpr int NOPS = NPV + NQK;
  const char* vb = (const char*)sv;
  const char* kb = (const char*)sk;

  // operand i: PV (ks = i / (D/32), cb = i % (D/32)), then QK (t = k / 2, mb = k % 2)
  auto load = [&](int i) -> u32x4 {
    if (i < NPV) {
      const int ks = i / (D / 32), cb = i % (D / 32);
      return *(const u32x4*)(vb + vaddr + 16 * (2 * ks * D + 32 * cb));
    }
    const int k = i - NPV, t = k / 2, mb = k % 2;
    return *(const u32x4*)(kb + (kaddr ^ (32u * t)) + mb * 32 * G::NCH * 16);
  };

  u32x4 ring[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i)
    if (i < NOPS) ring[i] = load(i);
  if constexpr (QK) {
    s[0] = zero16();
    s[1] = zero16();
  }
#pragma unroll
  for (int i = 0; i < NOPS; ++i) {
    const bf16x8 a = as_bf16x8(ring[i % kDepth]);
    if (i + kDepth < NOPS) ring[i % kDepth] = load(i + kDepth);
    if (i < NPV) {
      const int ks = i / (D / 32), cb = i % (D / 32);
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[ks], acc[cb], 0, 0, 0);
    } else {
      const int k = i - NPV, t = k / 2, mb = k % 2;
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[mb], 0, 0, 0);
    }
  }
  // S^T register r of block mb now holds key 32*mb + 16*(r/8) + 8*h + r%8

  // issue order: the first reads, then alternate one MFMA with one read
  __builtin_amdgcn_sched_group_barrier(0x100, NOPS < kDepth ? NOPS : kDepth, 0);
#pragma unroll
  for (int i = 0; i < NOPS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + kDepth < NOPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// ---- VALU phase: online softmax of one tile ----

struct RowState {
  float m;       // running max, log2 units (-inf before the first visible key)
  float l;       // this lane's partial row sum (its half of each 32-key block)
  unsigned steps, rescales;
  bool first;
  bool rescale;  // wave-uniform: O must be multiplied by alpha before the next PV product
  float alpha;
};

template <int D, bool CAUSAL, bool POLY, bool MASK>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[2], bf16x8 (&p)[4], RowState& st, int kv0,
                                             int qi, int N, float c, float tau, int h) {
  const float NEG_INF = -__builtin_inff();
  if constexpr (MASK) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * mb + 16 * (r >> 3) + 8 * h + (r & 7);
        const bool ok = key < N && (!CAUSAL || key <= qi);
        s[mb][r] = ok ? s[mb][r] : NEG_INF;
      }
  }

  float mx = NEG_INF;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
  mx = half_swap_max(mx);
  const float mt = (mx == NEG_INF) ? NEG_INF : mx * c;

  if (!st.first) ++st.steps;
  st.rescale = false;
  if (__ballot(mt > st.m + tau)) {
    const float m_new = fmaxf(st.m, mt);
    st.alpha = (m_new == NEG_INF) ? 1.f : exp2_sel<POLY>(st.m - m_new);
    st.l *= st.alpha;
    st.m = m_new;
    st.rescale = true;
    if (!st.first) ++st.rescales;
  }
  st.first = false;
  const float mu = (st.m == NEG_INF) ? 0.f : st.m;

  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
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
}

template <int D, bool CAUSAL, bool POLY>
__device__ __forceinline__ void softmax_any(bool masked, f32x16 (&s)[2], bf16x8 (&p)[4],
                                            RowState& st, int kv0, int qi, int N, float c,
                                            float tau, int h) {
  if (masked)
    softmax_tile<D, CAUSAL, POLY, true>(s, p, st, kv0, qi, N, c, tau, h);
  else
    softmax_tile<D, CAUSAL, POLY, false>(s, p, st, kv0, qi, N, c, tau, h);
}

template <int D, bool CAUSAL, bool POLY>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                     int Hq, int Hkv, int N, int nqb, float c, float tau, uint32_t qsign,
                     unsigned long long* __restrict__ stats) {
  using G = Geo<D>;
  __shared__ u32x4 sk[2][G::KUNITS];
  __shared__ u32x4 sv[2][G::VUNITS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = lane & 31, h = lane >> 5;
  const bool lead = wave < kWaves / 2;   // group A leads, group B trails by one phase

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
  RowState st{-__builtin_inff(), 0.f, 0u, 0u, true, false, 1.f};

  // Tiles of 64 keys this workgroup visits, and which of them touch this wave's rows.
  const int kv_end = CAUSAL ? min(N, Q0 + kBr) : N;
  const int n = (kv_end + kBc - 1) / kBc;
  const int wave_end = CAUSAL ? min(N, q0 + kRowsPerWave) : N;   // keys this wave can see
  const bool wave_live = q0 < N;
  auto active = [&](int j) { return wave_live && j * kBc < wave_end; };
  auto masked = [&](int j) {
    const int kv0 = j * kBc;
    return (CAUSAL && kv0 + kBc - 1 > q0) || (kv0 + kBc > N);
  };

  auto tile_rsrc = [&](const uint16_t* head, int kv0) {
    return make_rsrc(head + (size_t)kv0 * D, (N - kv0) * G::ROW_BYTES);
  };
  // Stage t of the pipeline holds K tile t+1 and V tile t.
  auto load_stage = [&](Stage<D>& s, int t) {
    if (t + 1 < n) load_k<D>(s, tile_rsrc(Kh, (t + 1) * kBc), tid);
    load_v<D>(s, tile_rsrc(Vh, t * kBc), tid);
  };
  auto store_stage = [&](const Stage<D>& s, int t) {
    if (t + 1 < n) store_k<D>(s, sk[t & 1], tid);
    store_v<D>(s, sv[t & 1], tid);
  };

  // Per-lane operand addresses (bytes within a tile).
  const uint32_t kaddr = (uint32_t)(perm_row(n32) * G::NCH * 16) ^
                         (uint32_t)(16 * (h ^ ((n32 & 15) >> G::SW_SHIFT)));
  const uint32_t vaddr = (uint32_t)(16 * (h * D + n32));

  // ---- prologue: K tile 0 -> sk[1], stage 0 -> buffer 0, stage 1 in registers ----
  Stage<D> stg;
  {
    Stage<D> s0;
    load_k<D>(s0, tile_rsrc(Kh, 0), tid);
    load_stage(stg, 0);
    store_k<D>(s0, sk[1], tid);
    store_stage(stg, 0);
  }
  if (n > 1) load_stage(stg, 1);
  lds_barrier();
  if (!lead) lds_barrier();

  f32x16 s[2];
  bf16x8 p[4];
  if (active(0)) mfma_phase<D, false, true>(sv[0], sk[1], p, acc, qf, s, vaddr, kaddr);
  lds_barrier();

  for (int j = 0; j < n; ++j) {
    // VALU phase: softmax of tile j.  A wave whose rows see no key of the tile
    // (causal, past its diagonal) contributes P = 0 to the shared MFMA code.
    if (active(j)) {
      softmax_any<D, CAUSAL, POLY>(masked(j), s, p, st, j * kBc, qi, N, c, tau, h);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      st.rescale = false;
    }
    lds_barrier();

    // MFMA phase: stage j+1 to LDS, prefetch stage j+2, PV of tile j, QK of tile j+1
    // (in the last iteration the QK half reads a stale buffer and its result is unused).
    if (j + 1 < n) {
      store_stage(stg, j + 1);
      if (j + 2 < n) load_stage(stg, j + 2);
    }
    const u32x4* svj = sv[j & 1];
    const u32x4* skj = sk[j & 1];
    if (st.rescale) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= st.alpha;
      mfma_phase<D, true, true>(svj, skj, p, acc, qf, s, vaddr, kaddr);
    } else {
      mfma_phase<D, true, true>(svj, skj, p, acc, qf, s, vaddr, kaddr);
    }
    lds_barrier();
  }
  if (lead) lds_barrier();

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
  if (stats != nullptr && lane == 0 && wave_live) {
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
