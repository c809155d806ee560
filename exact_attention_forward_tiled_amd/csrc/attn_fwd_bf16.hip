// bf16 fused attention forward for gfx950 (CDNA4).
//
// Work split.  One workgroup = 8 waves = 256 query rows of one (batch, query
// head); each wave owns 32 query rows.  K/V are streamed through LDS in tiles
// of 64 keys, so the N x N score matrix never leaves registers
// ("FlashAttention-4发布：原生支持Blackwell…", section "从V1到V4",
// FlashAttention (2022) entry).
//
// Software pipeline.  Each wave works through the key tiles with three
// tiles in flight: while its VALU computes the online softmax of tile j, the
// matrix unit runs O^T += V^T P^T for tile j-1 and S^T = K Q^T for tile j+1.
// The three streams are independent, so they are issued as one interleaved
// instruction sequence ("one MFMA, one LDS operand read, a few VALU
// instructions").  Both waves of a SIMD do this, so two waves feed the VALU
// while the matrix unit stays busy.  This is the CDNA form of overlapping the
// softmax stage with the tensor-core stage ("FlashAttention-4 de NVIDIA…",
// section "La ventaja técnica", the pipeline of load / MMA / softmax / correction
// roles; "Hardware-Aware FP4 FlashAttention-4", section "1. Direct-P…", keeping
// the exponential work off the critical path between the two matrix products).
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
  // LDS: two K and two V^T tiles, reused after the last tile by the epilogue (8 KiB per wave)
  static constexpr int STAGE_UNITS = 2 * KUNITS + 2 * VUNITS;
  static constexpr int EPI_UNITS = kWaves * kRowsPerWave * 16;
  static constexpr int LDS_UNITS = STAGE_UNITS > EPI_UNITS ? STAGE_UNITS : EPI_UNITS;
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

// Exponential split: NP of each lane's 16 score pairs per tile go to the cubic, the
// rest to v_exp_f32 ("FlashAttention-4 de NVIDIA…", section "La ventaja técnica":
// exponentials shared between the special-function unit and the FMA units).  The
// cubic pairs are spread evenly over the tile (pair e is one when the running count
// e*NP/16 steps up there).  NP = 0: hardware only; NP = 16: cubic only.
__device__ __forceinline__ constexpr bool pair_on_poly(int np, int e) {
  return (e + 1) * np / 16 > e * np / 16;
}

template <int NP>
__device__ __forceinline__ float exp2_pair(float x, int e) {
  return pair_on_poly(NP, e) ? exp2_poly(x) : __builtin_amdgcn_exp2f(x);
}

// Row of the K tile read by MFMA row m of a 32-row block: bits 2 and 3 swapped.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// max of two floats as one v_max_f32.  fmaxf on values the compiler cannot prove canonical
// (a lane swap's output, a loop-carried maximum) adds a quieting max per operand; the
// operands here are scores or -inf, never signalling NaNs.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// ---- one pipeline step ----
//
// MFMA stream: O^T += V^T P^T for the previous tile (D/32 accumulator blocks x 4
// key steps of 16), then S^T = K Q^T for the next tile (2 key blocks of 32 x
// D/16 steps); every A operand comes from LDS through a ring of registers
// filled kDepth MFMAs ahead.  VALU stream: the online softmax of the current
// tile, cut into per-MFMA slots (row max, threshold test, new reference max,
// then the exponentials two scores at a time).  Each slot issues one MFMA, one
// operand read and its share of the softmax; scheduling barriers between the
// slots keep that interleave in the final instruction order.

constexpr int kDepth = 4;

struct RowState {
  float m;       // running max, log2 units (-inf before the first visible key)
  float l;       // this lane's partial row sum (its half of each 32-key block)
};

template <int D, bool PV, bool QK, bool MODS = false>
struct StepShape {
  static constexpr int NPV = PV ? 4 * (D / 32) : 0;
  static constexpr int NQK = QK ? 2 * (D / 16) : 0;
  static constexpr int NOPS = NPV + NQK;
  // softmax slot plan, spread evenly over the MFMA slots: row max over 32 scores in
  // MAXS slots, threshold test, new reference max, the 16 score pairs over the
  // following slots, the row-sum update in the last slot; the staging of the next
  // K/V stage sits in the middle slot.  With score modifications (MODS) the max phase
  // also turns every score into its modified log2-domain value, so it gets more slots.
  static constexpr int MAXS = MODS ? (NOPS >= 32 ? 16 : 8) : (NOPS >= 32 ? 8 : 4);
  static_assert(32 % MAXS == 0, "every slot of the max phase takes the same share of the 32 scores");
  static constexpr int TEST = MAXS;
  static constexpr int MNEW = MAXS + 1;
  static constexpr int PAIR0 = MAXS + 2;
  static constexpr int PAIR_SLOTS = NOPS - 1 - PAIR0;
  static constexpr int LSUM = NOPS - 1;
  static constexpr int MID = NOPS / 2;
  // score pairs [pair_lo(k), pair_lo(k + 1)) go to slot k (at most MAXQ per slot)
  static constexpr int pair_lo(int k) {
    return k <= PAIR0 ? 0 : (k >= PAIR0 + PAIR_SLOTS ? 16 : ((k - PAIR0) * 16 + PAIR_SLOTS - 1) / PAIR_SLOTS);
  }
  static constexpr int MAXQ = (16 + PAIR_SLOTS - 1) / (PAIR_SLOTS > 0 ? PAIR_SLOTS : 1);
  static_assert(!(PV && QK) || PAIR_SLOTS >= 4, "softmax must fit in the MFMA slots");
};

// Operand i of a step: PV (ks = i / (D/32), cb = i % (D/32)), then QK (t = k/2, mb = k%2).
template <int D, int NPV>
__device__ __forceinline__ u32x4 load_operand(const char* vb, const char* kb, uint32_t vaddr,
                                              uint32_t kaddr, int i) {
  using G = Geo<D>;
  if (i < NPV) {
    const int ks = i / (D / 32), cb = i % (D / 32);
    return *(const u32x4*)(vb + vaddr + 16 * (2 * ks * D + 32 * cb));
  }
  const int k = i - NPV, t = k / 2, mb = k % 2;
  return *(const u32x4*)(kb + (kaddr ^ (32u * t)) + mb * 32 * G::NCH * 16);
}

template <int D, int NPV>
__device__ __forceinline__ void issue_mfma(int i, const u32x4& op, const bf16x8 (&pp)[4],
                                           f32x16 (&acc)[D / 32], const bf16x8 (&qf)[D / 16],
                                           f32x16 (&sn)[2]) {
  const bf16x8 a = as_bf16x8(op);
  if (i < NPV) {
    const int ks = i / (D / 32), cb = i % (D / 32);
    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pp[ks], acc[cb], 0, 0, 0);
  } else {
    const int k = i - NPV, t = k / 2, mb = k % 2;
    sn[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], sn[mb], 0, 0, 0);
  }
}

// MFMAs only (pipeline prologue and the final PV product).
template <int D, bool PV, bool QK>
__device__ __forceinline__ void mfma_only(const u32x4* svp, const u32x4* skn,
                                          const bf16x8 (&pp)[4], f32x16 (&acc)[D / 32],
                                          const bf16x8 (&qf)[D / 16], f32x16 (&sn)[2],
                                          uint32_t vaddr, uint32_t kaddr) {
  using SS = StepShape<D, PV, QK>;
  const char* vb = (const char*)svp;
  const char* kb = (const char*)skn;
  u32x4 ring[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i)
    if (i < SS::NOPS) ring[i] = load_operand<D, SS::NPV>(vb, kb, vaddr, kaddr, i);
  if constexpr (QK) {
    sn[0] = zero16();
    sn[1] = zero16();
  }
#pragma unroll
  for (int i = 0; i < SS::NOPS; ++i) {
    const u32x4 op = ring[i % kDepth];
    if (i + kDepth < SS::NOPS)
      ring[i % kDepth] = load_operand<D, SS::NPV>(vb, kb, vaddr, kaddr, i + kDepth);
    issue_mfma<D, SS::NPV>(i, op, pp, acc, qf, sn);
  }
}

// Score modifications (the FlexAttention news page, body: ALiBi and soft-capping among
// the patterns the FA4 backend serves), switched at compile time; the values are per
// lane.  In log2 units, on the scaled score s:
//   soft-capping  t = C log2(e) tanh(s / C),  tanh(x) = 1 - 2 / (1 + 2^(2 x log2 e))
//   ALiBi         t -= a_h log2(e) |i - j|
struct ScoreMod {
  float alibi;    // ALiBi slope of this query head, log2 units per key of distance
  float k2;       // soft-capping: 2 |scale| log2(e) / C (raw MFMA score to 2 x log2 e)
  float ccap;     // soft-capping: C log2(e)
  int qi;         // this lane's query row
};

// One pipeline step: PV of tile j-1 (pp, V^T tile in svp), QK of tile j+1 into
// sn (K tile in skn), and the online softmax of tile j (sc -> pc), interleaved.
// MASK: keys outside [klo, khi] (this lane's visible range) or past N get -inf; klo
// applies with BAND (a sliding window and/or documents), khi when causal or with BAND.
// Returns whether any row of the wave raised its reference max by more than tau;
// then O must be multiplied by alpha before the next PV product.
template <int D, bool CAUSAL, int NP, bool MASK, bool BAND, bool ALIBI, bool SOFTCAP, class Mid>
__device__ __forceinline__ bool step(const u32x4* svp, const u32x4* skn, const bf16x8 (&pp)[4],
                                     f32x16 (&acc)[D / 32], const bf16x8 (&qf)[D / 16],
                                     f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pc)[4],
                                     RowState& st, float& alpha, int kv0, int klo, int khi, int N,
                                     float c,
                                     float tau, int h, uint32_t vaddr, uint32_t kaddr,
                                     const ScoreMod& sm, Mid&& mid) {
  constexpr bool MODS = ALIBI || SOFTCAP;
  using SS = StepShape<D, true, true, MODS>;
  const float NEG_INF = -__builtin_inff();
  const char* vb = (const char*)svp;
  const char* kb = (const char*)skn;

  if constexpr (MASK) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * mb + 16 * (r >> 3) + 8 * h + (r & 7);
        const bool ok = key < N && (!(CAUSAL || BAND) || key <= khi) && (!BAND || key >= klo);
        sc[mb][r] = ok ? sc[mb][r] : NEG_INF;
      }
  }

  u32x4 ring[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i) ring[i] = load_operand<D, SS::NPV>(vb, kb, vaddr, kaddr, i);
  sn[0] = zero16();
  sn[1] = zero16();

  float mx = NEG_INF, mt = NEG_INF, mu = 0.f;
  bool any = false;
  // ALiBi: key - query of register r of block mb is dbase + 32 mb + 16 (r / 8) + r % 8
  const float dbase = ALIBI ? (float)(kv0 + 8 * h - sm.qi) : 0.f;
  // the modified score, log2 units (masked scores stay -inf)
  auto modified = [&](float s, int mb, int r) {
    float t;
    if constexpr (SOFTCAP) {
      const float y = __builtin_amdgcn_exp2f(s * sm.k2);
      t = __builtin_fmaf(-2.f * sm.ccap, __builtin_amdgcn_rcpf(y + 1.f), sm.ccap);
      if constexpr (MASK) t = (s == NEG_INF) ? NEG_INF : t;
    } else {
      t = s * c;
    }
    if constexpr (ALIBI) {
      const float dd = dbase + (float)(32 * mb + 16 * (r >> 3) + (r & 7));
      t = __builtin_fmaf(-sm.alibi, __builtin_fabsf(dd), t);
    }
    return t;
  };
  u32x4 pk[4];
  // -0 is the additive identity the compiler may fold, so the first add to each partial sum
  // disappears (+0 is not: +0 + -0 = +0)
  float ls[4] = {-0.f, -0.f, -0.f, -0.f};

#pragma unroll
  for (int k = 0; k < SS::NOPS; ++k) {
    const u32x4 op = ring[k % kDepth];
    if (k + kDepth < SS::NOPS)
      ring[k % kDepth] = load_operand<D, SS::NPV>(vb, kb, vaddr, kaddr, k + kDepth);
    issue_mfma<D, SS::NPV>(k, op, pp, acc, qf, sn);

    if (k < SS::MAXS) {                // row max over this slot's share of the 32 scores
      constexpr int per = 32 / SS::MAXS;
#pragma unroll
      for (int u = 0; u < per; ++u) {
        const int idx = k * per + u;
        if constexpr (MODS) {
          sc[idx >> 4][idx & 15] = modified(sc[idx >> 4][idx & 15], idx >> 4, idx & 15);
          // a use in this slot keeps the compiler from sinking the work out of it
          asm volatile("" ::"v"(sc[idx >> 4][idx & 15]));
        }
        mx = fmaxf(mx, sc[idx >> 4][idx & 15]);
      }
    } else if (k == SS::TEST) {        // whole row (other half-wave), threshold test
      mx = half_swap_max(mx);
      // an unmasked tile holds a finite score for every row: the -inf guard is for masks
      if constexpr (MASK) mt = (mx == NEG_INF) ? NEG_INF : (MODS ? mx : mx * c);
      else mt = MODS ? mx : mx * c;
      any = __ballot(mt > st.m + tau) != 0;
    } else if (k == SS::MNEW) {        // thresholded update of the reference max
      const float m_up = vmax(st.m, mt);   // unconditional, so the choice is a select
      const float m_new = any ? m_up : st.m;
      if constexpr (MASK) {
        alpha = (m_new == NEG_INF) ? 1.f : exp2_sel<NP == 16>(st.m - m_new);
        mu = (m_new == NEG_INF) ? 0.f : m_new;
      } else {
        // m_new is finite; on a row's first tile st.m = -inf and alpha = 2^-inf = 0
        alpha = exp2_sel<NP == 16>(st.m - m_new);
        mu = m_new;
      }
      st.m = m_new;
    } else if (k == SS::LSUM) {
      st.l = __builtin_fmaf(st.l, alpha, (ls[0] + ls[1]) + (ls[2] + ls[3]));
      asm volatile("" ::"v"(st.l));
    }
    if (k >= SS::PAIR0 && k < SS::LSUM) {
#pragma unroll
      for (int q = 0; q < SS::MAXQ; ++q) {   // score pairs scheduled in this slot
        const int e = SS::pair_lo(k) + q;
        if (e < SS::pair_lo(k + 1)) {
          const int mb = e >> 3, hf = (e >> 2) & 1, ee = e & 3;
          const float s0 = sc[mb][hf * 8 + 2 * ee], s1 = sc[mb][hf * 8 + 2 * ee + 1];
          float e0 = exp2_pair<NP>(MODS ? s0 - mu : __builtin_fmaf(s0, c, -mu), e);
          float e1 = exp2_pair<NP>(MODS ? s1 - mu : __builtin_fmaf(s1, c, -mu), e);
          if constexpr (MASK) {
            e0 = (s0 == NEG_INF) ? 0.f : e0;
            e1 = (s1 == NEG_INF) ? 0.f : e1;
          }
          pk[mb * 2 + hf][ee] = pack_bf16x2(e0, e1);
          ls[ee] += e0 + e1;
          // a use in this slot keeps the compiler from sinking the work out of it
          asm volatile("" ::"v"(pk[mb * 2 + hf][ee]), "v"(ls[ee]));
        }
      }
    }
    if (k == SS::MID) mid();
    __builtin_amdgcn_sched_barrier(0);
  }
  // S^T register r of block mb (next tile) holds key 32*mb + 16*(r/8) + 8*h + r%8
#pragma unroll
  for (int i = 0; i < 4; ++i) pc[i] = as_bf16x8(pk[i]);
  return any;
}

template <int D, bool CAUSAL, int NP, bool BAND, bool ALIBI, bool SOFTCAP>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                     int Hq, int Hkv, int N, int nqb, float c, float tau, uint32_t qsign,
                     int window_arg, const int* __restrict__ doc_off, int n_docs_arg,
                     const float* __restrict__ alibi_slopes, float k2, float ccap,
                     unsigned long long* __restrict__ stats) {
  using G = Geo<D>;
  __shared__ u32x4 lds[G::LDS_UNITS];
  u32x4 (*sk)[G::KUNITS] = reinterpret_cast<u32x4 (*)[G::KUNITS]>(lds);
  u32x4 (*sv)[G::VUNITS] = reinterpret_cast<u32x4 (*)[G::VUNITS]>(lds + 2 * G::KUNITS);

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index through readfirstlane: the compiler then knows it is uniform, and the
  // per-wave branches of the diagonal tiles (which contain barriers) are scalar branches
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

  ScoreMod sm;
  sm.alibi = ALIBI ? alibi_slopes[hq] * kLog2e : 0.f;
  sm.k2 = k2;
  sm.ccap = ccap;
  sm.qi = qi;

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = zero16();
  RowState st{-__builtin_inff(), 0.f};
  unsigned n_steps = 0, n_rescales = 0;
  bool first = true;

  // Keys this lane sees: [klo, khi].  Without BAND: up to its query when causal.  With
  // BAND, row i sees [row_lo(i), row_hi(i)]: the causal limit, a window W (from i - W + 1,
  // and up to i + W - 1 when not causal) and/or i's document (offsets doc_off[0..n_docs]).
  // Both bounds are non-decreasing in i, so the first and last rows of a workgroup or a
  // wave bound its keys.
  constexpr int kNoBound = 0x7fffffff;
  const int window = BAND ? window_arg : 0;   // 0 without the band instantiation
  const int n_docs = BAND ? n_docs_arg : 0;
  // [lo, hi] of row i (0 <= i < N); the document search is clamped so that any offsets
  // stay within doc_off[0..n_docs] and give lo <= i <= hi
  auto row_bounds = [&](int i, int& lo, int& hi) {
    lo = window ? max(0, i - window + 1) : 0;
    hi = CAUSAL ? i : (window ? min(N - 1, i + window - 1) : N - 1);
    if (n_docs > 0) {
      int a = 0, z = n_docs;   // the document d with doc_off[d] <= i < doc_off[d + 1]
      while (z - a > 1) {
        const int m = (a + z) >> 1;
        if (doc_off[m] <= i) a = m;
        else z = m;
      }
      lo = max(lo, min(doc_off[a], i));
      hi = min(hi, max(doc_off[a + 1] - 1, i));
    }
  };
  int klo = -kNoBound, khi = CAUSAL ? qi : kNoBound;
  if (BAND) row_bounds(min(qi, N - 1), klo, khi);
  // Tiles of 64 keys this workgroup visits, t0 .. t0 + n - 1 (local index j = tile - t0);
  // a band skips the tiles below its lower edge.
  int wg_lo_first = 0, wg_hi_first = 0, wg_lo_last = 0, wg_hi_last = 0;
  if (BAND) {
    row_bounds(Q0, wg_lo_first, wg_hi_first);
    row_bounds(min(Q0 + kBr - 1, N - 1), wg_lo_last, wg_hi_last);
  }
  const int t0 = BAND ? wg_lo_first / kBc : 0;
  const int kv_end = BAND ? wg_hi_last + 1 : (CAUSAL ? min(N, Q0 + kBr) : N);
  const int n = (kv_end + kBc - 1) / kBc - t0;
  const bool wave_live = q0 < N;
  int w_lo_first = 0, w_hi_first = 0, w_lo_last = 0, w_hi_last = 0;
  if (BAND) {
    row_bounds(min(q0, N - 1), w_lo_first, w_hi_first);
    row_bounds(min(q0 + kRowsPerWave - 1, N - 1), w_lo_last, w_hi_last);
  }
  const int wave_end = BAND ? w_hi_last + 1                          // keys this wave can see
                            : (CAUSAL ? min(N, q0 + kRowsPerWave) : N);
  const int wave_lo = BAND ? w_lo_first : 0;                          // the wave's lowest key
  auto active = [&](int j) {
    return wave_live && (t0 + j) * kBc < wave_end && (!BAND || (t0 + j + 1) * kBc > wave_lo);
  };
  // Tiles [0, lo_wg) hold keys below some row's lower edge: masked for every wave.
  int lo_wg = 0;
  if (BAND) {
    const int x = wg_lo_last;   // the largest lower edge of the workgroup's rows
    lo_wg = x > t0 * kBc ? min(n, (x + kBc - 1) / kBc - t0) : 0;
  }
  // Per wave: tiles [lo_wg, n_vis) need no element mask, tiles [n_vis, n_w) do, and tiles
  // [n_w, n) are entirely masked (keys past the wave's last visible key), so the wave
  // skips their products and only keeps up its share of the staging.
  const int n_w = wave_live ? (wave_end + kBc - 1) / kBc - t0 : n;
  const int n_vis = BAND ? max(0, min((w_hi_first + 1) / kBc, N / kBc) - t0)
                         : min(CAUSAL ? (q0 + 1) / kBc : n, N / kBc);

  auto tile_rsrc = [&](const uint16_t* head, int kv0) {
    return make_rsrc(head + (size_t)kv0 * D, (N - kv0) * G::ROW_BYTES);
  };
  // Stage t (read by pipeline step t from buffer t & 1) holds K tile t+1 and V tile t-1
  // (local indices).
  auto load_stage = [&](Stage<D>& s, int t) {
    if (t + 1 < n) load_k<D>(s, tile_rsrc(Kh, (t0 + t + 1) * kBc), tid);
    if (t >= 1 && t - 1 < n) load_v<D>(s, tile_rsrc(Vh, (t0 + t - 1) * kBc), tid);
  };
  auto store_stage = [&](const Stage<D>& s, int t) {
    if (t + 1 < n) store_k<D>(s, sk[t & 1], tid);
    if (t >= 1 && t - 1 < n) store_v<D>(s, sv[t & 1], tid);
  };

  // Per-lane operand addresses (bytes within a tile).
  const uint32_t kaddr = (uint32_t)(perm_row(n32) * G::NCH * 16) ^
                         (uint32_t)(16 * (h ^ ((n32 & 15) >> G::SW_SHIFT)));
  const uint32_t vaddr = (uint32_t)(16 * (h * D + n32));

  // ---- prologue: K tile 0 -> sk[1]; stage 0 (K tile 1, V^T = 0) -> buffer 0;
  //      stage 1 (K tile 2, V tile 0) in registers; S of tile 0 ----
  Stage<D> stg;
  {
    Stage<D> s0;
    load_k<D>(s0, tile_rsrc(Kh, t0 * kBc), tid);
    load_stage(stg, 0);
    store_k<D>(s0, sk[1], tid);
    store_stage(stg, 0);
    for (int u = tid; u < G::VUNITS; u += kThreads) sv[0][u] = u32x4{0u, 0u, 0u, 0u};
  }
  load_stage(stg, 1);   // V tile 0 always exists; K tile 2 only if n > 2
  lds_barrier();

  // S of the current tile and of the next one, P of the current tile and the previous one.
  f32x16 s_cur[2], s_nxt[2];
  bf16x8 p_prev[4], p_cur[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p_prev[i] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  mfma_only<D, false, true>(sv[0], sk[1], p_prev, acc, qf, s_cur, vaddr, kaddr);
  lds_barrier();

  // One pipeline step j: the rescale of O decided by step j-1 (a rare branch,
  // kept outside the interleaved region), then PV of tile j-1, QK of tile j+1 and
  // the softmax of tile j as one straight-line region; then the staging of the
  // next stage and one barrier.
  bool any_prev = false;
  float alpha_prev = 1.f;
  auto rescale = [&]() {
    if (any_prev) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha_prev;
    }
  };
  auto finish_step = [&](int j, bool any, float alpha) {
    any_prev = any;
    alpha_prev = alpha;
    if (active(j)) {
      if (!first) {
        ++n_steps;
        n_rescales += any ? 1u : 0u;
      }
      first = false;
    }
    lds_barrier();
  };
  auto advance = [&]() {   // the next tile's S and this tile's P become current / previous
#pragma unroll
    for (int i = 0; i < 2; ++i) s_cur[i] = s_nxt[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) p_prev[i] = p_cur[i];
  };

  // Staging inside step j (no branches, so it stays in the interleaved region):
  // stage j+1 from registers to LDS (buffer (j+1)&1, last read in step j-1), then
  // the loads of stage j+2.  Past the last tile the K part writes a buffer half
  // that is never read and the loads are clamped to the last tile (in bounds,
  // unused).
  auto staging = [&](int j) {
    store_k<D>(stg, sk[(j + 1) & 1], tid);
    store_v<D>(stg, sv[(j + 1) & 1], tid);
    load_k<D>(stg, tile_rsrc(Kh, (t0 + min(j + 3, n - 1)) * kBc), tid);
    load_v<D>(stg, tile_rsrc(Vh, (t0 + min(j + 1, n - 1)) * kBc), tid);
  };

  // Tiles [lo_wg, n_full) need no element mask for any row of the workgroup: causal, the
  // keys below the workgroup's first query; with a band, the keys up to its first row's
  // upper edge; otherwise the whole 64-key tiles.
  const int n_full = BAND ? max(0, (wg_hi_first + 1) / kBc - t0)
                          : (CAUSAL ? min(Q0, N) / kBc : N / kBc);
  int j = 0;
  // The window's lower edge: masked steps for every wave.
  for (; j < lo_wg; ++j) {
    rescale();
    float alpha;
    const bool any = step<D, CAUSAL, NP, true, BAND, ALIBI, SOFTCAP>(
        sv[j & 1], sk[j & 1], p_prev, acc, qf, s_cur, s_nxt, p_cur, st, alpha, (t0 + j) * kBc,
        klo, khi, N, c, tau, h, vaddr, kaddr, sm, [&]() { staging(j); });
    finish_step(j, any, alpha);
    advance();
  }
  // Unmasked tiles two at a time, with the roles of the S and P registers swapped in
  // the second step, so that no register copies are needed.
  for (; j + 1 < n_full; j += 2) {
    float alpha;
    rescale();
    bool any = step<D, CAUSAL, NP, false, BAND, ALIBI, SOFTCAP>(
        sv[j & 1], sk[j & 1], p_prev, acc, qf, s_cur, s_nxt, p_cur, st, alpha, (t0 + j) * kBc, klo, khi, N, c,
        tau, h, vaddr, kaddr, sm, [&]() { staging(j); });
    finish_step(j, any, alpha);
    rescale();
    any = step<D, CAUSAL, NP, false, BAND, ALIBI, SOFTCAP>(
        sv[(j + 1) & 1], sk[(j + 1) & 1], p_cur, acc, qf, s_nxt, s_cur, p_prev, st, alpha,
        (t0 + j + 1) * kBc, klo, khi, N, c, tau, h, vaddr, kaddr, sm, [&]() { staging(j + 1); });
    finish_step(j + 1, any, alpha);
  }
  for (; j < n_full; ++j) {
    rescale();
    float alpha;
    const bool any = step<D, CAUSAL, NP, false, BAND, ALIBI, SOFTCAP>(
        sv[j & 1], sk[j & 1], p_prev, acc, qf, s_cur, s_nxt, p_cur, st, alpha, (t0 + j) * kBc, klo, khi, N, c,
        tau, h, vaddr, kaddr, sm, [&]() { staging(j); });
    finish_step(j, any, alpha);
    advance();
  }
  // The diagonal tiles (and a ragged tail), in per-wave loops (wave-uniform bounds,
  // each tile in exactly one loop, one barrier per tile): unmasked while the wave
  // sees the whole tile, masked on its partial tiles, then its last PV product, then
  // staging only for the tiles that are entirely masked for it.
  for (; j < n_vis; ++j) {
    rescale();
    float alpha;
    const bool any = step<D, CAUSAL, NP, false, BAND, ALIBI, SOFTCAP>(
        sv[j & 1], sk[j & 1], p_prev, acc, qf, s_cur, s_nxt, p_cur, st, alpha, (t0 + j) * kBc, klo, khi, N, c,
        tau, h, vaddr, kaddr, sm, [&]() { staging(j); });
    finish_step(j, any, alpha);
    advance();
  }
  for (; j < n_w; ++j) {
    rescale();
    float alpha;
    const bool any = step<D, CAUSAL, NP, true, BAND, ALIBI, SOFTCAP>(
        sv[j & 1], sk[j & 1], p_prev, acc, qf, s_cur, s_nxt, p_cur, st, alpha, (t0 + j) * kBc, klo, khi, N, c,
        tau, h, vaddr, kaddr, sm, [&]() { staging(j); });
    finish_step(j, any, alpha);
    advance();
  }
  // ---- last PV product (tile n_w-1, V tile in stage n_w) ----
  rescale();
  mfma_only<D, true, false>(sv[j & 1], sk[j & 1], p_prev, acc, qf, s_nxt, vaddr, kaddr);
  if (j < n) {
    staging(j);
    lds_barrier();
    for (++j; j < n; ++j) {
      staging(j);
      lds_barrier();
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) ----
  // O goes out through LDS so that every store instruction writes whole rows: each
  // lane holds 16-byte pieces of one query row, so storing straight from registers
  // would touch 32 rows per instruction.  After a barrier (every wave is done with
  // the K/V buffers) each wave writes its 32 x 64 half tiles into its own 8 KiB of
  // them, chunk c of row r at (c ^ (r % 16)) (conflict-free both ways), and reads
  // them back as 4 rows x 256 B per instruction.
  const float ltot = half_swap_sum(st.l);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  lds_barrier();
  {
    u32x4* tb = lds + wave * (kRowsPerWave * 16);
    float* Obase = O + ((size_t)(b * Hq + hq) * N + q0) * D;
#pragma unroll
    for (int half = 0; half < D / 64; ++half) {
#pragma unroll
      for (int cbl = 0; cbl < 2; ++cbl)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int cb = 2 * half + cbl, c = 8 * cbl + 2 * a4 + h;
          const f32x4 out = {acc[cb][4 * a4] * inv, acc[cb][4 * a4 + 1] * inv,
                             acc[cb][4 * a4 + 2] * inv, acc[cb][4 * a4 + 3] * inv};
          tb[n32 * 16 + (c ^ (n32 & 15))] = __builtin_bit_cast(u32x4, out);
        }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + (lane >> 4), c = lane & 15;
        const u32x4 val = tb[r * 16 + (c ^ (r & 15))];
        if (q0 + r < N) *(u32x4*)(Obase + (size_t)r * D + 64 * half + 4 * c) = val;
      }
    }
  }
  if (qi < N && h == 0)
    LSE[(size_t)(b * Hq + hq) * N + qi] =
        ltot > 0.f ? (st.m + __builtin_log2f(ltot)) * kLn2 : -__builtin_inff();
  if (stats != nullptr && lane == 0 && wave_live) {
    atomicAdd(stats, (unsigned long long)n_steps);
    atomicAdd(stats + 1, (unsigned long long)n_rescales);
  }
  if (stats != nullptr && threadIdx.x == 0) {
    atomicAdd(stats + 2, __builtin_amdgcn_s_memtime() - clk0);
    atomicAdd(stats + 3, __builtin_amdgcn_s_memrealtime() - ref0);
  }
}

template <int D, bool CAUSAL, int NP, bool BAND, bool ALIBI, bool SOFTCAP>
hipError_t launch_one(const FwdArgs& a) {
  const int nqb = (a.N + kBr - 1) / kBr;
  const long long grid = (long long)a.B * a.Hq * nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const float k2 = SOFTCAP ? 2.f * a.c / a.softcap : 0.f;
  const float ccap = SOFTCAP ? a.softcap * kLog2e : 0.f;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, NP, BAND, ALIBI, SOFTCAP>), dim3((unsigned)grid),
                     dim3(kThreads), 0, (hipStream_t)a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, a.lse, a.Hq, a.Hkv, a.N, nqb,
                     a.c, a.tau, a.qsign, a.window, a.doc_offsets, a.n_docs, a.alibi, k2, ccap,
                     a.stats);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool BAND>
hipError_t launch_np(const FwdArgs& a) {
  switch (a.poly_pairs) {
    case 0: return launch_one<D, CAUSAL, 0, BAND, false, false>(a);
    case 4: return launch_one<D, CAUSAL, 4, BAND, false, false>(a);
    case 8: return launch_one<D, CAUSAL, 8, BAND, false, false>(a);
    case 12: return launch_one<D, CAUSAL, 12, BAND, false, false>(a);
    case 16: return launch_one<D, CAUSAL, 16, BAND, false, false>(a);
    default: return hipErrorInvalidValue;
  }
}

// Score modifications run with the hardware exponential only.
template <int D, bool CAUSAL, bool BAND>
hipError_t launch_mod(const FwdArgs& a) {
  const bool al = a.alibi != nullptr, cap = a.softcap > 0.f;
  if (!al && !cap) return launch_np<D, CAUSAL, BAND>(a);
  if (a.poly_pairs != 0) return hipErrorNotSupported;
  if (al && cap) return launch_one<D, CAUSAL, 0, BAND, true, true>(a);
  if (al) return launch_one<D, CAUSAL, 0, BAND, true, false>(a);
  return launch_one<D, CAUSAL, 0, BAND, false, true>(a);
}

template <int D, bool CAUSAL>
hipError_t launch_band(const FwdArgs& a) {
  return (a.window || a.n_docs > 0) ? launch_mod<D, CAUSAL, true>(a) : launch_mod<D, CAUSAL, false>(a);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch_band<128, true>(a) : launch_band<128, false>(a);
  return a.causal ? launch_band<64, true>(a) : launch_band<64, false>(a);
}

}  // namespace attn
