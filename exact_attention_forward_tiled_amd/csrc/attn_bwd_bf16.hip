// bf16 attention backward: dQ, dK, dV from the saved LSE.
//
// The forward keeps only O and the row log-sum-exp; the backward recomputes the
// probabilities from them instead of storing the N x N matrix ("FlashAttention-4
// 发布：原生支持Blackwell…", section "从V1到V4", FlashAttention (2022) entry:
// tiling plus recomputation; "Hardware-Aware FP4 FlashAttention-4", section
// "2. Causal Backward Cuantizado": the forward saves the LSE and the backward
// rebuilds the probabilities from it).  With s = scale q.k and P = exp(s - LSE):
//   D_i  = dO_i . O_i                         (delta_kernel)
//   dS   = P * (dO V^T - D)
//   dV   = P^T dO,  dK = scale dS^T Q          (dkdv_kernel, one workgroup per key block)
//   dQ   = scale dS K                          (dq_kernel, one workgroup per query block)
// Each kernel recomputes S and dP for its own orientation, so every output is
// written once by one workgroup: no atomics, deterministic results.  The forward's
// masks (causal, sliding window, documents) and score modifications (soft-capping,
// ALiBi) apply unchanged: P comes from the modified, masked score, and soft-capping
// multiplies dS by its derivative.
//
// All products run on v_mfma_f32_32x32x16_bf16.  Operand layouts (probed): lane l
// holds A[l % 32][8*(l / 32) + i] and B[8*(l / 32) + i][l % 32], i = 0..7;
// accumulator register r of lane l is C[8*(r / 4) + 4*(l / 32) + r % 4][l % 32].
// Reading the A rows in the order pi(m) (bits 2 and 3 of m swapped) makes
// register r of the product hold row 16*(r / 8) + 8*(l / 32) + r % 8 of the
// 32-row block, which is exactly the k index the B operand of the next product
// expects from that lane: the probabilities go from one MFMA to the next
// without any data movement.

#include <mutex>
#include <type_traits>

#include "../../include/attn.h"
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kBWaves = 4;
constexpr int kBThreads = kBWaves * 64;
constexpr int kBBlock = kBWaves * 32;    // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kBTile = 64;               // queries (dK/dV) or keys (dQ) staged per loop step
constexpr int kSub = 32;                 // rows per MFMA block: a step is two such halves
constexpr int kColStride = kBTile * 2 + 16;  // bytes per staged transposed column (padded)

__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// row of the 32-row block held by accumulator register r of lane half h (after pi)
__device__ __forceinline__ int acc_row(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// bf16 B operand (8 k values) from accumulator registers 8c .. 8c + 7.
__device__ __forceinline__ u32x4 pack_chunk(const f32x16& x, int c) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(x[8 * c + 2 * i], x[8 * c + 2 * i + 1]);
  return r;
}

// Staged tile: 64 rows x D bf16 of two tensors, row-major (rows padded by 16 bytes: the
// 16 rows read together start 4 banks apart) and transposed.
template <int D>
struct alignas(16) BTile {
  static constexpr int kRow = D * 2 + 16;   // bytes per staged row
  float s0[kBTile];                   // per-row scalars (LSE, D) of the dK/dV tile
  float s1[kBTile];
  uint8_t a[kBTile * kRow];           // tensor A, row r at r * kRow
  uint8_t b[kBTile * kRow];           // tensor B
  uint8_t at[D * kColStride];         // A transposed: column d at d * kColStride, 64 rows
  uint8_t bt[D * kColStride];         // B transposed
};

// One thread's share of a staged tile pair: D / 32 units of 16 bytes of each tensor.
// Unit u is row u % 64, bytes 16 * (u / 64) .. + 15, so the lanes of a wave take 64
// consecutive rows: their 2-byte writes into the transposed copy fall on 32 distinct
// dwords of one column instead of piling onto two banks.
template <int D>
struct StageRegs {
  static constexpr int kUnits = kBTile * D * 2 / 16 / kBThreads;
  u32x4 a[kUnits], b[kUnits];
};

// Fetch rows r0 .. r0 + 63 of two [N, D] bf16 tensors into registers (rows past N read
// as row N - 1: in bounds; their contributions are masked by the caller).
template <int D>
__device__ __forceinline__ void stage_load(StageRegs<D>& sr, const uint16_t* A,
                                           const uint16_t* B, int r0, int N) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < StageRegs<D>::kUnits; ++u) {
    const int unit = tid + u * kBThreads;
    const int row = unit % kBTile, c16 = unit / kBTile;
    const int gr = min(r0 + row, N - 1);
    sr.a[u] = *(const u32x4*)(A + (size_t)gr * D + 8 * c16);
    sr.b[u] = *(const u32x4*)(B + (size_t)gr * D + 8 * c16);
  }
}

__device__ __forceinline__ void put_transposed(uint8_t* t, const u32x4& v, int row, int c16) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *(uint16_t*)(t + (8 * c16 + i) * kColStride + 2 * row) = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
}

// Write the fetched rows into LDS: both tensors row-major, and transposed where asked.
template <int D>
__device__ __forceinline__ void stage_store(BTile<D>& t, const StageRegs<D>& sr,
                                            bool transposed_a, bool transposed_b) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < StageRegs<D>::kUnits; ++u) {
    const int unit = tid + u * kBThreads;
    const int row = unit % kBTile, c16 = unit / kBTile;
    *(u32x4*)(t.a + row * BTile<D>::kRow + 16 * c16) = sr.a[u];
    *(u32x4*)(t.b + row * BTile<D>::kRow + 16 * c16) = sr.b[u];
    if (transposed_a) put_transposed(t.at, sr.a[u], row, c16);
    if (transposed_b) put_transposed(t.bt, sr.b[u], row, c16);
  }
}

__device__ __forceinline__ u32x4 lds_u32x4(const uint8_t* p) { return *(const u32x4*)p; }

// The masks beyond the causal one, as in the forward: a sliding window W (key j visible
// from query i when i - W < j, and j < i + W without the causal mask) and packed documents
// (both in one document).  Key j is visible from query i iff lo(i) <= j <= hi(i) (keys()),
// equivalently qlo(j) <= i <= qhi(j) (queries()); all four bounds are non-decreasing, so
// the first and last rows of a block bound the band of the whole block.
struct Band {
  int N, window, n_docs;
  const int* doc_off;
  // the document [s, e) holding position i; the search reads only doc_off[0 .. n_docs],
  // and the clamps keep s <= i < e whatever the offsets hold
  __device__ void doc_of(int i, int& s, int& e) const {
    int a = 0, z = n_docs;
    while (z - a > 1) {
      const int m = (a + z) >> 1;
      if (doc_off[m] <= i) a = m;
      else z = m;
    }
    s = min(doc_off[a], i);
    e = max(doc_off[a + 1], i + 1);
  }
  // keys seen by query i (0 <= i < N)
  template <bool CAUSAL>
  __device__ void keys(int i, int& lo, int& hi) const {
    lo = window ? max(0, i - window + 1) : 0;
    hi = CAUSAL ? i : (window ? min(N - 1, i + window - 1) : N - 1);
    if (n_docs > 0) {
      int ds, de;
      doc_of(i, ds, de);
      lo = max(lo, ds);
      hi = min(hi, de - 1);
    }
  }
  // queries that see key j (0 <= j < N)
  template <bool CAUSAL>
  __device__ void queries(int j, int& lo, int& hi) const {
    lo = CAUSAL ? j : (window ? max(0, j - window + 1) : 0);
    hi = window ? min(N - 1, j + window - 1) : N - 1;
    if (n_docs > 0) {
      int ds, de;
      doc_of(j, ds, de);
      lo = max(lo, ds);
      hi = min(hi, de - 1);
    }
  }
};

// D_i = dO_i . O_i, HD / 8 threads per row (8 elements each).
template <int HD>
__global__ void delta_kernel(const float* __restrict__ O, const uint16_t* __restrict__ dO,
                             float* __restrict__ D, long long rows) {
  constexpr int kParts = HD / 8;
  const long long row = (long long)blockIdx.x * (256 / kParts) + (threadIdx.x / kParts);
  const int part = threadIdx.x % kParts;
  float acc = 0.f;
  if (row < rows) {
    const f32x4* o = (const f32x4*)(O + row * HD + 8 * part);
    const u32x4 g = *(const u32x4*)(dO + row * HD + 8 * part);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x4 ov = o[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = g[2 * i + (e >> 1)];
        const float gv = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
        acc = __builtin_fmaf(ov[e], gv, acc);
      }
    }
  }
#pragma unroll
  for (int off = kParts / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, kParts);
  if (row < rows && part == 0) D[row] = acc;
}

// The forward's score modifications, on the scaled score s (log2 units below): soft-capping
// t = C tanh(s / C), then the ALiBi bias t -= a_h |i - j|.  P is rebuilt from the modified
// score, and the cap's chain rule multiplies dS by dt/ds = 1 - tanh(s / C)^2.
struct Mods {
  const float* alibi;   // Hq slopes (natural units), or null
  float k2;             // soft-capping: 2 scale log2(e) / C (raw q.k to 2 s log2(e) / C); 0 = off
  float ccap;           // soft-capping: C log2(e)
};

// dK, dV for 128 keys of one (batch, kv head): each wave owns 32 keys; the loop runs
// over the group's query heads and their 64-query tiles (causal: only tiles that reach
// the workgroup's keys; BAND: only tiles within the keys' window and documents).
template <int D, bool CAUSAL, bool BAND, bool MODS>
__global__ __launch_bounds__(kBThreads) void dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, float* __restrict__ dK,
    float* __restrict__ dV, int Hq, int Hkv, int N, int nkb, float c, float scale, Band band,
    Mods mods) {
  __shared__ BTile<D> tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = lane & 31, h = lane >> 5;
  // the key blocks of one kv head run on one XCD (its Q / dO tiles stay in that L2);
  // causal: the blocks with the most query tiles (the lowest keys) first
  const WorkItem wi = decode_workgroup(blockIdx.x, gridDim.x, Hkv, 1, nkb, CAUSAL);
  const int kb = wi.qb_rank, hkv = wi.hkv, b = wi.b;
  const int group = Hq / Hkv;
  const int K0 = kb * kBBlock;
  const int kw0 = K0 + wave * 32;           // this wave's keys
  const int key = kw0 + n32;                // this lane's key (accumulator column)

  const size_t khead = (size_t)(b * Hkv + hkv) * N;
  // K^T and V^T as B operands: lane holds K[key][16c + 8h .. +7] for each d chunk c
  u32x4 kop[D / 16], vop[D / 16];
  {
    const int kr = min(key, N - 1);
    const uint16_t* krow = K + (khead + kr) * D;
    const uint16_t* vrow = V + (khead + kr) * D;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      kop[cc] = *(const u32x4*)(krow + 16 * cc + 8 * h);
      vop[cc] = *(const u32x4*)(vrow + 16 * cc + 8 * h);
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }

  // query tiles [qt0, qt1) reach the workgroup's keys; BAND: this lane's key is seen by
  // queries [kq_lo, kq_hi], this wave's keys by [wq_lo, wq_hi]
  int qt0 = CAUSAL ? K0 / kBTile : 0, qt1 = (N + kBTile - 1) / kBTile;
  int kq_lo = 0, kq_hi = 0, wq_lo = 0, wq_hi = 0;
  if (BAND) {
    int lo, hi, lo2, hi2;
    band.queries<CAUSAL>(K0, lo, hi);
    band.queries<CAUSAL>(min(K0 + kBBlock - 1, N - 1), lo2, hi2);
    qt0 = lo / kBTile;
    qt1 = hi2 / kBTile + 1;
    band.queries<CAUSAL>(min(key, N - 1), kq_lo, kq_hi);
    band.queries<CAUSAL>(min(kw0, N - 1), wq_lo, hi);
    band.queries<CAUSAL>(min(kw0 + 31, N - 1), lo, wq_hi);
    // the same in every lane of the wave: kept in scalar registers
    wq_lo = __builtin_amdgcn_readfirstlane(wq_lo);
    wq_hi = __builtin_amdgcn_readfirstlane(wq_hi);
  }
  const int pm = perm_row(n32);
  // (query head, query tile) steps in order; the next step's rows are fetched into
  // registers while the current one computes
  const int steps_per_head = qt1 - qt0;
  const int nsteps = group * steps_per_head;
  auto step_q0 = [&](int st) { return (qt0 + st % steps_per_head) * kBTile; };
  auto step_qhead = [&](int st) {
    return (size_t)(b * Hq + hkv * group + st / steps_per_head) * N;
  };
  StageRegs<D> sr;
  float lse_next = 0.f, d_next = 0.f;
  auto fetch = [&](int st) {
    const size_t qh = step_qhead(st);
    const int q0 = step_q0(st);
    stage_load(sr, Q + qh * D, dO + qh * D, q0, N);
    if (tid < kBTile) {
      const int qr = q0 + tid;
      lse_next = qr < N ? LSE[qh + qr] : -__builtin_inff();
      d_next = qr < N ? Delta[qh + qr] : 0.f;
    }
  };
  if (nsteps > 0) fetch(0);
  for (int st = 0; st < nsteps; ++st) {
    const int q0 = step_q0(st);
    // ALiBi slope of this step's query head, log2 units (0: no bias)
    const float slope2 =
        (MODS && mods.alibi != nullptr)
            ? mods.alibi[hkv * group + st / steps_per_head] * kLog2e : 0.f;
    {
      __syncthreads();
      stage_store(tile, sr, true, true);
      if (tid < kBTile) {
        // rows past N or without visible keys: +inf makes their weights 0
        tile.s0[tid] = (lse_next == -__builtin_inff()) ? __builtin_inff() : lse_next * kLog2e;
        tile.s1[tid] = d_next;
      }
      __syncthreads();
      if (st + 1 < nsteps) fetch(st + 1);
      // this wave's keys all lie after the tile's last query (or outside its band):
      // nothing visible
      if (!BAND && CAUSAL && kw0 > q0 + kBTile - 1) continue;
      if (BAND && (kw0 >= N || q0 > wq_hi || q0 + kBTile - 1 < wq_lo)) continue;
      // one 32-query half: S and dP, then P and dS, then the dK / dV products
      auto half = [&](int sub) {
        const int qs = q0 + kSub * sub;
        // S = Q_pi K^T and dP = dO_pi V^T (queries x keys; rows permuted), each as two
        // accumulation chains over alternate d chunks
        f32x16 s = zero16(), dp = zero16(), s2 = zero16(), dp2 = zero16();
#pragma unroll
        for (int cc = 0; cc < D / 16; cc += 2) {
          const uint8_t* qr = tile.a + (kSub * sub + pm) * BTile<D>::kRow + 32 * cc + 16 * h;
          const uint8_t* gr = tile.b + (kSub * sub + pm) * BTile<D>::kRow + 32 * cc + 16 * h;
          s = mfma_bf16(lds_u32x4(qr), kop[cc], s);
          dp = mfma_bf16(lds_u32x4(gr), vop[cc], dp);
          s2 = mfma_bf16(lds_u32x4(qr + 32), kop[cc + 1], s2);
          dp2 = mfma_bf16(lds_u32x4(gr + 32), vop[cc + 1], dp2);
        }
        // this lane's 16 query rows: acc_row(r, h) = 8h + r (r < 8), 16 + 8h + r - 8
        f32x4 l4[4], d4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = kSub * sub + 16 * (i >> 1) + 8 * h + 4 * (i & 1);
          l4[i] = *(const f32x4*)(tile.s0 + r0);
          d4[i] = *(const f32x4*)(tile.s1 + r0);
        }
        // P and dS; register r holds query qs + acc_row(r, h) for this lane's key.  CAP:
        // soft-capping (a uniform choice, made once around the loop)
        f32x16 p, ds;
        auto elements = [&](auto cap_tag) {
          constexpr bool CAP = decltype(cap_tag)::value;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = acc_row(r, h);
            float x, dfac = 1.f;
            if constexpr (MODS) {
              const float raw = s[r] + s2[r];
              float t = raw * c;
              if constexpr (CAP) {
                const float y = __builtin_amdgcn_exp2f(raw * mods.k2);
                const float th = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(y + 1.f), 1.f);
                t = mods.ccap * th;
                dfac = __builtin_fmaf(-th, th, 1.f);
              }
              t = __builtin_fmaf(-slope2, __builtin_fabsf((float)(key - (qs + qi))), t);
              x = t - l4[r >> 2][r & 3];
            } else {
              x = __builtin_fmaf(s[r] + s2[r], c, -l4[r >> 2][r & 3]);
            }
            // non-short-circuit: evaluated whole, so no branch per element
            const bool vis = BAND ? ((key < N) & (qs + qi >= kq_lo) & (qs + qi <= kq_hi))
                                  : (key < N && (!CAUSAL || key <= qs + qi));
            const float pr = vis ? __builtin_amdgcn_exp2f(x) : 0.f;
            p[r] = pr;
            const float g = pr * (dp[r] + dp2[r] - d4[r >> 2][r & 3]);
            ds[r] = CAP ? g * dfac : g;
          }
        };
        if constexpr (MODS) {
          if (mods.k2 != 0.f) elements(std::true_type{});
          else elements(std::false_type{});
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = acc_row(r, h);
            const float x = __builtin_fmaf(s[r] + s2[r], c, -l4[r >> 2][r & 3]);
            // non-short-circuit: evaluated whole, so no branch per element
            const bool vis = BAND ? ((key < N) & (qs + qi >= kq_lo) & (qs + qi <= kq_hi))
                                  : (key < N && (!CAUSAL || key <= qs + qi));
            const float pr = vis ? __builtin_amdgcn_exp2f(x) : 0.f;
            p[r] = pr;
            ds[r] = pr * (dp[r] + dp2[r] - d4[r >> 2][r & 3]);
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS (d x keys), over the two 16-query chunks
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const u32x4 pb = pack_chunk(p, q2), db = pack_chunk(ds, q2);
#pragma unroll
          for (int dbk = 0; dbk < D / 32; ++dbk) {
            const int dcol = 32 * dbk + n32;
            const int off = dcol * kColStride + 2 * kSub * sub + 32 * q2 + 16 * h;
            dv[dbk] = mfma_bf16(lds_u32x4(tile.bt + off), pb, dv[dbk]);
            dk[dbk] = mfma_bf16(lds_u32x4(tile.at + off), db, dk[dbk]);
          }
        }
      };
      // The two halves are independent until they meet in dK / dV.  Unrolled (non-causal),
      // the compiler overlaps one half's exponentials with the other's products; in the
      // causal and band forms, with their masks, both halves' scores live at once push the
      // K / V operands into AGPRs (415 register moves per step against 128), so the halves
      // run one after the other.
      if constexpr (CAUSAL || BAND || MODS) {
#pragma unroll 1
        for (int sub = 0; sub < kBTile / kSub; ++sub) half(sub);
      } else {
#pragma unroll
        for (int sub = 0; sub < kBTile / kSub; ++sub) half(sub);
      }
    }
  }
  // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane holds d 32dbk + 8a + 4h + 0..3 of its key
  if (key < N) {
    float* dkrow = dK + (khead + key) * D;
    float* dvrow = dV + (khead + key) * D;
#pragma unroll
    for (int dbk = 0; dbk < D / 32; ++dbk)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int col = 32 * dbk + 8 * a4 + 4 * h;
        f32x4 kv = {dk[dbk][4 * a4] * scale, dk[dbk][4 * a4 + 1] * scale,
                    dk[dbk][4 * a4 + 2] * scale, dk[dbk][4 * a4 + 3] * scale};
        f32x4 vv = {dv[dbk][4 * a4], dv[dbk][4 * a4 + 1], dv[dbk][4 * a4 + 2],
                    dv[dbk][4 * a4 + 3]};
        *(f32x4*)(dkrow + col) = kv;
        *(f32x4*)(dvrow + col) = vv;
      }
  }
}

// dQ for 128 queries of one (batch, query head): each wave owns 32 queries; the loop
// runs over 64-key tiles (causal: up to the workgroup's last query; BAND: the tiles within
// the queries' window and documents).
// (The body; the kernels below set the waves per SIMD.)
// CAP: the soft-capping path is compiled in (MODS with ALiBi only leaves it out).
template <int D, bool CAUSAL, bool BAND, bool MODS, bool CAP_ON = MODS>
__device__ __forceinline__ void dq_body(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, float* __restrict__ dQ,
    int Hq, int Hkv, int N, int nqb, float c, float scale, Band band, Mods mods) {
  __shared__ BTile<D> tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = lane & 31, h = lane >> 5;
  // the query blocks of one kv head's query heads run on one XCD (its K / V tiles stay
  // in that L2); causal: the longest (highest) query blocks first
  const int group = Hq / Hkv;
  const WorkItem wi = decode_workgroup(blockIdx.x, gridDim.x, Hkv, group, nqb, CAUSAL);
  const int qb = CAUSAL ? nqb - 1 - wi.qb_rank : wi.qb_rank;
  const int hkv = wi.hkv, b = wi.b, hq = hkv * group + wi.g;
  const int Q0 = qb * kBBlock;
  const int qw0 = Q0 + wave * 32;
  const int qi = qw0 + n32;                 // this lane's query (accumulator column)

  const size_t qhead = (size_t)(b * Hq + hq) * N;
  const size_t khead = (size_t)(b * Hkv + hkv) * N;
  // Q^T and dO^T as B operands: lane holds Q[qi][16c + 8h .. +7]
  u32x4 qop[D / 16], gop[D / 16];
  float lse2 = __builtin_inff(), dlt = 0.f;
  {
    const int qr = min(qi, N - 1);
    const uint16_t* qrow = Q + (qhead + qr) * D;
    const uint16_t* grow = dO + (qhead + qr) * D;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      qop[cc] = *(const u32x4*)(qrow + 16 * cc + 8 * h);
      gop[cc] = *(const u32x4*)(grow + 16 * cc + 8 * h);
    }
    if (qi < N) {
      const float l = LSE[qhead + qi];
      lse2 = (l == -__builtin_inff()) ? __builtin_inff() : l * kLog2e;
      dlt = Delta[qhead + qi];
    }
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = zero16();

  // key tiles [kt0, kt1) reach the workgroup's queries; BAND: this lane's query sees keys
  // [q_lo, q_hi], this wave's queries see [w_lo, w_hi]
  int kt0 = 0, kt1 = ((CAUSAL ? min(N, Q0 + kBBlock) : N) + kBTile - 1) / kBTile;
  int q_lo = 0, q_hi = 0, w_lo = 0, w_hi = 0;
  if (BAND) {
    int lo, hi, lo2, hi2;
    band.keys<CAUSAL>(Q0, lo, hi);
    band.keys<CAUSAL>(min(Q0 + kBBlock - 1, N - 1), lo2, hi2);
    kt0 = lo / kBTile;
    kt1 = hi2 / kBTile + 1;
    band.keys<CAUSAL>(min(qi, N - 1), q_lo, q_hi);
    band.keys<CAUSAL>(min(qw0, N - 1), w_lo, hi);
    band.keys<CAUSAL>(min(qw0 + 31, N - 1), lo, w_hi);
    // the same in every lane of the wave: kept in scalar registers
    w_lo = __builtin_amdgcn_readfirstlane(w_lo);
    w_hi = __builtin_amdgcn_readfirstlane(w_hi);
  }
  const int pm = perm_row(n32);
  // the next key tile is fetched into registers while the current one computes
  StageRegs<D> sr;
  if (kt1 > kt0) stage_load(sr, K + khead * D, V + khead * D, kt0 * kBTile, N);
  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * kBTile;
    __syncthreads();
    stage_store(tile, sr, true, false);
    __syncthreads();
    if (kt + 1 < kt1) stage_load(sr, K + khead * D, V + khead * D, k0 + kBTile, N);
    if (!BAND && CAUSAL && k0 > qw0 + 31) continue;
    if (BAND && (qw0 >= N || k0 > w_hi || k0 + kBTile - 1 < w_lo)) continue;
    // one 32-key half: S^T and dP^T, then dS^T, then the dQ products
    constexpr bool kTwoChains = !((BAND || MODS) && D == 128);
    // ALiBi slope of this query head, log2 units (0: no bias)
    const float slope2 = (MODS && mods.alibi != nullptr) ? mods.alibi[hq] * kLog2e : 0.f;
    auto half = [&](int sub) {
      const int ks = k0 + kSub * sub;
      // S^T = K_pi Q^T and dP^T = V_pi dO^T (keys x queries; rows permuted), two chains
      // each; one each in the band form at d = 128, whose bounds leave no room for four
      f32x16 s = zero16(), dp = zero16(), s2 = zero16(), dp2 = zero16();
#pragma unroll
      for (int cc = 0; cc < D / 16; cc += 2) {
        const uint8_t* kr = tile.a + (kSub * sub + pm) * BTile<D>::kRow + 32 * cc + 16 * h;
        const uint8_t* vr = tile.b + (kSub * sub + pm) * BTile<D>::kRow + 32 * cc + 16 * h;
        s = mfma_bf16(lds_u32x4(kr), qop[cc], s);
        dp = mfma_bf16(lds_u32x4(vr), gop[cc], dp);
        if constexpr (kTwoChains) {
          s2 = mfma_bf16(lds_u32x4(kr + 32), qop[cc + 1], s2);
          dp2 = mfma_bf16(lds_u32x4(vr + 32), gop[cc + 1], dp2);
        } else {
          s = mfma_bf16(lds_u32x4(kr + 32), qop[cc + 1], s);
          dp = mfma_bf16(lds_u32x4(vr + 32), gop[cc + 1], dp);
        }
      }
      // dS^T; register r holds key ks + acc_row(r, h) for this lane's query.  CAP:
      // soft-capping (a uniform choice, made once around the loop)
      f32x16 ds;
      auto elements = [&](auto cap_tag) {
      constexpr bool CAP = decltype(cap_tag)::value;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = ks + acc_row(r, h);
        // non-short-circuit: evaluated whole, so no branch per element (causal: kj <= qi
        // < N implies kj < N)
        const bool vis = BAND     ? ((qi < N) & (kj >= q_lo) & (kj <= q_hi))
                         : CAUSAL ? ((qi < N) & (kj <= qi))
                                  : ((kj < N) & (qi < N));
        const float sv = kTwoChains ? s[r] + s2[r] : s[r];
        const float dpv = kTwoChains ? dp[r] + dp2[r] : dp[r];
        // hidden: 2^-inf = 0 (a select, not a branch around the exponential)
        if constexpr (MODS) {
          float t = sv * c, dfac = 1.f;
          if constexpr (CAP) {
            const float y = __builtin_amdgcn_exp2f(sv * mods.k2);
            const float th = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(y + 1.f), 1.f);
            t = mods.ccap * th;
            dfac = __builtin_fmaf(-th, th, 1.f);
          }
          t = __builtin_fmaf(-slope2, __builtin_fabsf((float)(kj - qi)), t);
          const float x = vis ? t - lse2 : -__builtin_inff();
          const float g = __builtin_amdgcn_exp2f(x) * (dpv - dlt);
          ds[r] = CAP ? g * dfac : g;
        } else {
          const float x = vis ? __builtin_fmaf(sv, c, -lse2) : -__builtin_inff();
          ds[r] = __builtin_amdgcn_exp2f(x) * (dpv - dlt);
        }
      }
      };
      if (CAP_ON && mods.k2 != 0.f) elements(std::true_type{});
      else elements(std::false_type{});
      // dQ^T += K^T dS^T (d x queries), over the two 16-key chunks
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const u32x4 db = pack_chunk(ds, k2);
#pragma unroll
        for (int dbk = 0; dbk < D / 32; ++dbk) {
          const int dcol = 32 * dbk + n32;
          const int off = dcol * kColStride + 2 * kSub * sub + 32 * k2 + 16 * h;
          dq[dbk] = mfma_bf16(lds_u32x4(tile.at + off), db, dq[dbk]);
        }
      }
    };
    // unrolled, one half's exponentials overlap the other's products; the band and
    // modified forms' extra work would push that past the 256 registers of two waves per SIMD
    if constexpr (BAND || MODS) {
#pragma unroll 1
      for (int sub = 0; sub < kBTile / kSub; ++sub) half(sub);
    } else {
#pragma unroll
      for (int sub = 0; sub < kBTile / kSub; ++sub) half(sub);
    }
  }
  if (qi < N) {
    float* row = dQ + (qhead + qi) * D;
#pragma unroll
    for (int dbk = 0; dbk < D / 32; ++dbk)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 v = {dq[dbk][4 * a4] * scale, dq[dbk][4 * a4 + 1] * scale,
                   dq[dbk][4 * a4 + 2] * scale, dq[dbk][4 * a4 + 3] * scale};
        *(f32x4*)(row + 32 * dbk + 8 * a4 + 4 * h) = v;
      }
  }
}

// Two waves per SIMD (at most 256 registers each; two workgroups' tiles fit the CU's LDS),
// so one workgroup's products overlap the other's exponentials and staging.
template <int D, bool CAUSAL, bool BAND, bool MODS, bool CAP_ON = MODS>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, float* __restrict__ dQ,
    int Hq, int Hkv, int N, int nqb, float c, float scale, Band band, Mods mods) {
  dq_body<D, CAUSAL, BAND, MODS, CAP_ON>(Q, K, V, dO, LSE, Delta, dQ, Hq, Hkv, N, nqb, c, scale,
                                         band, mods);
}

// The same at one wave per SIMD (up to 512 registers): the soft-capping form at d = 128,
// whose per-element work does not fit the 256 registers of two waves per SIMD.
template <int D, bool CAUSAL, bool BAND, bool MODS>
__global__ __launch_bounds__(kBThreads) void dq_kernel_1w(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, float* __restrict__ dQ,
    int Hq, int Hkv, int N, int nqb, float c, float scale, Band band, Mods mods) {
  dq_body<D, CAUSAL, BAND, MODS>(Q, K, V, dO, LSE, Delta, dQ, Hq, Hkv, N, nqb, c, scale, band,
                                 mods);
}

template <int D, bool CAUSAL, bool BAND, bool MODS>
hipError_t launch_bwd_t(const BwdArgs& a) {
  const long long rows = (long long)a.B * a.Hq * a.N;
  constexpr int kRowsPerBlock = 256 / (D / 8);
  hipLaunchKernelGGL(delta_kernel<D>, dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(256), 0, (hipStream_t)a.stream, a.o, (const uint16_t*)a.dout, a.delta,
                     rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (a.N + kBBlock - 1) / kBBlock;
  const Band band{a.N, a.window, a.n_docs, a.doc_offsets};
  const Mods mods{a.alibi, a.softcap > 0.f ? 2.f * a.c / a.softcap : 0.f,
                  a.softcap * kLog2e};
  hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, BAND, MODS>), dim3((unsigned)(a.B * a.Hkv * nb)),
                     dim3(kBThreads), 0, (hipStream_t)a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                     a.delta, a.dk, a.dv, a.Hq, a.Hkv, a.N, nb, a.c, a.scale, band, mods);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(a.B * a.Hq * nb));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kBThreads), 0, (hipStream_t)a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.delta, a.dq, a.Hq, a.Hkv, a.N, nb, a.c,
                       a.scale, band, mods);
  };
  if constexpr (MODS && D == 128) {
    if (a.softcap > 0.f) go(dq_kernel_1w<D, CAUSAL, BAND, MODS>);
    else go(dq_kernel<D, CAUSAL, BAND, MODS, false>);   // ALiBi only: two waves per SIMD
  } else {
    go(dq_kernel<D, CAUSAL, BAND, MODS>);
  }
  return hipGetLastError();
}

template <int D, bool MODS>
hipError_t launch_bwd_dm(const BwdArgs& a) {
  const bool band = a.window > 0 || a.n_docs > 0;
  if (a.causal)
    return band ? launch_bwd_t<D, true, true, MODS>(a) : launch_bwd_t<D, true, false, MODS>(a);
  return band ? launch_bwd_t<D, false, true, MODS>(a) : launch_bwd_t<D, false, false, MODS>(a);
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  return (a.alibi != nullptr || a.softcap > 0.f) ? launch_bwd_dm<D, true>(a)
                                                 : launch_bwd_dm<D, false>(a);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.d == 128) return launch_bwd_d<128>(a);
  if (a.d == 64) return launch_bwd_d<64>(a);
  return hipErrorNotSupported;
}

}  // namespace attn

// Workspace of the allocation-free backward (attn_bwd_noalloc): D_i for up to
// ATTN_NOALLOC_MAX_ROWS rows.  Each GPU holds its own copy for the life of the process;
// every call on a GPU shares it.  In host code this name is a stand-in, not a device
// address: the kernels get the address resolved by noalloc_scratch below.
static __device__ __align__(256) float scratch[ATTN_NOALLOC_MAX_ROWS];

namespace attn {

// Device address of `scratch` on the current device, resolved once per device.
hipError_t noalloc_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace attn
