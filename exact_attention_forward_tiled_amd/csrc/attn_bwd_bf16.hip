// bf16 attention backward: dQ, dK, dV from the saved LSE.
//
// The forward keeps only O and the row log-sum-exp; the backward recomputes the
// probabilities from them instead of storing the N x N matrix ("FlashAttention-4
// 发布：原生支持Blackwell…", section "从V1到V4", FlashAttention (2022) entry:
// tiling plus recomputation; "Hardware-Aware FP4 FlashAttention-4", section
// "2. Causal Backward Cuantizado": the forward saves the LSE and the backward
// rebuilds the probabilities from it).  With s = scale q.k and P = exp(s - LSE):
//   D_i  = dO_i . O_i                         (dq_kernel, for its own query rows, into the
//                                              caller's workspace)
//   dS   = P * (dO V^T - D)
//   dQ   = scale dS K                          (dq_kernel, one workgroup per query block;
//                                              launched first)
//   dV   = P^T dO,  dK = scale dS^T Q          (dkdv_kernel, one workgroup per key block,
//                                              two waves of different roles per 32 keys;
//                                              reads D from the workspace)
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
constexpr int kBBlock = kBWaves * 32;    // keys per dK / dV workgroup
constexpr int kBTile = 64;               // queries (dK/dV) or keys (dQ) staged per loop step
constexpr int kSub = 32;                 // rows per MFMA block: a step is two such halves
constexpr int kQWaves = 8;               // dQ workgroup: 8 waves of 32 queries each
constexpr int kQThreads = kQWaves * 64;
constexpr int kQBlock = kQWaves * 32;    // queries per dQ workgroup

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

// The forward's score modifications, on the scaled score s (log2 units below): soft-capping
// t = C tanh(s / C), then the ALiBi bias t -= a_h |i - j|.  P is rebuilt from the modified
// score, and the cap's chain rule multiplies dS by dt/ds = 1 - tanh(s / C)^2.
struct Mods {
  const float* alibi;   // Hq slopes (natural units), or null
  float k2;             // soft-capping: 2 scale log2(e) / C (raw q.k to 2 s log2(e) / C); 0 = off
  float ccap;           // soft-capping: C log2(e)
};

// One query tile of the dK/dV loop in LDS, with its per-row scalars.  Each tensor is
// stored by 16-byte column chunks: chunk c of row r at (c * 68 + r) * 16, the 64 rows of a
// chunk followed by 4 units of padding.  Three access patterns then touch every bank once
// per pass: 16 lanes reading one chunk of 16 different rows (the row operands), 32 lanes
// reading 8 bytes of 4 chunks x 4 rows (the transposing reads), and 16 lanes writing
// consecutive rows of one chunk (the staging).
template <int D>
struct alignas(16) QTile {
  static constexpr int kChunk = (kBTile + 4) * 16;   // bytes per column chunk
  float l2[kBTile];                   // LSE in log2 units (+inf: the row has no weight)
  float dl[kBTile];                   // D_i
  uint8_t q[D / 8 * kChunk];
  uint8_t g[D / 8 * kChunk];          // dO
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane t
// returns element t % 4 of the 8-byte words addressed by lanes t / 4, t / 4 + 4, t / 4 + 8,
// t / 4 + 12 (probed).  When lane a of the group addresses the 8 bytes holding columns
// 4 (a % 4) .. + 3 of row a / 4 of a bf16 tile, lane t receives column t of four
// consecutive rows.
__device__ __forceinline__ uint2 lds_tr16(const uint8_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

// A operand (8 consecutive k = rows of the tile, one m = column per lane) from a QTile
// tensor: lane l holds rows r0 + 8 (l / 32) + 0..7 of column c0 + l % 32, when p is the
// lane's address of row r0 + 8 (l / 32) + (l % 16) / 4, column c0 + 16 ((l / 16) % 2) +
// 4 (l % 4) (rows r + 4 lie 64 bytes further on in a chunk).
__device__ __forceinline__ u32x4 lds_tr_operand(const uint8_t* p) {
  const uint2 lo = lds_tr16(p), hi = lds_tr16(p + 64);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

constexpr int kKVThreads = 2 * kBThreads;    // dK/dV workgroup: two waves per 32 keys
constexpr int kRing = 4;                     // dK/dV: LDS operand reads in flight per product

// dK, dV for 128 keys of one (batch, kv head).  The loop runs over the group's query
// heads and their 64-query tiles (causal: only tiles that reach the workgroup's keys;
// BAND: only tiles within the keys' window and documents).
//
// Two waves own each 32 keys, with different roles, so that each needs half the
// registers and two waves share every SIMD (one's elementwise work runs beside the
// other's products):
//   P wave  (waves 0-3): S = Q K^T, P; dV^T += dO^T P
//   dS wave (waves 4-7): dP = dO V^T; dS = P (dP - D); dK^T += Q^T dS
// P crosses from one to the other through LDS in fp32 (with soft-capping, P times the
// cap's derivative, which is all dS needs of it).  The query tiles are double-buffered:
// the next tile is fetched into registers at the top of a step and written to the other
// buffer after the middle barrier.  Q^T and dO^T come from the row-major tile through
// transposing reads.
template <int D, bool CAUSAL, bool BAND, bool MODS>
__global__ __launch_bounds__(kKVThreads) void dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, float* __restrict__ dK,
    float* __restrict__ dV, int Hq, int Hkv, int N, int nkb, float c, float scale, Band band,
    Mods mods) {
  using Tile = QTile<D>;
  constexpr int kChunk = Tile::kChunk;
  constexpr int kUnits = kBTile * D * 2 / 16 / kKVThreads;   // 16-byte units per thread
  __shared__ Tile tiles[2];
  __shared__ f32x4 xchg[kBWaves][kBTile / 8][64];            // P: [pair][register quad][lane]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (kBWaves - 1);
  const bool p_role = wave < kBWaves;
  const int n32 = lane & 31, h = lane >> 5;
  // the key blocks of one kv head run on one XCD (its Q / dO tiles stay in that L2);
  // causal: the blocks with the most query tiles (the lowest keys) first
  const WorkItem wi = decode_workgroup(blockIdx.x, gridDim.x, Hkv, 1, nkb, CAUSAL);
  const int kb = wi.qb_rank, hkv = wi.hkv, b = wi.b;
  const int group = Hq / Hkv;
  const int K0 = kb * kBBlock;
  const int kw0 = K0 + pair * 32;           // this wave's keys
  const int key = kw0 + n32;                // this lane's key (accumulator column)
  const size_t khead = (size_t)(b * Hkv + hkv) * N;

  // query tiles [qt0, qt1) reach the workgroup's keys; BAND: this lane's key is seen by
  // queries [kq_lo, kq_hi], this wave's keys by [wq_lo, wq_hi], every key of the wave by
  // [fq_lo, fq_hi]
  int qt0 = CAUSAL ? K0 / kBTile : 0, qt1 = (N + kBTile - 1) / kBTile;
  int kq_lo = 0, kq_hi = 0, wq_lo = 0, wq_hi = 0, fq_lo = 0, fq_hi = -1;
  if (BAND) {
    int lo, hi, lo2, hi2;
    band.queries<CAUSAL>(K0, lo, hi);
    band.queries<CAUSAL>(min(K0 + kBBlock - 1, N - 1), lo2, hi2);
    qt0 = lo / kBTile;
    qt1 = hi2 / kBTile + 1;
    band.queries<CAUSAL>(min(key, N - 1), kq_lo, kq_hi);
    band.queries<CAUSAL>(min(kw0, N - 1), wq_lo, fq_hi);
    band.queries<CAUSAL>(min(kw0 + 31, N - 1), fq_lo, wq_hi);
    // the same in every lane of the wave: kept in scalar registers
    wq_lo = __builtin_amdgcn_readfirstlane(wq_lo);
    wq_hi = __builtin_amdgcn_readfirstlane(wq_hi);
    fq_lo = __builtin_amdgcn_readfirstlane(fq_lo);
    fq_hi = __builtin_amdgcn_readfirstlane(fq_hi);
  }
  // lane offsets: S / dP A operands (rows in the order pi, chunk 2 cc + h) and the
  // transposed operands (row 8 h + (lane % 16) / 4, column 16 ((lane / 16) % 2) +
  // 4 (lane % 4): chunk 2 ((lane / 16) % 2) + (lane % 4) / 2, byte 8 (lane % 2))
  const int a_off = h * kChunk + perm_row(n32) * 16;
  const int t_off = (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) * kChunk +
                    (8 * h + ((lane & 15) >> 2)) * 16 + 8 * (lane & 1);
  // (query head, query tile) steps in order
  const int steps_per_head = qt1 - qt0;
  const int nsteps = group * steps_per_head;
  auto step_q0 = [&](int st) { return (qt0 + st % steps_per_head) * kBTile; };
  auto step_qhead = [&](int st) {
    return (size_t)(b * Hq + hkv * group + st / steps_per_head) * N;
  };
  // staging: unit u of a thread is row unit % 64, bytes 16 (unit / 64) .. + 15 (rows past
  // N read as row N - 1: in bounds; their LSE of +inf gives them no weight)
  u32x4 sq[kUnits], sg[kUnits];
  float lse_next = 0.f, d_next = 0.f;
  auto fetch = [&](int st) {
    const size_t qh = step_qhead(st);
    const int q0 = step_q0(st);
    const uint16_t* qb = Q + qh * D;
    const uint16_t* gb = dO + qh * D;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int unit = tid + u * kKVThreads;
      const int gr = min(q0 + unit % kBTile, N - 1);
      sq[u] = *(const u32x4*)(qb + (size_t)gr * D + 8 * (unit / kBTile));
      sg[u] = *(const u32x4*)(gb + (size_t)gr * D + 8 * (unit / kBTile));
    }
    if (tid < kBTile) {
      const int qr = q0 + tid;
      lse_next = qr < N ? LSE[qh + qr] : -__builtin_inff();
      d_next = qr < N ? Delta[qh + qr] : 0.f;
    }
  };
  auto store = [&](Tile& t) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int unit = tid + u * kKVThreads;
      const int off = (unit / kBTile) * kChunk + (unit % kBTile) * 16;
      *(u32x4*)(t.q + off) = sq[u];
      *(u32x4*)(t.g + off) = sg[u];
    }
    if (tid < kBTile) {
      // rows past N or without visible keys: +inf makes their weights 0
      t.l2[tid] = (lse_next == -__builtin_inff()) ? __builtin_inff() : lse_next * kLog2e;
      t.dl[tid] = d_next;
    }
  };
  // this wave's keys all lie after the tile's last query (or outside its band): nothing
  // visible in the step
  auto idle_at = [&](int q0) {
    return BAND ? (kw0 >= N || q0 > wq_hi || q0 + kBTile - 1 < wq_lo)
                : (CAUSAL && kw0 > q0 + kBTile - 1);
  };
  // one 32 x 32 product set: acc = X_pi Y^T over d, X rows from the tile, Y^T in registers
  auto rows_product = [&](const uint8_t* x, const u32x4 (&y)[D / 16], int sub) {
    f32x16 acc = zero16();
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc)
      acc = mfma_bf16(lds_u32x4(x + 2 * cc * kChunk + kSub * sub * 16 + a_off), y[cc], acc);
    return acc;
  };
  // Both 32-query halves of a product, as one sequence of MFMAs whose LDS operands are read
  // kRing products ahead (one read and one product per scheduling slot); left to itself the
  // compiler reads each operand just before its product and waits for it.
  // a0 / a1 = X_pi Y^T over d for the two halves, the halves' products interleaved:
  auto rows_product_pair = [&](const uint8_t* x, const u32x4 (&y)[D / 16], f32x16& a0,
                               f32x16& a1) {
    constexpr int NK = 2 * (D / 16);
    auto rd = [&](int k) {
      return lds_u32x4(x + 2 * (k >> 1) * kChunk + kSub * (k & 1) * 16 + a_off);
    };
    u32x4 ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) ring[i] = rd(i);
    a0 = zero16();
    a1 = zero16();
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const u32x4 op = ring[k % kRing];
      if (k + kRing < NK) ring[k % kRing] = rd(k + kRing);
      if (k & 1) a1 = mfma_bf16(op, y[k >> 1], a1);
      else a0 = mfma_bf16(op, y[k >> 1], a0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // acc[dbk] += X^T B over both halves (B = b0 for queries 0-31, b1 for 32-63), X^T from the
  // tile by transposing reads, each accumulator's products in query order:
  auto cols_product_pair = [&](f32x16 (&acc)[D / 32], const uint8_t* x, const u32x4 (&b0)[2],
                               const u32x4 (&b1)[2]) {
    constexpr int NK = 4 * (D / 32);
    auto rd = [&](int k) {
      const int sub = k / (2 * (D / 32)), q2 = (k / (D / 32)) & 1, dbk = k % (D / 32);
      return lds_tr_operand(x + 4 * dbk * kChunk + (kSub * sub + 16 * q2) * 16 + t_off);
    };
    u32x4 ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) ring[i] = rd(i);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int sub = k / (2 * (D / 32)), q2 = (k / (D / 32)) & 1, dbk = k % (D / 32);
      const u32x4 op = ring[k % kRing];
      if (k + kRing < NK) ring[k % kRing] = rd(k + kRing);
      acc[dbk] = mfma_bf16(op, sub ? b1[q2] : b0[q2], acc[dbk]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto write_out = [&](float* dst, const f32x16 (&acc)[D / 32], float mul) {
    if (key < N) {
      float* row = dst + (khead + key) * D;
#pragma unroll
      for (int dbk = 0; dbk < D / 32; ++dbk)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          f32x4 v = {acc[dbk][4 * a4] * mul, acc[dbk][4 * a4 + 1] * mul,
                     acc[dbk][4 * a4 + 2] * mul, acc[dbk][4 * a4 + 3] * mul};
          *(f32x4*)(row + 32 * dbk + 8 * a4 + 4 * h) = v;
        }
    }
  };

  if (nsteps > 0) {
    fetch(0);
    store(tiles[0]);
  }
  __syncthreads();
  if (p_role) {
    // K^T as B operand: lane holds K[key][16c + 8h .. +7] for each d chunk c
    u32x4 kop[D / 16];
    {
      const uint16_t* krow = K + (khead + min(key, N - 1)) * D;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) kop[cc] = *(const u32x4*)(krow + 16 * cc + 8 * h);
      // wait for the operands here: left pending into the loop, they would make every
      // step wait for its own prefetch of the next tile as well
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) asm volatile("" ::"v"(kop[cc]));
    }
    f32x16 dv[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dv[i] = zero16();
    for (int st = 0; st < nsteps; ++st) {
      const Tile& tl = tiles[st & 1];
      const int q0 = step_q0(st);
      if (st + 1 < nsteps) fetch(st + 1);
      const bool idle = idle_at(q0);
      // ALiBi slope of this step's query head, log2 units (0: no bias)
      const float slope2 =
          (MODS && mods.alibi != nullptr)
              ? mods.alibi[hkv * group + st / steps_per_head] * kLog2e : 0.f;
      u32x4 pb[2][2];
      // P of one half; register r holds query q0 + 32 sub + acc_row(r, h) for this lane's
      // key.  CAP: soft-capping; MASKED: some pair of the step is hidden (uniform choices)
      auto half = [&](auto cap_tag, auto mask_tag, int sub) {
        constexpr bool CAP = decltype(cap_tag)::value;
        constexpr bool MASKED = decltype(mask_tag)::value;
        const f32x16 s = rows_product(tl.q, kop, sub);
        // register r holds query qs + c(r), c(r) = 16 (r / 8) + r % 8: the masks and the
        // ALiBi distance compare per-lane differences with these constants
        const int qs = q0 + kSub * sub + 8 * h;
        const int kd = key - qs;
        f32x4 l4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          l4[i] = *(const f32x4*)(tl.l2 + kSub * sub + 16 * (i >> 1) + 8 * h + 4 * (i & 1));
        f32x16 p, pd;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          constexpr int kC[16] = {0, 1, 2, 3, 4, 5, 6, 7, 16, 17, 18, 19, 20, 21, 22, 23};
          const int cr = kC[r];
          float x, dfac = 1.f;
          if constexpr (MODS) {
            float t = s[r] * c;
            if constexpr (CAP) {
              const float y = __builtin_amdgcn_exp2f(s[r] * mods.k2);
              const float th = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(y + 1.f), 1.f);
              t = mods.ccap * th;
              dfac = __builtin_fmaf(-th, th, 1.f);
            }
            t = __builtin_fmaf(-slope2, __builtin_fabsf((float)(kd - cr)), t);
            x = t - l4[r >> 2][r & 3];
          } else {
            x = __builtin_fmaf(s[r], c, -l4[r >> 2][r & 3]);
          }
          float pr;
          if constexpr (MASKED) {
            // non-short-circuit: evaluated whole, so no branch per element
            const bool vis = BAND ? ((key < N) & (cr >= kq_lo - qs) & (cr <= kq_hi - qs))
                                  : (key < N && (!CAUSAL || kd <= cr));
            pr = vis ? __builtin_amdgcn_exp2f(x) : 0.f;
          } else {
            pr = __builtin_amdgcn_exp2f(x);
          }
          p[r] = pr;
          pd[r] = CAP ? pr * dfac : pr;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xchg[pair][4 * sub + i][lane] = f32x4{pd[4 * i], pd[4 * i + 1], pd[4 * i + 2], pd[4 * i + 3]};
        pb[sub][0] = pack_chunk(p, 0);
        pb[sub][1] = pack_chunk(p, 1);
      };
      auto phase1 = [&](auto cap_tag, auto mask_tag) {
        half(cap_tag, mask_tag, 0);
        half(cap_tag, mask_tag, 1);
      };
      if (!idle) {
        // every key of the wave is visible from every query of the step (query rows past
        // N need no mask: their LSE of +inf gives them weight 0)
        const bool full = BAND ? (kw0 + 31 < N && q0 >= fq_lo && q0 + kBTile - 1 <= fq_hi)
                               : (kw0 + 31 < N && (!CAUSAL || kw0 + 31 <= q0));
        if constexpr (MODS) {
          if (mods.k2 != 0.f) {
            if (full) phase1(std::true_type{}, std::false_type{});
            else phase1(std::true_type{}, std::true_type{});
          } else {
            if (full) phase1(std::false_type{}, std::false_type{});
            else phase1(std::false_type{}, std::true_type{});
          }
        } else {
          if (full) phase1(std::false_type{}, std::false_type{});
          else phase1(std::false_type{}, std::true_type{});
        }
      }
      __syncthreads();
      // dV^T += dO^T P
      if (!idle) cols_product_pair(dv, tl.g, pb[0], pb[1]);
      if (st + 1 < nsteps) store(tiles[(st + 1) & 1]);
      __syncthreads();
    }
    write_out(dV, dv, 1.f);
  } else {
    // V^T as B operand
    u32x4 vop[D / 16];
    {
      const uint16_t* vrow = V + (khead + min(key, N - 1)) * D;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) vop[cc] = *(const u32x4*)(vrow + 16 * cc + 8 * h);
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) asm volatile("" ::"v"(vop[cc]));
    }
    f32x16 dk[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dk[i] = zero16();
    for (int st = 0; st < nsteps; ++st) {
      const Tile& tl = tiles[st & 1];
      const int q0 = step_q0(st);
      if (st + 1 < nsteps) fetch(st + 1);
      const bool idle = idle_at(q0);
      f32x16 dp0, dp1;
      if (!idle) rows_product_pair(tl.g, vop, dp0, dp1);
      __syncthreads();
      // the dS wave's dS and dK are this phase's longest chain (the P wave only has its dV
      // products): its instructions go first when both waves of the SIMD are ready
      __builtin_amdgcn_s_setprio(1);
      if (!idle) {
        // dS = P (dP - D) for both halves, then dK^T += Q^T dS
        u32x4 db[2][2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const f32x16& dp = sub ? dp1 : dp0;
          f32x16 ds;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 pd = xchg[pair][4 * sub + i][lane];
            const f32x4 d4 =
                *(const f32x4*)(tl.dl + kSub * sub + 16 * (i >> 1) + 8 * h + 4 * (i & 1));
#pragma unroll
            for (int e = 0; e < 4; ++e) ds[4 * i + e] = pd[e] * (dp[4 * i + e] - d4[e]);
          }
          db[sub][0] = pack_chunk(ds, 0);
          db[sub][1] = pack_chunk(ds, 1);
        }
        cols_product_pair(dk, tl.q, db[0], db[1]);
      }
      __builtin_amdgcn_s_setprio(0);
      if (st + 1 < nsteps) store(tiles[(st + 1) & 1]);
      __syncthreads();
    }
    write_out(dK, dk, scale);
  }
}

// One key tile of the dQ loop in LDS: K and V stored by 16-byte column chunks, as QTile.
template <int D>
struct alignas(16) KVTile {
  static constexpr int kChunk = (kBTile + 4) * 16;   // bytes per column chunk
  uint8_t k[D / 8 * kChunk];
  uint8_t v[D / 8 * kChunk];
};

// dQ for 256 queries of one (batch, query head), and D = dO . O for those queries (written
// to the workspace for the dK / dV kernel): each wave owns 32 queries; the loop runs over
// 64-key tiles (causal: up to the workgroup's last query; BAND: the tiles within
// the queries' window and documents).  The key tiles are double-buffered: the next tile is
// loaded straight into the other buffer (direct-to-LDS, no registers) at the top of a step
// and waited for at the step's one barrier.  K^T comes from the stored K rows through
// transposing reads.
// (The body; the kernels below set the waves per SIMD.)
// CAP: the soft-capping path is compiled in (MODS with ALiBi only leaves it out).
template <int D, bool CAUSAL, bool BAND, bool MODS, bool CAP_ON = MODS>
__device__ __forceinline__ void dq_body(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ O, float* __restrict__ Delta,
    float* __restrict__ dQ, int Hq, int Hkv, int N, int nqb, float c, float scale, Band band,
    Mods mods) {
  using Tile = KVTile<D>;
  constexpr int kChunk = Tile::kChunk;
  __shared__ Tile tiles[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, h = lane >> 5;
  // the query blocks of one kv head's query heads run on one XCD (its K / V tiles stay
  // in that L2); causal: the longest (highest) query blocks first
  const int group = Hq / Hkv;
  const WorkItem wi = decode_workgroup(blockIdx.x, gridDim.x, Hkv, group, nqb, CAUSAL);
  const int qb = CAUSAL ? nqb - 1 - wi.qb_rank : wi.qb_rank;
  const int hkv = wi.hkv, b = wi.b, hq = hkv * group + wi.g;
  const int Q0 = qb * kQBlock;
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
    // D = dO . O for this lane's query: the lane holds dO at d = 16 cc + 8 h .. + 7; the
    // other half-wave holds the rest of the row
    const float* orow = O + (qhead + qr) * D;
    float part = 0.f;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      const f32x4 o0 = *(const f32x4*)(orow + 16 * cc + 8 * h);
      const f32x4 o1 = *(const f32x4*)(orow + 16 * cc + 8 * h + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = gop[cc][e >> 1];
        const float gv = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
        part = __builtin_fmaf(e < 4 ? o0[e] : o1[e - 4], gv, part);
      }
    }
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                               false, false);
    dlt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (qi < N) {
      const float l = LSE[qhead + qi];
      lse2 = (l == -__builtin_inff()) ? __builtin_inff() : l * kLog2e;
      if (h == 0) Delta[qhead + qi] = dlt;   // for the dK / dV kernel, launched after this one
    }
    // wait for the operands here: left pending into the loop, they would make every step
    // wait for its own prefetch of the next tile as well
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) asm volatile("" ::"v"(qop[cc]), "v"(gop[cc]));
    asm volatile("" ::"v"(lse2), "v"(dlt));
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = zero16();

  // key tiles [kt0, kt1) reach the workgroup's queries; BAND: this lane's query sees keys
  // [q_lo, q_hi], this wave's queries see [w_lo, w_hi] together and [f_lo, f_hi] each
  int kt0 = 0, kt1 = ((CAUSAL ? min(N, Q0 + kQBlock) : N) + kBTile - 1) / kBTile;
  int q_lo = 0, q_hi = 0, w_lo = 0, w_hi = 0, f_lo = 0, f_hi = -1;
  if (BAND) {
    int lo, hi, lo2, hi2;
    band.keys<CAUSAL>(Q0, lo, hi);
    band.keys<CAUSAL>(min(Q0 + kQBlock - 1, N - 1), lo2, hi2);
    kt0 = lo / kBTile;
    kt1 = hi2 / kBTile + 1;
    band.keys<CAUSAL>(min(qi, N - 1), q_lo, q_hi);
    band.keys<CAUSAL>(min(qw0, N - 1), w_lo, f_hi);
    band.keys<CAUSAL>(min(qw0 + 31, N - 1), f_lo, w_hi);
    // the same in every lane of the wave: kept in scalar registers
    w_lo = __builtin_amdgcn_readfirstlane(w_lo);
    w_hi = __builtin_amdgcn_readfirstlane(w_hi);
    f_lo = __builtin_amdgcn_readfirstlane(f_lo);
    f_hi = __builtin_amdgcn_readfirstlane(f_hi);
  }
  // lane offsets: S^T / dP^T A operands (rows in the order pi, chunk 2 cc + h) and the
  // transposed K operand (as in the dK/dV kernel)
  const int a_off = h * kChunk + perm_row(n32) * 16;
  const int t_off = (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) * kChunk +
                    (8 * h + ((lane & 15) >> 2)) * 16 + 8 * (lane & 1);
  // staging: unit u of a thread is row unit % 64, chunk unit / 64 (rows past N read as row
  // N - 1: in bounds; their keys are masked)

  // ALiBi slope of this query head, log2 units (0: no bias)
  const float slope2 = (MODS && mods.alibi != nullptr) ? mods.alibi[hq] * kLog2e : 0.f;
  // the next tile straight from global memory into LDS: one wave-wide 16-byte load per
  // 64-row column chunk (lane = row, consecutive LDS slots); waited for at the barrier
  auto fetch_lds = [&](int kt, Tile& t) {
    const size_t gr = khead + min(kt * kBTile + lane, N - 1);
#pragma unroll
    for (int i = 0; i < 2 * (D / 8) / kQWaves; ++i) {
      const int cid = wave + i * kQWaves;
      const int c = cid % (D / 8);
      const bool isv = cid >= D / 8;
      const uint16_t* src = (isv ? V : K) + gr * D + 8 * c;
      const uint32_t lds = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)((isv ? t.v : t.k) + c * kChunk));
      // written out rather than the builtin, with which the compiler makes the next LDS read
      // of any address wait for these loads.  m0 is a register the compiler reserves: no
      // other code in these kernels uses it, so its clobber needs no save or restore.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
                   : "memory", "m0");
#pragma clang diagnostic pop
    }
  };
  if (kt1 > kt0) fetch_lds(kt0, tiles[0]);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  for (int kt = kt0; kt < kt1; ++kt) {
    const Tile& tl = tiles[(kt - kt0) & 1];
    const int k0 = kt * kBTile;
    if (kt + 1 < kt1) fetch_lds(kt + 1, tiles[(kt + 1 - kt0) & 1]);
    // this wave's queries see none of the tile's keys: nothing to do in this step
    const bool idle = BAND ? (qw0 >= N || k0 > w_hi || k0 + kBTile - 1 < w_lo)
                           : (CAUSAL && k0 > qw0 + 31);
    // one 32-key half: S^T and dP^T, then dS^T, then the dQ products
    auto half = [&](int sub) {
      // register r holds key ks + c(r), c(r) = 16 (r / 8) + r % 8, for this lane's query
      const int ks = k0 + kSub * sub + 8 * h;
      const int qd = qi - ks;
      // S^T = K_pi Q^T and dP^T = V_pi dO^T (keys x queries; rows permuted); the two
      // chains alternate, so neither product waits on its own previous one
      f32x16 s = zero16(), dp = zero16();
      {
        // each LDS operand read kRing products ahead (one read and one product per
        // scheduling slot), as in the dK / dV kernel
        constexpr int NK = 2 * (D / 16);
        auto rd = [&](int k) {
          return lds_u32x4(((k & 1) ? tl.v : tl.k) + 2 * (k >> 1) * kChunk + kSub * sub * 16 +
                           a_off);
        };
        u32x4 ring[kRing];
#pragma unroll
        for (int i = 0; i < kRing; ++i) ring[i] = rd(i);
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          const u32x4 op = ring[k % kRing];
          if (k + kRing < NK) ring[k % kRing] = rd(k + kRing);
          if (k & 1) dp = mfma_bf16(op, gop[k >> 1], dp);
          else s = mfma_bf16(op, qop[k >> 1], s);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // dS^T.  CAP: soft-capping; MASKED: some (key, query) pair of the half is hidden
      // (uniform choices)
      f32x16 ds;
      auto elements = [&](auto cap_tag, auto mask_tag) {
        constexpr bool CAP = decltype(cap_tag)::value;
        constexpr bool MASKED = decltype(mask_tag)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          constexpr int kC[16] = {0, 1, 2, 3, 4, 5, 6, 7, 16, 17, 18, 19, 20, 21, 22, 23};
          const int cr = kC[r];
          float x;
          float dfac = 1.f;
          if constexpr (MODS) {
            float t = s[r] * c;
            if constexpr (CAP) {
              const float y = __builtin_amdgcn_exp2f(s[r] * mods.k2);
              const float th = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(y + 1.f), 1.f);
              t = mods.ccap * th;
              dfac = __builtin_fmaf(-th, th, 1.f);
            }
            t = __builtin_fmaf(-slope2, __builtin_fabsf((float)(cr - qd)), t);
            x = t - lse2;
          } else {
            x = __builtin_fmaf(s[r], c, -lse2);
          }
          if constexpr (MASKED) {
            // non-short-circuit: evaluated whole, so no branch per element (causal:
            // key <= query < N implies key < N); hidden: 2^-inf = 0
            const bool vis = BAND     ? ((qi < N) & (cr >= q_lo - ks) & (cr <= q_hi - ks))
                             : CAUSAL ? ((qi < N) & (cr <= qd))
                                      : ((cr < N - ks) & (qi < N));
            x = vis ? x : -__builtin_inff();
          }
          const float g = __builtin_amdgcn_exp2f(x) * (dp[r] - dlt);
          ds[r] = CAP ? g * dfac : g;
        }
      };
      // every key of the half is visible from every query of the wave
      const int kh = k0 + kSub * sub;
      const bool full = BAND ? (qw0 + 31 < N && kh >= f_lo && kh + kSub - 1 <= f_hi)
                             : (qw0 + 31 < N && kh + kSub - 1 < N &&
                                (!CAUSAL || kh + kSub - 1 <= qw0));
      if constexpr (MODS) {
        // (the modified forms take the masked path only: two copies would not fit)
        if (CAP_ON && mods.k2 != 0.f) elements(std::true_type{}, std::true_type{});
        else elements(std::false_type{}, std::true_type{});
      } else {
        if (full) elements(std::false_type{}, std::false_type{});
        else elements(std::false_type{}, std::true_type{});
      }
      // dQ^T += K^T dS^T (d x queries), over the two 16-key chunks; K^T by transposing reads,
      // through an operand ring.  Raised priority: the other wave on this SIMD then does its
      // element work beside these products instead of taking turns with them
      __builtin_amdgcn_s_setprio(1);
      {
        constexpr int NK = 2 * (D / 32);
        const u32x4 dbs[2] = {pack_chunk(ds, 0), pack_chunk(ds, 1)};
        auto rd = [&](int k) {
          const int k2 = k / (D / 32), dbk = k % (D / 32);
          return lds_tr_operand(tl.k + 4 * dbk * kChunk + (kSub * sub + 16 * k2) * 16 + t_off);
        };
        u32x4 ring[kRing];
#pragma unroll
        for (int i = 0; i < kRing; ++i) ring[i] = rd(i);
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          const u32x4 op = ring[k % kRing];
          if (k + kRing < NK) ring[k % kRing] = rd(k + kRing);
          dq[k % (D / 32)] = mfma_bf16(op, dbs[k / (D / 32)], dq[k % (D / 32)]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    if (!idle) {
      // the band and modified forms' extra work would not fit two halves at once in the
      // 256 registers of two waves per SIMD
      if constexpr (BAND || MODS) {
#pragma unroll 1
        for (int sub = 0; sub < kBTile / kSub; ++sub) half(sub);
      } else {
#pragma unroll
        for (int sub = 0; sub < kBTile / kSub; ++sub) half(sub);
      }
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// One workgroup of 8 waves per CU, two waves per SIMD (at most 256 registers each): every
// staged K / V tile serves 256 queries.  CAP_ON: the soft-capping path is compiled in.
template <int D, bool CAUSAL, bool BAND, bool MODS, bool CAP_ON = MODS>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ O, float* __restrict__ Delta,
    float* __restrict__ dQ, int Hq, int Hkv, int N, int nqb, float c, float scale, Band band,
    Mods mods) {
  dq_body<D, CAUSAL, BAND, MODS, CAP_ON>(Q, K, V, dO, LSE, O, Delta, dQ, Hq, Hkv, N, nqb, c,
                                         scale, band, mods);
}

template <int D, bool CAUSAL, bool BAND, bool MODS>
hipError_t launch_bwd_t(const BwdArgs& a) {
  const int nb = (a.N + kBBlock - 1) / kBBlock;     // dK / dV: key blocks
  const int nqb = (a.N + kQBlock - 1) / kQBlock;    // dQ: query blocks
  const Band band{a.N, a.window, a.n_docs, a.doc_offsets};
  const Mods mods{a.alibi, a.softcap > 0.f ? 2.f * a.c / a.softcap : 0.f,
                  a.softcap * kLog2e};
  // dQ first: it also computes D = dO . O for its rows into the workspace
  const dim3 grid((unsigned)(a.B * a.Hq * nqb));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kQThreads), 0, (hipStream_t)a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.o, a.delta, a.dq, a.Hq, a.Hkv, a.N, nqb,
                       a.c, a.scale, band, mods);
  };
  if constexpr (MODS && D == 128) {
    // ALiBi alone: the soft-capping path compiled out (fewer registers and instructions)
    if (a.softcap > 0.f) go(dq_kernel<D, CAUSAL, BAND, MODS, true>);
    else go(dq_kernel<D, CAUSAL, BAND, MODS, false>);
  } else {
    go(dq_kernel<D, CAUSAL, BAND, MODS>);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, BAND, MODS>), dim3((unsigned)(a.B * a.Hkv * nb)),
                     dim3(kKVThreads), 0, (hipStream_t)a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                     a.delta, a.dk, a.dv, a.Hq, a.Hkv, a.N, nb, a.c, a.scale, band, mods);
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
