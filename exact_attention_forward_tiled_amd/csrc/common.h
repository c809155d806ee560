// Device-side vector types and small helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Max over the two 32-lane halves of a wave (lane l and lane l ^ 32).
__device__ __forceinline__ float max_across_halves(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  return x + __shfl_xor(x, 32);
}

// Pack two fp32 into a bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Workgroup -> (batch, kv head, query head in the group, query block rank).
// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).  When
// the kv heads split evenly over the XCDs, each XCD gets a contiguous range of
// kv heads, so the query heads sharing a kv head and all their query blocks
// read K/V through the same L2.  Within an XCD the dispatch order is: causal,
// query block outermost with the heaviest (longest key range) first, so the
// XCD's CUs take the longest work first and end together; non-causal, query
// heads of a group, then query blocks, then kv heads.  Rank 0 is the heaviest
// query block when causal (the caller maps rank -> block).
struct WorkItem {
  int b, hkv, g, qb_rank;
};

__device__ __forceinline__ WorkItem decode_workgroup(int w, int G, int Hkv, int group, int nqb,
                                                     bool causal) {
  const int nkv = G / (group * nqb);   // B * Hkv
  WorkItem it;
  int kv;
  if (nkv % 8 == 0) {
    const int x = w % 8, r = w / 8;    // XCD and dispatch rank within it
    const int kv_per = nkv / 8;
    int kvl;
    if (causal) {
      it.qb_rank = r / (kv_per * group);
      const int t = r % (kv_per * group);
      kvl = t / group;
      it.g = t % group;
    } else {
      it.g = r % group;
      it.qb_rank = (r / group) % nqb;
      kvl = r / (group * nqb);
    }
    kv = x * kv_per + kvl;
  } else {
    // uneven split: plain order; causal, heaviest query blocks first across the grid
    const int hw = nkv * group;
    const int r = causal ? w % hw : w / nqb;
    it.qb_rank = causal ? w / hw : w % nqb;
    it.g = r % group;
    kv = r / group;
  }
  it.hkv = kv % Hkv;
  it.b = kv / Hkv;
  return it;
}

}  // namespace attn
