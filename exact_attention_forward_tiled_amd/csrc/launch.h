// Internal interface between the C-ABI entry points (attn_api.cpp) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, N, d, causal;
  float c;          // |scale| * log2(e): scores to log2 units
  float tau;        // rescale threshold, log2 units
  uint32_t qsign;   // 0x80008000 flips the sign of every bf16 Q element (scale < 0)
  int poly_pairs;   // of each lane's 16 score pairs per tile, how many use the cubic exp2
                    // (0, 4, 8, 12 or 16; the rest use v_exp_f32)
  int window;       // sliding window W (0: none; 1 <= W < N): key j visible from query i
                    // only when i - W < j, and j < i + W without the causal mask
  const float* alibi;   // device, Hq ALiBi slopes (natural-log units per key), or null
  float softcap;    // soft-capping C (0: off)
  const int* doc_offsets;   // device, n_docs + 1 document offsets (0, ..., N), or null
  int n_docs;       // documents (0: no document masking)
  unsigned long long* stats;
  void* stream;
};

// Block-scaled (MXFP4 / MXFP8) forward: element codes and E8M0 scales.
struct MxArgs {
  const uint8_t *qc, *qs, *kc, *ks, *vtc, *vts;
  float* o;
  float* lse;
  int B, Hq, Hkv, N, d, causal;
  float c;          // |scale| * log2(e): scores to log2 units
  float tau;
  uint32_t qsign;   // flips the sign bit of every Q element (scale < 0): 0x88888888 for E2M1
                    // nibbles, 0x80808080 for E4M3 bytes
  int window;       // sliding window W (0: none; 1 <= W < N)
  const int* doc_offsets;   // device, n_docs + 1 document offsets, or null
  int n_docs;       // documents (0: no document masking)
  unsigned long long* stats;
  void* stream;
};

// bf16 backward (d = 64 or 128): gradients of the forward from its saved O and LSE.
struct BwdArgs {
  const void* q;        // bf16 [B, Hq, N, d]
  const void* k;        // bf16 [B, Hkv, N, d]
  const void* v;        // bf16 [B, Hkv, N, d]
  const float* o;       // fp32 [B, Hq, N, d], the forward's output
  const float* lse;     // fp32 [B, Hq, N], the forward's LSE (natural log)
  const void* dout;     // bf16 [B, Hq, N, d]
  float* dq;            // fp32 [B, Hq, N, d]
  float* dk;            // fp32 [B, Hkv, N, d]
  float* dv;            // fp32 [B, Hkv, N, d]
  float* delta;         // fp32 [B, Hq, N] workspace (D_i = dO_i . O_i)
  int B, Hq, Hkv, N, d, causal;
  int window;           // sliding window W (0: none; 1 <= W < N), as in FwdArgs
  const int* doc_offsets;   // device, n_docs + 1 document offsets (0, ..., N), or null
  int n_docs;           // documents (0: no document masking)
  const float* alibi;   // device, Hq ALiBi slopes, or null
  float softcap;        // soft-capping C (0: off)
  float c;              // scale * log2(e)
  float scale;
  void* stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);
// Device address of the allocation-free backward's static workspace on the current device.
hipError_t noalloc_scratch(float** out);
hipError_t launch_fwd_mxfp4(const MxArgs& a);
hipError_t launch_fwd_mxfp8(const MxArgs& a);
hipError_t launch_quantize_rows(const float* x, uint8_t* codes, uint8_t* scales, long long rows,
                                int cols, void* stream);
hipError_t launch_quantize_cols_t(const float* x, uint8_t* codes, uint8_t* scales, int batch,
                                  int rows, int cols, void* stream);
hipError_t launch_quantize8_rows(const float* x, uint8_t* codes, uint8_t* scales, long long rows,
                                 int cols, void* stream);
hipError_t launch_quantize8_cols_t(const float* x, uint8_t* codes, uint8_t* scales, int batch,
                                   int rows, int cols, void* stream);

}  // namespace attn
