// C-ABI entry points of libattn: argument validation, then one kernel launch
// on the caller's stream.  Nothing here allocates or synchronises.

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/attn.h"
#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  g_last_hip_error = (int)e;
  return ATTN_EHIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_opts(const attn_opts* o) {
  if (!(o->tau >= 0.f && o->tau <= ATTN_TAU_MAX)) return ATTN_EINVAL;   // also rejects NaN
  if (o->exp_mode != ATTN_EXP_HW && o->exp_mode != ATTN_EXP_POLY && o->exp_mode != ATTN_EXP_MIX)
    return ATTN_EINVAL;
  if (o->exp_mode == ATTN_EXP_MIX && !(o->poly_frac >= 0.f && o->poly_frac <= 1.f))
    return ATTN_EINVAL;
  if (o->window < 0) return ATTN_EINVAL;
  if (!(o->softcap >= 0.f) || !isfinite(o->softcap)) return ATTN_EINVAL;
  if (o->doc_offsets != nullptr && o->n_docs < 1) return ATTN_EINVAL;
  return ATTN_OK;
}

// Score pairs per lane and tile (of 16) whose exponential is the cubic.
int poly_pairs(const attn_opts* o) {
  if (o->exp_mode == ATTN_EXP_HW) return 0;
  if (o->exp_mode == ATTN_EXP_POLY) return 16;
  return 4 * (int)lrintf(o->poly_frac * 4.f);   // nearest quarter
}

int check_common(int B, int Hq, int Hkv, int N, int d, int causal, float scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_EINVAL;
  if (!isfinite(scale)) return ATTN_EINVAL;
  // every flat row index b*Hq*N + h*N + i must fit in 32 bits
  if ((long long)B * Hq * N >= (1LL << 31)) return ATTN_EUNSUPPORTED;
  // the forwards address one head's K and V tiles through buffer descriptors with 32-bit
  // byte offsets: one head's bf16 K (N * d * 2 bytes) must stay under 2 GiB
  if ((long long)N * d * 2 >= (1LL << 31)) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

// Shared validation and launch of the block-scaled forwards (MXFP4 and MXFP8).
// band_ok: the forward takes a sliding window and document offsets (both forwards do).
int mx_fwd(hipError_t (*launch)(const attn::MxArgs&), uint32_t qsign, bool band_ok,
           const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
           const uint8_t* vtc, const uint8_t* vts, float* o, float* lse, int B, int Hq, int Hkv,
           int N, int d, int causal, float scale, const attn_opts* opts, void* stream) {
  if (!qc || !qs || !kc || !ks || !vtc || !vts || !o || !lse) return ATTN_EINVAL;
  if (!aligned(qc, 16) || !aligned(kc, 16) || !aligned(vtc, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(ks, 4))
    return ATTN_EINVAL;
  int st = check_common(B, Hq, Hkv, N, d, causal, scale);
  if (st != ATTN_OK) return st;
  attn_opts def;
  attn_default_opts(&def);
  const attn_opts* op = opts ? opts : &def;
  st = check_opts(op);
  if (st != ATTN_OK) return st;
  if (d != 128 || N % 32 != 0 || op->alibi_slopes != nullptr || op->softcap != 0.f)
    return ATTN_EUNSUPPORTED;
  if (!band_ok && (op->window != 0 || op->doc_offsets != nullptr)) return ATTN_EUNSUPPORTED;

  attn::MxArgs a;
  a.qc = qc; a.qs = qs; a.kc = kc; a.ks = ks; a.vtc = vtc; a.vts = vts;
  a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d; a.causal = causal;
  a.c = fabsf(scale) * 1.4426950408889634f;
  a.qsign = scale < 0.f ? qsign : 0u;
  a.tau = op->tau;
  // a window at least N wide hides nothing: run the plain mask
  a.window = op->window >= N ? 0 : op->window;
  a.doc_offsets = op->doc_offsets;
  a.n_docs = op->doc_offsets != nullptr ? op->n_docs : 0;
  if (a.n_docs > N) return ATTN_EINVAL;   // documents are non-empty
  a.stats = op->stats;
  a.stream = stream;
  hipError_t e = launch(a);
  if (e == hipErrorNotSupported) return ATTN_EUNSUPPORTED;
  return hip_status(e);
}

// Validation of the backward's arguments and the kernel arguments; nothing is launched.
int bwd_args(attn::BwdArgs& a, const void* q, const void* k, const void* v, const float* o,
             const float* lse, const void* dout, float* dq, float* dk, float* dv, float* delta,
             int B, int Hq, int Hkv, int N, int d, int causal, float scale,
             const attn_opts* opts, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return ATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(delta, 4))
    return ATTN_EINVAL;
  int st = check_common(B, Hq, Hkv, N, d, causal, scale);
  if (st != ATTN_OK) return st;
  attn_opts def;
  attn_default_opts(&def);
  const attn_opts* op = opts ? opts : &def;
  st = check_opts(op);
  if (st != ATTN_OK) return st;
  if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
  if ((long long)B * Hkv * ((N + 127) / 128) >= (1LL << 31) ||
      (long long)B * Hq * ((N + 127) / 128) >= (1LL << 31))
    return ATTN_EUNSUPPORTED;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv; a.delta = delta;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d; a.causal = causal;
  // a window at least N wide hides nothing: run the plain mask
  a.window = op->window >= N ? 0 : op->window;
  a.doc_offsets = op->doc_offsets;
  a.n_docs = op->doc_offsets != nullptr ? op->n_docs : 0;
  if (a.n_docs > N) return ATTN_EINVAL;   // documents are non-empty
  a.alibi = op->alibi_slopes;
  a.softcap = op->softcap;
  a.c = scale * 1.4426950408889634f;
  a.scale = scale;
  a.stream = stream;
  return ATTN_OK;
}

}  // namespace

extern "C" {

void attn_default_opts(attn_opts* opts) {
  if (opts == nullptr) return;
  opts->tau = 8.0f;
  opts->exp_mode = ATTN_EXP_HW;
  opts->poly_frac = 0.5f;
  opts->stats = nullptr;
  opts->window = 0;
  opts->alibi_slopes = nullptr;
  opts->softcap = 0.f;
  opts->doc_offsets = nullptr;
  opts->n_docs = 0;
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported shape or format";
    case ATTN_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

int attn_fwd_ex(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
                int Hkv, int N, int d, int causal, float scale, const attn_opts* opts,
                void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return ATTN_EINVAL;
  int st = check_common(B, Hq, Hkv, N, d, causal, scale);
  if (st != ATTN_OK) return st;
  attn_opts def;
  attn_default_opts(&def);
  const attn_opts* op = opts ? opts : &def;
  st = check_opts(op);
  if (st != ATTN_OK) return st;
  if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;

  attn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d; a.causal = causal;
  a.c = fabsf(scale) * 1.4426950408889634f;
  a.tau = op->tau;
  a.qsign = scale < 0.f ? 0x80008000u : 0u;
  a.poly_pairs = poly_pairs(op);
  // a window at least N wide hides nothing: run the plain mask
  a.window = op->window >= N ? 0 : op->window;
  a.alibi = op->alibi_slopes;
  a.softcap = op->softcap;
  a.doc_offsets = op->doc_offsets;
  a.n_docs = op->doc_offsets != nullptr ? op->n_docs : 0;
  if (a.n_docs > N) return ATTN_EINVAL;   // documents are non-empty
  if ((a.alibi != nullptr || a.softcap > 0.f) && op->exp_mode != ATTN_EXP_HW)
    return ATTN_EUNSUPPORTED;
  a.stats = op->stats;
  a.stream = stream;
  return hip_status(attn::launch_fwd_bf16(a));
}

int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
             int Hkv, int N, int d, int causal, float scale) {
  return attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, nullptr, nullptr);
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv, float* delta, int B, int Hq,
                int Hkv, int N, int d, int causal, float scale, const attn_opts* opts,
                void* stream) {
  attn::BwdArgs a;
  const int st = bwd_args(a, q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal,
                          scale, opts, stream);
  if (st != ATTN_OK) return st;
  hipError_t e = attn::launch_bwd_bf16(a);
  if (e == hipErrorNotSupported) return ATTN_EUNSUPPORTED;
  return hip_status(e);
}

int attn_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, float* delta, int B, int Hq,
             int Hkv, int N, int d, int causal, float scale, void* stream) {
  return attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal, scale,
                     nullptr, stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const float* o,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv, int B,
                     int Hq, int Hkv, int N, int d, int causal, float scale,
                     const attn_opts* opts, void* stream) {
  attn::BwdArgs a;
  // validate everything first (dq stands in for the workspace pointer: non-null, aligned)
  const int st = bwd_args(a, q, k, v, o, lse, dout, dq, dk, dv, dq, B, Hq, Hkv, N, d, causal,
                          scale, opts, stream);
  if (st != ATTN_OK) return st;
  if ((long long)B * Hq * N > ATTN_NOALLOC_MAX_ROWS) return ATTN_EUNSUPPORTED;
  hipError_t e = attn::noalloc_scratch(&a.delta);
  if (e != hipSuccess) return hip_status(e);
  e = attn::launch_bwd_bf16(a);
  if (e == hipErrorNotSupported) return ATTN_EUNSUPPORTED;
  return hip_status(e);
}

int attn_fwd_mxfp4_ex(const uint8_t* q4, const uint8_t* qs, const uint8_t* k4, const uint8_t* ks,
                      const uint8_t* vt4, const uint8_t* vts, float* o, float* lse, int B, int Hq,
                      int Hkv, int N, int d, int causal, float scale, const attn_opts* opts,
                      void* stream) {
  return mx_fwd(attn::launch_fwd_mxfp4, 0x88888888u, true, q4, qs, k4, ks, vt4, vts, o, lse, B, Hq, Hkv,
                N, d, causal, scale, opts, stream);
}

int attn_fwd_mxfp4(const uint8_t* q4, const uint8_t* qs, const uint8_t* k4, const uint8_t* ks,
                   const uint8_t* vt4, const uint8_t* vts, float* o, float* lse, int B, int Hq,
                   int Hkv, int N, int d, int causal, float scale) {
  return attn_fwd_mxfp4_ex(q4, qs, k4, ks, vt4, vts, o, lse, B, Hq, Hkv, N, d, causal, scale,
                           nullptr, nullptr);
}

int attn_quantize_mxfp4_rows(const float* x, uint8_t* codes, uint8_t* scales, long long rows,
                             int cols, void* stream) {
  if (!x || !codes || !scales) return ATTN_EINVAL;
  if (rows < 1 || cols < 32 || cols % 32 != 0) return ATTN_EINVAL;
  if (!aligned(x, 16)) return ATTN_EINVAL;
  return hip_status(attn::launch_quantize_rows(x, codes, scales, rows, cols, stream));
}

int attn_quantize_mxfp4_cols_t(const float* x, uint8_t* codes, uint8_t* scales, int batch,
                               int rows, int cols, void* stream) {
  if (!x || !codes || !scales) return ATTN_EINVAL;
  if (batch < 1 || rows < 32 || rows % 32 != 0 || cols < 1) return ATTN_EINVAL;
  if ((long long)batch * rows * cols >= (1LL << 40)) return ATTN_EUNSUPPORTED;
  return hip_status(attn::launch_quantize_cols_t(x, codes, scales, batch, rows, cols, stream));
}

int attn_fwd_mxfp8_ex(const uint8_t* q8, const uint8_t* qs, const uint8_t* k8, const uint8_t* ks,
                      const uint8_t* vt8, const uint8_t* vts, float* o, float* lse, int B, int Hq,
                      int Hkv, int N, int d, int causal, float scale, const attn_opts* opts,
                      void* stream) {
  return mx_fwd(attn::launch_fwd_mxfp8, 0x80808080u, true, q8, qs, k8, ks, vt8, vts, o, lse, B, Hq, Hkv,
                N, d, causal, scale, opts, stream);
}

int attn_fwd_mxfp8(const uint8_t* q8, const uint8_t* qs, const uint8_t* k8, const uint8_t* ks,
                   const uint8_t* vt8, const uint8_t* vts, float* o, float* lse, int B, int Hq,
                   int Hkv, int N, int d, int causal, float scale) {
  return attn_fwd_mxfp8_ex(q8, qs, k8, ks, vt8, vts, o, lse, B, Hq, Hkv, N, d, causal, scale,
                           nullptr, nullptr);
}

int attn_quantize_mxfp8_rows(const float* x, uint8_t* codes, uint8_t* scales, long long rows,
                             int cols, void* stream) {
  if (!x || !codes || !scales) return ATTN_EINVAL;
  if (rows < 1 || cols < 32 || cols % 32 != 0) return ATTN_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16)) return ATTN_EINVAL;
  return hip_status(attn::launch_quantize8_rows(x, codes, scales, rows, cols, stream));
}

int attn_quantize_mxfp8_cols_t(const float* x, uint8_t* codes, uint8_t* scales, int batch,
                               int rows, int cols, void* stream) {
  if (!x || !codes || !scales) return ATTN_EINVAL;
  if (batch < 1 || rows < 32 || rows % 32 != 0 || cols < 1) return ATTN_EINVAL;
  if (!aligned(codes, 16)) return ATTN_EINVAL;
  if ((long long)batch * rows * cols >= (1LL << 40)) return ATTN_EUNSUPPORTED;
  return hip_status(attn::launch_quantize8_cols_t(x, codes, scales, batch, rows, cols, stream));
}

}  // extern "C"
