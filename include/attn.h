/*
 * attn.h -- C ABI of libattn: fused, tiled, exact attention forward on gfx950.
 *
 * Operation.  For every batch b, query head hq and query row i:
 *     s_ij   = scale * sum_c q[b,hq,i,c] * k[b,hk,j,c]        hk = hq / (Hq/Hkv)
 *     s_ij   = -inf  when causal and j > i
 *     O[i,:] = sum_j exp(s_ij - m_i) v[b,hk,j,:] / sum_j exp(s_ij - m_i),  m_i = max_j s_ij
 *     LSE_i  = m_i + ln(sum_j exp(s_ij - m_i))                  (natural log)
 * This is the FlashAttention forward: the N x N score matrix is never stored;
 * K/V are streamed in tiles and the softmax is carried online
 * ("FlashAttention-4发布：原生支持Blackwell…", section "从V1到V4", FlashAttention
 * (2022) entry: tiling and recomputation keep memory O(N); FlashAttention-2
 * entry: grouped-query attention).  The running row maximum is only moved,
 * and the output only rescaled, when a tile's maximum exceeds it by more than
 * a threshold tau ("FlashAttention-4 de NVIDIA: Un instrument…", section
 * "La ventaja técnica", and the aigc.bar page, section "FlashAttention-4：为
 * Blackwell而生的性能猛兽": rescaling only when the maximum changes enough);
 * this is exact in exact arithmetic.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, owned
 *    by the caller.  The library allocates no device memory, keeps no state
 *    between calls (except a thread-local last HIP error) and never
 *    synchronises: work is queued on the given stream (the null stream for the
 *    short forms) and outputs are valid once that stream has completed it.
 *  - Outputs must not alias inputs.
 *  - Arguments are validated before anything is launched; on error nothing is
 *    written.  Return codes are attn_status values; no C++ exception crosses
 *    the ABI.
 *  - Size limits (attention calls): B*Hq*N < 2^31 rows, and one head's bf16 K
 *    under 2 GiB (N*d*2 < 2^31, i.e. N < 2^23 at d = 128); larger requests return
 *    ATTN_EUNSUPPORTED (the kernels address rows and a head's K/V tiles with
 *    32-bit offsets).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_EINVAL = -1,        /* null pointer, non-positive size, Hq % Hkv != 0, causal not 0/1,
                                non-finite scale, bad option value */
    ATTN_EUNSUPPORTED = -2,  /* valid request the library does not implement (e.g. d not 64/128,
                                sizes past the limits below) */
    ATTN_EHIP = -3           /* a HIP runtime call or kernel launch failed; see attn_last_hip_error */
} attn_status;

/* Exponential used for the softmax weights. */
enum attn_exp_mode {
    ATTN_EXP_HW = 0,         /* hardware v_exp_f32 */
    ATTN_EXP_POLY = 1,       /* VALU cubic polynomial for 2^f on [0,1) plus exponent add
                                ("FlashAttention-4 de NVIDIA…", section "La ventaja técnica":
                                exponentials approximated by cubic polynomials on the FMA units) */
    ATTN_EXP_MIX = 2         /* a fraction poly_frac of the score elements on the cubic, the rest
                                on v_exp_f32 (same section: the exponential work shared between
                                the special-function unit and the FMA units) */
};

/* Largest accepted rescale threshold (log2 units): weights up to 2^64 times the row sum
 * stay far inside fp32, and the MXFP4 / MXFP8 weight scale exponents (tau - 2, tau - 7)
 * stay below the E8M0 NaN code. */
#define ATTN_TAU_MAX 64.0f

typedef struct attn_opts {
    float tau;               /* rescale threshold in log2 units, 0 <= tau <= ATTN_TAU_MAX
                                (else ATTN_EINVAL); 0 rescales on every increase of the
                                maximum (the textbook online softmax).  Stale weights reach
                                2^tau, so the bound keeps the fp32 sums and the E8M0 weight
                                scales of the block-scaled forwards far from overflow. */
    int exp_mode;            /* attn_exp_mode */
    float poly_frac;         /* ATTN_EXP_MIX only: fraction of the score elements whose
                                exponential is the cubic, in [0, 1]; the kernel uses the nearest
                                multiple of 1/4 (each lane's 16 score pairs of a 64-key tile are
                                split 4 ways, the cubic pairs spread evenly); otherwise ignored */
    unsigned long long* stats; /* nullable DEVICE pointer to 4 counters, accumulated atomically:
                                [0] wave-tile steps after each wave's first tile,
                                [1] rescale events among those steps.  Skip ratio = 1 - [1]/[0].
                                [2] shader-clock cycles and [3] 100 MHz reference-clock ticks
                                from start to end of each workgroup (its first wave), summed:
                                the mean shader clock is [2] / [3] * 100 MHz. */
    int window;              /* sliding window W >= 0 (the FlexAttention news page names sliding
                                window attention among the patterns the FA4 backend serves; it
                                prints no definition).  W = 0: no window.  W >= 1: key j is
                                visible from query i only when i - W < j, and, without the
                                causal mask, also j < i + W.  Tiles wholly outside the band are
                                skipped.  All three forwards and the backward. */
    const float* alibi_slopes; /* nullable DEVICE pointer to Hq floats, one ALiBi slope a_h per
                                query head (the same page names ALiBi; no definition printed):
                                the scaled score of query i and key j gets -a_h |i - j| added
                                before the mask.  Caller-owned, read during the call. */
    float softcap;           /* soft-capping C >= 0 (same page): 0 = off; C > 0 replaces the
                                scaled score s by C tanh(s / C), before the ALiBi bias and the
                                mask.  Both modifications need the hardware exponential
                                (ATTN_EUNSUPPORTED otherwise) and the bf16 forward (the MXFP4
                                forward returns ATTN_EUNSUPPORTED). */
    const int* doc_offsets;  /* nullable DEVICE pointer to n_docs + 1 ints: document masking (the
                                same page names it; no definition printed).  The sequence holds
                                n_docs documents packed back to back, 0 = o[0] < o[1] < ... <
                                o[n_docs] = N, the same layout for every batch entry; key j is
                                visible from query i only when both lie in one document (on top
                                of the causal mask and the window).  Tiles outside a workgroup's
                                documents are skipped.  Offsets that break the order give
                                unspecified values but every read stays within the array.
                                All three forwards and the backward. */
    int n_docs;              /* number of documents (>= 1 when doc_offsets is set; else ignored) */
} attn_opts;

/* Default options: tau = 8, hardware exp (poly_frac 0.5 for ATTN_EXP_MIX), no stats, no
   window, no ALiBi, no soft-capping, no documents. */
void attn_default_opts(attn_opts* opts);

/*
 * bf16 forward.
 *   q    bf16 [B, Hq,  N, d]      k, v  bf16 [B, Hkv, N, d]
 *   o    fp32 [B, Hq,  N, d]      lse   fp32 [B, Hq, N]   (natural log)
 *   d in {64, 128}; N >= 1 (any value; the tail tile is masked); causal in {0, 1}
 *   (key j visible to query i iff j <= i); scale finite (any sign).
 */
int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
             int B, int Hq, int Hkv, int N, int d, int causal, float scale);

/* As attn_fwd, with options (nullable: defaults) and a hipStream_t (nullable: null stream). */
int attn_fwd_ex(const void* q, const void* k, const void* v, float* o, float* lse,
                int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                const attn_opts* opts, void* stream);

/*
 * MXFP4 forward with Direct-P ("Hardware-Aware FP4 FlashAttention-4", section
 * "1. Direct-P para Inferencia Directa"): QK^T and PV run on the scaled FP4
 * MFMA; the softmax weights are mapped straight to E2M1 codes with one
 * power-of-two scale per 32 keys (relative to an integer running maximum), and
 * the denominator is accumulated from those same codes and scales.
 *   q4, k4   E2M1 codes [B, H*, N, d/2]  (two codes per byte: element 2i in the low nibble)
 *   qs, ks   E8M0 scales [B, H*, N, d/32] (block of 32 along d)
 *   vt4      E2M1 codes of V transposed [B, Hkv, d, N/2] (block of 32 along keys)
 *   vts      E8M0 scales [B, Hkv, d, N/32]
 *   o fp32 [B, Hq, N, d], lse fp32 [B, Hq, N]
 *   d = 128; N a multiple of 32 (else ATTN_EUNSUPPORTED).
 */
int attn_fwd_mxfp4(const uint8_t* q4, const uint8_t* qs, const uint8_t* k4, const uint8_t* ks,
                   const uint8_t* vt4, const uint8_t* vts, float* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale);

int attn_fwd_mxfp4_ex(const uint8_t* q4, const uint8_t* qs, const uint8_t* k4, const uint8_t* ks,
                      const uint8_t* vt4, const uint8_t* vts, float* o, float* lse,
                      int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                      const attn_opts* opts, void* stream);

/*
 * MXFP4 quantisation of fp32 inputs (OCP MX v1.0 rule: shared exponent
 * floor(log2(amax)) - 2 per block of 32, elements rounded to nearest E2M1
 * magnitude with ties to even, saturating at 6; an all-zero block gets
 * exponent 0; a value that rounds to 0 is stored as +0).
 *
 * attn_quantize_mxfp4_rows: x fp32 [rows, cols] -> codes [rows, cols/2], scales [rows, cols/32]
 *   (blocks along the contiguous axis; used for Q and K with cols = d).
 * attn_quantize_mxfp4_cols_t: x fp32 [batch, rows, cols] -> codes [batch, cols, rows/2],
 *   scales [batch, cols, rows/32] (blocks along rows, output transposed; used for V with
 *   rows = N keys, cols = d).
 * cols (resp. rows) must be a positive multiple of 32.
 */
int attn_quantize_mxfp4_rows(const float* x, uint8_t* codes, uint8_t* scales,
                             long long rows, int cols, void* stream);
int attn_quantize_mxfp4_cols_t(const float* x, uint8_t* codes, uint8_t* scales,
                               int batch, int rows, int cols, void* stream);

/*
 * MXFP8 forward ("Hardware-Aware FP4 FlashAttention-4", section "Resultados",
 * sets its FP4 path beside an FP8 one; section "2. Causal Backward Cuantizado"
 * keeps P and V in FP8; the aigc.bar page, section "从V1到V4", credits
 * FlashAttention-3 with FP8).  Operands are OCP MXFP8: E4M3 elements, one E8M0
 * scale per 32.  QK^T and PV run on the scaled FP8 MFMA; the softmax weights,
 * taken relative to an integer running maximum m, are rounded to E4M3 with one
 * power-of-two scale per 32 keys, E = floor(block max of t - m) - 7 with
 * t = scale * q.k * log2(e), and the denominator is summed from those same
 * rounded weights.
 *   q8, k8   E4M3 codes [B, H*, N, d]  (one byte per element)
 *   qs, ks   E8M0 scales [B, H*, N, d/32] (block of 32 along d)
 *   vt8      E4M3 codes of V transposed [B, Hkv, d, N] (block of 32 along keys)
 *   vts      E8M0 scales [B, Hkv, d, N/32]
 *   o fp32 [B, Hq, N, d], lse fp32 [B, Hq, N]  (natural log)
 *   d = 128; N a multiple of 32 (else ATTN_EUNSUPPORTED); codes must not hold the NaN
 *   patterns 0x7F / 0xFF (the quantisers below never write them).  Options: tau,
 *   stats, the sliding window and the document offsets as for the bf16 forward; ALiBi
 *   and soft-capping are ATTN_EUNSUPPORTED.
 */
int attn_fwd_mxfp8(const uint8_t* q8, const uint8_t* qs, const uint8_t* k8, const uint8_t* ks,
                   const uint8_t* vt8, const uint8_t* vts, float* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale);

int attn_fwd_mxfp8_ex(const uint8_t* q8, const uint8_t* qs, const uint8_t* k8, const uint8_t* ks,
                      const uint8_t* vt8, const uint8_t* vts, float* o, float* lse,
                      int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                      const attn_opts* opts, void* stream);

/*
 * MXFP8 quantisation of fp32 inputs (OCP MX v1.0 rule for E4M3: shared exponent
 * floor(log2(amax)) - 8 per block of 32, clamped to [-127, 127]; elements rounded to
 * the nearest E4M3 value with ties to even, saturating at +-448; an all-zero block gets
 * exponent 0; a value that rounds to 0 is stored as +0).
 *
 * attn_quantize_mxfp8_rows: x fp32 [rows, cols] -> codes [rows, cols], scales [rows, cols/32].
 * attn_quantize_mxfp8_cols_t: x fp32 [batch, rows, cols] -> codes [batch, cols, rows],
 *   scales [batch, cols, rows/32] (blocks along rows, output transposed; used for V).
 * cols (resp. rows) must be a positive multiple of 32; codes 16-byte aligned.
 */
int attn_quantize_mxfp8_rows(const float* x, uint8_t* codes, uint8_t* scales,
                             long long rows, int cols, void* stream);
int attn_quantize_mxfp8_cols_t(const float* x, uint8_t* codes, uint8_t* scales,
                               int batch, int rows, int cols, void* stream);

/*
 * bf16 backward: the gradients of the bf16 forward (same masks, scale and GQA map), with
 * the probabilities rebuilt from the forward's saved LSE instead of a stored N x N matrix
 * ("FlashAttention-4发布：原生支持Blackwell…", section "从V1到V4", FlashAttention (2022)
 * entry: tiling plus recomputation; "Hardware-Aware FP4 FlashAttention-4", section
 * "2. Causal Backward Cuantizado": the forward saves the LSE for the backward).  With
 * s = scale q.k (masked: -inf) and P = exp(s - LSE):
 *     D = rowsum(dO * O),  dS = P * (dO V^T - D)
 *     dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO   (dK, dV summed over the query
 *                                                          heads that share a kv head)
 *   q bf16 [B, Hq, N, d]; k, v bf16 [B, Hkv, N, d]; o fp32 [B, Hq, N, d] and lse fp32
 *   [B, Hq, N] as written by attn_fwd on the same inputs; dout bf16 [B, Hq, N, d];
 *   dq fp32 [B, Hq, N, d], dk, dv fp32 [B, Hkv, N, d] (outputs, every element written);
 *   delta: caller-owned device workspace of B*Hq*N floats (overwritten; holds D afterwards).
 *   d in {64, 128} (else ATTN_EUNSUPPORTED); any N >= 1; causal in {0, 1}; scale finite.
 *   Two kernels are queued on `stream` (null: the null stream): dQ, which also writes D
 *   into the workspace, then dK / dV, which reads it; no atomics, so the results are
 *   deterministic.
 */
int attn_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, float* delta,
             int B, int Hq, int Hkv, int N, int d, int causal, float scale, void* stream);

/*
 * bf16 backward with the forward's options: opts->window, opts->doc_offsets / n_docs,
 * opts->alibi_slopes and opts->softcap (the same meaning, ranges and errors as for
 * attn_fwd_ex; pass the options the forward ran with).  A window at least N wide is no
 * window; the tiles wholly outside a block's band are skipped in both gradient kernels.
 * With the score modifications P is rebuilt from the modified score, and soft-capping
 * multiplies dS by its derivative 1 - tanh(s / C)^2 (the ALiBi bias does not depend on
 * q or k).  tau, exp_mode, poly_frac and stats are forward-only and ignored (still
 * validated).  opts NULL = attn_bwd.  The document offsets and slopes are read on
 * `stream` during the call.
 */
int attn_bwd_ex(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv, float* delta,
                int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                const attn_opts* opts, void* stream);

/*
 * The bf16 backward without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, meaning and errors as attn_bwd_ex, except that D (B*Hq*N
 * floats) goes to a static device array of the library, ATTN_NOALLOC_MAX_ROWS floats
 * (8 MiB) on each GPU, held until the process ends.  B*Hq*N > ATTN_NOALLOC_MAX_ROWS ->
 * ATTN_EUNSUPPORTED.  Nothing is allocated: not by the library, not through any other
 * library.  The array's device address is looked up once per device (on the first call
 * with that device current).  Every call overwrites all of D before reading it, so nothing
 * carries over between calls; but calls on one GPU share the array, so calls that overlap
 * in time on one GPU (other streams, other threads) race and must be serialised by the
 * caller.
 */
#define ATTN_NOALLOC_MAX_ROWS (1 << 21)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const float* o,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv,
                     int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     const attn_opts* opts, void* stream);

/* Static description of a status code; never NULL. */
const char* attn_strerror(int status);

/* The hipError_t value behind the last ATTN_EHIP returned on this thread (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
