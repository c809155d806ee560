/* Host-side sanitizer run of libattn's C ABI: every entry point's argument checks, the
 * option defaults and the status strings, with the host code built under AddressSanitizer
 * and UndefinedBehaviorSanitizer.  No kernel is launched and no device is needed: every
 * call here is rejected before the library touches the device.  Prints "ok" and exits 0
 * when every call returns the documented status. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attn.h"

static int failures = 0;
#define EXPECT(call, want)                                                      \
  do {                                                                          \
    int got_ = (call);                                                          \
    if (got_ != (want)) {                                                       \
      fprintf(stderr, "%s:%d: %s returned %d, want %d\n", __FILE__, __LINE__, #call, \
              got_, (want));                                                    \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

int main(void) {
  /* 16-byte aligned, never dereferenced: every call below fails validation first */
  void* p = (void*)(uintptr_t)4096;
  float* f = (float*)p;
  const uint8_t* u = (const uint8_t*)p;
  attn_opts o;
  memset(&o, 0x5A, sizeof o);
  attn_default_opts(&o);
  attn_default_opts(NULL);
  if (o.tau != 8.0f || o.exp_mode != ATTN_EXP_HW || o.stats || o.window || o.alibi_slopes ||
      o.softcap != 0.0f || o.doc_offsets || o.n_docs) {
    fprintf(stderr, "attn_default_opts left a field unset\n");
    ++failures;
  }
  /* bf16 forward */
  EXPECT(attn_fwd(NULL, p, p, f, f, 1, 2, 1, 16, 64, 0, 0.1f), ATTN_EINVAL);
  EXPECT(attn_fwd(p, p, p, f, f, 0, 2, 1, 16, 64, 0, 0.1f), ATTN_EINVAL);
  EXPECT(attn_fwd(p, p, p, f, f, 1, 6, 4, 16, 64, 0, 0.1f), ATTN_EINVAL);
  EXPECT(attn_fwd(p, p, p, f, f, 1, 2, 1, 16, 64, 2, 0.1f), ATTN_EINVAL);
  EXPECT(attn_fwd(p, p, p, f, f, 1, 2, 1, 16, 96, 0, 0.1f), ATTN_EUNSUPPORTED);
  EXPECT(attn_fwd(p, p, p, f, f, 1 << 16, 1 << 10, 1, 1 << 10, 64, 0, 0.1f), ATTN_EUNSUPPORTED);
  attn_opts bad = o;
  bad.tau = 65.0f;
  EXPECT(attn_fwd_ex(p, p, p, f, f, 1, 2, 1, 16, 64, 0, 0.1f, &bad, NULL), ATTN_EINVAL);
  bad = o;
  bad.exp_mode = 7;
  EXPECT(attn_fwd_ex(p, p, p, f, f, 1, 2, 1, 16, 64, 0, 0.1f, &bad, NULL), ATTN_EINVAL);
  bad = o;
  bad.doc_offsets = (const int*)p;
  bad.n_docs = 17;
  EXPECT(attn_fwd_ex(p, p, p, f, f, 1, 2, 1, 16, 64, 0, 0.1f, &bad, NULL), ATTN_EINVAL);
  bad = o;
  bad.softcap = 2.0f;
  bad.exp_mode = ATTN_EXP_POLY;
  EXPECT(attn_fwd_ex(p, p, p, f, f, 1, 2, 1, 16, 64, 0, 0.1f, &bad, NULL), ATTN_EUNSUPPORTED);
  /* block-scaled forwards */
  EXPECT(attn_fwd_mxfp4(u, u, u, u, u, NULL, f, f, 1, 1, 1, 64, 128, 0, 0.1f), ATTN_EINVAL);
  EXPECT(attn_fwd_mxfp4(u, u, u, u, u, u, f, f, 1, 1, 1, 48, 128, 0, 0.1f), ATTN_EUNSUPPORTED);
  bad = o;
  bad.window = -8;
  EXPECT(attn_fwd_mxfp4_ex(u, u, u, u, u, u, f, f, 1, 1, 1, 64, 128, 0, 0.1f, &bad, NULL),
         ATTN_EINVAL);
  bad = o;
  bad.softcap = 2.0f;
  EXPECT(attn_fwd_mxfp4_ex(u, u, u, u, u, u, f, f, 1, 1, 1, 64, 128, 0, 0.1f, &bad, NULL),
         ATTN_EUNSUPPORTED);
  EXPECT(attn_fwd_mxfp8(u, u, u, u, u, u, f, f, 1, 1, 1, 64, 64, 0, 0.1f), ATTN_EUNSUPPORTED);
  EXPECT(attn_fwd_mxfp8_ex(u, u, u, u, u, u, f, f, 1, 3, 2, 64, 128, 0, 0.1f, &o, NULL),
         ATTN_EINVAL);
  /* quantisers */
  EXPECT(attn_quantize_mxfp4_rows(f, (uint8_t*)p, (uint8_t*)p, 4, 48, NULL), ATTN_EINVAL);
  EXPECT(attn_quantize_mxfp4_cols_t(f, (uint8_t*)p, (uint8_t*)p, 1, 40, 8, NULL), ATTN_EINVAL);
  EXPECT(attn_quantize_mxfp8_rows(NULL, (uint8_t*)p, (uint8_t*)p, 4, 64, NULL), ATTN_EINVAL);
  EXPECT(attn_quantize_mxfp8_cols_t(f, (uint8_t*)p, (uint8_t*)p, 0, 64, 8, NULL), ATTN_EINVAL);
  /* backward, with and without a workspace */
  EXPECT(attn_bwd(p, p, p, f, f, p, f, f, f, NULL, 1, 2, 1, 16, 64, 0, 0.1f, NULL), ATTN_EINVAL);
  EXPECT(attn_bwd(p, p, p, f, f, p, f, f, f, f, 1, 2, 1, 16, 96, 0, 0.1f, NULL),
         ATTN_EUNSUPPORTED);
  bad = o;
  bad.window = -3;
  EXPECT(attn_bwd_ex(p, p, p, f, f, p, f, f, f, f, 1, 2, 1, 16, 64, 0, 0.1f, &bad, NULL),
         ATTN_EINVAL);
  EXPECT(attn_bwd_noalloc(p, p, p, f, f, NULL, f, f, f, 1, 2, 1, 16, 64, 0, 0.1f, NULL, NULL),
         ATTN_EINVAL);
  EXPECT(attn_bwd_noalloc(p, p, p, f, f, p, f, f, f, 64, 64, 8, 1024, 128, 0, 0.1f, NULL, NULL),
         ATTN_EUNSUPPORTED);
  /* status strings */
  for (int s = -5; s <= 1; ++s)
    if (attn_strerror(s) == NULL || strlen(attn_strerror(s)) == 0) ++failures;
  if (attn_last_hip_error() != 0) ++failures;
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
