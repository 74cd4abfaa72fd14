// Host-side driver of the library's validation layer, built with AddressSanitizer
// on the host code only.  It calls every entry point declared in rmm.h with
// arguments the validation rejects (so no kernel is launched), queries every
// workspace size over a range of shapes, and answers k_from_rho queries read
// from stdin ("rho_as_hex_bits d" per line -> "k" per line).  Any heap or
// stack misuse in the host code aborts the process with an ASan report.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rmm.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(call);                                                       \
    if (got_ != (want)) {                                                               \
      fprintf(stderr, "line %d: %s returned %d, want %d (%s)\n", __LINE__, #call, got_, \
              (want), rmm_last_error());                                                \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main(int argc, char **argv) {
  void *F = (void *)0x10000;   // never dereferenced: every call below is rejected first
  float *Ff = (float *)F;
  int32_t *Fi = (int32_t *)F;
  const int INV = RMM_ERR_INVALID_ARG, UNS = RMM_ERR_UNSUPPORTED, WSE = RMM_ERR_WORKSPACE;

  EXPECT(rmm_version() >= 100, 1);
  for (int s = -1; s < 8; ++s) EXPECT(strlen(rmm_status_string(s)) > 0, 1);
  EXPECT(rmm_k_from_rho(0.5, 10, NULL), INV);
  EXPECT(rmm_k_from_rho(0.0, 10, (int64_t *)F), INV);
  EXPECT(rmm_k_pad(0), 0);
  EXPECT(rmm_k_pad(65), 128);

  // column norms, top-k, products
  EXPECT(rmm_colnorm(RMM_BF16, NULL, 4, 4, 4, 1, 0, Ff, NULL, 0, NULL), INV);
  EXPECT(rmm_colnorm(RMM_BF16, F, 4, 8, 4, 1, 0, Ff, NULL, 0, NULL), INV);
  EXPECT(rmm_colnorm((rmm_dtype_t)7, F, 4, 8, 8, 1, 0, Ff, NULL, 0, NULL), INV);
  EXPECT(rmm_colnorm(RMM_BF16, F, 65536, 4096, 4096, 1, 0, Ff, F,
                     rmm_colnorm_workspace_bytes(RMM_BF16, 65536, 4096, 1) - 1, NULL), WSE);
  EXPECT(rmm_topk(Ff, 1, 10, 11, Fi, NULL, 0, NULL), INV);
  EXPECT(rmm_topk(Ff, 70000, 10, 5, Fi, NULL, 0, NULL), INV);
  EXPECT(rmm_gemm(RMM_BF16, F, 64, F, 32, Fi, 16, 64, 32, 65, F, 32, F, 1 << 30, NULL), INV);
  EXPECT(rmm_gemm(RMM_BF16, F, 64, F, 32, Fi, 16, 64, 32, 8, F, 32, F,
                  rmm_gemm_workspace_bytes(RMM_BF16, 16, 32, 8) - 1, NULL), WSE);
  EXPECT(rmm_gemm_scored(RMM_BF16, F, 64, F, 32, Fi, 16, 64, 32, 8, F, 32, NULL, F, 1 << 30, NULL), INV);
  EXPECT(rmm_gemm_scored(RMM_BF16, F, 64, F, 32, Fi, 16, 64, 32, 8, F, 32, Ff, F,
                         rmm_gemm_scored_workspace_bytes(RMM_BF16, 16, 32, 8) - 1, NULL), WSE);
  EXPECT(rmm_gemm_noalloc(RMM_BF16, F, 4096, F, 28672, Fi, 16384, 4096, 28672, 3277, F, 28672, NULL), UNS);
  EXPECT(rmm_gemm_noalloc(RMM_BF16, F, 64, F, 32, Fi, 16, 64, 32, 65, F, 32, NULL), INV);
  EXPECT(rmm_gemm_w8(F, 64, F, 40, Ff, Fi, 16, 64, 32, 8, F, 32, F, 1 << 30, NULL), UNS);
  EXPECT(rmm_gemm_w8(F, 64, F, 32, NULL, Fi, 16, 64, 32, 8, F, 32, F, 1 << 30, NULL), INV);
  EXPECT(rmm_swiglu_scored(F, 64, F, 64, 100, 60, F, 64, Ff, F, 1 << 30, NULL), UNS);
  EXPECT(rmm_swiglu_scored(F, 63, F, 64, 100, 64, F, 64, Ff, F, 1 << 30, NULL), INV);
  EXPECT(rmm_rmsnorm_scored(F, 1024, F, -1.f, 100, 1024, F, 1024, Ff, F, 1 << 30, NULL), INV);
  EXPECT(rmm_rmsnorm_scored(F, 1000, F, 1e-5f, 100, 1000, F, 1000, Ff, F, 1 << 30, NULL), UNS);

  // attention
  EXPECT(rmm_qk(F, 64, 6, 128, 768, 128, F, 64, 4, 8192, 64, 32, 0, Ff, 4096, 64, Fi, NULL, F, 1 << 30, NULL), INV);
  EXPECT(rmm_qk(F, 64, 4, 128, 512, 128, F, 64, 2, (int64_t)128 << 25, (int64_t)1 << 25, 64, 1, Ff, 4096, 64,
                Fi, NULL, F, 1 << 30, NULL), UNS);
  EXPECT(rmm_qk(F, 64, 4, 128, 512, 128, F, 64, 2, 8192, 64, 64, 0, Ff, 4096, 64, Fi, NULL, F,
                rmm_qk_workspace_bytes(64, 4, 128, 64) - 1, NULL), WSE);
  EXPECT(rmm_pv(F, 4, 64, 64, 4096, 64, F, 2, 128, 256, 128, 65, 0, F, 512, 128, Fi, NULL, F, 1 << 30, NULL), INV);
  EXPECT(rmm_pv(F, 4, 64, 64, (int64_t)64 << 24, (int64_t)1 << 24, F, 2, 128, 256, 128, 32, 1, F, 512, 128, Fi,
                NULL, F, 1 << 30, NULL), UNS);
  EXPECT(rmm_attention(F, 64, 4, 64, 256, 64, F, 64, 2, 4096, 64, F, 128, 64, 32, 32, 1, F, 256, 64, Fi, Fi,
                       NULL, NULL, F, 1 << 30, NULL), UNS);
  EXPECT(rmm_attention(F, 65, 4, 128, 512, 128, F, 64, 2, 8192, 64, F, 256, 128, 32, 32, 1, F, 512, 128, Fi, Fi,
                       NULL, NULL, F, 1 << 30, NULL), INV);
  EXPECT(rmm_attention_decode_batch(F, 1024, 128, F, 256000, 128000, 1000, F, 256000, 256, 128, Fi, Fi, 9000, 8,
                                    2, 128, 1000, 64, 500, F, 1024, 128, Fi, Fi, NULL, F, 1 << 30, NULL), INV);
  EXPECT(rmm_attention_decode_batch(F, 1024, 128, F, 256000, 128000, 1000, F, 256000, 252, 128, Fi, Fi, 4, 8,
                                    2, 128, 1000, 64, 500, F, 1024, 128, Fi, Fi, NULL, F, 1 << 30, NULL), UNS);

  // workspace queries over a spread of shapes (host arithmetic only)
  size_t acc = 0;
  for (int64_t m = 1; m <= (1 << 16); m *= 4)
    for (int64_t d = 1; d <= (1 << 15); d *= 8)
      for (int64_t b = 1; b <= 64; b *= 8) {
        acc += rmm_colnorm_workspace_bytes(RMM_BF16, m, d, b) + rmm_colnorm_workspace_bytes(RMM_F32, m, d, b);
        acc += rmm_gemm_workspace_bytes(RMM_BF16, m, d, d) + rmm_gemm_w8_workspace_bytes(m, d, d);
        acc += rmm_gemm_scored_workspace_bytes(RMM_BF16, m, d, d) + rmm_gemm_scored_workspace_bytes(RMM_F32, m, d, d);
        acc += rmm_qk_workspace_bytes(m, b, 128, 64) + rmm_pv_workspace_bytes(b, m, d, d);
        acc += rmm_attention_workspace_bytes(m, m, b, 128, 64, m) + rmm_swiglu_scored_workspace_bytes(m, d);
        acc += rmm_attention_decode_batch_workspace_bytes(b, 8, 128, d, d) + rmm_rmsnorm_scored_workspace_bytes(m, 512);
      }
  EXPECT(acc > 0, 1);

  // timing registry: host bookkeeping only while nothing is recorded
  EXPECT(rmm_timing_set_tag("asan/driver"), RMM_OK);
  EXPECT(rmm_timing_set_tag(NULL), RMM_OK);
  EXPECT(rmm_timing_reset(), RMM_OK);
  EXPECT(rmm_timing_count(), 0);

  // k_from_rho queries from stdin
  if (argc > 1 && strcmp(argv[1], "k") == 0) {
    char hex[64];
    long long d;
    while (scanf("%63s %lld", hex, &d) == 2) {
      const uint64_t bits = strtoull(hex, NULL, 16);
      double rho;
      memcpy(&rho, &bits, sizeof(rho));
      int64_t k = -1;
      const rmm_status_t st = rmm_k_from_rho(rho, (int64_t)d, &k);
      printf("%lld\n", st == RMM_OK ? (long long)k : -(long long)st);
    }
  }
  fprintf(stderr, "abi_driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
