// Host-side checks of the C ABI (config defaults, validation, workspace sizes,
// early rejections), built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code only; the device launchers are replaced by stubs, so no
// GPU is needed and no device code runs.
#include <math.h>
#include <stdio.h>
#include <string.h>
#include "sparsepr.h"
static int fails = 0;
#define EXPECT(c) do { if (!(c)) { ++fails; printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); } } while (0)
int main() {
  sparsepr_config c;
  const int Ns[] = {2, 7, 64, 100, 1000, 1024, 4097, 32760, 75600};
  for (int d : {64, 128}) {
    for (int N : Ns) {
      EXPECT(sparsepr_config_default(N, d, &c) == SPARSEPR_OK);
      EXPECT(sparsepr_validate(&c, 1, 2, N, d, SPARSEPR_BF16) == SPARSEPR_OK);
      for (int dt : {SPARSEPR_BF16, SPARSEPR_FP32})
        for (int B : {1, 2}) {
          size_t bytes = 0;
          EXPECT(sparsepr_workspace_size(&c, B, 3, N, d, dt, &bytes) == SPARSEPR_OK && bytes > 0);
        }
    }
  }
  EXPECT(sparsepr_config_default(1024, 96, &c) == SPARSEPR_ERR_INVALID_ARG);
  EXPECT(sparsepr_config_default(1, 64, &c) == SPARSEPR_ERR_INVALID_ARG);
  EXPECT(sparsepr_config_default(1024, 64, nullptr) == SPARSEPR_ERR_INVALID_ARG);
  // invalid settings, one at a time
  struct Bad { const char* what; void (*f)(sparsepr_config*); };
  const Bad bad[] = {
      {"density nan", [](sparsepr_config* x) { x->density = NAN; }},
      {"density 0", [](sparsepr_config* x) { x->density = 0.f; }},
      {"probes < 0", [](sparsepr_config* x) { x->probe_rows = -1; }},
      {"probes > N", [](sparsepr_config* x) { x->probe_rows = 5000; }},
      {"G_K 0", [](sparsepr_config* x) { x->n_kv_groups = 0; }},
      {"G_Q huge", [](sparsepr_config* x) { x->n_q_groups = 1 << 20; }},
      {"rank < 0", [](sparsepr_config* x) { x->residual_rank = -3; }},
      {"lambda inf", [](sparsepr_config* x) { x->ridge_lambda = INFINITY; }},
      {"iters 0", [](sparsepr_config* x) { x->kmeans_iters = 0; }},
      {"sample 0", [](sparsepr_config* x) { x->n_sample_q = 0; }},
      {"rK 0", [](sparsepr_config* x) { x->key_coord_rank = 0; }},
      {"scale < 0", [](sparsepr_config* x) { x->scale = -1.f; }},
      {"cut 1", [](sparsepr_config* x) { x->rank_cut = 1.f; }},
      {"mode 7", [](sparsepr_config* x) { x->partition_mode = 7; }},
      {"ridge mode 9", [](sparsepr_config* x) { x->ridge_mode = 9; }},
      {"router 5", [](sparsepr_config* x) { x->router = 5; }},
      {"alpha 0", [](sparsepr_config* x) { x->router = SPARSEPR_ROUTER_ALPHA; x->alpha = 0.f; }},
      {"rank cap 0", [](sparsepr_config* x) { x->rank_cap = 0.f; }},
      {"rank cap 1.5", [](sparsepr_config* x) { x->rank_cap = 1.5f; }},
      {"svd weighted 2", [](sparsepr_config* x) { x->svd_weighted = 2; }},
      {"centred -1", [](sparsepr_config* x) { x->centred_query_coords = -1; }},
  };
  for (const Bad& b : bad) {
    sparsepr_config x;
    sparsepr_config_default(4096, 128, &x);
    b.f(&x);
    size_t bytes = 0;
    const bool ok = sparsepr_validate(&x, 1, 2, 4096, 128, SPARSEPR_BF16) == SPARSEPR_ERR_INVALID_ARG &&
                    sparsepr_workspace_size(&x, 1, 2, 4096, 128, SPARSEPR_BF16, &bytes) == SPARSEPR_ERR_INVALID_ARG;
    if (!ok) printf("not rejected: %s\n", b.what);
    EXPECT(ok);
  }
  // shapes
  sparsepr_config_default(4096, 128, &c);
  EXPECT(sparsepr_validate(&c, 0, 2, 4096, 128, SPARSEPR_BF16) == SPARSEPR_ERR_INVALID_ARG);
  EXPECT(sparsepr_validate(&c, 1, 2, 4096, 80, SPARSEPR_BF16) != SPARSEPR_OK);
  EXPECT(sparsepr_validate(&c, 1, 2, 4096, 128, 7) != SPARSEPR_OK);
  // the allocation-free call rejects an oversized request before any device work
  sparsepr_tensors io;
  memset(&io, 0, sizeof(io));
  io.B = 1; io.H = 40; io.N = 75600; io.d = 128; io.dtype = SPARSEPR_BF16;
  const long long st[4] = {40LL * 75600 * 128, 75600LL * 128, 128, 1};
  memcpy(io.q_strides, st, sizeof(st)); memcpy(io.k_strides, st, sizeof(st));
  memcpy(io.v_strides, st, sizeof(st)); memcpy(io.o_strides, st, sizeof(st));
  io.q = io.k = io.v = (const void*)0x1000; io.o = (void*)0x2000;
  sparsepr_config_default(75600, 128, &c);
  EXPECT(sparsepr_attention_noalloc(&c, &io, nullptr, nullptr) == SPARSEPR_ERR_WORKSPACE);
  EXPECT(sparsepr_attention(&c, nullptr, nullptr, 0, nullptr, nullptr) == SPARSEPR_ERR_INVALID_ARG);
  EXPECT(strlen(sparsepr_status_string(SPARSEPR_ERR_HIP)) > 0);
  printf("host checks done, %d failures\n", fails);
  return fails ? 1 : 0;
}
