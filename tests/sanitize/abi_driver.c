/* Host-side paths of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer: parameter derivation, sizes, the state
 * layout, status strings and the argument checks every entry makes before
 * touching a device (no GPU is used: every call here returns before its
 * first HIP call). Exits 0 when every result is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "still.h"

static int fails = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

static still_params base(void) {
  still_params p;
  memset(&p, 0, sizeof(p));
  p.abi_version = STILL_ABI_VERSION;
  p.dtype = STILL_DTYPE_BF16;
  p.batch = 2;
  p.n_q_heads = 8;
  p.n_kv_heads = 2;
  p.head_dim = 128;
  p.window = 64;
  p.chunk = 64;
  p.budget = 512;
  p.t_max = 64;
  return p;
}

int main(void) {
  /* sizes over a grid of valid shapes, and their consistency */
  const int dims[2] = {64, 128}, chunks[4] = {16, 32, 64, 128}, groups[4] = {1, 2, 4, 8};
  const int windows[4] = {1, 17, 128, 256};
  for (int a = 0; a < 2; ++a)
    for (int c = 0; c < 4; ++c)
      for (int g = 0; g < 4; ++g)
        for (int w = 0; w < 4; ++w) {
          still_params p = base();
          p.head_dim = dims[a];
          p.chunk = chunks[c];
          p.n_q_heads = 2 * groups[g];
          p.window = windows[w];
          p.budget = windows[w] + 3 * chunks[c];
          p.t_max = 5;
          const int lam = still_lambda(&p);
          EXPECT(lam == (3 * chunks[c]) / 5);
          const int64_t sb = still_state_bytes(&p);
          still_state_layout L;
          EXPECT(still_state_layout_get(&p, &L) == STILL_OK);
          EXPECT(sb == L.unit_bytes * p.batch * p.n_kv_heads);
          EXPECT(L.S < L.z && L.z < L.pool_k && L.meta + 32 <= L.unit_bytes);
          for (int64_t n = 1; n <= 70000; n = n * 3 + 1) {
            const int64_t ws = still_workspace_bytes(&p, n);
            EXPECT(ws > 0);
            EXPECT(ws >= still_workspace_bytes(&p, n > 1 ? n - 1 : 1));
          }
          p.flags = STILL_FLAG_ROUTE(STILL_ROUTE_EXTERNAL) | STILL_FLAG_MERGE_SUM;
          EXPECT(still_lambda(&p) == lam);
        }
  /* invalid and unsupported parameters */
  still_params p = base();
  EXPECT(still_lambda(NULL) == STILL_EINVAL);
  p.abi_version = 99;
  EXPECT(still_lambda(&p) == STILL_EINVAL);
  p = base();
  p.n_q_heads = 6;
  EXPECT(still_state_bytes(&p) == STILL_EUNSUPPORTED);
  p = base();
  p.head_dim = 96;
  EXPECT(still_workspace_bytes(&p, 100) == STILL_EUNSUPPORTED);
  p = base();
  p.flags = STILL_FLAG_SOFTMAX_ONLY | STILL_FLAG_MERGE_SUM;
  EXPECT(still_lambda(&p) == STILL_EINVAL);
  p = base();
  p.flags = STILL_FLAG_ROUTE(9);
  EXPECT(still_lambda(&p) == STILL_EINVAL);
  p = base();
  p.budget = 10;
  EXPECT(still_lambda(&p) == STILL_EINVAL);
  /* argument checks before any launch (never dereferenced) */
  p = base();
  void* f = (void*)(uintptr_t)(1u << 20);
  float* ff = (float*)f;
  int32_t* fi = (int32_t*)f;
  const int64_t ws = still_workspace_bytes(&p, 1000);
  EXPECT(still_prefill(&p, 1000, NULL, f, f, f, ff, f, fi, ff, f, f, (size_t)ws, NULL) == STILL_EINVAL);
  EXPECT(still_prefill(&p, 0, f, f, f, f, ff, f, fi, ff, f, f, (size_t)ws, NULL) == STILL_EINVAL);
  EXPECT(still_prefill(&p, 1000, f, f, f, f, ff, f, fi, ff, f, f, (size_t)ws - 1, NULL) == STILL_EWORKSPACE);
  EXPECT(still_prefill(&p, 1000, (char*)f + 4, f, f, f, ff, f, fi, ff, f, f, (size_t)ws, NULL) == STILL_EINVAL);
  EXPECT(still_prefill_partials(&p, 1000, f, f, f, f, ff, f, fi, ff, f, f, (size_t)ws, NULL, ff, NULL, ff, ff) ==
         STILL_EINVAL);
  p.flags = STILL_FLAG_ROUTE(STILL_ROUTE_EXTERNAL);
  EXPECT(still_prefill(&p, 1000, f, f, f, f, ff, f, fi, NULL, f, f, (size_t)ws, NULL) == STILL_EINVAL);
  EXPECT(still_decode_step(&p, 1000, f, f, f, f, ff, f, f, fi, NULL, 0, NULL) == STILL_EUNSUPPORTED);
  p = base();
  EXPECT(still_decode_step(&p, 0, f, f, f, f, ff, f, f, fi, NULL, 0, NULL) == STILL_EINVAL);
  p.batch = 64;
  p.n_q_heads = 32;
  p.n_kv_heads = 8;
  EXPECT(still_prefill_noalloc(&p, 65536, f, f, f, f, ff, f, fi, ff, f, NULL) == STILL_ESCRATCH);
  EXPECT(still_noalloc_scratch_bytes() > 0);
  for (int rc = -8; rc <= 1; ++rc) EXPECT(still_status_str(rc) != NULL && strlen(still_status_str(rc)) > 0);
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  else printf("abi host paths: all checks passed\n");
  return fails ? 1 : 0;
}
