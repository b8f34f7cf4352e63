/* A plain C caller of libsrat through include/srat.h only (no Python, no
 * torch): it exercises the host-side entry points -- version, descriptor
 * validation, workspace queries and the recompute planner -- and prints
 * their results for the test that compares them with the oracle. */
#include <stdio.h>
#include <string.h>

#include "srat.h"

int main(void) {
  printf("version %d\n", srat_version());

  /* attention descriptor: b 1, s 2048, 12 heads of 128, causal, bf16 */
  srat_attn_desc a;
  memset(&a, 0, sizeof a);
  a.dtype = SRAT_BF16;
  a.causal = 1;
  a.b = 1; a.s = 2048; a.hq = 12; a.hkv = 12; a.d = 128;
  const int64_t row = a.hq * a.d, batch = a.s * row;
  int64_t st[3] = {batch, row, a.d};
  memcpy(a.q_stride, st, sizeof st); memcpy(a.k_stride, st, sizeof st);
  memcpy(a.v_stride, st, sizeof st); memcpy(a.o_stride, st, sizeof st);
  a.scale = 0.08838834764831845f;
  a.p_drop = 0.1f;
  size_t ws = 0;
  int rc = srat_attn_core_bwd_workspace(&a, &ws);
  printf("bwd_workspace rc %d bytes %zu\n", rc, ws);
  a.d = 48;
  rc = srat_attn_core_bwd_workspace(&a, &ws);
  printf("bad_head_dim rc %d msg %s\n", rc, srat_last_error());

  /* the Recomputing Activations plate's Llama 3 70B example */
  srat_layer_desc l;
  memset(&l, 0, sizeof l);
  l.s = 8192; l.b = 1; l.h = 8192; l.a = 64; l.layers = 80;
  l.n_params = 70000000000LL; l.t = 1; l.sequence_parallel = 0; l.causal = 1;
  const char* names[3] = {"none", "selective", "full"};
  for (int pol = SRAT_RECOMPUTE_NONE; pol <= SRAT_RECOMPUTE_FULL; ++pol) {
    double bytes = 0, extra = 0;
    rc = srat_activation_bytes(&l, pol, &bytes, &extra);
    printf("policy %s rc %d bytes_per_layer %.17g extra %.17g\n", names[pol], rc, bytes, extra);
  }
  const double budgets[4] = {2e12, 183e9, 100e9, 10.75e9};
  for (int i = 0; i < 4; ++i) {
    srat_recompute_plan p;
    rc = srat_plan_recompute(&l, budgets[i], &p);
    printf("plan %.17g rc %d none %lld selective %lld full %lld bytes %.17g extra %.17g\n", budgets[i], rc,
           (long long)p.layers_none, (long long)p.layers_selective, (long long)p.layers_full,
           p.activation_bytes, p.extra_compute);
  }
  srat_recompute_plan p;
  rc = srat_plan_recompute(&l, 10.7e9, &p);
  printf("too_small rc %d\n", rc);
  return 0;
}
