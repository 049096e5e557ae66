/* A plain C caller of libmoedecode: only the header and the shared library,
 * no Python and no device.  It checks that the declared entry points link and
 * that the host-side validation answers as the header states (every call here
 * fails validation or is pure host arithmetic, so nothing touches a GPU).
 * Built and run by tests/test_capi_host.py; prints "ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_decode.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__);    \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main(void) {
  moe_dims d;
  memset(&d, 0, sizeof d);
  d.hidden = 2560;
  d.n_experts = 512;
  d.top_k = 8;
  d.inter = 768;
  d.n_shared = 1;
  size_t bytes = 0;
  CHECK(moe_workspace_size(&d, 1, 1, &bytes) == MOE_OK && bytes > 0);
  size_t b16 = 0;
  CHECK(moe_workspace_size(&d, MOE_MAX_ROWS, 16, &b16) == MOE_OK && b16 > bytes);
  CHECK(moe_workspace_size(&d, MOE_MAX_ROWS + 1, 1, &bytes) == MOE_E_UNSUPPORTED);
  CHECK(moe_workspace_size(NULL, 1, 1, &bytes) == MOE_E_ARG);
  d.expert_format = MOE_EXPERT_FP8_B128;
  d.inter = 192;  /* not a whole number of 128-blocks */
  CHECK(moe_workspace_size(&d, 1, 1, &bytes) == MOE_E_UNSUPPORTED);
  d.inter = 768;
  CHECK(moe_workspace_size(&d, 1, 1, &bytes) == MOE_OK);
  d.expert_format = MOE_EXPERT_BF16;

  /* validation before any device work: null pointers, sizes, alignment, workspace */
  void* A = (void*)(uintptr_t)(1u << 20);       /* never dereferenced */
  void* BAD = (void*)((uintptr_t)(1u << 20) + 2);
  const size_t big = (size_t)1 << 30;
  int32_t* ip = (int32_t*)A;
  float* fp = (float*)A;
  const uint16_t* hp = (const uint16_t*)A;
  CHECK(moe_router_topk(&d, 0, hp, hp, NULL, ip, fp, NULL, A, big, NULL) == MOE_E_ARG);
  CHECK(moe_router_topk(&d, 1, NULL, hp, NULL, ip, fp, NULL, A, big, NULL) == MOE_E_ARG);
  CHECK(moe_router_topk(&d, 1, (const uint16_t*)BAD, hp, NULL, ip, fp, NULL, A, big, NULL) ==
        MOE_E_ALIGN);
  CHECK(moe_router_topk(&d, 1, hp, hp, NULL, ip, fp, NULL, A, 4096, NULL) == MOE_E_WORKSPACE);
  moe_layer_weights w;
  memset(&w, 0, sizeof w);
  w.w_router = hp;
  w.w_gate_up = A;
  w.w_down = A;
  CHECK(moe_experts_fused(&d, 1, hp, ip, fp, &w, A, 2, A, big, NULL) == MOE_E_ARG);
  CHECK(moe_layer_chain(&d, 1, 2, &w, hp, A, MOE_OUT_BF16, MOE_CHAIN_LAYER_ONLY, NULL, NULL, A,
                        big, NULL) == MOE_E_UNSUPPORTED);
  CHECK(lmhead_argmax(1, 2560, 0, hp, hp, ip, NULL, A, big, NULL) == MOE_E_ARG);
  CHECK(moe_expert_prefetch(&d, &w, ip, -1, NULL) == MOE_E_ARG);
  CHECK(moe_expert_prefetch(&d, &w, NULL, 0, NULL) == MOE_OK);
  CHECK(strcmp(moe_status_str(MOE_E_TIMEOUT), "device wait passed its deadline") == 0);
  printf("ok\n");
  return 0;
}
