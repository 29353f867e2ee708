/* A plain C client of the library's public headers: it compiles with a C compiler
 * against include/ alone, links against libgqa_decode.so, and exercises the calls that
 * need no GPU -- options, the plans, workspace sizes, status strings and the host-side
 * argument checks. Prints one line per check; exits non-zero on the first mismatch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gqa_decode.h"
#include "gqla_absorb.h"

#define CHECK(cond, what)                              \
  do {                                                 \
    if (!(cond)) {                                     \
      fprintf(stderr, "c_client: FAILED %s\n", what);  \
      return 1;                                        \
    }                                                  \
    printf("ok %s\n", what);                           \
  } while (0)

int main(void) {
  gqa_decode_opts o;
  gqa_decode_opts_init(&o);
  CHECK(o.struct_size == sizeof(gqa_decode_opts), "opts_init sets struct_size");
  CHECK(gqa_abi_version() == GQA_ABI_VERSION, "abi version");

  /* a contiguous bf16 cache of 4096 tokens; B=16, H=32, G=8, d_h=128, q_len=1 */
  o.cache_capacity = 4096;
  o.num_splits = 100; /* a fixed workgroup count keeps the plan device-independent */
  gqa_plan plan;
  memset(&plan, 0, sizeof(plan));
  CHECK(gqa_decode_plan(16, 32, 8, 128, 1, &o, &plan) == GQA_OK, "plan");
  CHECK(plan.policy == GQA_POLICY_MFMA && plan.schedule == 1 && plan.rows == 4, "plan: matrix cores, persistent");
  CHECK(plan.workgroups == 100 && plan.workspace_bytes > 0, "plan: workgroups and workspace");
  size_t ws = 0;
  CHECK(gqa_decode_workspace_size(16, 32, 8, 128, 1, &o, &ws) == GQA_OK && ws == plan.workspace_bytes,
        "workspace size agrees with the plan");

  /* argument errors come back before any HIP call: fake aligned pointers are never used */
  const void* P = (const void*)(uintptr_t)4096;
  int32_t* report = (int32_t*)(uintptr_t)4096;
  CHECK(gqa_decode(P, P, P, (const int32_t*)P, NULL, (void*)P, 16, 32, 3, 128, 1, 0.1f, NULL, &o) ==
            GQA_ERR_INVALID_ARGUMENT,
        "H % G != 0 is rejected");
  CHECK(gqa_decode(P, P, P, (const int32_t*)P, NULL, (void*)P, 16, 32, 8, 96, 1, 0.1f, NULL, &o) ==
            GQA_ERR_UNSUPPORTED,
        "d_h 96 is unsupported");
  CHECK(gqa_decode(P, P, P, (const int32_t*)P, NULL, (void*)P, 16, 32, 8, 128, 1, 0.1f, NULL, &o) ==
            GQA_ERR_WORKSPACE,
        "a missing workspace is reported");
  CHECK(gqa_decode_check_inputs(NULL, NULL, 16, 1, NULL, &o, report) == GQA_ERR_INVALID_ARGUMENT,
        "check_inputs needs seq_lens");
  CHECK(gqla_absorb_decode_append(P, NULL, P, P, (void*)P, (const int32_t*)P, NULL, (void*)P, 2, 16, 2, 128, 512,
                                  1, 0.1f, NULL, &o) == GQA_ERR_INVALID_ARGUMENT,
        "the latent append needs c_new");
  CHECK(strlen(gqa_status_string(GQA_ERR_WORKSPACE)) > 0, "status strings");
  return 0;
}
