/* Host-only use of the C ABI from plain C: every call below carries an
 * argument the library must reject before touching the GPU, so this runs on
 * a machine without one.  Exit status 0 when every status matches. */
#include <stdio.h>
#include <stddef.h>
#include <stdint.h>

#include "specopd.h"

static int fails = 0;
#define EXPECT(call, want)                                                          \
  do {                                                                              \
    specopd_status got_ = (call);                                                   \
    if (got_ != (want)) {                                                           \
      fprintf(stderr, "%s:%d: %s -> %d (%s), want %d\n", __FILE__, __LINE__, #call, \
              (int)got_, specopd_status_string(got_), (int)(want));                 \
      ++fails;                                                                      \
    }                                                                               \
  } while (0)

int main(void) {
  void* fake = (void*)(uintptr_t)0x7f0000000000ull; /* aligned, never dereferenced */
  size_t bytes = 0;

  if (specopd_version() != SPECOPD_VERSION) {
    fprintf(stderr, "version %d != %d\n", specopd_version(), SPECOPD_VERSION);
    ++fails;
  }

  specopd_tree_attn_desc td = {1, 128, 4, 4, 8, 2, 128, SPECOPD_BF16, 10000.0f, 0.0f, 0u};
  EXPECT(specopd_tree_attn_workspace_size(&td, &bytes), SPECOPD_OK);
  if (bytes == 0) ++fails;
  td.D = 96;
  EXPECT(specopd_tree_attn_workspace_size(&td, &bytes), SPECOPD_ERR_UNSUPPORTED);
  td.D = 128;
  EXPECT(specopd_tree_attn_fwd(&td, fake, fake, fake, fake, fake, fake, fake, fake, NULL, fake,
                               1u << 30, NULL),
         SPECOPD_ERR_INVALID_ARGUMENT); /* null output */
  EXPECT(specopd_tree_attn_fwd(NULL, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                               1u << 30, NULL),
         SPECOPD_ERR_INVALID_ARGUMENT);

  specopd_e2etv_desc ed = {4, 7, 151936, SPECOPD_BF16, SPECOPD_F32, 0.0, 1.0f, 0u, 0, 0};
  EXPECT(specopd_e2etv_workspace_size(&ed, &bytes), SPECOPD_OK);
  {
    char* f = (char*)fake; /* distinct, aligned stand-ins: no argument aliases another */
    EXPECT(specopd_e2etv_fwd_bwd(&ed, f, f + 16, NULL, (const int32_t*)(f + 32), NULL, NULL,
                                 (double*)(f + 48), f + 64, NULL, 0, NULL),
           SPECOPD_ERR_WORKSPACE);
    /* a target-row index without a row count */
    EXPECT(specopd_e2etv_fwd_bwd(&ed, f, f + 16, (const int32_t*)(f + 96), (const int32_t*)(f + 32),
                                 NULL, NULL, (double*)(f + 48), f + 64, f + 128, 1u << 30, NULL),
           SPECOPD_ERR_INVALID_ARGUMENT);
  }
  ed.Wn = 65;
  EXPECT(specopd_e2etv_workspace_size(&ed, &bytes), SPECOPD_ERR_UNSUPPORTED);

  specopd_prefill_desc pd = {2, 300, 8, 2, 128, SPECOPD_BF16, 10000.0f, 0.0f, 0u};
  EXPECT(specopd_prefill_workspace_size(&pd, &bytes), SPECOPD_OK);
  EXPECT(specopd_prefill_fwd(&pd, fake, fake, fake, fake, fake, fake, fake, 1, NULL),
         SPECOPD_ERR_INVALID_ARGUMENT); /* cache_k aliases q */
  pd.Hq = 7;
  EXPECT(specopd_prefill_workspace_size(&pd, &bytes), SPECOPD_ERR_INVALID_ARGUMENT);

  EXPECT(specopd_kernel_time(3, NULL, NULL), SPECOPD_ERR_INVALID_ARGUMENT);
  EXPECT(specopd_kernel_time(8, NULL, NULL), SPECOPD_ERR_INVALID_ARGUMENT);

  specopd_qsa_desc qd = {1, 4096, 8, 10, 128, 64, 10000.0f, 0.0f, 0u};
  EXPECT(specopd_qsa_workspace_size(&qd, &bytes), SPECOPD_OK);
  EXPECT(specopd_qsa_select_fwd(&qd, fake, fake, fake, fake, (const float*)fake, (const int32_t*)fake,
                                (const int32_t*)fake, (const int32_t*)fake, NULL, (float*)fake, NULL,
                                fake, bytes, NULL),
         SPECOPD_ERR_INVALID_ARGUMENT); /* no selection output */
  EXPECT(specopd_qsa_trunk_groups_fwd(&qd, fake, (const float*)fake, fake, NULL),
         SPECOPD_ERR_INVALID_ARGUMENT); /* the cache aliases the raw keys */
  qd.Di = 96;
  EXPECT(specopd_qsa_workspace_size(&qd, &bytes), SPECOPD_ERR_UNSUPPORTED);

  specopd_lmhead_e2etv_desc ld = {64, 8, 151936, 4096, 4608, 0.0, 1.0f, 0u};
  EXPECT(specopd_lmhead_e2etv_workspace_size(&ld, &bytes), SPECOPD_OK);
  EXPECT(specopd_lmhead_e2etv_fwd_bwd(&ld, fake, fake, fake, fake, (const int32_t*)fake,
                                      (const int32_t*)fake, NULL, NULL, NULL, NULL, fake, bytes, NULL),
         SPECOPD_ERR_INVALID_ARGUMENT); /* no loss output */
  ld.H = 4100;
  EXPECT(specopd_lmhead_e2etv_workspace_size(&ld, &bytes), SPECOPD_ERR_UNSUPPORTED);

  if (fails) fprintf(stderr, "%d mismatches\n", fails);
  return fails ? 1 : 0;
}
