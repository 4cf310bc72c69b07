/* Host-side paths of the C ABI (include/mk.h) that need no GPU: argument
 * checks, status strings, the two-wave rule, and a workspace / schedule
 * creation that fails at its first HIP call when no GPU is present (its
 * clean-up path).  Built with the host code under AddressSanitizer and
 * LeakSanitizer (tests/test_host_asan.py); exits 0 when every call returns
 * what the header states. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mk.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main(void) {
  mk_config cfg;
  mk_config_default(&cfg);
  expect(cfg.minibatch_rows, 0, "default minibatch_rows");
  expect(cfg.precision, MK_BF16, "default precision");
  expect((int)(cfg.ring_bytes >> 20), 256, "default ring MiB");

  mk_workspace* ws = (mk_workspace*)0x1;
  expect(mk_workspace_create(NULL, 1024, 256, 128, 8, 2, &ws), MK_ERR_NULL, "create: NULL config");
  expect(mk_workspace_create(&cfg, 1024, 256, 128, 8, 2, NULL), MK_ERR_NULL, "create: NULL out");
  expect(mk_workspace_create(&cfg, 1024, 100, 128, 8, 2, &ws), MK_ERR_SHAPE, "create: H not a multiple of 256");
  expect(ws == NULL, 1, "create: *out cleared on error");
  expect(mk_workspace_create(&cfg, 0, 256, 128, 8, 2, &ws), MK_ERR_SHAPE, "create: no rows");
  expect(mk_workspace_create(&cfg, 1024, 256, 128, 0, 2, &ws), MK_ERR_LIMIT, "create: no experts");
  expect(mk_workspace_create(&cfg, 1024, 256, 128, 8, 33, &ws), MK_ERR_LIMIT, "create: k above 32");
  mk_config bad = cfg;
  bad.precision = 7;
  expect(mk_workspace_create(&bad, 1024, 256, 128, 8, 2, &ws), MK_ERR_CONFIG, "create: precision");
  bad = cfg;
  bad.ring_bytes = (int64_t)1 << 31;
  expect(mk_workspace_create(&bad, 1024, 256, 128, 8, 2, &ws), MK_ERR_LIMIT, "create: ring of 2 GiB");
  bad = cfg;
  bad.fused_forward = 1;
  bad.precision = MK_MXFP8;
  expect(mk_workspace_create(&bad, 1024, 256, 256, 8, 2, &ws), MK_ERR_CONFIG, "create: fused MXFP8");
  bad = cfg;
  bad.minibatch_rows = 8;
  expect(mk_workspace_create(&bad, 8 * 65536, 256, 128, 8, 2, &ws), MK_ERR_LIMIT, "create: minibatch count");

  /* a valid request: MK_ERR_HIP without a GPU (the partly built workspace is
   * released), MK_OK with one */
  int rc = mk_workspace_create(&cfg, 1024, 256, 128, 8, 2, &ws);
  if (rc == MK_OK) {
    mk_schedule* sc = NULL;
    expect(mk_schedule_create(ws, &sc), MK_OK, "schedule create");
    expect(mk_schedule_destroy(sc), MK_OK, "schedule destroy");
    expect(mk_workspace_destroy(ws), MK_OK, "workspace destroy");
  } else {
    expect(rc, MK_ERR_HIP, "create without a GPU");
    expect(ws == NULL, 1, "create without a GPU: *out");
  }

  mk_schedule* sc = (mk_schedule*)0x1;
  expect(mk_schedule_create(NULL, &sc), MK_ERR_NULL, "schedule create: NULL workspace");
  expect(mk_forward(NULL, NULL, MK_FULL_LAYER, NULL, NULL, NULL, NULL, NULL, NULL), MK_ERR_NULL, "forward: NULL");
  expect(mk_backward(NULL, NULL, MK_FULL_LAYER, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
         MK_ERR_NULL, "backward: NULL");
  expect(mk_timing_enable(NULL, 1), MK_ERR_NULL, "timing enable: NULL");
  expect(mk_timing_phases(NULL, 0u), MK_ERR_NULL, "timing phases: NULL");
  expect(mk_debug_fused_waits(NULL, 0, 0), MK_ERR_NULL, "debug waits: NULL");
  expect(mk_mxfp8_quantize(NULL, 4, 48, NULL, NULL, NULL) != MK_OK, 1, "quantize: bad K or NULL");
  expect(mk_build_schedule_static(NULL, 16, 0, 16, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
         MK_ERR_LIMIT, "static schedule: no experts");
  expect(mk_build_schedule_static(NULL, -1, 8, 16, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
         MK_ERR_SHAPE, "static schedule: negative rows");

  expect(mk_two_wave_rows(7168, 2048, 256, 256, 256) == 8192, 1, "two-wave rule at H=7168, I=2048");
  const int codes[] = {MK_OK, MK_ERR_NULL, MK_ERR_SHAPE, MK_ERR_RING, MK_ERR_LIMIT, MK_ERR_HIP, MK_ERR_STATE,
                       MK_ERR_UNSUPPORTED, MK_ERR_CONFIG, 12345};
  for (size_t i = 0; i < sizeof(codes) / sizeof(codes[0]); ++i) {
    const char* s = mk_status_string(codes[i]);
    if (!s || !strlen(s)) {
      fprintf(stderr, "status string of %d empty\n", codes[i]);
      ++failures;
    }
  }
  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("host checks ok\n");
  return failures ? 1 : 0;
}
