/* Calls every entry point of include/iha.h with arguments the host-side validation must
 * reject, and checks the status codes.  Each call returns before any device work, so this
 * runs without a GPU; built with the host code of the library under AddressSanitizer and
 * UndefinedBehaviorSanitizer. */
#include <stdio.h>
#include <string.h>

#include "iha.h"

static int failures = 0;

static void expect(iha_status got, iha_status want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL: %s: got %s, want %s\n", what, iha_status_str(got), iha_status_str(want));
    ++failures;
  }
}

int main(void) {
  iha_problem p;
  memset(&p, 0, sizeof(p));
  p.B = 2; p.N = 100; p.D = 256; p.H = 2; p.P = 2; p.mask = IHA_MASK_WINDOW; p.window = 25;
  p.dtype = IHA_BF16;
  size_t ws = 0;
  uint32_t plan = 0;
  expect(iha_workspace_bytes(&p, &ws), IHA_OK, "workspace of a valid problem");
  if (ws == 0) { fprintf(stderr, "FAIL: zero workspace\n"); ++failures; }
  expect(iha_plan(&p, &plan), IHA_OK, "plan of a valid problem");
  expect(iha_workspace_bytes(NULL, &ws), IHA_ERR_INVALID_ARG, "null problem");
  expect(iha_workspace_bytes(&p, NULL), IHA_ERR_INVALID_ARG, "null size");
  iha_problem q = p;
  q.D = 255; expect(iha_workspace_bytes(&q, &ws), IHA_ERR_SHAPE, "D not a multiple of H");
  q = p; q.window = 0; expect(iha_workspace_bytes(&q, &ws), IHA_ERR_EMPTY_ROW, "window 0");
  q = p; q.H = 1; q.D = 96; expect(iha_workspace_bytes(&q, &ws), IHA_ERR_UNSUPPORTED, "d = 96");
  q = p; q.N = 0; expect(iha_workspace_bytes(&q, &ws), IHA_ERR_INVALID_ARG, "N = 0");
  q = p; q.flags = 0x80; expect(iha_workspace_bytes(&q, &ws), IHA_ERR_INVALID_ARG, "unknown flag");
  q = p; q.reserved = 1; expect(iha_workspace_bytes(&q, &ws), IHA_ERR_INVALID_ARG, "reserved field");
  q = p; q.flags = IHA_FLAG_FUSED_COLLAPSE; expect(iha_workspace_bytes(&q, &ws), IHA_OK, "fused collapse flag");
  q.dtype = IHA_F32; q.D = 64; q.H = 4;
  expect(iha_workspace_bytes(&q, &ws), IHA_ERR_UNSUPPORTED, "fused collapse with fp32 inputs");
  q = p; q.mask = 3; expect(iha_plan(&q, &plan), IHA_ERR_INVALID_ARG, "unknown mask");
  q = p; q.dtype = 5; expect(iha_plan(&q, &plan), IHA_ERR_INVALID_ARG, "unknown dtype");
  q = p; q.B = (int64_t)1 << 40; expect(iha_plan(&q, &plan), IHA_ERR_SHAPE, "too many tokens");

  /* Fake but 256-byte aligned addresses: validation must return before dereferencing them. */
  char* fake = (char*)(uintptr_t)0x100000;
  const float* af = (const float*)fake;
  expect(iha_forward(&p, NULL, fake, fake, fake, af, af, af, af, (float*)fake, fake, ws, NULL),
         IHA_ERR_INVALID_ARG, "null X");
  expect(iha_forward(&p, fake + 2, fake, fake, fake, af, af, af, af, (float*)fake, fake, ws, NULL),
         IHA_ERR_INVALID_ARG, "misaligned X");
  expect(iha_forward(&p, fake, fake, fake, fake, af, af, af, af, (float*)fake, fake, ws - 1, NULL),
         IHA_ERR_WORKSPACE, "short workspace");
  expect(iha_forward(&p, fake, fake, fake, fake, af, af, af, af, (float*)fake, fake + 16, ws, NULL),
         IHA_ERR_WORKSPACE, "misaligned workspace");
  q = p; q.window = -3;
  expect(iha_forward(&q, fake, fake, fake, fake, af, af, af, af, (float*)fake, fake, ws, NULL),
         IHA_ERR_EMPTY_ROW, "negative window");
  expect(iha_forward_timed(&p, fake, fake, fake, fake, af, af, af, af, (float*)fake, fake, ws, NULL, NULL),
         IHA_ERR_INVALID_ARG, "timed without events");

  expect(iha_attention(1, 64, 2, 96, IHA_MASK_CAUSAL, 0, 0.1f, fake, fake, fake, (float*)fake, 0, NULL, NULL),
         IHA_ERR_UNSUPPORTED, "attention d = 96");
  expect(iha_attention(1, 64, 2, 128, IHA_MASK_WINDOW, 0, 0.1f, fake, fake, fake, (float*)fake, 0, NULL, NULL),
         IHA_ERR_EMPTY_ROW, "attention window 0");
  expect(iha_attention(1, 64, 2, 128, IHA_MASK_CAUSAL, 0, -1.f, fake, fake, fake, (float*)fake, 0, NULL, NULL),
         IHA_ERR_INVALID_ARG, "attention negative scale");
  expect(iha_attention(1, 64, 2, 128, IHA_MASK_CAUSAL, 0, 0.1f, fake, fake, fake, (float*)fake,
                       IHA_FLAG_CHECK, NULL, NULL),
         IHA_ERR_WORKSPACE, "attention check without a flag buffer");

  size_t bws = 0;
  expect(iha_attention_backward_workspace(1, 64, 2, 128, &bws), IHA_OK, "backward workspace");
  expect(iha_attention_backward_workspace(1, 64, 2, 128, NULL), IHA_ERR_INVALID_ARG, "backward null size");
  expect(iha_attention_backward(1, 64, 2, 128, IHA_MASK_CAUSAL, 0, 0.1f, fake, fake, fake, fake,
                                (float*)fake, (float*)fake, (float*)fake, fake, bws - 1, NULL),
         IHA_ERR_WORKSPACE, "backward short workspace");
  expect(iha_attention_backward(1, 64, 2, 64, IHA_MASK_WINDOW, 0, 0.1f, fake, fake, fake, fake,
                                (float*)fake, (float*)fake, (float*)fake, fake, bws, NULL),
         IHA_ERR_EMPTY_ROW, "backward window 0");
  size_t nws = 0;
  expect(iha_nexus_inner_workspace(1, 64, 2, 128, &nws), IHA_OK, "nexus workspace");
  expect(iha_nexus_inner_workspace(1, 64, 2, 96, &nws), IHA_ERR_UNSUPPORTED, "nexus d = 96");
  expect(iha_nexus_inner(1, 64, 2, 128, IHA_MASK_WINDOW, 0, 0.1f, fake, (float*)fake, 0, fake, nws, NULL),
         IHA_ERR_EMPTY_ROW, "nexus window 0");
  expect(iha_nexus_inner(1, 64, 2, 128, IHA_MASK_CAUSAL, 0, 0.1f, fake, (float*)fake, 0, fake, nws - 1, NULL),
         IHA_ERR_WORKSPACE, "nexus short workspace");
  expect(iha_nexus_inner(1, 64, 2, 128, IHA_MASK_CAUSAL, 0, 0.1f, fake + 8, (float*)fake, 0, fake, nws, NULL),
         IHA_ERR_INVALID_ARG, "nexus misaligned Q");
  size_t lws = 0;
  float* ff = (float*)fake;
  expect(iha_backward_workspace(&p, &lws), IHA_OK, "layer backward workspace");
  q = p; q.dtype = IHA_F32;
  expect(iha_backward_workspace(&q, &lws), IHA_ERR_UNSUPPORTED, "layer backward fp32");
  expect(iha_backward(&p, fake, fake, fake, fake, af, af, af, af, af, ff, ff, ff, ff, ff, ff, ff, ff, fake,
                      lws - 1, NULL),
         IHA_ERR_WORKSPACE, "layer backward short workspace");
  expect(iha_backward(&p, fake, fake, fake, fake, af, af, af, af, NULL, ff, ff, ff, ff, ff, ff, ff, ff, fake,
                      lws, NULL),
         IHA_ERR_INVALID_ARG, "layer backward null G");
  expect(iha_backward(&p, fake, fake, fake, fake, af, af, af, af, af, ff, ff, ff, ff, ff, ff, ff, ff + 2, fake,
                      lws, NULL),
         IHA_ERR_INVALID_ARG, "layer backward misaligned dR");
  for (int s = 0; s <= 8; ++s)
    if (!iha_status_str((iha_status)s) || !strncmp(iha_status_str((iha_status)s), "IHA_ERR_UNKNOWN", 15)) {
      fprintf(stderr, "FAIL: no name for status %d\n", s);
      ++failures;
    }
  printf("abi driver: %s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
