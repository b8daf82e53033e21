/* Host-side driver for the AddressSanitizer build of the C ABI (CPU only).
 *
 * Calls every entry point with arguments that its host-side checks reject
 * (null, misaligned or too-small buffers, shapes outside the domain), plus
 * the size queries, status strings and kernel-choice overrides, so that the
 * checks, the workspace arithmetic and the string tables run under ASan.
 * Nothing here reaches a kernel launch: every call must return before it
 * touches the GPU.  Exits 0 when every call returned the expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mova.h"

static int failures = 0;

static void expect(const char* what, long long got, long long want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

/* Aligned, non-null device-pointer stand-ins: the host code checks them but
 * never dereferences them. */
static void* const P = (void*)(uintptr_t)0x100000;
static void* const Q = (void*)(uintptr_t)0x200000;
static void* const MIS = (void*)(uintptr_t)0x100008; /* 8-byte aligned only */

int main(void) {
  const size_t bad = (size_t)-1;

  /* Version, status strings (every code and a few outside the range). */
  expect("version", mova_version() > 0, 1);
  for (int s = -16; s <= 16; ++s) {
    const char* str = mova_status_str(s);
    expect("status string", str != NULL && strlen(str) > 0, 1);
  }

  /* Workspace queries over valid and invalid shapes. */
  for (int T = 0; T <= 70000; T = T ? T * 3 + 1 : 1)
    for (int k = 1; k <= 8; ++k) {
      const size_t n = mova_workspace_bytes(T, 2560, 64, k, 8, 128);
      expect("workspace in domain", n != bad, 1);
      const size_t f = mova_ffn_workspace_bytes(T, 2560, 100, k, 768, 768);
      expect("ffn workspace in domain", f != bad, 1);
    }
  expect("workspace E > 64", mova_workspace_bytes(16, 2560, 65, 4, 8, 128) == bad, 1);
  expect("workspace k > 8", mova_workspace_bytes(16, 2560, 64, 9, 8, 128) == bad, 1);
  expect("workspace d % 64", mova_workspace_bytes(16, 2500, 64, 4, 8, 128) == bad, 1);
  expect("workspace N % 64", mova_workspace_bytes(16, 2560, 64, 4, 3, 20) == bad, 1);
  expect("workspace T < 0", mova_workspace_bytes(-1, 2560, 64, 4, 8, 128) == bad, 1);
  expect("dense workspace d % 64", mova_dense_workspace_bytes(16, 100, 8, 128) == bad, 1);
  expect("ffn workspace E > 128", mova_ffn_workspace_bytes(16, 2560, 129, 8, 768, 0) == bad, 1);

  /* Routing only. */
  int32_t* I = (int32_t*)Q;
  float* W = (float*)Q;
  expect("route T = 0", mova_route(NULL, NULL, NULL, 0, 2560, 64, 4, 2.5f, NULL, NULL, NULL), MOVA_OK);
  expect("route null x", mova_route(NULL, P, NULL, 16, 2560, 64, 4, 2.5f, I, W, NULL), MOVA_ERR_INVALID_ARG);
  expect("route E > 64", mova_route(P, P, NULL, 16, 2560, 65, 4, 2.5f, I, W, NULL), MOVA_ERR_UNSUPPORTED);
  expect("route misaligned", mova_route(MIS, P, NULL, 16, 2560, 64, 4, 2.5f, I, W, NULL),
         MOVA_ERR_INVALID_ARG);

  /* Value forward: null, misaligned, too-small workspace, bad shapes. */
  const size_t need = mova_workspace_bytes(64, 2560, 64, 4, 8, 128);
  expect("forward null x", mova_value_forward(NULL, P, NULL, P, 64, 2560, 64, 4, 2.5f, 8, 128, P, NULL,
                                              NULL, P, need, NULL), MOVA_ERR_INVALID_ARG);
  expect("forward misaligned out", mova_value_forward(P, P, NULL, P, 64, 2560, 64, 4, 2.5f, 8, 128, MIS,
                                                      NULL, NULL, P, need, NULL), MOVA_ERR_INVALID_ARG);
  expect("forward small workspace", mova_value_forward(P, P, NULL, P, 64, 2560, 64, 4, 2.5f, 8, 128, P,
                                                       NULL, NULL, P, need - 1, NULL), MOVA_ERR_WORKSPACE);
  expect("forward no workspace", mova_value_forward(P, P, NULL, P, 64, 2560, 64, 4, 2.5f, 8, 128, P, NULL,
                                                    NULL, NULL, need, NULL), MOVA_ERR_WORKSPACE);
  expect("forward k > E", mova_value_forward(P, P, NULL, P, 64, 2560, 2, 4, 2.5f, 8, 128, P, NULL, NULL,
                                             P, need, NULL), MOVA_ERR_UNSUPPORTED);
  expect("forward heads", mova_value_forward(P, P, NULL, P, 64, 2560, 64, 4, 2.5f, 0, 128, P, NULL, NULL,
                                             P, need, NULL), MOVA_ERR_INVALID_ARG);
  expect("forward T = 0", mova_value_forward(NULL, NULL, NULL, NULL, 0, 2560, 64, 4, 2.5f, 8, 128, NULL,
                                             NULL, NULL, NULL, 0, NULL), MOVA_OK);

  /* Paged store. */
  const int64_t* S = (const int64_t*)Q;
  expect("paged negative blocks", mova_value_forward_paged(P, P, NULL, P, 64, 2560, 64, 4, 2.5f, 8, 128, P,
                                                           -1, 16, S, NULL, NULL, NULL, P, need, NULL),
         MOVA_ERR_INVALID_ARG);
  expect("paged null slots", mova_value_forward_paged(P, P, NULL, P, 64, 2560, 64, 4, 2.5f, 8, 128, P, 16,
                                                      16, NULL, NULL, NULL, NULL, P, need, NULL),
         MOVA_ERR_INVALID_ARG);
  expect("paged small workspace", mova_value_forward_paged(P, P, NULL, P, 64, 2560, 64, 4, 2.5f, 8, 128, P,
                                                           16, 16, S, NULL, NULL, NULL, P, 16, NULL),
         MOVA_ERR_WORKSPACE);

  /* Rebuild from stored routing, records. */
  expect("from routing null ids", mova_value_from_routing(P, NULL, W, P, 64, 2560, 64, 4, 8, 128, P, P,
                                                          need, NULL), MOVA_ERR_INVALID_ARG);
  expect("from routing small workspace", mova_value_from_routing(P, I, W, P, 64, 2560, 64, 4, 8, 128, P, P,
                                                                 8, NULL), MOVA_ERR_WORKSPACE);
  uint32_t* R = (uint32_t*)Q;
  expect("record k > 5", mova_value_forward_record(P, P, NULL, P, 64, 2560, 64, 6, 2.5f, 8, 128, P, R, Q,
                                                   P, need, NULL), MOVA_ERR_UNSUPPORTED);
  expect("record null ids", mova_value_forward_record(P, P, NULL, P, 64, 2560, 64, 4, 2.5f, 8, 128, P, NULL,
                                                      Q, P, need, NULL), MOVA_ERR_INVALID_ARG);
  expect("from record null ids", mova_value_from_record(P, NULL, Q, P, 64, 2560, 64, 4, 8, 128, P, P, need,
                                                        NULL), MOVA_ERR_INVALID_ARG);

  /* The entry point that allocates nothing: shape errors and calls larger
   * than its scratch are refused before any device lookup. */
  expect("noalloc E > 64", mova_value_forward_noalloc(P, P, NULL, P, 16, 2560, 65, 4, 2.5f, 8, 128, P, NULL,
                                                      NULL, NULL), MOVA_ERR_UNSUPPORTED);
  expect("noalloc T < 0", mova_value_forward_noalloc(P, P, NULL, P, -1, 2560, 64, 4, 2.5f, 8, 128, P, NULL,
                                                     NULL, NULL), MOVA_ERR_INVALID_ARG);
  int big = 1;
  while (mova_workspace_bytes(big, 2560, 64, 4, 8, 128) <= (size_t)MOVA_NOALLOC_SCRATCH_BYTES) big *= 2;
  expect("noalloc beyond scratch", mova_value_forward_noalloc(P, P, NULL, P, big, 2560, 64, 4, 2.5f, 8, 128,
                                                              P, NULL, NULL, NULL), MOVA_ERR_SCRATCH);

  /* Dense projection and FFN. */
  expect("dense null x", mova_dense_value_proj(NULL, P, 64, 2560, 8, 128, P, P, 1 << 20, NULL),
         MOVA_ERR_INVALID_ARG);
  expect("dense d % 64", mova_dense_value_proj(P, P, 64, 2500, 8, 128, P, P, 1 << 20, NULL),
         MOVA_ERR_UNSUPPORTED);
  expect("ffn pack bad shape", mova_ffn_pack_gate_up(P, P, 100, 770, 2560, Q, NULL) < 0, 1);
  expect("ffn E > 128", mova_ffn_moe_forward(P, P, NULL, P, P, 129, 8, 768, NULL, NULL, 0, 64, 2560, 2.5f,
                                             P, NULL, NULL, P, 1 << 30, NULL), MOVA_ERR_UNSUPPORTED);
  expect("ffn null x", mova_ffn_moe_forward(NULL, P, NULL, P, P, 100, 8, 768, NULL, NULL, 0, 64, 2560, 2.5f,
                                            P, NULL, NULL, P, 1 << 30, NULL), MOVA_ERR_INVALID_ARG);

  /* Kernel-choice overrides: range checks and round trips. */
  for (int key = -2; key < MOVA_OVERRIDE_COUNT + 2; ++key) {
    const int in = key >= 0 && key < MOVA_OVERRIDE_COUNT;
    expect("override get", mova_debug_override_get(key), in ? 0 : -1);
    expect("override set 1", mova_debug_override(key, 1), in ? MOVA_OK : MOVA_ERR_INVALID_ARG);
    expect("override set 99", mova_debug_override(key, 99), MOVA_ERR_INVALID_ARG);
    if (in) {
      expect("override round trip", mova_debug_override_get(key), 1);
      expect("override reset", mova_debug_override(key, 0), MOVA_OK);
    }
  }

  if (failures == 0) printf("asan host driver: ok\n");
  return failures == 0 ? 0 : 1;
}
