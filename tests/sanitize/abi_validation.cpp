// Host-side driver for the sanitizer build of libkda's validation layer:
// calls every entry point of include/kda.h with invalid arguments (bad
// sizes, NULL or misaligned pointers, short workspaces, unsupported shapes),
// so that each call returns a status before any HIP call, and checks the
// statuses.  Built with AddressSanitizer and UndefinedBehaviorSanitizer on
// the host code only, without device code; it never launches a kernel.
#include <stdint.h>
#include <stdio.h>

#include "kda.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  char* const P = reinterpret_cast<char*>(0x100000);   // 256-aligned fake
  char* const MIS = reinterpret_cast<char*>(0x100002); // misaligned
  float* const F = reinterpret_cast<float*>(P);
  const int32_t* const I = reinterpret_cast<const int32_t*>(P);
  const size_t big = (size_t)1 << 40;

  expect("version", kda_abi_version(), KDA_ABI_VERSION);
  for (int s = -6; s <= 1; ++s)
    if (!kda_status_string(s)) ++failures;
  expect("ws size bad N", (int)kda_prefill_workspace_size(0, 10, 1, 128, 128, 64), 0);
  expect("ws size bad C", (int)kda_prefill_workspace_size(1, 10, 1, 128, 128, 48), 0);
  if (kda_prefill_workspace_size(1, 8192, 96, 128, 128, 64) == 0) ++failures;

  // fixed-length prefill
  expect("chunked B=0", kda_prefill_chunked(P, P, P, F, F, nullptr, nullptr, P, 0, 128, 2, 128, 128, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("chunked C=48", kda_prefill_chunked(P, P, P, F, F, nullptr, nullptr, P, 1, 128, 2, 128, 128, 48, 1.f, 0, P, big, nullptr), KDA_ERR_UNSUPPORTED);
  expect("chunked dtype", kda_prefill_chunked(P, P, P, F, F, nullptr, nullptr, P, 1, 128, 2, 128, 128, 64, 1.f, 3, P, big, nullptr), KDA_ERR_UNSUPPORTED);
  expect("chunked q NULL", kda_prefill_chunked(nullptr, P, P, F, F, nullptr, nullptr, P, 1, 128, 2, 128, 128, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("chunked k misaligned", kda_prefill_chunked(P, MIS, P, F, F, nullptr, nullptr, P, 1, 128, 2, 128, 128, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("chunked ws small", kda_prefill_chunked(P, P, P, F, F, nullptr, nullptr, P, 1, 128, 2, 128, 128, 64, 1.f, 0, P, 1000, nullptr), KDA_ERR_WORKSPACE);

  // varlen and its forms
  expect("varlen N=0", kda_prefill_varlen(P, P, P, F, F, I, 0, 100, 64, nullptr, nullptr, P, 2, 64, 64, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("varlen cu NULL", kda_prefill_varlen(P, P, P, F, F, nullptr, 2, 100, 64, nullptr, nullptr, P, 2, 64, 64, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("varlen maxlen 0", kda_prefill_varlen(P, P, P, F, F, I, 2, 100, 0, nullptr, nullptr, P, 2, 64, 64, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("varlen ws small", kda_prefill_varlen(P, P, P, F, F, I, 2, 100, 64, nullptr, nullptr, P, 2, 64, 64, 64, 1.f, 0, P, 10, nullptr), KDA_ERR_WORKSPACE);
  expect("prep q NULL", kda_prefill_varlen_prep(nullptr, P, P, F, F, I, 2, 300, 200, 2, 64, 64, 32, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("recur o NULL", kda_prefill_varlen_recur(I, 2, 300, 200, nullptr, nullptr, nullptr, 2, 64, 64, 32, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("ckpt every 48", kda_prefill_varlen_ckpt(P, P, P, F, F, I, 2, 300, 200, nullptr, nullptr, P, 2, 64, 64, 32, 1.f, 0, 48, F, big, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("ckpt buffer small", kda_prefill_varlen_ckpt(P, P, P, F, F, I, 2, 300, 200, nullptr, nullptr, P, 2, 64, 64, 32, 1.f, 0, 64, F, 131071, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("ckpt_at n<0", kda_prefill_varlen_ckpt_at(P, P, P, F, F, I, 2, 300, 200, nullptr, nullptr, P, 2, 64, 64, 32, 1.f, 0, I, I, -1, F, big, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("ckpt_at pos NULL", kda_prefill_varlen_ckpt_at(P, P, P, F, F, I, 2, 300, 200, nullptr, nullptr, P, 2, 64, 64, 32, 1.f, 0, nullptr, I, 3, F, big, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("gated z NULL", kda_prefill_varlen_gated(P, P, P, F, F, I, 2, 100, 64, nullptr, nullptr, nullptr, F, 1e-6f, P, 2, 64, 64, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("gated eps<0", kda_prefill_varlen_gated(P, P, P, F, F, I, 2, 100, 64, nullptr, nullptr, P, F, -1.f, P, 2, 64, 64, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);
  expect("noalloc too big", kda_prefill_varlen_noalloc(P, P, P, F, F, I, 1, 8192, 8192, nullptr, nullptr, P, 96, 128, 128, 64, 1.f, 0, nullptr), KDA_ERR_SCRATCH);
  expect("noalloc C=8", kda_prefill_varlen_noalloc(P, P, P, F, F, I, 2, 100, 64, nullptr, nullptr, P, 2, 64, 64, 8, 1.f, 0, nullptr), KDA_ERR_UNSUPPORTED);
  expect("prologue w NULL", kda_prefill_varlen_prologue(P, P, P, nullptr, F, F, I, 2, 100, 64, nullptr, nullptr, P, 2, 64, 64, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);

  // decode, epilogue, speculative verify and commit
  expect("decode B=0", kda_decode_step(P, P, P, F, F, F, P, 0, 2, 128, 128, 1.f, 0, nullptr), KDA_ERR_INVALID_ARG);
  expect("decode state NULL", kda_decode_step(P, P, P, F, F, nullptr, P, 2, 2, 128, 128, 1.f, 0, nullptr), KDA_ERR_INVALID_ARG);
  expect("decode gated z NULL", kda_decode_step_gated(P, P, P, F, F, F, nullptr, F, 1e-6f, P, 2, 2, 128, 128, 1.f, 0, nullptr), KDA_ERR_INVALID_ARG);
  expect("epilogue tokens<0", kda_output_norm_gate(P, P, F, 1e-6f, P, -1, 2, 128, 0, nullptr), KDA_ERR_INVALID_ARG);
  expect("epilogue tokens=0", kda_output_norm_gate(P, P, F, 1e-6f, P, 0, 2, 128, 0, nullptr), KDA_OK);
  expect("verify T=17", kda_spec_verify(P, P, P, F, F, F, P, F, 2, 17, 2, 128, 128, 1.f, 0, nullptr), KDA_ERR_UNSUPPORTED);
  expect("commit acc NULL", kda_spec_commit(P, F, F, nullptr, F, 2, 4, 2, 128, 128, 0, nullptr), KDA_ERR_INVALID_ARG);
  expect("step k_prev NULL", kda_spec_step(nullptr, F, F, I, 4, P, P, P, F, F, F, P, F, 2, 4, 2, 128, 128, 1.f, 0, nullptr), KDA_ERR_INVALID_ARG);
  expect("step T_prev=17", kda_spec_step(P, F, F, I, 17, P, P, P, F, F, F, P, F, 2, 4, 2, 128, 128, 1.f, 0, nullptr), KDA_ERR_UNSUPPORTED);
  expect("decode pool idx NULL", kda_decode_step_indexed(P, P, P, F, F, F, nullptr, 4, P, 2, 2, 128, 128, 1.f, 0, nullptr), KDA_ERR_INVALID_ARG);
  expect("prefill pool slots 0", kda_prefill_varlen_indexed(P, P, P, F, F, I, 2, 100, 64, F, I, nullptr, 0, P, 2, 128, 128, 64, 1.f, 0, P, big, nullptr), KDA_ERR_INVALID_ARG);

  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("sanitized validation layer: all statuses as expected\n");
  return 0;
}
