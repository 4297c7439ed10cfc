// A consumer of libkda that uses only the C ABI (include/kda.h) and the HIP
// runtime: no Python, no torch.  It reads one problem from a file, runs
// kda_prefill_varlen (append-prefill from initial states) and then
// kda_decode_step on the final states, and writes the results to a file.
//
// Input file (little-endian): 8 int64 header words
//   N, total_T, H, D, C, dtype (0 bf16, 1 fp32), decode present (0/1),
//   and the output scale's float32 bits
// followed by the byte blocks, each exactly as the library takes it:
//   cu_seqlens int32 [N+1]; q, k [total_T, H, D] dtype; v [total_T, H, D]
//   dtype; g [total_T, H, D] fp32; beta [total_T, H] fp32;
//   initial_state [N, H, D, D] fp32; and, when decode is present,
//   dq, dk, dv [N, H, D] dtype, dg [N, H, D] fp32, dbeta [N, H] fp32.
// Output file: o [total_T, H, D] dtype, final_state [N, H, D, D] fp32, and,
// with decode, decode o [N, H, D] dtype and the state after it.
//
// usage: kda_from_c IN OUT      exit status 0 on success
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kda.h"

namespace {

#define HIP_OK(x)                                                        \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_)); \
      std::exit(2);                                                      \
    }                                                                    \
  } while (0)

bool read_exact(std::FILE* f, void* p, size_t n) {
  return n == 0 || std::fread(p, 1, n, f) == n;
}

// Reads n bytes from f into a new device buffer.
void* upload(std::FILE* f, size_t n) {
  std::vector<char> h(n);
  if (!read_exact(f, h.data(), n)) {
    std::fprintf(stderr, "input file too short\n");
    std::exit(2);
  }
  void* d = nullptr;
  HIP_OK(hipMalloc(&d, n > 0 ? n : 1));
  if (n) HIP_OK(hipMemcpy(d, h.data(), n, hipMemcpyHostToDevice));
  return d;
}

void download(std::FILE* f, const void* d, size_t n) {
  std::vector<char> h(n);
  if (n) HIP_OK(hipMemcpy(h.data(), d, n, hipMemcpyDeviceToHost));
  if (n && std::fwrite(h.data(), 1, n, f) != n) {
    std::fprintf(stderr, "cannot write the output file\n");
    std::exit(2);
  }
}

int check(const char* what, int32_t st) {
  if (st != KDA_OK) {
    std::fprintf(stderr, "%s: %s (%d)\n", what, kda_status_string(st), st);
    return 1;
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  std::FILE* in = std::fopen(argv[1], "rb");
  if (!in) {
    std::fprintf(stderr, "cannot open %s\n", argv[1]);
    return 2;
  }
  int64_t hdr[8];
  if (!read_exact(in, hdr, sizeof(hdr))) {
    std::fprintf(stderr, "input file too short\n");
    return 2;
  }
  const int32_t N = (int32_t)hdr[0], H = (int32_t)hdr[2], D = (int32_t)hdr[3];
  const int32_t C = (int32_t)hdr[4], dtype = (int32_t)hdr[5];
  const int64_t T = hdr[1];
  const bool decode = hdr[6] != 0;
  const uint32_t scale_bits = (uint32_t)hdr[7];
  float scale;
  std::memcpy(&scale, &scale_bits, 4);
  if (N <= 0 || T < 0 || H <= 0 || D <= 0 || (dtype != 0 && dtype != 1)) {
    std::fprintf(stderr, "bad header\n");
    return 2;
  }
  const size_t es = dtype == KDA_DTYPE_BF16 ? 2 : 4;
  const size_t tok = (size_t)T * H * D, st_n = (size_t)N * H * D * D;
  std::vector<int32_t> cu(N + 1);
  if (!read_exact(in, cu.data(), cu.size() * 4)) {
    std::fprintf(stderr, "input file too short\n");
    return 2;
  }
  int32_t maxlen = 0;
  for (int32_t n = 0; n < N; ++n)
    maxlen = cu[n + 1] - cu[n] > maxlen ? cu[n + 1] - cu[n] : maxlen;
  void* d_cu = nullptr;
  HIP_OK(hipMalloc(&d_cu, cu.size() * 4));
  HIP_OK(hipMemcpy(d_cu, cu.data(), cu.size() * 4, hipMemcpyHostToDevice));
  void* q = upload(in, tok * es);
  void* k = upload(in, tok * es);
  void* v = upload(in, tok * es);
  void* g = upload(in, tok * 4);
  void* beta = upload(in, (size_t)T * H * 4);
  void* state = upload(in, st_n * 4);
  void *dq = nullptr, *dk = nullptr, *dv = nullptr, *dg = nullptr,
       *dbeta = nullptr;
  const size_t dtok = (size_t)N * H * D;
  if (decode) {
    dq = upload(in, dtok * es);
    dk = upload(in, dtok * es);
    dv = upload(in, dtok * es);
    dg = upload(in, dtok * 4);
    dbeta = upload(in, (size_t)N * H * 4);
  }
  std::fclose(in);

  void *o = nullptr, *ws = nullptr, *od = nullptr;
  HIP_OK(hipMalloc(&o, tok * es > 0 ? tok * es : 1));
  const size_t ws_bytes = kda_prefill_workspace_size(N, T, H, D, D, C);
  if (ws_bytes == 0) {
    std::fprintf(stderr, "unsupported sizes\n");
    return 1;
  }
  HIP_OK(hipMalloc(&ws, ws_bytes));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  // final states written over the initial ones (the header allows it)
  int rc = check("kda_prefill_varlen",
                 kda_prefill_varlen(q, k, v, (const float*)g,
                                    (const float*)beta, (const int32_t*)d_cu,
                                    N, T, maxlen, (const float*)state,
                                    (float*)state, o, H, D, D, C,
                                    scale, dtype, ws,
                                    ws_bytes, stream));
  std::FILE* out = std::fopen(argv[2], "wb");
  if (!out) {
    std::fprintf(stderr, "cannot open %s\n", argv[2]);
    return 2;
  }
  HIP_OK(hipStreamSynchronize(stream));
  download(out, o, tok * es);
  download(out, state, st_n * 4);
  if (decode && rc == 0) {
    HIP_OK(hipMalloc(&od, dtok * es));
    rc |= check("kda_decode_step",
                kda_decode_step(dq, dk, dv, (const float*)dg,
                                (const float*)dbeta, (float*)state, od, N, H,
                                D, D, scale, dtype,
                                stream));
    HIP_OK(hipStreamSynchronize(stream));
    download(out, od, dtok * es);
    download(out, state, st_n * 4);
  }
  std::fclose(out);
  // an argument the library must reject, with nothing enqueued
  if (kda_decode_step(dq, dk, dv, (const float*)dg, (const float*)dbeta,
                      (float*)state, od, N, H, 40, 40, 1.f, dtype,
                      stream) != KDA_ERR_UNSUPPORTED) {
    std::fprintf(stderr, "an unsupported head dim was not rejected\n");
    rc = 1;
  }
  HIP_OK(hipStreamDestroy(stream));
  for (void* p : {d_cu, q, k, v, g, beta, state, dq, dk, dv, dg, dbeta, o,
                  ws, od})
    if (p) HIP_OK(hipFree(p));
  return rc;
}
