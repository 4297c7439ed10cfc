// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Per-(head, chunk slot) block of the prefill workspace, written by the
// chunk-prep kernel and read by the chunk-recurrence kernel.  All bf16
// except gamma:
//   W    [C][Dk]   (I + A)^-1 diag(beta) Khat
//   Qh   [C][Dk]   q * exp(a)
//   KbT  [Dk][C]   (k * exp(a_last - a))^T
//   UtT  [Dv][C]   ((I + A)^-1 diag(beta) v)^T
//   M    [C][C]    decayed Q K^T, lower triangle incl. diagonal, zero above
//   gamma[Dk] fp32 exp(a_last)
struct WsLayout {
  int C, Dk, Dv;
  size_t off_W, off_Qh, off_KbT, off_UtT, off_M, off_gamma, block_bytes;
  __host__ __device__ static WsLayout make(int C, int Dk, int Dv) {
    WsLayout l;
    l.C = C; l.Dk = Dk; l.Dv = Dv;
    size_t o = 0;
    l.off_W = o;     o += (size_t)C * Dk * 2;
    l.off_Qh = o;    o += (size_t)C * Dk * 2;
    l.off_KbT = o;   o += (size_t)Dk * C * 2;
    l.off_UtT = o;   o += (size_t)Dv * C * 2;
    l.off_M = o;     o += (size_t)C * C * 2;
    l.off_gamma = o; o += (size_t)Dk * 4;
    l.block_bytes = (o + 255) / 256 * 256;
    return l;
  }
};

// Number of chunk slots for N sequences of total_T tokens.  The chunk of
// sequence n that starts at packed token t0 uses slot t0 / C + n; these are
// distinct and below total_T / C + N.
inline int64_t num_slots(int32_t N, int64_t total_T, int32_t C) {
  return total_T / C + N;
}

struct PrefillArgs {
  const void* q; const void* k; const void* v;
  const float* g; const float* beta;
  const int32_t* cu_seqlens;   // device, or nullptr for fixed length
  int32_t T_fixed;             // fixed length when cu_seqlens == nullptr
  int32_t N;                   // sequences
  int64_t total_T;
  int32_t max_chunks;          // ceil(max_seqlen / C)
  const float* initial_state;
  float* final_state;
  void* o;
  int32_t H;
  float scale;
  char* ws;
  int64_t nslots;
};

struct DecodeArgs {
  const void* q; const void* k; const void* v;
  const float* g; const float* beta;
  float* state; void* o;
  int32_t B, H;
  float scale;
};

// Launch a kernel whose only parameter is `arg`; returns the launch status
// of this very launch (not an earlier, unrelated error).
template <typename Kern, typename Arg>
inline hipError_t launch_kernel(Kern kernel, dim3 grid, dim3 block,
                                hipStream_t s, const Arg& arg) {
  void* args[] = {const_cast<Arg*>(&arg)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                         args, 0, s);
}

// Return hipSuccess or the launch error.
hipError_t launch_decode(const DecodeArgs& a, int D, bool bf16_io,
                         hipStream_t s);
hipError_t launch_prep(const PrefillArgs& a, int D, int C, bool bf16_io,
                       hipStream_t s);
hipError_t launch_recur(const PrefillArgs& a, int D, int C, bool bf16_io,
                        hipStream_t s);

}  // namespace kda
