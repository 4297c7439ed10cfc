// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Per-(head, chunk slot) block of the prefill workspace, written by the
// chunk-prep kernel and read by the chunk-recurrence kernel.  Every matrix is
// stored fragment-major: the 16x32 bf16 MFMA operand fragment that a wave
// reads with one 16-byte load per lane is 1 KB, stored contiguously in lane
// order (lane l = row%16 + 16*((col%32)/8) holds row, cols 8*(l/16)..+7 of
// its 32-column group), so each load instruction of the recurrence reads one
// contiguous kilobyte.
//   W    fragments (m, kk)  : rows of (I + A)^-1 diag(beta) Khat       [C x Dk]
//   Qh   fragments (m, kk)  : q * exp(a)                              [C x Dk]
//   KbT  fragments (ct, cs) : (k * exp(a_last - a))^T                 [Dk x C]
//   M    fragments (m, cs)  : decayed Q K^T, lower incl. diag, 0 above [C x C];
//                             only fragments with 2 cs <= m are written (the
//                             others are entirely above the diagonal, zero,
//                             and never read)
//   UtT  fragments (jt, m)  : ((I + A)^-1 diag(beta) v)^T, 8 bytes per lane
//                             (row j = 16jt + l%16, cols 16m + 4(l/16)..+3)
//   gamma[Dk] fp32          : exp(a_last)
// m / ct / jt index 16-row tiles, kk / cs 32-column groups.  Fragment slots
// of lanes past Dk or C (only when Dk or C is 16) are never read.
struct WsLayout {
  int C, Dk, Dv, kst, cst, mt;
  size_t off_W, off_Qh, off_KbT, off_UtT, off_M, off_gamma, block_bytes;
  __host__ __device__ static WsLayout make(int C, int Dk, int Dv) {
    WsLayout l;
    l.C = C; l.Dk = Dk; l.Dv = Dv;
    l.kst = (Dk + 31) / 32;
    l.cst = (C + 31) / 32;
    l.mt = C / 16;
    size_t o = 0;
    l.off_W = o;     o += (size_t)l.mt * l.kst * 1024;
    l.off_Qh = o;    o += (size_t)l.mt * l.kst * 1024;
    l.off_KbT = o;   o += (size_t)(Dk / 16) * l.cst * 1024;
    l.off_UtT = o;   o += (size_t)(Dv / 16) * l.mt * 512;
    l.off_M = o;     o += (size_t)l.mt * l.cst * 1024;
    l.off_gamma = o; o += (size_t)Dk * 4;
    l.block_bytes = (o + 255) / 256 * 256;
    return l;
  }
  // bf16 element offset of (row, col) inside a 16x32-fragment-major matrix
  // whose column groups per 16-row tile number `groups`.
  __host__ __device__ static size_t frag16(int row, int col, int groups) {
    const int f = (row >> 4) * groups + (col >> 5);
    const int lane = (row & 15) + 16 * ((col & 31) >> 3);
    return ((size_t)f * 64 + lane) * 8 + (col & 7);
  }
  // bf16 element offset of U~^T (j, r) for the 8-byte-per-lane fragments.
  __host__ __device__ static size_t frag_ut(int j, int r, int mt) {
    const int f = (j >> 4) * mt + (r >> 4);
    const int lane = (j & 15) + 16 * ((r & 15) >> 2);
    return ((size_t)f * 64 + lane) * 4 + (r & 3);
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
  // head dims as stored (multiples of 16, at most the kernels' tile D):
  // rows of q, k, g and of the state hold dk channels, rows of v, o and the
  // state's columns dv; channels past them are zero inside the kernels
  int32_t dk, dv;
  float scale;
  char* ws;
  int64_t nslots;
  float* ckpt_states;          // state checkpoints, or nullptr
  // Where the checkpoints fall.  Interval mode (ckpt_pos == nullptr): every
  // ckpt_every tokens of each sequence (a multiple of C).  List mode: the
  // positions ckpt_pos[cu_ckpt[n] .. cu_ckpt[n+1]-1] (device int32) of
  // sequence n, checkpoint j going to slot j of ckpt_states [n_ckpt, ...].
  int32_t ckpt_every;
  const int32_t* ckpt_pos;
  const int32_t* cu_ckpt;
  int32_t n_ckpt;
  // Input prologue fused into the chunk-prep kernel when conv_w != nullptr:
  // q, k, v then hold the short convolutions' inputs, g the decay gate's
  // pre-activation a (g = -5 sigmoid(a)) and beta the pre-activation b
  // (beta = sigmoid(b)); conv_w is [3, H, D, 4] fp32 (taps of q, k, v).
  const float* conv_w;
  // Output epilogue fused into the recurrence when gate_z != nullptr: the
  // outputs are written as y = o * rsqrt(mean(o^2) + gate_eps) * gate_w *
  // sigmoid(gate_z) per (token, head) row; gate_z [total_T, H, Dv] in the
  // storage dtype, gate_w [Dv] fp32.
  const void* gate_z;
  const float* gate_w;
  float gate_eps;
  // States kept in a pool (state_idx != nullptr): sequence n's initial and
  // final states are row state_idx[n] of initial_state / final_state, both
  // [pool_slots, H, dk, dv].  A slot outside [0, pool_slots) marks padding
  // (zero start, no state read or written); has_initial[n] == 0, when
  // has_initial is given, starts sequence n from zero.
  const int32_t* state_idx;
  const int32_t* has_initial;
  int32_t pool_slots;
};

struct SpecArgs {
  const void* q; const void* k; const void* v;   // [B, T, H, D]
  const float* g; const float* beta;             // [B, T, H, D], [B, T, H]
  float* state;                                  // [B, H, D, D]
  void* o;                                       // [B, T, H, D] (verify)
  float* u;                                      // [B, T, H, D] fp32
  const int32_t* accepted;                       // [B] (commit)
  int32_t B, T, H;
  int32_t dk, dv;                                // head dims as stored
  float scale;
  // previous draft, committed before the verify (step): its k, g and u
  // [B, T_prev, H, D] and accepted counts [B]; T_prev = 0 when none
  const void* k_prev; const float* g_prev; const float* u_prev;
  const int32_t* accepted_prev;
  int32_t T_prev;
  // state pool (state_idx != nullptr): sequence b's state is row
  // state_idx[b] of `state` [pool_slots, H, dk, dv]; a slot outside
  // [0, pool_slots) is padding (zero state, nothing read or written)
  const int32_t* state_idx;
  int32_t pool_slots;
};

enum class SpecMode { kVerify, kCommit, kStep };

struct DecodeArgs {
  const void* q; const void* k; const void* v;
  const float* g; const float* beta;
  float* state; void* o;
  int32_t B, H;
  int32_t dk, dv;                                // head dims as stored
  float scale;
  // output epilogue fused into the decode step (when z != nullptr): o is
  // replaced by o * rsqrt(mean(o^2) + eps) * w * sigmoid(z)
  const void* z; const float* w; float eps;
  // state pool (state_idx != nullptr): sequence b's state is row
  // state_idx[b] of `state` [pool_slots, H, dk, dv]; a slot outside
  // [0, pool_slots) is padding (zero start, nothing read or written)
  const int32_t* state_idx;
  int32_t pool_slots;
};

struct EpilogueArgs {
  const void* o; const void* z; const float* w; void* y;
  int64_t rows;                // tokens * heads
  int32_t dv;                  // channels of a row as stored
  float eps;
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

// Compute units of the current device (queried once per device).
int device_cus();

// Return hipSuccess or the launch error.
hipError_t launch_decode(const DecodeArgs& a, int D, bool bf16_io,
                         hipStream_t s);
hipError_t launch_prep(const PrefillArgs& a, int D, int C, bool bf16_io,
                       hipStream_t s);
hipError_t launch_recur(const PrefillArgs& a, int D, int C, bool bf16_io,
                        hipStream_t s);
hipError_t launch_spec(const SpecArgs& a, int D, bool bf16_io, SpecMode mode,
                       hipStream_t s);
int max_spec_tokens();
hipError_t launch_epilogue(const EpilogueArgs& a, int D, bool bf16_io,
                           hipStream_t s);

}  // namespace kda
