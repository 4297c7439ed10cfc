// Decode step: one token per sequence, the fp32 state read once and written
// once in place.
//
// Per (sequence, head), with alpha = exp(g) and the decayed state aS:
//   x = (aS)^T k,  y = (aS)^T q,  u = beta (v - x)
//   o = scale * (y + (q . k) u)          (= scale * S_new^T q)
//   S_new = aS + k u^T
// This is the per-token form of "Kimi K3: The Manos, The Mythos, The
// Legendos", section "FlashKDA algorithm" (decode follows the recurrence
// token by token); expanding S_new^T q lets the output come from the same
// single pass over the state.  Section "Complexity analysis" of that page:
// about 7 D^2 FLOPs and 8 D^2 bytes (fp32 state in and out) per head, so the
// kernel is bound by HBM bandwidth and uses no matrix cores.
//
// Mapping: one workgroup per (sequence, head).  Thread (rg, cg) owns the
// float4 column group cg of rows rg, rg + RG, rg + 2 RG, ...; a wave reads
// and writes whole contiguous rows (fully coalesced 16-byte accesses), the
// slice stays in registers between the reduction and the write-back.  The
// state is touched exactly once per step, so its loads and stores may carry
// the non-temporal cache policy (kNt) to keep it from displacing other data
// in the caches.

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

template <typename Tio, int D, int NT, bool kNt, bool kGated, bool kExact>
__global__ __launch_bounds__(NT, (NT >= 1024 && sizeof(Tio) == 2) ? 8 : 1)
void decode_kernel(DecodeArgs a) {
  constexpr int CG = D / 4;       // float4 column groups
  constexpr int RG = NT / CG;     // row groups
  constexpr int RPT = D / RG;     // rows per thread
  constexpr int NW = NT / 64;     // waves
  static_assert(NT % CG == 0 && D % RG == 0, "decode tiling");
  // a wave holds 64 / CG lanes of each column group (CG divides 32)
  static_assert(32 % CG == 0 && NT >= 64, "decode lane grouping");

  __shared__ float s_alpha[D], s_k[D], s_q[D];
  // cross-wave partial sums: with many waves, one thread per (component,
  // column group) sums the waves and every thread then reads 9 totals,
  // instead of every thread reading every wave's partials (16x the LDS
  // traffic at 16 waves)
  constexpr bool kTwoLevel = NW >= 8;
  __shared__ float4 s_red[kTwoLevel ? 1 : NW][CG][3];
  __shared__ float s_part[kTwoLevel ? NW : 1][9][CG];
  __shared__ float s_fin[kTwoLevel ? 9 : 1][CG];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  // the stored slice is dk x dv (<= D x D); rows past dk and column groups
  // past dv are zero here and never stored.  kExact: dk = dv = D, known at
  // compile time (constant strides, no masks)
  const int dk = kExact ? D : a.dk, dv = kExact ? D : a.dv;
  const bool col_ok = 4 * cg < dv;
  // the state slice: row bh of [B, H, dk, dv], or, with a state pool, row
  // (state_idx[b], h) of [pool_slots, H, dk, dv].  A padding entry (slot out
  // of range) gets an empty buffer: its state loads read 0 and its stores
  // are dropped, so it runs from a zero state and touches no state.
  size_t srow = bh;
  bool s_ok = true;
  if (a.state_idx) {
    const int32_t r = a.state_idx[bh / a.H];
    s_ok = r >= 0 && r < a.pool_slots;
    srow = s_ok ? (size_t)r * a.H + bh % a.H : 0;
  }
  float* S = a.state + srow * dk * dv;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(S, s_ok ? dk * dv * 4 : 0);
  constexpr int kPol = kNt ? kCachePolicyNt : 0;
  auto soff = [&](int c) {
    return (c < dk && col_ok) ? (uint32_t)((c * dv + 4 * cg) * 4) : kOffNone;
  };

  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(rs, soff(rg + RG * i),
                                                      0, kPol));

  const Tio* q = static_cast<const Tio*>(a.q) + (size_t)bh * dk;
  const Tio* k = static_cast<const Tio*>(a.k) + (size_t)bh * dk;
  if (tid < D) {
    const bool ok = tid < dk;
    s_alpha[tid] =
        ok ? __builtin_amdgcn_exp2f(a.g[(size_t)bh * dk + tid] * kLog2e) : 1.f;
    s_k[tid] = ok ? io<Tio>::to_f(k[tid]) : 0.f;
    s_q[tid] = ok ? io<Tio>::to_f(q[tid]) : 0.f;
  }
  __syncthreads();

  // per-thread partial sums over its rows, then over the lanes of the wave
  // with the same column group (shuffles), then over the waves (LDS)
  float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
  float qk = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    const float al = s_alpha[c], kc = s_k[c], qc = s_q[c];
    s[i].x *= al; s[i].y *= al; s[i].z *= al; s[i].w *= al;
    x[0] += s[i].x * kc; x[1] += s[i].y * kc; x[2] += s[i].z * kc; x[3] += s[i].w * kc;
    y[0] += s[i].x * qc; y[1] += s[i].y * qc; y[2] += s[i].z * qc; y[3] += s[i].w * qc;
    qk += qc * kc;
  }
  // lanes l and l ^ off share a column group for every off in CG..32
#pragma unroll
  for (int off = 32; off >= CG; off >>= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] += __shfl_xor(x[j], off);
      y[j] += __shfl_xor(y[j], off);
    }
    qk += __shfl_xor(qk, off);
  }
  float4 X = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 Y = make_float4(0.f, 0.f, 0.f, 0.f);
  float QK = 0.f;
  if constexpr (kTwoLevel) {
    if ((tid & 63) < CG) {
      const int w = tid / 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s_part[w][j][cg] = x[j];
        s_part[w][4 + j][cg] = y[j];
      }
      s_part[w][8][cg] = qk;
    }
    __syncthreads();
    if (tid < 9 * CG) {
      const int comp = tid / CG, c = tid % CG;
      float t = 0.f;
#pragma unroll
      for (int r = 0; r < NW; ++r) t += s_part[r][comp][c];
      s_fin[comp][c] = t;
    }
    __syncthreads();
    X = make_float4(s_fin[0][cg], s_fin[1][cg], s_fin[2][cg], s_fin[3][cg]);
    Y = make_float4(s_fin[4][cg], s_fin[5][cg], s_fin[6][cg], s_fin[7][cg]);
    QK = s_fin[8][cg];
  } else {
    if ((tid & 63) < CG) {
      const int w = tid / 64;
      s_red[w][cg][0] = make_float4(x[0], x[1], x[2], x[3]);
      s_red[w][cg][1] = make_float4(y[0], y[1], y[2], y[3]);
      s_red[w][cg][2] = make_float4(qk, 0.f, 0.f, 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NW; ++r) {
      const float4 xr = s_red[r][cg][0], yr = s_red[r][cg][1];
      X.x += xr.x; X.y += xr.y; X.z += xr.z; X.w += xr.w;
      Y.x += yr.x; Y.y += yr.y; Y.z += yr.z; Y.w += yr.w;
      QK += s_red[r][cg][2].x;
    }
  }

  const Tio* v = static_cast<const Tio*>(a.v) + (size_t)bh * dv + 4 * cg;
  const float beta = a.beta[bh];
  float vv[4] = {0.f, 0.f, 0.f, 0.f};
  if (col_ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = io<Tio>::to_f(v[i]);
  }
  float4 u;
  u.x = beta * (vv[0] - X.x);
  u.y = beta * (vv[1] - X.y);
  u.z = beta * (vv[2] - X.z);
  u.w = beta * (vv[3] - X.w);

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    const float kc = s_k[c];
    float4 w;
    w.x = s[i].x + kc * u.x; w.y = s[i].y + kc * u.y;
    w.z = s[i].z + kc * u.z; w.w = s[i].w + kc * u.w;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), rs,
                                           soff(c), 0, kPol);
  }

  // output (after the state stores, so that the state's registers are free)
  if (rg == 0) {
    Tio* o = static_cast<Tio*>(a.o) + (size_t)bh * dv + 4 * cg;
    float ov[4] = {a.scale * (Y.x + QK * u.x), a.scale * (Y.y + QK * u.y),
                   a.scale * (Y.z + QK * u.z), a.scale * (Y.w + QK * u.w)};
    if (kGated) {
      // output epilogue ("Kimi K3: The Manos, The Mythos, The Legendos",
      // section "Kimi Linear": per-head norm, then the output gate); the
      // CG lanes of this row are lanes 0 .. CG-1 of wave 0
      float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
      for (int m = CG / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
      const float r = rsqrtf(ss / (float)dv + a.eps);
      const Tio* z = static_cast<const Tio*>(a.z) + (size_t)bh * dv + 4 * cg;
      if (col_ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gate = 1.f / (1.f + __builtin_amdgcn_exp2f(
                                              -io<Tio>::to_f(z[i]) * kLog2e));
          ov[i] = ov[i] * r * a.w[4 * cg + i] * gate;
        }
      }
    }
    if (col_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = io<Tio>::from_f(ov[i]);
    }
  }

}

// Launch shape: one float4 per thread and row group, at most 1024 threads
// per workgroup (D^2 / 4 below D = 64).  At D = 128, 1024 threads hold 4 rows
// each in 44 VGPRs (46 with the fused output epilogue, 50-53 in the
// run-time-stride variants), so two workgroups (128 KB of state loads) are
// in flight per CU.  The state is touched once per step, so its accesses carry the
// non-temporal policy (measured: the kernel's own time then covers all of
// its traffic, and back-to-back steps run at the streaming ceiling).
// Head dims equal to the tile run a variant with compile-time strides
// (measured: the run-time strides and masks cost the 128 x 128 step ~5 %).
template <typename Tio, int D>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  constexpr int T = (D * D / 4) < 1024 ? (D * D / 4) : 1024;
  const unsigned blocks = (unsigned)a.B * (unsigned)a.H;
  const bool exact = a.dk == D && a.dv == D;
  if (a.z)  // fused output epilogue
    return exact ? launch_kernel(decode_kernel<Tio, D, T, true, true, true>,
                                 dim3(blocks), dim3(T), st, a)
                 : launch_kernel(decode_kernel<Tio, D, T, true, true, false>,
                                 dim3(blocks), dim3(T), st, a);
  return exact ? launch_kernel(decode_kernel<Tio, D, T, true, false, true>,
                               dim3(blocks), dim3(T), st, a)
               : launch_kernel(decode_kernel<Tio, D, T, true, false, false>,
                               dim3(blocks), dim3(T), st, a);
}

template <typename Tio>
hipError_t launch_d(const DecodeArgs& a, int D, hipStream_t st) {
  switch (D) {
    case 16: return launch<Tio, 16>(a, st);
    case 32: return launch<Tio, 32>(a, st);
    case 64: return launch<Tio, 64>(a, st);
    case 128: return launch<Tio, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int D, bool bf16_io,
                         hipStream_t st) {
  return bf16_io ? launch_d<bf16>(a, D, st) : launch_d<float>(a, D, st);
}

}  // namespace kda
