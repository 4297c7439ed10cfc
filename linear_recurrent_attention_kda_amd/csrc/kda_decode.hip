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
// slice stays in registers between the reduction and the write-back.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

template <typename Tio, int D, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a) {
  constexpr int CG = D / 4;       // float4 column groups
  constexpr int RG = NT / CG;     // row groups
  constexpr int RPT = D / RG;     // rows per thread
  static_assert(NT % CG == 0 && D % RG == 0, "decode tiling");

  __shared__ float s_alpha[D], s_k[D], s_q[D];
  __shared__ float4 s_red[RG][CG][3];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  float* S = a.state + (size_t)bh * D * D;

  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = *reinterpret_cast<const float4*>(S + (size_t)(rg + RG * i) * D +
                                            4 * cg);

  const Tio* q = static_cast<const Tio*>(a.q) + (size_t)bh * D;
  const Tio* k = static_cast<const Tio*>(a.k) + (size_t)bh * D;
  if (tid < D) {
    s_alpha[tid] = __builtin_amdgcn_exp2f(a.g[(size_t)bh * D + tid] * kLog2e);
    s_k[tid] = io<Tio>::to_f(k[tid]);
    s_q[tid] = io<Tio>::to_f(q[tid]);
  }
  __syncthreads();

  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  float qk = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    const float al = s_alpha[c], kc = s_k[c], qc = s_q[c];
    s[i].x *= al; s[i].y *= al; s[i].z *= al; s[i].w *= al;
    x.x += s[i].x * kc; x.y += s[i].y * kc; x.z += s[i].z * kc; x.w += s[i].w * kc;
    y.x += s[i].x * qc; y.y += s[i].y * qc; y.z += s[i].z * qc; y.w += s[i].w * qc;
    qk += qc * kc;
  }
  s_red[rg][cg][0] = x;
  s_red[rg][cg][1] = y;
  s_red[rg][cg][2] = make_float4(qk, 0.f, 0.f, 0.f);
  __syncthreads();

  float4 X = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 Y = make_float4(0.f, 0.f, 0.f, 0.f);
  float QK = 0.f;
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const float4 xr = s_red[r][cg][0], yr = s_red[r][cg][1];
    X.x += xr.x; X.y += xr.y; X.z += xr.z; X.w += xr.w;
    Y.x += yr.x; Y.y += yr.y; Y.z += yr.z; Y.w += yr.w;
    QK += s_red[r][cg][2].x;
  }

  const Tio* v = static_cast<const Tio*>(a.v) + (size_t)bh * D + 4 * cg;
  const float beta = a.beta[bh];
  float4 u;
  u.x = beta * (io<Tio>::to_f(v[0]) - X.x);
  u.y = beta * (io<Tio>::to_f(v[1]) - X.y);
  u.z = beta * (io<Tio>::to_f(v[2]) - X.z);
  u.w = beta * (io<Tio>::to_f(v[3]) - X.w);

  if (rg == 0) {
    Tio* o = static_cast<Tio*>(a.o) + (size_t)bh * D + 4 * cg;
    o[0] = io<Tio>::from_f(a.scale * (Y.x + QK * u.x));
    o[1] = io<Tio>::from_f(a.scale * (Y.y + QK * u.y));
    o[2] = io<Tio>::from_f(a.scale * (Y.z + QK * u.z));
    o[3] = io<Tio>::from_f(a.scale * (Y.w + QK * u.w));
  }

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    const float kc = s_k[c];
    float4 w;
    w.x = s[i].x + kc * u.x; w.y = s[i].y + kc * u.y;
    w.z = s[i].z + kc * u.z; w.w = s[i].w + kc * u.w;
    *reinterpret_cast<float4*>(S + (size_t)c * D + 4 * cg) = w;
  }
}

template <typename Tio, int D>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  constexpr int NT = (D * D / 4) < 256 ? (D * D / 4) : 256;
  const unsigned blocks = (unsigned)a.B * (unsigned)a.H;
  return launch_kernel(decode_kernel<Tio, D, NT>, dim3(blocks), dim3(NT), st,
                       a);
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
