// Speculative-decode verify and commit.
//
// "Model evolution after DeepSeek V3" (uncledou.site), section four
// (speculative sampling has become standard): decode is bound by memory
// bandwidth, so a cheap draft proposes several tokens, the large model
// checks them in one parallel pass and keeps the ones it agrees with.  For a
// KDA layer this means running T draft tokens through the recurrence from a
// cached state, emitting every draft position's output, and afterwards
// advancing the state by only the accepted prefix.
//
// verify: per (sequence, head), the fp32 state is read once into registers
//   and the T tokens are applied in order, exactly as the decode kernel
//   applies one token:
//     aS = Diag(exp g_t) S;  x = (aS)^T k_t;  y = (aS)^T q_t
//     u_t = beta_t (v_t - x);  o_t = scale (y + (q_t . k_t) u_t)
//     S = aS + k_t u_t^T
//   o_t and the fp32 pseudo-values u_t are written; the state in memory is
//   left unchanged, so rejecting any suffix costs nothing.
// commit: per (sequence, head), with a = accepted[sequence] (clamped to
//   [0, T]) the state is read once, the a updates S = Diag(exp g_t) S +
//   k_t u_t^T are applied with the decode kernel's arithmetic, and the state
//   is written once (not at all when a = 0).
// step: commit of the previous draft's accepted prefix followed by verify
//   of the new draft, in one pass: the state is read once, the accepted
//   updates are applied and the state is written (when any was accepted),
//   and the new draft is run from the registers.
// State traffic per head: verify reads 4 d^2 bytes and commit reads and
// writes 8 d^2, against 8 d^2 per accepted token for single decode steps; a
// step reads and writes 8 d^2 where commit then verify move 12 d^2.
#include <stdlib.h>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kMaxSpecT = 16;

// Thread (rg, cg) owns the float4 column group cg of rows rg, rg + RG, ...
// (the decode kernel's mapping); a wave holds 64 / CG lanes of each column
// group.
template <int D, int NT>
struct SpecTiling {
  static constexpr int CG = D / 4;
  static constexpr int RG = NT / CG;
  static constexpr int RPT = D / RG;
  static constexpr int NW = NT / 64;
  static_assert(NT % CG == 0 && D % RG == 0 && 32 % CG == 0 && NT >= 64,
                "spec tiling");
};

// The commit's update of one state row group by token t: per element the
// rounded product s <- alpha s, then one fused multiply-add s <- k u + s.
// Both roundings are spelled out (no contraction left to the compiler), so
// the commit and step kernels round alike whatever their unrolling.
__device__ __forceinline__ void commit_update(float4& s, float al, float kc,
                                              const float4& u) {
#pragma clang fp contract(off)
  s.x = s.x * al; s.y = s.y * al; s.z = s.z * al; s.w = s.w * al;
  s.x = __builtin_fmaf(kc, u.x, s.x); s.y = __builtin_fmaf(kc, u.y, s.y);
  s.z = __builtin_fmaf(kc, u.z, s.z); s.w = __builtin_fmaf(kc, u.w, s.w);
}

// The state slice of (sequence, head) bh: row bh of [B, H, dk, dv], or,
// with a state pool, row (state_idx[b], h) of [pool_slots, H, dk, dv].  A
// padding entry (slot out of range) gets an empty buffer: its state loads
// read 0 and its stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t spec_state(const SpecArgs& a,
                                                            int bh, int dk,
                                                            int dv) {
  size_t row = bh;
  bool ok = true;
  if (a.state_idx) {
    const int32_t r = a.state_idx[bh / a.H];
    ok = r >= 0 && r < a.pool_slots;
    row = ok ? (size_t)r * a.H + bh % a.H : 0;
  }
  return make_rsrc(a.state + row * dk * dv, ok ? dk * dv * 4 : 0);
}

template <typename Tio, int D, int NT, bool kStep>
__global__ __launch_bounds__(NT) void spec_verify_kernel(SpecArgs a) {
  // every fused multiply-add below is written out: the verify and step
  // instantiations then round alike
#pragma clang fp contract(off)
  using Ti = SpecTiling<D, NT>;
  constexpr int CG = Ti::CG, RG = Ti::RG, RPT = Ti::RPT, NW = Ti::NW;
  __shared__ float s_alpha[kMaxSpecT][D], s_k[kMaxSpecT][D], s_q[kMaxSpecT][D];
  __shared__ float4 s_red[2][NW][CG][3];

  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int T = a.T;
  // the stored slice is dk x dv (<= D x D); padded rows and column groups
  // are zero here and never stored
  const int dk = a.dk, dv = a.dv;
  const bool col_ok = 4 * cg < dv;
  const __amdgpu_buffer_rsrc_t rs = spec_state(a, bh, dk, dv);

  // a step touches the state once (read, then write): non-temporal
  constexpr int kPolicy = kStep ? kCachePolicyNt : 0;
  auto soff = [&](int c) {
    return (c < dk && col_ok) ? (uint32_t)((c * dv + 4 * cg) * 4) : kOffNone;
  };
  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(rs, soff(rg + RG * i),
                                                      0, kPolicy));

  if constexpr (kStep) {
    // commit of the previous draft's first `acc` tokens (uniform per
    // workgroup), exactly as spec_commit_kernel applies them
    int acc = a.T_prev > 0 ? a.accepted_prev[b] : 0;
    acc = acc < 0 ? 0 : (acc > a.T_prev ? a.T_prev : acc);
    if (acc > 0) {
      for (int e = tid; e < acc * D; e += NT) {
        const int t = e / D, c = e % D;
        const size_t row = ((size_t)b * a.T_prev + t) * a.H + h;
        const bool ok = c < dk;
        s_alpha[t][c] =
            ok ? __builtin_amdgcn_exp2f(a.g_prev[row * dk + c] * kLog2e)
               : 1.f;
        s_k[t][c] = ok ? io<Tio>::to_f(
                             static_cast<const Tio*>(a.k_prev)[row * dk + c])
                       : 0.f;
      }
      __syncthreads();
      for (int t = 0; t < acc; ++t) {
        const size_t row = ((size_t)b * a.T_prev + t) * a.H + h;
        const float4 u =
            col_ok ? *reinterpret_cast<const float4*>(a.u_prev + row * dv +
                                                      4 * cg)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int c = rg + RG * i;
          commit_update(s[i], s_alpha[t][c], s_k[t][c], u);
        }
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, s[i]), rs, soff(rg + RG * i), 0,
            kCachePolicyNt);
      // the staging arrays are refilled below, and u (which may be u_prev)
      // is written only after every thread's reads of u_prev
      __syncthreads();
    }
  }

  // token t of sequence b, head h: row (b * T + t) * H + h
  for (int e = tid; e < T * D; e += NT) {
    const int t = e / D, c = e % D;
    const size_t row = ((size_t)b * T + t) * a.H + h;
    const bool ok = c < dk;
    s_alpha[t][c] =
        ok ? __builtin_amdgcn_exp2f(a.g[row * dk + c] * kLog2e) : 1.f;
    s_k[t][c] =
        ok ? io<Tio>::to_f(static_cast<const Tio*>(a.k)[row * dk + c]) : 0.f;
    s_q[t][c] =
        ok ? io<Tio>::to_f(static_cast<const Tio*>(a.q)[row * dk + c]) : 0.f;
  }
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = rg + RG * i;
      const float al = s_alpha[t][c], kc = s_k[t][c], qc = s_q[t][c];
      s[i].x = s[i].x * al; s[i].y = s[i].y * al;
      s[i].z = s[i].z * al; s[i].w = s[i].w * al;
      x[0] = __builtin_fmaf(s[i].x, kc, x[0]);
      x[1] = __builtin_fmaf(s[i].y, kc, x[1]);
      x[2] = __builtin_fmaf(s[i].z, kc, x[2]);
      x[3] = __builtin_fmaf(s[i].w, kc, x[3]);
      y[0] = __builtin_fmaf(s[i].x, qc, y[0]);
      y[1] = __builtin_fmaf(s[i].y, qc, y[1]);
      y[2] = __builtin_fmaf(s[i].z, qc, y[2]);
      y[3] = __builtin_fmaf(s[i].w, qc, y[3]);
      qk = __builtin_fmaf(qc, kc, qk);
    }
#pragma unroll
    for (int off = 32; off >= CG; off >>= 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] += __shfl_xor(x[j], off);
        y[j] += __shfl_xor(y[j], off);
      }
      qk += __shfl_xor(qk, off);
    }
    // double-buffered by token parity: one barrier per token
    float4 (*red)[CG][3] = s_red[t & 1];
    if ((tid & 63) < CG) {
      const int w = tid / 64;
      red[w][cg][0] = make_float4(x[0], x[1], x[2], x[3]);
      red[w][cg][1] = make_float4(y[0], y[1], y[2], y[3]);
      red[w][cg][2] = make_float4(qk, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    float4 X = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 Y = make_float4(0.f, 0.f, 0.f, 0.f);
    float QK = 0.f;
#pragma unroll
    for (int r = 0; r < NW; ++r) {
      const float4 xr = red[r][cg][0], yr = red[r][cg][1];
      X.x += xr.x; X.y += xr.y; X.z += xr.z; X.w += xr.w;
      Y.x += yr.x; Y.y += yr.y; Y.z += yr.z; Y.w += yr.w;
      QK += red[r][cg][2].x;
    }
    const size_t row = ((size_t)b * T + t) * a.H + h;
    const Tio* v = static_cast<const Tio*>(a.v) + row * dv + 4 * cg;
    const float beta = a.beta[row];
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
    if (rg == 0 && col_ok) {
      Tio* o = static_cast<Tio*>(a.o) + row * dv + 4 * cg;
      o[0] = io<Tio>::from_f(a.scale * __builtin_fmaf(QK, u.x, Y.x));
      o[1] = io<Tio>::from_f(a.scale * __builtin_fmaf(QK, u.y, Y.y));
      o[2] = io<Tio>::from_f(a.scale * __builtin_fmaf(QK, u.z, Y.z));
      o[3] = io<Tio>::from_f(a.scale * __builtin_fmaf(QK, u.w, Y.w));
      *reinterpret_cast<float4*>(a.u + row * dv + 4 * cg) = u;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float kc = s_k[t][rg + RG * i];
      s[i].x = __builtin_fmaf(kc, u.x, s[i].x);
      s[i].y = __builtin_fmaf(kc, u.y, s[i].y);
      s[i].z = __builtin_fmaf(kc, u.z, s[i].z);
      s[i].w = __builtin_fmaf(kc, u.w, s[i].w);
    }
  }
}

template <typename Tio, int D, int NT>
__global__ __launch_bounds__(NT) void spec_commit_kernel(SpecArgs a) {
  using Ti = SpecTiling<D, NT>;
  constexpr int CG = Ti::CG, RG = Ti::RG, RPT = Ti::RPT;
  __shared__ float s_alpha[kMaxSpecT][D], s_k[kMaxSpecT][D];

  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int T = a.T;
  int acc = a.accepted[b];
  acc = acc < 0 ? 0 : (acc > T ? T : acc);
  if (acc == 0) return;  // uniform: the state stays as it is

  const int dk = a.dk, dv = a.dv;
  const bool col_ok = 4 * cg < dv;
  const __amdgpu_buffer_rsrc_t rs = spec_state(a, bh, dk, dv);
  auto soff = [&](int c) {
    return (c < dk && col_ok) ? (uint32_t)((c * dv + 4 * cg) * 4) : kOffNone;
  };
  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(rs, soff(rg + RG * i),
                                                      0, kCachePolicyNt));
  for (int e = tid; e < acc * D; e += NT) {
    const int t = e / D, c = e % D;
    const size_t row = ((size_t)b * T + t) * a.H + h;
    const bool ok = c < dk;
    s_alpha[t][c] =
        ok ? __builtin_amdgcn_exp2f(a.g[row * dk + c] * kLog2e) : 1.f;
    s_k[t][c] =
        ok ? io<Tio>::to_f(static_cast<const Tio*>(a.k)[row * dk + c]) : 0.f;
  }
  __syncthreads();
  for (int t = 0; t < acc; ++t) {
    const size_t row = ((size_t)b * T + t) * a.H + h;
    const float4 u =
        col_ok ? *reinterpret_cast<const float4*>(a.u + row * dv + 4 * cg)
               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = rg + RG * i;
      commit_update(s[i], s_alpha[t][c], s_k[t][c], u);
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(u32x4, s[i]), rs, soff(rg + RG * i), 0,
        kCachePolicyNt);
}

// Threads per workgroup, capped by D^2 / 4.  Commit streams the state like
// the decode kernel (1024 threads at D = 128).  Verify reduces across the
// waves once per token, and every thread reads every wave's partial sums, so
// it uses 4 waves (256 threads, 16 rows per thread at D = 128): a sixth of
// the LDS traffic per token of 16 waves, and four workgroups per CU.
template <int D, int CAP>
constexpr int spec_threads() {
  return (D * D / 4) < CAP ? (D * D / 4) : CAP;
}

template <typename Tio, int D>
hipError_t launch_d(const SpecArgs& a, SpecMode mode, hipStream_t st) {
  const unsigned blocks = (unsigned)a.B * (unsigned)a.H;
  if (mode == SpecMode::kCommit) {
    constexpr int NT = spec_threads<D, 1024>();
    return launch_kernel(spec_commit_kernel<Tio, D, NT>, dim3(blocks),
                         dim3(NT), st, a);
  }
  constexpr int NT = spec_threads<D, 256>();
  if (mode == SpecMode::kStep)
    return launch_kernel(spec_verify_kernel<Tio, D, NT, true>, dim3(blocks),
                         dim3(NT), st, a);
  return launch_kernel(spec_verify_kernel<Tio, D, NT, false>, dim3(blocks),
                       dim3(NT), st, a);
}

template <typename Tio>
hipError_t launch_t(const SpecArgs& a, int D, SpecMode mode, hipStream_t st) {
  switch (D) {
    case 16: return launch_d<Tio, 16>(a, mode, st);
    case 32: return launch_d<Tio, 32>(a, mode, st);
    case 64: return launch_d<Tio, 64>(a, mode, st);
    case 128: return launch_d<Tio, 128>(a, mode, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int max_spec_tokens() { return kMaxSpecT; }

hipError_t launch_spec(const SpecArgs& a, int D, bool bf16_io, SpecMode mode,
                       hipStream_t st) {
  return bf16_io ? launch_t<bf16>(a, D, mode, st)
                 : launch_t<float>(a, D, mode, st);
}

}  // namespace kda
