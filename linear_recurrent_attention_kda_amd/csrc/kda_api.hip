// C-ABI entry points of libkda (declared and documented in include/kda.h):
// argument validation on the host, then kernel launches on the caller's
// stream.  Validation touches no HIP API, so an invalid call returns before
// anything is enqueued.
#include "../../include/kda.h"

#include <limits.h>

#include <atomic>
#include <mutex>

#include "kda_internal.hpp"

// Prefill workspace of kda_prefill_varlen_noalloc: a fixed device array that
// each GPU the library runs on holds until the process ends.  In host code
// this name is only a stand-in for the array: its device address comes from
// hipGetSymbolAddress (scratch_ptr below), never from the name itself.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, fetched once per device
// (each GPU holds its own copy at its own address).  nullptr on failure.
void* scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q)
      return nullptr;
    addr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Head dims: any multiple of 16 up to 128, d_k and d_v independently.  The
// kernels are compiled for square tiles of 16, 32, 64 or 128 channels; a
// call runs on the smallest tile that holds both dims, with the channels
// past them zero inside the kernels (the state's padded rows and columns
// stay zero: their k, q and v entries are zero).
bool supported_dim(int32_t d) { return d >= 16 && d <= 128 && d % 16 == 0; }
bool supported_dims(int32_t Dk, int32_t Dv) {
  return supported_dim(Dk) && supported_dim(Dv);
}
int32_t tile_dim(int32_t Dk, int32_t Dv) {
  const int32_t m = Dk > Dv ? Dk : Dv;
  return m <= 16 ? 16 : m <= 32 ? 32 : m <= 64 ? 64 : 128;
}

bool supported_chunk(int32_t C) { return C == 16 || C == 32 || C == 64; }

// Shape / dtype checks shared by both prefill entry points.
kda_status_t check_prefill_common(int32_t H, int32_t Dk, int32_t Dv,
                                  int32_t C, int32_t dtype) {
  if (H <= 0 || Dk <= 0 || Dv <= 0 || C <= 0) return KDA_ERR_INVALID_ARG;
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32)
    return KDA_ERR_UNSUPPORTED;
  if (!supported_dims(Dk, Dv) || !supported_chunk(C))
    return KDA_ERR_UNSUPPORTED;
  // The kernels address each chunk's token rows (and the input prologue's
  // three rows before them) through 32-bit buffer offsets, with masked
  // lanes parked just below 2^32: C + 8 rows of H heads must stay well
  // under 4 GiB (H <= 116,508 at d = 128, C = 64 in fp32).
  if ((int64_t)(C + 8) * H * tile_dim(Dk, Dv) * 4 > 0xFFFF0000LL)
    return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

// Stages of a prefill call: the chunk-prep kernel (writes the workspace) and
// the chunk-recurrence kernel (reads it).
constexpr int kStagePrep = 1, kStageRecur = 2, kStagesBoth = 3;

// With validate_only, every check except the workspace's runs and nothing is
// launched.
kda_status_t run_prefill(kda::PrefillArgs& a, int32_t C, int32_t dtype,
                         void* workspace, size_t workspace_bytes, void* stream,
                         int stages = kStagesBoth,
                         bool validate_only = false) {
  const int32_t D = tile_dim(a.dk, a.dv);
  const size_t need =
      kda_prefill_workspace_size(a.N, a.total_T, a.H, a.dk, a.dv, C);
  if (need == 0) return KDA_ERR_INVALID_ARG;
  // the prep kernel indexes its (sequence, chunk, head) items in 32 bits
  if ((int64_t)a.N * a.max_chunks * a.H >= ((int64_t)1 << 31))
    return KDA_ERR_UNSUPPORTED;
  if (validate_only) return KDA_OK;
  if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return KDA_ERR_INVALID_ARG;
  a.ws = static_cast<char*>(workspace);
  a.nslots = kda::num_slots(a.N, a.total_T, C);
  const bool bf16_io = dtype == KDA_DTYPE_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((stages & kStagePrep) && a.total_T > 0 && a.max_chunks > 0) {
    if (kda::launch_prep(a, D, C, bf16_io, st) != hipSuccess)
      return KDA_ERR_LAUNCH;
  }
  if ((stages & kStageRecur) &&
      kda::launch_recur(a, D, C, bf16_io, st) != hipSuccess)
    return KDA_ERR_LAUNCH;
  return KDA_OK;
}

kda_status_t check_tensors(int64_t tokens, const void* q, const void* k,
                           const void* v, const float* g, const float* beta,
                           const void* o) {
  if (tokens > 0) {
    if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(g, 16) || !aligned(o, 16) || !aligned(beta, 4))
      return KDA_ERR_INVALID_ARG;
  }
  return KDA_OK;
}

// State checkpoints requested by a prefill call: none, every `every` tokens
// of each sequence, or at the listed positions (see kda.h).
// A state pool for the prefill's initial and final states (both the pool).
struct PoolOpts {
  const int32_t* idx = nullptr;
  const int32_t* has_initial = nullptr;
  int32_t slots = 0;
};

struct CkptOpts {
  enum Mode { kNone, kEvery, kList } mode = kNone;
  int32_t every = 0;
  const int32_t* pos = nullptr;
  const int32_t* cu = nullptr;
  int32_t n = 0;
  float* states = nullptr;
  size_t bytes = 0;
};

// Validates the checkpoint request and fills its part of the launch args.
kda_status_t set_ckpt(const CkptOpts& ck, int64_t total_T, int32_t H,
                      int32_t Dk, int32_t Dv, int32_t C, kda::PrefillArgs& a) {
  a.ckpt_states = nullptr;
  a.ckpt_every = 0;
  a.ckpt_pos = nullptr;
  a.cu_ckpt = nullptr;
  a.n_ckpt = 0;
  if (ck.mode == CkptOpts::kNone) return KDA_OK;
  int64_t slots = 0;
  if (ck.mode == CkptOpts::kEvery) {
    if (ck.every <= 0 || ck.every % C != 0) return KDA_ERR_INVALID_ARG;
    slots = total_T / ck.every;
  } else {
    if (ck.n < 0) return KDA_ERR_INVALID_ARG;
    slots = ck.n;
    if (slots > 0 && (!ck.pos || !ck.cu || !aligned(ck.pos, 4) ||
                      !aligned(ck.cu, 4)))
      return KDA_ERR_INVALID_ARG;
  }
  if (slots == 0) return KDA_OK;  // no checkpoint can be written
  if (!ck.states || !aligned(ck.states, 16)) return KDA_ERR_INVALID_ARG;
  const double need = (double)slots * H * Dk * Dv * 4.0;
  if (need > 9.0e18 || (double)ck.bytes < need) return KDA_ERR_INVALID_ARG;
  a.ckpt_states = ck.states;
  if (ck.mode == CkptOpts::kEvery) {
    a.ckpt_every = ck.every;
  } else {
    a.ckpt_pos = ck.pos;
    a.cu_ckpt = ck.cu;
    a.n_ckpt = ck.n;
  }
  return KDA_OK;
}

// Varlen prefill, with the requested state checkpoints.
kda_status_t prefill_varlen(const void* q, const void* k, const void* v,
                            const float* g, const float* beta,
                            const int32_t* cu_seqlens, int32_t N,
                            int64_t total_T, int32_t max_seqlen,
                            const float* initial_state, float* final_state,
                            void* o, int32_t H, int32_t Dk, int32_t Dv,
                            int32_t C, float scale, int32_t dtype,
                            const CkptOpts& ck, const float* conv_w,
                            void* workspace, size_t workspace_bytes,
                            void* stream, int stages = kStagesBoth,
                            bool validate_only = false,
                            const void* gate_z = nullptr,
                            const float* gate_w = nullptr,
                            float gate_eps = 0.f,
                            const PoolOpts& pool = PoolOpts{}) {
  if (N <= 0 || total_T < 0 || max_seqlen < 0) return KDA_ERR_INVALID_ARG;
  if (total_T > 0 && max_seqlen == 0) return KDA_ERR_INVALID_ARG;
  kda_status_t st = check_prefill_common(H, Dk, Dv, C, dtype);
  if (st != KDA_OK) return st;
  if (!cu_seqlens || !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARG;
  if (stages == kStagesBoth) {
    st = check_tensors(total_T, q, k, v, g, beta, o);
  } else if (stages == kStagePrep) {
    // the inputs only (o is not touched)
    st = check_tensors(total_T, q, k, v, g, beta, q);
  } else if (total_T > 0 && (!o || !aligned(o, 16))) {
    st = KDA_ERR_INVALID_ARG;  // the recurrence: o only
  }
  if (st != KDA_OK) return st;
  if ((initial_state && !aligned(initial_state, 16)) ||
      (final_state && !aligned(final_state, 16)))
    return KDA_ERR_INVALID_ARG;
  if ((int64_t)(tile_dim(Dk, Dv) / 16) * H * N > INT_MAX)
    return KDA_ERR_UNSUPPORTED;
  // the input prologue's taps are per channel of q, k and v alike
  if (conv_w && Dk != Dv) return KDA_ERR_UNSUPPORTED;
  const int64_t maxlen = max_seqlen < total_T ? max_seqlen : total_T;

  kda::PrefillArgs a{};
  st = set_ckpt(ck, total_T, H, Dk, Dv, C, a);
  if (st != KDA_OK) return st;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.cu_seqlens = cu_seqlens;
  a.T_fixed = 0;
  a.N = N;
  a.total_T = total_T;
  a.max_chunks = (int32_t)((maxlen + C - 1) / C);
  a.initial_state = initial_state;
  a.final_state = final_state;
  a.o = o;
  a.H = H;
  a.dk = Dk;
  a.dv = Dv;
  a.scale = scale;
  a.conv_w = conv_w;
  a.gate_z = gate_z;
  a.gate_w = gate_w;
  a.gate_eps = gate_eps;
  a.state_idx = pool.idx;
  a.has_initial = pool.has_initial;
  a.pool_slots = pool.slots;
  return run_prefill(a, C, dtype, workspace, workspace_bytes, stream, stages,
                     validate_only);
}

kda_status_t decode_step(const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float* state,
                         void* o, const void* z, const float* w, float eps,
                         int32_t B, int32_t H, int32_t Dk, int32_t Dv,
                         float scale, int32_t dtype, void* stream,
                         const int32_t* state_idx = nullptr,
                         int32_t pool_slots = 0) {
  if (B <= 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_ERR_INVALID_ARG;
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32)
    return KDA_ERR_UNSUPPORTED;
  if (!supported_dims(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > INT_MAX) return KDA_ERR_UNSUPPORTED;
  kda_status_t st = check_tensors((int64_t)B, q, k, v, g, beta, o);
  if (st != KDA_OK) return st;
  if (!state || !aligned(state, 16)) return KDA_ERR_INVALID_ARG;

  kda::DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.state = state;
  a.o = o;
  a.B = B;
  a.H = H;
  a.dk = Dk;
  a.dv = Dv;
  a.scale = scale;
  a.z = z;
  a.w = w;
  a.eps = eps;
  a.state_idx = state_idx;
  a.pool_slots = pool_slots;
  if (kda::launch_decode(a, tile_dim(Dk, Dv), dtype == KDA_DTYPE_BF16,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_LAUNCH;
  return KDA_OK;
}

// One speculative step (the commit of the previous draft, then the verify
// of the next), on a state array or a state pool.  T == 0 commits only;
// T_prev == 0 verifies only; with both 0 there is nothing to do.
kda_status_t spec_step(const void* k_prev, const float* g_prev,
                       const float* u_prev, const int32_t* accepted_prev,
                       int32_t T_prev, const void* q, const void* k,
                       const void* v, const float* g, const float* beta,
                       float* state, void* o, float* u, int32_t B, int32_t T,
                       int32_t H, int32_t Dk, int32_t Dv, float scale,
                       int32_t dtype, void* stream,
                       const int32_t* state_idx, int32_t pool_slots) {
  if (B <= 0 || H <= 0 || T < 0 || Dk <= 0 || Dv <= 0 || T_prev < 0)
    return KDA_ERR_INVALID_ARG;
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32)
    return KDA_ERR_UNSUPPORTED;
  if (!supported_dims(Dk, Dv) || T > kda::max_spec_tokens() ||
      T_prev > kda::max_spec_tokens())
    return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > INT_MAX) return KDA_ERR_UNSUPPORTED;
  if (!state || !aligned(state, 16)) return KDA_ERR_INVALID_ARG;
  if (T > 0) {
    kda_status_t st = check_tensors((int64_t)B * T, q, k, v, g, beta, o);
    if (st != KDA_OK) return st;
    if (!u || !aligned(u, 16)) return KDA_ERR_INVALID_ARG;
  }
  if (T_prev > 0) {
    if (!k_prev || !g_prev || !u_prev || !accepted_prev)
      return KDA_ERR_INVALID_ARG;
    if (!aligned(k_prev, 16) || !aligned(g_prev, 16) || !aligned(u_prev, 16) ||
        !aligned(accepted_prev, 4))
      return KDA_ERR_INVALID_ARG;
    // u may reuse u_prev's buffer only row for row: with another draft
    // length, one workgroup's new rows would be another's previous ones
    if (T > 0 && u == u_prev && T != T_prev) return KDA_ERR_INVALID_ARG;
  }
  if (T == 0 && T_prev == 0) return KDA_OK;  // nothing to do
  kda::SpecArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.state = state;
  a.o = o;
  a.u = u;
  a.B = B; a.T = T; a.H = H;
  a.dk = Dk; a.dv = Dv;
  a.scale = scale;
  a.T_prev = T_prev;
  if (T_prev > 0) {
    a.k_prev = k_prev; a.g_prev = g_prev; a.u_prev = u_prev;
    a.accepted_prev = accepted_prev;
  }
  a.state_idx = state_idx;
  a.pool_slots = pool_slots;
  if (kda::launch_spec(a, tile_dim(Dk, Dv), dtype == KDA_DTYPE_BF16,
                       kda::SpecMode::kStep,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_LAUNCH;
  return KDA_OK;
}

}  // namespace

extern "C" {

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int32_t status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported size, chunk or dtype";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
    case KDA_ERR_SCRATCH:
      return "problem needs more workspace than the fixed scratch buffer";
  }
  return "unknown status";
}

size_t kda_prefill_workspace_size(int32_t N, int64_t total_T, int32_t H,
                                  int32_t Dk, int32_t Dv, int32_t C) {
  if (N <= 0 || total_T < 0 || H <= 0 || !supported_dims(Dk, Dv) ||
      !supported_chunk(C))
    return 0;
  const int32_t D = tile_dim(Dk, Dv);
  const kda::WsLayout lay = kda::WsLayout::make(C, D, D);
  const int64_t slots = kda::num_slots(N, total_T, C);
  return (size_t)slots * (size_t)H * lay.block_bytes;
}

kda_status_t kda_prefill_chunked(const void* q, const void* k, const void* v,
                                 const float* g, const float* beta,
                                 const float* initial_state,
                                 float* final_state, void* o, int32_t B,
                                 int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                                 int32_t C, float scale, int32_t dtype,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (B <= 0 || T < 0) return KDA_ERR_INVALID_ARG;
  kda_status_t st = check_prefill_common(H, Dk, Dv, C, dtype);
  if (st != KDA_OK) return st;
  const int64_t total = (int64_t)B * T;
  st = check_tensors(total, q, k, v, g, beta, o);
  if (st != KDA_OK) return st;
  if ((initial_state && !aligned(initial_state, 16)) ||
      (final_state && !aligned(final_state, 16)))
    return KDA_ERR_INVALID_ARG;
  if ((int64_t)(tile_dim(Dk, Dv) / 16) * H * B > INT_MAX)
    return KDA_ERR_UNSUPPORTED;

  kda::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.cu_seqlens = nullptr;
  a.T_fixed = T;
  a.N = B;
  a.total_T = total;
  a.max_chunks = (T + C - 1) / C;
  a.initial_state = initial_state;
  a.final_state = final_state;
  a.o = o;
  a.H = H;
  a.dk = Dk;
  a.dv = Dv;
  a.scale = scale;
  return run_prefill(a, C, dtype, workspace, workspace_bytes, stream);
}

kda_status_t kda_prefill_varlen(const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const int32_t* cu_seqlens, int32_t N,
                                int64_t total_T, int32_t max_seqlen,
                                const float* initial_state,
                                float* final_state, void* o, int32_t H,
                                int32_t Dk, int32_t Dv, int32_t C, float scale,
                                int32_t dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return prefill_varlen(q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen,
                        initial_state, final_state, o, H, Dk, Dv, C, scale,
                        dtype, CkptOpts{}, nullptr, workspace,
                        workspace_bytes, stream);
}

kda_status_t kda_prefill_varlen_gated(
    const void* q, const void* k, const void* v, const float* g,
    const float* beta, const int32_t* cu_seqlens, int32_t N, int64_t total_T,
    int32_t max_seqlen, const float* initial_state, float* final_state,
    const void* z, const float* w, float eps, void* y, int32_t H, int32_t Dk,
    int32_t Dv, int32_t C, float scale, int32_t dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (!(eps >= 0.f)) return KDA_ERR_INVALID_ARG;
  if (total_T > 0 && (!z || !w || !aligned(z, 16) || !aligned(w, 16)))
    return KDA_ERR_INVALID_ARG;
  // every check of the prefill, and the workspace, before the first launch
  kda_status_t st = prefill_varlen(
      q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen, initial_state,
      final_state, y, H, Dk, Dv, C, scale, dtype, CkptOpts{}, nullptr,
      workspace, workspace_bytes, stream, kStagesBoth, true);
  if (st != KDA_OK) return st;
  const size_t need = kda_prefill_workspace_size(N, total_T, H, Dk, Dv, C);
  if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return KDA_ERR_INVALID_ARG;
  const int64_t rows = total_T * H;  // the epilogue's grid, as in its entry
  if (rows / (1024 / tile_dim(Dv, Dv)) >= ((int64_t)1 << 31))
    return KDA_ERR_UNSUPPORTED;
  // The fused kernel holds whole rows, i.e. one workgroup per (sequence,
  // head) instead of one per d_v slice.  Measured on MI355X it is faster
  // than the plain recurrence followed by the epilogue pass once there are
  // at least two such workgroups per compute unit (768 pairs: 4.13 against
  // 4.27 ms), and slower below (96 pairs: 1.06 against 0.75 ms).
  if (total_T == 0 || (int64_t)N * H >= 2 * (int64_t)kda::device_cus())
    return prefill_varlen(q, k, v, g, beta, cu_seqlens, N, total_T,
                          max_seqlen, initial_state, final_state, y, H, Dk,
                          Dv, C, scale, dtype, CkptOpts{}, nullptr,
                          workspace, workspace_bytes, stream, kStagesBoth,
                          false, total_T > 0 ? z : nullptr, w, eps);
  st = prefill_varlen(q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen,
                      initial_state, final_state, y, H, Dk, Dv, C, scale,
                      dtype, CkptOpts{}, nullptr, workspace, workspace_bytes,
                      stream);
  if (st != KDA_OK) return st;
  kda::EpilogueArgs e{};
  e.o = y; e.z = z; e.w = w; e.y = y;
  e.rows = rows;
  e.dv = Dv;
  e.eps = eps;
  if (kda::launch_epilogue(e, tile_dim(Dv, Dv), dtype == KDA_DTYPE_BF16,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_LAUNCH;
  return KDA_OK;
}

kda_status_t kda_prefill_varlen_noalloc(
    const void* q, const void* k, const void* v, const float* g,
    const float* beta, const int32_t* cu_seqlens, int32_t N, int64_t total_T,
    int32_t max_seqlen, const float* initial_state, float* final_state,
    void* o, int32_t H, int32_t Dk, int32_t Dv, int32_t C, float scale,
    int32_t dtype, void* stream) {
  const size_t need = kda_prefill_workspace_size(N, total_T, H, Dk, Dv, C);
  void* ws = nullptr;
  if (need > 0) {  // (need == 0: invalid sizes, reported below)
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
    // every other check runs before the first HIP call
    const kda_status_t st = prefill_varlen(
        q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen, initial_state,
        final_state, o, H, Dk, Dv, C, scale, dtype, CkptOpts{}, nullptr,
        nullptr, 0, stream, kStagesBoth, /*validate_only=*/true);
    if (st != KDA_OK) return st;
    ws = scratch_ptr();
    if (!ws) return KDA_ERR_LAUNCH;
  }
  return prefill_varlen(q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen,
                        initial_state, final_state, o, H, Dk, Dv, C, scale,
                        dtype, CkptOpts{}, nullptr, ws,
                        (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}

kda_status_t kda_prefill_varlen_prep(const void* q, const void* k,
                                     const void* v, const float* g,
                                     const float* beta,
                                     const int32_t* cu_seqlens, int32_t N,
                                     int64_t total_T, int32_t max_seqlen,
                                     int32_t H, int32_t Dk, int32_t Dv,
                                     int32_t C, int32_t dtype, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return prefill_varlen(q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen,
                        nullptr, nullptr, nullptr, H, Dk, Dv, C, 1.0f, dtype,
                        CkptOpts{}, nullptr, workspace, workspace_bytes,
                        stream, kStagePrep);
}

kda_status_t kda_prefill_varlen_recur(const int32_t* cu_seqlens, int32_t N,
                                      int64_t total_T, int32_t max_seqlen,
                                      const float* initial_state,
                                      float* final_state, void* o, int32_t H,
                                      int32_t Dk, int32_t Dv, int32_t C,
                                      float scale, int32_t dtype,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return prefill_varlen(nullptr, nullptr, nullptr, nullptr, nullptr,
                        cu_seqlens, N, total_T, max_seqlen, initial_state,
                        final_state, o, H, Dk, Dv, C, scale, dtype,
                        CkptOpts{}, nullptr, workspace, workspace_bytes,
                        stream, kStageRecur);
}

kda_status_t kda_prefill_varlen_ckpt(
    const void* q, const void* k, const void* v, const float* g,
    const float* beta, const int32_t* cu_seqlens, int32_t N, int64_t total_T,
    int32_t max_seqlen, const float* initial_state, float* final_state,
    void* o, int32_t H, int32_t Dk, int32_t Dv, int32_t C, float scale,
    int32_t dtype, int32_t ckpt_every, float* ckpt_states, size_t ckpt_bytes,
    void* workspace, size_t workspace_bytes, void* stream) {
  CkptOpts ck;
  ck.mode = CkptOpts::kEvery;
  ck.every = ckpt_every;
  ck.states = ckpt_states;
  ck.bytes = ckpt_bytes;
  return prefill_varlen(q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen,
                        initial_state, final_state, o, H, Dk, Dv, C, scale,
                        dtype, ck, nullptr, workspace, workspace_bytes,
                        stream);
}

kda_status_t kda_prefill_varlen_ckpt_at(
    const void* q, const void* k, const void* v, const float* g,
    const float* beta, const int32_t* cu_seqlens, int32_t N, int64_t total_T,
    int32_t max_seqlen, const float* initial_state, float* final_state,
    void* o, int32_t H, int32_t Dk, int32_t Dv, int32_t C, float scale,
    int32_t dtype, const int32_t* ckpt_pos, const int32_t* cu_ckpt,
    int32_t n_ckpt, float* ckpt_states, size_t ckpt_bytes, void* workspace,
    size_t workspace_bytes, void* stream) {
  CkptOpts ck;
  ck.mode = CkptOpts::kList;
  ck.pos = ckpt_pos;
  ck.cu = cu_ckpt;
  ck.n = n_ckpt;
  ck.states = ckpt_states;
  ck.bytes = ckpt_bytes;
  return prefill_varlen(q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen,
                        initial_state, final_state, o, H, Dk, Dv, C, scale,
                        dtype, ck, nullptr, workspace, workspace_bytes,
                        stream);
}

kda_status_t kda_prefill_varlen_prologue(
    const void* xq, const void* xk, const void* xv, const float* conv_w,
    const float* a, const float* b, const int32_t* cu_seqlens, int32_t N,
    int64_t total_T, int32_t max_seqlen, const float* initial_state,
    float* final_state, void* o, int32_t H, int32_t Dk, int32_t Dv, int32_t C,
    float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (!conv_w || !aligned(conv_w, 16)) return KDA_ERR_INVALID_ARG;
  return prefill_varlen(xq, xk, xv, a, b, cu_seqlens, N, total_T, max_seqlen,
                        initial_state, final_state, o, H, Dk, Dv, C, scale,
                        dtype, CkptOpts{}, conv_w, workspace,
                        workspace_bytes, stream);
}

kda_status_t kda_decode_step(const void* q, const void* k, const void* v,
                             const float* g, const float* beta, float* state,
                             void* o, int32_t B, int32_t H, int32_t Dk,
                             int32_t Dv, float scale, int32_t dtype,
                             void* stream) {
  return decode_step(q, k, v, g, beta, state, o, nullptr, nullptr, 0.f, B, H,
                     Dk, Dv, scale, dtype, stream);
}

kda_status_t kda_decode_step_gated(const void* q, const void* k,
                                   const void* v, const float* g,
                                   const float* beta, float* state,
                                   const void* z, const float* w, float eps,
                                   void* y, int32_t B, int32_t H, int32_t Dk,
                                   int32_t Dv, float scale, int32_t dtype,
                                   void* stream) {
  if (!z || !w || !aligned(z, 16) || !aligned(w, 16) || !(eps >= 0.f))
    return KDA_ERR_INVALID_ARG;
  return decode_step(q, k, v, g, beta, state, y, z, w, eps, B, H, Dk, Dv,
                     scale, dtype, stream);
}

kda_status_t kda_output_norm_gate(const void* o, const void* z,
                                  const float* w, float eps, void* y,
                                  int64_t tokens, int32_t H, int32_t Dv,
                                  int32_t dtype, void* stream) {
  if (tokens < 0 || H <= 0 || Dv <= 0 || !(eps >= 0.f))
    return KDA_ERR_INVALID_ARG;
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32)
    return KDA_ERR_UNSUPPORTED;
  if (!supported_dim(Dv)) return KDA_ERR_UNSUPPORTED;
  if (tokens == 0) return KDA_OK;
  if (!o || !z || !w || !y) return KDA_ERR_INVALID_ARG;
  if (!aligned(o, 16) || !aligned(z, 16) || !aligned(w, 16) ||
      !aligned(y, 16))
    return KDA_ERR_INVALID_ARG;
  const int64_t rows = tokens * H;
  // the grid covers rows in groups of 256 / (D / 4), D the tile
  const int32_t D = tile_dim(Dv, Dv);
  if (rows / (1024 / D) >= ((int64_t)1 << 31)) return KDA_ERR_UNSUPPORTED;
  kda::EpilogueArgs a{};
  a.o = o; a.z = z; a.w = w; a.y = y;
  a.rows = rows;
  a.dv = Dv;
  a.eps = eps;
  if (kda::launch_epilogue(a, D, dtype == KDA_DTYPE_BF16,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_LAUNCH;
  return KDA_OK;
}

kda_status_t kda_spec_verify(const void* q, const void* k, const void* v,
                             const float* g, const float* beta,
                             const float* state, void* o, float* u, int32_t B,
                             int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                             float scale, int32_t dtype, void* stream) {
  if (B <= 0 || H <= 0 || T <= 0 || Dk <= 0 || Dv <= 0)
    return KDA_ERR_INVALID_ARG;
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32)
    return KDA_ERR_UNSUPPORTED;
  if (!supported_dims(Dk, Dv) || T > kda::max_spec_tokens())
    return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > INT_MAX) return KDA_ERR_UNSUPPORTED;
  kda_status_t st = check_tensors((int64_t)B * T, q, k, v, g, beta, o);
  if (st != KDA_OK) return st;
  if (!state || !aligned(state, 16) || !u || !aligned(u, 16))
    return KDA_ERR_INVALID_ARG;
  kda::SpecArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.state = const_cast<float*>(state);
  a.o = o;
  a.u = u;
  a.B = B; a.T = T; a.H = H;
  a.dk = Dk; a.dv = Dv;
  a.scale = scale;
  if (kda::launch_spec(a, tile_dim(Dk, Dv), dtype == KDA_DTYPE_BF16,
                       kda::SpecMode::kVerify,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_LAUNCH;
  return KDA_OK;
}

kda_status_t kda_spec_commit(const void* k, const float* g, const float* u,
                             const int32_t* accepted, float* state, int32_t B,
                             int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                             int32_t dtype, void* stream) {
  if (B <= 0 || H <= 0 || T <= 0 || Dk <= 0 || Dv <= 0)
    return KDA_ERR_INVALID_ARG;
  if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_FP32)
    return KDA_ERR_UNSUPPORTED;
  if (!supported_dims(Dk, Dv) || T > kda::max_spec_tokens())
    return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > INT_MAX) return KDA_ERR_UNSUPPORTED;
  if (!k || !g || !u || !accepted || !state) return KDA_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(g, 16) || !aligned(u, 16) ||
      !aligned(state, 16) || !aligned(accepted, 4))
    return KDA_ERR_INVALID_ARG;
  kda::SpecArgs a{};
  a.k = k; a.g = g;
  a.u = const_cast<float*>(u);
  a.accepted = accepted;
  a.state = state;
  a.B = B; a.T = T; a.H = H;
  a.dk = Dk; a.dv = Dv;
  if (kda::launch_spec(a, tile_dim(Dk, Dv), dtype == KDA_DTYPE_BF16,
                       kda::SpecMode::kCommit,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_LAUNCH;
  return KDA_OK;
}

kda_status_t kda_spec_step(const void* k_prev, const float* g_prev,
                           const float* u_prev, const int32_t* accepted_prev,
                           int32_t T_prev, const void* q, const void* k,
                           const void* v, const float* g, const float* beta,
                           float* state, void* o, float* u, int32_t B,
                           int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                           float scale, int32_t dtype, void* stream) {
  return spec_step(k_prev, g_prev, u_prev, accepted_prev, T_prev, q, k, v, g,
                   beta, state, o, u, B, T, H, Dk, Dv, scale, dtype, stream,
                   nullptr, 0);
}

kda_status_t kda_spec_step_indexed(
    const void* k_prev, const float* g_prev, const float* u_prev,
    const int32_t* accepted_prev, int32_t T_prev, const void* q,
    const void* k, const void* v, const float* g, const float* beta,
    float* state_pool, const int32_t* state_idx, int32_t pool_slots, void* o,
    float* u, int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
    float scale, int32_t dtype, void* stream) {
  if (pool_slots <= 0 || !state_idx || !aligned(state_idx, 4))
    return KDA_ERR_INVALID_ARG;
  return spec_step(k_prev, g_prev, u_prev, accepted_prev, T_prev, q, k, v, g,
                   beta, state_pool, o, u, B, T, H, Dk, Dv, scale, dtype,
                   stream, state_idx, pool_slots);
}

kda_status_t kda_decode_step_gated_indexed(
    const void* q, const void* k, const void* v, const float* g,
    const float* beta, float* state_pool, const int32_t* state_idx,
    int32_t pool_slots, const void* z, const float* w, float eps, void* y,
    int32_t B, int32_t H, int32_t Dk, int32_t Dv, float scale, int32_t dtype,
    void* stream) {
  if (pool_slots <= 0 || !state_idx || !aligned(state_idx, 4))
    return KDA_ERR_INVALID_ARG;
  if (!z || !w || !aligned(z, 16) || !aligned(w, 16) || !(eps >= 0.f))
    return KDA_ERR_INVALID_ARG;
  return decode_step(q, k, v, g, beta, state_pool, y, z, w, eps, B, H, Dk, Dv,
                     scale, dtype, stream, state_idx, pool_slots);
}

kda_status_t kda_decode_step_indexed(const void* q, const void* k,
                                     const void* v, const float* g,
                                     const float* beta, float* state_pool,
                                     const int32_t* state_idx,
                                     int32_t pool_slots, void* o, int32_t B,
                                     int32_t H, int32_t Dk, int32_t Dv,
                                     float scale, int32_t dtype,
                                     void* stream) {
  if (pool_slots <= 0 || !state_idx || !aligned(state_idx, 4))
    return KDA_ERR_INVALID_ARG;
  return decode_step(q, k, v, g, beta, state_pool, o, nullptr, nullptr, 0.f,
                     B, H, Dk, Dv, scale, dtype, stream, state_idx,
                     pool_slots);
}

kda_status_t kda_prefill_varlen_indexed(
    const void* q, const void* k, const void* v, const float* g,
    const float* beta, const int32_t* cu_seqlens, int32_t N, int64_t total_T,
    int32_t max_seqlen, float* state_pool, const int32_t* state_idx,
    const int32_t* has_initial, int32_t pool_slots, void* o, int32_t H,
    int32_t Dk, int32_t Dv, int32_t C, float scale, int32_t dtype,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (pool_slots <= 0 || !state_pool || !state_idx || !aligned(state_idx, 4) ||
      (has_initial && !aligned(has_initial, 4)))
    return KDA_ERR_INVALID_ARG;
  PoolOpts pool;
  pool.idx = state_idx;
  pool.has_initial = has_initial;
  pool.slots = pool_slots;
  return prefill_varlen(q, k, v, g, beta, cu_seqlens, N, total_T, max_seqlen,
                        state_pool, state_pool, o, H, Dk, Dv, C, scale, dtype,
                        CkptOpts{}, nullptr, workspace, workspace_bytes,
                        stream, kStagesBoth, false, nullptr, nullptr, 0.f,
                        pool);
}

}  // extern "C"
