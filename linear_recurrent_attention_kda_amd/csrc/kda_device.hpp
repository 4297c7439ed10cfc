// Device helpers shared by the libkda kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Storage types of q, k, v, o.
template <typename T> struct io;
template <> struct io<bf16> {
  static __device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
  static __device__ __forceinline__ bf16 from_f(float x) { return (bf16)x; }
};
template <> struct io<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};

// Eight consecutive elements of a storage-dtype row as floats (16-byte
// aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const bf16x8 v = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Eight consecutive storage-dtype elements kept raw in registers (a
// prefetch buffer), converted to float on use.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) {
    v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r,
                                           uint32_t off) {
    v = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  __device__ __forceinline__ void zero() {
    v = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  }
  __device__ __forceinline__ void set(const float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
  }
};
template <> struct Raw8<float> {
  float4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const float4*>(p);
    hi = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r,
                                           uint32_t off) {
    lo = __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    hi = __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
  }
  __device__ __forceinline__ void zero() {
    lo = hi = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
    x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
  }
  __device__ __forceinline__ void set(const float (&x)[8]) {
    lo = make_float4(x[0], x[1], x[2], x[3]);
    hi = make_float4(x[4], x[5], x[6], x[7]);
  }
};

// Eight consecutive elements of an LDS row (bf16 or fp32) as floats, and
// the reverse.
__device__ __forceinline__ void lds_get8(const bf16* p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
__device__ __forceinline__ void lds_get8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void lds_put8(bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void lds_put8(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)x[i];
  return r;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}

// D += A(16x32) * B(32x16), bf16 operands, fp32 accumulate.  Lane l holds
// row (l % 16) of A and column (l % 16) of B, each with the 8 contraction
// indices of lane group l / 16 (the same indices for A and B); D element
// (4 * (l / 16) + i, l % 16) is acc[i].
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// D += A(16x4) * B(4x16) in fp32.  Lane l holds A(l % 16, l / 16) and
// B(l / 16, l % 16); D as above.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Buffer resource over [base, base + bytes): buffer loads past the end
// return 0 and buffer stores past the end are dropped by the hardware, which
// lets partial chunks use the same unconditional memory instructions as
// full ones.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes,
                                           0x00020000);
}
// A buffer offset past every buffer the kernels build (each covers less than
// 4 GiB - 256 bytes): a masked lane's load through it returns 0 and its store
// is dropped, without a branch around the memory instruction.
constexpr uint32_t kOffNone = 0xFFFFFF00u;

// Cache-policy operand of the buffer intrinsics on gfx950: the "nt"
// (non-temporal, streaming) bit.
constexpr int kCachePolicyNt = 2;
// Raw buffer loads (out-of-range -> 0).
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r,
                                                 uint32_t off) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ uint4 buffer_load_16(__amdgpu_buffer_rsrc_t r,
                                                uint32_t off) {
  return __builtin_bit_cast(uint4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Four elements x * scale at byte offset `off` of buffer r.
__device__ __forceinline__ void buffer_store4(bf16*, __amdgpu_buffer_rsrc_t r,
                                              uint32_t off, f32x4 x,
                                              float scale) {
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (bf16)(x[i] * scale);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off,
                                        0, 0);
}
__device__ __forceinline__ void buffer_store4(float*, __amdgpu_buffer_rsrc_t r,
                                              uint32_t off, f32x4 x,
                                              float scale) {
  const f32x4 v = x * scale;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off,
                                         0, 0);
}

// Four storage-dtype elements at byte offset `off` of buffer r, as floats
// (out of range: zeros).  The pointer argument only selects the dtype.
__device__ __forceinline__ f32x4 load4(const bf16*, __amdgpu_buffer_rsrc_t r,
                                       uint32_t off) {
  const bf16x4 v = __builtin_bit_cast(
      bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 load4(const float*, __amdgpu_buffer_rsrc_t r,
                                       uint32_t off) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Four consecutive storage-dtype elements (8-byte aligned for bf16, 16-byte
// for fp32) from x * scale.
__device__ __forceinline__ void store4(bf16* p, f32x4 x, float scale) {
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (bf16)(x[i] * scale);
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, f32x4 x, float scale) {
  *reinterpret_cast<float4*>(p) =
      make_float4(x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale);
}

}  // namespace kda

#include "kda_internal.hpp"

namespace kda {

constexpr float kLog2e = 1.4426950408889634f;

// Wait until at most N vector-memory operations of this wave are
// outstanding (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; the
// exp and lgkm counters at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) |
                             (15 << 8));
}

// LDS-direct copies (global_load_lds): lane l's n bytes from src land at
// lds + n * l (n = 16 or 4), so a wave moves one contiguous block per
// instruction.  `lds` must be the same for every lane of the wave.
__device__ __forceinline__ void copy16_to_lds(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
}

// Workgroup barrier without the memory fences of __syncthreads(), for a wave
// that makes its LDS writes visible by waiting on its own counters (the
// empty asm statements keep the compiler from moving memory accesses across).
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Token range [bos, eos) of sequence n, clamped into [0, total_T] so that an
// invalid cu_seqlens can never index outside the packed tensors.
__device__ __forceinline__ void seq_bounds(const PrefillArgs& a, int n,
                                           int64_t& bos, int64_t& eos) {
  if (a.cu_seqlens) {
    int64_t b = a.cu_seqlens[n], e = a.cu_seqlens[n + 1];
    b = b < 0 ? 0 : (b > a.total_T ? a.total_T : b);
    e = e < b ? b : (e > a.total_T ? a.total_T : e);
    bos = b;
    eos = e;
  } else {
    bos = (int64_t)n * a.T_fixed;
    eos = bos + a.T_fixed;
  }
}

// Where sequence n's initial and final states live: row n of the
// [N, H, dk, dv] arrays, or, with a state pool, row state_idx[n] of the
// [pool_slots, H, dk, dv] pool.  A pool slot outside [0, pool_slots) marks
// a padding entry: it starts from zero and no state is read or written for
// it.  has_initial[n] == 0 starts sequence n from zero (its final state is
// still written).  `base` is the element offset of head h's slice.
struct StateSlot {
  size_t base;
  bool load, store;
};
__device__ __forceinline__ StateSlot state_slot(const PrefillArgs& a, int n,
                                                int h, int dk, int dv) {
  int64_t row = n;
  bool ok = true, init = true;
  if (a.state_idx) {
    const int32_t r = a.state_idx[n];
    ok = r >= 0 && r < a.pool_slots;
    row = ok ? r : 0;
    if (a.has_initial) init = a.has_initial[n] != 0;
  }
  StateSlot s;
  s.base = ((size_t)row * a.H + h) * (size_t)dk * dv;
  s.load = ok && init && a.initial_state != nullptr;
  s.store = ok && a.final_state != nullptr;
  return s;
}

// Chunks of sequence [bos, eos) that the recurrence walks: never more than
// the chunk-prep grid covered (max_chunks, from the caller's max_seqlen), so
// a max_seqlen below a sequence's length leaves that sequence's later tokens
// unprocessed instead of reading workspace slots nobody wrote.
__device__ __forceinline__ int64_t seq_chunks(const PrefillArgs& a,
                                              int64_t bos, int64_t eos,
                                              int C) {
  const int64_t n = (eos - bos + C - 1) / C;
  return n < a.max_chunks ? n : a.max_chunks;
}

// State checkpoints of one sequence ("Kimi K3: The Manos, The Mythos, The
// Legendos", section "KDA prefix cache management": the fixed-size state is
// saved every so many tokens and at prompt boundaries).  The recurrence
// holds the state at every chunk boundary.  After each chunk it asks
// `due(done)`, with `done` the tokens of the sequence processed so far (a
// multiple of C, or the sequence length after a partial last chunk), and
// while that is true stores the state to `slot` and calls `next()`.  Every
// member has the same value in all threads of the workgroup.
struct CkptCursor {
  static constexpr int64_t kNone = INT64_MAX;
  const int32_t* pos;  // list mode: ckpt_pos; interval mode: nullptr
  int64_t at;          // tokens done at the pending checkpoint, or kNone
  int64_t slot;        // its slot in ckpt_states
  int64_t len;         // tokens of the sequence
  int32_t every;       // interval mode: the interval
  int32_t j, jend;     // list mode: pending entry of pos, end of the entries

  __device__ __forceinline__ void init(const PrefillArgs& a, int n,
                                       int64_t bos, int64_t eos) {
    pos = a.ckpt_pos;
    len = eos - bos;
    every = a.ckpt_every;
    if (pos) {
      // this sequence's entries, clamped into [0, n_ckpt]
      int32_t b = a.cu_ckpt[n], e = a.cu_ckpt[n + 1];
      b = b < 0 ? 0 : (b > a.n_ckpt ? a.n_ckpt : b);
      e = e < b ? b : (e > a.n_ckpt ? a.n_ckpt : e);
      j = __builtin_amdgcn_readfirstlane(b);
      jend = __builtin_amdgcn_readfirstlane(e);
      load();
    } else {
      j = jend = 0;
      at = every <= len ? every : kNone;
      slot = (bos + every) / every - 1;
    }
  }
  // True when a checkpoint falls exactly at `done` tokens.  List entries
  // that were passed without an exact match (not a multiple of C and not the
  // sequence length, out of increasing order, or <= 0) are skipped and their
  // slots left untouched.
  __device__ __forceinline__ bool due(int64_t done) {
    if (pos) {
      while (at < done) {
        ++j;
        load();
      }
    }
    return at == done;
  }
  __device__ __forceinline__ void next() {
    if (pos) {
      ++j;
      load();
    } else {
      at = at + every <= len ? at + every : kNone;
      slot += 1;
    }
  }

 private:
  __device__ __forceinline__ void load() {
    if (j < jend) {
      at = __builtin_amdgcn_readfirstlane(pos[j]);
      slot = j;
    } else {
      at = kNone;
    }
  }
};

}  // namespace kda
