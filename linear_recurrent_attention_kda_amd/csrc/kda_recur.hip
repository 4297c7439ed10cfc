// Chunk-recurrence kernel: the sequential part of chunked prefill.
// "Kimi K3: The Manos, The Mythos, The Legendos" (SemiAnalysis), section
// "FlashKDA algorithm": the second kernel runs the chunk-level recurrence
// over the tensors the chunk-prep kernel wrote.  Per chunk, with the fp32
// state S (d_k x d_v) entering the chunk:
//
//   U  = U~ - W S                      (pseudo-values of the chunk)
//   O  = scale * (Q^ S + M U)          (outputs of the chunk's tokens)
//   S <- diag(gamma) S + K-bar^T U     (state after the chunk)
//
// Columns of S evolve independently, so one workgroup owns a BV-wide slice
// of d_v for one (sequence, head) and walks that sequence's chunks in
// order.  The slice stays in MFMA accumulators (fp32) for the whole
// sequence; its bf16 copy in LDS is the matrix-core operand.  The three
// C x D by D x BV products and the C x C by C x BV product use
// v_mfma_f32_16x16x32_bf16; the g >= -5 bound keeps every operand that the
// chunk-prep kernel scaled inside the bf16 range ("Two Paths: Kimi K3 vs
// DeepSeek V4 Architecture Divergence", section "Hardware Adaptation").
//
// Launch: one workgroup per (d_v slice, head, sequence), 256 threads.  On
// MI355X consecutive workgroup ids go round-robin over the 8 XCDs (each with
// its own L2); ids are remapped so that the slices of one head run on one
// XCD and share its L2 copy of the head's chunk tensors.
#include <atomic>

#include "kda_device.hpp"

namespace kda {
namespace {

// Operands of one chunk that one wave needs, loaded straight into registers
// in MFMA operand layout.  Wave w owns U/O row tile m (all its jt tiles) and
// state tiles ct0 .. ct0 + NCT - 1, so no two waves of a workgroup load the
// same bytes.
template <int KSTEPS, int CSTEPS, int UPW, int NCT>
struct ChunkOps {
  bf16x8 w[KSTEPS], qh[KSTEPS];   // rows of W and Q^ (row tile m)
  bf16x8 m[CSTEPS];               // row tile m of M
  bf16x8 kb[NCT][CSTEPS];         // rows of K-bar^T (state row tiles)
  uint2 ut[UPW];                  // U~^T, 4 rows of one column per tile
  float4 gm[NCT];                 // gamma for the 4 state rows of the lane
};

// XCD-aware block id.  Workgroup b runs on XCD b % 8 (round-robin
// dispatch).  Logical id = pair * nvt + slice, pair = sequence * H + head.
// The slices of one (sequence, head) pair run on one XCD and share its L2,
// and the pairs are dealt to the XCDs in turn (pair p on XCD p % 8), so every
// XCD gets the same share of every sequence, whatever the sequence lengths.
// Without a multiple of 8 pairs the ids are used as they are.
__device__ __forceinline__ unsigned xcd_logical_id(unsigned b, unsigned total,
                                                   unsigned nvt) {
  const unsigned pairs = total / nvt;
  if ((pairs & 7u) != 0u) return b;
  const unsigned x = b & 7u, k = b >> 3;
  return (x + 8u * (k / nvt)) * nvt + k % nvt;
}

template <typename Tout, int D, int C, int BV, int PF, int NW, bool kCkpt,
          bool kGated>
__global__ __launch_bounds__(64 * NW) void recur_kernel(PrefillArgs a) {
  constexpr int K = D, V = D;
  constexpr int NVT = V / BV;              // d_v slices per head
  constexpr int KT = K / 16, JT = BV / 16; // 16x16 tiles of the slice
  constexpr int NST = KT * JT;             // state tiles
  constexpr int SPW = (NST + NW - 1) / NW; // state tiles per wave
  constexpr int MT = C / 16;               // 16-row tiles of a chunk
  constexpr int NUT = MT * JT;             // U / O tiles per chunk
  constexpr int UPW = (NUT + NW - 1) / NW; // U / O tiles per wave
  constexpr int NCT = SPW >= JT ? SPW / JT : 1;  // state row tiles per wave
  constexpr int KSTEPS = (K + 31) / 32;
  constexpr int CSTEPS = (C + 31) / 32;
  constexpr int SP = K + 8, UP = C + 8;    // padded LDS strides (bf16)
  static_assert(V % BV == 0 && BV % 16 == 0, "slice width");
  static_assert(UPW <= JT && (SPW % JT == 0 || SPW < JT), "wave tiling");
  static_assert(!kGated || BV == V, "the fused epilogue needs whole rows");
  using Ops = ChunkOps<KSTEPS, CSTEPS, UPW, NCT>;

  __shared__ __attribute__((aligned(16))) bf16 s_SbT[BV][SP];  // S^T, bf16
  __shared__ __attribute__((aligned(16))) bf16 s_UbT[BV][UP];  // U^T, bf16
  // fused epilogue: per-wave row sums of squares, when a row's columns are
  // spread over several waves
  __shared__ float s_ss[kGated && UPW < JT ? NW : 1][16];

  const unsigned bid = xcd_logical_id(blockIdx.x, gridDim.x, NVT);
  const int vt = bid % NVT;
  const int h = (bid / NVT) % a.H;
  const int n = bid / (NVT * a.H);
  const int j0 = vt * BV;
  const int H = a.H;
  // the stored state and output rows hold dk x dv and dv channels (<= D):
  // a slice entirely past dv has nothing to do; padded rows and columns are
  // zero in the accumulators and never stored
  const int dk = a.dk, dv = a.dv;
  if (j0 >= dv) return;  // uniform over the workgroup

  int64_t bos, eos;
  seq_bounds(a, n, bos, eos);
  const WsLayout lay = WsLayout::make(C, K, V);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = lane & 15, kg = lane >> 4;

  // this wave's tiles
  const int u0 = wave * UPW;                 // first U/O tile
  const bool has_u = u0 < NUT;
  const int mrow = has_u ? u0 / JT : 0;      // its row tile
  const int s0t = wave * SPW;                // first state tile
  const int ct0 = s0t / JT;
  const bool has_s = s0t < NST;

  // For the production shapes every lane guard below is a compile-time
  // "true", so the loop's loads and stores are branch-free and the compiler
  // can count outstanding memory operations exactly (a branch makes it wait
  // for all of them, which would serialise the prefetch).
  constexpr bool kFullK = K % 32 == 0;      // every lane's column group < K
  constexpr bool kFullC = C % 32 == 0;      // every lane's row group < C
  constexpr bool kAllU = NUT % NW == 0;     // every wave owns U/O tiles
  constexpr bool kAllS = NST % NW == 0;     // every wave owns state tiles

  // ---- initial state -> accumulators (D layout: row c = 16ct + 4kg + e,
  //      column j = 16jt + rl) and its bf16 copy -----------------------------
  f32x4 S[SPW];
  const StateSlot slot = state_slot(a, n, h, dk, dv);
  const size_t sbase = slot.base;
  // element (row, col) of a stored dk x dv state slice, -1 when padded
  auto sidx = [&](int row, int col) -> int64_t {
    return (row < dk && col < dv) ? (int64_t)row * dv + col : -1;
  };
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = s0t + i;
    S[i] = zero4();
    if (t < NST) {
      const int ct = t / JT, jt = t % JT;
      if (slot.load) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t ix = sidx(16 * ct + 4 * kg + e, j0 + 16 * jt + rl);
          S[i][e] = ix >= 0 ? a.initial_state[sbase + ix] : 0.f;
        }
      }
      bf16x4 sb;
#pragma unroll
      for (int e = 0; e < 4; ++e) sb[e] = (bf16)S[i][e];
      *reinterpret_cast<bf16x4*>(&s_SbT[16 * jt + rl][16 * ct + 4 * kg]) = sb;
    }
  }

  const int64_t nchunks = seq_chunks(a, bos, eos, C);
  const char* ws_head = a.ws + (size_t)h * a.nslots * lay.block_bytes;
  CkptCursor ck;
  if (kCkpt) ck.init(a, n, bos, eos);

  // Loads of chunk ci's operands, in three groups issued as soon as the
  // registers they fill are free: W, Q^ and U~ (read by the U phase), M (the
  // O phase), K-bar^T and gamma (the state update).  Spreading them lets the
  // address unit work through one group while the wave computes.  ci is
  // clamped to the last chunk (a harmless duplicate load) instead of
  // branching.
  struct Blk {
    const bf16 *W, *Qh, *KbT, *UtT, *M;
    const float* G;
  };
  auto chunk_blk = [&](int64_t ci) {
    ci = ci < nchunks ? ci : nchunks - 1;
    const int64_t slot = (bos + ci * C) / C + n;
    const char* blk = ws_head + (size_t)slot * lay.block_bytes;
    Blk b;
    b.W = reinterpret_cast<const bf16*>(blk + lay.off_W);
    b.Qh = reinterpret_cast<const bf16*>(blk + lay.off_Qh);
    b.KbT = reinterpret_cast<const bf16*>(blk + lay.off_KbT);
    b.UtT = reinterpret_cast<const bf16*>(blk + lay.off_UtT);
    b.M = reinterpret_cast<const bf16*>(blk + lay.off_M);
    b.G = reinterpret_cast<const float*>(blk + lay.off_gamma);
    return b;
  };
  auto load_u = [&](Ops& op, const Blk& b) {
    if (kAllU || has_u) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int c0 = 32 * kk + 8 * kg;
        if (kFullK || c0 < K) {
          // fragment (mrow, kk), this lane's 16 bytes: one contiguous 1 KB
          op.w[kk] = load_bf16x8(b.W + ((mrow * lay.kst + kk) * 64 + lane) * 8);
          op.qh[kk] = load_bf16x8(b.Qh + ((mrow * lay.kst + kk) * 64 + lane) * 8);
        }
      }
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        const int jt = (u0 + i) % JT;
        if (kAllU || u0 + i < NUT)
          op.ut[i] = *reinterpret_cast<const uint2*>(
              b.UtT + ((((j0 >> 4) + jt) * lay.mt + mrow) * 64 + lane) * 4);
      }
    }
  };
  auto load_m = [&](Ops& op, const Blk& b) {
    if (kAllU || has_u) {
#pragma unroll
      for (int cs = 0; cs < CSTEPS; ++cs) {
        const int s0 = 32 * cs + 8 * kg;   // M is zero above the diagonal
        if (kFullC || s0 < C)
          // (fragments with 2 cs > mrow are never written, and the product
          // below skips them; the load stays branch-free)
          op.m[cs] = load_bf16x8(b.M + ((mrow * lay.cst + cs) * 64 + lane) * 8);
      }
    }
  };
  auto load_s = [&](Ops& op, const Blk& b) {
    if (kAllS || has_s) {
#pragma unroll
      for (int lc = 0; lc < NCT; ++lc) {
        const int ct = ct0 + lc;
#pragma unroll
        for (int cs = 0; cs < CSTEPS; ++cs) {
          const int s0 = 32 * cs + 8 * kg;
          if (kFullC || s0 < C)
            op.kb[lc][cs] =
                load_bf16x8(b.KbT + ((ct * lay.cst + cs) * 64 + lane) * 8);
        }
        op.gm[lc] = *reinterpret_cast<const float4*>(b.G + 16 * ct + 4 * kg);
      }
    }
  };
  auto load_ops = [&](Ops& op, int64_t ci) {
    const Blk b = chunk_blk(ci);
    load_u(op, b);
    load_m(op, b);
    load_s(op, b);
  };

  Tout* o = static_cast<Tout*>(a.o);
  // byte offset of this lane's 4 outputs in row r, tile jt of the chunk's
  // output buffer (base at column j0), or out of range past dv
  auto ooff = [&](int r, int jt) -> uint32_t {
    return j0 + 16 * jt + 4 * kg < dv
               ? (uint32_t)(((int64_t)r * H * dv + 16 * jt + 4 * kg) *
                            sizeof(Tout))
               : kOffNone;
  };

  // One chunk of the recurrence with its operands already in registers;
  // each operand group is refilled with chunk `next` once consumed.
  auto process = [&](Ops& op, int64_t ci, int64_t next) {
    const Blk nb = chunk_blk(next);
    const int64_t t0 = bos + ci * C;
    const int L = (eos - t0) < C ? (int)(eos - t0) : C;
    // outputs of this chunk and slice: rows r < L at stride H*V elements
    const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(
        o + (t0 * H + h) * (int64_t)dv + j0,
        (uint32_t)(((int64_t)(L - 1) * H * dv + BV) * sizeof(Tout)));
    __syncthreads();  // S^T copy complete; U^T buffer free

    // U = U~ - W S,  O^T = S^T Q^^T.  Every S^T fragment of the phase is
    // read before the first product so that the LDS latencies overlap.
    bf16x8 sbf[UPW][KSTEPS];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int jt = (u0 + i) % JT;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        // per-lane guards only select operands; every lane runs the MFMA
        const int c0 = 32 * kk + 8 * kg;
        sbf[i][kk] = zero_bf16x8();
        if ((kAllU || u0 + i < NUT) && (kFullK || c0 < K))
          sbf[i][kk] = *reinterpret_cast<const bf16x8*>(&s_SbT[16 * jt + rl][c0]);
      }
    }
    f32x4 Ot[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      Ot[i] = zero4();
      if (kAllU || u0 + i < NUT) {
        const int jt = (u0 + i) % JT;
        f32x4 wsacc = zero4();
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          wsacc = mfma_bf16(op.w[kk], sbf[i][kk], wsacc);
          Ot[i] = mfma_bf16(sbf[i][kk], op.qh[kk], Ot[i]);
        }
        const bf16x4 ut = __builtin_bit_cast(bf16x4, op.ut[i]);
        bf16x4 ub;
#pragma unroll
        for (int e = 0; e < 4; ++e) ub[e] = (bf16)((float)ut[e] - wsacc[e]);
        *reinterpret_cast<bf16x4*>(&s_UbT[16 * jt + rl][16 * mrow + 4 * kg]) =
            ub;
      }
    }
    load_u(op, nb);
    __syncthreads();  // U^T complete

    // U^T fragments, read once for both products below
    bf16x8 ubf[JT][CSTEPS];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
#pragma unroll
      for (int cs = 0; cs < CSTEPS; ++cs) {
        const int s0 = 32 * cs + 8 * kg;
        ubf[jt][cs] = zero_bf16x8();
        if (kFullC || s0 < C)
          ubf[jt][cs] = *reinterpret_cast<const bf16x8*>(&s_UbT[16 * jt + rl][s0]);
      }
    }

    // fused epilogue: the gate pre-activations and weights of this wave's
    // outputs, issued before the products that finish them
    f32x4 zg[kGated ? UPW : 1], wg[kGated ? UPW : 1];
    if constexpr (kGated) {
      const __amdgpu_buffer_rsrc_t zrsrc = make_rsrc(
          static_cast<const Tout*>(a.gate_z) + (t0 * H + h) * (int64_t)dv,
          (uint32_t)(((int64_t)(L - 1) * H * dv + dv) * sizeof(Tout)));
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        const int jt = (u0 + i) % JT;
        const int r = 16 * mrow + rl;
        zg[i] = load4(static_cast<const Tout*>(nullptr), zrsrc,
                      ooff(r, jt));
        const float4 w4 =
            16 * jt + 4 * kg < dv
                ? *reinterpret_cast<const float4*>(a.gate_w + 16 * jt + 4 * kg)
                : make_float4(0.f, 0.f, 0.f, 0.f);
        wg[i] = f32x4{w4.x, w4.y, w4.z, w4.w};
      }
    }

    // O^T += U^T M^T; store O (rows >= L fall outside the buffer: dropped)
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      if (kAllU || u0 + i < NUT) {
        const int jt = (u0 + i) % JT;
#pragma unroll
        for (int cs = 0; cs < CSTEPS; ++cs)
          if (2 * cs <= mrow)  // M is zero right of that
            Ot[i] = mfma_bf16(ubf[jt][cs], op.m[cs], Ot[i]);
        if constexpr (!kGated) {
          const int r = 16 * mrow + rl;
          buffer_store4(o, orsrc,
                        ooff(r, jt),
                        Ot[i], a.scale);
        }
      }
    }
    if constexpr (kGated) {
      // y = o rsqrt(mean(o^2) + eps) w sigmoid(z) per (token, head) row
      // ("Kimi K3: The Manos, The Mythos, The Legendos", section "Kimi
      // Linear": per-head output norm and output gate).  Lane (rl, kg)
      // holds columns 16 jt + 4 kg .. + 3 of row 16 mrow + rl.
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        if (kAllU || u0 + i < NUT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = Ot[i][e] * a.scale;
            ss += x * x;
          }
        }
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      if constexpr (UPW < JT) {
        // the row's other columns belong to the waves with the same row
        // tile: add their partial sums through LDS
        if (kg == 0) s_ss[wave][rl] = (kAllU || has_u) ? ss : 0.f;
        __syncthreads();
        ss = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2)
          if (w2 * UPW < NUT && (w2 * UPW) / JT == mrow) ss += s_ss[w2][rl];
      }
      const float rn = rsqrtf(ss / (float)dv + a.gate_eps);
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        if (kAllU || u0 + i < NUT) {
          const int jt = (u0 + i) % JT;
          const int r = 16 * mrow + rl;
          f32x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gate = __builtin_amdgcn_rcpf(
                1.f + __builtin_amdgcn_exp2f(-zg[i][e] * kLog2e));
            y[e] = Ot[i][e] * a.scale * rn * wg[i][e] * gate;
          }
          buffer_store4(o, orsrc,
                        ooff(r, jt),
                        y, 1.f);
        }
      }
    }
    load_m(op, nb);

    // S <- diag(gamma) S + K-bar^T U
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = s0t + i;
      if (kAllS || t < NST) {
        // tiles s0t .. s0t + SPW - 1 cover whole rows ct0 .. ct0 + NCT - 1
        // (or part of one row when SPW < JT)
        constexpr bool kRows = SPW >= JT;
        const int lc = kRows ? i / JT : 0;
        const int jt = kRows ? i % JT : t % JT;
        const int ct = ct0 + lc;
        const float4 gm = op.gm[lc];
        S[i][0] *= gm.x; S[i][1] *= gm.y; S[i][2] *= gm.z; S[i][3] *= gm.w;
#pragma unroll
        for (int cs = 0; cs < CSTEPS; ++cs)
          S[i] = mfma_bf16(op.kb[lc][cs], ubf[jt][cs], S[i]);
        bf16x4 sb;
#pragma unroll
        for (int e = 0; e < 4; ++e) sb[e] = (bf16)S[i][e];
        *reinterpret_cast<bf16x4*>(&s_SbT[16 * jt + rl][16 * ct + 4 * kg]) = sb;
      }
    }
    // state checkpoints after this chunk: "Kimi K3: The Manos, The Mythos,
    // The Legendos", section "KDA prefix cache management".  The condition
    // is uniform over the workgroup.
    if (kCkpt) {
      const int64_t done = (ci + 1) * C < eos - bos ? (ci + 1) * C : eos - bos;
      while (ck.due(done)) {
        float* dst = a.ckpt_states + ((size_t)ck.slot * H + h) * (size_t)dk * dv;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
          const int t = s0t + i;
          if (kAllS || t < NST) {
            const int ct = t / JT, jt = t % JT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int64_t ix = sidx(16 * ct + 4 * kg + e, j0 + 16 * jt + rl);
              if (ix >= 0) dst[ix] = S[i][e];
            }
          }
        }
        ck.next();
      }
    }
    load_s(op, nb);
  };

  // PF register sets: chunk ci computes while chunks ci + 1 .. ci + PF - 1
  // are in flight; the set freed by ci is refilled with ci + PF.
  Ops ops[PF];
#pragma unroll
  for (int f = 0; f < PF; ++f) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) ops[f].w[kk] = ops[f].qh[kk] = zero_bf16x8();
#pragma unroll
    for (int cs = 0; cs < CSTEPS; ++cs) {
      ops[f].m[cs] = zero_bf16x8();
#pragma unroll
      for (int lc = 0; lc < NCT; ++lc) ops[f].kb[lc][cs] = zero_bf16x8();
    }
#pragma unroll
    for (int i = 0; i < UPW; ++i) ops[f].ut[i] = make_uint2(0u, 0u);
#pragma unroll
    for (int lc = 0; lc < NCT; ++lc)
      ops[f].gm[lc] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // The loop body has no branch, so every path into its header agrees on
  // the order of outstanding loads and the compiler waits only for the set
  // it is about to use.
  if (nchunks > 0) {
#pragma unroll
    for (int f = 0; f < PF; ++f) load_ops(ops[f], f);
    int64_t ci = 0;
    for (; ci + PF <= nchunks; ci += PF) {
#pragma unroll
      for (int f = 0; f < PF; ++f) process(ops[f], ci + f, ci + f + PF);
    }
#pragma unroll
    for (int f = 0; f < PF - 1; ++f)
      if (ci + f < nchunks) process(ops[f], ci + f, ci + f + PF);
  }

  if (slot.store) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = s0t + i;
      if (t < NST) {
        const int ct = t / JT, jt = t % JT;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t ix = sidx(16 * ct + 4 * kg + e, j0 + 16 * jt + rl);
          if (ix >= 0) a.final_state[sbase + ix] = S[i][e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Streamed variant: a fifth wave copies each chunk's operands from the
// workspace into one of two LDS buffers with LDS-direct loads
// (global_load_lds: every lane's 16 bytes land at the buffer offset plus
// 16 x lane, so one instruction moves one contiguous 1 KB fragment), and
// the four compute waves read them with 16-byte LDS reads.  The compute
// waves then issue no global loads at all: the address unit's back-pressure
// and the loads' latency fall on the loader wave.
//
// Operands of chunk ci are split in two parts by when they are consumed:
//   part A: W, Q^ and this slice's U~^T   (read before the mid-chunk barrier)
//   part B: K-bar^T, M and gamma           (read after it)
// With X_ci / Y_ci the chunk's first / mid-chunk barrier, the loader issues
// part B of chunk ci + 1 after X_ci (its buffer's previous part B, chunk
// ci - 1's, was consumed before X_ci) and part A of chunk ci + 2 after Y_ci
// (chunk ci's part A was consumed before Y_ci), then waits until only that
// last part A is outstanding, so that both parts of chunk ci + 1 have landed
// before X_ci+1.  Loads complete in order for the counter, so one wait
// with the count of part A's instructions does this.
template <int D, int C, int BV>
struct OpBuf {
  static constexpr int MT = C / 16, KST = D / 32, CST = C / 32, KT = D / 16;
  static constexpr int JT = BV / 16;
  static constexpr int W = 0;                          // MT*KST fragments
  static constexpr int QH = W + MT * KST * 1024;       // MT*KST fragments
  static constexpr int KB = QH + MT * KST * 1024;      // KT*CST fragments
  static constexpr int M = KB + KT * CST * 1024;       // MT*CST fragments
  static constexpr int U = M + MT * CST * 1024;        // JT*MT of 512 B
  static constexpr int G = U + JT * MT * 512;          // D floats
  static constexpr int BYTES = G + D * 4;
  static constexpr int NA = 2 * MT * KST + JT * MT / 2;  // part A copies
  static_assert(D % 32 == 0 && C % 32 == 0 && (JT * MT) % 2 == 0 &&
                D % 64 == 0, "streamed operand layout");
  static_assert(NA <= 63, "one counter wait covers part A");
};

template <typename Tout, int D, int C, int BV, bool kCkpt>
__global__ __launch_bounds__(320, 1) void recur_stream_kernel(PrefillArgs a) {
  constexpr int NW = 4;                    // compute waves; wave 4 loads
  constexpr int K = D, V = D;
  constexpr int NVT = V / BV;
  constexpr int KT = K / 16, JT = BV / 16;
  constexpr int NST = KT * JT;
  constexpr int SPW = NST / NW;
  constexpr int MT = C / 16;
  constexpr int NUT = MT * JT;
  constexpr int UPW = NUT / NW;
  constexpr int NCT = SPW >= JT ? SPW / JT : 1;
  constexpr int KSTEPS = K / 32, CSTEPS = C / 32;
  constexpr int SP = K + 8, UP = C + 8;
  using OB = OpBuf<D, C, BV>;
  static_assert(NUT % NW == 0 && NST % NW == 0 && UPW <= JT &&
                (SPW % JT == 0 || SPW < JT), "wave tiling");
  static_assert(2 * OB::BYTES + (BV * SP + BV * UP) * 2 <= 160 * 1024,
                "LDS budget");

  __shared__ __attribute__((aligned(16))) bf16 s_SbT[BV][SP];
  __shared__ __attribute__((aligned(16))) bf16 s_UbT[BV][UP];
  __shared__ __attribute__((aligned(1024))) char s_ops[2][OB::BYTES];

  const unsigned bid = xcd_logical_id(blockIdx.x, gridDim.x, NVT);
  const int vt = bid % NVT;
  const int h = (bid / NVT) % a.H;
  const int n = bid / (NVT * a.H);
  const int j0 = vt * BV;
  const int H = a.H;
  // stored dims (<= D); see recur_kernel
  const int dk = a.dk, dv = a.dv;
  if (j0 >= dv) return;  // uniform: every wave, the loader included

  int64_t bos, eos;
  seq_bounds(a, n, bos, eos);
  const WsLayout lay = WsLayout::make(C, K, V);
  const int64_t nchunks = seq_chunks(a, bos, eos, C);
  const char* ws_head = a.ws + (size_t)h * a.nslots * lay.block_bytes;
  auto chunk_ptr = [&](int64_t ci) {
    ci = ci < nchunks ? ci : nchunks - 1;  // past the end: a harmless reload
    const int64_t slot = (bos + ci * C) / C + n;
    return ws_head + (size_t)slot * lay.block_bytes;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (wave == NW) {
    // ---- loader wave --------------------------------------------------
    auto copy1k = [&](const char* src, int dst) {
      copy16_to_lds(src + 16 * lane, &s_ops[0][0] + dst);
    };
    auto issue_a = [&](int64_t ci, int b) {
      const char* blk = chunk_ptr(ci);
      const int base = b * OB::BYTES;
#pragma unroll
      for (int f = 0; f < 2 * OB::MT * OB::KST; ++f)
        copy1k(blk + lay.off_W + 1024 * f, base + OB::W + 1024 * f);
      const char* ut = blk + lay.off_UtT + (size_t)(j0 / 16) * lay.mt * 512;
#pragma unroll
      for (int f = 0; f < JT * MT / 2; ++f)
        copy1k(ut + 1024 * f, base + OB::U + 1024 * f);
    };
    auto issue_b = [&](int64_t ci, int b) {
      const char* blk = chunk_ptr(ci);
      const int base = b * OB::BYTES;
#pragma unroll
      for (int f = 0; f < KT * CSTEPS; ++f)
        copy1k(blk + lay.off_KbT + 1024 * f, base + OB::KB + 1024 * f);
#pragma unroll
      for (int f = 0; f < MT * CSTEPS; ++f)  // fragments (m, cs), 2 cs <= m
        if (2 * (f % CSTEPS) <= f / CSTEPS)
          copy1k(blk + lay.off_M + 1024 * f, base + OB::M + 1024 * f);
#pragma unroll
      for (int f = 0; f < D / 64; ++f)  // gamma: 256 B per instruction
        copy4_to_lds(blk + lay.off_gamma + 256 * f + 4 * lane,
                       &s_ops[0][0] + base + OB::G + 256 * f);
    };
    if (nchunks > 0) {
      issue_a(0, 0);
      issue_b(0, 0);
      issue_a(1, 1);
      wait_vmcnt<OB::NA>();                 // chunk 0 has landed
      for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int b = (int)(ci & 1);
        raw_barrier();                      // X_ci
        issue_b(ci + 1, b ^ 1);
        raw_barrier();                      // Y_ci
        issue_a(ci + 2, b);
        wait_vmcnt<OB::NA>();               // chunk ci + 1 has landed
      }
      wait_vmcnt<0>();  // no copy may land after the workgroup's LDS is gone
    }
    return;
  }

  // ---- compute waves ----------------------------------------------------
  CkptCursor ck;
  if (kCkpt) ck.init(a, n, bos, eos);
  const int rl = lane & 15, kg = lane >> 4;
  const int u0 = wave * UPW;
  const int mrow = u0 / JT;
  const int s0t = wave * SPW;
  const int ct0 = s0t / JT;

  f32x4 S[SPW];
  const StateSlot slot = state_slot(a, n, h, dk, dv);
  const size_t sbase = slot.base;
  // element (row, col) of a stored dk x dv state slice, -1 when padded
  auto sidx = [&](int row, int col) -> int64_t {
    return (row < dk && col < dv) ? (int64_t)row * dv + col : -1;
  };
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = s0t + i;
    const int ct = t / JT, jt = t % JT;
    S[i] = zero4();
    if (slot.load) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ix = sidx(16 * ct + 4 * kg + e, j0 + 16 * jt + rl);
        S[i][e] = ix >= 0 ? a.initial_state[sbase + ix] : 0.f;
      }
    }
    bf16x4 sb;
#pragma unroll
    for (int e = 0; e < 4; ++e) sb[e] = (bf16)S[i][e];
    *reinterpret_cast<bf16x4*>(&s_SbT[16 * jt + rl][16 * ct + 4 * kg]) = sb;
  }

  Tout* o = static_cast<Tout*>(a.o);
  auto ooff = [&](int r, int jt) -> uint32_t {  // as in recur_kernel
    return j0 + 16 * jt + 4 * kg < dv
               ? (uint32_t)(((int64_t)r * H * dv + 16 * jt + 4 * kg) *
                            sizeof(Tout))
               : kOffNone;
  };
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const char* ob = &s_ops[ci & 1][0];
    const int64_t t0 = bos + ci * C;
    const int L = (eos - t0) < C ? (int)(eos - t0) : C;
    const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(
        o + (t0 * H + h) * (int64_t)dv + j0,
        (uint32_t)(((int64_t)(L - 1) * H * dv + BV) * sizeof(Tout)));
    __syncthreads();  // X_ci: S^T copy complete, U^T free, operands landed

    // U = U~ - W S,  O^T = S^T Q^^T
    bf16x8 w[KSTEPS], qh[KSTEPS], sbf[UPW][KSTEPS];
    uint2 ut[UPW];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      w[kk] = *reinterpret_cast<const bf16x8*>(
          ob + OB::W + ((mrow * KSTEPS + kk) * 64 + lane) * 16);
      qh[kk] = *reinterpret_cast<const bf16x8*>(
          ob + OB::QH + ((mrow * KSTEPS + kk) * 64 + lane) * 16);
    }
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int jt = (u0 + i) % JT;
      ut[i] = *reinterpret_cast<const uint2*>(
          ob + OB::U + ((jt * MT + mrow) * 64 + lane) * 8);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        sbf[i][kk] = *reinterpret_cast<const bf16x8*>(
            &s_SbT[16 * jt + rl][32 * kk + 8 * kg]);
    }
    f32x4 Ot[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int jt = (u0 + i) % JT;
      f32x4 wsacc = zero4();
      Ot[i] = zero4();
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        wsacc = mfma_bf16(w[kk], sbf[i][kk], wsacc);
        Ot[i] = mfma_bf16(sbf[i][kk], qh[kk], Ot[i]);
      }
      const bf16x4 u4 = __builtin_bit_cast(bf16x4, ut[i]);
      bf16x4 ub;
#pragma unroll
      for (int e = 0; e < 4; ++e) ub[e] = (bf16)((float)u4[e] - wsacc[e]);
      *reinterpret_cast<bf16x4*>(&s_UbT[16 * jt + rl][16 * mrow + 4 * kg]) = ub;
    }
    __syncthreads();  // Y_ci: U^T complete

    bf16x8 ubf[JT][CSTEPS], mf[CSTEPS], kb[NCT][CSTEPS];
    float4 gm[NCT];
#pragma unroll
    for (int cs = 0; cs < CSTEPS; ++cs) {
      mf[cs] = zero_bf16x8();
      if (2 * cs <= mrow)  // the others were not copied (zero)
        mf[cs] = *reinterpret_cast<const bf16x8*>(
            ob + OB::M + ((mrow * CSTEPS + cs) * 64 + lane) * 16);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
        ubf[jt][cs] = *reinterpret_cast<const bf16x8*>(
            &s_UbT[16 * jt + rl][32 * cs + 8 * kg]);
    }
#pragma unroll
    for (int lc = 0; lc < NCT; ++lc) {
      const int ct = ct0 + lc;
#pragma unroll
      for (int cs = 0; cs < CSTEPS; ++cs)
        kb[lc][cs] = *reinterpret_cast<const bf16x8*>(
            ob + OB::KB + ((ct * CSTEPS + cs) * 64 + lane) * 16);
      gm[lc] = *reinterpret_cast<const float4*>(ob + OB::G +
                                                (16 * ct + 4 * kg) * 4);
    }

    // O^T += U^T M^T; store O (rows >= L fall outside the buffer: dropped)
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int jt = (u0 + i) % JT;
#pragma unroll
      for (int cs = 0; cs < CSTEPS; ++cs)
        if (2 * cs <= mrow) Ot[i] = mfma_bf16(ubf[jt][cs], mf[cs], Ot[i]);
      const int r = 16 * mrow + rl;
      buffer_store4(o, orsrc,
                    ooff(r, jt),
                    Ot[i], a.scale);
    }

    // S <- diag(gamma) S + K-bar^T U
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      constexpr bool kRows = SPW >= JT;
      const int t = s0t + i;
      const int lc = kRows ? i / JT : 0;
      const int jt = kRows ? i % JT : t % JT;
      const int ct = ct0 + lc;
      const float4 g4 = gm[lc];
      S[i][0] *= g4.x; S[i][1] *= g4.y; S[i][2] *= g4.z; S[i][3] *= g4.w;
#pragma unroll
      for (int cs = 0; cs < CSTEPS; ++cs)
        S[i] = mfma_bf16(kb[lc][cs], ubf[jt][cs], S[i]);
      bf16x4 sb;
#pragma unroll
      for (int e = 0; e < 4; ++e) sb[e] = (bf16)S[i][e];
      *reinterpret_cast<bf16x4*>(&s_SbT[16 * jt + rl][16 * ct + 4 * kg]) = sb;
    }
    // state checkpoints after this chunk (uniform over the workgroup)
    if (kCkpt) {
      const int64_t done = (ci + 1) * C < eos - bos ? (ci + 1) * C : eos - bos;
      while (ck.due(done)) {
        float* dst = a.ckpt_states + ((size_t)ck.slot * H + h) * (size_t)dk * dv;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
          const int t = s0t + i;
          const int ct = t / JT, jt = t % JT;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t ix = sidx(16 * ct + 4 * kg + e, j0 + 16 * jt + rl);
            if (ix >= 0) dst[ix] = S[i][e];
          }
        }
        ck.next();
      }
    }
  }

  if (slot.store) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = s0t + i;
      const int ct = t / JT, jt = t % JT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ix = sidx(16 * ct + 4 * kg + e, j0 + 16 * jt + rl);
        if (ix >= 0) a.final_state[sbase + ix] = S[i][e];
      }
    }
  }
}

// Slice width.  Wider slices re-read the per-chunk tensors fewer times and
// do more matrix work per chunk loaded; narrower ones give more workgroups
// when there are few (sequence, head) pairs.  Measured on MI355X: 96 heads
// run fastest at 64 (192 workgroups), 32 heads at 16 (256 workgroups);
// 128-wide slices were slower on both.
inline int pick_bv(int D, int64_t units) {
  const int cus = device_cus();
  int bv = 16;
  if (D >= 64 && units * (D / 64) >= cus / 2)
    bv = 64;
  else if (D >= 32 && units * (D / 32) >= cus)
    bv = 32;
  return D == 16 ? 16 : bv;
}

// Two register operand sets in flight and 4 waves per workgroup: a third
// set, or 8 waves (also with the outputs' products given to their own
// waves), measured no faster on MI355X.
// Variant choice for D = 128, C = 64: the streamed variant serves the
// 64-wide slices.  Measured on MI355X: it runs the 96-head prefill workload
// (64-wide slices) in 287 us against 301 us, and the 32-head long workload
// (16-wide slices) 4 % slower.
template <typename Tout, int D, int C, int BV>
hipError_t launch_w(const PrefillArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(D / BV) * (unsigned)a.H * (unsigned)a.N;
  // state checkpoints: their own compile-time variant of each kernel
  if constexpr (D == 128 && C == 64 && BV == 64) {
    return a.ckpt_states
               ? launch_kernel(recur_stream_kernel<Tout, D, C, BV, true>,
                               dim3(blocks), dim3(320), st, a)
               : launch_kernel(recur_stream_kernel<Tout, D, C, BV, false>,
                               dim3(blocks), dim3(320), st, a);
  } else {
    return a.ckpt_states
               ? launch_kernel(recur_kernel<Tout, D, C, BV, 2, 4, true, false>,
                               dim3(blocks), dim3(256), st, a)
               : launch_kernel(recur_kernel<Tout, D, C, BV, 2, 4, false, false>,
                               dim3(blocks), dim3(256), st, a);
  }
}

// Output epilogue fused into the recurrence: the row norm needs every value
// channel of a row in one workgroup, so the slice is all of d_v (one
// workgroup per (sequence, head)).  At d = 128 the whole-row slice keeps one
// operand set in flight (two would spill registers).
template <typename Tout, int D, int C>
hipError_t launch_gated(const PrefillArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)a.H * (unsigned)a.N;
  constexpr int PF = D == 128 ? 1 : 2;
  return launch_kernel(recur_kernel<Tout, D, C, D, PF, 4, false, true>,
                       dim3(blocks), dim3(256), st, a);
}

// Only the slice widths pick_bv can return are instantiated: 64 or 16 at
// D = 128 and 64, 32 or 16 at D = 32, 16 at D = 16.
template <typename Tout, int D, int C>
hipError_t launch(const PrefillArgs& a, hipStream_t st) {
  if (a.gate_z) return launch_gated<Tout, D, C>(a, st);
  const int bv = pick_bv(D, (int64_t)a.N * a.H);
  if constexpr (D >= 64) {
    if (bv == 64) return launch_w<Tout, D, C, 64>(a, st);
  } else if constexpr (D == 32) {
    if (bv == 32) return launch_w<Tout, D, C, 32>(a, st);
  }
  return launch_w<Tout, D, C, 16>(a, st);
}

template <typename Tout, int D>
hipError_t launch_c(const PrefillArgs& a, int C, hipStream_t st) {
  switch (C) {
    case 16: return launch<Tout, D, 16>(a, st);
    case 32: return launch<Tout, D, 32>(a, st);
    case 64: return launch<Tout, D, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename Tout>
hipError_t launch_dc(const PrefillArgs& a, int D, int C, hipStream_t st) {
  switch (D) {
    case 16: return launch_c<Tout, 16>(a, C, st);
    case 32: return launch_c<Tout, 32>(a, C, st);
    case 64: return launch_c<Tout, 64>(a, C, st);
    case 128: return launch_c<Tout, 128>(a, C, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Compute units of the current device, queried once per device and cached
// (the query is not repeated on every launch).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return 256;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

hipError_t launch_recur(const PrefillArgs& a, int D, int C, bool bf16_io,
                        hipStream_t st) {
  return bf16_io ? launch_dc<bf16>(a, D, C, st)
                 : launch_dc<float>(a, D, C, st);
}

}  // namespace kda
