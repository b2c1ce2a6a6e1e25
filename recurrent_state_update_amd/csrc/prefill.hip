// Chunked (SSD) prefill of packed variable-length sequences, gfx950.
//
// Each sequence is cut into chunks of Q tokens from its first row.  Inside a chunk the output is
// the causally masked product Y = (M o L) X of the Mamba study notes (echobase-5bl.pages.dev,
// "Mamba and Attention"),
//   M[i][j] = (C_i . B_j) exp(a_i - a_j) Delta_j   (j <= i),
// with a the chunk-local cumulative sum of Delta*A, plus exp(a_i) C_i h_in for the state h_in
// entering the chunk; the state leaving a chunk is the affine step
//   h_out = exp(a_last) h_in + sum_j exp(a_last - a_j) Delta_j x_j B_j^T
// that links chunks ("Hybrid SSM / Mamba models and non-KV state", mlinterviewnotes.com ch. 7.3:
// chunked-prefill handoff, affine-composition passage, SSD chunk-scan call site: chunks stitched by
// a small inter-chunk scan).
//
// Two launches on one stream:
//   1. bc_kernel    per (chunk, group): conv + SiLU of the group's B and C channels, Delta and its
//                   chunk-local cumsum for the group's heads, and C B^T of the causal pairs on MFMA
//                   (shared by the group's heads), written as operand planes in the order the
//                   second launch reads them;
//   2. walk_kernel  per (sequence, head, part of the head's channels): walks the sequence's chunks
//                   in order with the running state in MFMA accumulators (the inter-chunk pass on
//                   chip): conv + SiLU of the part's x channels into LDS, the outputs
//                   (C h_in + (M o L) X + D x, gated) and the state update on MFMA, checkpoint and
//                   final states and windows into their slots.
// With SPLIT every product operand is a bf16 hi plane plus a bf16 lo plane and each product
// takes three MFMAs (fp32-level accuracy, used for fp32 state); otherwise operands are single
// bf16 planes with fp32 accumulation.
#include <cstddef>
#include <cstring>
#include <type_traits>

#include "device_common.h"
#include "prefill.h"

namespace m2 {

// Eight consecutive fp32 values -> an io tensor (16-byte aligned position).
__device__ __forceinline__ void store8_any(void* p, int64_t i, int is_bf16, const float (&v)[8]) {
  if (is_bf16) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = from_f32<bf16>(v[e]);
    *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p) + i) = o;
  } else {
    float* d = static_cast<float*>(p) + i;
    *reinterpret_cast<floatx4*>(d) = floatx4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<floatx4*>(d + 4) = floatx4{v[4], v[5], v[6], v[7]};
  }
}

// A wave-uniform read of read-only data (launch tables, per-head parameters) through the
// constant address space, so that it becomes a scalar-memory load: it does not join the
// in-order vector-memory counter that covers prefetches in flight.
template <typename T> __device__ __forceinline__ T load_uniform(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "whole dwords");
  typedef const __attribute__((address_space(4))) int cint;
  const cint* q = (const cint*)p;
  struct W { int w[sizeof(T) / 4]; } w;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) w.w[i] = q[i];
  return __builtin_bit_cast(T, w);
}

// A wave-uniform value the compiler cannot see through.  Folding it into an index inside a
// loop keeps the compiler from hoisting everything derived from that index out of the loop
// (which, for values that are cheap to recompute, costs registers the loop needs).
__device__ __forceinline__ int opaque_uniform(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value, so that
// branches on it are scalar branches rather than exec-masked ones.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }



typedef uint16_t u16;
typedef u16 u16x4 __attribute__((ext_vector_type(4)));
typedef u16 u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ u16 bits_of(bf16 v) { return __builtin_bit_cast(u16, v); }
__device__ __forceinline__ bf16 bf_of(u16 v) { return __builtin_bit_cast(bf16, v); }
__device__ __forceinline__ float f_of(u16 v) { return static_cast<float>(bf_of(v)); }

// fp32 -> (hi, lo) bf16 bit patterns.
__device__ __forceinline__ void split2(float v, u16& hi, u16& lo) {
  const bf16 h = from_f32<bf16>(v);
  hi = bits_of(h);
  lo = bits_of(from_f32<bf16>(v - static_cast<float>(h)));
}

// Two fp32 values -> two bf16 (round to nearest even) in one word, `lo` in the low half (one
// v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2v));
}
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// A fragment from bf16 planes in LDS: row `row`, K positions kb + kmap(q, 0..7).
template <bool SPLIT>
__device__ __forceinline__ Frag<SPLIT> lds_frag(const u16* base, int64_t plane, int ld, int row, int kb, int q) {
  Frag<SPLIT> f;
  const u16* p = base + row * ld + kb + 4 * q;
  const u16x4 a = *reinterpret_cast<const u16x4*>(p);
  const u16x4 b = *reinterpret_cast<const u16x4*>(p + 16);
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.hi[e] = bf_of(a[e]); f.hi[e + 4] = bf_of(b[e]); }
  if (SPLIT) {
    const u16x4 c = *reinterpret_cast<const u16x4*>(p + plane);
    const u16x4 d = *reinterpret_cast<const u16x4*>(p + plane + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.lo[e] = bf_of(c[e]); f.lo[e + 4] = bf_of(d[e]); }
  }
  return f;
}

// A workgroup barrier that orders LDS accesses only: the wave's LDS operations complete before
// it, but its global loads (prefetches) stay in flight across it (a full __syncthreads waits for
// every outstanding global access too).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup b of a launch runs on XCD b % 8 (the dispatcher deals workgroups round-robin over
// the 8 XCDs, each with its own L2).  This maps b to a logical index in units of `unit`
// consecutive indices: unit u runs on XCD u % 8, and each XCD takes its units in order, so work
// listed first starts first on every XCD (a tail of fewer than 8 units keeps the dispatch order).
// A bijection on [0, n), n a multiple of `unit`.
__device__ __forceinline__ int xcd_units(int b, int n, int unit) {
  const int x = b % 8, j = b / 8, rounds = n / (8 * unit);
  if (j >= rounds * unit) return b;
  return (8 * (j / unit) + x) * unit + j % unit;
}

constexpr int kThreads = 512;

// ------------------------------------------------------------------ launch tables
// The packed tables inside the first launch's own kernel arguments.
__device__ __forceinline__ const __attribute__((address_space(4))) unsigned char* arg_tables() {
  typedef const __attribute__((address_space(4))) unsigned char kbyte;
  return (kbyte*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(BcArgs, t);
}

// The walk's PrefillParams argument, read through a pointer the compiler cannot see through:
// fields needed only on rare paths (checkpoints, the end of a sequence) are loaded there instead
// of being held in scalar registers across the whole chunk loop.  (Accesses through pointers read
// this way are flat ones, so the chunk loop's own accesses keep using the argument itself.)
__device__ __forceinline__ PrefillParams opaque_params() {
  typedef const __attribute__((address_space(4))) uint32_t ConstWord;
  ConstWord* p = (ConstWord*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  // a word-wise copy: only the words a caller reads survive, as scalar loads
  PrefillParams r;
  uint32_t* d = reinterpret_cast<uint32_t*>(&r);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(PrefillParams) / 4); ++i) d[i] = p[i];
  return r;
}

// One workgroup of the first launch: copy the tables from the kernel arguments to the workspace,
// where the later launch reads them (tab_inline is a multiple of 16 bytes).
__device__ __forceinline__ void table_copy_block(const PrefillParams& a) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) i32x4 kquad;
  kquad* src = reinterpret_cast<kquad*>(arg_tables());
  i32x4* dst = reinterpret_cast<i32x4*>(const_cast<SeqEntry*>(a.seqs));
  for (int i = threadIdx.x; i < a.tab_inline / 16; i += blockDim.x) dst[i] = src[i];
}

// 2^x as the bare hardware instruction: results below 2^-126 flush to zero, which only drops
// terms that are negligible against the rest of a sum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;

// Position of d_state (or token) index k inside a 32-wide K-step in the permuted storage of the
// operand planes: the 8 values lane l of an MFMA operand holds (K positions kmap(l / 16, 0..7))
// are stored contiguously, at 8 * (l / 16).
__device__ __forceinline__ int perm32(int k) { return ((k & 15) >> 2) * 8 + ((k >> 4) & 1) * 4 + (k & 3); }

// Raw (pre-conv) input of channel col of a token row, 8 consecutive channels.
template <bool IOBF> struct Raw8;
template <> struct Raw8<true> {
  u16x8 v;
  __device__ __forceinline__ void load(const void* p, int64_t i) { v = *reinterpret_cast<const u16x8*>(static_cast<const u16*>(p) + i); }
  __device__ __forceinline__ float at(int e) const { return f_of(v[e]); }
  __device__ __forceinline__ void zero() { v = u16x8{0, 0, 0, 0, 0, 0, 0, 0}; }
};
template <> struct Raw8<false> {
  floatx4 v0, v1;
  __device__ __forceinline__ void load(const void* p, int64_t i) {
    const float* f = static_cast<const float*>(p) + i;
    v0 = *reinterpret_cast<const floatx4*>(f);
    v1 = *reinterpret_cast<const floatx4*>(f + 4);
  }
  __device__ __forceinline__ float at(int e) const { return e < 4 ? v0[e] : v1[e - 4]; }
  __device__ __forceinline__ void zero() { v0 = v1 = floatx4{0.f, 0.f, 0.f, 0.f}; }
};

__device__ __forceinline__ float window_value(const PrefillParams& a, int slot, int cc, int col) {
  const int64_t i = ((int64_t)slot * a.sh.Cd + cc) * (a.sh.W - 1) + col;
  return a.conv_bf16 ? to_f32(static_cast<const bf16*>(a.conv)[i]) : static_cast<const float*>(a.conv)[i];
}
__device__ __forceinline__ void window_store(const PrefillParams& a, int slot, int cc, int col, float v) {
  const int64_t i = ((int64_t)slot * a.sh.Cd + cc) * (a.sh.W - 1) + col;
  if (a.conv_bf16) static_cast<bf16*>(a.conv)[i] = from_f32<bf16>(v);
  else static_cast<float*>(a.conv)[i] = v;
}

// Conv taps of channel cc as four taps applied to rows tau-3 .. tau (a kernel narrower than 4
// gets leading zero taps), and the bias.
__device__ __forceinline__ void taps4(const PrefillParams& a, int cc, float (&w)[4], float& b) {
  const int W = a.sh.W;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = k >= 4 - W ? a.conv_w[(int64_t)cc * W + k - (4 - W)] : 0.f;
  b = a.conv_b[cc];
}

// ------------------------------------------------------------------ 1. B, C, Delta and C B^T per (chunk, group)
// One workgroup of 512 threads per (chunk, group).
//  a. causal conv + SiLU of the group's B and C channels over the chunk's tokens (items of 8
//     channels x 8 tokens; the W-1 rows before a sequence come from the slot's window or are
//     zero): B rows to LDS, C rows to the workspace in the permuted order of the C h_in operand;
//  b. Delta = softplus(dt + dt_bias) and the chunk-local inclusive cumsum of Delta*A for the
//     group's heads (one wave per head, a wave scan);
//  c. B transposed to the workspace in the permuted order of the state product's operand;
//  d. C B^T for the 72 causal (row tile, K-step) pairs on MFMA (two row tiles per wave, w and
//     15 - w), formed transposed so that each lane holds exactly the 8 values the output
//     product's operand fragment needs, written as one 16-byte (bf16) or 32-byte (fp32) piece.
template <bool SPLIT, int N> struct BcLds {
  static constexpr int NP = N < 32 ? 32 : N;
  static constexpr int NPL = SPLIT ? 2 : 1;
  static constexpr int LDB = NP + 4;                       // u16 pitch of the post-conv B rows
  static constexpr int PLANE = kMaxRowTiles * 16 * LDB;   // u16
  static constexpr int OFF_TAPS = NPL * PLANE * 2;         // bytes: taps [2N][4], then bias [2N]
  static constexpr int BYTES = OFF_TAPS + 2 * N * 5 * 4;
};

template <bool SPLIT, int N, bool IOBF>
__global__ __launch_bounds__(kThreads) void bc_kernel(BcArgs args) {
  const PrefillParams& a = args.p;
  typedef BcLds<SPLIT, N> L;
  constexpr int NP = L::NP, NPL = L::NPL, NK = NP / 32, LDB = L::LDB;
  extern __shared__ __align__(16) unsigned char bc_smem[];
  u16* const sB = reinterpret_cast<u16*>(bc_smem);
  const unsigned char* tab = a.tab_inline > 0 ? (const unsigned char*)arg_tables()
                                              : reinterpret_cast<const unsigned char*>(a.seqs);
  const SeqEntry* seqs = reinterpret_cast<const SeqEntry*>(tab);
  const ChunkEntry* chunks = reinterpret_cast<const ChunkEntry*>(tab + a.tab_chunks);
  const int G = a.sh.G;
  if ((int)blockIdx.x >= a.num_chunks * G) {   // trailing workgroup (inline tables only)
    table_copy_block(a);
    return;
  }
  const int c = blockIdx.x / G, g = blockIdx.x % G;
  const ChunkEntry ch = load_uniform(&chunks[c]);
  const SeqEntry sq = load_uniform(&seqs[ch.seq]);
  const int len = ch.len, QC = a.QC;
  const int I = a.sh.I, GN = G * N, W1 = a.sh.W - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t cg = (int64_t)c * G + g;
  u16* const cf = a.Cf + cg * QC * NP;

  // Requests first, work second: the step sizes' dt values, the group's conv taps (to LDS), and
  // the raw B/C rows of this thread's conv items all go out before any of them is waited for.
  // b0. dt of the wave's heads (wave w: heads w, w + 8, ...; lane l: tokens 4l .. 4l+3), two heads
  // at a time
  const int hpg = a.sh.H / G;
  constexpr int HB = 2;
  // raw values (converted when used, so no load waits for its own result)
  typedef typename std::conditional<IOBF, u16, float>::type DtRaw;
  DtRaw dtv[HB][4];
  auto load_dt = [&](int hh0) {
#pragma unroll
    for (int b = 0; b < HB; ++b) {
      const int hh = min(hh0 + 8 * b, hpg - 1), h = g * hpg + hh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = min(lane * 4 + e, len - 1);
        dtv[b][e] = static_cast<const DtRaw*>(a.dt)[(int64_t)(ch.t0 + i) * a.dt_stride + h];
      }
    }
  };
  load_dt(wave);
  // a1. conv + SiLU: thread (octet o, token blocks tb0 + TBS m); octets [0, OCT) are B channels,
  // [OCT, 2 OCT) C channels (past N: zeros); rows outside the sequence or past the chunk read a
  // valid row of the chunk (rows before the sequence are then replaced by the slot's window or
  // zeros)
  constexpr int OCT = NP / 8, NOCT = 2 * OCT, TBS = kThreads / NOCT;
  constexpr int NIT = (kMaxRowTiles * 2 + TBS - 1) / TBS;
  constexpr int PRE = 1;   // items whose rows are requested ahead (fp32 rows: one)
  const int ntb = (len + 7) / 8;
  const int o = tid % NOCT, tb0 = tid / NOCT;
  const bool isC = o >= OCT;
  const int n0 = (o % OCT) * 8;
  const bool chan_ok = n0 < N;
  const void* const src = isC ? a.C : a.B;
  const int64_t stride = isC ? a.C_stride : a.B_stride;
  const int64_t col = (int64_t)g * N + (chan_ok ? n0 : 0);
  Raw8<IOBF> raw[PRE][11];
  auto load_rows = [&](int m, Raw8<IOBF> (&r)[11]) {
    const int j0 = 8 * (tb0 + TBS * m);
#pragma unroll
    for (int k = 0; k < 11; ++k) {
      const int jj = min(max(j0 - 3 + k, -min(3, ch.tau0)), len - 1);   // a row of the sequence
      r[k].load(src, (int64_t)(sq.t0 + ch.tau0 + jj) * stride + col);
    }
  };
#pragma unroll
  for (int m = 0; m < PRE; ++m) load_rows(m, raw[m]);
  // the conv taps and bias of the group's B and C channels, to LDS (requested after the rows)
  float* const sTap = reinterpret_cast<float*>(bc_smem + L::OFF_TAPS);
  for (int i = tid; i < 2 * N; i += kThreads) {
    const int cc = I + (i >= N ? GN : 0) + g * N + i % N;
    float w[4], b;
    taps4(a, cc, w, b);
    *reinterpret_cast<floatx4*>(sTap + 4 * i) = floatx4{w[0], w[1], w[2], w[3]};
    sTap[8 * N + i] = b;
  }
  __syncthreads();   // the taps in LDS
  const int cc0 = I + (isC ? GN : 0) + g * N + n0;
  float wt[8][4], bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int ci = (isC ? N : 0) + (chan_ok ? n0 + e : 0);
    const floatx4 w4 = *reinterpret_cast<const floatx4*>(sTap + 4 * ci);
#pragma unroll
    for (int k = 0; k < 4; ++k) wt[e][k] = w4[k];
    bias[e] = sTap[8 * N + ci];
  }
#pragma unroll
  for (int m = 0; m < NIT; ++m) {
    const int tb = tb0 + TBS * m, j0 = 8 * tb;
    if (tb >= ntb) break;
    Raw8<IOBF> rr[11];
    if (PRE == NIT) {
#pragma unroll
      for (int k = 0; k < 11; ++k) rr[k] = raw[PRE == NIT ? m : 0][k];
    } else {
      load_rows(m, rr);
    }
    // the raw rows; a row past the chunk holds a row of the chunk (finite: the outputs it feeds
    // are past the chunk, where the walk gives them zero weight or discards them)
    float xr[11][8];
#pragma unroll
    for (int k = 0; k < 11; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xr[k][e] = rr[k].at(e);
    }
    if (ch.tau0 + j0 < 3) {   // rare: rows before the sequence, from the slot's window or zero
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int tau = ch.tau0 + j0 - 3 + k;
        if (tau < 0) {
          const bool w = sq.has_init && tau >= -W1 && chan_ok;
#pragma unroll
          for (int e = 0; e < 8; ++e) xr[k][e] = w ? window_value(a, sq.slot, cc0 + e, W1 + tau) : 0.f;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = bias[e];
#pragma unroll
        for (int k = 0; k < 4; ++k) x += wt[e][k] * xr[r + k][e];
        v[e] = chan_ok ? silu(x) : 0.f;   // d_state padding: zeros
      }
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        hw[mm] = pack_bf16x2(v[2 * mm], v[2 * mm + 1]);
        if (SPLIT) lw[mm] = pack_bf16x2(v[2 * mm] - lo_f32(hw[mm]), v[2 * mm + 1] - hi_f32(hw[mm]));
      }
      const int j = j0 + r;
      if (!isC) {
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          const uint32_t* x = pl == 0 ? hw : lw;
          uint32_t* d = reinterpret_cast<uint32_t*>(sB + pl * L::PLANE + j * LDB + n0);
          *reinterpret_cast<uint2*>(d) = uint2{x[0], x[1]};
          *reinterpret_cast<uint2*>(d + 2) = uint2{x[2], x[3]};
        }
      } else {
        // channels n0 .. n0+3 and n0+4 .. n0+7 land at two 4-element runs of the permuted row
        const int p0 = (n0 & ~31) + perm32(n0 & 31), p1 = (n0 & ~31) + perm32((n0 + 4) & 31);
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          const uint32_t* x = pl == 0 ? hw : lw;
          u16* d = cf + pl * a.Cf_plane + (int64_t)j * NP;
          *reinterpret_cast<uint2*>(d + p0) = uint2{x[0], x[1]};
          *reinterpret_cast<uint2*>(d + p1) = uint2{x[2], x[3]};
        }
      }
    }
  }
  // B rows past the conv items, up to the operand capacity: zero (the C B^T K-steps read them)
  for (int i = tid; i < (QC - ntb * 8) * (NP / 4); i += kThreads) {
    const int j = ntb * 8 + i / (NP / 4), n = (i % (NP / 4)) * 4;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl) *reinterpret_cast<u16x4*>(sB + pl * L::PLANE + j * LDB + n) = u16x4{0, 0, 0, 0};
  }

  // b. Delta and the chunk-local cumsum for the group's heads; lane l owns tokens 4l .. 4l+3
  {
    const int64_t T = a.total_tokens;
    for (int hh0 = wave; hh0 < hpg; hh0 += 8 * HB) {
      if (hh0 != wave) load_dt(hh0);
#pragma unroll
      for (int b = 0; b < HB; ++b) {
        const int hh = hh0 + 8 * b;
        if (hh >= hpg) break;
        const int h = g * hpg + hh;
        const float A = a.A[h], dtb = a.dt_bias[h];
        float d[4], sc[4], run = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = lane * 4 + e;
          float dt;
          if constexpr (IOBF) dt = f_of(dtv[b][e]);
          else dt = dtv[b][e];
          d[e] = i < len ? softplus(dt + dtb) : 0.f;
          run += d[e] * A;
          sc[e] = run;
        }
        float incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float t = __shfl_up(incl, off);
          if (lane >= off) incl += t;
        }
        const float excl = incl - run;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = lane * 4 + e;
          if (i < len) {
            a.delta[(int64_t)h * T + ch.t0 + i] = d[e];
            a.dA[(int64_t)h * T + ch.t0 + i] = excl + sc[e];
          }
        }
      }
    }
  }
  __syncthreads();

  // c. B transposed: lane per state column n (consecutive lanes read consecutive LDS words),
  // one 32-token K-step per item, written as 64 contiguous bytes in the permuted token order
  for (int item = tid; item < N * (QC / 32); item += kThreads) {
    const int n = item % N, kb = (item / N) * 32;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl) {
      u16* d = a.Btf + pl * a.Btf_plane + (cg * N + n) * QC + kb;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        u16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = sB[pl * L::PLANE + (kb + kmap(qq, e)) * LDB + n];
        *reinterpret_cast<u16x8*>(d + 8 * qq) = o;
      }
    }
  }

  // d. C B^T of the causal pairs: A = B rows j (K = d_state, from LDS), B = C columns i (K =
  // d_state, from the permuted C rows just written); the accumulator of the two 16-token halves
  // jt of K-step k holds, in lane l, G[16 rt + l % 16][32 k + kmap(l / 16, 4 jt + r)]
#pragma unroll 1
  for (int t = 0; t < 2; ++t) {
    const int rt = t == 0 ? wave : kMaxRowTiles - 1 - wave;
    if (rt * 16 >= len) continue;
    const int i = rt * 16 + l16;
    Frag<SPLIT> fc[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const u16* p = cf + (int64_t)i * NP + 32 * ks + 8 * q;
      const u16x8 hi = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) fc[ks].hi[e] = bf_of(hi[e]);
      if (SPLIT) {
        const u16x8 lo = *reinterpret_cast<const u16x8*>(p + a.Cf_plane);
#pragma unroll
        for (int e = 0; e < 8; ++e) fc[ks].lo[e] = bf_of(lo[e]);
      }
    }
#pragma unroll 1
    for (int k = 0; k <= (rt >> 1); ++k) {
      floatx4 gt[2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        gt[jt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks)
          gt[jt] = mma<SPLIT>(lds_frag<SPLIT>(sB, L::PLANE, LDB, 32 * k + 16 * jt + l16, 32 * ks, q), fc[ks], gt[jt]);
      }
      // lane-major, 8 bf16 values per lane (16 with fp32 state: the hi values, then the lo values)
      const int64_t gi = ((cg * kGPairs + pair_index(rt, k)) * 64 + lane) * 8 * NPL;
      u16x8 oh, ol;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u16 hi, lo = 0;
        const float v = gt[e >> 2][e & 3];
        if (SPLIT) split2(v, hi, lo);
        else hi = bits_of(from_f32<bf16>(v));
        oh[e] = hi;
        ol[e] = lo;
      }
      u16* const gp = static_cast<u16*>(a.Gf) + gi;
      *reinterpret_cast<u16x8*>(gp) = oh;
      if (SPLIT) *reinterpret_cast<u16x8*>(gp + 8) = ol;
    }
  }
}

// ------------------------------------------------------------------ 2. the walk over each sequence's chunks
// One workgroup of 512 threads per (sequence, head, part of PP head_dim channels) walks the
// sequence's chunks in order with the running state h (PP x N) in fp32 MFMA accumulators, so the
// state passes from chunk to chunk on chip.  The conv of a chunk runs one step ahead of the
// chunk's products, into the other of two LDS buffers, so that one barrier per step orders every
// LDS access.  Step k:
//  B. causal conv + SiLU of chunk k+1's x channels straight from its raw rows (requested during
//     step k-1, the W-1 rows before the chunk included) -> x^T, (w x)^T (w_j = exp(a_last - a_j)
//     Delta_j) and (c x)^T (c_j: the column factors of the output product) as bf16 planes;
//  C. outputs of chunk k, formed transposed, Y^T = h_in^T (exp(a) C)^T + X^T (M o L)^T, two
//     16-token row tiles per wave (w and 15 - w), so that a lane holds four consecutive channels
//     of one token: C h_in from the permuted C rows, then (M o L) X from the C B^T blocks of the
//     causal pairs masked by the decay (below the diagonal by a recurrence over the K-steps' last
//     tokens whose factors are all <= 1; on the diagonal block the exponent is taken directly,
//     with the causal mask and D on the diagonal), then the gate y = acc * SiLU(z);
//  D. h <- exp(a_last) h + (w x)^T B over chunk k's tokens (wave w: state columns 16w ..), with
//     the next steps' loads issued between its K-steps;
//  T. per-token decay tables of chunk k+2 (log2 units) into the third of three table sets;
//  H. the state leaving chunk k -> the other LDS state buffer (bf16 planes), read by step k+1;
//  E. after a checkpoint chunk, the state (rounded) and the raw-input window into the slot.
// After the last chunk the state and the window go to the sequence's slot.  The part-0
// workgroup of a group's first head also writes the windows of the group's B and C channels.
template <bool SPLIT, int PP, int N> struct WalkLds {
  static constexpr int NP = N < 32 ? 32 : N;
  static constexpr int NPL = SPLIT ? 2 : 1;
  static constexpr int LDX = kMaxRowTiles * 16 + 4;    // u16 pitch of an x^T row (tokens)
  static constexpr int LDH = NP + 4;                   // u16 pitch of a state row
  static constexpr int XPL = PP * LDX;                 // u16 per plane
  static constexpr int HPL = PP * LDH;
  static constexpr int TSET = 4 * 256 * 4;             // bytes of a chunk's tables: a2, b2, cw, ws
  static constexpr int HBUF = NPL * HPL * 2;           // bytes of a state buffer
  static constexpr int PBUF = 3 * NPL * XPL * 2;       // bytes of a plane buffer: (c x)^T, x^T, (w x)^T
  static constexpr int OFF_TAB = 0;                                     // three table sets
  static constexpr int OFF_TAPS = OFF_TAB + 3 * TSET;                   // taps [PP][4], bias [PP]
  static constexpr int OFF_W0 = OFF_TAPS + PP * 5 * 4;                  // raw rows -3 .. -1 [3][PP]
  static constexpr int OFF_H = (OFF_W0 + 3 * PP * 4 + 15) / 16 * 16;   // two state buffers
  static constexpr int OFF_P = OFF_H + 2 * HBUF;                        // two plane buffers
  static constexpr int BYTES = OFF_P + 2 * PBUF;
  static constexpr bool FITS = BYTES <= 160 * 1024;
};

template <bool SPLIT, int PP, int N, bool IOBF, bool ZYV>
__global__ __launch_bounds__(kThreads) void walk_kernel(PrefillParams a) {
  typedef WalkLds<SPLIT, PP, N> L;
  typedef typename std::conditional<SPLIT, float, bf16>::type TS;
  constexpr int NP = L::NP, NPL = L::NPL, NK = NP / 32, PT = PP / 16;
  constexpr int NT = N / 16;                     // state column tiles (one per wave)
  constexpr int LDX = L::LDX, LDH = L::LDH, XPL = L::XPL;
  // The channel of the part (row of the planes and of the state) that MFMA row m of channel
  // block pt stands for: with two blocks, rows 4q .. 4q+3 of blocks 0 and 1 (the accumulator
  // values of lane group q) are channels 8q .. 8q+7, so a lane's outputs, gate inputs and state
  // values are 8 adjacent channels (one 16-byte access for bf16).  Every operand read from the
  // planes and the state rows uses the same map, so the products are unchanged.
  auto chan = [](int pt, int m) { return PT == 2 ? 8 * (m >> 2) + 4 * pt + (m & 3) : 16 * pt + m; };
  extern __shared__ __align__(16) unsigned char wk_smem[];
  float* const sTap = reinterpret_cast<float*>(wk_smem + L::OFF_TAPS);
  float* const sBias = sTap + PP * 4;
  float* const sW0 = reinterpret_cast<float*>(wk_smem + L::OFF_W0);
  auto tab = [&](int s) { return reinterpret_cast<float*>(wk_smem + L::OFF_TAB + s * L::TSET); };
  auto hbuf = [&](int b) { return reinterpret_cast<u16*>(wk_smem + L::OFF_H + b * L::HBUF); };
  auto pbuf = [&](int b) { return reinterpret_cast<u16*>(wk_smem + L::OFF_P + b * L::PBUF); };

  const int H = a.sh.H, P = a.sh.P, G = a.sh.G, hpg = H / G, nparts = a.nparts;
  // the workgroups of one (sequence, group) run on one XCD, so the group's C, B^T and C B^T blocks
  // of a chunk come from memory once for its heads; the (sequence, group) units are dealt over the
  // XCDs in table order (longest sequences first)
  const int lg = xcd_units(blockIdx.x, gridDim.x, hpg * nparts);
  const int part = lg % nparts, rest = lg / nparts;
  const int hh = rest % hpg, g = (rest / hpg) % G, s = rest / H;
  const int h = g * hpg + hh;
  const SeqEntry sq = load_uniform(&a.seqs[s]);
  if (sq.nchunk == 0) return;
  const int c0 = h * P + part * PP;   // first x channel and output column of this part
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), q = lane >> 4, l16 = lane & 15;
  const int W1 = a.sh.W - 1, QC = a.QC;
  const int64_t T = a.total_tokens;
  const float Dh = load_uniform(&a.D[h]);
  const bool bc_windows = hh == 0 && part == 0;   // this workgroup also writes the group's B/C windows

  // ---- set-up: taps, the raw rows before the sequence, the state rows' padding past d_state
  for (int i = tid; i < PP * 4; i += kThreads) {
    const int cl = i / 4, k = i % 4, W = W1 + 1;
    sTap[i] = k >= 4 - W ? a.conv_w[(int64_t)(c0 + cl) * W + k - (4 - W)] : 0.f;
  }
  for (int i = tid; i < PP; i += kThreads) sBias[i] = a.conv_b[c0 + i];
  for (int i = tid; i < 3 * PP; i += kThreads) {
    const int tau = i / PP - 3, cl = i % PP;
    sW0[i] = (sq.has_init && tau >= -W1) ? window_value(a, sq.slot, c0 + cl, W1 + tau) : 0.f;
  }
  if (NP > N) {
    u16* const h0 = hbuf(0);   // both buffers: 2 NPL consecutive planes
    for (int i = tid; i < 2 * NPL * PP * (NP - N); i += kThreads) {
      const int pl = i / (PP * (NP - N)), p = (i / (NP - N)) % PP, n = N + i % (NP - N);
      h0[pl * L::HPL + p * LDH + n] = 0;
    }
  }
  // the state: wave w holds columns 16w .. 16w+15 for all PT row tiles (lane: rows 4q + r, column l16)
  const bool st_on = wave < NT;
  floatx4 accS[PT];
  {
    const TS* const init = static_cast<const TS*>(a.ssm) + ((int64_t)sq.slot * H + h) * P * N + (int64_t)part * PP * N;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      accS[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (sq.has_init && st_on) {
#pragma unroll
        for (int r = 0; r < 4; ++r) accS[pt][r] = to_f32(init[chan(pt, 4 * q + r) * N + wave * 16 + l16]);
      }
    }
  }
  // the state (bf16 planes) -> LDS state buffer b
  auto put_state = [&](int b) {
    if (!st_on) return;
    u16* const hb = hbuf(b);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u16 hi, lo = 0;
        if (SPLIT) split2(accS[pt][r], hi, lo);
        else hi = bits_of(from_f32<bf16>(accS[pt][r]));
        u16* d = hb + chan(pt, 4 * q + r) * LDH + wave * 16 + l16;
        d[0] = hi;
        if (SPLIT) d[L::HPL] = lo;
      }
    }
  };

  // ---- the conv items: thread (channel pair cp, group of TPT tokens); its raw rows j0-3 ..
  // j0+TPT-1 of the chunk (rows before the sequence come from the slot's window in LDS; rows past
  // the chunk repeat its last row: finite, and their token weights are zero)
  constexpr int NCP = PP / 2, TPT = PP == 32 ? 8 : 4, NRW = TPT + 3;
  static_assert(NCP * (kMaxRowTiles * 16 / TPT) == kThreads, "one conv item per thread");
  const int cp = tid % NCP, j0 = TPT * (tid / NCP), ccl = 2 * cp;
  typedef typename std::conditional<IOBF, uint32_t, f32x2>::type RawPair;
  constexpr int ES = IOBF ? 2 : 4;   // bytes of an x or z element
  // Rows of a chunk are addressed as a wave-uniform base (the chunk's first row read) plus a
  // 32-bit byte offset per lane: row pitches are below 16 MiB (checked by the host) and a chunk
  // spans at most 262 rows.
  const uint32_t xsb = (uint32_t)(a.x_stride * ES), xcol = (uint32_t)((c0 + ccl) * ES);
  RawPair rr[NRW];
  auto prefetch_raw = [&](const PrefillParams& ap, const ChunkEntry& nc) {
    const int lo = -min(3, nc.tau0), span = nc.len - 1 - lo;
    const char* const base = static_cast<const char*>(ap.x) + (int64_t)(nc.t0 + lo) * ap.x_stride * ES;
    const int u0 = j0 - 3 - lo;
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
      const uint32_t u = (uint32_t)min(max(u0 + r, 0), span);
      rr[r] = *reinterpret_cast<const RawPair*>(base + (__umul24(u, xsb) + xcol));
    }
  };
  // the conv of one chunk into plane buffer pl with its tables tb; `mid` runs once the raw rows
  // are in registers (it issues stores: by then no load that the conv waits for is in flight)
  auto conv_chunk = [&](u16* pl, const float* tb, int tau0, auto mid) {
    float rw[NRW][2];
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
      if constexpr (IOBF) { rw[r][0] = lo_f32(rr[r]); rw[r][1] = hi_f32(rr[r]); }
      else { rw[r][0] = rr[r][0]; rw[r][1] = rr[r][1]; }
    }
    // a chunk that starts fewer than 3 rows into its sequence: the rows before the sequence
    // (offset tau0 + r - 3 < 0) come from the slot's window
    if (tau0 < 3 && j0 == 0) {
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        if (tau0 + r < 3) { rw[r][0] = sW0[(tau0 + r) * PP + ccl]; rw[r][1] = sW0[(tau0 + r) * PP + ccl + 1]; }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
    float wsv[TPT], cwv[TPT];
#pragma unroll
    for (int m = 0; m < TPT / 4; ++m) {
      const floatx4 w4 = *reinterpret_cast<const floatx4*>(tb + 768 + j0 + 4 * m);
      const floatx4 c4 = *reinterpret_cast<const floatx4*>(tb + 512 + j0 + 4 * m);
#pragma unroll
      for (int e = 0; e < 4; ++e) { wsv[4 * m + e] = w4[e]; cwv[4 * m + e] = c4[e]; }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const floatx4 w4 = *reinterpret_cast<const floatx4*>(sTap + (ccl + e) * 4);
      const float b = sBias[ccl + e];
      float xv[TPT], wv[TPT], cv[TPT];
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        float x = b;
#pragma unroll
        for (int k = 0; k < 4; ++k) x += w4[k] * rw[r + k][e];
        x = silu(x);
        xv[r] = x;
        wv[r] = x * wsv[r];
        cv[r] = x * cwv[r];
      }
      auto put = [&](u16* base, const float (&v)[TPT]) {
        uint32_t hw[TPT / 2], lw[TPT / 2];
#pragma unroll
        for (int m = 0; m < TPT / 2; ++m) {
          hw[m] = pack_bf16x2(v[2 * m], v[2 * m + 1]);
          if (SPLIT) lw[m] = pack_bf16x2(v[2 * m] - lo_f32(hw[m]), v[2 * m + 1] - hi_f32(hw[m]));
        }
        uint32_t* d = reinterpret_cast<uint32_t*>(base + (ccl + e) * LDX + j0);
#pragma unroll
        for (int m = 0; m < TPT / 4; ++m) *reinterpret_cast<uint2*>(d + 2 * m) = uint2{hw[2 * m], hw[2 * m + 1]};
        if (SPLIT) {
          uint32_t* dl = reinterpret_cast<uint32_t*>(base + XPL + (ccl + e) * LDX + j0);
#pragma unroll
          for (int m = 0; m < TPT / 4; ++m) *reinterpret_cast<uint2*>(dl + 2 * m) = uint2{lw[2 * m], lw[2 * m + 1]};
        }
      };
      put(pl, cv);
      put(pl + NPL * XPL, xv);
      put(pl + 2 * NPL * XPL, wv);
    }
  };

  // ---- a chunk's token values (one token per thread) and its decay tables
  // (waves 0-3 only: thread j holds token j; the tables are written by those threads)
  float pd = 0.f, pa = 0.f;
  auto prefetch_tok = [&](const PrefillParams& ap, const ChunkEntry& nc) {
    if (wave < 4) {
      const int j = min(tid, nc.len - 1);
      pd = ap.delta[(int64_t)h * T + nc.t0 + j];
      pa = ap.dA[(int64_t)h * T + nc.t0 + j];
    }
  };
  auto put_tables = [&](float* tb, const ChunkEntry& nc) {
    const float al = load_uniform(&a.dA[(int64_t)h * T + nc.t0 + nc.len - 1]);
    if (tid < 256) {
      // a at the last token of the token's 32-token K-step (or of the chunk): lane j | 31 holds
      // token min(j | 31, len - 1)
      const float pr = __shfl(pa, lane | 31);
      const bool ok = tid < nc.len;
      tb[tid] = ok ? pa * kLog2e : -INFINITY;
      tb[256 + tid] = ok ? pa * kLog2e - __builtin_amdgcn_logf(pd) : 0.f;
      tb[512 + tid] = ok ? fast_exp2((pr - pa) * kLog2e) * pd : 0.f;
      tb[768 + tid] = ok ? fast_exp2((al - pa) * kLog2e) * pd : 0.f;
    }
  };

  const int rts[2] = {wave, kMaxRowTiles - 1 - wave};
  const int m0 = wave >> 1;           // K-steps below row tile 0 (7 - m0 below row tile 1)
  // the diagonal block of a row tile, lane (q, l16): row 4q + e against column l16 -> the causal
  // mask as an exponent offset (0, or -inf above the diagonal) and D on the diagonal
  float dmask[4], ddiag[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dmask[e] = e <= l16 - 4 * q ? 0.f : -INFINITY;
    ddiag[e] = e == l16 - 4 * q ? Dh : 0.f;
  }

  // ---- the output product's operands of a chunk, requested a step ahead (while the previous
  // chunk's state product runs): C columns and C B^T blocks of this wave's row tiles (below-diagonal
  // blocks of tile 0 in gb[0 .. m0-1], of tile 1 from gb[6] down; the diagonal blocks in gd), and z
  // (4 channels of one token per lane and column tile)
  typedef typename std::conditional<IOBF, u16x4, floatx4>::type ZQuad;
  const uint32_t zsb = (uint32_t)(a.z_stride * ES);
  Frag<SPLIT> cfr[2][NK];
  Frag<SPLIT> gb[7], gd[2];
  ZQuad zr[2][PT];
  // Every load is issued unconditionally (row tiles past the chunk read row tile 0 instead): the
  // in-order memory counter then lets each later wait cover exactly the loads it needs.  Step 0 /
  // 1 is the diagonal block and z of tile 0 / 1, step 2 + k is C B^T slot k.
  auto load_op = [&](const PrefillParams& ap, int step, int cidx, const ChunkEntry& nc) {
    const int64_t cgn = (int64_t)cidx * G + g;
    const bool v0 = rts[0] * 16 < nc.len, v1 = rts[1] * 16 < nc.len;
    const int rv[2] = {v0 ? rts[0] : 0, v1 ? rts[1] : 0};   // the row tile each load reads
    auto load_g = [&](int rt, int k, Frag<SPLIT>& dst) {
      const u16* const gp = static_cast<const u16*>(ap.Gf) + ((cgn * kGPairs + pair_index(rt, k)) * 64 + lane) * 8 * NPL;
      const u16x8 hi = *reinterpret_cast<const u16x8*>(gp);
#pragma unroll
      for (int e = 0; e < 8; ++e) dst.hi[e] = bf_of(hi[e]);
      if constexpr (SPLIT) {
        const u16x8 lo = *reinterpret_cast<const u16x8*>(gp + 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst.lo[e] = bf_of(lo[e]);
      }
    };
    if (step < 2) {
      const int t = step;
      const int i = rv[t] * 16 + l16;
      load_g(rv[t], rv[t] >> 1, gd[t]);
      const char* const zb = static_cast<const char*>(ap.z) + (int64_t)nc.t0 * ap.z_stride * ES;
      const uint32_t zrow = __umul24((uint32_t)(i < nc.len ? i : 0), zsb);
      if constexpr (ZYV && IOBF && PT == 2) {   // channels 8q .. 8q+7: one 16-byte load (aligned: ZYV)
        const u16x8 z8 = *reinterpret_cast<const u16x8*>(zb + (zrow + (uint32_t)((c0 + chan(0, 4 * q)) * ES)));
        zr[t][0] = u16x4{z8[0], z8[1], z8[2], z8[3]};
        zr[t][1] = u16x4{z8[4], z8[5], z8[6], z8[7]};
      } else {
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const char* const zp = zb + (zrow + (uint32_t)((c0 + chan(pt, 4 * q)) * ES));
        if constexpr (ZYV) {
          if constexpr (IOBF) zr[t][pt] = *reinterpret_cast<const u16x4*>(zp);
          else zr[t][pt] = *reinterpret_cast<const floatx4*>(zp);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (IOBF) zr[t][pt][r] = reinterpret_cast<const u16*>(zp)[r];
            else zr[t][pt][r] = reinterpret_cast<const float*>(zp)[r];
          }
        }
      }
      }
    } else {
      // slot k: a below-diagonal block of tile 0 (k < m0) or of tile 1 (K-step 6 - k)
      const int k = step - 2;
      const int rt = k < m0 ? rv[0] : rv[1];
      const int kk = k < m0 ? k : 6 - k;
      load_g(rt, min(kk, rt >> 1), gb[k]);
    }
  };
  // the C columns of row tile t of this wave
  auto load_c = [&](const PrefillParams& ap, int t, int cidx, const ChunkEntry& nc) {
    const u16* const cfb = ap.Cf + ((int64_t)cidx * G + g) * QC * NP;
    const int i = (rts[t] * 16 < nc.len ? rts[t] : 0) * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const u16* p = cfb + (int64_t)i * NP + 32 * ks + 8 * q;
      const u16x8 hi = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) cfr[t][ks].hi[e] = bf_of(hi[e]);
      if (SPLIT) {
        const u16x8 lo = *reinterpret_cast<const u16x8*>(p + ap.Cf_plane);
#pragma unroll
        for (int e = 0; e < 8; ++e) cfr[t][ks].lo[e] = bf_of(lo[e]);
      }
    }
  };

  // A chunk's gated outputs stay in registers until the next step's conv has its raw rows, and
  // are stored then (lane: channels c0 + 16 pt + 4q .. +3 of row yrow[t] of that chunk).
  // Loads and stores share one counter, and any wait while both are in flight has to wait for all
  // of them: the stores go out when the conv's loads have arrived, and the conv's arithmetic
  // covers them before the output phase's first wait.
  floatx4 ys[2][PT];
  int yrow[2] = {-1, -1};                 // row inside the stored chunk, -1 for none
  char* ybase = static_cast<char*>(a.y);  // the stored chunk's first row
  const int yes = a.y_bf16 ? 2 : 4;
  const uint32_t ysb = (uint32_t)(a.y_stride * yes);
  auto store_y = [&](const PrefillParams& ap) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (yrow[t] < 0) continue;
      const uint32_t yr = __umul24((uint32_t)yrow[t], ysb);
      if (ZYV && PT == 2 && ap.y_bf16) {   // channels 8q .. 8q+7: one 16-byte store (aligned: ZYV)
        u16x8 o;
#pragma unroll
        for (int r = 0; r < 8; ++r) o[r] = bits_of(from_f32<bf16>(ys[t][r >> 2][r & 3]));
        *reinterpret_cast<u16x8*>(ybase + (yr + (uint32_t)((c0 + chan(0, 4 * q)) * yes))) = o;
        yrow[t] = -1;
        continue;
      }
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        char* const yp = ybase + (yr + (uint32_t)((c0 + chan(pt, 4 * q)) * yes));
        const floatx4 yv = ys[t][pt];
        if (ap.y_bf16) {
          u16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = bits_of(from_f32<bf16>(yv[r]));
          if constexpr (ZYV) {
            *reinterpret_cast<u16x4*>(yp) = o;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) reinterpret_cast<u16*>(yp)[r] = o[r];
          }
        } else {
          if constexpr (ZYV) {
            *reinterpret_cast<floatx4*>(yp) = yv;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) reinterpret_cast<float*>(yp)[r] = yv[r];
          }
        }
      }
      yrow[t] = -1;
    }
  };

  // ---- before the first step: tables of chunks 0 and 1, the conv of chunk 0, the entering state
  {
    const ChunkEntry f0 = load_uniform(&a.chunks[sq.chunk0]);
    const ChunkEntry f1 = load_uniform(&a.chunks[sq.chunk0 + min(1, sq.nchunk - 1)]);
    prefetch_raw(a, f0);
    prefetch_tok(a, f0);
    put_tables(tab(0), f0);
    prefetch_tok(a, f1);
    put_tables(tab(1), f1);
    lds_sync();   // taps, window rows, tables
    conv_chunk(pbuf(0), tab(0), f0.tau0, [] {});
    put_state(0);
    __builtin_amdgcn_sched_barrier(0);
    prefetch_raw(a, f1);
#pragma unroll
    for (int st = 0; st < 9; ++st) load_op(a, st, sq.chunk0, f0);
    load_c(a, 0, sq.chunk0, f0);
    __builtin_amdgcn_sched_barrier(0);
    lds_sync();
  }

  int ts0 = 0, ts1 = 1, ts2 = 2;   // table sets of chunks k, k+1, k+2
  for (int kc = 0; kc < sq.nchunk; ++kc) {
    const int pb = kc & 1;
    const int cidx = sq.chunk0 + kc;
    const ChunkEntry ch = load_uniform(&a.chunks[cidx]);
    const int cnext = sq.chunk0 + min(kc + 1, sq.nchunk - 1);   // past the last chunk: the last again
    const ChunkEntry nx = load_uniform(&a.chunks[cnext]);
    const int cnn = sq.chunk0 + min(kc + 2, sq.nchunk - 1);
    const ChunkEntry nx2 = load_uniform(&a.chunks[cnn]);
    const int len = ch.len;
    const float alast = load_uniform(&a.dA[(int64_t)h * T + ch.t0 + len - 1]);
    const int64_t cg = (int64_t)cidx * G + g;
    const float* const sA2 = tab(ts0);
    const float* const sB2 = sA2 + 256;
    const u16* const sXC = pbuf(pb);
    const u16* const sXT = sXC + NPL * XPL;
    const u16* const sXW = sXT + NPL * XPL;
    const u16* const sH = hbuf(pb);

    // ---- B. the conv of the next chunk; the outputs held in registers are stored once its raw
    // rows are in.  With bf16 operands it runs first (the previous chunk's outputs); with
    // fp32-faithful operands after the outputs (this chunk's), so that it covers the latency of
    // the state product's B^T, whose registers would not fit during the output phase
    auto phase_b = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      if (kc + 1 < sq.nchunk) conv_chunk(pbuf(pb ^ 1), tab(ts1), nx.tau0, [&] { store_y(a); });
      else store_y(a);
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (!SPLIT) phase_b();

    const bool vt[2] = {rts[0] * 16 < len, rts[1] * 16 < len};
    // ---- loads of the state product's operand (bf16: under the output product; fp32-faithful
    // planes: after it, so that their registers are free during it)
    const int nkb = (len + 31) / 32;
    Frag<SPLIT> bt[kMaxRowTiles / 2];
    const u16* const btb = a.Btf + (cg * N + (st_on ? wave : 0) * 16 + l16) * QC + 8 * q;
    // K-steps k0 .. k1-1, unconditional: K-steps past the chunk read its last K-step again
    auto load_bt = [&](const PrefillParams& ap, int k0, int k1) {
#pragma unroll
      for (int kb = k0; kb < k1; ++kb) {
        const int kr = min(kb, nkb - 1);
        const u16x8 hi = *reinterpret_cast<const u16x8*>(btb + 32 * kr);
#pragma unroll
        for (int e = 0; e < 8; ++e) bt[kb].hi[e] = bf_of(hi[e]);
        if (SPLIT) {
          const u16x8 lo = *reinterpret_cast<const u16x8*>(btb + ap.Btf_plane + 32 * kr);
#pragma unroll
          for (int e = 0; e < 8; ++e) bt[kb].lo[e] = bf_of(lo[e]);
        }
      }
    };

    // ---- C. outputs of this wave's row tiles, one copy of the code per number of K-steps below
    // tile 0, so the K-step loops have fixed trip counts.
    auto phase_c = [&](auto m0c) {
    constexpr int M0 = decltype(m0c)::value;
    constexpr int MT[2] = {M0, 7 - M0};   // K-steps below each row tile; K-step MT[t] holds its diagonal
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!vt[t]) {
        yrow[t] = -1;
        if (t == 0) {
          load_c(a, 1, cidx, ch);
          if (!SPLIT) load_bt(a, 0, 8);
        }
        continue;
      }
      const int rt = rts[t];
      const int i = rt * 16 + l16;
      const float a2i = sA2[i];
      // C h_in first, then the K-steps entirely below the tile by a Horner recurrence over their
      // last tokens R(k): acc <- 2^(a2_R(k) - a2_R(k-1)) acc + (c x)_k^T (C B^T)_k^T (a2_R(-1) = 0,
      // every factor <= 1), with the column factors c_j = exp(a_R(k) - a_j) Delta_j folded into x;
      // at the end the row factor 2^(a2_i - a2_R(last)) gives every term its full decay
      // (each product's LDS operand is read one product ahead, so its latency hides under the
      // previous product)
      floatx4 acc[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
      {
        constexpr int NI = NK * PT;   // product i: K-step i / PT of row block i % PT
        Frag<SPLIT> hf[2];
        hf[0] = lds_frag<SPLIT>(sH, L::HPL, LDH, chan(0, l16), 0, q);
        // fp32-faithful planes: the two low-order products go to a second accumulator, so the
        // dependent chain through each accumulator is half as long
        floatx4 accl[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) accl[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (i + 1 < NI) hf[(i + 1) & 1] = lds_frag<SPLIT>(sH, L::HPL, LDH, chan((i + 1) % PT, l16), 32 * ((i + 1) / PT), q);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (SPLIT) mma_split2(hf[i & 1], cfr[t][i / PT], acc[i % PT], accl[i % PT]);
          else acc[i % PT] = mma<SPLIT>(hf[i & 1], cfr[t][i / PT], acc[i % PT]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (SPLIT) {
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) acc[pt] += accl[pt];
        }
      }
      // the next operands, requested under this tile's products: tile 1's C columns and (bf16) the
      // state product's B^T
      __builtin_amdgcn_sched_barrier(0);
      if (t == 0) {
        load_c(a, 1, cidx, ch);
        if (!SPLIT) load_bt(a, 0, 8);
      }
      __builtin_amdgcn_sched_barrier(0);
      float aprev = 0.f;
      {
        Frag<SPLIT> xf[2][PT];   // the (c x) operands of K-step k + 1 are read during K-step k
        if (MT[t] > 0) {
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) xf[0][pt] = lds_frag<SPLIT>(sXC, XPL, LDX, chan(pt, l16), 0, q);
        }
#pragma unroll
        for (int k = 0; k < MT[t]; ++k) {
          const int jk = 32 * k;
          if (k + 1 < MT[t]) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) xf[(k + 1) & 1][pt] = lds_frag<SPLIT>(sXC, XPL, LDX, chan(pt, l16), jk + 32, q);
          }
          __builtin_amdgcn_sched_barrier(0);
          const float aR = sA2[jk + 31];
          const float sk = fast_exp2(aR - aprev);
          aprev = aR;
          const Frag<SPLIT>& gk = t == 0 ? gb[k] : gb[6 - k];
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pt][r] *= sk;
            acc[pt] = mma<SPLIT>(xf[k & 1][pt], gk, acc[pt]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      {
        const float rfac = fast_exp2(a2i - aprev);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pt][r] *= rfac;
      }
      // the diagonal K-step: the 16-token block on the diagonal takes its exponents directly, with
      // the causal mask and D on the diagonal; the other half lies entirely below the tile (odd
      // tiles) or entirely above it (even tiles)
      {
        const int jk = 32 * MT[t];
        const floatx4 bd = *reinterpret_cast<const floatx4*>(&sB2[16 * rt + 4 * q]);
        float gv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gv[e] = static_cast<float>(gd[t].hi[e]);
          if (SPLIT) gv[e] += static_cast<float>(gd[t].lo[e]);
        }
        float mv[8];
        if (rt & 1) {
          const floatx4 bb = *reinterpret_cast<const floatx4*>(&sB2[jk + 4 * q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mv[e + 4] = fmaf(fast_exp2((a2i + dmask[e]) - bd[e]), gv[e + 4], ddiag[e]);
            mv[e] = fast_exp2(a2i - bb[e]) * gv[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mv[e] = fmaf(fast_exp2((a2i + dmask[e]) - bd[e]), gv[e], ddiag[e]);
            mv[e + 4] = 0.f;
          }
        }
        const Frag<SPLIT> mf = make_frag<SPLIT>(mv);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          acc[pt] = mma<SPLIT>(lds_frag<SPLIT>(sXT, XPL, LDX, chan(pt, l16), jk, q), mf, acc[pt]);
      }
      // the gate: lane holds channels c0 + 16 pt + 4q .. +3 of token i
      yrow[t] = i < len ? i : -1;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float zv;
          if constexpr (IOBF) zv = f_of(zr[t][pt][r]);
          else zv = zr[t][pt][r];
          ys[t][pt][r] = acc[pt][r] * silu(zv);
        }
      }
    }
    };
    switch (m0) {
      case 0: phase_c(std::integral_constant<int, 0>{}); break;
      case 1: phase_c(std::integral_constant<int, 1>{}); break;
      case 2: phase_c(std::integral_constant<int, 2>{}); break;
      default: phase_c(std::integral_constant<int, 3>{}); break;
    }
    ybase = static_cast<char*>(a.y) + (int64_t)ch.t0 * a.y_stride * yes;
    // fp32-faithful planes: the state product's B^T, now that the output operands' registers are
    // free (requested during the outputs it made them spill); the conv then covers its latency
    if constexpr (SPLIT) {
      load_bt(a, 0, 8);
      phase_b();
    }


    // ---- D. the state: h <- exp(a_last) h + (w x)^T B over the chunk's tokens.  Between its
    // K-steps the next steps' loads are issued, in the order they are consumed: token values
    // (tables at the end of this step), raw rows (next step's conv), output operands (next step's
    // output product).
    __builtin_amdgcn_sched_barrier(0);
    prefetch_tok(a, nx2);
    __builtin_amdgcn_sched_barrier(0);
    const float dec = fast_exp2(alast * kLog2e);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) accS[pt][r] *= dec;
    // every K-step, also past a short chunk's end: there the (w x) rows are zeros and the B^T
    // operand repeats the last K-step, so the products add nothing and no branch is needed
    Frag<SPLIT> wf[2][PT];   // the (w x) operands of K-step kb + 1 are read during K-step kb
    floatx4 accSl[PT];       // fp32-faithful planes: the low-order products, added at the end
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) accSl[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) wf[0][pt] = lds_frag<SPLIT>(sXW, XPL, LDX, chan(pt, l16), 0, q);
#pragma unroll
    for (int kb = 0; kb < kMaxRowTiles / 2; ++kb) {
      if (kb + 1 < kMaxRowTiles / 2) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) wf[(kb + 1) & 1][pt] = lds_frag<SPLIT>(sXW, XPL, LDX, chan(pt, l16), 32 * kb + 32, q);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (st_on) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          if constexpr (SPLIT) mma_split2(wf[kb & 1][pt], bt[kb], accS[pt], accSl[pt]);
          else accS[pt] = mma<SPLIT>(wf[kb & 1][pt], bt[kb], accS[pt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kb == 0) prefetch_raw(a, nx2);
      if (kb >= 1) load_op(a, kb - 1, cnext, nx);
      if (kb == 7) load_op(a, 7, cnext, nx), load_op(a, 8, cnext, nx), load_c(a, 0, cnext, nx);
      __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (SPLIT) {
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) accS[pt] += accSl[pt];
    }

    // ---- T, H. tables of chunk k+2; the state leaving this chunk for the next step's outputs
    if (kc + 2 < sq.nchunk) put_tables(tab(ts2), nx2);
    put_state(pb ^ 1);

    // ---- E. a checkpoint after this chunk: the state (rounded) and the raw-input window
    if (ch.ckpt_slot >= 0) {
      const PrefillParams ar = opaque_params();
      const SeqEntry sqr = load_uniform(&ar.seqs[s]);
      if (st_on) {
        TS* const dst = static_cast<TS*>(ar.ssm) + ((int64_t)ch.ckpt_slot * H + h) * P * N + (int64_t)part * PP * N;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[chan(pt, 4 * q + r) * N + wave * 16 + l16] = from_f32<TS>(accS[pt][r]);
      }
      const int tau = ch.tau0 + len;
      for (int i = tid; i < W1 * PP; i += kThreads) {
        const int kk = i / PP, cl = i % PP, pos = tau - W1 + kk;
        const float v = pos >= 0 ? load_any(ar.x, (int64_t)(sqr.t0 + pos) * ar.x_stride + c0 + cl, ar.io_bf16)
                                 : sW0[(3 + pos) * PP + cl];
        window_store(ar, ch.ckpt_slot, c0 + cl, kk, v);
      }
      if (bc_windows) {
        const int I = ar.sh.I, GN = ar.sh.G * N;
        for (int i = tid; i < W1 * 2 * N; i += kThreads) {
          const int kk = i / (2 * N), cl = i % (2 * N);
          const bool isC = cl >= N;
          const int n = cl % N, cc = I + (isC ? GN : 0) + g * N + n, off = tau - W1 + kk;
          float v;
          if (off >= 0) {
            v = isC ? load_any(ar.C, (int64_t)(sqr.t0 + off) * ar.C_stride + g * N + n, ar.io_bf16)
                    : load_any(ar.B, (int64_t)(sqr.t0 + off) * ar.B_stride + g * N + n, ar.io_bf16);
          } else {
            v = sqr.has_init ? window_value(ar, sqr.slot, cc, W1 + off) : 0.f;
          }
          window_store(ar, ch.ckpt_slot, cc, kk, v);
        }
      }
      // drain the checkpoint stores (this also waits for the next step's loads, on checkpoint
      // chunks only): past this branch only loads are in flight on either path
      __builtin_amdgcn_s_waitcnt(0);
    }
    lds_sync();   // this step's LDS reads and writes are done
    const int tr = ts0;
    ts0 = ts1;
    ts1 = ts2;
    ts2 = tr;
  }

  store_y(a);   // the last chunk's outputs
  // ---- the final state and window into the sequence's slot
  const PrefillParams ar = opaque_params();
  const SeqEntry sqr = load_uniform(&ar.seqs[s]);
  if (st_on) {
    TS* const head_state = static_cast<TS*>(ar.ssm) + ((int64_t)sqr.slot * H + h) * P * N + (int64_t)part * PP * N;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) head_state[chan(pt, 4 * q + r) * N + wave * 16 + l16] = from_f32<TS>(accS[pt][r]);
  }
  {
    const int tau = sqr.len;
    for (int i = tid; i < W1 * PP; i += kThreads) {
      const int kk = i / PP, cl = i % PP, pos = tau - W1 + kk;
      const float v = pos >= 0 ? load_any(ar.x, (int64_t)(sqr.t0 + pos) * ar.x_stride + c0 + cl, ar.io_bf16)
                               : sW0[(3 + pos) * PP + cl];
      window_store(ar, sqr.slot, c0 + cl, kk, v);
    }
  }
  if (bc_windows) {
    // the group's B and C windows: values may come from the slot's own window (a sequence shorter
    // than W-1 rows), so every value is read before any is written
    constexpr int BIT = (3 * 2 * N + kThreads - 1) / kThreads;
    float vals[BIT];
    const int I = ar.sh.I, GN = ar.sh.G * N;
    const int tau = sqr.len;
#pragma unroll
    for (int b = 0; b < BIT; ++b) {
      const int i = tid + b * kThreads;
      vals[b] = 0.f;
      if (i < W1 * 2 * N) {
        const int kk = i / (2 * N), cl = i % (2 * N);
        const bool isC = cl >= N;
        const int n = cl % N, cc = I + (isC ? GN : 0) + g * N + n, off = tau - W1 + kk;
        if (off >= 0) {
          vals[b] = isC ? load_any(ar.C, (int64_t)(sqr.t0 + off) * ar.C_stride + g * N + n, ar.io_bf16)
                        : load_any(ar.B, (int64_t)(sqr.t0 + off) * ar.B_stride + g * N + n, ar.io_bf16);
        } else if (sqr.has_init) {
          vals[b] = window_value(ar, sqr.slot, cc, W1 + off);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < BIT; ++b) {
      const int i = tid + b * kThreads;
      if (i < W1 * 2 * N) {
        const int kk = i / (2 * N), cl = i % (2 * N);
        const bool isC = cl >= N;
        window_store(ar, sqr.slot, I + (isC ? GN : 0) + g * N + cl % N, kk, vals[b]);
      }
    }
  }
}

// ------------------------------------------------------------------ launch
// Allow `bytes` of dynamic LDS for a kernel (idempotent; called before each launch).
static hipError_t set_lds_attr(const void* fn, int bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <bool SPLIT, int N, bool IOBF>
static hipError_t launch_bc(const PrefillParams& p, const InlineTables* inl, hipStream_t s) {
  BcArgs ba;
  ba.p = p;
  if (p.tab_inline > 0) memcpy(&ba.t, inl, (size_t)p.tab_inline);
  typedef BcLds<SPLIT, N> L;
  const hipError_t e = set_lds_attr(reinterpret_cast<const void*>(&bc_kernel<SPLIT, N, IOBF>), L::BYTES);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(p.num_chunks * p.sh.G) + (p.tab_inline > 0 ? 1u : 0u));
  hipLaunchKernelGGL((bc_kernel<SPLIT, N, IOBF>), grid, dim3(kThreads), L::BYTES, s, ba);
  return hipGetLastError();
}

template <bool SPLIT, int PP, int N, bool IOBF, bool ZYV>
static hipError_t launch_walk_z(const PrefillParams& p, hipStream_t s) {
  typedef WalkLds<SPLIT, PP, N> L;
  static_assert(L::FITS, "walk LDS");
  const hipError_t e = set_lds_attr(reinterpret_cast<const void*>(&walk_kernel<SPLIT, PP, N, IOBF, ZYV>), L::BYTES);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(p.num_seqs * p.sh.H * p.nparts));
  hipLaunchKernelGGL((walk_kernel<SPLIT, PP, N, IOBF, ZYV>), grid, dim3(kThreads), L::BYTES, s, p);
  return hipGetLastError();
}

template <bool SPLIT, int PP, int N, bool IOBF>
static hipError_t launch_walk(const PrefillParams& p, hipStream_t s) {
  return p.zy_vec ? launch_walk_z<SPLIT, PP, N, IOBF, true>(p, s) : launch_walk_z<SPLIT, PP, N, IOBF, false>(p, s);
}

template <bool SPLIT, int N>
static hipError_t launch_sn(const PrefillParams& p, const InlineTables* inl, hipStream_t s) {
  hipError_t e = p.io_bf16 ? launch_bc<SPLIT, N, true>(p, inl, s) : launch_bc<SPLIT, N, false>(p, inl, s);
  if (e != hipSuccess) return e;
  if constexpr (SPLIT) {
    return p.io_bf16 ? launch_walk<SPLIT, 16, N, true>(p, s) : launch_walk<SPLIT, 16, N, false>(p, s);
  } else {
    if (prefill_part(p.sh.P, false) == 16)
      return p.io_bf16 ? launch_walk<SPLIT, 16, N, true>(p, s) : launch_walk<SPLIT, 16, N, false>(p, s);
    return p.io_bf16 ? launch_walk<SPLIT, 32, N, true>(p, s) : launch_walk<SPLIT, 32, N, false>(p, s);
  }
}

template <int N>
static hipError_t launch_n(const PrefillParams& p, const InlineTables* inl, hipStream_t s) {
  return p.ssm_bf16 ? launch_sn<false, N>(p, inl, s) : launch_sn<true, N>(p, inl, s);
}

bool prefill_supported(int P, int N, int W) {
  const bool p_ok = P == 16 || P == 32 || P == 64 || P == 128;
  const bool n_ok = N == 16 || N == 32 || N == 64 || N == 128;
  return p_ok && n_ok && W >= 2 && W <= 4;
}

hipError_t launch_prefill(const PrefillParams& p, const InlineTables* inl, hipStream_t s) {
  if (p.num_chunks == 0) return hipSuccess;
  if (p.tab_inline < 0 || p.tab_inline > kInlineTableBytes || p.tab_inline % 16 != 0 || (p.tab_inline > 0 && !inl))
    return hipErrorInvalidValue;
  if (!prefill_supported(p.sh.P, p.sh.N, p.sh.W) || p.nparts * prefill_part(p.sh.P, !p.ssm_bf16) != p.sh.P || p.Q > 256 ||
      p.QC % 32 != 0 || p.QC < p.Q)
    return hipErrorInvalidValue;
  switch (p.sh.N) {
    case 16: return launch_n<16>(p, inl, s);
    case 32: return launch_n<32>(p, inl, s);
    case 64: return launch_n<64>(p, inl, s);
    case 128: return launch_n<128>(p, inl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m2
