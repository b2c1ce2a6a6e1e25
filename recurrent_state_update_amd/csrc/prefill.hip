// Chunked (SSD) prefill of packed variable-length sequences, gfx950.
//
// Each sequence is cut into chunks of Q tokens from its first row.  Inside a
// chunk the output is the causally masked product Y = (M o L) X of the Mamba study notes
// (echobase-5bl.pages.dev, "Mamba and Attention"),
//   M[i][j] = (C_i . B_j) exp(a_i - a_j) Delta_j   (j <= i),
// with a the chunk-local cumulative sum of Delta*A, plus exp(a_i) C_i h_in
// for the state h_in entering the chunk; chunk end states follow
// h_out = exp(a_last) h_in + sum_j exp(a_last - a_j) Delta_j x_j B_j^T, the
// affine step that links chunks ("Hybrid SSM / Mamba models and
// non-KV state", mlinterviewnotes.com ch. 7.3: chunked-prefill handoff,
// affine-composition passage, SSD chunk-scan call site).
//
// Launch sequence (one stream):
//   1. conv_kernel        causal conv + SiLU of every (token, channel), written as bf16
//                         operand planes in the layouts the products read; its leading
//                         workgroups compute Delta = softplus(dt + dt_bias) and the chunk-local
//                         cumsum of Delta*A
//   2. chunk_state_kernel per (chunk, head): the chunk's end state from a zero state (MFMA); its
//                         trailing workgroups write the checkpoint conv windows
//   3. state_pass_kernel  per (sequence, head): the affine step through the sequence's chunks ->
//                         state entering each chunk (operand planes), checkpoint and final
//                         states into their slots; the final conv windows
//   4. chunk_out_group_kernel  per (chunk, group): outputs (MFMA) of the group's heads in turn,
//                         C B^T formed once; chunk_out_kernel per (chunk, head) for hi/lo planes
//                         and head_dim 128
// With SPLIT every product operand is a bf16 hi plane plus a bf16 lo plane and
// each product takes three MFMAs (fp32-level accuracy, used for fp32 state);
// otherwise operands are single bf16 planes with fp32 accumulation.
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


constexpr int kScanThreads = 512;
constexpr int kStateThreads = 512;

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

// The same fragment's values as fp32 (hi + lo).
template <bool SPLIT>
__device__ __forceinline__ void lds_vals(const u16* base, int64_t plane, int ld, int row, int kb, int q, float (&v)[8]) {
  const u16* p = base + row * ld + kb + 4 * q;
  const u16x4 a = *reinterpret_cast<const u16x4*>(p);
  const u16x4 b = *reinterpret_cast<const u16x4*>(p + 16);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = f_of(a[e]); v[e + 4] = f_of(b[e]); }
  if (SPLIT) {
    const u16x4 c = *reinterpret_cast<const u16x4*>(p + plane);
    const u16x4 d = *reinterpret_cast<const u16x4*>(p + plane + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] += f_of(c[e]); v[e + 4] += f_of(d[e]); }
  }
}

// Copy rows of 8-element vectors from global bf16 planes into LDS planes.  Row r of the
// source starts at src + r * src_ld.  Rows at or past valid_rows and columns at or past
// valid_cols are written as zero and never read from global memory.
template <int NPL>
__device__ __forceinline__ void stage_rows(u16* dst, int64_t dst_plane, int dst_ld, const u16* src, int64_t src_plane,
                                           int64_t src_ld, int rows, int cols, int valid_rows, int valid_cols,
                                           int tid, int nthreads) {
  const int vpr = cols / 8;
  for (int idx = tid; idx < rows * vpr; idx += nthreads) {
    const int r = idx / vpr, c = (idx % vpr) * 8;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl) {
      u16x8 v = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      const u16* s = src + pl * src_plane + r * src_ld + c;
      if (r < valid_rows) {
        if (c + 8 <= valid_cols) {
          v = *reinterpret_cast<const u16x8*>(s);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (c + e < valid_cols) ? s[e] : u16(0);
        }
      }
      u16* d = dst + pl * dst_plane + r * dst_ld + c;
      *reinterpret_cast<u16x4*>(d) = u16x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<u16x4*>(d + 4) = u16x4{v[4], v[5], v[6], v[7]};
    }
  }
}

// Register prefetch of a staged block: ITEMS 8-element vectors per plane of a (rows x cols)
// tile, held in registers until written to LDS.  Every thread issues the same number of 16-byte
// loads with no branch (vectors outside the valid region read the tile's first vector; source
// rows are whole multiples of 8 elements, so a vector that starts inside a row stays inside
// it), and nothing touches the loaded registers until store(), which zeroes what lies outside
// the valid region.  The loads therefore stay in flight until the block is stored.
template <int NPL, int ITEMS> struct TilePrefetch {
  u16x8 v[ITEMS][NPL];

  __device__ __forceinline__ void load(const u16* src, int64_t src_plane, int64_t src_ld, int rows, int cols,
                                       int valid_rows, int valid_cols, int tid, int nthreads) {
    const int vpr = cols / 8;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * nthreads;
      const int r = idx / vpr, c = (idx % vpr) * 8;
      const bool in = idx < rows * vpr && r < valid_rows && c < valid_cols;
      const int off = in ? r * (int)src_ld + c : 0;   // offsets inside one tile fit in 32 bits
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) v[it][pl] = *reinterpret_cast<const u16x8*>(src + pl * src_plane + off);
    }
  }

  __device__ __forceinline__ void store(u16* dst, int64_t dst_plane, int dst_ld, int rows, int cols, int valid_rows,
                                        int valid_cols, int tid, int nthreads) const {
    const int vpr = cols / 8;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * nthreads;
      if (idx < rows * vpr) {
        const int r = idx / vpr, c = (idx % vpr) * 8;
        const bool in = r < valid_rows;
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          u16x8 x = v[it][pl];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (in && c + e < valid_cols) ? x[e] : u16(0);
          u16* d = dst + pl * dst_plane + r * dst_ld + c;
          *reinterpret_cast<u16x4*>(d) = u16x4{x[0], x[1], x[2], x[3]};
          *reinterpret_cast<u16x4*>(d + 4) = u16x4{x[4], x[5], x[6], x[7]};
        }
      }
    }
  }

  // store() for a tile known to be entirely valid: no masking.
  __device__ __forceinline__ void store_full(u16* dst, int64_t dst_plane, int dst_ld, int rows, int cols, int tid,
                                             int nthreads) const {
    const int vpr = cols / 8;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * nthreads;
      if (idx < rows * vpr) {
        const int r = idx / vpr, c = (idx % vpr) * 8;
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          u16* d = dst + pl * dst_plane + r * dst_ld + c;
          const u16x8 x = v[it][pl];
          *reinterpret_cast<u16x4*>(d) = u16x4{x[0], x[1], x[2], x[3]};
          *reinterpret_cast<u16x4*>(d + 4) = u16x4{x[4], x[5], x[6], x[7]};
        }
      }
    }
  }
};

// Workgroup b of a launch runs on XCD b % 8 (the dispatcher deals workgroups round-robin over
// the 8 XCDs, each with its own L2).  This maps b to a logical index so that every XCD receives
// one contiguous range of logical indices (a bijection on [0, n)).
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
  const int x = b % 8, full = n / 8, rem = n % 8;
  return x * full + min(x, rem) + b / 8;
}

// ------------------------------------------------------------------ 1a. Delta, cumsum
// Run by the first workgroups of the conv launch (they depend on nothing the conv writes and
// overlap its memory traffic).  One wave per (chunk, head); lane l owns rows 4l .. 4l+3 of the
// chunk (Q <= 256).
__device__ __forceinline__ void dt_block(const PrefillParams& a, const ChunkEntry* chunks, int b) {
  const int hq = (a.sh.H + 3) / 4;
  const ChunkEntry ch = load_uniform(&chunks[b / hq]);
  const int lane = threadIdx.x & 63;
  const int h = (b % hq) * 4 + (threadIdx.x >> 6);
  if (h >= a.sh.H) return;
  const float A = a.A[h], bias = a.dt_bias[h];
  float d[4], s[4];
  float run = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = lane * 4 + e;
    d[e] = i < ch.len ? softplus(load_any(a.dt, (int64_t)(ch.t0 + i) * a.dt_stride + h, a.io_bf16) + bias) : 0.f;
    run += d[e] * A;
    s[e] = run;
  }
  float incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  const float excl = incl - run;
  const int64_t T = a.total_tokens;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = lane * 4 + e;
    if (i < ch.len) {
      a.delta[(int64_t)h * T + ch.t0 + i] = d[e];
      a.dA[(int64_t)h * T + ch.t0 + i] = excl + s[e];
    }
  }
}

// ------------------------------------------------------------------ 1b. conv
// One-dimensional grid over (chunk, 64-token part, 256 channels), channel block fastest, so that
// workgroups running together read neighbouring pieces of the same token rows; 256 threads.
// Thread (octet o, group t) convolves channels 8o .. 8o+7 over tokens 8t .. 8t+7 of its part: the
// W-1 halo rows and its 8 rows are requested together (16-byte loads), the taps and SiLU run in
// fp32, and the results are rounded to the operand planes.  B and C rows go out straight from
// registers (32 lanes cover 512 contiguous bytes of a row); x and B also go into a
// channel-major LDS tile, each thread's block transposed in registers so that it writes 8-byte
// runs of 4 tokens, from which the transposed planes are written with consecutive lanes
// on consecutive 16-byte pieces of one row.  In a channel row, token group t sits at position
// t ^ (row / 8 % 8): the eight channel octets of one token group then fall in distinct banks.
// A conv workgroup covers 256 channels x 64 tokens: 512-byte pieces of each input row, and one
// 64-token block of the transposed planes per channel (measured: 64 channels x 256 tokens 7%
// slower, 128 x 128 2% slower).
constexpr int kConvCB = 256;
constexpr int kConvTQ = 64 * 256 / kConvCB;   // tokens per workgroup
constexpr int kConvNH = 256 / kConvTQ;        // workgroups per (chunk, channel block)
constexpr int kConvLD = kConvTQ + 8;   // u16 pitch of a channel row of the LDS tile (16-byte aligned)
__device__ __forceinline__ int conv_tpos(int row, int grp) { return 8 * (grp ^ ((row >> 3) & 7)); }

template <bool SPLIT> struct ConvLds {
  static constexpr int NPL = SPLIT ? 2 : 1;
  static constexpr int BYTES = NPL * kConvCB * kConvLD * 2;
};

template <bool IOBF> __device__ __forceinline__ void load_row8(const void* p, int64_t i, float (&o)[8]) {
  if (IOBF) {
    const u16x8 v = *reinterpret_cast<const u16x8*>(static_cast<const u16*>(p) + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = f_of(v[e]);
  } else {
    const floatx4 a = *reinterpret_cast<const floatx4*>(static_cast<const float*>(p) + i);
    const floatx4 b = *reinterpret_cast<const floatx4*>(static_cast<const float*>(p) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[e + 4] = b[e]; }
  }
}

// The packed tables inside the conv launch's own kernel arguments.
__device__ __forceinline__ const __attribute__((address_space(4))) unsigned char* conv_arg_tables() {
  typedef const __attribute__((address_space(4))) unsigned char kbyte;
  return (kbyte*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(ConvArgs, t);
}

// One workgroup of the conv launch: copy the tables from the kernel arguments to the workspace,
// where the later launches read them (tab_inline is a multiple of 16 bytes).
__device__ __forceinline__ void table_copy_block(const PrefillParams& a) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) i32x4 kquad;
  kquad* src = reinterpret_cast<kquad*>(conv_arg_tables());
  i32x4* dst = reinterpret_cast<i32x4*>(const_cast<SeqEntry*>(a.seqs));
  for (int i = threadIdx.x; i < a.tab_inline / 16; i += blockDim.x) dst[i] = src[i];
}

template <int W, bool SPLIT, bool IOBF>
__global__ __launch_bounds__(256) void conv_kernel(ConvArgs args) {
  const PrefillParams& a = args.p;
  constexpr int CB = kConvCB;
  constexpr int NPL = ConvLds<SPLIT>::NPL;
  constexpr int PLANE = CB * kConvLD;
  constexpr int R = 8;
  extern __shared__ __align__(16) unsigned char conv_smem[];
  u16* const s_t = reinterpret_cast<u16*>(conv_smem);
  // this launch reads the tables where the host put them: its own arguments or the workspace
  const unsigned char* tab = a.tab_inline > 0 ? (const unsigned char*)conv_arg_tables()
                                              : reinterpret_cast<const unsigned char*>(a.seqs);
  const SeqEntry* seqs = reinterpret_cast<const SeqEntry*>(tab);
  const ChunkEntry* chunks = reinterpret_cast<const ChunkEntry*>(tab + a.tab_chunks);
  const int ndt = a.num_chunks * ((a.sh.H + 3) / 4);   // leading workgroups: Delta and cumsum
  if ((int)blockIdx.x < ndt) {
    dt_block(a, chunks, blockIdx.x);
    return;
  }
  const int bx = blockIdx.x - ndt;
  const int ncb = (a.sh.Cd + CB - 1) / CB;
  if (bx >= a.num_chunks * ncb * kConvNH) {   // trailing workgroup (inline tables only)
    table_copy_block(a);
    return;
  }
  const int64_t chunk = bx / (ncb * kConvNH);
  const int rem = bx % (ncb * kConvNH);
  const int tq0 = (rem / ncb) * kConvTQ;   // first token of this workgroup inside the chunk
  const ChunkEntry ch = load_uniform(&chunks[chunk]);
  const SeqEntry sq = load_uniform(&seqs[ch.seq]);
  const int Cd = a.sh.Cd, I = a.sh.I, GN = a.sh.G * a.sh.N, P = a.sh.P, N = a.sh.N, H = a.sh.H, G = a.sh.G;
  const int Q = a.Q, len = ch.len;
  const int c0 = (rem % ncb) * CB;
  const int tid = threadIdx.x;
  const int oc = tid % (CB / 8), tg = tid / (CB / 8);   // 32 channel octets x 8 token groups
  const int c = c0 + 8 * oc;
  const int j0 = tq0 + 8 * tg;
  if (c < Cd && j0 < len) {
    const void* src;
    int64_t col, stride;
    if (c < I) { src = a.x; col = c; stride = a.x_stride; }
    else if (c < I + GN) { src = a.B; col = c - I; stride = a.B_stride; }
    else { src = a.C; col = c - I - GN; stride = a.C_stride; }
    // inputs: rows outside the sequence read the chunk's first row and are replaced below.
    // bf16 rows stay packed until used (half the registers of fp32 copies).
    typedef typename std::conditional<IOBF, u16x8, float[8]>::type Row;
    Row in_raw[R + W - 1];
#pragma unroll
    for (int k = 0; k < R + W - 1; ++k) {
      const int tau = ch.tau0 + j0 - (W - 1) + k;   // offset inside the sequence
      const bool ok = tau >= 0 && j0 - (W - 1) + k < len;
      const int64_t i = (ok ? sq.t0 + tau : ch.t0) * stride + col;
      if constexpr (IOBF) in_raw[k] = *reinterpret_cast<const u16x8*>(static_cast<const u16*>(src) + i);
      else load_row8<false>(src, i, in_raw[k]);
    }
    auto in_at = [&](int k, int e) -> float {
      if constexpr (IOBF) return f_of(in_raw[k][e]);
      else return in_raw[k][e];
    };
    float halo[W - 1][8];   // the rows before the sequence start, when the chunk begins it
    float w[8][W], bias[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int k = 0; k < W; ++k) w[e][k] = a.conv_w[(int64_t)(c + e) * W + k];
      bias[e] = a.conv_b[c + e];
    }
    const bool seq_start = ch.tau0 + j0 < W - 1;   // uniform per thread group; rare
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) halo[k][e] = in_at(k, e);
    }
    if (seq_start) {   // halo before the sequence start: the slot's window or zeros
#pragma unroll
      for (int k = 0; k < W - 1; ++k) {
        const int tau = ch.tau0 + j0 - (W - 1) + k;
        if (tau < 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float v = 0.f;
            if (sq.has_init) {
              const int64_t wi = ((int64_t)sq.slot * Cd + c + e) * (W - 1) + (W - 1 + tau);
              v = a.conv_bf16 ? to_f32(static_cast<const bf16*>(a.conv)[wi]) : static_cast<const float*>(a.conv)[wi];
            }
            halo[k][e] = v;
          }
        }
      }
    }
    // token j0 + r, channels c .. c+7 (zero past the chunk): B and C rows straight to global;
    // x and B collected per channel (tv[e][r]) for the channel-major LDS tile
    u16* const brow = c < I + GN ? a.Br + (chunk * Q + j0) * GN + (c - I) : a.Cr + (chunk * Q + j0) * GN + (c - I - GN);
    const int64_t bplane = c < I + GN ? a.Br_plane : a.Cr_plane;
    u16x4 tv[8], tl[8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      u16x8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = bias[e];
#pragma unroll
        for (int k = 0; k < W; ++k) v += w[e][k] * (r + k < W - 1 ? halo[r + k][e] : in_at(r + k, e));
        v = j0 + r < len ? silu(v) : 0.f;
        u16 hi, lo = 0;
        if (SPLIT) split2(v, hi, lo);
        else hi = bits_of(from_f32<bf16>(v));
        hv[e] = hi;
        lv[e] = lo;
      }
      if (c >= I && j0 + r < len) {
        *reinterpret_cast<u16x8*>(brow + (int64_t)r * GN) = hv;
        if (SPLIT) *reinterpret_cast<u16x8*>(brow + bplane + (int64_t)r * GN) = lv;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        tv[e][r & 3] = hv[e];
        tl[e][r & 3] = lv[e];
      }
      if ((r & 3) == 3 && c < I + GN) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = 8 * oc + e;
          u16* d = s_t + row * kConvLD + conv_tpos(row, tg) + (r & 4);
          *reinterpret_cast<u16x4*>(d) = tv[e];
          if (SPLIT) *reinterpret_cast<u16x4*>(d + PLANE) = tl[e];
        }
      }
    }
  }
  if (c0 >= I + GN) return;   // C channels only: nothing transposed (uniform per workgroup)
  __syncthreads();
  // x and B transposed: lane per 8-token group, consecutive lanes along one channel row
  const int ngr = len > tq0 ? (min(len - tq0, kConvTQ) + 7) / 8 : 0;
  for (int idx = tid; idx < CB * ngr; idx += 256) {
    const int g = idx % ngr, ccl = idx / ngr;
    const int tg8 = tq0 + 8 * g;
    const int cc = c0 + ccl;
    if (cc >= I + GN) continue;
    u16* dst;
    int64_t pstride;
    const int QB = (Q + kPB - 1) / kPB, blk = tg8 / kPB, off = tg8 % kPB;
    if (cc < I) {
      const int h = cc / P, p = cc % P;
      dst = a.xT + (((chunk * H + h) * QB + blk) * P + p) * kPB + off;
      pstride = a.xT_plane;
    } else {
      const int gg = (cc - I) / N, n = (cc - I) % N;
      dst = a.Bt + (((chunk * G + gg) * QB + blk) * N + n) * kPB + off;
      pstride = a.Bt_plane;
    }
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
      *reinterpret_cast<u16x8*>(dst + pl * pstride) =
          *reinterpret_cast<const u16x8*>(s_t + pl * PLANE + ccl * kConvLD + conv_tpos(ccl, g));
  }
}

// State tiles (P/16 x N/16 of 16x16) spread over the NW waves of a workgroup.  When the
// shape allows, each wave owns PER_WAVE tiles of one tile row (ALIGNED), so the x-side operand
// of the state product is read once per K-step and shared by all of the wave's tiles.
template <int P, int N, int NW> struct StateTiles {
  static constexpr int PT = P / 16;
  static constexpr int NT = N / 16;
  static constexpr int TOTAL = PT * NT;
  static constexpr bool ALIGNED = PT <= NW && NW % PT == 0 && NT % (NW / PT) == 0;
  static constexpr int WPR = ALIGNED ? NW / PT : 1;                       // waves per tile row
  static constexpr int PER_WAVE = ALIGNED ? NT / WPR : (TOTAL + NW - 1) / NW;
  __device__ static bool valid(int w, int m) { return ALIGNED || w * PER_WAVE + m < TOTAL; }
  __device__ static int pt(int w, int m) { return ALIGNED ? w / WPR : (w * PER_WAVE + m) / NT; }
  __device__ static int nt(int w, int m) { return ALIGNED ? (w % WPR) * PER_WAVE + m : (w * PER_WAVE + m) % NT; }
};

template <typename TS>
__device__ __forceinline__ void store_state_tile(void* pool, int64_t base, int N, int p, int n, const floatx4& v) {
  TS* d = static_cast<TS*>(pool) + base;
#pragma unroll
  for (int r = 0; r < 4; ++r) d[(int64_t)(p + r) * N + n] = from_f32<TS>(v[r]);
}

// ------------------------------------------------------------------ 2a. conv windows
// The raw inputs of the W-1 rows before position tau of sequence we.seq (from the slot's window,
// or zeros, before the sequence start) into slot we.slot, channels c_first, c_first + c_step, ...
// Checkpoint windows are written by the trailing workgroups of the chunk-state launch, after the
// conv launch has read every initial window; final windows, which overwrite the sequence's own
// slot, by the state-pass launch, after every checkpoint window that reads the initial window.
__device__ __forceinline__ void window_write(const PrefillParams& a, const WindowEntry& we, const SeqEntry& sq,
                                             int c_first, int c_step) {
  const int Cd = a.sh.Cd, I = a.sh.I, GN = a.sh.G * a.sh.N, W1 = a.sh.W - 1;
  for (int c = c_first; c < Cd; c += c_step) {
    const void* src;
    int64_t col, stride;
    if (c < I) { src = a.x; col = c; stride = a.x_stride; }
    else if (c < I + GN) { src = a.B; col = c - I; stride = a.B_stride; }
    else { src = a.C; col = c - I - GN; stride = a.C_stride; }
    float v[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      if (k >= W1) break;
      const int pos = we.tau - W1 + k;
      if (pos >= 0) {
        v[k] = load_any(src, (int64_t)(sq.t0 + pos) * stride + col, a.io_bf16);
      } else if (sq.has_init) {
        const int64_t wi = ((int64_t)sq.slot * Cd + c) * W1 + (W1 + pos);
        v[k] = a.conv_bf16 ? to_f32(static_cast<const bf16*>(a.conv)[wi]) : static_cast<const float*>(a.conv)[wi];
      } else {
        v[k] = 0.f;
      }
    }
    const int64_t wo = ((int64_t)we.slot * Cd + c) * W1;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      if (k >= W1) break;
      if (a.conv_bf16) static_cast<bf16*>(a.conv)[wo + k] = from_f32<bf16>(v[k]);
      else static_cast<float*>(a.conv)[wo + k] = v[k];
    }
  }
}

// ------------------------------------------------------------------ 2b. chunk end states
// Per (chunk, HPW heads of one group), 512 threads: each head's end state from a zero state,
//   S_c = sum_j exp(a_last - a_j) Delta_j x_j B_j^T,
// in MFMA accumulators over staged blocks of kWB tokens, the next block held in registers while
// the current one is used; the group's B block is staged once for the workgroup's heads.
// Written to the chunk-state array through an LDS tile as 16-byte pieces of rows: fp32 with
// hi/lo planes (fp32 state), bf16 otherwise.
constexpr int kWB = kPB;   // one block of the transposed planes

template <bool SPLIT, int P, int N, int HPW> struct WalkLds {
  static constexpr int NPL = SPLIT ? 2 : 1;
  static constexpr int LDX = kWB + 4;   // 34 dwords per row: the 16 rows of a fragment hit distinct banks
  static constexpr int XROWS = HPW * P;                     // x rows of all the workgroup's heads
  static constexpr int XT_OFF = 0;                          // u16 offsets
  static constexpr int BT_OFF = XT_OFF + NPL * XROWS * LDX;
  static constexpr int STAGE_END = BT_OFF + NPL * N * LDX;
  // end-state staging (overlays the blocks): fp32 rows of N + 4, or bf16 rows of N + 8
  static constexpr int LDS_ST = SPLIT ? N + 4 : N + 8;
  static constexpr int ST_END = XROWS * LDS_ST * (SPLIT ? 2 : 1);
  static constexpr int U16S = STAGE_END > ST_END ? STAGE_END : ST_END;
  static constexpr int IT_XT = (XROWS * (kWB / 8) + kStateThreads - 1) / kStateThreads;
  static constexpr int IT_BT = (N * (kWB / 8) + kStateThreads - 1) / kStateThreads;
};

template <bool SPLIT, int P, int N, int HPW>
__global__ __launch_bounds__(kStateThreads) void chunk_state_kernel(PrefillParams a) {
  typedef WalkLds<SPLIT, P, N, HPW> L;
  constexpr int WPH = (kStateThreads / 64) / HPW;   // waves per head
  typedef StateTiles<P, N, WPH> ST;
  constexpr int NPL = L::NPL, LDX = L::LDX;
  __shared__ __align__(16) u16 smem_w[L::U16S];
  __shared__ __align__(16) float sW[HPW * 256];
  u16* const sXT = smem_w + L::XT_OFF;
  u16* const sBT = smem_w + L::BT_OFF;
  const int H = a.sh.H, G = a.sh.G, Q = a.Q;
  const int nh = H / HPW;                      // workgroups per chunk
  const int nmain = a.num_chunks * nh;
  if ((int)blockIdx.x >= nmain) {   // trailing workgroups: conv windows, nh per window
    const int w = blockIdx.x - nmain;
    const WindowEntry we = load_uniform(&a.windows[w / nh]);
    window_write(a, we, load_uniform(&a.seqs[we.seq]), (w % nh) * kStateThreads + threadIdx.x, nh * kStateThreads);
    return;
  }
  // The workgroups of one (chunk, group) read the same B blocks: consecutive logical indices,
  // all on one XCD (one L2), so that the blocks come from memory once.
  const int hpg = (H / G) / HPW;               // workgroups per (chunk, group)
  const int lg = xcd_contiguous(blockIdx.x, nmain);
  const int c = lg / hpg / G, g = lg / hpg % G;
  const int h0 = (g * hpg + lg % hpg) * HPW;
  const ChunkEntry ch = load_uniform(&a.chunks[c]);
  const int len = ch.len;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();
  const int hw = wave / WPH, wh = wave % WPH;   // this wave's head and its index among the head's waves
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t T = a.total_tokens;
  const int64_t PN = (int64_t)P * N;
  const int QB = (Q + kPB - 1) / kPB;

  // x rows of the HPW heads (row r: head r / P, channel r % P; a head's blocks are QB * P * kPB
  // apart), requested like TilePrefetch: branch-free, clamped, masked when stored
  // two register sets, two blocks in flight: set k holds the blocks jb with jb / kWB % 2 == k
  u16x8 xv[2][L::IT_XT][NPL];
  TilePrefetch<NPL, L::IT_BT> pb[2];
  auto prefetch = [&](int k, int jb) {
    const u16* xb = a.xT + (((int64_t)c * H + h0) * QB + jb / kPB) * P * kPB;
#pragma unroll
    for (int it = 0; it < L::IT_XT; ++it) {
      const int idx = tid + it * kStateThreads;
      const int r = idx / (kWB / 8), cc = (idx % (kWB / 8)) * 8;
      const bool in = idx < L::XROWS * (kWB / 8) && cc < len - jb;
      const int off = in ? (r / P) * QB * P * kPB + (r % P) * kPB + cc : 0;
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) xv[k][it][pl] = *reinterpret_cast<const u16x8*>(xb + pl * a.xT_plane + off);
    }
    pb[k].load(a.Bt + (((int64_t)c * G + g) * QB + jb / kPB) * N * kPB, a.Bt_plane, kPB, N, kWB, N, len - jb, tid,
            kStateThreads);
  };
  // weights w_j = exp(a_last - a_j) Delta_j of the chunk's tokens (head tid / 256), requested
  // before the blocks so that their use waits for nothing else
  const int whh = min(tid >> 8, HPW - 1);
  const int64_t wbase = (int64_t)(h0 + whh) * T + ch.t0;
  const int wj = min(tid & 255, len - 1);
  const float aj = a.dA[wbase + wj], dj = a.delta[wbase + wj], alast = a.dA[wbase + len - 1];
  prefetch(0, 0);
  prefetch(1, kWB < len ? kWB : 0);
  if ((tid >> 8) < HPW) sW[tid] = (tid & 255) < len ? __expf(alast - aj) * dj : 0.f;

  floatx4 acc[ST::PER_WAVE];
#pragma unroll
  for (int m = 0; m < ST::PER_WAVE; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int k, int jb) {
    __syncthreads();   // all reads of the previous block are done (and sW is written)
    // x goes to LDS already scaled by w_j (one rounding of the product, as the operand needs),
    // so the K-steps read it as a finished fragment
#pragma unroll
    for (int it = 0; it < L::IT_XT; ++it) {
      const int idx = tid + it * kStateThreads;
      if (idx < L::XROWS * (kWB / 8)) {
        const int r = idx / (kWB / 8), cc = (idx % (kWB / 8)) * 8;
        const float* w = sW + (r / P) * 256 + jb + cc;
        const floatx4 w0 = *reinterpret_cast<const floatx4*>(w);
        const floatx4 w1 = *reinterpret_cast<const floatx4*>(w + 4);
        u16x8 hv, lv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float xf = f_of(xv[k][it][0][e]);
          if (SPLIT) xf += f_of(xv[k][it][NPL - 1][e]);
          xf = jb + cc + e < len ? xf * (e < 4 ? w0[e] : w1[e - 4]) : 0.f;
          u16 hi, lo = 0;
          if (SPLIT) split2(xf, hi, lo);
          else hi = bits_of(from_f32<bf16>(xf));
          hv[e] = hi;
          lv[e] = lo;
        }
        u16* d = sXT + r * LDX + cc;
        *reinterpret_cast<u16x4*>(d) = u16x4{hv[0], hv[1], hv[2], hv[3]};
        *reinterpret_cast<u16x4*>(d + 4) = u16x4{hv[4], hv[5], hv[6], hv[7]};
        if (SPLIT) {
          *reinterpret_cast<u16x4*>(d + L::XROWS * LDX) = u16x4{lv[0], lv[1], lv[2], lv[3]};
          *reinterpret_cast<u16x4*>(d + L::XROWS * LDX + 4) = u16x4{lv[4], lv[5], lv[6], lv[7]};
        }
      }
    }
    pb[k].store(sBT, N * LDX, LDX, N, kWB, N, len - jb, tid, kStateThreads);   // one path: precise waits
    __syncthreads();
    // the block after next into this set; one straight path (past the last block the current
    // one is fetched again and not used)
    prefetch(k, jb + 2 * kWB < len ? jb + 2 * kWB : jb);
    const u16* const sXh = sXT + hw * P * LDX;   // this wave's head
#pragma unroll
    for (int kb = 0; kb < kWB; kb += 32) {
      if (jb + kb >= len) break;
      // x-side operand of tile row pt: (w x)^T over the K-step's tokens, staged scaled
      auto xfrag = [&](int pt) { return lds_frag<SPLIT>(sXh, L::XROWS * LDX, LDX, pt * 16 + l16, kb, q); };
      if (ST::ALIGNED) {
        const Frag<SPLIT> fa = xfrag(ST::pt(wh, 0));
        Frag<SPLIT> fb[ST::PER_WAVE];
#pragma unroll
        for (int m = 0; m < ST::PER_WAVE; ++m)
          fb[m] = lds_frag<SPLIT>(sBT, N * LDX, LDX, ST::nt(wh, m) * 16 + l16, kb, q);
#pragma unroll
        for (int m = 0; m < ST::PER_WAVE; ++m) acc[m] = mma<SPLIT>(fa, fb[m], acc[m]);
      } else {
#pragma unroll
        for (int m = 0; m < ST::PER_WAVE; ++m) {
          if (ST::valid(wh, m)) {
            const Frag<SPLIT> fa = xfrag(ST::pt(wh, m));
            const Frag<SPLIT> fb = lds_frag<SPLIT>(sBT, N * LDX, LDX, ST::nt(wh, m) * 16 + l16, kb, q);
            acc[m] = mma<SPLIT>(fa, fb, acc[m]);
          }
        }
      }
    }
  };
  // a chunk has at most 256 / kWB blocks: straight-line code keeps every wait exact
#pragma unroll
  for (int b = 0; b < 256 / kWB; ++b) {
    if (b * kWB >= len) break;
    step(b & 1, b * kWB);
  }

  // the end states -> LDS rows -> 16-byte stores
  __syncthreads();   // the last block's reads are done before the staging overlays it
#pragma unroll
  for (int m = 0; m < ST::PER_WAVE; ++m) {
    if (ST::valid(wh, m)) {
      const int pt = ST::pt(wh, m), nt = ST::nt(wh, m);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (hw * P + pt * 16 + 4 * q + r) * L::LDS_ST + nt * 16 + l16;
        if (SPLIT) reinterpret_cast<float*>(smem_w)[i] = acc[m][r];
        else smem_w[i] = bits_of(from_f32<bf16>(acc[m][r]));
      }
    }
  }
  __syncthreads();
  constexpr int VPR = SPLIT ? N / 4 : N / 8;   // 16-byte pieces per row
  for (int idx = tid; idx < L::XROWS * VPR; idx += kStateThreads) {
    const int row = idx / VPR, cv = idx % VPR;   // row = head * P + p
    const int64_t o = ((int64_t)c * H + h0) * PN + (int64_t)row * N;   // heads are PN apart
    if (SPLIT) {
      float* dst = static_cast<float*>(a.cstate) + o + cv * 4;
      *reinterpret_cast<floatx4*>(dst) =
          *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(smem_w) + row * L::LDS_ST + cv * 4);
    } else {
      u16* dst = static_cast<u16*>(a.cstate) + o + cv * 8;
      *reinterpret_cast<u16x8*>(dst) = *reinterpret_cast<const u16x8*>(smem_w + row * L::LDS_ST + cv * 8);
    }
  }
}

// ------------------------------------------------------------------ 3. pass over each sequence's chunks
// Per (sequence, head, 2048 state elements), 256 threads of 8 elements each (part 0 also writes the
// sequence's final conv window): the affine step
//   h <- exp(a_last(c)) h + S_c
// through the sequence's chunks from its initial state (the slot's, or zero).  Before each chunk
// the state entering it goes out as the output kernel's bf16 operand planes; after a chunk that
// ends on a checkpoint, and after the last one, the state is rounded into its slot.  Eight
// chunks at a time: their end states and log decays are all requested before the first is used
// (one straight path; past the last chunk the last one is read again and not used).
template <typename TSS, typename TS>
__global__ __launch_bounds__(256) void state_pass_kernel(PrefillParams a) {
  const SeqEntry sq = load_uniform(&a.seqs[blockIdx.x]);
  if (sq.nchunk == 0) return;
  const int h = blockIdx.y, H = a.sh.H;
  if (blockIdx.z == 0) {   // the final conv window, spread over the sequence's H workgroups of part 0
    const WindowEntry we = {(int32_t)blockIdx.x, sq.len, sq.slot, 0};
    window_write(a, we, sq, h * 256 + threadIdx.x, H * 256);
  }
  const int PN = a.sh.P * a.sh.N;
  const int e8 = (blockIdx.z * 256 + threadIdx.x) * 8;
  if (e8 >= PN) return;
  const int64_t head_off = (int64_t)h * PN + e8;
  const int64_t T = a.total_tokens;
  constexpr bool SPLIT = std::is_same<TSS, float>::value;
  float hs[8];
  if (sq.has_init) {
    const TS* src = static_cast<const TS*>(a.ssm) + (int64_t)sq.slot * H * PN + head_off;
#pragma unroll
    for (int e = 0; e < 8; ++e) hs[e] = to_f32(src[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) hs[e] = 0.f;
  }
  auto store_state = [&](int slot) {
    TS* d = static_cast<TS*>(a.ssm) + (int64_t)slot * H * PN + head_off;
    if (std::is_same<TS, float>::value) {
      *reinterpret_cast<floatx4*>(d) = floatx4{hs[0], hs[1], hs[2], hs[3]};
      *reinterpret_cast<floatx4*>(d + 4) = floatx4{hs[4], hs[5], hs[6], hs[7]};
    } else {
      u16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = bits_of(from_f32<bf16>(hs[e]));
      *reinterpret_cast<u16x8*>(d) = o;
    }
  };
  constexpr int D = 8;
  for (int k0 = 0; k0 < sq.nchunk; k0 += D) {
    float sc[D][8], dec[D];
    int ck[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const int c = sq.chunk0 + min(k0 + k, sq.nchunk - 1);
      const ChunkEntry ch = load_uniform(&a.chunks[c]);
      dec[k] = load_uniform(&a.dA[(int64_t)h * T + ch.t0 + ch.len - 1]);
      ck[k] = ch.ckpt_slot;
      const int64_t so = (int64_t)c * H * PN + head_off;
      if (SPLIT) {
        const floatx4 v0 = *reinterpret_cast<const floatx4*>(static_cast<const float*>(a.cstate) + so);
        const floatx4 v1 = *reinterpret_cast<const floatx4*>(static_cast<const float*>(a.cstate) + so + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { sc[k][e] = v0[e]; sc[k][e + 4] = v1[e]; }
      } else {
        const u16x8 v = *reinterpret_cast<const u16x8*>(static_cast<const u16*>(a.cstate) + so);
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[k][e] = f_of(v[e]);
      }
    }
#pragma unroll
    for (int k = 0; k < D; ++k) {
      if (k0 + k >= sq.nchunk) break;
      const int c = sq.chunk0 + k0 + k;
      u16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u16 vh, vl = 0;
        if (SPLIT) split2(hs[e], vh, vl);
        else vh = bits_of(from_f32<bf16>(hs[e]));
        hi[e] = vh;
        lo[e] = vl;
      }
      u16* dst = a.hin + (int64_t)c * H * PN + head_off;
      *reinterpret_cast<u16x8*>(dst) = hi;
      if (SPLIT) *reinterpret_cast<u16x8*>(dst + a.hin_plane) = lo;
      const float decay = __expf(dec[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) hs[e] = decay * hs[e] + sc[k][e];
      if (ck[k] >= 0) store_state(ck[k]);
    }
  }
  store_state(sq.slot);
}

// ------------------------------------------------------------------ 4. chunk outputs
// Per (chunk, head), 512 threads; wave w owns the 16-row tiles w and 15 - w of the chunk
// (equal causal work per wave for Q = 256).  Y = exp(a_i) C_i h_in + (M o L) X + D x, gated.
// Tokens per staged block: two K-steps with single bf16 planes, one with hi/lo planes.
template <bool SPLIT> struct OutBlock { static constexpr int JB = SPLIT ? 32 : 64; };

template <bool SPLIT, int P, int N> struct OutLds {
  static constexpr int kOB = OutBlock<SPLIT>::JB;
  static constexpr int NPL = SPLIT ? 2 : 1;
  // row pitches of 2 (mod 32) dwords: the 16 rows of a fragment read land in distinct banks
  static constexpr int LDH = N + 4;      // entering state [p][n]
  static constexpr int LDB = N + 4;      // B rows [j][n]
  static constexpr int LDX = kOB + 4;    // x transposed [p][j]
  static constexpr int H_OFF = 0;
  static constexpr int BR_OFF = H_OFF + NPL * P * LDH;
  static constexpr int XT_OFF = BR_OFF + NPL * kOB * LDB;
  static constexpr int U16_END = XT_OFF + NPL * P * LDX;
  static constexpr int F_OFF = (U16_END * 2 + 15) / 16 * 16;   // bytes
  // output staging after the products: one 16-row fp32 tile per wave (overlays the above)
  static constexpr int LDO = P + 4;
  static constexpr int OUT_BYTES = 8 * 16 * LDO * 4;
  static constexpr int BYTES = F_OFF + 3 * 256 * 4 > OUT_BYTES ? F_OFF + 3 * 256 * 4 : OUT_BYTES;
  static constexpr int IT_BR = (kOB * (N / 8) + kScanThreads - 1) / kScanThreads;
  static constexpr int IT_XT = (P * (kOB / 8) + kScanThreads - 1) / kScanThreads;
};

// C rows of a wave's two row tiles as B-operand fragments of G^T (zero past the chunk).
template <bool SPLIT, int N, int NK>
__device__ __forceinline__ void load_c_frags(const PrefillParams& a, int c, int g, int len, const int (&rts)[2],
                                             int nrt, int q, int l16, Frag<SPLIT> (&cf)[2][NK]) {
  constexpr int NPL = SPLIT ? 2 : 1;
  const int GN = a.sh.G * N;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int rt = rts[t];
    const int i = rt * 16 + l16;
    const u16* crow = a.Cr + ((int64_t)c * a.Q + i) * GN + g * N;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) {
        u16x4 lo4 = u16x4{0, 0, 0, 0}, hi4 = u16x4{0, 0, 0, 0};
        const int n = ks * 32 + 4 * q;
        if (rt < nrt && i < len) {
          if (n < N) lo4 = *reinterpret_cast<const u16x4*>(crow + pl * a.Cr_plane + n);
          if (n + 16 < N) hi4 = *reinterpret_cast<const u16x4*>(crow + pl * a.Cr_plane + n + 16);
        }
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) { f[e] = bf_of(lo4[e]); f[e + 4] = bf_of(hi4[e]); }
        if (pl == 0) cf[t][ks].hi = f;
        else cf[t][ks].lo = f;
      }
    }
  }
}

// G^T = B C^T for the 32 tokens of a K-step and the 16 rows of one tile (two 16x16 halves).
template <bool SPLIT, int NK>
__device__ __forceinline__ void gt_tile(const Frag<SPLIT> (&cft)[NK], const Frag<SPLIT> (&fb)[2][NK],
                                        floatx4 (&gtt)[2]) {
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    gtt[jt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) gtt[jt] = mma<SPLIT>(fb[jt][ks], cft[ks], gtt[jt]);
  }
}

// Decay mask of one row tile -> the A operand of (M o L) X, with D x riding on the diagonal.
// Below the diagonal (every token of the K-step precedes every row), exp(a_i - a_j) =
// exp(a_i - a_ref) exp(a_ref - a_j) with a_ref the cumsum at the K-step's last token: both
// factors are <= 1, one exp per row and a column table cw.  On the diagonal the exponent is
// taken directly, and entries above it are selected away.
template <bool SPLIT>
__device__ __forceinline__ Frag<SPLIT> decay_mask(const floatx4 (&gtt)[2], int rt, int jk, int len, float aref,
                                                  const float (&cw)[8], const float* sA, const float* sD, float Dh,
                                                  int q, int l16) {
  const int i = rt * 16 + l16;
  const bool row_ok = i < len;
  const float ai = sA[i & 255];
  float mv[8];
  if (jk + 31 < rt * 16) {
    const float rf = row_ok ? __expf(ai - aref) : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) mv[e] = gtt[e >> 2][e & 3] * rf * cw[e];
  } else {
    const floatx4 a0 = *reinterpret_cast<const floatx4*>(&sA[jk + 4 * q]);
    const floatx4 a1 = *reinterpret_cast<const floatx4*>(&sA[jk + 16 + 4 * q]);
    const floatx4 d0 = *reinterpret_cast<const floatx4*>(&sD[jk + 4 * q]);
    const floatx4 d1 = *reinterpret_cast<const floatx4*>(&sD[jk + 16 + 4 * q]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = jk + kmap(q, e);
      const float aj = e < 4 ? a0[e & 3] : a1[e & 3];
      const float dj = e < 4 ? d0[e & 3] : d1[e & 3];
      // branch-free: every factor is finite, so the causal mask is a multiply by 0 or 1
      const float keep = (row_ok && j <= i) ? 1.f : 0.f;
      const float v = gtt[e >> 2][e & 3] * __expf(fminf(ai - aj, 0.f)) * dj + (j == i ? Dh : 0.f);
      mv[e] = v * keep;
    }
  }
  return make_frag<SPLIT>(mv);
}

template <bool SPLIT, int P, int N>
__global__ __launch_bounds__(kScanThreads) void chunk_out_kernel(PrefillParams a) {
  typedef OutLds<SPLIT, P, N> L;
  constexpr int kOB = L::kOB;
  constexpr int NPL = L::NPL;
  constexpr int PT = P / 16;
  constexpr int NK = N / 32 > 0 ? N / 32 : 1;   // K-steps over the state dimension
  extern __shared__ __align__(16) unsigned char smem_raw[];
  u16* const smem = reinterpret_cast<u16*>(smem_raw);
  u16* const sH = smem + L::H_OFF;
  u16* const sBr = smem + L::BR_OFF;
  u16* const sXT = smem + L::XT_OFF;
  float* const sA = reinterpret_cast<float*>(smem_raw + L::F_OFF);
  float* const sD = sA + 256;
  float* const sCw = sD + 256;   // exp(a_ref - a_j) Delta_j, a_ref = cumsum at the last token of j's K-step

  const int c = blockIdx.x;
  const ChunkEntry ch = load_uniform(&a.chunks[c]);
  const int len = ch.len;
  const int h = blockIdx.y, H = a.sh.H, G = a.sh.G, Q = a.Q;
  const int GN = G * N;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t T = a.total_tokens;
  // uniform: held in a scalar register, so no later vector-memory wait depends on it
  const float Dh = load_uniform(&a.D[h]);
  const int nrt = Q / 16;
  const int rts[2] = {wave, 15 - wave};

  TilePrefetch<NPL, L::IT_BR> pbr;
  TilePrefetch<NPL, L::IT_XT> pxt;
  auto prefetch = [&](int jb) {
    pbr.load(a.Br + ((int64_t)c * Q + jb) * GN + g * N, a.Br_plane, GN, kOB, N, len - jb, N, tid, kScanThreads);
    pxt.load(a.xT + (((int64_t)c * H + h) * ((Q + kPB - 1) / kPB) + jb / kPB) * P * kPB + jb % kPB, a.xT_plane,
             kPB, P, kOB, P, len - jb, tid, kScanThreads);
  };
  prefetch(0);

  // C rows of this wave's row tiles as fragments
  Frag<SPLIT> cf[2][NK];
  load_c_frags<SPLIT, N, NK>(a, c, g, len, rts, nrt, q, l16, cf);
  // per-token tables and the entering state
  {
    const float* dAh = a.dA + (int64_t)h * T + ch.t0;
    const float* dh = a.delta + (int64_t)h * T + ch.t0;
    for (int j = tid; j < 256; j += kScanThreads) {
      const bool ok = j < len;
      const float aj = ok ? dAh[j] : 0.f, dj = ok ? dh[j] : 0.f;
      const int jr = min((j | 31), len - 1);   // last token of j's K-step
      sA[j] = aj;
      sD[j] = dj;
      sCw[j] = ok ? __expf(dAh[jr] - aj) * dj : 0.f;
    }
    stage_rows<NPL>(sH, P * L::LDH, L::LDH, a.hin + ((int64_t)c * H + h) * P * N, a.hin_plane, N, P, N, P, N, tid,
                    kScanThreads);
  }
  __syncthreads();

  // Row-tile validity is uniform per wave, so every branch below is a scalar branch and each
  // code path is straight-line MFMA work the compiler can schedule freely.
  const bool v0 = rts[0] < nrt && rts[0] * 16 < len;
  const bool v1 = rts[1] < nrt && rts[1] * 16 < len;

  // the entering-state term exp(a_i) C_i h_in (C fragments of invalid rows are zero)
  floatx4 acc[2][PT];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    acc[0][pt] = floatx4{0.f, 0.f, 0.f, 0.f};
    acc[1][pt] = floatx4{0.f, 0.f, 0.f, 0.f};
    Frag<SPLIT> fh[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      fh[ks] = lds_frag<SPLIT>(sH, P * L::LDH, L::LDH, pt * 16 + l16, N >= 32 ? ks * 32 : 0, q);
      if (N < 32) {   // upper K half is padding
#pragma unroll
        for (int e = 4; e < 8; ++e) { fh[ks].hi[e] = bf_of(0); if (SPLIT) fh[ks].lo[e] = bf_of(0); }
      }
    }
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      acc[0][pt] = mma<SPLIT>(cf[0][ks], fh[ks], acc[0][pt]);
      acc[1][pt] = mma<SPLIT>(cf[1][ks], fh[ks], acc[1][pt]);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ii = rts[t] * 16 + 4 * q + r;
      const float sc = ii < len ? __expf(sA[ii & 255]) : 0.f;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[t][pt][r] *= sc;
    }
  }

  auto gmat = [&](const Frag<SPLIT> (&cft)[NK], const Frag<SPLIT> (&fb)[2][NK], floatx4 (&gtt)[2]) {
    gt_tile<SPLIT, NK>(cft, fb, gtt);
  };
  auto mask = [&](const floatx4 (&gtt)[2], int rt, int jk, float aref, const float (&cw)[8]) {
    return decay_mask<SPLIT>(gtt, rt, jk, len, aref, cw, sA, sD, Dh, q, l16);
  };

  for (int jb = 0; jb < len; jb += kOB) {
    __syncthreads();   // all reads of the previous block are done
    pbr.store(sBr, kOB * L::LDB, L::LDB, kOB, N, len - jb, N, tid, kScanThreads);
    pxt.store(sXT, P * L::LDX, L::LDX, P, kOB, P, len - jb, tid, kScanThreads);
    __syncthreads();
    prefetch(jb + kOB < len ? jb + kOB : jb);   // unconditional: one straight path
#pragma unroll
    for (int kb = 0; kb < kOB; kb += 32) {
      const int jk = jb + kb;   // first token of this K-step
      if (jk >= len) break;
      const bool a0 = v0 && jk <= rts[0] * 16 + 15;
      const bool a1 = v1 && jk <= rts[1] * 16 + 15;
      if (!(a0 || a1)) continue;
      Frag<SPLIT> fb[2][NK];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          fb[jt][ks] = lds_frag<SPLIT>(sBr, kOB * L::LDB, L::LDB, kb + jt * 16 + l16, N >= 32 ? ks * 32 : 0, q);
          if (N < 32) {
#pragma unroll
            for (int e = 4; e < 8; ++e) { fb[jt][ks].hi[e] = bf_of(0); if (SPLIT) fb[jt][ks].lo[e] = bf_of(0); }
          }
        }
      }
      Frag<SPLIT> fx[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) fx[pt] = lds_frag<SPLIT>(sXT, P * L::LDX, L::LDX, pt * 16 + l16, kb, q);
      float cw[8];
      {
        const floatx4 c0 = *reinterpret_cast<const floatx4*>(&sCw[jk + 4 * q]);
        const floatx4 c1 = *reinterpret_cast<const floatx4*>(&sCw[jk + 16 + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) { cw[e] = c0[e]; cw[e + 4] = c1[e]; }
      }
      const float aref = sA[min(jk + 31, len - 1)];
      if (a0 && a1) {
        floatx4 g0[2], g1[2];
        gmat(cf[0], fb, g0);
        gmat(cf[1], fb, g1);
        const Frag<SPLIT> m0 = mask(g0, rts[0], jk, aref, cw);
        const Frag<SPLIT> m1 = mask(g1, rts[1], jk, aref, cw);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          acc[0][pt] = mma<SPLIT>(m0, fx[pt], acc[0][pt]);
          acc[1][pt] = mma<SPLIT>(m1, fx[pt], acc[1][pt]);
        }
      } else if (a1) {
        floatx4 g1[2];
        gmat(cf[1], fb, g1);
        const Frag<SPLIT> m1 = mask(g1, rts[1], jk, aref, cw);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[1][pt] = mma<SPLIT>(m1, fx[pt], acc[1][pt]);
      } else {
        floatx4 g0[2];
        gmat(cf[0], fb, g0);
        const Frag<SPLIT> m0 = mask(g0, rts[0], jk, aref, cw);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[0][pt] = mma<SPLIT>(m0, fx[pt], acc[0][pt]);
      }
    }
  }

  // outputs y = acc * SiLU(z).  Each wave stages one 16-row tile at a time in its own fp32 LDS
  // region and reads it back as 8 consecutive columns per lane, so that z is read and y written
  // with 16-byte accesses (element accesses when the caller's rows are not 16-byte aligned).
  __syncthreads();   // every wave is done with the staged blocks
  float* const sO = reinterpret_cast<float*>(smem_raw) + wave * 16 * L::LDO;
  constexpr int CG = P / 8;   // 8-column groups per row
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int rt = rts[t];
    if (!(t == 0 ? v0 : v1)) continue;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sO[(4 * q + r) * L::LDO + pt * 16 + l16] = acc[t][pt][r];
#pragma unroll
    for (int it = lane; it < 16 * CG; it += 64) {
      const int rr = it / CG, c8 = (it % CG) * 8;
      const int ii = rt * 16 + rr;
      if (ii >= len) continue;
      const floatx4 o0 = *reinterpret_cast<const floatx4*>(&sO[rr * L::LDO + c8]);
      const floatx4 o1 = *reinterpret_cast<const floatx4*>(&sO[rr * L::LDO + c8 + 4]);
      const int64_t row = ch.t0 + ii;
      const int col = h * P + c8;
      float v[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
      if (a.zy_vec) {
        float zf[8];
        load8_any(a.z, row * a.z_stride + col, a.io_bf16, zf);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= silu(zf[e]);
        store8_any(a.y, row * a.y_stride + col, a.y_bf16, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float zv = load_any(a.z, row * a.z_stride + col + e, a.io_bf16);
          store_any(a.y, row * a.y_stride + col + e, v[e] * silu(zv), a.y_bf16);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ 4b. helpers of the grouped output kernel
// 2^x and log2(x) as the bare hardware instructions: results below 2^-126 flush to zero, which
// only drops terms that are negligible against the rest of a sum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ 4c. chunk outputs, a group's heads in turn
// Per (chunk, group, part of the group's heads), 512 threads, single bf16 operand planes.  C B^T
// depends on the chunk and group only: each wave forms its nine (row tile, K-step) slots once,
// from the chunk's B rows staged in LDS and its C rows held as register fragments, and keeps
// them in fp32 registers for all of the workgroup's heads; the same C fragments serve C h_in.
// Heads alternate between two LDS buffers, so one barrier per head suffices: a head's x, entering
// state and Delta values are requested into registers while the previous head is computed.  The
// products are formed transposed, Y^T = h_in^T (exp(a) C)^T + X^T (M o L)^T, so that a lane's
// accumulator holds four consecutive channels of one token: z is read and y written straight from
// registers as pieces of token rows.  Wave w owns the row tiles w and 15 - w.  Decay factors are
// taken as powers of two from per-head tables kept in log2 units:
//   sA2[j] = a_j log2(e),  sB2[j] = a_j log2(e) - log2(Delta_j),  sCw[j] = exp(a_ref - a_j) Delta_j
// (a_ref = the cumsum at the last token of j's K-step); rows past the chunk get sA2 = -inf, so
// every factor of theirs is zero.
template <int P, int N> struct GroupLds {
  static constexpr int QM = 256;
  static constexpr int LDB = N + 4;    // B rows [j][n] (set-up only, overlaid by the buffers)
  static constexpr int LDX = QM + 4;   // x transposed [p][j]
  static constexpr int LDH = N + 4;    // entering state [p][n]
  static constexpr int BUF = P * LDX + P * LDH;   // u16 per head buffer
  static constexpr int U16_END = 2 * BUF > QM * LDB ? 2 * BUF : QM * LDB;
  static constexpr int F_OFF = (U16_END * 2 + 15) / 16 * 16;   // bytes: two sets of sA2, sB2, sCw
  static constexpr int LDO = P + 4;                              // output staging [row][p], fp32
  static constexpr int O_OFF = F_OFF + 2 * 3 * 256 * 4;          // bytes: one 16-row tile per wave
  static constexpr int BYTES = O_OFF + 8 * 16 * LDO * 4;
  static constexpr bool FITS = BYTES <= 160 * 1024 && P <= 64;
  static constexpr int IT_BR = (QM * (N / 8) + 511) / 512;
  static constexpr int IT_XT = (P * (QM / 8) + 511) / 512;
  static constexpr int IT_H = (P * (N / 8) + 511) / 512;
};

template <int P, int N>
__global__ __launch_bounds__(512) void chunk_out_group_kernel(PrefillParams a, int heads_per_wg) {
  typedef GroupLds<P, N> L;
  constexpr int PT = P / 16;
  constexpr int NK = N / 32 > 0 ? N / 32 : 1;
  constexpr float kLog2e = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  u16* const smem = reinterpret_cast<u16*>(smem_raw);
  float* const ftab = reinterpret_cast<float*>(smem_raw + L::F_OFF);

  const int c = blockIdx.x;
  const ChunkEntry ch = load_uniform(&a.chunks[c]);
  const int len = ch.len;
  const int H = a.sh.H, G = a.sh.G, Q = a.Q, GN = G * N;
  const int hpg = H / G;
  const int parts = hpg / heads_per_wg;
  const int g = blockIdx.y / parts;
  const int h0 = g * hpg + (blockIdx.y % parts) * heads_per_wg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t T = a.total_tokens;
  const int nrt = Q / 16;
  const int rts[2] = {wave, 15 - wave};
  const bool vt[2] = {rts[0] < nrt && rts[0] * 16 < len, rts[1] < nrt && rts[1] * 16 < len};
  const int QB = (Q + kPB - 1) / kPB;
  const bool zpre = a.io_bf16 && a.zy_vec;
  const int m0 = wave >> 1;
  const int mt[2] = {m0, 7 - m0};   // K-steps below each tile; K-step mt[t] holds its diagonal
  constexpr int CG = P / 8;                   // 8-channel groups of an output row
  constexpr int ZI = (16 * CG + 63) / 64;     // output items (8 channels of one token) per lane per tile
  float* const sO = reinterpret_cast<float*>(smem_raw + L::O_OFF) + wave * 16 * L::LDO;

  TilePrefetch<1, L::IT_XT> px;
  TilePrefetch<1, L::IT_H> ph;
  float pa, pd, pr;
  auto prefetch = [&](int h) {
    px.load(a.xT + ((int64_t)c * H + h) * QB * P * kPB, 0, kPB, QB * P, kPB, QB * P, kPB, tid, 512);
    ph.load(a.hin + ((int64_t)c * H + h) * P * N, 0, N, P, N, P, N, tid, 512);
    const int j = min(tid, len - 1);
    const float* dAh = a.dA + (int64_t)h * T + ch.t0;
    pa = dAh[j];
    pd = a.delta[(int64_t)h * T + ch.t0 + j];
    pr = dAh[min(j | 31, len - 1)];
  };
  prefetch(h0);

  // C B^T slots, fp32: below-diagonal slots of tile 0 in gb[0 .. m0-1] and of tile 1 from gb[6]
  // downwards (constant indices for both tiles), the diagonal slots in gd
  Frag<false> cf[2][NK];
  floatx4 gb[7][2], gd[2][2];
  {
    u16* const sBr = smem;
    TilePrefetch<1, L::IT_BR> pb;
    pb.load(a.Br + (int64_t)c * Q * GN + g * N, 0, GN, L::QM, N, len, N, tid, 512);
    load_c_frags<false, N, NK>(a, c, g, len, rts, nrt, q, l16, cf);
    pb.store(sBr, 0, L::LDB, L::QM, N, len, N, tid, 512);
    __syncthreads();
    auto slot = [&](int t, int ks, floatx4 (&out)[2]) {
      Frag<false> fb[2][NK];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          fb[jt][kk] = lds_frag<false>(sBr, 0, L::LDB, 32 * ks + jt * 16 + l16, N >= 32 ? kk * 32 : 0, q);
          if (N < 32) {
#pragma unroll
            for (int e = 4; e < 8; ++e) fb[jt][kk].hi[e] = bf_of(0);
          }
        }
      }
      if (t == 0) gt_tile<false, NK>(cf[0], fb, out);
      else gt_tile<false, NK>(cf[1], fb, out);
    };
#pragma unroll
    for (int k = 0; k < 7; ++k) {
      gb[k][0] = gb[k][1] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (k < m0) {
        if (vt[0]) slot(0, k, gb[k]);
      } else if (vt[1]) {
        slot(1, 6 - k, gb[k]);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      gd[t][0] = gd[t][1] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (vt[t]) slot(t, mt[t], gd[t]);
    }
    __syncthreads();   // B rows are overwritten by the head buffers below
  }

  for (int hh = 0; hh < heads_per_wg; ++hh) {
    const int h = h0 + hh;
    u16* const sXT = smem + (hh & 1) * L::BUF;
    u16* const sH = sXT + P * L::LDX;
    float* const sA2 = ftab + (hh & 1) * 768;
    float* const sB2 = sA2 + 256;
    float* const sCw = sB2 + 256;
    // this head's x blocks [QB][P][kPB] -> sXT[p][token] (tokens past the chunk zeroed), its
    // entering state and its tables, into the buffer last read two heads ago
    if (len == QB * kPB) {
#pragma unroll
      for (int it = 0; it < L::IT_XT; ++it) {
        const int idx = tid + it * 512;
        const int r = idx / (kPB / 8), cc = (idx % (kPB / 8)) * 8;
        if (r < QB * P) {
          const u16x8 x = px.v[it][0];
          u16* d = sXT + (r % P) * L::LDX + (r / P) * kPB + cc;
          *reinterpret_cast<u16x4*>(d) = u16x4{x[0], x[1], x[2], x[3]};
          *reinterpret_cast<u16x4*>(d + 4) = u16x4{x[4], x[5], x[6], x[7]};
        }
      }
    } else {
#pragma unroll
      for (int it = 0; it < L::IT_XT; ++it) {
        const int idx = tid + it * 512;
        const int r = idx / (kPB / 8), cc = (idx % (kPB / 8)) * 8;
        if (r < QB * P) {
          const int j = (r / P) * kPB + cc;
          u16x8 x = px.v[it][0];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = j + e < len ? x[e] : u16(0);
          u16* d = sXT + (r % P) * L::LDX + j;
          *reinterpret_cast<u16x4*>(d) = u16x4{x[0], x[1], x[2], x[3]};
          *reinterpret_cast<u16x4*>(d + 4) = u16x4{x[4], x[5], x[6], x[7]};
        }
      }
    }
    ph.store(sH, 0, L::LDH, P, N, P, N, tid, 512);
    if (tid < 256) {
      const bool ok = tid < len;
      sA2[tid] = ok ? pa * kLog2e : -INFINITY;
      sB2[tid] = ok ? pa * kLog2e - __builtin_amdgcn_logf(pd) : 0.f;
      sCw[tid] = ok ? fast_exp2((pr - pa) * kLog2e) * pd : 0.f;
    }
    __syncthreads();
    const float Dh = load_uniform(&a.D[h]);
    // z of both tiles as 16-byte row pieces (the output items below), then the next head's
    // operands (unconditional: one straight path); rows past the chunk read the chunk's first row
    u16x8 zr[2][ZI];
    if (zpre) {
      const u16* zbase = static_cast<const u16*>(a.z) + ch.t0 * a.z_stride + h * P;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int k = 0; k < ZI; ++k) {
          const int it = min(lane + 64 * k, 16 * CG - 1);
          const int ii = rts[t] * 16 + it / CG;
          zr[t][k] = *reinterpret_cast<const u16x8*>(zbase + (ii < len ? ii : 0) * (int)a.z_stride + (it % CG) * 8);
        }
      }
    }
    prefetch(min(h + 1, h0 + heads_per_wg - 1));

#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!vt[t]) continue;
      const int rt = rts[t];
      const int i = rt * 16 + l16;
      const float a2i = sA2[i];
      // exp(a_i) h_in^T C_i^T first (state dimension in the kmap order of the C fragments), then
      // (M o L) X accumulates on top
      floatx4 acc[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          Frag<false> fh = lds_frag<false>(sH, 0, L::LDH, pt * 16 + l16, N >= 32 ? ks * 32 : 0, q);
          if (N < 32) {
#pragma unroll
            for (int e = 4; e < 8; ++e) fh.hi[e] = bf_of(0);
          }
          acc[pt] = mfma_bf16(fh.hi, cf[t][ks].hi, acc[pt]);
        }
      }
      {
        const float sc = fast_exp2(a2i);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pt][r] *= sc;
      }

      // (M o L) X over the K-steps entirely below the tile: exp(a_i - a_j) = 2^(a2_i - a2_ref)
      // times the column factor, with a_ref the cumsum at the K-step's last token (both <= 1)
#pragma unroll
      for (int k = 0; k < 7; ++k) {
        if (k >= mt[t]) break;
        const int jk = 32 * k;
        Frag<false> fx[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) fx[pt] = lds_frag<false>(sXT, 0, L::LDX, pt * 16 + l16, jk, q);
        const floatx4 c0 = *reinterpret_cast<const floatx4*>(&sCw[jk + 4 * q]);
        const floatx4 c1 = *reinterpret_cast<const floatx4*>(&sCw[jk + 16 + 4 * q]);
        const float rf = fast_exp2(a2i - sA2[jk + 31]);
        const floatx4(&gs)[2] = t == 0 ? gb[k] : gb[6 - k];
        float mv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mv[e] = gs[0][e] * (rf * c0[e]);
          mv[e + 4] = gs[1][e] * (rf * c1[e]);
        }
        const Frag<false> mf = make_frag<false>(mv);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = mfma_bf16(fx[pt].hi, mf.hi, acc[pt]);
      }

      // the diagonal K-step: the 16-token block on the diagonal takes its exponents directly, with
      // the causal mask and D x on the diagonal; the other block lies entirely below the tile (odd
      // tiles, direct exponents) or entirely above it (even tiles, zero)
      {
        const int jk = 32 * mt[t];
        Frag<false> fx[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) fx[pt] = lds_frag<false>(sXT, 0, L::LDX, pt * 16 + l16, jk, q);
        const int dsel = l16 - 4 * q;
        const floatx4 bd = *reinterpret_cast<const floatx4*>(&sB2[16 * rt + 4 * q]);
        float mv[8];
        if (rt & 1) {
          const floatx4 bb = *reinterpret_cast<const floatx4*>(&sB2[jk + 4 * q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = fast_exp2(a2i - bd[e]) * gd[t][1][e];
            mv[e + 4] = (e <= dsel ? v : 0.f) + (e == dsel ? Dh : 0.f);
            mv[e] = fast_exp2(a2i - bb[e]) * gd[t][0][e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = fast_exp2(a2i - bd[e]) * gd[t][0][e];
            mv[e] = (e <= dsel ? v : 0.f) + (e == dsel ? Dh : 0.f);
            mv[e + 4] = 0.f;
          }
        }
        const Frag<false> mf = make_frag<false>(mv);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = mfma_bf16(fx[pt].hi, mf.hi, acc[pt]);
      }

      // y = acc * SiLU(z) through this wave's LDS tile: the accumulators go in as 16-byte pieces
      // of token rows, and eight lanes then cover one row's channels, so z and y move as 16-byte
      // pieces of whole rows
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) *reinterpret_cast<floatx4*>(&sO[l16 * L::LDO + pt * 16 + 4 * q]) = acc[pt];
#pragma unroll
      for (int k = 0; k < ZI; ++k) {
        const int it = lane + 64 * k;
        if (it >= 16 * CG) continue;
        const int rr = it / CG, c8 = (it % CG) * 8;
        const int ii = rt * 16 + rr;
        if (ii >= len) continue;
        const floatx4 o0 = *reinterpret_cast<const floatx4*>(&sO[rr * L::LDO + c8]);
        const floatx4 o1 = *reinterpret_cast<const floatx4*>(&sO[rr * L::LDO + c8 + 4]);
        float v[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
        const int64_t row = ch.t0 + ii + opaque_uniform(0);   // keeps these addresses inside the loop
        const int col = h * P + c8;
        if (zpre) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= silu(f_of(zr[t][k][e]));
          store8_any(a.y, row * a.y_stride + col, a.y_bf16, v);
        } else if (a.zy_vec) {
          float zf[8];
          load8_any(a.z, row * a.z_stride + col, a.io_bf16, zf);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= silu(zf[e]);
          store8_any(a.y, row * a.y_stride + col, a.y_bf16, v);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float zv = load_any(a.z, row * a.z_stride + col + e, a.io_bf16);
            store_any(a.y, row * a.y_stride + col + e, v[e] * silu(zv), a.y_bf16);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ 4d. chunk outputs with hi/lo planes, a group's heads in turn
// fp32 state: every operand is a bf16 hi plane plus a lo plane and each product takes three
// MFMAs.  Per (chunk, group, part of the group's heads), 512 threads, as the single-plane kernel
// above, with what the doubled operands leave room for: C B^T is formed once per workgroup (split
// products) and kept in fp32 registers; the C fragments of C h_in are read per head, state
// dimension contiguous per lane; one LDS buffer (x, entering state and output staging take
// 136 KB), so a head's operands are requested while the previous head writes its last tile.
template <int P, int N> struct GroupSplitLds {
  static constexpr int QM = 256;
  static constexpr int LDB = N + 4;      // B rows [j][n], hi and lo (set-up only, overlaid below)
  static constexpr int LDX = QM + 4;     // x transposed [p][j], hi and lo
  static constexpr int LDH = N + 8;      // entering state [p][n], hi and lo, 16-byte aligned rows
  static constexpr int LDO = P + 4;      // output staging [row][p], fp32, one 16-row tile per wave
  static constexpr int XPL = P * LDX;    // u16 plane strides
  static constexpr int HPL = P * LDH;
  static constexpr int H_OFF = 2 * XPL;  // u16 offsets
  static constexpr int O_OFF = H_OFF + 2 * HPL;
  static constexpr int HEAD_END = O_OFF + 8 * 16 * LDO * 2;   // fp32 staging counted in u16
  static constexpr int SETUP_END = 2 * QM * LDB;
  static constexpr int U16_END = HEAD_END > SETUP_END ? HEAD_END : SETUP_END;
  static constexpr int F_OFF = (U16_END * 2 + 15) / 16 * 16;   // bytes: sA2, sB2, sCw
  static constexpr int BYTES = F_OFF + 3 * 256 * 4;
  static constexpr bool FITS = BYTES <= 160 * 1024 && P <= 64;
  static constexpr int IT_BR = (QM * (N / 8) + 511) / 512;
  static constexpr int IT_XT = (P * (QM / 8) + 511) / 512;
  static constexpr int IT_H = (P * (N / 8) + 511) / 512;
};

template <int P, int N>
__global__ __launch_bounds__(512) void chunk_out_group_split_kernel(PrefillParams a, int heads_per_wg) {
  typedef GroupSplitLds<P, N> L;
  constexpr int PT = P / 16;
  constexpr int NK = N / 32 > 0 ? N / 32 : 1;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr int CG = P / 8;                   // 8-channel groups of an output row
  constexpr int ZI = (16 * CG + 63) / 64;     // output items (8 channels of one token) per lane per tile
  extern __shared__ __align__(16) unsigned char smem_raw[];
  u16* const smem = reinterpret_cast<u16*>(smem_raw);

  const int c = blockIdx.x;
  const ChunkEntry ch = load_uniform(&a.chunks[c]);
  const int len = ch.len;
  const int H = a.sh.H, G = a.sh.G, Q = a.Q, GN = G * N;
  const int hpg = H / G;
  const int parts = hpg / heads_per_wg;
  const int g = blockIdx.y / parts;
  const int h0 = g * hpg + (blockIdx.y % parts) * heads_per_wg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t T = a.total_tokens;
  const int nrt = Q / 16;
  const int rts[2] = {wave, 15 - wave};
  const bool vt[2] = {rts[0] < nrt && rts[0] * 16 < len, rts[1] < nrt && rts[1] * 16 < len};
  const int QB = (Q + kPB - 1) / kPB;
  const int m0 = wave >> 1;
  const int mt[2] = {m0, 7 - m0};   // K-steps below each tile; K-step mt[t] holds its diagonal

  TilePrefetch<2, L::IT_XT> px;
  TilePrefetch<2, L::IT_H> ph;
  float pa, pd, pr;
  auto prefetch = [&](int h) {
    px.load(a.xT + ((int64_t)c * H + h) * QB * P * kPB, a.xT_plane, kPB, QB * P, kPB, QB * P, kPB, tid, 512);
    ph.load(a.hin + ((int64_t)c * H + h) * P * N, a.hin_plane, N, P, N, P, N, tid, 512);
    const int j = min(tid, len - 1);
    const float* dAh = a.dA + (int64_t)h * T + ch.t0;
    pa = dAh[j];
    pd = a.delta[(int64_t)h * T + ch.t0 + j];
    pr = dAh[min(j | 31, len - 1)];
  };
  prefetch(h0);

  // C B^T slots in fp32 (split products): below-diagonal slots of tile 0 in gb[0 .. m0-1] and of
  // tile 1 from gb[6] downwards, the diagonal slots in gd
  floatx4 gb[7][2], gd[2][2];
  {
    u16* const sBr = smem;
    TilePrefetch<2, L::IT_BR> pb;
    pb.load(a.Br + (int64_t)c * Q * GN + g * N, a.Br_plane, GN, L::QM, N, len, N, tid, 512);
    Frag<true> cf[2][NK];
    load_c_frags<true, N, NK>(a, c, g, len, rts, nrt, q, l16, cf);
    pb.store(sBr, L::QM * L::LDB, L::LDB, L::QM, N, len, N, tid, 512);
    __syncthreads();
    auto slot = [&](int t, int ks, floatx4 (&out)[2]) {
      Frag<true> fb[2][NK];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          fb[jt][kk] = lds_frag<true>(sBr, L::QM * L::LDB, L::LDB, 32 * ks + jt * 16 + l16, N >= 32 ? kk * 32 : 0, q);
          if (N < 32) {
#pragma unroll
            for (int e = 4; e < 8; ++e) { fb[jt][kk].hi[e] = bf_of(0); fb[jt][kk].lo[e] = bf_of(0); }
          }
        }
      }
      if (t == 0) gt_tile<true, NK>(cf[0], fb, out);
      else gt_tile<true, NK>(cf[1], fb, out);
    };
#pragma unroll
    for (int k = 0; k < 7; ++k) {
      gb[k][0] = gb[k][1] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (k < m0) {
        if (vt[0]) slot(0, k, gb[k]);
      } else if (vt[1]) {
        slot(1, 6 - k, gb[k]);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      gd[t][0] = gd[t][1] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (vt[t]) slot(t, mt[t], gd[t]);
    }
  }

  const u16* const cbase = a.Cr + (int64_t)c * Q * GN + g * N;
  for (int hh = 0; hh < heads_per_wg; ++hh) {
    const int h = h0 + hh;
    // LDS bases through an opaque zero: the per-lane addresses derived from them stay inside the
    // head loop instead of being hoisted out of it and spilled
    const int zo = opaque_uniform(0);
    u16* const sXT = smem + zo;
    u16* const sH = smem + L::H_OFF + zo;
    float* const sA2 = reinterpret_cast<float*>(smem_raw + L::F_OFF) + zo;
    float* const sB2 = sA2 + 256;
    float* const sCw = sB2 + 256;
    float* const sO = reinterpret_cast<float*>(smem + L::O_OFF) + wave * 16 * L::LDO + zo;
    __syncthreads();   // the set-up or the previous head is done with the LDS buffer
    // this head's x blocks [QB][P][kPB] -> sXT[p][token] (hi, lo; tokens past the chunk zeroed),
    // its entering state and its tables
#pragma unroll
    for (int it = 0; it < L::IT_XT; ++it) {
      const int idx = tid + it * 512;
      const int r = idx / (kPB / 8), cc = (idx % (kPB / 8)) * 8;
      if (r < QB * P) {
        const int j = (r / P) * kPB + cc;
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
          u16x8 x = px.v[it][pl];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = j + e < len ? x[e] : u16(0);
          u16* d = sXT + pl * L::XPL + (r % P) * L::LDX + j;
          *reinterpret_cast<u16x4*>(d) = u16x4{x[0], x[1], x[2], x[3]};
          *reinterpret_cast<u16x4*>(d + 4) = u16x4{x[4], x[5], x[6], x[7]};
        }
      }
    }
    ph.store(sH, L::HPL, L::LDH, P, N, P, N, tid, 512);
    if (tid < 256) {
      const bool ok = tid < len;
      sA2[tid] = ok ? pa * kLog2e : -INFINITY;
      sB2[tid] = ok ? pa * kLog2e - __builtin_amdgcn_logf(pd) : 0.f;
      sCw[tid] = ok ? fast_exp2((pr - pa) * kLog2e) * pd : 0.f;
    }
    __syncthreads();
    const float Dh = load_uniform(&a.D[h]);
    const bool zpre = a.io_bf16 && a.zy_vec;

#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!vt[t]) continue;
      const int rt = rts[t];
      const int i = rt * 16 + l16;
      const float a2i = sA2[i];
      // z of this tile (bf16 io: 16-byte row pieces, the output items below)
      u16x8 zr[ZI];
      if (zpre) {
        const u16* zbase = static_cast<const u16*>(a.z) + ch.t0 * a.z_stride + h * P;
#pragma unroll
        for (int k = 0; k < ZI; ++k) {
          const int it = min(lane + 64 * k, 16 * CG - 1);
          const int ii = rt * 16 + it / CG;
          zr[k] = *reinterpret_cast<const u16x8*>(zbase + (ii < len ? ii : 0) * (int)a.z_stride + (it % CG) * 8);
        }
      }
      // exp(a_i) h_in^T C_i^T: C row i from global (hi, lo), n = 32 ks + 8 q .. + 7
      floatx4 acc[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
      {
        const int ii = i < len ? i : 0;
        Frag<true> fc[NK];
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const int n = ks * 32 + 8 * q;
          const u16* cr = cbase + ii * GN + (n < N ? n : 0);
          const u16x8 ch8 = *reinterpret_cast<const u16x8*>(cr);
          const u16x8 cl8 = *reinterpret_cast<const u16x8*>(cr + a.Cr_plane);
          const bool ok = n < N && i < len;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            fc[ks].hi[e] = bf_of(ok ? ch8[e] : u16(0));
            fc[ks].lo[e] = bf_of(ok ? cl8[e] : u16(0));
          }
        }
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const int n = ks * 32 + 8 * q;
          const bool ok = n < N;
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
            const u16* hp = sH + (pt * 16 + l16) * L::LDH + (ok ? n : 0);
            const u16x8 hh8 = *reinterpret_cast<const u16x8*>(hp);
            const u16x8 hl8 = *reinterpret_cast<const u16x8*>(hp + L::HPL);
            Frag<true> fh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              fh.hi[e] = bf_of(ok ? hh8[e] : u16(0));
              fh.lo[e] = bf_of(ok ? hl8[e] : u16(0));
            }
            acc[pt] = mma<true>(fh, fc[ks], acc[pt]);
          }
        }
        const float sc = fast_exp2(a2i);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pt][r] *= sc;
      }

      // (M o L) X below the diagonal: exp(a_i - a_j) = 2^(a2_i - a2_ref) times the column factor
#pragma unroll
      for (int k = 0; k < 7; ++k) {
        if (k >= mt[t]) break;
        const int jk = 32 * k;
        Frag<true> fx[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) fx[pt] = lds_frag<true>(sXT, L::XPL, L::LDX, pt * 16 + l16, jk, q);
        const floatx4 c0 = *reinterpret_cast<const floatx4*>(&sCw[jk + 4 * q]);
        const floatx4 c1 = *reinterpret_cast<const floatx4*>(&sCw[jk + 16 + 4 * q]);
        const float rf = fast_exp2(a2i - sA2[jk + 31]);
        const floatx4(&gs)[2] = t == 0 ? gb[k] : gb[6 - k];
        float mv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mv[e] = gs[0][e] * (rf * c0[e]);
          mv[e + 4] = gs[1][e] * (rf * c1[e]);
        }
        const Frag<true> mf = make_frag<true>(mv);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = mma<true>(fx[pt], mf, acc[pt]);
      }

      // the diagonal K-step (as in the single-plane kernel)
      {
        const int jk = 32 * mt[t];
        Frag<true> fx[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) fx[pt] = lds_frag<true>(sXT, L::XPL, L::LDX, pt * 16 + l16, jk, q);
        const int dsel = l16 - 4 * q;
        const floatx4 bd = *reinterpret_cast<const floatx4*>(&sB2[16 * rt + 4 * q]);
        float mv[8];
        if (rt & 1) {
          const floatx4 bb = *reinterpret_cast<const floatx4*>(&sB2[jk + 4 * q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = fast_exp2(a2i - bd[e]) * gd[t][1][e];
            mv[e + 4] = (e <= dsel ? v : 0.f) + (e == dsel ? Dh : 0.f);
            mv[e] = fast_exp2(a2i - bb[e]) * gd[t][0][e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = fast_exp2(a2i - bd[e]) * gd[t][0][e];
            mv[e] = (e <= dsel ? v : 0.f) + (e == dsel ? Dh : 0.f);
            mv[e + 4] = 0.f;
          }
        }
        const Frag<true> mf = make_frag<true>(mv);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = mma<true>(fx[pt], mf, acc[pt]);
      }

      // the next head's operands go out before this workgroup's last tile is written (the last
      // reads of x and h are behind; they land in LDS after the next barrier)
      if (t == 1 || !vt[1]) prefetch(min(h + 1, h0 + heads_per_wg - 1));

      // y = acc * SiLU(z) through this wave's LDS tile, z and y as 16-byte row pieces
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) *reinterpret_cast<floatx4*>(&sO[l16 * L::LDO + pt * 16 + 4 * q]) = acc[pt];
#pragma unroll
      for (int k = 0; k < ZI; ++k) {
        const int it = lane + 64 * k;
        if (it >= 16 * CG) continue;
        const int rr = it / CG, c8 = (it % CG) * 8;
        const int ii = rt * 16 + rr;
        if (ii >= len) continue;
        const floatx4 o0 = *reinterpret_cast<const floatx4*>(&sO[rr * L::LDO + c8]);
        const floatx4 o1 = *reinterpret_cast<const floatx4*>(&sO[rr * L::LDO + c8 + 4]);
        float v[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
        const int64_t row = ch.t0 + ii + opaque_uniform(0);   // keeps these addresses inside the loop
        const int col = h * P + c8;
        if (zpre) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= silu(f_of(zr[k][e]));
          store8_any(a.y, row * a.y_stride + col, a.y_bf16, v);
        } else if (a.zy_vec) {
          float zf[8];
          load8_any(a.z, row * a.z_stride + col, a.io_bf16, zf);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= silu(zf[e]);
          store8_any(a.y, row * a.y_stride + col, a.y_bf16, v);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float zv = load_any(a.z, row * a.z_stride + col + e, a.io_bf16);
            store_any(a.y, row * a.y_stride + col + e, v[e] * silu(zv), a.y_bf16);
          }
        }
      }
    }
    if (!vt[0] && !vt[1]) prefetch(min(h + 1, h0 + heads_per_wg - 1));   // waves with no tile
  }
}

// ------------------------------------------------------------------ launch
// Allow `bytes` of dynamic LDS for a kernel (idempotent; called before each launch).
static hipError_t set_lds_attr(const void* fn, int bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// Workgroups per (chunk, group) of the grouped output kernels: the whole group in one unless
// that leaves CUs idle (then the group's heads are split evenly).
static int group_parts(const PrefillParams& a) {
  static int num_cu = 0;
  if (num_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || num_cu < 1)
      num_cu = 256;
  }
  const int hpg = a.sh.H / a.sh.G;
  int parts = 1;
  while ((int64_t)a.num_chunks * a.sh.G * parts < num_cu && parts < hpg) {
    int next = parts + 1;
    while (hpg % next != 0) ++next;
    parts = next;
  }
  return parts;
}

template <bool SPLIT, int P, int N>
static hipError_t launch_states_and_outputs(const PrefillParams& a, hipStream_t s) {
  // two heads of a group per workgroup share the staged B blocks; one with hi/lo planes (two
  // measured no faster there)
  bool two = false;
  if constexpr (!SPLIT) {
    if ((a.sh.H / a.sh.G) % 2 == 0) {
      two = true;
      hipLaunchKernelGGL((chunk_state_kernel<SPLIT, P, N, 2>), dim3((a.num_chunks + a.num_windows) * (a.sh.H / 2)),
                         dim3(kStateThreads), 0, s, a);
    }
  }
  if (!two)
    hipLaunchKernelGGL((chunk_state_kernel<SPLIT, P, N, 1>), dim3((a.num_chunks + a.num_windows) * a.sh.H),
                       dim3(kStateThreads), 0, s, a);
  const dim3 gp(a.num_seqs, a.sh.H, (P * N / 8 + 255) / 256);
  // hi/lo planes go with fp32 state: fp32 chunk states; bf16 state: bf16 chunk states
  if (SPLIT) hipLaunchKernelGGL((state_pass_kernel<float, float>), gp, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((state_pass_kernel<bf16, bf16>), gp, dim3(256), 0, s, a);
  if (!SPLIT && GroupLds<P, N>::FITS) {
    const int hpg = a.sh.H / a.sh.G;
    const int parts = group_parts(a);
    typedef GroupLds<P, N> L;
    const hipError_t e = set_lds_attr(reinterpret_cast<const void*>(&chunk_out_group_kernel<P, N>), L::BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_out_group_kernel<P, N>), dim3(a.num_chunks, a.sh.G * parts), dim3(512), L::BYTES, s, a,
                       hpg / parts);
    return hipSuccess;
  }
  if (SPLIT && GroupSplitLds<P, N>::FITS) {
    typedef GroupSplitLds<P, N> L;
    const hipError_t e = set_lds_attr(reinterpret_cast<const void*>(&chunk_out_group_split_kernel<P, N>), L::BYTES);
    if (e != hipSuccess) return e;
    const int hpg = a.sh.H / a.sh.G;
    hipLaunchKernelGGL((chunk_out_group_split_kernel<P, N>), dim3(a.num_chunks, a.sh.G * group_parts(a)), dim3(512),
                       L::BYTES, s, a, hpg / group_parts(a));
    return hipSuccess;
  }
  typedef OutLds<SPLIT, P, N> L;
  const hipError_t e = set_lds_attr(reinterpret_cast<const void*>(&chunk_out_kernel<SPLIT, P, N>), L::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_out_kernel<SPLIT, P, N>), dim3(a.num_chunks, a.sh.H), dim3(kScanThreads), L::BYTES, s,
                     a);
  return hipSuccess;
}

template <int P, int N>
static hipError_t launch_pn(const PrefillParams& a, hipStream_t s) {
  return a.ssm_bf16 ? launch_states_and_outputs<false, P, N>(a, s) : launch_states_and_outputs<true, P, N>(a, s);
}

template <int P>
static hipError_t launch_p(const PrefillParams& a, hipStream_t s) {
  switch (a.sh.N) {
    case 16: return launch_pn<P, 16>(a, s);
    case 32: return launch_pn<P, 32>(a, s);
    case 64: return launch_pn<P, 64>(a, s);
    case 128: return launch_pn<P, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

bool prefill_supported(int P, int N, int W) {
  const bool p_ok = P == 16 || P == 32 || P == 64 || P == 128;
  const bool n_ok = N == 16 || N == 32 || N == 64 || N == 128;
  return p_ok && n_ok && W >= 2 && W <= 4;
}

hipError_t launch_prefill(const PrefillParams& a, const InlineTables* inl, hipStream_t s) {
  if (a.num_chunks == 0) return hipSuccess;
  if (a.tab_inline < 0 || a.tab_inline > kInlineTableBytes || a.tab_inline % 16 != 0 || (a.tab_inline > 0 && !inl))
    return hipErrorInvalidValue;
  ConvArgs ca;
  ca.p = a;
  if (a.tab_inline > 0) memcpy(&ca.t, inl, (size_t)a.tab_inline);
  // Delta/cumsum workgroups first, then (chunk, token part, channel block) with the channel block
  // fastest, then the table copy
  const unsigned per_chunk = (unsigned)((a.sh.H + 3) / 4 + (a.sh.Cd + kConvCB - 1) / kConvCB * kConvNH);
  const dim3 gc((unsigned)a.num_chunks * per_chunk + (a.tab_inline > 0 ? 1u : 0u));
  const bool split = !a.ssm_bf16;
  hipError_t ea = hipSuccess;
#define M2_CONV_IO(WW, SP, IO)                                                                           \
  {                                                                                                      \
    ea = set_lds_attr(reinterpret_cast<const void*>(&conv_kernel<WW, SP, IO>), ConvLds<SP>::BYTES);      \
    hipLaunchKernelGGL((conv_kernel<WW, SP, IO>), gc, dim3(256), ConvLds<SP>::BYTES, s, ca);             \
  }
#define M2_CONV(WW)                                                                                       \
  if (split) {                                                                                            \
    if (a.io_bf16) M2_CONV_IO(WW, true, true) else M2_CONV_IO(WW, true, false)                            \
  } else {                                                                                                \
    if (a.io_bf16) M2_CONV_IO(WW, false, true) else M2_CONV_IO(WW, false, false)                          \
  }
  switch (a.sh.W) {
    case 2: M2_CONV(2) break;
    case 3: M2_CONV(3) break;
    case 4: M2_CONV(4) break;
    default: return hipErrorInvalidValue;
  }
#undef M2_CONV
#undef M2_CONV_IO
  if (ea != hipSuccess) return ea;
  hipError_t e = hipErrorInvalidValue;
  switch (a.sh.P) {
    case 16: e = launch_p<16>(a, s); break;
    case 32: e = launch_p<32>(a, s); break;
    case 64: e = launch_p<64>(a, s); break;
    case 128: e = launch_p<128>(a, s); break;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace m2
