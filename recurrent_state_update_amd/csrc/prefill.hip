// Chunked (SSD) prefill of packed variable-length sequences, gfx950.
//
// Each sequence is cut into chunks of Q tokens from its first row, and runs
// of consecutive chunks form segments.  Inside a chunk the output is the
// causally masked product Y = (M o L) X of the Mamba study notes
// (echobase-5bl.pages.dev, "Mamba and Attention"),
//   M[i][j] = (C_i . B_j) exp(a_i - a_j) Delta_j   (j <= i),
// with a the chunk-local cumulative sum of Delta*A, plus exp(a_i) C_i h_in
// for the state h_in entering the chunk; chunk end states follow
// h_out = exp(a_last) h_in + sum_j exp(a_last - a_j) Delta_j x_j B_j^T, the
// affine step that links chunks and segments ("Hybrid SSM / Mamba models and
// non-KV state", mlinterviewnotes.com ch. 7.3: chunked-prefill handoff,
// affine-composition passage, SSD chunk-scan call site).
//
// Launch sequence (one stream):
//   1. conv_kernel       causal conv + SiLU of every (token, channel), written as bf16
//                        operand planes in the layouts the products read
//   2. dt_kernel         Delta = softplus(dt + dt_bias) and the chunk-local cumsum of Delta*A
//   3. seg_state_kernel  per (segment, head): end state of the segment from a zero state (MFMA);
//                        skipped for each sequence's last segment
//   4. seg_pass_kernel   per (sequence, head): scan over segments -> state entering each segment
//   5. seg_scan_kernel   per (segment, head): walks its chunks with the state in MFMA
//                        accumulators: outputs (MFMA), state update (MFMA), checkpoint and
//                        final states rounded into their slots
//   6. window_kernel     final and checkpoint conv windows (raw inputs) into their slots
// With SPLIT every product operand is a bf16 hi plane plus a bf16 lo plane and
// each product takes three MFMAs (fp32-level accuracy, used for fp32 state);
// otherwise operands are single bf16 planes with fp32 accumulation.
#include "device_common.h"
#include "kernels.h"

namespace m2 {

constexpr int kJB = 32;          // tokens per staged block (one MFMA K-step)
#ifndef M2_SCAN_WAVES_PER_EU
#define M2_SCAN_WAVES_PER_EU 1
#endif
#ifndef M2_SCAN_PREFETCH
#define M2_SCAN_PREFETCH 1
#endif
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

// Register prefetch of a staged block: ITEMS 8-element vectors per plane, taken from a
// (rows x cols) tile exactly as stage_rows does, held in registers until written to LDS.
template <int NPL, int ITEMS> struct TilePrefetch {
  u16x8 v[ITEMS][NPL];

  __device__ __forceinline__ void load(const u16* src, int64_t src_plane, int64_t src_ld, int rows, int cols,
                                       int valid_rows, int valid_cols, int tid, int nthreads) {
    const int vpr = cols / 8;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * nthreads;
      const int r = idx / vpr, c = (idx % vpr) * 8;
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) {
        u16x8 x = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (idx < rows * vpr && r < valid_rows) {
          const u16* s = src + pl * src_plane + r * src_ld + c;
          if (c + 8 <= valid_cols) {
            x = *reinterpret_cast<const u16x8*>(s);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (c + e < valid_cols) ? s[e] : u16(0);
          }
        }
        v[it][pl] = x;
      }
    }
  }

  __device__ __forceinline__ void store(u16* dst, int64_t dst_plane, int dst_ld, int rows, int cols, int tid,
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

// ------------------------------------------------------------------ 1. conv
// Workgroup per (chunk, 64 channels), 256 threads.  Thread (octet o, token group tg) convolves
// channels 8o .. 8o+7 over its rows with 16-byte input loads and writes each row's 8 results to
// LDS as one 16-byte store per operand plane.  The tile is then written out: x and B transposed
// (consecutive lanes on consecutive channels, 8 tokens per 16-byte store), and B and C rows.
constexpr int kConvCB = 64;
constexpr int kConvLD = kConvCB + 8;   // u16 pitch of the LDS rows (16-byte aligned)

template <bool SPLIT> struct ConvLds {
  static constexpr int NPL = SPLIT ? 2 : 1;
  static constexpr int BYTES = NPL * 256 * kConvLD * 2;
};

template <int W, bool SPLIT>
__global__ __launch_bounds__(256) void conv_kernel(PrefillParams a) {
  constexpr int CB = kConvCB;
  constexpr int NPL = ConvLds<SPLIT>::NPL;
  constexpr int PLANE = 256 * kConvLD;
  extern __shared__ __align__(16) unsigned char conv_smem[];
  u16* const s_t = reinterpret_cast<u16*>(conv_smem);
  const ChunkEntry ch = a.chunks[blockIdx.x];
  const SeqEntry sq = a.seqs[ch.seq];
  const int Cd = a.sh.Cd, I = a.sh.I, GN = a.sh.G * a.sh.N, P = a.sh.P, N = a.sh.N, H = a.sh.H, G = a.sh.G;
  const int Q = a.Q, len = ch.len;
  const int c0 = blockIdx.y * CB;
  const int tid = threadIdx.x;
  const int oc = tid % (CB / 8), tg = tid / (CB / 8);   // 8 octets x 32 token groups
  const int c = c0 + 8 * oc;
  if (c < Cd) {
    const void* src;
    int64_t col, stride;
    if (c < I) { src = a.x; col = c; stride = a.x_stride; }
    else if (c < I + GN) { src = a.B; col = c - I; stride = a.B_stride; }
    else { src = a.C; col = c - I - GN; stride = a.C_stride; }
    const int per = (len + 31) / 32;
    const int j0 = tg * per, j1 = min(len, j0 + per);
    if (j0 < j1) {
      float win[W - 1][8];
#pragma unroll
      for (int k = 0; k < W - 1; ++k) {
        const int tau = ch.tau0 + j0 - (W - 1) + k;   // offset inside the sequence
        if (tau >= 0) {
          load8_any(src, (int64_t)(sq.t0 + tau) * stride + col, a.io_bf16, win[k]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float v = 0.f;
            if (sq.has_init) {
              const int64_t wi = ((int64_t)sq.slot * Cd + c + e) * (W - 1) + (W - 1 + tau);
              v = a.conv_bf16 ? to_f32(static_cast<const bf16*>(a.conv)[wi]) : static_cast<const float*>(a.conv)[wi];
            }
            win[k][e] = v;
          }
        }
      }
      float w[8][W], bias[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int k = 0; k < W; ++k) w[e][k] = a.conv_w[(int64_t)(c + e) * W + k];
        bias[e] = a.conv_b[c + e];
      }
      for (int j = j0; j < j1; j += 4) {
        float u[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (j + r < j1) load8_any(src, (int64_t)(ch.t0 + j + r) * stride + col, a.io_bf16, u[r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (j + r < j1) {
            u16x8 hv, lv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float v = bias[e];
#pragma unroll
              for (int k = 0; k < W - 1; ++k) v += w[e][k] * win[k][e];
              v += w[e][W - 1] * u[r][e];
              v = silu(v);
              if (SPLIT) {
                u16 hi, lo;
                split2(v, hi, lo);
                hv[e] = hi;
                lv[e] = lo;
              } else {
                hv[e] = bits_of(from_f32<bf16>(v));
              }
            }
            *reinterpret_cast<u16x8*>(s_t + (j + r) * kConvLD + 8 * oc) = hv;
            if (SPLIT) *reinterpret_cast<u16x8*>(s_t + PLANE + (j + r) * kConvLD + 8 * oc) = lv;
#pragma unroll
            for (int k = 0; k < W - 2; ++k)
#pragma unroll
              for (int e = 0; e < 8; ++e) win[k][e] = win[k + 1][e];
#pragma unroll
            for (int e = 0; e < 8; ++e) win[W - 2][e] = u[r][e];
          }
        }
      }
    }
  }
  __syncthreads();
  const int64_t chunk = blockIdx.x;
  // channel-major outputs (x transposed, B transposed): lane per channel, 8 rows per store
  const int ngr = (len + 7) / 8;
  for (int idx = tid; idx < CB * ngr; idx += 256) {
    const int ccl = idx % CB, j = (idx / CB) * 8;
    const int cc = c0 + ccl;
    if (cc >= I + GN) continue;
    u16* dst;
    int64_t pstride;
    if (cc < I) {
      const int h = cc / P, p = cc % P;
      dst = a.xT + ((chunk * H + h) * P + p) * Q + j;
      pstride = a.xT_plane;
    } else {
      const int g = (cc - I) / N, n = (cc - I) % N;
      dst = a.Bt + ((chunk * G + g) * N + n) * Q + j;
      pstride = a.Bt_plane;
    }
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl) {
      u16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = s_t[pl * PLANE + (j + e) * kConvLD + ccl];
      if (j + 8 <= len) {
        *reinterpret_cast<u16x8*>(dst + pl * pstride) = v;
      } else {
        for (int e = 0; e < 8 && j + e < len; ++e) dst[pl * pstride + e] = v[e];
      }
    }
  }
  // token-major outputs (B rows, C rows): thread per (row, 8 channels)
  for (int idx = tid; idx < len * (CB / 8); idx += 256) {
    const int j = idx / (CB / 8), cc = c0 + (idx % (CB / 8)) * 8;
    if (cc < I || cc >= Cd) continue;
    u16* dst;
    int64_t pstride;
    if (cc < I + GN) {
      dst = a.Br + (chunk * Q + j) * GN + (cc - I);
      pstride = a.Br_plane;
    } else {
      dst = a.Cr + (chunk * Q + j) * GN + (cc - I - GN);
      pstride = a.Cr_plane;
    }
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
      *reinterpret_cast<u16x8*>(dst + pl * pstride) =
          *reinterpret_cast<const u16x8*>(s_t + pl * PLANE + j * kConvLD + (cc - c0));
  }
}

// ------------------------------------------------------------------ 2. Delta, cumsum
// One wave per (chunk, head); lane l owns rows 4l .. 4l+3 of the chunk (Q <= 256).
__global__ __launch_bounds__(256) void dt_kernel(PrefillParams a) {
  const ChunkEntry ch = a.chunks[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
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

// State tiles (P/16 x N/16 of 16x16) spread over the 8 waves of a workgroup.
template <int P, int N> struct StateTiles {
  static constexpr int NT = N / 16;
  static constexpr int TOTAL = (P / 16) * NT;
  static constexpr int PER_WAVE = (TOTAL + 7) / 8;
};

// ------------------------------------------------------------------ 3. segment end states
template <bool SPLIT, int P, int N>
__global__ __launch_bounds__(kStateThreads) void seg_state_kernel(PrefillParams a) {
  constexpr int NPL = SPLIT ? 2 : 1;
  constexpr int LDX = kJB + 4;   // 18 dwords: conflict-free fragment rows
  typedef StateTiles<P, N> ST;
  __shared__ u16 sXT[NPL * P * LDX];
  __shared__ u16 sBT[NPL * N * LDX];
  __shared__ float sW[256];
  const SegEntry sg = a.segs[blockIdx.x];
  if (sg.is_last) return;
  const int h = blockIdx.y, H = a.sh.H, G = a.sh.G, Q = a.Q;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t T = a.total_tokens;
  floatx4 acc[ST::PER_WAVE];
#pragma unroll
  for (int k = 0; k < ST::PER_WAVE; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
  float logdecay = 0.f;
  for (int c = sg.chunk0; c < sg.chunk0 + sg.nchunk; ++c) {
    const ChunkEntry ch = a.chunks[c];
    const int len = ch.len;
    const float* dAh = a.dA + (int64_t)h * T + ch.t0;
    const float* dh = a.delta + (int64_t)h * T + ch.t0;
    const float alast = dAh[len - 1];
    logdecay += alast;
    __syncthreads();
    for (int j = tid; j < 256; j += kStateThreads) sW[j] = j < len ? __expf(alast - dAh[j]) * dh[j] : 0.f;
    const float decay = __expf(alast);
#pragma unroll
    for (int k = 0; k < ST::PER_WAVE; ++k) acc[k] *= decay;
    for (int jb = 0; jb < len; jb += kJB) {
      __syncthreads();
      stage_rows<NPL>(sXT, P * LDX, LDX, a.xT + (((int64_t)c * H + h) * P) * Q + jb, a.xT_plane, Q, P, kJB,
                      P, len - jb, tid, kStateThreads);
      stage_rows<NPL>(sBT, N * LDX, LDX, a.Bt + (((int64_t)c * G + g) * N) * Q + jb, a.Bt_plane, Q, N, kJB,
                      N, len - jb, tid, kStateThreads);
      __syncthreads();
      int cur_pt = -1;
      Frag<SPLIT> fa;
#pragma unroll
      for (int m = 0; m < ST::PER_WAVE; ++m) {
        const int k = wave * ST::PER_WAVE + m;
        if (k < ST::TOTAL) {
          const int pt = k / ST::NT, nt = k % ST::NT;
          if (pt != cur_pt) {
            float v[8];
            lds_vals<SPLIT>(sXT, P * LDX, LDX, pt * 16 + l16, 0, q, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= sW[jb + kmap(q, e)];
            fa = make_frag<SPLIT>(v);
            cur_pt = pt;
          }
          const Frag<SPLIT> fb = lds_frag<SPLIT>(sBT, N * LDX, LDX, nt * 16 + l16, 0, q);
          acc[m] = mma<SPLIT>(fa, fb, acc[m]);
        }
      }
    }
  }
  float* out = a.seg_state + ((int64_t)blockIdx.x * H + h) * P * N;
#pragma unroll
  for (int m = 0; m < ST::PER_WAVE; ++m) {
    const int k = wave * ST::PER_WAVE + m;
    if (k < ST::TOTAL) {
      const int pt = k / ST::NT, nt = k % ST::NT;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(pt * 16 + 4 * q + r) * N + nt * 16 + l16] = acc[m][r];
    }
  }
  if (tid == 0) a.seg_decay[(int64_t)blockIdx.x * H + h] = logdecay;
}

// ------------------------------------------------------------------ 4. scan over segments
template <typename TS>
__global__ __launch_bounds__(256) void seg_pass_kernel(PrefillParams a) {
  const SeqEntry sq = a.seqs[blockIdx.x];
  if (sq.nseg == 0) return;
  const int h = blockIdx.y, H = a.sh.H;
  const int PN = a.sh.P * a.sh.N;
  const int e4 = (blockIdx.z * 256 + threadIdx.x) * 4;
  if (e4 >= PN) return;
  const int64_t head_off = (int64_t)h * PN + e4;
  floatx4 hs = floatx4{0.f, 0.f, 0.f, 0.f};
  if (sq.has_init) {
    const TS* src = static_cast<const TS*>(a.ssm) + (int64_t)sq.slot * H * PN + head_off;
#pragma unroll
    for (int e = 0; e < 4; ++e) hs[e] = to_f32(src[e]);
  }
  constexpr int D = 8;
  for (int s0 = 0; s0 < sq.nseg; s0 += D) {
    floatx4 sc[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const int s = sq.seg0 + s0 + k;
      if (s0 + k < sq.nseg && !a.segs[s].is_last)
        sc[k] = *reinterpret_cast<const floatx4*>(a.seg_state + (int64_t)s * H * PN + head_off);
    }
#pragma unroll
    for (int k = 0; k < D; ++k) {
      if (s0 + k < sq.nseg) {
        const int s = sq.seg0 + s0 + k;
        *reinterpret_cast<floatx4*>(a.seg_state + (int64_t)s * H * PN + head_off) = hs;
        if (!a.segs[s].is_last) hs = __expf(a.seg_decay[(int64_t)s * H + h]) * hs + sc[k];
      }
    }
  }
}

// ------------------------------------------------------------------ 5. segment walk
// Tokens per staged block in the segment walk: two K-steps with single bf16 planes, one with
// hi/lo planes (the register prefetch of a block doubles with two planes).
template <bool SPLIT> struct ScanBlock { static constexpr int JB = SPLIT ? 32 : 64; };

template <bool SPLIT, int P, int N> struct ScanLds {
  static constexpr int kSJB = ScanBlock<SPLIT>::JB;
  static constexpr int NPL = SPLIT ? 2 : 1;
  // row pitches of 2 (mod 32) dwords: the 16 rows of a fragment read land in distinct banks
  static constexpr int LDH = N + 4;      // state operand rows [p][n]
  static constexpr int LDB = N + 4;      // B rows [j][n]
  static constexpr int LDX = kSJB + 4;   // transposed blocks [p or n][j]
  static constexpr int H_OFF = 0;
  static constexpr int BR_OFF = H_OFF + NPL * P * LDH;
  static constexpr int XT_OFF = BR_OFF + NPL * kSJB * LDB;
  static constexpr int BT_OFF = XT_OFF + NPL * P * LDX;
  static constexpr int U16_END = BT_OFF + NPL * N * LDX;
  static constexpr int F_OFF = (U16_END * 2 + 15) / 16 * 16;   // bytes
  static constexpr int BYTES = F_OFF + 4 * 256 * 4;
  // staging vectors per thread
  static constexpr int IT_BR = (kSJB * (N / 8) + kScanThreads - 1) / kScanThreads;
  static constexpr int IT_XT = (P * (kSJB / 8) + kScanThreads - 1) / kScanThreads;
  static constexpr int IT_BT = (N * (kSJB / 8) + kScanThreads - 1) / kScanThreads;
};

template <typename TS>
__device__ __forceinline__ void store_state_tile(void* pool, int64_t base, int N, int p, int n, const floatx4& v) {
  TS* d = static_cast<TS*>(pool) + base;
#pragma unroll
  for (int r = 0; r < 4; ++r) d[(int64_t)(p + r) * N + n] = from_f32<TS>(v[r]);
}

template <bool SPLIT, int P, int N> struct ScanPrefetch {
  typedef ScanLds<SPLIT, P, N> L;
  static constexpr int kSJB = L::kSJB;
  TilePrefetch<L::NPL, L::IT_BR> br;
  TilePrefetch<L::NPL, L::IT_XT> xt;
  TilePrefetch<L::NPL, L::IT_BT> bt;

  __device__ __forceinline__ void load(const PrefillParams& a, int c, int jb, int len, int h, int g, int tid) {
    const int Q = a.Q, H = a.sh.H, G = a.sh.G, GN = G * N;
    br.load(a.Br + ((int64_t)c * Q + jb) * GN + g * N, a.Br_plane, GN, kSJB, N, len - jb, N, tid, kScanThreads);
    xt.load(a.xT + (((int64_t)c * H + h) * P) * Q + jb, a.xT_plane, Q, P, kSJB, P, len - jb, tid, kScanThreads);
    bt.load(a.Bt + (((int64_t)c * G + g) * N) * Q + jb, a.Bt_plane, Q, N, kSJB, N, len - jb, tid, kScanThreads);
  }
  __device__ __forceinline__ void store(u16* sBr, u16* sXT, u16* sBT, int tid) const {
    br.store(sBr, kSJB * L::LDB, L::LDB, kSJB, N, tid, kScanThreads);
    xt.store(sXT, P * L::LDX, L::LDX, P, kSJB, tid, kScanThreads);
    bt.store(sBT, N * L::LDX, L::LDX, N, kSJB, tid, kScanThreads);
  }
};

template <bool SPLIT, int P, int N>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(M2_SCAN_WAVES_PER_EU)))
void seg_scan_kernel(PrefillParams a) {
  typedef ScanLds<SPLIT, P, N> L;
  typedef StateTiles<P, N> ST;
  constexpr int kSJB = L::kSJB;
  constexpr int NPL = L::NPL;
  constexpr int PT = P / 16;
  constexpr int NK = N / 32 > 0 ? N / 32 : 1;   // K-steps over the state dimension
  extern __shared__ __align__(16) unsigned char smem_raw[];
  u16* const smem = reinterpret_cast<u16*>(smem_raw);
  u16* const sH = smem + L::H_OFF;
  u16* const sBr = smem + L::BR_OFF;
  u16* const sXT = smem + L::XT_OFF;
  u16* const sBT = smem + L::BT_OFF;
  float* const sA = reinterpret_cast<float*>(smem_raw + L::F_OFF);
  float* const sD = sA + 256;
  float* const sW = sD + 256;
  float* const sCw = sW + 256;   // exp(a_ref - a_j) Delta_j, a_ref = cumsum at the last token of j's K-step

  const SegEntry sg = a.segs[blockIdx.x];
  const SeqEntry sq = a.seqs[sg.seq];
  const int h = blockIdx.y, H = a.sh.H, G = a.sh.G, Q = a.Q;
  const int GN = G * N;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t T = a.total_tokens;
  const float Dh = a.D[h];
  const int64_t slot_elems = (int64_t)H * P * N;

  // running state in accumulator layout: tile (pt, nt), lane holds h[pt*16 + 4q + r][nt*16 + l16]
  floatx4 hacc[ST::PER_WAVE];
  {
    const float* hin = a.seg_state + ((int64_t)blockIdx.x * H + h) * P * N;
#pragma unroll
    for (int m = 0; m < ST::PER_WAVE; ++m) {
      const int k = wave * ST::PER_WAVE + m;
      hacc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (k < ST::TOTAL) {
        const int pt = k / ST::NT, nt = k % ST::NT;
#pragma unroll
        for (int r = 0; r < 4; ++r) hacc[m][r] = hin[(pt * 16 + 4 * q + r) * N + nt * 16 + l16];
      }
    }
  }
  // row tiles of this wave: wave and 15 - wave (balanced causal work for Q = 256)
  const int nrt = Q / 16;
  const int rts[2] = {wave, 15 - wave};
  const int c_end = sg.chunk0 + sg.nchunk;

  ScanPrefetch<SPLIT, P, N> pf;
#if M2_SCAN_PREFETCH
  pf.load(a, sg.chunk0, 0, a.chunks[sg.chunk0].len, h, g, tid);
#endif

  for (int c = sg.chunk0; c < c_end; ++c) {
    const ChunkEntry ch = a.chunks[c];
    const int len = ch.len;
    const float* dAh = a.dA + (int64_t)h * T + ch.t0;
    const float* dh = a.delta + (int64_t)h * T + ch.t0;
    const float alast = dAh[len - 1];
    __syncthreads();   // previous chunk's LDS reads are done
    for (int j = tid; j < 256; j += kScanThreads) {
      const bool ok = j < len;
      const float aj = ok ? dAh[j] : 0.f, dj = ok ? dh[j] : 0.f;
      const int jr = min((j | 31), len - 1);   // last token of j's K-step
      sA[j] = aj;
      sD[j] = dj;
      sW[j] = ok ? __expf(alast - aj) * dj : 0.f;
      sCw[j] = ok ? __expf(dAh[jr] - aj) * dj : 0.f;
    }
    // state entering the chunk -> operand planes [p][n]
#pragma unroll
    for (int m = 0; m < ST::PER_WAVE; ++m) {
      const int k = wave * ST::PER_WAVE + m;
      if (k < ST::TOTAL) {
        const int pt = k / ST::NT, nt = k % ST::NT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int idx = (pt * 16 + 4 * q + r) * L::LDH + nt * 16 + l16;
          u16 hi, lo = 0;
          if (SPLIT) split2(hacc[m][r], hi, lo);
          else hi = bits_of(from_f32<bf16>(hacc[m][r]));
          sH[idx] = hi;
          if (SPLIT) sH[P * L::LDH + idx] = lo;
        }
      }
    }
    // C rows of this wave's row tiles as fragments (global loads issued before the barrier)
    Frag<SPLIT> cf[2][NK];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rt = rts[t];
      const int i = rt * 16 + l16;
      if (!(rt < nrt && rt * 16 < len)) continue;
      const u16* crow = a.Cr + ((int64_t)c * Q + i) * GN + g * N;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          u16x4 lo4 = u16x4{0, 0, 0, 0}, hi4 = u16x4{0, 0, 0, 0};
          const int n = ks * 32 + 4 * q;
          if (i < len) {
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
    __syncthreads();

    // the entering-state term
    floatx4 acc[2][PT];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rt = rts[t];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[t][pt] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (!(rt < nrt && rt * 16 < len)) continue;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          Frag<SPLIT> fh = lds_frag<SPLIT>(sH, P * L::LDH, L::LDH, pt * 16 + l16, N >= 32 ? ks * 32 : 0, q);
          if (N < 32) {   // upper K half is padding
#pragma unroll
            for (int e = 4; e < 8; ++e) { fh.hi[e] = bf_of(0); if (SPLIT) fh.lo[e] = bf_of(0); }
          }
          acc[t][pt] = mma<SPLIT>(cf[t][ks], fh, acc[t][pt]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = rt * 16 + 4 * q + r;
        const float sc = ii < len ? __expf(sA[ii]) : 0.f;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[t][pt][r] *= sc;
      }
    }

    // the chunk's state update starts from the decayed entering state
    const float decay = __expf(alast);
#pragma unroll
    for (int m = 0; m < ST::PER_WAVE; ++m) hacc[m] *= decay;

    for (int jb = 0; jb < len; jb += kSJB) {
      __syncthreads();   // all reads of the previous block are done
#if M2_SCAN_PREFETCH
      pf.store(sBr, sXT, sBT, tid);
      __syncthreads();
      // prefetch the next block (next chunk's first block at the end of this chunk)
      if (jb + kSJB < len) pf.load(a, c, jb + kSJB, len, h, g, tid);
      else if (c + 1 < c_end) pf.load(a, c + 1, 0, a.chunks[c + 1].len, h, g, tid);
#else
      pf.load(a, c, jb, len, h, g, tid);
      pf.store(sBr, sXT, sBT, tid);
      __syncthreads();
#endif

#pragma unroll
      for (int kb = 0; kb < kSJB; kb += 32) {
        const int jk = jb + kb;   // first token of this K-step
        if (jk >= len) break;
        // diagonal blocks: G^T tiles -> M -> (M o L) X  (D x rides on the diagonal of M).
        // Each B-row and x fragment is read from LDS once and used for both row tiles.
        bool act[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) act[t] = rts[t] < nrt && rts[t] * 16 < len && jk <= rts[t] * 16 + 15;
        if (act[0] || act[1]) {
          floatx4 gt[2][2];
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) gt[t][jt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const bool need0 = act[0] && jk + 16 * jt <= rts[0] * 16 + 15;
            const bool need1 = act[1] && jk + 16 * jt <= rts[1] * 16 + 15;
            if (!(need0 || need1)) continue;
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) {
              Frag<SPLIT> fb = lds_frag<SPLIT>(sBr, kSJB * L::LDB, L::LDB, kb + jt * 16 + l16,
                                               N >= 32 ? ks * 32 : 0, q);
              if (N < 32) {
#pragma unroll
                for (int e = 4; e < 8; ++e) { fb.hi[e] = bf_of(0); if (SPLIT) fb.lo[e] = bf_of(0); }
              }
              if (need0) gt[0][jt] = mma<SPLIT>(fb, cf[0][ks], gt[0][jt]);
              if (need1) gt[1][jt] = mma<SPLIT>(fb, cf[1][ks], gt[1][jt]);
            }
          }
          // decay mask.  Below the diagonal (every token of the K-step precedes every row),
          // exp(a_i - a_j) = exp(a_i - a_ref) exp(a_ref - a_j) with a_ref the cumsum at the
          // K-step's last token: both factors are <= 1, one exp per row and a column table.
          // On the diagonal the exponent is taken directly.
          Frag<SPLIT> fm[2];
          float cw[8];
          {
            const floatx4 c0 = *reinterpret_cast<const floatx4*>(&sCw[jk + 4 * q]);
            const floatx4 c1 = *reinterpret_cast<const floatx4*>(&sCw[jk + 16 + 4 * q]);
#pragma unroll
            for (int e = 0; e < 4; ++e) { cw[e] = c0[e]; cw[e + 4] = c1[e]; }
          }
          const float aref = sA[min(jk + 31, len - 1)];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int i = rts[t] * 16 + l16;
            const bool row_ok = act[t] && i < len;
            const float ai = row_ok ? sA[i] : 0.f;
            float mv[8];
            if (jk + 31 < rts[t] * 16) {
              const float rf = row_ok ? __expf(ai - aref) : 0.f;
#pragma unroll
              for (int e = 0; e < 8; ++e) mv[e] = gt[t][e >> 2][e & 3] * rf * cw[e];
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int j = jk + kmap(q, e);
                float v = 0.f;
                if (row_ok && j <= i) {
                  v = gt[t][e >> 2][e & 3] * __expf(ai - sA[j]) * sD[j];
                  if (j == i) v += Dh;
                }
                mv[e] = v;
              }
            }
            fm[t] = make_frag<SPLIT>(mv);
          }
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
            const Frag<SPLIT> fx = lds_frag<SPLIT>(sXT, P * L::LDX, L::LDX, pt * 16 + l16, kb, q);
            if (act[0]) acc[0][pt] = mma<SPLIT>(fm[0], fx, acc[0][pt]);
            if (act[1]) acc[1][pt] = mma<SPLIT>(fm[1], fx, acc[1][pt]);
          }
        }
        // state update: h += (w x)^T B over this K-step's tokens
        int cur_pt = -1;
        Frag<SPLIT> fa;
#pragma unroll
        for (int m = 0; m < ST::PER_WAVE; ++m) {
          const int k = wave * ST::PER_WAVE + m;
          if (k < ST::TOTAL) {
            const int pt = k / ST::NT, nt = k % ST::NT;
            if (pt != cur_pt) {
              float v[8];
              lds_vals<SPLIT>(sXT, P * L::LDX, L::LDX, pt * 16 + l16, kb, q, v);
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] *= sW[jk + kmap(q, e)];
              fa = make_frag<SPLIT>(v);
              cur_pt = pt;
            }
            const Frag<SPLIT> fb = lds_frag<SPLIT>(sBT, N * L::LDX, L::LDX, nt * 16 + l16, kb, q);
            hacc[m] = mma<SPLIT>(fa, fb, hacc[m]);
          }
        }
      }
    }

    // outputs: y = acc gated by SiLU(z); lane holds rows rt*16 + 4q + r, columns pt*16 + l16
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rt = rts[t];
      if (rt >= nrt || rt * 16 >= len) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = rt * 16 + 4 * q + r;
        if (ii < len) {
          const int64_t row = ch.t0 + ii;
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) {
            const int col = h * P + pt * 16 + l16;
            const float zv = load_any(a.z, row * a.z_stride + col, a.io_bf16);
            store_any(a.y, row * a.y_stride + col, acc[t][pt][r] * silu(zv), a.y_bf16);
          }
        }
      }
    }

    // checkpoint and final states, rounded to the state dtype
    const int dsts[2] = {ch.ckpt_slot, ch.is_last ? sq.slot : -1};
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (dsts[d] < 0) continue;
      const int64_t base = (int64_t)dsts[d] * slot_elems + (int64_t)h * P * N;
#pragma unroll
      for (int m = 0; m < ST::PER_WAVE; ++m) {
        const int k = wave * ST::PER_WAVE + m;
        if (k < ST::TOTAL) {
          const int pt = k / ST::NT, nt = k % ST::NT;
          if (a.ssm_bf16) store_state_tile<bf16>(a.ssm, base, N, pt * 16 + 4 * q, nt * 16 + l16, hacc[m]);
          else store_state_tile<float>(a.ssm, base, N, pt * 16 + 4 * q, nt * 16 + l16, hacc[m]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ 6. conv windows
template <int W>
__global__ __launch_bounds__(256) void window_kernel(PrefillParams a) {
  const WindowEntry we = a.windows[blockIdx.x];
  const SeqEntry sq = a.seqs[we.seq];
  const int Cd = a.sh.Cd, I = a.sh.I, GN = a.sh.G * a.sh.N;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= Cd) return;
  const void* src;
  int64_t col, stride;
  if (c < I) { src = a.x; col = c; stride = a.x_stride; }
  else if (c < I + GN) { src = a.B; col = c - I; stride = a.B_stride; }
  else { src = a.C; col = c - I - GN; stride = a.C_stride; }
  float v[W - 1];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int pos = we.tau - (W - 1) + k;
    if (pos >= 0) {
      v[k] = load_any(src, (int64_t)(sq.t0 + pos) * stride + col, a.io_bf16);
    } else if (sq.has_init) {
      const int64_t wi = ((int64_t)sq.slot * Cd + c) * (W - 1) + (W - 1 + pos);
      v[k] = a.conv_bf16 ? to_f32(static_cast<const bf16*>(a.conv)[wi]) : static_cast<const float*>(a.conv)[wi];
    } else {
      v[k] = 0.f;
    }
  }
  const int64_t wo = ((int64_t)we.slot * Cd + c) * (W - 1);
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    if (a.conv_bf16) static_cast<bf16*>(a.conv)[wo + k] = from_f32<bf16>(v[k]);
    else static_cast<float*>(a.conv)[wo + k] = v[k];
  }
}

// ------------------------------------------------------------------ launch
// Allow `bytes` of dynamic LDS for a kernel (idempotent; called before each launch).
static hipError_t set_lds_attr(const void* fn, int bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <bool SPLIT, int P, int N>
static hipError_t launch_segments(const PrefillParams& a, hipStream_t s) {
  hipLaunchKernelGGL((seg_state_kernel<SPLIT, P, N>), dim3(a.num_segments, a.sh.H), dim3(kStateThreads), 0, s, a);
  const int PN = P * N;
  const dim3 gp(a.num_seqs, a.sh.H, (PN / 4 + 255) / 256);
  if (a.ssm_bf16) hipLaunchKernelGGL(seg_pass_kernel<bf16>, gp, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(seg_pass_kernel<float>, gp, dim3(256), 0, s, a);
  typedef ScanLds<SPLIT, P, N> L;
  const hipError_t e = set_lds_attr(reinterpret_cast<const void*>(&seg_scan_kernel<SPLIT, P, N>), L::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((seg_scan_kernel<SPLIT, P, N>), dim3(a.num_segments, a.sh.H), dim3(kScanThreads), L::BYTES, s,
                     a);
  return hipSuccess;
}

template <int P, int N>
static hipError_t launch_pn(const PrefillParams& a, hipStream_t s) {
  return a.ssm_bf16 ? launch_segments<false, P, N>(a, s) : launch_segments<true, P, N>(a, s);
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

hipError_t launch_prefill(const PrefillParams& a, hipStream_t s) {
  if (a.num_chunks == 0) return hipSuccess;
  const dim3 gc(a.num_chunks, (a.sh.Cd + kConvCB - 1) / kConvCB);
  const bool split = !a.ssm_bf16;
  hipError_t ea = hipSuccess;
#define M2_CONV(WW)                                                                                        \
  if (split) {                                                                                             \
    ea = set_lds_attr(reinterpret_cast<const void*>(&conv_kernel<WW, true>), ConvLds<true>::BYTES);        \
    hipLaunchKernelGGL((conv_kernel<WW, true>), gc, dim3(256), ConvLds<true>::BYTES, s, a);                \
  } else {                                                                                                 \
    ea = set_lds_attr(reinterpret_cast<const void*>(&conv_kernel<WW, false>), ConvLds<false>::BYTES);     \
    hipLaunchKernelGGL((conv_kernel<WW, false>), gc, dim3(256), ConvLds<false>::BYTES, s, a);             \
  }
  switch (a.sh.W) {
    case 2: M2_CONV(2) break;
    case 3: M2_CONV(3) break;
    case 4: M2_CONV(4) break;
    default: return hipErrorInvalidValue;
  }
#undef M2_CONV
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(dt_kernel, dim3(a.num_chunks, (a.sh.H + 3) / 4), dim3(256), 0, s, a);
  hipError_t e = hipErrorInvalidValue;
  switch (a.sh.P) {
    case 16: e = launch_p<16>(a, s); break;
    case 32: e = launch_p<32>(a, s); break;
    case 64: e = launch_p<64>(a, s); break;
    case 128: e = launch_p<128>(a, s); break;
  }
  if (e != hipSuccess) return e;
  if (a.num_windows > 0) {
    const dim3 gw(a.num_windows, (a.sh.Cd + 255) / 256);
    switch (a.sh.W) {
      case 2: hipLaunchKernelGGL(window_kernel<2>, gw, dim3(256), 0, s, a); break;
      case 3: hipLaunchKernelGGL(window_kernel<3>, gw, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL(window_kernel<4>, gw, dim3(256), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace m2
