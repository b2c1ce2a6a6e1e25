// Chunked (SSD) prefill of packed variable-length sequences, gfx950.
//
// The sequence is cut into chunks of Q tokens starting at each sequence's
// first row.  Inside a chunk the output is the causally masked product
// Y = (M o L) X of the Mamba study notes (echobase-5bl.pages.dev, "Mamba and
// Attention"), M[i][j] = (C_i . B_j) exp(a_i - a_j) Delta_j, with a the
// chunk-local cumulative sum of Delta*A; chunks are linked by a scan over
// their end states, each chunk handing its state to the next
// ("Hybrid SSM / Mamba models and non-KV state", mlinterviewnotes.com
// ch. 7.3: the chunked-prefill handoff and the SSD chunk-scan call site).
//
// Launch sequence (one stream):
//   1. conv_kernel         causal depthwise conv + SiLU of every (token, channel)
//   2. dt_kernel           Delta = softplus(dt + dt_bias) and the chunk-local cumsum of Delta*A
//   3. chunk_state_kernel  S_c = sum_j exp(a_last - a_j) Delta_j x_j B_j^T  (MFMA)
//   4. state_pass_kernel   h_c = exp(a_last) h_{c-1} + S_c along each sequence; the state
//                          entering each chunk replaces S_c; final and checkpoint states
//                          go to their pool slots rounded to the state dtype
//   5. chunk_scan_kernel   y = C h_{c-1} exp(a_i) + (M o L) X + D x, gated by SiLU(z)  (MFMA)
//   6. window_kernel       final and checkpoint conv windows (raw inputs) into their slots
// With SPLIT the MFMA operands are split into bf16 hi + lo parts and each
// product takes three bf16 MFMAs, which keeps fp32-level accuracy for fp32
// state; otherwise operands are rounded to bf16 (fp32 accumulate).
#include "device_common.h"
#include "kernels.h"

namespace m2 {

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ const void* io_col(const PrefillParams& a, int c, int64_t& col, int64_t& stride) {
  const int I = a.sh.I, GN = a.sh.G * a.sh.N;
  if (c < I) { col = c; stride = a.x_stride; return a.x; }
  if (c < I + GN) { col = c - I; stride = a.B_stride; return a.B; }
  col = c - I - GN;
  stride = a.C_stride;
  return a.C;
}

// ------------------------------------------------------------------ 1. conv
template <int W>
__global__ __launch_bounds__(256) void conv_kernel(PrefillParams a) {
  const ChunkEntry ch = a.chunks[blockIdx.x];
  const SeqEntry sq = a.seqs[ch.seq];
  const int Cd = a.sh.Cd;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= Cd) return;
  int64_t col, stride;
  const void* src = io_col(a, c, col, stride);
  float win[W - 1];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int tau = ch.tau0 - (W - 1) + k;
    if (tau >= 0) {
      win[k] = load_any(src, (int64_t)(sq.t0 + tau) * stride + col, a.io_bf16);
    } else if (sq.has_init) {
      const int64_t wi = ((int64_t)sq.slot * Cd + c) * (W - 1) + (W - 1 + tau);
      win[k] = a.conv_bf16 ? to_f32(static_cast<const bf16*>(a.conv)[wi]) : static_cast<const float*>(a.conv)[wi];
    } else {
      win[k] = 0.f;
    }
  }
  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = a.conv_w[(int64_t)c * W + k];
  const float bias = a.conv_b[c];
  float* out = a.act + (int64_t)ch.t0 * Cd + c;
#pragma unroll 8
  for (int i = 0; i < ch.len; ++i) {
    const float u = load_any(src, (int64_t)(ch.t0 + i) * stride + col, a.io_bf16);
    float v = bias;
#pragma unroll
    for (int k = 0; k < W - 1; ++k) v += w[k] * win[k];
    v += w[W - 1] * u;
    out[(int64_t)i * Cd] = silu(v);
#pragma unroll
    for (int k = 0; k < W - 2; ++k) win[k] = win[k + 1];
    win[W - 2] = u;
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

// ------------------------------------------------------------------ 3. chunk states
// Workgroup per (chunk, head).  S[p][n] = sum_j (w_j x_j[p]) B_j[n] with
// w_j = exp(a_last - a_j) Delta_j.  32-token blocks of x (transposed, weighted)
// and B (transposed) are staged in LDS; wave w owns p-tiles w, w+4, ...
template <bool SPLIT, int P, int N>
__global__ __launch_bounds__(256) void chunk_state_kernel(PrefillParams a) {
  constexpr int PT = P / 16, NT = N / 16;
  constexpr int PTW = (PT + 3) / 4;   // p-tiles per wave
  constexpr int LDJ = 36;             // row pitch (floats) of the transposed tiles
  __shared__ float sX[P * LDJ];
  __shared__ float sB[N * LDJ];
  __shared__ float sW[256];

  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkEntry ch = a.chunks[c];
  const int I = a.sh.I, Cd = a.sh.Cd, G = a.sh.G;
  const int g = h / (a.sh.H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t T = a.total_tokens;
  const float* dAh = a.dA + (int64_t)h * T + ch.t0;
  const float* dh = a.delta + (int64_t)h * T + ch.t0;
  const float alast = dAh[ch.len - 1];
  for (int j = tid; j < 256; j += 256) sW[j] = j < ch.len ? __expf(alast - dAh[j]) * dh[j] : 0.f;

  floatx4 acc[PTW][NT];
#pragma unroll
  for (int t = 0; t < PTW; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[t][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int jb = 0; jb < ch.len; jb += 32) {
    __syncthreads();
    // stage x^T (weighted) and B^T for rows jb .. jb+31
    for (int idx = tid; idx < 32 * (P / 4); idx += 256) {
      const int jj = idx / (P / 4), p4 = (idx % (P / 4)) * 4;
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      if (jb + jj < ch.len) {
        v = *reinterpret_cast<const floatx4*>(a.act + (int64_t)(ch.t0 + jb + jj) * Cd + h * P + p4);
        v *= sW[jb + jj];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[(p4 + e) * LDJ + jj] = v[e];
    }
    for (int idx = tid; idx < 32 * (N / 4); idx += 256) {
      const int jj = idx / (N / 4), n4 = (idx % (N / 4)) * 4;
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      if (jb + jj < ch.len)
        v = *reinterpret_cast<const floatx4*>(a.act + (int64_t)(ch.t0 + jb + jj) * Cd + I + g * N + n4);
#pragma unroll
      for (int e = 0; e < 4; ++e) sB[(n4 + e) * LDJ + jj] = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < PTW; ++t) {
      const int pt = wave + 4 * t;
      if (pt < PT) {
        float av[8];
        const floatx4 a0 = *reinterpret_cast<const floatx4*>(&sX[(pt * 16 + l16) * LDJ + 4 * q]);
        const floatx4 a1 = *reinterpret_cast<const floatx4*>(&sX[(pt * 16 + l16) * LDJ + 16 + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) { av[e] = a0[e]; av[e + 4] = a1[e]; }
        const Frag<SPLIT> fa = make_frag<SPLIT>(av);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float bv[8];
          const floatx4 b0 = *reinterpret_cast<const floatx4*>(&sB[(nt * 16 + l16) * LDJ + 4 * q]);
          const floatx4 b1 = *reinterpret_cast<const floatx4*>(&sB[(nt * 16 + l16) * LDJ + 16 + 4 * q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) { bv[e] = b0[e]; bv[e + 4] = b1[e]; }
          acc[t][nt] = mma<SPLIT>(fa, make_frag<SPLIT>(bv), acc[t][nt]);
        }
      }
    }
  }
  // acc[t][nt] lane holds S[p = pt*16 + 4q + r][n = nt*16 + l16]
  float* out = a.states + ((int64_t)c * a.sh.H + h) * P * N;
#pragma unroll
  for (int t = 0; t < PTW; ++t) {
    const int pt = wave + 4 * t;
    if (pt < PT) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[(pt * 16 + 4 * q + r) * N + nt * 16 + l16] = acc[t][nt][r];
    }
  }
}

// ------------------------------------------------------------------ 4. state passing
// Thread per 4 state elements of one head of one sequence, walking its chunks
// in order, eight chunk states in flight.
template <typename TS>
__device__ __forceinline__ void store_state4(void* pool, int64_t i, const floatx4& v) {
  TS* p = static_cast<TS*>(pool) + i;
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = from_f32<TS>(v[e]);
}

template <typename TS>
__global__ __launch_bounds__(256) void state_pass_kernel(PrefillParams a) {
  const SeqEntry sq = a.seqs[blockIdx.x];
  if (sq.nchunk == 0) return;
  const int h = blockIdx.y;
  const int PN = a.sh.P * a.sh.N;
  const int e4 = (blockIdx.z * 256 + threadIdx.x) * 4;
  if (e4 >= PN) return;
  const int64_t T = a.total_tokens;
  const int64_t head_off = (int64_t)h * PN + e4;
  const int64_t slot_stride = (int64_t)a.sh.H * PN;
  floatx4 hs = floatx4{0.f, 0.f, 0.f, 0.f};
  if (sq.has_init) {
    const TS* src = static_cast<const TS*>(a.ssm) + sq.slot * slot_stride + head_off;
#pragma unroll
    for (int e = 0; e < 4; ++e) hs[e] = to_f32(src[e]);
  }
  constexpr int D = 8;
  for (int c0 = 0; c0 < sq.nchunk; c0 += D) {
    floatx4 sc[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
      if (c0 + k < sq.nchunk)
        sc[k] = *reinterpret_cast<const floatx4*>(a.states + (int64_t)(sq.chunk0 + c0 + k) * a.sh.H * PN + head_off);
    }
#pragma unroll
    for (int k = 0; k < D; ++k) {
      if (c0 + k < sq.nchunk) {
        const int c = sq.chunk0 + c0 + k;
        const ChunkEntry ch = a.chunks[c];
        *reinterpret_cast<floatx4*>(a.states + (int64_t)c * a.sh.H * PN + head_off) = hs;
        const float decay = __expf(a.dA[(int64_t)h * T + ch.t0 + ch.len - 1]);
        hs = decay * hs + sc[k];
        if (ch.ckpt_slot >= 0) store_state4<TS>(a.ssm, ch.ckpt_slot * slot_stride + head_off, hs);
      }
    }
  }
  store_state4<TS>(a.ssm, sq.slot * slot_stride + head_off, hs);
}

// ------------------------------------------------------------------ 5. chunk outputs
// Workgroup per (chunk, head, 64-row block); wave w owns rows i0 + 16w .. +15.
template <bool SPLIT, int P, int N>
__global__ __launch_bounds__(256) void chunk_scan_kernel(PrefillParams a) {
  constexpr int PT = P / 16;
  constexpr int NK = (N + 31) / 32;    // K-steps over the state dimension
  constexpr int LDB = N + 4;           // row pitch of the staged B block
  constexpr int LDJ = 36;              // row pitch of the staged x^T block
  __shared__ float sB[32 * LDB];
  __shared__ float sX[P * LDJ];
  __shared__ float sdA[256];
  __shared__ float sD[256];

  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkEntry ch = a.chunks[c];
  const int rb0 = blockIdx.z * 64;
  if (rb0 >= ch.len) return;
  const int I = a.sh.I, Cd = a.sh.Cd, G = a.sh.G;
  const int g = h / (a.sh.H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int i0 = rb0 + wave * 16;
  const int64_t T = a.total_tokens;
  const int jend = min(rb0 + 64, ch.len);
  for (int j = tid; j < 256; j += 256) {
    sdA[j] = j < ch.len ? a.dA[(int64_t)h * T + ch.t0 + j] : 0.f;
    sD[j] = j < ch.len ? a.delta[(int64_t)h * T + ch.t0 + j] : 0.f;
  }

  // C rows of this wave as fragments (lane: row i0 + l16, K positions kmap)
  const int irow = i0 + l16;
  const bool row_ok = irow < ch.len;
  const float* crow = a.act + (int64_t)(ch.t0 + irow) * Cd + I + G * N + g * N;
  Frag<SPLIT> cf[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    float v[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int n = ks * 32 + half * 16 + 4 * q;
      floatx4 t = floatx4{0.f, 0.f, 0.f, 0.f};
      if (row_ok && n < N) t = *reinterpret_cast<const floatx4*>(crow + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[half * 4 + e] = t[e];
    }
    cf[ks] = make_frag<SPLIT>(v);
  }

  // contribution of the state entering the chunk: acc[pt] = C h_prev^T
  floatx4 acc[PT];
  const float* hp = a.states + ((int64_t)c * a.sh.H + h) * P * N;
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    acc[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      float v[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int n = ks * 32 + half * 16 + 4 * q;
        floatx4 t = floatx4{0.f, 0.f, 0.f, 0.f};
        if (n < N) t = *reinterpret_cast<const floatx4*>(hp + (pt * 16 + l16) * N + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[half * 4 + e] = t[e];
      }
      acc[pt] = mma<SPLIT>(cf[ks], make_frag<SPLIT>(v), acc[pt]);
    }
  }
  __syncthreads();   // sdA ready
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * q + r;
    const float s = i < ch.len ? __expf(sdA[i]) : 0.f;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) acc[pt][r] *= s;
  }

  const float dAi = row_ok ? sdA[irow] : 0.f;
  for (int jb = 0; jb < jend; jb += 32) {
    __syncthreads();
    for (int idx = tid; idx < 32 * (N / 4); idx += 256) {
      const int jj = idx / (N / 4), n4 = (idx % (N / 4)) * 4;
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      if (jb + jj < ch.len)
        v = *reinterpret_cast<const floatx4*>(a.act + (int64_t)(ch.t0 + jb + jj) * Cd + I + g * N + n4);
      *reinterpret_cast<floatx4*>(&sB[jj * LDB + n4]) = v;
    }
    for (int idx = tid; idx < 32 * (P / 4); idx += 256) {
      const int jj = idx / (P / 4), p4 = (idx % (P / 4)) * 4;
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      if (jb + jj < ch.len)
        v = *reinterpret_cast<const floatx4*>(a.act + (int64_t)(ch.t0 + jb + jj) * Cd + h * P + p4);
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[(p4 + e) * LDJ + jj] = v[e];
    }
    __syncthreads();
    if (jb <= i0 + 15 && i0 < ch.len) {
      // G^T tiles: lane holds G[i0 + l16][jb + 16 jt + 4q + r]
      floatx4 gt[2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        gt[jt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          float v[8];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int n = ks * 32 + half * 16 + 4 * q;
            floatx4 t = floatx4{0.f, 0.f, 0.f, 0.f};
            if (n < N) t = *reinterpret_cast<const floatx4*>(&sB[(jt * 16 + l16) * LDB + n]);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[half * 4 + e] = t[e];
          }
          gt[jt] = mma<SPLIT>(make_frag<SPLIT>(v), cf[ks], gt[jt]);
        }
      }
      float m[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = jb + (e >> 2) * 16 + 4 * q + (e & 3);
        m[e] = (row_ok && j <= irow) ? gt[e >> 2][e & 3] * __expf(dAi - sdA[j]) * sD[j] : 0.f;
      }
      const Frag<SPLIT> fm = make_frag<SPLIT>(m);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        float v[8];
        const floatx4 x0 = *reinterpret_cast<const floatx4*>(&sX[(pt * 16 + l16) * LDJ + 4 * q]);
        const floatx4 x1 = *reinterpret_cast<const floatx4*>(&sX[(pt * 16 + l16) * LDJ + 16 + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = x0[e]; v[e + 4] = x1[e]; }
        acc[pt] = mma<SPLIT>(fm, make_frag<SPLIT>(v), acc[pt]);
      }
    }
  }

  // y = acc + D x, gated; lane holds rows i0 + 4q + r, column pt*16 + l16
  const float Dh = a.D[h];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * q + r;
    if (i < ch.len) {
      const int64_t row = ch.t0 + i;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int col = h * P + pt * 16 + l16;
        const float xv = a.act[row * Cd + col];
        const float zv = load_any(a.z, row * a.z_stride + col, a.io_bf16);
        store_any(a.y, row * a.y_stride + col, (acc[pt][r] + Dh * xv) * silu(zv), a.y_bf16);
      }
    }
  }
}

// ------------------------------------------------------------------ 6. conv windows
template <int W>
__global__ __launch_bounds__(256) void window_kernel(PrefillParams a) {
  const WindowEntry we = a.windows[blockIdx.x];
  const SeqEntry sq = a.seqs[we.seq];
  const int Cd = a.sh.Cd;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= Cd) return;
  int64_t col, stride;
  const void* src = io_col(a, c, col, stride);
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
template <bool SPLIT, int P, int N>
static void launch_mfma(const PrefillParams& a, hipStream_t s) {
  hipLaunchKernelGGL((chunk_state_kernel<SPLIT, P, N>), dim3(a.num_chunks, a.sh.H), dim3(256), 0, s, a);
  const int PN = P * N;
  const dim3 gp(a.num_seqs, a.sh.H, (PN / 4 + 255) / 256);
  if (a.ssm_bf16) hipLaunchKernelGGL(state_pass_kernel<bf16>, gp, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(state_pass_kernel<float>, gp, dim3(256), 0, s, a);
  hipLaunchKernelGGL((chunk_scan_kernel<SPLIT, P, N>), dim3(a.num_chunks, a.sh.H, (a.Q + 63) / 64), dim3(256),
                     0, s, a);
}

template <int P, int N>
static void launch_pn(const PrefillParams& a, hipStream_t s) {
  if (a.ssm_bf16) launch_mfma<false, P, N>(a, s);
  else launch_mfma<true, P, N>(a, s);
}

template <int P>
static bool launch_p(const PrefillParams& a, int N, hipStream_t s) {
  switch (N) {
    case 16: launch_pn<P, 16>(a, s); return true;
    case 32: launch_pn<P, 32>(a, s); return true;
    case 64: launch_pn<P, 64>(a, s); return true;
    case 128: launch_pn<P, 128>(a, s); return true;
    case 256: launch_pn<P, 256>(a, s); return true;
    default: return false;
  }
}

bool prefill_supported(int P, int N, int W) {
  const bool p_ok = P == 16 || P == 32 || P == 64 || P == 128;
  const bool n_ok = N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
  return p_ok && n_ok && W >= 2 && W <= 4;
}

hipError_t launch_prefill(const PrefillParams& a, hipStream_t s) {
  if (a.num_chunks == 0) return hipSuccess;
  const dim3 gc(a.num_chunks, (a.sh.Cd + 255) / 256);
  switch (a.sh.W) {
    case 2: hipLaunchKernelGGL(conv_kernel<2>, gc, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(conv_kernel<3>, gc, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(conv_kernel<4>, gc, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(dt_kernel, dim3(a.num_chunks, (a.sh.H + 3) / 4), dim3(256), 0, s, a);
  bool ok = false;
  switch (a.sh.P) {
    case 16: ok = launch_p<16>(a, a.sh.N, s); break;
    case 32: ok = launch_p<32>(a, a.sh.N, s); break;
    case 64: ok = launch_p<64>(a, a.sh.N, s); break;
    case 128: ok = launch_p<128>(a, a.sh.N, s); break;
  }
  if (!ok) return hipErrorInvalidValue;
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
