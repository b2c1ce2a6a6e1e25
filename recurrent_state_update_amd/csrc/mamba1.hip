// Mamba1 decode step over a slot pool, gfx950: the second recurrent family the
// pool holds.  The recurrence is the one of the Mamba study notes
// (echobase-5bl.pages.dev, "Mamba" equations) with the Mamba1 shapes of the
// state-shape table on the same page: a (D, N) state, one decay per channel
// and state index exp(Delta_d A[d][n]), B and C shared by all channels, the
// short conv over the D channels of x.
//
// One workgroup of 256 threads covers a block of channels of one sequence.
// Phase 1: one thread per channel shifts the conv window, convolves, applies
// SiLU and softplus, and stages x_d and Delta_d in LDS with the row's B and C.
// Phase 2: a channel's N state values are split over N/VEC lanes, each with one
// 16-byte non-temporal access (requested before phase 1, so the load overlaps
// it); the lanes update their values, reduce h' C over the channel's lanes with
// xor shuffles, and the first lane writes y_d = (sum + D_d x_d) SiLU(z_d).
// HBM-bound: per sequence the state is read and written once.
#include "device_common.h"
#include "mamba1.h"

namespace m2 {

constexpr int kM1Threads = 256;

template <typename T> struct M1Vec;
template <> struct M1Vec<float> { typedef floatx4 type; };
template <> struct M1Vec<bf16> { typedef bf16x8 type; };

__device__ __forceinline__ int m1_uniform(const int32_t* p) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  return *(const cint*)p;
}

template <typename TS, int N, int W>
__global__ __launch_bounds__(kM1Threads) void mamba1_decode_kernel(Mamba1Params a) {
  typedef typename M1Vec<TS>::type vec_t;
  constexpr int VEC = 16 / sizeof(TS);      // state values per 16-byte access
  constexpr int LPC = N / VEC;              // lanes per channel
  static_assert(LPC >= 1 && LPC <= 64 && (64 % LPC) == 0, "unsupported d_state");
  constexpr int CPW = kM1Threads / LPC;     // channels per workgroup
  __shared__ float s_x[CPW], s_dl[CPW], s_B[N], s_C[N];

  const int b = blockIdx.y;
  const int d0 = blockIdx.x * CPW;
  const int tid = threadIdx.x;
  const int D = a.D;
  const int slot = m1_uniform(a.slots + b);
  if (slot < 0 || slot >= a.num_slots) {   // padding row: no pool access, zero outputs
    if (tid < CPW && d0 + tid < D) store_any(a.y, b * a.y_stride + d0 + tid, 0.f, a.y_bf16);
    return;
  }
  // this lane's state values, requested first
  const int c = tid / LPC, sub = tid % LPC;
  const int d = d0 + c;
  const int n0 = sub * VEC;
  TS* const st = static_cast<TS*>(a.ssm) + ((int64_t)slot * D + d) * N + n0;
  vec_t h;
  if (d < D) h = __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(st));

  // ---------------------------------------------------------------- phase 1
  if (tid < CPW && d0 + tid < D) {
    const int dc = d0 + tid;
    float win[W - 1];
    const int64_t woff = ((int64_t)slot * D + dc) * (W - 1);
#pragma unroll
    for (int k = 0; k < W - 1; ++k) win[k] = load_any(a.conv, woff + k, a.conv_bf16);
    const float u = load_any(a.x, b * a.x_stride + dc, a.io_bf16);
    float v = a.conv_b[dc];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) v += a.conv_w[(int64_t)dc * W + k] * win[k];
    v += a.conv_w[(int64_t)dc * W + W - 1] * u;
    s_x[tid] = silu(v);
    s_dl[tid] = softplus(load_any(a.dt, b * a.dt_stride + dc, a.io_bf16) + a.dt_bias[dc]);
#pragma unroll
    for (int k = 0; k < W - 2; ++k) store_any(a.conv, woff + k, win[k + 1], a.conv_bf16);
    store_any(a.conv, woff + W - 2, u, a.conv_bf16);
  }
  for (int n = tid; n < N; n += kM1Threads) {
    s_B[n] = load_any(a.B, b * a.B_stride + n, a.io_bf16);
    s_C[n] = load_any(a.C, b * a.C_stride + n, a.io_bf16);
  }
  __syncthreads();

  // ---------------------------------------------------------------- phase 2
  float part = 0.f;
  if (d < D) {
    const float x = s_x[c], dl = s_dl[c];
    const float dx = dl * x;
    const float* Ar = a.A + (int64_t)d * N + n0;
    vec_t o;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float al = __builtin_amdgcn_exp2f(dl * Ar[e] * 1.4426950408889634f);
      const float hn = al * to_f32(h[e]) + dx * s_B[n0 + e];
      part += hn * s_C[n0 + e];
      o[e] = from_f32<TS>(hn);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<vec_t*>(st));
  }
#pragma unroll
  for (int m = LPC / 2; m >= 1; m /= 2) part += __shfl_xor(part, m);
  if (d < D && sub == 0) {
    const float yv = part + a.Dk[d] * s_x[c];
    const float zv = load_any(a.z, b * a.z_stride + d, a.io_bf16);
    store_any(a.y, b * a.y_stride + d, yv * silu(zv), a.y_bf16);
  }
}

template <typename TS, int N>
static hipError_t launch_m1w(const Mamba1Params& p, int W, int batch, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(TS);
  constexpr int CPW = kM1Threads / (N / VEC);
  const dim3 grid((p.D + CPW - 1) / CPW, batch), block(kM1Threads);
  switch (W) {
    case 2: hipLaunchKernelGGL((mamba1_decode_kernel<TS, N, 2>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((mamba1_decode_kernel<TS, N, 3>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((mamba1_decode_kernel<TS, N, 4>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TS>
static hipError_t launch_m1n(const Mamba1Params& p, int N, int W, int batch, hipStream_t s) {
  switch (N) {
    case 8: return launch_m1w<TS, 8>(p, W, batch, s);
    case 16: return launch_m1w<TS, 16>(p, W, batch, s);
    case 32: return launch_m1w<TS, 32>(p, W, batch, s);
    case 64: return launch_m1w<TS, 64>(p, W, batch, s);
    case 128: return launch_m1w<TS, 128>(p, W, batch, s);
    case 256: return launch_m1w<TS, 256>(p, W, batch, s);
    default: return hipErrorInvalidValue;
  }
}

bool mamba1_supported(int N, int W) {
  return (N == 8 || N == 16 || N == 32 || N == 64 || N == 128 || N == 256) && W >= 2 && W <= 4;
}

hipError_t launch_mamba1_decode(const Mamba1Params& p, int N, int W, int batch, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  return p.ssm_bf16 ? launch_m1n<bf16>(p, N, W, batch, s) : launch_m1n<float>(p, N, W, batch, s);
}

}  // namespace m2

// ============================================================================ prefill
// Three launches: (1) each chunk's end state from a zero state and its per-channel sum of Delta,
// all chunks at once; (2) per (sequence, channel, state index) the pass through the sequence's
// chunks, h <- exp(A sum Delta) h + S_c, writing the state entering each chunk; (3) each chunk's
// tokens again from its entering state, with the outputs, the checkpoint states at their tokens
// and the final state.  Launches (1) and (3) give a channel's state values to N/8 lanes of one
// wave, run the token recurrence in fp32 registers (inputs of the next token requested before the
// current one is computed) and reduce h C over the channel's lanes with xor shuffles.
namespace m2 {

constexpr int kM1PThreads = 64;
constexpr int kM1PV = 8;   // state values per lane

template <int W> struct M1Tok {   // one token's inputs for one lane
  float u, dt, z;
  float B[kM1PV], C[kM1PV];
};

template <bool OUT, int N, int W>
__device__ __forceinline__ void m1_load_tok(const Mamba1PrefillParams& a, int64_t row, int d, int n0,
                                            M1Tok<W>& t) {
  t.u = load_any(a.x, row * a.x_stride + d, a.io_bf16);
  t.dt = load_any(a.dt, row * a.dt_stride + d, a.io_bf16);
  load8_any(a.B, row * a.B_stride + n0, a.io_bf16, t.B);
  if (OUT) {
    t.z = load_any(a.z, row * a.z_stride + d, a.io_bf16);
    load8_any(a.C, row * a.C_stride + n0, a.io_bf16, t.C);
  }
}

// OUT = false: launch (1); OUT = true: launch (3).
template <typename TS, bool OUT, int N, int W>
__global__ __launch_bounds__(kM1PThreads) void mamba1_chunk_kernel(Mamba1PrefillParams a) {
  constexpr int LPC = N / kM1PV;
  constexpr int CPW = kM1PThreads / LPC;
  const int ci = blockIdx.y;
  const M1Chunk ch = a.chunks[ci];
  const M1Seq sq = a.seqs[ch.seq];
  const int lane = threadIdx.x;
  const int c = lane / LPC, sub = lane % LPC;
  const int d = blockIdx.x * CPW + c;
  const int n0 = sub * kM1PV;
  const bool on = d < a.D;
  const int dd = on ? d : 0;   // lanes past D run on channel 0 and store nothing
  const int D = a.D;
  const float kLog2e = 1.4426950408889634f;
  float A2[kM1PV], h[kM1PV];
#pragma unroll
  for (int e = 0; e < kM1PV; ++e) A2[e] = a.A[(int64_t)dd * N + n0 + e] * kLog2e;
  if (OUT) {
    const float* hin = a.Hin + ((int64_t)ci * D + dd) * N + n0;
#pragma unroll
    for (int e = 0; e < kM1PV; ++e) h[e] = hin[e];
  } else {
#pragma unroll
    for (int e = 0; e < kM1PV; ++e) h[e] = 0.f;
  }
  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = a.conv_w[(int64_t)dd * W + k];
  const float cb = a.conv_b[dd], bias = a.dt_bias[dd], Dd = a.Dk[dd];
  // the W-1 raw inputs before the chunk: earlier rows of the sequence, else the slot's window
  float win[W - 1];
  float* const w0 = a.Win0 + ((int64_t)ch.seq * D + dd) * (W - 1);
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int tau = ch.tau0 - (W - 1) + k;
    if (tau >= 0) win[k] = load_any(a.x, (int64_t)(sq.t0 + tau) * a.x_stride + dd, a.io_bf16);
    else if (OUT) win[k] = w0[W - 1 + tau];   // the slot's window, as launch (1) read it
    else if (sq.has_init) win[k] = load_any(a.conv, ((int64_t)sq.slot * D + dd) * (W - 1) + (W - 1 + tau), a.conv_bf16);
    else win[k] = 0.f;
  }
  if (!OUT && ch.tau0 == 0 && on && sub == 0) {
#pragma unroll
    for (int k = 0; k < W - 1; ++k) w0[k] = win[k];
  }
  auto store_state = [&](int slot) {
    TS* st = static_cast<TS*>(a.ssm) + ((int64_t)slot * D + d) * N + n0;
#pragma unroll
    for (int e = 0; e < kM1PV; ++e) st[e] = from_f32<TS>(h[e]);
    if (sub == 0) {
#pragma unroll
      for (int k = 0; k < W - 1; ++k) store_any(a.conv, ((int64_t)slot * D + d) * (W - 1) + k, win[k], a.conv_bf16);
    }
  };
  float sumd = 0.f;
  M1Tok<W> cur, nxt;
  if (ch.len > 0) m1_load_tok<OUT, N, W>(a, ch.t0, dd, n0, nxt);
  for (int t = 0; t < ch.len; ++t) {
    cur = nxt;
    if (t + 1 < ch.len) m1_load_tok<OUT, N, W>(a, ch.t0 + t + 1, dd, n0, nxt);
    float v = cb;
#pragma unroll
    for (int k = 0; k < W - 1; ++k) v += w[k] * win[k];
    v += w[W - 1] * cur.u;
#pragma unroll
    for (int k = 0; k < W - 2; ++k) win[k] = win[k + 1];
    win[W - 2] = cur.u;
    const float xv = silu(v);
    const float dl = softplus(cur.dt + bias);
    const float dx = dl * xv;
    sumd += dl;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < kM1PV; ++e) {
      h[e] = __builtin_amdgcn_exp2f(dl * A2[e]) * h[e] + dx * cur.B[e];
      if (OUT) part += h[e] * cur.C[e];
    }
    if (OUT) {
#pragma unroll
      for (int m = LPC / 2; m >= 1; m /= 2) part += __shfl_xor(part, m);
      if (on && sub == 0)
        store_any(a.y, (int64_t)(ch.t0 + t) * a.y_stride + d, (part + Dd * xv) * silu(cur.z), a.y_bf16);
      if (a.ckpt_interval > 0 && on) {
        const int64_t p = (int64_t)sq.start_pos + ch.tau0 + t + 1;
        if (p % a.ckpt_interval == 0) {
          const int64_t k = p / a.ckpt_interval - sq.start_pos / a.ckpt_interval - 1;
          if (k >= 0 && k < sq.nck) {
            const int slot = a.ck[sq.ck0 + k];
            if (slot >= 0 && slot < a.num_slots) store_state(slot);
          }
        }
      }
    }
  }
  if (!on) return;
  if (OUT) {
    if (ch.tau0 + ch.len == sq.len) store_state(sq.slot);
  } else {
    float* s = a.S + ((int64_t)ci * D + d) * N + n0;
#pragma unroll
    for (int e = 0; e < kM1PV; ++e) s[e] = h[e];
    if (sub == 0) a.SD[(int64_t)ci * D + d] = sumd;
  }
}

// Launch (2): one thread per (channel, state index) of one sequence.
template <typename TS>
__global__ __launch_bounds__(256) void mamba1_pass_kernel(Mamba1PrefillParams a, int N) {
  const M1Seq sq = a.seqs[blockIdx.y];
  const int64_t DN = (int64_t)a.D * N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= DN || sq.len == 0) return;
  const int d = (int)(i / N);
  float h = sq.has_init ? to_f32(static_cast<const TS*>(a.ssm)[(int64_t)sq.slot * DN + i]) : 0.f;
  const float A2 = a.A[i] * 1.4426950408889634f;
  for (int cj = sq.chunk0; cj < a.num_chunks && a.chunks[cj].seq == (int)blockIdx.y; ++cj) {
    a.Hin[(int64_t)cj * DN + i] = h;
    h = __builtin_amdgcn_exp2f(A2 * a.SD[(int64_t)cj * a.D + d]) * h + a.S[(int64_t)cj * DN + i];
  }
}

template <typename TS, int N>
static hipError_t launch_m1p_n(const Mamba1PrefillParams& a, int W, hipStream_t s) {
  constexpr int CPW = kM1PThreads / (N / kM1PV);
  const dim3 gc((a.D + CPW - 1) / CPW, a.num_chunks), gp((unsigned)(((int64_t)a.D * N + 255) / 256), a.num_seqs);
#define M1P_W(WW)                                                                                   \
  hipLaunchKernelGGL((mamba1_chunk_kernel<TS, false, N, WW>), gc, dim3(kM1PThreads), 0, s, a);      \
  hipLaunchKernelGGL((mamba1_pass_kernel<TS>), gp, dim3(256), 0, s, a, N);                          \
  hipLaunchKernelGGL((mamba1_chunk_kernel<TS, true, N, WW>), gc, dim3(kM1PThreads), 0, s, a);
  switch (W) {
    case 2: M1P_W(2) break;
    case 3: M1P_W(3) break;
    case 4: M1P_W(4) break;
    default: return hipErrorInvalidValue;
  }
#undef M1P_W
  return hipGetLastError();
}

template <typename TS>
static hipError_t launch_m1p(const Mamba1PrefillParams& a, int N, int W, hipStream_t s) {
  switch (N) {
    case 8: return launch_m1p_n<TS, 8>(a, W, s);
    case 16: return launch_m1p_n<TS, 16>(a, W, s);
    case 32: return launch_m1p_n<TS, 32>(a, W, s);
    case 64: return launch_m1p_n<TS, 64>(a, W, s);
    case 128: return launch_m1p_n<TS, 128>(a, W, s);
    case 256: return launch_m1p_n<TS, 256>(a, W, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mamba1_prefill(const Mamba1PrefillParams& a, int N, int W, hipStream_t s) {
  if (a.num_chunks == 0) return hipSuccess;
  return a.ssm_bf16 ? launch_m1p<bf16>(a, N, W, s) : launch_m1p<float>(a, N, W, s);
}

}  // namespace m2
