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
