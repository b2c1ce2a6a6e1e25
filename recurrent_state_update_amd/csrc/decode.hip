// Fused Mamba2 decode step over a slot pool, gfx950.
//
// One workgroup of 512 threads (eight wave64s) per (sequence row, group), rows fastest in the grid.
// Phase 1 shifts the conv window of the group's channels (x of its heads,
// then its B and C), applies the depthwise conv and SiLU, and stages the
// activations in LDS, together with Delta = softplus(dt + dt_bias) and
// alpha = exp(Delta * A) for its heads and the gate SiLU(z) of its rows.  Phase 2 streams the (P, N) state of
// each head through HBM with 16-byte loads: every lane owns one 16-byte
// column slice of a state row, updates h' = alpha h + Delta x B, accumulates
// h' C, and writes h' back rounded to the state dtype.  The reduction over N
// is a butterfly over the LPR lanes that share a row which scatters the row
// sums across lanes, so the row outputs y = C h' + D x gated by SiLU(z) come
// out one per lane.
//
// The method is the Mamba recurrence of the Mamba study notes
// (echobase-5bl.pages.dev, "Mamba" equations) on the slot pool of
// "Hybrid SSM / Mamba models and non-KV state" (mlinterviewnotes.com,
// ch. 7.3: temporal state (H, P, N) and conv window (d_conv, W-1) per slot).
#include "device_common.h"
#include "kernels.h"

namespace m2 {

// Shape of the launch, the fastest combination measured on MI355X for the 8B-hybrid decode:
// state rows per lane batch, threads per workgroup, minimum waves per SIMD the register budget
// must allow.
constexpr int kDecodeRows = 8;
constexpr int kDecodeThreads = 512;
constexpr int kDecodeWavesPerEU = 1;

// The state is streamed once per step: non-temporal loads and stores keep it from displacing
// reusable lines in the caches.
template <typename V> __device__ __forceinline__ V ld_state(const V* p) { return __builtin_nontemporal_load(p); }
template <typename V> __device__ __forceinline__ void st_state(V* p, const V& v) { __builtin_nontemporal_store(v, p); }

template <typename T> struct Vec16;
template <> struct Vec16<float> { typedef floatx4 type; };
template <> struct Vec16<bf16> { typedef bf16x8 type; };

// Butterfly over the lanes that share a row: M partial row sums per lane,
// xor-offsets O, O/2, ..., 1.  While a lane holds more than one value, each
// step halves its list (the lane with bit O set keeps the upper half), so the
// sums end up scattered across lanes; afterwards plain xor-adds finish the sum.
// On return acc[k] holds the full sum of row index sel + k.
template <int M, int O> struct RowReduce {
  static __device__ __forceinline__ void run(float* acc, int lane, int& sel) {
    if constexpr (O == 0) {
      return;
    } else if constexpr (M > 1) {
      const bool up = (lane & O) != 0;
#pragma unroll
      for (int k = 0; k < M / 2; ++k) {
        const float send = up ? acc[k] : acc[k + M / 2];
        const float keep = up ? acc[k + M / 2] : acc[k];
        acc[k] = keep + __shfl_xor(send, O);
      }
      if (up) sel += M / 2;
      RowReduce<M / 2, O / 2>::run(acc, lane, sel);
    } else {
      acc[0] += __shfl_xor(acc[0], O);
      RowReduce<1, O / 2>::run(acc, lane, sel);
    }
  }
};

template <typename TS, int N, int W>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(kDecodeWavesPerEU)))
void decode_kernel(DecodeParams a) {
  typedef typename Vec16<TS>::type vec_t;
  constexpr int VEC = 16 / sizeof(TS);   // state elements per 16-byte access
  constexpr int LPR = N / VEC;           // lanes per state row
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "unsupported d_state");
  constexpr int RPI = 64 / LPR;          // rows per wave-wide access
  constexpr int U0 = kDecodeRows / RPI;
  constexpr int U = U0 < 1 ? 1 : (U0 > 16 ? 16 : U0);   // accesses in flight per lane
  constexpr int RB = RPI * U;            // rows per batch
  constexpr int MF = U > LPR ? U / LPR : 1;             // row sums held per lane at the end
  constexpr int DUP = U < LPR ? LPR / U : 1;            // lanes holding the same row sum

  const int b = blockIdx.x;   // rows fastest: consecutive workgroups (dealt round-robin over the XCDs) take
  const int g = blockIdx.y;   // the same group of different rows (measured 0.8% faster than groups fastest)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hpg = a.H / a.G;
  const int P = a.P;
  const int nx = hpg * P;
  const int slot = a.slots[b];

  if (slot < 0 || slot >= a.num_slots) {   // padding row: no pool access, zero output
    for (int i = tid; i < nx; i += blockDim.x) store_any(a.y, b * a.y_stride + g * nx + i, 0.f, a.y_bf16);
    return;
  }

  extern __shared__ float smem[];
  float* s_act = smem;                  // [x of the group's heads | B_g | C_g]
  float* s_delta = smem + nx + 2 * N;   // [hpg]
  float* s_alpha = s_delta + hpg;       // [hpg]
  float* s_gate = s_alpha + hpg;        // [nx] SiLU(z) of the group's rows

  // ---------------------------------------------------------------- state geometry
  const int sub = lane % LPR;
  const int rsub = lane / LPR;
  const int n0 = sub * VEC;
  const int nwaves = blockDim.x >> 6;
  TS* const base = static_cast<TS*>(a.ssm) + ((int64_t)slot * a.H + g * hpg) * P * N;
  // Flattened (head, row batch) tiles of this wave; with prefetch the next
  // tile's loads are issued before the current tile is computed.
  const int nbat = (P + RB - 1) / RB;
  const int my_heads = hpg > wave ? (hpg - wave + nwaves - 1) / nwaves : 0;
  const int ntile = my_heads * nbat;
  auto tile_ptr = [&](int t, int& hl, int& r0) -> TS* {
    hl = wave + (t / nbat) * nwaves;
    r0 = (t % nbat) * RB;
    return base + (int64_t)hl * P * N;
  };
  auto load_tile = [&](int t, vec_t (&d)[U]) {
    int hl, r0;
    const TS* st = tile_ptr(t, hl, r0);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int row = r0 + j * RPI + rsub;
      if (row < P) d[j] = ld_state(reinterpret_cast<const vec_t*>(st + (int64_t)row * N + n0));
    }
  };
  // one state tile held in registers ahead of the one in use; the first is requested before
  // the conv phase so that its latency overlaps it
  vec_t data[U], next[U];
  if (ntile > 0) load_tile(0, next);
  // ---------------------------------------------------------------- gate
  // SiLU(z) of the group's rows goes to LDS here, by the threads the conv pass leaves idle (all
  // threads when it leaves none), so that the state loop issues no global load besides the
  // state: a z load there would wait for the prefetched tile ahead of it in the memory counter.
  const int nch = nx + 2 * N;
  {
    const int nconv = (nch + 7) / 8 < (int)blockDim.x ? (nch + 7) / 8 : (int)blockDim.x;
    const int zn = nconv < (int)blockDim.x ? (int)blockDim.x - nconv : (int)blockDim.x;
    const int zt = nconv < (int)blockDim.x ? tid - nconv : tid;
    for (int i = zt; zt >= 0 && i < nx; i += zn)
      s_gate[i] = silu(load_any(a.z, b * a.z_stride + g * nx + i, a.io_bf16));
  }
  // ---------------------------------------------------------------- conv
  for (int ck = tid * 8; ck < nch; ck += blockDim.x * 8) {
    const void* src;
    int64_t si;
    int gc;
    if (ck < nx) {
      gc = g * nx + ck;
      src = a.x;
      si = b * a.x_stride + gc;
    } else if (ck < nx + N) {
      const int o = g * N + (ck - nx);
      gc = a.I + o;
      src = a.B;
      si = b * a.B_stride + o;
    } else {
      const int o = g * N + (ck - nx - N);
      gc = a.I + a.G * N + o;
      src = a.C;
      si = b * a.C_stride + o;
    }
    float u[8];
    load8_any(src, si, a.io_bf16, u);

    // 8 channels x (W-1) window values, contiguous and 16-byte aligned.
    float win[8 * (W - 1)];
    const int64_t woff = ((int64_t)slot * (a.I + 2 * a.G * N) + gc) * (W - 1);
    if (a.conv_bf16) {
      const bf16x8* wp = reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.conv) + woff);
#pragma unroll
      for (int v = 0; v < W - 1; ++v) {
        const bf16x8 t = wp[v];
#pragma unroll
        for (int e = 0; e < 8; ++e) win[8 * v + e] = static_cast<float>(t[e]);
      }
    } else {
      const floatx4* wp = reinterpret_cast<const floatx4*>(static_cast<const float*>(a.conv) + woff);
#pragma unroll
      for (int v = 0; v < 2 * (W - 1); ++v) {
        const floatx4 t = wp[v];
#pragma unroll
        for (int e = 0; e < 4; ++e) win[4 * v + e] = t[e];
      }
    }
    float wt[8 * W];
    const floatx4* wq = reinterpret_cast<const floatx4*>(a.conv_w + (int64_t)gc * W);
#pragma unroll
    for (int v = 0; v < 2 * W; ++v) {
      const floatx4 t = wq[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) wt[4 * v + e] = t[e];
    }
    float nw[8 * (W - 1)];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = a.conv_b[gc + c];
#pragma unroll
      for (int k = 0; k < W - 1; ++k) v += wt[c * W + k] * win[c * (W - 1) + k];
      v += wt[c * W + W - 1] * u[c];
      s_act[ck + c] = silu(v);
#pragma unroll
      for (int k = 0; k < W - 2; ++k) nw[c * (W - 1) + k] = win[c * (W - 1) + k + 1];
      nw[c * (W - 1) + W - 2] = u[c];
    }
    if (a.conv_bf16) {
      bf16x8* wp = reinterpret_cast<bf16x8*>(static_cast<bf16*>(a.conv) + woff);
#pragma unroll
      for (int v = 0; v < W - 1; ++v) {
        bf16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = from_f32<bf16>(nw[8 * v + e]);
        wp[v] = t;
      }
    } else {
      floatx4* wp = reinterpret_cast<floatx4*>(static_cast<float*>(a.conv) + woff);
#pragma unroll
      for (int v = 0; v < 2 * (W - 1); ++v) {
        floatx4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = nw[4 * v + e];
        wp[v] = t;
      }
    }
  }
  if (tid < hpg) {
    const int h = g * hpg + tid;
    const float d = softplus(load_any(a.dt, b * a.dt_stride + h, a.io_bf16) + a.dt_bias[h]);
    s_delta[tid] = d;
    s_alpha[tid] = expf(d * a.A[h]);
  }
  __syncthreads();

  // ---------------------------------------------------------------- state
  float Bv[VEC], Cv[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    Bv[e] = s_act[nx + n0 + e];
    Cv[e] = s_act[nx + N + n0 + e];
  }
  for (int t = 0; t < ntile; ++t) {
#pragma unroll
    for (int j = 0; j < U; ++j) data[j] = next[j];
    if (t + 1 < ntile) load_tile(t + 1, next);
    int hl, r0;
    TS* const st = tile_ptr(t, hl, r0);
    const float delta = s_delta[hl];
    const float alpha = s_alpha[hl];
    const int h = g * hpg + hl;
    const float* xs = s_act + hl * P;
    float acc[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int row = r0 + j * RPI + rsub;
      acc[j] = 0.f;
      if (row < P) {
        const float dx = delta * xs[row];
        vec_t o;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float hn = alpha * to_f32(data[j][e]) + dx * Bv[e];
          acc[j] += hn * Cv[e];
          o[e] = from_f32<TS>(hn);
        }
        st_state(reinterpret_cast<vec_t*>(st + (int64_t)row * N + n0), o);
      }
    }
    int sel = 0;
    RowReduce<U, LPR / 2>::run(acc, lane, sel);
    if ((lane % DUP) == 0) {
      const float Dh = a.D[h];
#pragma unroll
      for (int k = 0; k < MF; ++k) {
        const int row = r0 + (sel + k) * RPI + rsub;
        if (row < P) {
          const int64_t ci = (int64_t)h * P + row;
          const float yv = acc[k] + Dh * xs[row];
          store_any(a.y, b * a.y_stride + ci, yv * s_gate[hl * P + row], a.y_bf16);
        }
      }
    }
  }
}

template <typename TS, int N>
static hipError_t launch_w(const DecodeParams& p, int W, int batch, hipStream_t s) {
  const int hpg = p.H / p.G;
  const size_t lds = decode_lds_bytes(hpg, p.P, N);
  const dim3 grid(batch, p.G), block(kDecodeThreads);
#define D_LAUNCH(WW)                                                                                      \
  {                                                                                                       \
    if (lds > 65536) {                                                                                    \
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<TS, N, WW>),  \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);     \
      if (e != hipSuccess) return e;                                                                      \
    }                                                                                                     \
    hipLaunchKernelGGL((decode_kernel<TS, N, WW>), grid, block, lds, s, p);                              \
  }
  switch (W) {
    case 2: D_LAUNCH(2) break;
    case 3: D_LAUNCH(3) break;
    case 4: D_LAUNCH(4) break;
    default: return hipErrorInvalidValue;
  }
#undef D_LAUNCH
  return hipGetLastError();
}

template <typename TS>
static hipError_t launch_n(const DecodeParams& p, int N, int W, int batch, hipStream_t s) {
  switch (N) {
    case 16: return launch_w<TS, 16>(p, W, batch, s);
    case 32: return launch_w<TS, 32>(p, W, batch, s);
    case 64: return launch_w<TS, 64>(p, W, batch, s);
    case 128: return launch_w<TS, 128>(p, W, batch, s);
    case 256: return launch_w<TS, 256>(p, W, batch, s);
    default: return hipErrorInvalidValue;
  }
}

bool decode_supported(int /*ssm_bf16*/, int N, int W) {
  return (N == 16 || N == 32 || N == 64 || N == 128 || N == 256) && W >= 2 && W <= 4;
}

hipError_t launch_decode(const DecodeParams& p, int N, int W, int batch, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  return p.ssm_bf16 ? launch_n<bf16>(p, N, W, batch, s) : launch_n<float>(p, N, W, batch, s);
}

}  // namespace m2
