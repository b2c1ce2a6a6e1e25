// Multi-token (speculative) decode over a slot pool, gfx950.
//
// A speculative step feeds a sequence its verified token and its draft tokens
// at once, and must keep the state after each of them, because the verifier
// may accept any prefix of the drafts ("Hybrid SSM / Mamba models and non-KV
// state", mlinterviewnotes.com ch. 7.3: the conv state widened by num_spec
// columns and one state block per speculative token).  Here the state after
// token t is written, with its conv window, into a slot of its own, so the
// accepted position is a slot to switch to and every slot keeps the plain
// (H, P, N) + (d_conv, W-1) layout.
//
// The kernel is the decode kernel's layout run over K tokens: one workgroup of
// 1024 threads per (sequence, group).  Phase 1 (four channels per thread) slides
// each channel's window over the K inputs (conv + SiLU per token, the window after every token written to
// that token's slot) and stages the K activation sets in LDS.  Phase 2 reads
// each state tile once and applies the K tokens in order, storing the rounded
// state after each token (which is also what the next token reads, as in K
// single decode steps) and reducing each token's readout over N with the same
// butterfly, so the outputs and states equal K single decode steps bit for bit.
// HBM traffic per sequence: one state read, K state writes.
#include "device_common.h"
#include "spec_decode.h"

namespace m2 {

constexpr int kMultiThreads = 1024;   // one wave per head of a 16-head group (measured: 512 threads 3% slower)
constexpr int kMultiRows = 8;

template <typename T> struct MVec16;
template <> struct MVec16<float> { typedef floatx4 type; };
template <> struct MVec16<bf16> { typedef bf16x8 type; };

template <int M, int O> struct MRowReduce {
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
      MRowReduce<M / 2, O / 2>::run(acc, lane, sel);
    } else {
      acc[0] += __shfl_xor(acc[0], O);
      MRowReduce<1, O / 2>::run(acc, lane, sel);
    }
  }
};

__device__ __forceinline__ int uniform_slot(const int32_t* p) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  return *(const cint*)p;
}

template <typename TS, int N, int W>
__global__ __launch_bounds__(kMultiThreads) void decode_multi_kernel(MultiDecodeParams m) {
  const DecodeParams& a = m.d;
  typedef typename MVec16<TS>::type vec_t;
  constexpr int VEC = 16 / sizeof(TS);
  constexpr int LPR = N / VEC;
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "unsupported d_state");
  constexpr int RPI = 64 / LPR;
  constexpr int U0 = kMultiRows / RPI;
  constexpr int U = U0 < 1 ? 1 : (U0 > 16 ? 16 : U0);
  constexpr int RB = RPI * U;
  constexpr int MF = U > LPR ? U / LPR : 1;
  constexpr int DUP = U < LPR ? LPR / U : 1;

  const int b = blockIdx.x;   // rows fastest in the grid, as in the single-token decode
  const int g = blockIdx.y;
  const int K = m.K;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hpg = a.H / a.G;
  const int P = a.P;
  const int nx = hpg * P;
  const int nch = nx + 2 * N;
  const int slot = uniform_slot(a.slots + b);

  if (slot < 0 || slot >= a.num_slots) {   // padding row: no pool access, zero outputs
    for (int i = tid; i < K * nx; i += blockDim.x)
      store_any(a.y, (int64_t)(b * K + i / nx) * a.y_stride + g * nx + i % nx, 0.f, a.y_bf16);
    return;
  }

  extern __shared__ float smem[];
  float* s_act = smem;                     // [K][x of the group's heads | B_g | C_g]
  float* s_delta = smem + K * nch;         // [K][hpg]
  float* s_alpha = s_delta + K * hpg;      // [K][hpg]
  int* s_out = reinterpret_cast<int*>(s_alpha + K * hpg);   // [K] output slot per token (-1: none)
  float* s_gate = reinterpret_cast<float*>(s_out + K);      // [K][nx] SiLU(z) of the group's rows

  if (tid < K) {
    const int o = m.slots_out[(int64_t)b * K + tid];
    s_out[tid] = (o >= 0 && o < a.num_slots) ? o : -1;
  }

  // ---------------------------------------------------------------- state geometry
  const int sub = lane % LPR;
  const int rsub = lane / LPR;
  const int n0 = sub * VEC;
  const int nwaves = blockDim.x >> 6;
  const int64_t head0 = (int64_t)g * hpg;
  const TS* const base = static_cast<const TS*>(a.ssm) + ((int64_t)slot * a.H + head0) * P * N;
  const int nbat = (P + RB - 1) / RB;
  const int my_heads = hpg > wave ? (hpg - wave + nwaves - 1) / nwaves : 0;
  const int ntile = my_heads * nbat;
  auto tile_of = [&](int t, int& hl, int& r0) {
    hl = wave + (t / nbat) * nwaves;
    r0 = (t % nbat) * RB;
  };
  auto load_tile = [&](int t, vec_t (&d)[U]) {
    int hl, r0;
    tile_of(t, hl, r0);
    const TS* st = base + (int64_t)hl * P * N;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int row = r0 + j * RPI + rsub;
      if (row < P) d[j] = __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(st + (int64_t)row * N + n0));
    }
  };
  vec_t data[U], next[U];
  if (ntile > 0) load_tile(0, next);

  // ---------------------------------------------------------------- gate
  // SiLU(z) of the group's rows for every token goes to LDS here, by the threads the conv pass
  // leaves idle (all threads when it leaves none): a z load in the state loop would be issued
  // after the next tile's state loads and, the memory counter being in order, wait for them.
  {
    const int nconv = (nch + 3) / 4 < (int)blockDim.x ? (nch + 3) / 4 : (int)blockDim.x;
    const int zn = nconv < (int)blockDim.x ? (int)blockDim.x - nconv : (int)blockDim.x;
    const int zt = nconv < (int)blockDim.x ? tid - nconv : tid;
    for (int i = zt; zt >= 0 && i < K * nx; i += zn) {
      const int t = i / nx, c = i - t * nx;
      s_gate[i] = silu(load_any(a.z, (int64_t)(b * K + t) * a.z_stride + (int64_t)g * nx + c, a.io_bf16));
    }
  }

  // ---------------------------------------------------------------- conv over the K tokens
  // four channels per thread (what stays live across the token loop is their taps and windows)
  const int64_t cd = a.I + 2 * a.G * N;
  for (int ck = tid * 4; ck < nch; ck += blockDim.x * 4) {
    const void* src;
    int64_t col, stride;
    int gc;
    if (ck < nx) {
      gc = g * nx + ck;
      src = a.x;
      col = gc;
      stride = a.x_stride;
    } else if (ck < nx + N) {
      const int o = g * N + (ck - nx);
      gc = a.I + o;
      src = a.B;
      col = o;
      stride = a.B_stride;
    } else {
      const int o = g * N + (ck - nx - N);
      gc = a.I + a.G * N + o;
      src = a.C;
      col = o;
      stride = a.C_stride;
    }
    // 4 channels x (W-1) window values, contiguous: 8-byte pieces (bf16) or 16-byte (fp32)
    float win[4 * (W - 1)];
    const int64_t woff = ((int64_t)slot * cd + gc) * (W - 1);
    if (a.conv_bf16) {
      const uint2* wp = reinterpret_cast<const uint2*>(static_cast<const bf16*>(a.conv) + woff);
#pragma unroll
      for (int v = 0; v < W - 1; ++v) {
        const uint2 t = wp[v];
        win[4 * v + 0] = __uint_as_float(t.x << 16);
        win[4 * v + 1] = __uint_as_float(t.x & 0xffff0000u);
        win[4 * v + 2] = __uint_as_float(t.y << 16);
        win[4 * v + 3] = __uint_as_float(t.y & 0xffff0000u);
      }
    } else {
      const floatx4* wp = reinterpret_cast<const floatx4*>(static_cast<const float*>(a.conv) + woff);
#pragma unroll
      for (int v = 0; v < W - 1; ++v) {
        const floatx4 t = wp[v];
#pragma unroll
        for (int e = 0; e < 4; ++e) win[4 * v + e] = t[e];
      }
    }
    float wt[4 * W];
    const floatx4* wq = reinterpret_cast<const floatx4*>(a.conv_w + (int64_t)gc * W);
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const floatx4 t = wq[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) wt[4 * v + e] = t[e];
    }
    float bias[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bias[c] = a.conv_b[gc + c];
    for (int t = 0; t < K; ++t) {
      float u[4];
      const int64_t ui = (int64_t)(b * K + t) * stride + col;
      if (a.io_bf16) {
        const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const bf16*>(src) + ui);
        u[0] = __uint_as_float(r.x << 16);
        u[1] = __uint_as_float(r.x & 0xffff0000u);
        u[2] = __uint_as_float(r.y << 16);
        u[3] = __uint_as_float(r.y & 0xffff0000u);
      } else {
        const floatx4 r = *reinterpret_cast<const floatx4*>(static_cast<const float*>(src) + ui);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = r[e];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float v = bias[c];
#pragma unroll
        for (int k = 0; k < W - 1; ++k) v += wt[c * W + k] * win[c * (W - 1) + k];
        v += wt[c * W + W - 1] * u[c];
        s_act[t * nch + ck + c] = silu(v);
        // slide: the window after token t, rounded to the conv dtype as decode stores it
#pragma unroll
        for (int k = 0; k < W - 2; ++k) win[c * (W - 1) + k] = win[c * (W - 1) + k + 1];
        win[c * (W - 1) + W - 2] = a.conv_bf16 ? static_cast<float>(from_f32<bf16>(u[c])) : u[c];
      }
      const int o = uniform_slot(m.slots_out + (int64_t)b * K + t);
      if (o >= 0 && o < a.num_slots) {
        const int64_t ooff = ((int64_t)o * cd + gc) * (W - 1);
        if (a.conv_bf16) {
          uint2* wp = reinterpret_cast<uint2*>(static_cast<bf16*>(a.conv) + ooff);
#pragma unroll
          for (int v = 0; v < W - 1; ++v) {
            // the values are bf16 already: their upper halves are the bf16 bits
            const uint32_t b0 = __float_as_uint(win[4 * v + 0]) >> 16, b1 = __float_as_uint(win[4 * v + 1]) >> 16;
            const uint32_t b2 = __float_as_uint(win[4 * v + 2]) >> 16, b3 = __float_as_uint(win[4 * v + 3]) >> 16;
            wp[v] = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
          }
        } else {
          floatx4* wp = reinterpret_cast<floatx4*>(static_cast<float*>(a.conv) + ooff);
#pragma unroll
          for (int v = 0; v < W - 1; ++v) wp[v] = floatx4{win[4 * v], win[4 * v + 1], win[4 * v + 2], win[4 * v + 3]};
        }
      }
    }
  }
  for (int i = tid; i < K * hpg; i += blockDim.x) {
    const int t = i / hpg, hl = i % hpg;
    const int h = g * hpg + hl;
    const float d = softplus(load_any(a.dt, (int64_t)(b * K + t) * a.dt_stride + h, a.io_bf16) + a.dt_bias[h]);
    s_delta[i] = d;
    s_alpha[i] = expf(d * a.A[h]);
  }
  __syncthreads();

  // ---------------------------------------------------------------- state, K tokens per tile
  for (int ti = 0; ti < ntile; ++ti) {
#pragma unroll
    for (int j = 0; j < U; ++j) data[j] = next[j];
    if (ti + 1 < ntile) load_tile(ti + 1, next);
    int hl, r0;
    tile_of(ti, hl, r0);
    const int h = g * hpg + hl;
    const float Dh = a.D[h];
    for (int t = 0; t < K; ++t) {
      const float* act = s_act + t * nch;
      const float delta = s_delta[t * hpg + hl];
      const float alpha = s_alpha[t * hpg + hl];
      const float* xs = act + hl * P;
      float Bv[VEC], Cv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        Bv[e] = act[nx + n0 + e];
        Cv[e] = act[nx + N + n0 + e];
      }
      const int o = s_out[t];
      TS* const ost = o >= 0 ? static_cast<TS*>(a.ssm) + ((int64_t)o * a.H + head0 + hl) * P * N : nullptr;
      float acc[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int row = r0 + j * RPI + rsub;
        acc[j] = 0.f;
        if (row < P) {
          const float dx = delta * xs[row];
          vec_t nv;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float hn = alpha * to_f32(data[j][e]) + dx * Bv[e];
            acc[j] += hn * Cv[e];
            nv[e] = from_f32<TS>(hn);
          }
          data[j] = nv;
          if (o >= 0) __builtin_nontemporal_store(nv, reinterpret_cast<vec_t*>(ost + (int64_t)row * N + n0));
        }
      }
      int sel = 0;
      MRowReduce<U, LPR / 2>::run(acc, lane, sel);
      if ((lane % DUP) == 0) {
#pragma unroll
        for (int k = 0; k < MF; ++k) {
          const int row = r0 + (sel + k) * RPI + rsub;
          if (row < P) {
            const int64_t ci = (int64_t)h * P + row;
            const float yv = acc[k] + Dh * xs[row];
            store_any(a.y, (int64_t)(b * K + t) * a.y_stride + ci, yv * s_gate[t * nx + hl * P + row], a.y_bf16);
          }
        }
      }
    }
  }
}

template <typename TS, int N>
static hipError_t launch_mw(const MultiDecodeParams& p, int W, int batch, hipStream_t s) {
  const DecodeParams& d = p.d;
  const int hpg = d.H / d.G;
  const size_t lds = multi_decode_lds_bytes(hpg, d.P, N, p.K);
  const dim3 grid(batch, d.G), block(kMultiThreads);
#define MW_LAUNCH(WW)                                                                                         \
  {                                                                                                           \
    if (lds > 65536) {                                                                                        \
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_multi_kernel<TS, N, WW>), \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);         \
      if (e != hipSuccess) return e;                                                                          \
    }                                                                                                         \
    hipLaunchKernelGGL((decode_multi_kernel<TS, N, WW>), grid, block, lds, s, p);                            \
  }
  switch (W) {
    case 2: MW_LAUNCH(2) break;
    case 3: MW_LAUNCH(3) break;
    case 4: MW_LAUNCH(4) break;
    default: return hipErrorInvalidValue;
  }
#undef MW_LAUNCH
  return hipGetLastError();
}

template <typename TS>
static hipError_t launch_mn(const MultiDecodeParams& p, int N, int W, int batch, hipStream_t s) {
  switch (N) {
    case 16: return launch_mw<TS, 16>(p, W, batch, s);
    case 32: return launch_mw<TS, 32>(p, W, batch, s);
    case 64: return launch_mw<TS, 64>(p, W, batch, s);
    case 128: return launch_mw<TS, 128>(p, W, batch, s);
    case 256: return launch_mw<TS, 256>(p, W, batch, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_multi(const MultiDecodeParams& p, int N, int W, int batch, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (p.K < 1 || p.K > kMaxDecodeTokens) return hipErrorInvalidValue;
  return p.d.ssm_bf16 ? launch_mn<bf16>(p, N, W, batch, s) : launch_mn<float>(p, N, W, batch, s);
}

}  // namespace m2
