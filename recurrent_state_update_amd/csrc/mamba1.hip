// Mamba1 decode step over a slot pool, gfx950: the second recurrent family the
// pool holds.  The recurrence is the one of the Mamba study notes
// (echobase-5bl.pages.dev, "Mamba" equations) with the Mamba1 shapes of the
// state-shape table on the same page: a (D, N) state, one decay per channel
// and state index exp(Delta_d A[d][n]), B and C shared by all channels, the
// short conv over the D channels of x.
//
// One workgroup of 512 threads covers a block of channels of one sequence
// (with states of at most 32 bytes per channel, two channels per lane group).
// Phase 1: one thread per channel shifts the conv window, convolves, applies
// SiLU and softplus, and stages Delta_d, Delta_d x_d, D_d x_d and SiLU(z_d) in
// LDS with the row's B and C.
// Phase 2: a channel's N state values are split over N/VEC lanes, each with one
// 16-byte non-temporal access (requested before phase 1, so the load overlaps
// it); the lanes update their values, reduce h' C over the channel's lanes with
// xor shuffles, and the first lane writes y_d = (sum + D_d x_d) SiLU(z_d).
// HBM-bound: per sequence the state is read and written once.
#include "device_common.h"
#include "mamba1.h"

namespace m2 {

constexpr int kM1Threads = 512;



template <typename T> struct M1Vec;
template <> struct M1Vec<float> { typedef floatx4 type; };
template <> struct M1Vec<bf16> { typedef bf16x8 type; };

__device__ __forceinline__ int m1_uniform(const int32_t* p) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  return *(const cint*)p;
}

template <typename TS, int N> constexpr int m1_passes() { return N * (int)sizeof(TS) <= 32 ? 2 : 1; }

template <typename TS, int N, int W>
__global__ __launch_bounds__(kM1Threads) void mamba1_decode_kernel(Mamba1Params a) {
  typedef typename M1Vec<TS>::type vec_t;
  constexpr int VEC = 16 / sizeof(TS);      // state values per 16-byte access
  constexpr int LPC = N / VEC;              // lanes per channel
  static_assert(LPC >= 1 && LPC <= 64 && (64 % LPC) == 0, "unsupported d_state");
  constexpr int CPP = kM1Threads / LPC;     // channels per pass of the workgroup's lanes
  constexpr int NPASS = m1_passes<TS, N>(); // passes: with small states a lane holds two channels'
                                            // values, so twice the bytes are in flight
  constexpr int CPW = CPP * NPASS;          // channels per workgroup
  __shared__ float s_dl[CPW], s_dx[CPW], s_yx[CPW], s_g[CPW], s_B[N], s_C[N];

  const int b = blockIdx.y;
  const int d0 = blockIdx.x * CPW;
  const int tid = threadIdx.x;
  const int D = a.D;
  const int slot = m1_uniform(a.slots + b);
  if (slot < 0 || slot >= a.num_slots) {   // padding row: no pool access, zero outputs
    for (int i = tid; i < CPW; i += kM1Threads)
      if (d0 + i < D) store_any(a.y, b * a.y_stride + d0 + i, 0.f, a.y_bf16);
    return;
  }
  // this lane's state values (channel c + CPP p of pass p), requested first
  const int c = tid / LPC, sub = tid % LPC;
  const int n0 = sub * VEC;
  vec_t h[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int d = d0 + CPP * p + c;
    if (d < D) h[p] = __builtin_nontemporal_load(
        reinterpret_cast<const vec_t*>(static_cast<TS*>(a.ssm) + ((int64_t)slot * D + d) * N + n0));
  }

  // ---------------------------------------------------------------- phase 1
  // One copy per (conv dtype, io dtype), chosen once: with the element types known every load of
  // the phase is issued before the first conversion waits for one.
  auto phase1 = [&](auto tc, auto ti) {
    typedef decltype(tc) TC;
    typedef decltype(ti) TI;
    for (int ci = tid; ci < CPW; ci += kM1Threads) {
      if (d0 + ci >= D) break;
      const int dc = d0 + ci;
      const int64_t woff = ((int64_t)slot * D + dc) * (W - 1);
      TC* const wp = static_cast<TC*>(a.conv) + woff;
      TC wr[W - 1];
#pragma unroll
      for (int k = 0; k < W - 1; ++k) wr[k] = wp[k];
      const TI ur = static_cast<const TI*>(a.x)[b * a.x_stride + dc];
      const TI dtr = static_cast<const TI*>(a.dt)[b * a.dt_stride + dc];
      const TI zr = static_cast<const TI*>(a.z)[b * a.z_stride + dc];
      float wt[W];
#pragma unroll
      for (int k = 0; k < W; ++k) wt[k] = a.conv_w[(int64_t)dc * W + k];
      const float cb = a.conv_b[dc], dtb = a.dt_bias[dc], dk = a.Dk[dc];
      const float u = to_f32(ur);
      float v = cb + wt[W - 1] * u;
#pragma unroll
      for (int k = 0; k < W - 1; ++k) v += wt[k] * to_f32(wr[k]);
      const float x = silu(v), dl = softplus(to_f32(dtr) + dtb);
      s_dl[ci] = dl * 1.4426950408889634f;   // Delta log2 e: the decay exponent per unit of A
      s_dx[ci] = dl * x;                     // Delta x: the input's weight on B
      s_yx[ci] = dk * x;                     // the skip term D x
      s_g[ci] = silu(to_f32(zr));            // the gate
      // the window keeps raw inputs at the conv dtype: shift the stored words, append the input
#pragma unroll
      for (int k = 0; k < W - 2; ++k) wp[k] = wr[k + 1];
      wp[W - 2] = from_f32<TC>(u);
    }
    for (int n = tid; n < N; n += kM1Threads) {
      s_B[n] = to_f32(static_cast<const TI*>(a.B)[b * a.B_stride + n]);
      s_C[n] = to_f32(static_cast<const TI*>(a.C)[b * a.C_stride + n]);
    }
  };
  if (a.conv_bf16) {
    if (a.io_bf16) phase1(bf16(), bf16());
    else phase1(bf16(), 0.f);
  } else {
    if (a.io_bf16) phase1(0.f, bf16());
    else phase1(0.f, 0.f);
  }
  __syncthreads();

  // ---------------------------------------------------------------- phase 2
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int cc = CPP * p + c, d = d0 + cc;
    float part = 0.f;
    if (d < D) {
      const float dl = s_dl[cc], dx = s_dx[cc];
      const float* Ar = a.A + (int64_t)d * N + n0;
      vec_t o;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float al = __builtin_amdgcn_exp2f(dl * Ar[e]);
        const float hn = al * to_f32(h[p][e]) + dx * s_B[n0 + e];
        part += hn * s_C[n0 + e];
        o[e] = from_f32<TS>(hn);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<vec_t*>(static_cast<TS*>(a.ssm) + ((int64_t)slot * D + d) * N + n0));
    }
#pragma unroll
    for (int m = LPC / 2; m >= 1; m /= 2) part += __shfl_xor(part, m);
    if (d < D && sub == 0) {
      store_any(a.y, b * a.y_stride + d, (part + s_yx[cc]) * s_g[cc], a.y_bf16);
    }
  }
}

template <typename TS, int N>
static hipError_t launch_m1w(const Mamba1Params& p, int W, int batch, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(TS);
  constexpr int CPW = kM1Threads / (N / VEC) * m1_passes<TS, N>();
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
// Three launches: (1) the end state from a zero state and the per-channel sum of Delta of every
// chunk that is not its sequence's last (a last chunk's end state feeds nothing), all at once;
// (2) per (sequence, channel, state index) the pass through the sequence's chunks,
// h <- exp(A sum Delta) h + S_c, writing the state entering each chunk; (3) every chunk again
// from its entering state, with the outputs, the checkpoint states at their tokens and the final
// state.  With one chunk per sequence only launch (3) runs, from the slots' states.  Launches (1)
// and (3) take a 256-thread workgroup per (chunk, block of channels) and walk the chunk in blocks
// of 16 rows: the raw rows of the block are loaded cooperatively (the next block's requested
// while the current one runs), each (row, channel) gets its conv, Delta, Delta x, D x and
// silu(z) once, into LDS, and then the recurrence runs with a channel's state values spread over
// N/4 lanes in fp32 registers.  Rows go in groups of four: each lane keeps one partial h C per
// row, and the channel's lanes share out the four sums (a reduce-scatter over the lane quad), so
// every lane finishes one row's output.
namespace m2 {

constexpr int kM1PV = 4;      // state values per lane
constexpr int kM1G = 4;       // rows per output group
constexpr int kM1TB = 16;     // rows per staged block (a multiple of kM1G)
constexpr int kM1Ring = 32;   // rows of the raw-x ring: a block and the W-1 rows before it

template <typename TI> __device__ __forceinline__ float m1_ld(const void* p, int64_t i) {
  return to_f32(static_cast<const TI*>(p)[i]);
}

// v of the lane whose index differs in bit 0 (bit 1): DPP quad permutes
__device__ __forceinline__ float m1_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float m1_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Sums of the four row partials p[0..3] over a channel's LPC lanes.  LPC >= 4: on return s0 of
// lane `sub` is the sum of row (sub & 3), complete in every lane quad.  LPC == 2: s0 is the sum of
// row (sub & 1) and s1 that of row 2 + (sub & 1).
template <int LPC> __device__ __forceinline__ void m1_group_sums(const float (&p)[kM1G], int sub, float& s0, float& s1) {
  const bool b0 = sub & 1;
  if constexpr (LPC == 2) {
    s0 = (b0 ? p[1] : p[0]) + m1_xor1(b0 ? p[0] : p[1]);
    s1 = (b0 ? p[3] : p[2]) + m1_xor1(b0 ? p[2] : p[3]);
  } else {
    const bool b1 = sub & 2;
    const float q0 = (b1 ? p[2] : p[0]) + m1_xor2(b1 ? p[0] : p[2]);   // row 2 b1
    const float q1 = (b1 ? p[3] : p[1]) + m1_xor2(b1 ? p[1] : p[3]);   // row 2 b1 + 1
    float r = (b0 ? q1 : q0) + m1_xor1(b0 ? q0 : q1);
    if constexpr (LPC >= 8) r += __shfl_xor(r, 4);
    if constexpr (LPC >= 16) r += __shfl_xor(r, 8);
    if constexpr (LPC >= 32) r += __shfl_xor(r, 16);
    if constexpr (LPC >= 64) r += __shfl_xor(r, 32);
    s0 = r;
    s1 = 0.f;
  }
}

// OUT = false: launch (1); OUT = true: launch (3).  TI: the dtype of the x, z, dt, B, C rows.
template <typename TS, typename TI, bool OUT, int N, int W>
__global__ __launch_bounds__(256) void mamba1_chunk_kernel(Mamba1PrefillParams a) {
  constexpr int PV = kM1PV, G = kM1G, TB = kM1TB, R = kM1Ring;
  constexpr int LPC = N / PV;                // recurrence lanes per channel
  constexpr int CPW = 256 / LPC;             // channels per workgroup
  static_assert(LPC >= 2 && TB % G == 0 && TB + W - 1 <= R, "block shape");
  constexpr int RS = 256 / CPW;              // staging: row step of one thread
  constexpr int PP = (TB + RS - 1) / RS;     // staging: (row, channel) pairs per thread
  constexpr int BPT = (TB * N + 255) / 256;  // staging: B (and C) values per thread
  constexpr int NO = OUT ? TB : 1;
  __shared__ float xs[R][CPW];
  __shared__ float s_dl[TB][CPW], s_dx[TB][CPW];
  __shared__ float s_dy[NO][CPW], s_sz[NO][CPW];
  __shared__ __align__(16) float s_B[TB][N];
  __shared__ __align__(16) float s_C[NO][N];

  const int ci = blockIdx.y;
  const M1Chunk ch = a.chunks[ci];
  const M1Seq sq = a.seqs[ch.seq];
  const bool first = ch.tau0 == 0, last = ch.tau0 + ch.len == sq.len;
  if (!OUT && last) return;
  const int tid = threadIdx.x, D = a.D, d0 = blockIdx.x * CPW;

  // staging role: channel pc, rows pr0, pr0 + RS, ... (pr0 is the wave's index when a wave
  // covers whole rows)
  const int pc = tid % CPW;
  const int pr0 = CPW % 64 == 0 ? __builtin_amdgcn_readfirstlane(tid / CPW) : tid / CPW;
  const int pd = d0 + pc;
  const bool pon = pd < D;
  const int pdd = pon ? pd : 0;
  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = a.conv_w[(int64_t)pdd * W + k];
  const float cb = a.conv_b[pdd], bias = a.dt_bias[pdd];
  const float Dd = OUT ? a.Dk[pdd] : 0.f;

  // the W-1 raw inputs before the chunk: earlier rows of the sequence, else the slot's window
  // (launch (1) copies a first chunk's window aside for launch (3), whose last chunk rewrites the
  // slot's window while the first may still be reading it; a chunk that is both reads the slot)
  if (pr0 == 0) {
    float* const w0 = a.Win0 + ((int64_t)ch.seq * D + pdd) * (W - 1);
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
      const int tau = ch.tau0 - (W - 1) + k;
      float v;
      if (tau >= 0) v = m1_ld<TI>(a.x, (int64_t)(sq.t0 + tau) * a.x_stride + pdd);
      else if (OUT && !last) v = w0[k];
      else if (sq.has_init) v = load_any(a.conv, ((int64_t)sq.slot * D + pdd) * (W - 1) + k, a.conv_bf16);
      else v = 0.f;
      xs[k][pc] = v;
      if (!OUT && first && pon) w0[k] = v;
    }
  }

  // recurrence role: channel rc, state values n0 .. n0+PV-1
  const int rc = tid / LPC, sub = tid % LPC;
  const int rd = d0 + rc;
  const bool ron = rd < D;
  const int rdd = ron ? rd : 0;
  const int n0 = sub * PV;
  const float kLog2e = 1.4426950408889634f;
  float A2[PV], h[PV];
#pragma unroll
  for (int e = 0; e < PV; ++e) A2[e] = a.A[(int64_t)rdd * N + n0 + e] * kLog2e;
  if (OUT) {
    if (first && last) {   // a whole sequence: its slot is read and written by this lane alone
      const TS* st = static_cast<const TS*>(a.ssm) + ((int64_t)sq.slot * D + rdd) * N + n0;
#pragma unroll
      for (int e = 0; e < PV; ++e) h[e] = sq.has_init ? to_f32(st[e]) : 0.f;
    } else {
      const float* hin = a.Hin + ((int64_t)ci * D + rdd) * N + n0;
#pragma unroll
      for (int e = 0; e < PV; ++e) h[e] = hin[e];
    }
    // settle these loads here: left in flight they would make the row loop wait for every
    // memory access before each row
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  } else {
#pragma unroll
    for (int e = 0; e < PV; ++e) h[e] = 0.f;
  }
  // state and window after chunk row q (the window's raw rows are in the ring)
  auto store_state = [&](int slot, int q) {
    TS* st = static_cast<TS*>(a.ssm) + ((int64_t)slot * D + rd) * N + n0;
#pragma unroll
    for (int e = 0; e < PV; ++e) st[e] = from_f32<TS>(h[e]);
    if (sub == 0) {
#pragma unroll
      for (int k = 0; k < W - 1; ++k)
        store_any(a.conv, ((int64_t)slot * D + rd) * (W - 1) + k, xs[(q + 1 + k) & (R - 1)][rc], a.conv_bf16);
    }
  };

  float px[PP], pdt[PP], pz[OUT ? PP : 1], pB[BPT], pC[OUT ? BPT : 1];
  auto fetch = [&](int r0, int nb) {
#pragma unroll
    for (int m = 0; m < PP; ++m) {
      const int r = pr0 + m * RS;
      if (r < nb && pon) {
        const int64_t row = ch.t0 + r0 + r;
        px[m] = m1_ld<TI>(static_cast<const TI*>(a.x) + row * a.x_stride, (uint32_t)pd);
        pdt[m] = m1_ld<TI>(static_cast<const TI*>(a.dt) + row * a.dt_stride, (uint32_t)pd);
        if (OUT) pz[m] = m1_ld<TI>(static_cast<const TI*>(a.z) + row * a.z_stride, (uint32_t)pd);
      }
    }
#pragma unroll
    for (int m = 0; m < BPT; ++m) {
      const int i = tid + 256 * m, r = i / N, n = i % N;
      if (r < nb) {
        const int64_t row = ch.t0 + r0 + r;
        pB[m] = m1_ld<TI>(a.B, row * a.B_stride + n);
        if (OUT) pC[m] = m1_ld<TI>(a.C, row * a.C_stride + n);
      }
    }
  };

  float sumd = 0.f;
  fetch(0, ch.len < TB ? ch.len : TB);
  for (int r0 = 0; r0 < ch.len; r0 += TB) {
    const int nb = ch.len - r0 < TB ? ch.len - r0 : TB;
    const int ng = (nb + G - 1) / G * G;   // rows walked: the last group is padded with rows
                                           // that leave the state as it is (Delta = 0, B = 0)
    // stage the block's raw rows (rows past nb are left alone: the ring still holds older rows
    // that the final window may need)
#pragma unroll
    for (int m = 0; m < PP; ++m) {
      const int r = pr0 + m * RS;
      if (r < nb) xs[(r0 + r + W - 1) & (R - 1)][pc] = pon ? px[m] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < BPT; ++m) {
      const int i = tid + 256 * m, r = i / N;
      if (r < ng) {
        s_B[r][i % N] = r < nb ? pB[m] : 0.f;
        if (OUT) s_C[r][i % N] = r < nb ? pC[m] : 0.f;
      }
    }
    __syncthreads();
    // per (row, channel): conv over the ring, Delta, Delta x, D x, silu(z)
#pragma unroll
    for (int m = 0; m < PP; ++m) {
      const int r = pr0 + m * RS;
      if (r < nb) {
        float v = cb;
#pragma unroll
        for (int k = 0; k < W; ++k) v += w[k] * xs[(r0 + r + k) & (R - 1)][pc];
        const float xv = silu(v);
        const float dl = softplus((pon ? pdt[m] : 0.f) + bias);
        s_dl[r][pc] = dl;
        s_dx[r][pc] = dl * xv;
        if (OUT) {
          s_dy[r][pc] = Dd * xv;
          s_sz[r][pc] = silu(pon ? pz[m] : 0.f);
        }
      } else if (r < ng) {
        s_dl[r][pc] = 0.f;
        s_dx[r][pc] = 0.f;
      }
    }
    if (r0 + TB < ch.len) fetch(r0 + TB, ch.len - r0 - TB < TB ? ch.len - r0 - TB : TB);
    // the block's first checkpoint row: row t ends at absolute position p1 + t
    const int64_t p1 = (int64_t)sq.start_pos + ch.tau0 + r0 + 1;
    int tck = TB;   // none
    if (OUT && a.ckpt_interval > 0) {
      const int64_t rem = p1 % a.ckpt_interval;
      const int64_t t0 = rem == 0 ? 0 : a.ckpt_interval - rem;
      if (t0 < nb) tck = (int)t0;
    }
    __syncthreads();
    for (int t = 0; t < ng; t += G) {
      float part[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float dl = s_dl[t + g][rc], dx = s_dx[t + g][rc];
        float Bv[PV];
#pragma unroll
        for (int e = 0; e < PV; ++e) Bv[e] = s_B[t + g][n0 + e];
#pragma unroll
        for (int e = 0; e < PV; ++e) h[e] = __builtin_amdgcn_exp2f(dl * A2[e]) * h[e] + dx * Bv[e];
        if (!OUT) {
          sumd += dl;
        } else {
          part[g] = 0.f;
#pragma unroll
          for (int e = 0; e < PV; ++e) part[g] += h[e] * s_C[t + g][n0 + e];
          if (t + g == tck) {   // a checkpoint row (wave-uniform)
            const int64_t k = (p1 + t + g) / a.ckpt_interval - sq.start_pos / a.ckpt_interval - 1;
            if (ron && k >= 0 && k < sq.nck) {
              const int slot = a.ck[sq.ck0 + k];
              if (slot >= 0 && slot < a.num_slots) store_state(slot, r0 + t + g);
            }
            tck = (int64_t)tck + a.ckpt_interval < nb ? tck + a.ckpt_interval : TB;
          }
        }
      }
      if (OUT) {
        float s0, s1;
        m1_group_sums<LPC>(part, sub, s0, s1);
        // y of row t + tr: the lane's share of the group's outputs
        auto put = [&](int tr, float sum) {
          if (ron && tr < nb)
            store_any(a.y, (int64_t)(ch.t0 + r0 + tr) * a.y_stride + rd, (sum + s_dy[tr][rc]) * s_sz[tr][rc],
                      a.y_bf16);
        };
        if constexpr (LPC == 2) {
          put(t + sub, s0);
          put(t + 2 + sub, s1);
        } else {
          if (sub < 4) put(t + sub, s0);
        }
      }
    }
    __syncthreads();
  }
  if (!ron) return;
  if (OUT) {
    if (last) store_state(sq.slot, ch.len - 1);
  } else {
    float* s = a.S + ((int64_t)ci * D + rd) * N + n0;
#pragma unroll
    for (int e = 0; e < PV; ++e) s[e] = h[e];
    if (sub == 0) a.SD[(int64_t)ci * D + rd] = sumd;
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
  for (int cj = sq.chunk0;; ++cj) {
    a.Hin[(int64_t)cj * DN + i] = h;
    const M1Chunk c = a.chunks[cj];
    if (c.tau0 + c.len == sq.len) break;
    h = __builtin_amdgcn_exp2f(A2 * a.SD[(int64_t)cj * a.D + d]) * h + a.S[(int64_t)cj * DN + i];
  }
}

template <typename TS, typename TI, int N>
static hipError_t launch_m1p_n(const Mamba1PrefillParams& a, int W, hipStream_t s) {
  constexpr int CPW = 256 / (N / kM1PV);
  const dim3 gc((a.D + CPW - 1) / CPW, a.num_chunks), gp((unsigned)(((int64_t)a.D * N + 255) / 256), a.num_seqs);
#define M1P_W(WW)                                                                               \
  if (!a.whole_seqs) {                                                                          \
    hipLaunchKernelGGL((mamba1_chunk_kernel<TS, TI, false, N, WW>), gc, dim3(256), 0, s, a);        \
    hipLaunchKernelGGL((mamba1_pass_kernel<TS>), gp, dim3(256), 0, s, a, N);                    \
  }                                                                                             \
  hipLaunchKernelGGL((mamba1_chunk_kernel<TS, TI, true, N, WW>), gc, dim3(256), 0, s, a);
  switch (W) {
    case 2: M1P_W(2) break;
    case 3: M1P_W(3) break;
    case 4: M1P_W(4) break;
    default: return hipErrorInvalidValue;
  }
#undef M1P_W
  return hipGetLastError();
}

template <typename TS, typename TI>
static hipError_t launch_m1p(const Mamba1PrefillParams& a, int N, int W, hipStream_t s) {
  switch (N) {
    case 8: return launch_m1p_n<TS, TI, 8>(a, W, s);
    case 16: return launch_m1p_n<TS, TI, 16>(a, W, s);
    case 32: return launch_m1p_n<TS, TI, 32>(a, W, s);
    case 64: return launch_m1p_n<TS, TI, 64>(a, W, s);
    case 128: return launch_m1p_n<TS, TI, 128>(a, W, s);
    case 256: return launch_m1p_n<TS, TI, 256>(a, W, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mamba1_prefill(const Mamba1PrefillParams& a, int N, int W, hipStream_t s) {
  if (a.num_chunks == 0) return hipSuccess;
  if (a.ssm_bf16) return a.io_bf16 ? launch_m1p<bf16, bf16>(a, N, W, s) : launch_m1p<bf16, float>(a, N, W, s);
  return a.io_bf16 ? launch_m1p<float, bf16>(a, N, W, s) : launch_m1p<float, float>(a, N, W, s);
}

}  // namespace m2
