// int8 checkpoint store, gfx950: cached states kept apart from the active pool,
// the temporal state quantized once when stored and dequantized once into a
// fresh slot on a hit ("Hybrid SSM / Mamba models and non-KV state",
// mlinterviewnotes.com ch. 7.3, the SGLang passage on compressed checkpoints).
//
// Codes are symmetric int8 with one fp32 scale per (head, d_state index n),
// taken over the head_dim rows of that column (the k-channel: B is the key the
// state is written with).  All decisions are fp32:
//   amax = max_p |h[p][n]|,  scale = amax / 127,  inv = 127 / amax (both
//   correctly rounded), code = clamp(rint(h * inv), -127, 127); zero column:
//   scale 0, codes 0.  Restore: h = code * scale in fp32, rounded (RNE) to the
//   pool's dtype.  The conv window is copied in its own dtype.
//
// One launch per direction.  Workgroups [0, H) of a (pair, layer) each move one
// head; the rest copy the conv window, 4 KiB per workgroup.  A head's thread
// owns 8 consecutive columns and every (256 / (N/8))-th row; put keeps up to 8
// such rows in registers while the column maxima are reduced through LDS (a
// taller head reads its rows again, from cache), then quantizes them.
#include "device_common.h"
#include "int8_store.h"

namespace m2 {

constexpr int kQThreads = 256;
typedef unsigned short u16v8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int uniform_load_i32(const int32_t* p) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  return *(const cint*)p;
}

// 8 consecutive state values of one row as fp32.
__device__ __forceinline__ void load8(const char* base, bool bf, int64_t i, float (&v)[8]) {
  if (bf) {
    const u16v8 r = *reinterpret_cast<const u16v8*>(reinterpret_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __uint_as_float((uint32_t)r[e] << 16);
  } else {
    const float* p = reinterpret_cast<const float*>(base) + i;
    const floatx4 a = *reinterpret_cast<const floatx4*>(p), b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
  }
}

// Conv-window workgroups: copy 4 KiB pieces of one slot-layer's window.
__device__ __forceinline__ void conv_piece(const char* src, char* dst, uint64_t bytes, uint64_t g) {
  const uint64_t i = g * kQThreads + threadIdx.x;
  if (i < bytes / 16)
    reinterpret_cast<floatx4*>(dst)[i] = reinterpret_cast<const floatx4*>(src)[i];
}

// Rows a thread keeps in registers between the two passes; taller heads read their rows again.
constexpr int kQRows = 8;

template <bool BF>
__device__ __forceinline__ void load8t(const char* base, int64_t i, float (&v)[8]) {
  load8(base, BF, i, v);
}

template <bool BF>
__global__ __launch_bounds__(kQThreads) void int8_put_kernel(Int8StoreArgs a) {
  const int pair = blockIdx.y, layer = a.l0 + blockIdx.z;
  const int s = uniform_load_i32(a.slots + pair), e = uniform_load_i32(a.entries + pair);
  if (s < 0 || s >= a.num_slots || e < 0 || e >= a.num_entries) return;
  const int H = a.H, P = a.P, N = a.N;
  const int64_t pl = (int64_t)layer * a.num_slots + s;     // pool (layer, slot)
  const int64_t el = (int64_t)e * a.num_layers + layer;    // store (entry, layer)
  if ((int)blockIdx.x >= H) {
    conv_piece(a.conv + pl * a.conv_bytes, a.store_conv + el * a.conv_bytes, a.conv_bytes, blockIdx.x - H);
    return;
  }
  __shared__ float red[2048];       // [row group][N] partial maxima (row groups * N <= 2048)
  __shared__ float sinv[2048];      // per column: 127 / amax
  const int h = blockIdx.x;
  const int64_t PN = (int64_t)P * N;
  const char* src = a.ssm + ((pl * H + h) * PN) * (BF ? 2 : 4);
  int8_t* codes = a.codes + (el * H + h) * PN;
  float* scales = a.scales + (el * H + h) * N;
  const int cgs = N / 8, rstep = kQThreads / cgs;
  const int cg = threadIdx.x % cgs, r0 = threadIdx.x / cgs;
  const bool active = r0 < rstep;
  const bool held = P <= rstep * kQRows;   // every row of this thread fits in registers
  float v[kQRows][8];
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (active) {
    if (held) {
#pragma unroll
      for (int i = 0; i < kQRows; ++i) {   // all loads first, then the maxima
        const int r = r0 + i * rstep;
        if (r < P) load8t<BF>(src, (int64_t)r * N + 8 * cg, v[i]);
      }
#pragma unroll
      for (int i = 0; i < kQRows; ++i) {
        if (r0 + i * rstep < P) {
#pragma unroll
          for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], fabsf(v[i][k]));
        }
      }
    } else {
      for (int r = r0; r < P; r += rstep) {
        float t[8];
        load8t<BF>(src, (int64_t)r * N + 8 * cg, t);
#pragma unroll
        for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], fabsf(t[k]));
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) red[r0 * N + 8 * cg + k] = m[k];
  }
  __syncthreads();
  for (int n = threadIdx.x; n < N; n += kQThreads) {
    float amax = 0.f;
    for (int g = 0; g < rstep; ++g) amax = fmaxf(amax, red[g * N + n]);
    scales[n] = amax / 127.0f;
    sinv[n] = amax > 0.f ? 127.0f / amax : 0.f;
  }
  __syncthreads();
  if (!active) return;
  float inv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) inv[k] = sinv[8 * cg + k];
  auto store_row = [&](int r, const float (&t)[8]) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float q = fminf(fmaxf(rintf(t[k] * inv[k]), -127.f), 127.f);
      const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)q;
      if (k < 4) lo |= b << (8 * k);
      else hi |= b << (8 * (k - 4));
    }
    *reinterpret_cast<uint2*>(codes + (int64_t)r * N + 8 * cg) = make_uint2(lo, hi);
  };
  if (held) {
#pragma unroll
    for (int i = 0; i < kQRows; ++i) {
      const int r = r0 + i * rstep;
      if (r < P) store_row(r, v[i]);
    }
  } else {
    for (int r = r0; r < P; r += rstep) {
      float t[8];
      load8t<BF>(src, (int64_t)r * N + 8 * cg, t);
      store_row(r, t);
    }
  }
}

template <bool BF>
__global__ __launch_bounds__(kQThreads) void int8_get_kernel(Int8StoreArgs a) {
  const int pair = blockIdx.y, layer = a.l0 + blockIdx.z;
  const int e = uniform_load_i32(a.entries + pair), s = uniform_load_i32(a.slots + pair);
  if (s < 0 || s >= a.num_slots || e < 0 || e >= a.num_entries) return;
  const int H = a.H, P = a.P, N = a.N;
  const int64_t pl = (int64_t)layer * a.num_slots + s;
  const int64_t el = (int64_t)e * a.num_layers + layer;
  if ((int)blockIdx.x >= H) {
    conv_piece(a.store_conv + el * a.conv_bytes, a.conv + pl * a.conv_bytes, a.conv_bytes, blockIdx.x - H);
    return;
  }
  const int h = blockIdx.x;
  const int64_t PN = (int64_t)P * N;
  char* dst = a.ssm + ((pl * H + h) * PN) * (BF ? 2 : 4);
  const int8_t* codes = a.codes + (el * H + h) * PN;
  const float* scales = a.scales + (el * H + h) * N;
  const int cgs = N / 8, rstep = kQThreads / cgs;
  const int cg = threadIdx.x % cgs, r0 = threadIdx.x / cgs;
  if (r0 >= rstep) return;
  const floatx4 s0 = *reinterpret_cast<const floatx4*>(scales + 8 * cg);
  const floatx4 s1 = *reinterpret_cast<const floatx4*>(scales + 8 * cg + 4);
  const float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  auto restore_row = [&](int r, uint2 q) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t w = k < 4 ? q.x : q.y;
      v[k] = (float)(int8_t)(uint8_t)(w >> (8 * (k & 3))) * sc[k];
    }
    const int64_t i = (int64_t)r * N + 8 * cg;
    if (BF) {
      u16v8 o;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = __builtin_bit_cast(unsigned short, from_f32<bf16>(v[k]));
      *reinterpret_cast<u16v8*>(reinterpret_cast<uint16_t*>(dst) + i) = o;
    } else {
      float* d = reinterpret_cast<float*>(dst) + i;
      *reinterpret_cast<floatx4*>(d) = floatx4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<floatx4*>(d + 4) = floatx4{v[4], v[5], v[6], v[7]};
    }
  };
  // rows in batches of kQRows, every batch's loads issued before its stores
  for (int rb = r0; rb < P; rb += rstep * kQRows) {
    uint2 q[kQRows];
#pragma unroll
    for (int i = 0; i < kQRows; ++i) {
      const int r = rb + i * rstep;
      if (r < P) q[i] = *reinterpret_cast<const uint2*>(codes + (int64_t)r * N + 8 * cg);
    }
#pragma unroll
    for (int i = 0; i < kQRows; ++i) {
      const int r = rb + i * rstep;
      if (r < P) restore_row(r, q[i]);
    }
  }
}

static dim3 int8_grid(const Int8StoreArgs& a, int n, int nl) {
  const uint64_t conv_groups = (a.conv_bytes / 16 + kQThreads - 1) / kQThreads;
  return dim3((unsigned)(a.H + conv_groups), (unsigned)n, (unsigned)nl);
}

hipError_t launch_int8_put(const Int8StoreArgs& a, int n, int nl, hipStream_t s) {
  if (n == 0 || nl == 0) return hipSuccess;
  if (a.N % 8 != 0 || a.N / 8 > kQThreads || (kQThreads / (a.N / 8)) * a.N > 2048) return hipErrorInvalidValue;
  if (a.ssm_bf16) hipLaunchKernelGGL(int8_put_kernel<true>, int8_grid(a, n, nl), dim3(kQThreads), 0, s, a);
  else hipLaunchKernelGGL(int8_put_kernel<false>, int8_grid(a, n, nl), dim3(kQThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_int8_get(const Int8StoreArgs& a, int n, int nl, hipStream_t s) {
  if (n == 0 || nl == 0) return hipSuccess;
  if (a.N % 8 != 0 || a.N / 8 > kQThreads) return hipErrorInvalidValue;
  if (a.ssm_bf16) hipLaunchKernelGGL(int8_get_kernel<true>, int8_grid(a, n, nl), dim3(kQThreads), 0, s, a);
  else hipLaunchKernelGGL(int8_get_kernel<false>, int8_grid(a, n, nl), dim3(kQThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace m2
