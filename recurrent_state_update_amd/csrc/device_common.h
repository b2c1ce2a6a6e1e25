// Device helpers shared by the gfx950 kernels: dtype conversion, 16-byte
// vector access, the elementwise functions of the Mamba2 layer, and the
// bf16 MFMA tile product.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

typedef __bf16 bf16;
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ dtypes
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// Load one element of a tensor whose dtype is only known at run time
// (io tensors: 0 = fp32, 1 = bf16).  The branch is uniform across a launch.
__device__ __forceinline__ float load_any(const void* p, int64_t i, int is_bf16) {
  return is_bf16 ? static_cast<float>(static_cast<const bf16*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void store_any(void* p, int64_t i, float v, int is_bf16) {
  if (is_bf16) static_cast<bf16*>(p)[i] = from_f32<bf16>(v);
  else static_cast<float*>(p)[i] = v;
}

// Eight consecutive elements of an io tensor -> fp32 (16-byte aligned rows).
__device__ __forceinline__ void load8_any(const void* p, int64_t i, int is_bf16, float (&o)[8]) {
  if (is_bf16) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p) + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<float>(v[e]);
  } else {
    const floatx4 a = *reinterpret_cast<const floatx4*>(static_cast<const float*>(p) + i);
    const floatx4 b = *reinterpret_cast<const floatx4*>(static_cast<const float*>(p) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[e + 4] = b[e]; }
  }
}

// ------------------------------------------------------------------ math
// SiLU(v) = v / (1 + e^-v) with the hardware reciprocal (about 1 ulp) instead of an IEEE divide.
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// log(1 + e^v) from the hardware exp2 and log2.  Above 20 the value is v to fp32 resolution
// (the correction log1p(e^-v) < 2.1e-9); below, with e = e^v and u = 1 + e rounded,
// log(u) e / (u - 1) cancels the rounding of u (Goldberg's log1p identity), and is e itself
// when u rounds to 1.
__device__ __forceinline__ float softplus(float v) {
  if (v > 20.f) return v;
  const float e = __builtin_amdgcn_exp2f(v * 1.4426950408889634f);
  const float u = 1.f + e;
  const float um1 = u - 1.f;
  return um1 == 0.f ? e : __builtin_amdgcn_logf(u) * 0.6931471805599453f * e * __builtin_amdgcn_rcpf(um1);
}

// ------------------------------------------------------------------ MFMA
// 16x16x32 bf16 tile product on gfx950, fp32 accumulate.  For both operands,
// lane l holds 8 values of row/column (l % 16) at the K positions
//   k(q, e) = (e / 4) * 16 + 4 * q + (e % 4),   q = l / 16,
// the same map for A and B, so the contraction pairs them correctly.  The
// accumulator lane l holds D[4 * q + r][l % 16], r = 0..3.
__device__ __forceinline__ int kmap(int q, int e) { return (e >> 2) * 16 + 4 * q + (e & 3); }

__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// An operand fragment as bf16 (hi) plus, for fp32-faithful products, the
// bf16 rounding of the residual (lo): v ~= hi + lo to about 2^-17 relative.
template <bool SPLIT> struct Frag {
  bf16x8 hi;
  bf16x8 lo;
};

template <bool SPLIT> __device__ __forceinline__ Frag<SPLIT> make_frag(const float (&v)[8]) {
  Frag<SPLIT> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f.hi[e] = from_f32<bf16>(v[e]);
    if (SPLIT) f.lo[e] = from_f32<bf16>(v[e] - static_cast<float>(f.hi[e]));
  }
  return f;
}

// acc += a * b: one bf16 product, or hi*hi + hi*lo + lo*hi for SPLIT
// (the dropped lo*lo term is below 2^-16 of the product).
template <bool SPLIT>
__device__ __forceinline__ floatx4 mma(const Frag<SPLIT>& a, const Frag<SPLIT>& b, floatx4 acc) {
  if (SPLIT) {
    acc = mfma_bf16(a.lo, b.hi, acc);
    acc = mfma_bf16(a.hi, b.lo, acc);
  }
  return mfma_bf16(a.hi, b.hi, acc);
}
// The same three products of hi/lo operands, the high-order one into `hi` and the two low-order
// ones into `lo` (two independent accumulation chains; the caller adds them).
__device__ __forceinline__ void mma_split2(const Frag<true>& a, const Frag<true>& b, floatx4& hi, floatx4& lo) {
  lo = mfma_bf16(a.lo, b.hi, lo);
  hi = mfma_bf16(a.hi, b.hi, hi);
  lo = mfma_bf16(a.hi, b.lo, lo);
}

}  // namespace m2
