// Bit-exact slot-to-slot copy of a pool state object, gfx950.
//
// A cached state is copied into a fresh slot rather than shared, because the
// recurrence overwrites its slot in place ("Hybrid SSM / Mamba models and
// non-KV state", mlinterviewnotes.com ch. 7.3, SGLang checkpoint passage).
// Each workgroup moves a contiguous 32 KiB span of one (layer, pair) with
// 16-byte accesses, eight in flight per lane.
#include "device_common.h"
#include "kernels.h"

namespace m2 {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;
constexpr uint64_t kCopySpan = (uint64_t)kCopyThreads * kCopyUnroll * 16;

__global__ __launch_bounds__(kCopyThreads) void slot_copy_kernel(char* base, uint64_t bytes_per_slot,
                                                                 uint64_t layer_stride, int l0,
                                                                 int num_slots, const int32_t* src,
                                                                 const int32_t* dst) {
  const int pair = blockIdx.y;
  const int layer = l0 + blockIdx.z;
  const int s = src[pair];
  const int d = dst[pair];
  if (s < 0 || s >= num_slots || d < 0 || d >= num_slots || s == d) return;
  const uint64_t off = (uint64_t)blockIdx.x * kCopySpan;
  const uint64_t n16 = bytes_per_slot / 16;
  const floatx4* in = reinterpret_cast<const floatx4*>(base + layer * layer_stride + s * bytes_per_slot + off);
  floatx4* out = reinterpret_cast<floatx4*>(base + layer * layer_stride + d * bytes_per_slot + off);
  const uint64_t first = off / 16;
  floatx4 v[kCopyUnroll];
#pragma unroll
  for (int k = 0; k < kCopyUnroll; ++k) {
    const uint64_t i = (uint64_t)k * kCopyThreads + threadIdx.x;
    if (first + i < n16) v[k] = in[i];
  }
#pragma unroll
  for (int k = 0; k < kCopyUnroll; ++k) {
    const uint64_t i = (uint64_t)k * kCopyThreads + threadIdx.x;
    if (first + i < n16) out[i] = v[k];
  }
}

hipError_t launch_slot_copy(void* base, uint64_t bytes_per_slot, uint64_t layer_stride, int l0, int nl,
                            int num_slots, int n, const int32_t* src, const int32_t* dst, hipStream_t s) {
  if (n == 0 || nl == 0) return hipSuccess;
  const dim3 grid((unsigned)((bytes_per_slot + kCopySpan - 1) / kCopySpan), n, nl);
  hipLaunchKernelGGL(slot_copy_kernel, grid, dim3(kCopyThreads), 0, s, static_cast<char*>(base),
                     bytes_per_slot, layer_stride, l0, num_slots, src, dst);
  return hipGetLastError();
}

}  // namespace m2
