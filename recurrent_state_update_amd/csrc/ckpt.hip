// Bit-exact slot-to-slot copy of both pool state objects, gfx950; and the launch that carries
// host-built tables to device memory inside its own kernel arguments.
//
// A kept state needs a slot of its own: the live slot is updated in place by the next token, so
// the two cannot share storage ("Hybrid SSM / Mamba models and non-KV state",
// mlinterviewnotes.com ch. 7.3, SGLang checkpoint passage).
// One launch covers both objects: workgroups [0, groups of the SSM state) copy
// the SSM state, the rest the conv window, of one (pair, layer) each.  Each lane
// moves one 16-byte piece with a non-temporal load and store (the copy is
// streamed once and should not evict what the caches hold), so a workgroup
// covers 8 KiB.  Measured on 256 pairs of bf16 Nemotron-H layer states: many
// small workgroups stream fastest (8 KiB per 512-thread workgroup 6.33 TB/s;
// 32 KiB 5.73; 128 KiB with the next span's loads issued before the current
// span's stores 5.26).
#include <cstddef>
#include <cstring>

#include "device_common.h"
#include "kernels.h"

namespace m2 {

constexpr int kCopyThreads = 512;
constexpr uint64_t kCopyGroup = kCopyThreads;   // 16-byte pieces per workgroup

struct CopyObject {
  char* base;
  uint64_t bytes_per_slot;   // a multiple of 16
  uint64_t layer_stride;
  uint32_t groups;           // workgroups per (pair, layer)
};

// A wave-uniform int32 read through the constant address space (a scalar load).
__device__ __forceinline__ int uniform_i32(const int32_t* p) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  return *(const cint*)p;
}

__global__ __launch_bounds__(kCopyThreads) void slot_copy_kernel(CopyObject o0, CopyObject o1, int l0,
                                                                 int num_slots, const int32_t* src,
                                                                 const int32_t* dst) {
  const int pair = blockIdx.y;
  const int layer = l0 + blockIdx.z;
  const int s = uniform_i32(src + pair);
  const int d = uniform_i32(dst + pair);
  if (s < 0 || s >= num_slots || d < 0 || d >= num_slots || s == d) return;
  const bool first = blockIdx.x < o0.groups;
  const CopyObject& o = first ? o0 : o1;
  const uint64_t g = first ? blockIdx.x : blockIdx.x - o0.groups;
  const uint64_t n16 = o.bytes_per_slot / 16;
  char* lbase = o.base + (uint64_t)layer * o.layer_stride;
  const floatx4* in = reinterpret_cast<const floatx4*>(lbase + (uint64_t)s * o.bytes_per_slot);
  floatx4* out = reinterpret_cast<floatx4*>(lbase + (uint64_t)d * o.bytes_per_slot);
  const uint64_t i = g * kCopyGroup + threadIdx.x;
  if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(in + i), out + i);
}

hipError_t launch_slot_copy(void* ssm_base, uint64_t ssm_bytes_per_slot, void* conv_base,
                            uint64_t conv_bytes_per_slot, uint64_t num_slots, int l0, int nl, int n,
                            const int32_t* src, const int32_t* dst, hipStream_t s) {
  if (n == 0 || nl == 0) return hipSuccess;
  auto object = [&](void* base, uint64_t bytes) {
    CopyObject o;
    o.base = static_cast<char*>(base);
    o.bytes_per_slot = bytes;
    o.layer_stride = num_slots * bytes;
    o.groups = (uint32_t)((bytes / 16 + kCopyGroup - 1) / kCopyGroup);
    return o;
  };
  const CopyObject o0 = object(ssm_base, ssm_bytes_per_slot), o1 = object(conv_base, conv_bytes_per_slot);
  const dim3 grid(o0.groups + o1.groups, (unsigned)n, (unsigned)nl);
  hipLaunchKernelGGL(slot_copy_kernel, grid, dim3(kCopyThreads), 0, s, o0, o1, l0, (int)num_slots, src, dst);
  return hipGetLastError();
}

// ------------------------------------------------------------------ tables through kernel arguments
// Host-built launch tables reach device memory without a host-to-device copy: each launch carries
// up to kUploadBytes of them in its kernel arguments and writes them to dst.  No pinned host
// buffer, no allocation and no host wait are involved, and the launches order with the rest of
// the work on the stream.
constexpr int kUploadBytes = 3072;
struct alignas(16) UploadArgs {
  unsigned char* dst;
  int32_t bytes;   // a multiple of 16, at most kUploadBytes
  int32_t pad[1];
  unsigned char data[kUploadBytes];
};

__global__ __launch_bounds__(256) void table_upload_kernel(UploadArgs a) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) i32x4 kquad;
  kquad* src = reinterpret_cast<kquad*>((const __attribute__((address_space(4))) unsigned char*)
                                            __builtin_amdgcn_kernarg_segment_ptr() + offsetof(UploadArgs, data));
  i32x4* dst = reinterpret_cast<i32x4*>(a.dst);
  for (int i = threadIdx.x; i < a.bytes / 16; i += blockDim.x) dst[i] = src[i];
}

hipError_t launch_table_upload(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes % 16 != 0) return hipErrorInvalidValue;
  UploadArgs a;
  for (size_t off = 0; off < bytes; off += kUploadBytes) {
    const size_t n = bytes - off < (size_t)kUploadBytes ? bytes - off : (size_t)kUploadBytes;
    a.dst = static_cast<unsigned char*>(dst) + off;
    a.bytes = (int32_t)n;
    a.pad[0] = 0;
    memcpy(a.data, static_cast<const unsigned char*>(src) + off, n);
    hipLaunchKernelGGL(table_upload_kernel, dim3(1), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace m2
