// Internal launch interface between the C ABI (api.cpp) and the gfx950 decode and
// slot-copy kernels; the prefill has its own (prefill.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

struct LayerShape {
  int H, P, N, G, W;  // heads, head_dim, d_state, n_groups, conv kernel
  int I, Cd;          // H*P, H*P + 2*G*N
};

// Fused decode step.  ssm/conv point at the layer's first slot.
struct DecodeParams {
  void* ssm;
  void* conv;
  int num_slots;
  int ssm_bf16, conv_bf16, io_bf16, y_bf16;
  int H, P, G, I;
  const int32_t* slots;
  const void* x;
  const void* B;
  const void* C;
  const void* z;
  const void* dt;
  int64_t x_stride, B_stride, C_stride, z_stride, dt_stride;
  void* y;
  int64_t y_stride;
  const float* A;
  const float* D;
  const float* dt_bias;
  const float* conv_w;
  const float* conv_b;
};
hipError_t launch_decode(const DecodeParams& p, int N, int W, int batch, hipStream_t s);
bool decode_supported(int ssm_bf16, int N, int W);
// LDS of one decode workgroup: its group's x and gate rows, B, C, Delta and alpha (fp32).  Up to
// kMaxLdsBytes per workgroup on gfx950 (above 64 KiB the launch raises the kernel's limit).
constexpr size_t kMaxLdsBytes = 160 * 1024;
inline size_t decode_lds_bytes(int hpg, int P, int N) {
  return sizeof(float) * (2 * (size_t)hpg * P + 2 * (size_t)N + 2 * (size_t)hpg);
}

// Slot-to-slot copy of both state objects in one launch: for each object, bytes_per_slot bytes at
// base + layer*num_slots*bytes_per_slot + slot*bytes_per_slot, for layers [l0, l0+nl).  Byte
// counts per slot are multiples of 16.
hipError_t launch_slot_copy(void* ssm_base, uint64_t ssm_bytes_per_slot, void* conv_base,
                            uint64_t conv_bytes_per_slot, uint64_t num_slots, int l0, int nl, int n,
                            const int32_t* src, const int32_t* dst, hipStream_t s);

// Copy `bytes` (a multiple of 16) of host data to device memory at dst, ordered on stream s, by
// kernel launches that carry the data in their arguments (no host-to-device copy, no pinned
// buffer, no host wait).
hipError_t launch_table_upload(void* dst, const void* src, size_t bytes, hipStream_t s);

// The prefill scratch of the entry point that allocates nothing: a file-scope device array of
// kNoAllocScratchBytes per GPU.  *ptr receives its device address on the current device (looked
// up once per device).
constexpr uint64_t kNoAllocScratchBytes = 64ull << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace m2
