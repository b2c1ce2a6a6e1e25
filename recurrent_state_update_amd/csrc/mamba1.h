// Internal launch interface between the C ABI (api.cpp) and the gfx950 Mamba1 decode kernel.
#pragma once
#include "kernels.h"

namespace m2 {

struct Mamba1Params {
  void* ssm;            // [num_slots][D][N] of one layer
  void* conv;           // [num_slots][D][W-1] of one layer
  int num_slots;
  int ssm_bf16, conv_bf16, io_bf16, y_bf16;
  int D;
  const int32_t* slots;
  const void* x;
  const void* B;
  const void* C;
  const void* z;
  const void* dt;
  int64_t x_stride, B_stride, C_stride, z_stride, dt_stride;
  void* y;
  int64_t y_stride;
  const float* A;       // [D][N]
  const float* Dk;      // [D]
  const float* dt_bias;
  const float* conv_w;  // [D][W]
  const float* conv_b;
};
hipError_t launch_mamba1_decode(const Mamba1Params& p, int N, int W, int batch, hipStream_t s);
bool mamba1_supported(int N, int W);

}  // namespace m2
