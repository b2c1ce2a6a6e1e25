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

namespace m2 {

// Mamba1 prefill over packed sequences, in chunks of Q tokens from each sequence's first row.
struct M1Seq {      // one per sequence
  int32_t t0, len, slot, has_init, start_pos, ck0, nck, chunk0;
};
struct M1Chunk {    // one per chunk
  int32_t seq, t0, len, tau0;   // packed start row, rows, offset inside the sequence
};
struct Mamba1PrefillParams {
  void* ssm;            // [num_slots][D][N] of one layer
  void* conv;           // [num_slots][D][W-1] of one layer
  int num_slots;
  int ssm_bf16, conv_bf16, io_bf16, y_bf16;
  int D;
  const void* x;
  const void* B;
  const void* C;
  const void* z;
  const void* dt;
  int64_t x_stride, B_stride, C_stride, z_stride, dt_stride;
  void* y;
  int64_t y_stride;
  const float* A;
  const float* Dk;
  const float* dt_bias;
  const float* conv_w;
  const float* conv_b;
  int num_seqs, num_chunks, ckpt_interval;
  int whole_seqs;           // every chunk is a whole sequence: launches (1) and (2) are skipped
  const M1Seq* seqs;        // workspace tables
  const M1Chunk* chunks;
  const int32_t* ck;        // checkpoint slots, sequence s at ck[seqs[s].ck0 ...]
  float* S;                 // [chunks][D][N] each chunk's end state from a zero state
  float* SD;                // [chunks][D] each chunk's sum of Delta per channel
  float* Hin;               // [chunks][D][N] the state entering each chunk
  float* Win0;              // [seqs][D][W-1] the initial window of each sequence of several chunks,
                            // copied by launch (1) for launch (3), whose last chunk rewrites the slot
};
hipError_t launch_mamba1_prefill(const Mamba1PrefillParams& p, int N, int W, hipStream_t s);

}  // namespace m2
