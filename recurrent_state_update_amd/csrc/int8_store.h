// Internal launch interface between the C ABI (api.cpp) and the gfx950 int8 checkpoint-store kernels.
#pragma once
#include "kernels.h"

namespace m2 {

// int8 checkpoint store (int8_store.hip).  Pool objects at layer 0 of the pool; the store holds
// codes int8 [E][L][H][P][N], scales fp32 [E][L][H][N], conv windows [E][L][Cd][W-1] in the
// pool's conv dtype.  Pairs (slots[i], entries[i]) with an index out of range are skipped.
struct Int8StoreArgs {
  char* ssm;
  char* conv;
  int8_t* codes;
  float* scales;
  char* store_conv;
  uint64_t conv_bytes;   // one slot-layer's conv window (a multiple of 16)
  int H, P, N, ssm_bf16;
  int num_layers, num_slots, num_entries, l0;
  const int32_t* slots;
  const int32_t* entries;
};
hipError_t launch_int8_put(const Int8StoreArgs& a, int n, int nl, hipStream_t s);   // pool -> store
hipError_t launch_int8_get(const Int8StoreArgs& a, int n, int nl, hipStream_t s);   // store -> pool

}  // namespace m2
