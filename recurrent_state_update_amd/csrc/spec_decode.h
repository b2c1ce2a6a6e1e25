// Internal launch interface between the C ABI (api.cpp) and the gfx950 multi-token decode kernel.
#pragma once
#include "kernels.h"

namespace m2 {

constexpr int kMaxDecodeTokens = 8;   // tokens per sequence in one multi-token decode call

// Several decode tokens per sequence: rows b*K + t of x, B, C, z, dt and y; the state and window
// of slot d.slots[b] seed the row, and the state and window after token t go to slot
// slots_out[b*K + t] (skipped when out of range).  d.slots[b] out of range: padding row.
struct MultiDecodeParams {
  DecodeParams d;
  const int32_t* slots_out;
  int K;
};
hipError_t launch_decode_multi(const MultiDecodeParams& p, int N, int W, int batch, hipStream_t s);
// LDS of one multi-token workgroup: per token the group's activations, Delta, alpha and gate rows,
// and the output slots (at most kMaxLdsBytes).
inline size_t multi_decode_lds_bytes(int hpg, int P, int N, int K) {
  return sizeof(float) * ((size_t)K * (2 * (size_t)hpg * P + 2 * (size_t)N) + 2 * (size_t)K * hpg) +
         sizeof(int) * (size_t)K;
}

}  // namespace m2
