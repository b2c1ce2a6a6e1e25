// Internal launch interface between the C ABI (api.cpp) and the gfx950 chunked-prefill kernels.
#pragma once
#include "kernels.h"

namespace m2 {

// Chunked prefill.  Host-built tables live at the start of the workspace.
struct SeqEntry {     // one per sequence
  int32_t t0, len, slot, has_init;  // packed start row, rows, final slot, seed from slot
  int32_t chunk0, nchunk, pad0, pad1;
};
struct ChunkEntry {   // one per chunk
  int32_t seq, t0, len, tau0;       // packed start row, rows in chunk, offset inside the sequence
  int32_t ckpt_slot, is_last, pad0, pad1;
};

// Row tiles (16 tokens) of a chunk of at most 256 tokens, and the (row tile, 32-token K-step)
// pairs on or below the diagonal whose C B^T blocks the output product needs: row tile rt takes
// K-steps 0 .. rt/2, so there are 72 pairs; pair (rt, k) is stored at index pair_index(rt, k).
constexpr int kMaxRowTiles = 16;
constexpr int kGPairs = 72;
__host__ __device__ constexpr int pair_index(int rt, int k) {
  return (rt & 1) ? ((rt >> 1) + 1) * ((rt >> 1) + 1) + k : (rt >> 1) * ((rt >> 1) + 1) + k;
}

struct PrefillParams {
  void* ssm;
  void* conv;
  int ssm_bf16, conv_bf16, io_bf16, y_bf16;
  int zy_vec;          // z and y allow vector access of up to 8 elements (aligned bases and row pitches)
  LayerShape sh;
  int Q;               // chunk size (multiple of 16, at most 256)
  int QC;              // token capacity of a chunk's operand rows: Q rounded up to 32
  int nparts;          // head_dim parts per head in the walk (head_dim / part width)
  int num_seqs, num_chunks, total_tokens;
  const SeqEntry* seqs;        // the tables, packed in this order at the start of the workspace
  const ChunkEntry* chunks;
  int tab_chunks;              // byte offset of the chunk table from the sequence table
  int tab_inline;              // > 0: the tables (this many bytes) ride in the first launch's arguments
                               // and that launch writes them to the workspace; 0: already there
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
  // workspace arrays, per chunk and group: the post-conv B and C rows as bf16 operand planes (one
  // plane, or hi and lo planes for fp32-faithful products) in the order the output and state
  // products read them, and the C B^T blocks of the causal pairs
  float* delta;          // [H][T] Delta = softplus(dt + dt_bias)
  float* dA;             // [H][T] chunk-local inclusive cumsum of Delta*A
  uint16_t* Cf;          // [planes][chunks][G][QC][NP]  C rows, d_state permuted inside 32-blocks
  uint16_t* Btf;         // [planes][chunks][G][N][QC]   B transposed, tokens permuted inside 32-blocks
  void* Gf;              // [chunks][G][kGPairs][64 lanes][8]: bf16 with bf16 state, fp32 with fp32 state
  int64_t Cf_plane, Btf_plane;   // elements per plane
};
// Tables of up to kInlineTableBytes travel inside the first launch's kernel arguments: its
// workgroups read them from there and one extra workgroup writes them to the workspace for the
// later launch, so a call needs no host-to-device copy.
constexpr int kInlineTableBytes = 3072;
struct alignas(16) InlineTables {
  int32_t w[kInlineTableBytes / 4];
};
struct BcArgs {   // the first launch's one kernel argument
  PrefillParams p;
  InlineTables t;
};

// `inl` holds the packed tables when p.tab_inline > 0 (else it may be NULL).
hipError_t launch_prefill(const PrefillParams& p, const InlineTables* inl, hipStream_t s);
bool prefill_supported(int P, int N, int W);
// head_dim part width of the walk for head_dim P: 32 channels with a bf16 state, 16 with an fp32
// state (whose fp32-faithful operands take twice the registers)
inline int prefill_part(int P, bool fp32_state) { return fp32_state || P < 32 ? 16 : 32; }

}  // namespace m2
