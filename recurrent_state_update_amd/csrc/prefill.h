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
struct WindowEntry {  // one checkpoint conv-window write: window after `tau` rows of sequence `seq` -> slot
  int32_t seq, tau, slot, pad;
};

constexpr int kPB = 64;   // tokens per block of the transposed operand planes

struct PrefillParams {
  void* ssm;
  void* conv;
  int ssm_bf16, conv_bf16, io_bf16, y_bf16;
  int zy_vec;          // z and y rows allow 16-byte vector access (aligned bases and row pitches), and
                       // offsets inside a chunk's rows fit in 32 bits
  LayerShape sh;
  int Q;               // chunk size
  int num_seqs, num_chunks, num_windows, total_tokens;
  const SeqEntry* seqs;        // the tables, packed in this order at the start of the workspace
  const ChunkEntry* chunks;
  const WindowEntry* windows;
  int tab_chunks, tab_windows;   // byte offsets of the chunk and window tables from the sequence table
  int tab_inline;              // > 0: the tables (this many bytes) ride in the conv launch's arguments
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
  // workspace arrays.  Post-conv activations as bf16 operand planes (one plane, or hi and lo
  // planes for fp32-faithful products), chunk-blocked with Q rows per chunk:
  // x and B transposed in blocks of kPB tokens (QB = ceil(Q / kPB) blocks per chunk), each
  // block contiguous: [planes][chunks][H][QB][P][kPB] and [planes][chunks][G][QB][N][kPB]
  uint16_t* xT;
  uint16_t* Bt;
  uint16_t* Br;          // [planes][chunks][Q][G*N]    B, channels contiguous
  uint16_t* Cr;          // [planes][chunks][Q][G*N]    C, channels contiguous
  int64_t xT_plane, Bt_plane, Br_plane, Cr_plane;   // elements per plane
  float* delta;          // [H][T]
  float* dA;             // [H][T] chunk-local inclusive cumsum of Delta*A
  void* cstate;          // [chunks][H][P][N]: each chunk's end state from a zero state; fp32 with
                         // hi/lo planes, bf16 otherwise
  uint16_t* hin;         // [planes][chunks][H][P][N]: state entering each chunk, bf16 operand planes
  int64_t hin_plane;     // elements per plane
};
// Tables of up to kInlineTableBytes travel inside the conv launch's kernel arguments: its
// workgroups read them from there and one extra workgroup writes them to the workspace for the
// later launches, so a call needs no host-to-device copy.
constexpr int kInlineTableBytes = 3072;
struct alignas(16) InlineTables {
  int32_t w[kInlineTableBytes / 4];
};
struct ConvArgs {   // the conv launch's one kernel argument
  PrefillParams p;
  InlineTables t;
};

// `inl` holds the packed tables when p.tab_inline > 0 (else it may be NULL).
hipError_t launch_prefill(const PrefillParams& p, const InlineTables* inl, hipStream_t s);
bool prefill_supported(int P, int N, int W);

}  // namespace m2
