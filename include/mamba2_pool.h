/*
 * mamba2_pool.h -- C ABI of the Mamba2 selective-state update over a slot pool
 * (MI355X / gfx950 HIP library libmamba2pool.so).
 *
 * Pages cited:
 *   [SSM-hybrids] "Hybrid SSM / Mamba models and non-KV state"
 *                 (mlinterviewnotes.com, inference course, chapter 7.3)
 *   [notes]       Mamba study notes (echobase-5bl.pages.dev, log 2026.07.27.01)
 *
 * The method, per token t and head h of group g(h) = h / (H/G):
 *   window <- last W-1 raw inputs per conv channel; v = conv_b + sum_k conv_w[k]*window_k
 *   [x | B | C] = SiLU(v)            over d_conv = H*P + 2*G*N channels
 *   Delta = softplus(dt + dt_bias);  h <- exp(Delta*A) h + Delta * x B^T
 *   y = C h + D x;  out = y * SiLU(z)
 * ([notes] "Mamba" equations; [SSM-hybrids] the selective_state_update and
 * mamba_chunk_scan_combined call sites and the state-shape function.)
 *
 * Conventions for every entry point:
 *  - All device pointers are caller-owned device memory; the library never
 *    allocates device memory (the one exception is the static scratch array
 *    of mamba2_prefill_chunked_noalloc) and never frees caller memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream).  Pointers must stay valid until the
 *    stream has completed the work.  Host pointers are read before return.
 *  - Strides are in elements of the tensor's own dtype, between consecutive
 *    rows (tokens); the innermost dimension is contiguous.
 *  - On any status other than M2_OK nothing has been enqueued and the pool
 *    is untouched.  mamba2_last_error() gives a message (thread-local).
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Calls that update the same slot must not overlap in time (in-place update).
 */
#ifndef MAMBA2_POOL_H
#define MAMBA2_POOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum m2_status {
  M2_OK = 0,
  M2_ERR_ARG = 1,         /* null pointer, negative count, bad enum */
  M2_ERR_SHAPE = 2,       /* inconsistent sizes */
  M2_ERR_DTYPE = 3,       /* unsupported dtype value */
  M2_ERR_ALIGN = 4,       /* pointer or stride not 16-byte aligned */
  M2_ERR_SLOT = 5,        /* slot out of range, duplicated, or aliasing (host-visible slots) */
  M2_ERR_UNSUPPORTED = 6, /* shape outside the compiled kernel set */
  M2_ERR_HIP = 7,         /* a HIP runtime call failed */
  M2_ERR_WORKSPACE = 8    /* workspace missing or too small */
} m2_status;

typedef enum m2_dtype { M2_F32 = 0, M2_BF16 = 1 } m2_dtype;

/* State families a pool can hold ([sizing] and the state-shape and dtype tables of [notes],
 * section "MambaSpec"). */
typedef enum m2_family {
  M2_FAMILY_MAMBA2 = 0, /* temporal state (H, P, N), conv over [x | B | C] */
  M2_FAMILY_MAMBA1 = 1, /* temporal state (D, N), conv over the D channels of x */
  M2_FAMILY_GDN = 2,    /* temporal state (num_v_heads, head_v_dim, head_k_dim), conv over q, k, v */
  M2_FAMILY_KDA = 3     /* temporal state (num_heads, head_dim, head_dim), conv over q, k, v */
} m2_family;

/* Pool descriptor.  A pool is two dense caller-owned device tensors, one per
 * state object, indexed [layer, slot, ...] ([SSM-hybrids], MambaPool passage):
 *   ssm_base : [num_layers][num_slots][nheads][head_dim][d_state]   of ssm_dtype
 *   conv_base: [num_layers][num_slots][d_conv][conv_kernel-1]        of conv_dtype
 * with d_conv = nheads*head_dim + 2*n_groups*d_state; the conv window column
 * conv_kernel-2 is the newest input.  ssm_bytes / conv_bytes must equal the
 * dense sizes exactly.  Requirements: nheads % n_groups == 0, head_dim and
 * d_state multiples of 8, 2 <= conv_kernel <= 4, bases 16-byte aligned.
 * family M2_FAMILY_MAMBA1: nheads = D (a multiple of 8), head_dim = 1,
 * n_groups = 1, so the state is [D][N] and d_conv = D.
 * family M2_FAMILY_GDN: nheads = num_v_heads, head_dim = head_v_dim,
 * d_state = head_k_dim, n_groups = num_k_heads (q and k have num_k_heads heads
 * of head_k_dim, v has num_v_heads of head_v_dim, so d_conv has the formula
 * above); both objects bf16, the dtypes the [notes] table gives GDN.
 * family M2_FAMILY_KDA: nheads = num_heads, head_dim = d_state = head_dim,
 * n_groups = num_heads (q, k and v each num_heads x head_dim: d_conv =
 * 3 * num_heads * head_dim); conv bf16 and state fp32, as the [notes] table
 * gives KDA.  GDN and KDA pools hold, copy (mamba2_checkpoint_states) and
 * quantize (the int8 store) their states; the pages give no recurrence for
 * either, so the decode and prefill entry points refuse them
 * (M2_ERR_UNSUPPORTED). */
typedef struct m2_pool_desc {
  int32_t num_layers;
  int32_t num_slots;
  int32_t nheads;
  int32_t head_dim;
  int32_t d_state;
  int32_t n_groups;
  int32_t conv_kernel;
  int32_t ssm_dtype;  /* m2_dtype */
  int32_t conv_dtype; /* m2_dtype */
  int32_t family;     /* m2_family; 0 (Mamba2) for the Mamba2 decode and prefill entry points */
  void* ssm_base;
  void* conv_base;
  uint64_t ssm_bytes;
  uint64_t conv_bytes;
} m2_pool_desc;

/* Opaque host-side handle; holds the descriptor, no device or pinned host memory. */
typedef struct m2_pool m2_pool;

/* Per-layer parameters, fp32 device arrays:
 *   A[nheads] (negative, used as given: alpha = exp(Delta*A)), D[nheads],
 *   dt_bias[nheads], conv_w[d_conv][conv_kernel] (tap conv_kernel-1 multiplies
 *   the current token), conv_b[d_conv].  conv_w must be 16-byte aligned. */
typedef struct m2_layer_params {
  const float* A;
  const float* D;
  const float* dt_bias;
  const float* conv_w;
  const float* conv_b;
} m2_layer_params;

/* Validate `desc` and create a handle.  Host-only: makes no HIP call.
 * Errors: M2_ERR_ARG, M2_ERR_SHAPE, M2_ERR_DTYPE, M2_ERR_ALIGN. */
m2_status mamba2_pool_create(const m2_pool_desc* desc, m2_pool** out);

/* Free the handle (not the caller's tensors).  NULL is a no-op. */
void mamba2_pool_destroy(m2_pool* pool);

/* State bytes of one slot in one layer ([SSM-hybrids] state-shape function:
 * temporal state (H, P, N), conv state (d_conv, W-1)):
 *   *ssm_bytes  = nheads*head_dim*d_state*sizeof(ssm_dtype)
 *   *conv_bytes = d_conv*(conv_kernel-1)*sizeof(conv_dtype)
 * Host-only. */
m2_status mamba2_pool_info(const m2_pool* pool, uint64_t* ssm_bytes_per_slot_layer,
                           uint64_t* conv_bytes_per_slot_layer);

/* One decode token per batch row, in place on the pool.  Decode has no time
 * axis to parallelise, so each row is an elementwise state update on the slot
 * named by its index ([SSM-hybrids], the selective_state_update call site);
 * fused here with the conv window shift, SiLU, softplus and the gate of [notes]
 * ("Mamba" equations).
 *   slots      device int32[batch]; slot -1 marks a padding row: its slot is
 *              neither read nor written and its output row is set to zero.
 *              A device slot outside [0, num_slots) is treated as padding.
 *   slots_host optional host copy of `slots`; when given, the call checks range
 *              and duplicates and returns M2_ERR_SLOT before enqueueing anything.
 *   x [batch][H*P], B [batch][G*N], C [batch][G*N]: raw (pre-conv) inputs of
 *              io_dtype, row strides x_stride, B_stride, C_stride (a packed
 *              [x|B|C] row of width d_conv works with B = x + H*P, C = B + G*N).
 *   z [batch][H*P], dt [batch][H] of io_dtype.
 *   y [batch][H*P] of y_dtype: out = (C h + D x) * SiLU(z), written for every row.
 * x, B, C must be 16-byte aligned with 16-byte multiple row strides.
 * Duplicated slots in one call race; pass slots_host to have them rejected.
 * Errors: M2_ERR_ARG (NULL pool, params or slots, layer or batch out of
 * range), M2_ERR_DTYPE, M2_ERR_ALIGN, M2_ERR_SLOT (with slots_host),
 * M2_ERR_UNSUPPORTED (a Mamba1 pool, d_state outside {16, 32, 64, 128, 256},
 * or a group of heads whose rows need more than 160 KiB of LDS), M2_ERR_HIP
 * (launch failure).  On any error nothing is enqueued. */
m2_status mamba2_decode_step(m2_pool* pool, int32_t layer, const m2_layer_params* params,
                             int32_t batch, const int32_t* slots, const int32_t* slots_host,
                             const void* x, int64_t x_stride, const void* B, int64_t B_stride,
                             const void* C, int64_t C_stride, const void* z, int64_t z_stride,
                             const void* dt, int64_t dt_stride, int32_t io_dtype,
                             void* y, int64_t y_stride, int32_t y_dtype, void* stream);

/* Several decode tokens per sequence in one call: a verified token and its
 * drafts under speculative decoding, where the verifier may accept any prefix
 * of the drafts, so the state after every token has to survive
 * ([SSM-hybrids]: the conv state widened by num_spec columns and one state
 * block per speculative token).  Row b runs its num_tokens tokens as decode
 * steps in order from the state and window of slots_in[b] (left as they are
 * unless also an output slot); the state and window after token t are written
 * to slot slots_out[b*num_tokens + t], so accepting t+1 tokens means switching
 * the sequence to that slot.  The states, windows and outputs equal
 * num_tokens calls of mamba2_decode_step.
 *   num_tokens 1..8.
 *   slots_in   device int32[batch]; -1 (or any slot out of range) marks a
 *              padding row: nothing is read or written and its outputs are zero.
 *   slots_out  device int32[batch*num_tokens]; an entry out of range (e.g. -1)
 *              keeps no snapshot of that token.
 *   slots_in_host, slots_out_host optional host copies; when both are given the
 *              call checks ranges, distinct input slots, distinct output slots,
 *              and that no output slot is another row's input slot, and returns
 *              M2_ERR_SLOT otherwise.
 *   x, B, C, z, dt, y: as in mamba2_decode_step with batch*num_tokens rows,
 *              row b*num_tokens + t holding token t of sequence b.
 * Errors: as mamba2_decode_step, plus M2_ERR_UNSUPPORTED for num_tokens outside
 * 1..8, batch > 65535, or num_tokens whose per-token rows of one group need
 * more than 160 KiB of LDS. */
m2_status mamba2_decode_multi(m2_pool* pool, int32_t layer, const m2_layer_params* params,
                              int32_t batch, int32_t num_tokens, const int32_t* slots_in,
                              const int32_t* slots_out, const int32_t* slots_in_host,
                              const int32_t* slots_out_host, const void* x, int64_t x_stride,
                              const void* B, int64_t B_stride, const void* C, int64_t C_stride,
                              const void* z, int64_t z_stride, const void* dt, int64_t dt_stride,
                              int32_t io_dtype, void* y, int64_t y_stride, int32_t y_dtype,
                              void* stream);

/* Bytes of device workspace mamba2_prefill_chunked needs for a call with these
 * per-sequence host arguments (the same values the call takes: cu_seqlens
 * [num_seqs+1], start_pos [num_seqs] or NULL, chunk_size, ckpt_interval and the
 * checkpoint table ckpt_slots [num_seqs][max_ckpt] or NULL).  The library builds
 * the call's chunk table from them, so checkpoints that end a chunk early are
 * counted exactly; a workspace sized for one call fits every call whose chunk
 * table is no larger.  Host-only.
 * Errors: M2_ERR_ARG (NULL pool or bytes, negative counts, cu_seqlens or
 * ckpt_slots missing where needed), M2_ERR_SHAPE (cu_seqlens[0] != 0 or
 * decreasing; size overflow), M2_ERR_UNSUPPORTED (a Mamba1 pool, chunk_size). */
m2_status mamba2_prefill_workspace_size(const m2_pool* pool, int32_t num_seqs, const int32_t* cu_seqlens,
                                        const int32_t* start_pos, int32_t chunk_size, int32_t ckpt_interval,
                                        const int32_t* ckpt_slots, int32_t max_ckpt, uint64_t* bytes);

/* Chunked (SSD) prefill of packed variable-length sequences.  Each chunk's
 * own contribution is a causally masked matrix product, and the state is carried
 * from each chunk to the next by the affine step ([SSM-hybrids], the
 * mamba_chunk_scan_combined call site; [notes] "Mamba and Attention":
 * Y = (M o L) X with L the causal mask).  The result equals the token-by-token
 * recurrence up to rounding.
 * Host arrays (read before return):
 *   cu_seqlens int32[num_seqs+1], cu_seqlens[0] = 0, non-decreasing;
 *              sequence s owns packed rows [cu_seqlens[s], cu_seqlens[s+1]).
 *   slots      int32[num_seqs], distinct, in range: the final state and conv
 *              window of sequence s are written to slots[s].
 *   has_initial_state uint8[num_seqs]: nonzero seeds the recurrence and the conv
 *              halo from slots[s] (a chunk boundary hands the state from one
 *              launch to the next: [SSM-hybrids], chunked-prefill passage on
 *              has_initial_states_p); zero means a zero state and window, and the slot is not read.
 *   start_pos  int32[num_seqs] absolute position of the first row (tokens
 *              already absorbed into the slot); may be NULL (all zero).
 *   ckpt_slots int32[num_seqs][max_ckpt] or NULL.  With ckpt_interval > 0, entry k
 *              of sequence s receives the state and conv window after absolute
 *              position p, the k-th multiple of ckpt_interval with
 *              start_pos < p <= start_pos + L_s ([SSM-hybrids] "align" mode:
 *              states kept at block-aligned positions); -1 skips it.
 *              Checkpoint slots must be distinct and disjoint from `slots`.
 *              Positions need not lie on the chunk grid: a chunk that contains a
 *              checkpoint position ends there and the next chunk starts after it
 *              (the pages' "all" mode, one checkpoint every ckpt_interval tokens,
 *              is max_ckpt columns with every slot given).
 * Device tensors: x, B, C, z, dt, y as in mamba2_decode_step with rows = packed tokens
 * (x, B, C 16-byte aligned with 16-byte multiple row strides; the row strides of x, z
 * and y below 16 MiB, else M2_ERR_SHAPE).
 * chunk_size: multiple of 16, at most 256.  Chunks start at each sequence's
 * first row.  workspace: device memory of at least
 * mamba2_prefill_workspace_size(...) bytes, 256-byte aligned, used as scratch
 * and not read across calls.  Sequences with zero length leave their slot untouched.
 * Launch tables (32 bytes per sequence and per chunk) travel in kernel arguments: up to 3072 bytes in the first kernel's, more in
 * those of small upload launches ahead of it.  The call allocates nothing, enqueues
 * no host-to-device copy and never waits on the host.
 * With fp32 SSM state the contractions run in split-bf16 (three products)
 * for fp32-level accuracy; with bf16 state they run in bf16 with fp32 accumulate. */
m2_status mamba2_prefill_chunked(m2_pool* pool, int32_t layer, const m2_layer_params* params,
                                 int32_t num_seqs, const int32_t* cu_seqlens, const int32_t* slots,
                                 const uint8_t* has_initial_state, const int32_t* start_pos,
                                 const void* x, int64_t x_stride, const void* B, int64_t B_stride,
                                 const void* C, int64_t C_stride, const void* z, int64_t z_stride,
                                 const void* dt, int64_t dt_stride, int32_t io_dtype,
                                 void* y, int64_t y_stride, int32_t y_dtype,
                                 int32_t chunk_size, int32_t ckpt_interval, const int32_t* ckpt_slots,
                                 int32_t max_ckpt, void* workspace, uint64_t workspace_bytes,
                                 void* stream);

/* mamba2_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  The scratch comes from a static device array
 * of 64 MiB (67,108,864 bytes) that every GPU the library runs on holds from
 * library load until the process ends; the call itself allocates no device or
 * pinned memory (its host-side launch tables are built in ordinary host memory).
 * Arguments, results and errors are those of mamba2_prefill_chunked, plus
 * M2_ERR_WORKSPACE when mamba2_prefill_workspace_size for the same arguments
 * exceeds 64 MiB (at the 8B-hybrid layer shape, chunk 256: up to 8,960 tokens of
 * one sequence with bf16 state, 4,735 with fp32 state), and M2_ERR_HIP if the
 * array's address cannot be looked up.
 * All calls on one GPU share that GPU's array and nothing in it survives a call:
 * calls that overlap in time on one GPU (two streams, or two threads) race and
 * must not be issued. */
m2_status mamba2_prefill_chunked_noalloc(m2_pool* pool, int32_t layer, const m2_layer_params* params,
                                         int32_t num_seqs, const int32_t* cu_seqlens, const int32_t* slots,
                                         const uint8_t* has_initial_state, const int32_t* start_pos,
                                         const void* x, int64_t x_stride, const void* B, int64_t B_stride,
                                         const void* C, int64_t C_stride, const void* z, int64_t z_stride,
                                         const void* dt, int64_t dt_stride, int32_t io_dtype,
                                         void* y, int64_t y_stride, int32_t y_dtype,
                                         int32_t chunk_size, int32_t ckpt_interval, const int32_t* ckpt_slots,
                                         int32_t max_ckpt, void* stream);

/* Copy both state objects of slot src[i] into slot dst[i], bit-exact.  A
 * cached state is copied to a fresh slot instead of being shared, since the
 * recurrence overwrites its slot ([SSM-hybrids], SGLang checkpoint passage).
 *   layer      one layer, or -1 for every layer of the pool.
 *   src, dst   device int32[n]; pairs with an index outside [0, num_slots) are skipped.
 *   src_host, dst_host optional host copies; when given, the call checks range,
 *              src != dst, distinct dst and dst not used as a src, and returns
 *              M2_ERR_SLOT otherwise. */
m2_status mamba2_checkpoint_states(m2_pool* pool, int32_t layer, int32_t n, const int32_t* src,
                                   const int32_t* dst, const int32_t* src_host,
                                   const int32_t* dst_host, void* stream);

/* int8 checkpoint store: cached states held apart from the active pool, the
 * temporal state compressed to int8 when stored and expanded once into a fresh
 * pool slot on a prefix hit, the conv window kept in its own dtype
 * ([SSM-hybrids], the SGLang passage on int8 checkpoints: symmetric codes per
 * (head, k-channel), quantized once, about twice the cached states of bf16).
 * The k-channel is read as the d_state index n (B is the key the state is
 * written with), so one fp32 scale covers h[head][0..P-1][n].  Arithmetic is
 * fp32: amax = max_p |h[p][n]|; scale = amax / 127; code = rint(h * (127 / amax))
 * clamped to [-127, 127] (both quotients correctly rounded; a zero column gives
 * scale 0 and codes 0); restore: code * scale rounded (RNE) to the pool's ssm dtype.
 * A store of num_entries entries for a pool of L layers is three caller-owned,
 * dense, 16-byte aligned device arrays:
 *   codes  int8        [num_entries][L][nheads][head_dim][d_state]
 *   scales fp32        [num_entries][L][nheads][d_state]
 *   conv   conv_dtype  [num_entries][L][d_conv][conv_kernel-1]
 * The *_bytes fields must equal those dense sizes (mamba2_int8_store_size). */
typedef struct m2_int8_store {
  int32_t num_entries;
  int32_t reserved;
  void* codes;
  void* scales;
  void* conv;
  uint64_t codes_bytes;
  uint64_t scales_bytes;
  uint64_t conv_bytes;
} m2_int8_store;

/* Dense byte sizes of a store of num_entries entries for this pool.  Host-only. */
m2_status mamba2_int8_store_size(const m2_pool* pool, int32_t num_entries, uint64_t* codes_bytes,
                                 uint64_t* scales_bytes, uint64_t* conv_bytes);

/* Quantize slot slots[i] of the pool into store entry entries[i] (both state
 * objects), for one layer or, with layer = -1, every layer.
 *   slots, entries  device int32[n]; a pair with an index out of range is skipped.
 *   slots_host, entries_host optional host copies; when given, the call checks
 *              ranges and that entries are distinct, and returns M2_ERR_SLOT otherwise.
 * Errors: M2_ERR_ARG, M2_ERR_SHAPE (store sizes), M2_ERR_ALIGN, M2_ERR_UNSUPPORTED
 * (n > 65535, or d_state / 8 > 256), M2_ERR_SLOT, M2_ERR_HIP. */
m2_status mamba2_int8_store_put(m2_pool* pool, const m2_int8_store* store, int32_t layer, int32_t n,
                                const int32_t* slots, const int32_t* entries, const int32_t* slots_host,
                                const int32_t* entries_host, void* stream);

/* Restore store entry entries[i] into slot slots[i] of the pool (both state
 * objects), for one layer or every layer (layer = -1).  Same argument rules as
 * mamba2_int8_store_put, with the slots required distinct when host copies are given. */
m2_status mamba2_int8_store_get(m2_pool* pool, const m2_int8_store* store, int32_t layer, int32_t n,
                                const int32_t* entries, const int32_t* slots, const int32_t* entries_host,
                                const int32_t* slots_host, void* stream);

/* One Mamba1 decode token per batch row on a Mamba1 pool, in place: the
 * recurrence of [notes] ("Mamba": h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t,
 * y_t = C_t h_t) with the Mamba1 shapes of the vLLM state-shape table on the
 * same page: per channel d and state index n,
 *   x = SiLU(conv_b + sum_k conv_w[d][k] * window_k)     (window over x' only)
 *   Delta_d = softplus(dt_d + dt_bias_d)
 *   h'[d][n] = exp(Delta_d * A[d][n]) h[d][n] + Delta_d * x_d * B[n]
 *   y_d = sum_n C[n] h'[d][n] + D_d x_d;  out_d = y_d * SiLU(z_d)
 * params: A fp32 [D][N] (negative), D, dt_bias, conv_b [D], conv_w [D][W].
 * Rows: x [batch][D] (raw, before the conv), B and C [batch][N] (taken as
 * given), z and dt [batch][D] of io_dtype; y [batch][D].  slots, slots_host,
 * padding rows and alignment as in mamba2_decode_step.
 * Errors: as mamba2_decode_step; M2_ERR_UNSUPPORTED for a Mamba2 pool or
 * d_state outside {8, 16, 32, 64, 128, 256}. */
m2_status mamba1_decode_step(m2_pool* pool, int32_t layer, const m2_layer_params* params, int32_t batch,
                             const int32_t* slots, const int32_t* slots_host, const void* x, int64_t x_stride,
                             const void* B, int64_t B_stride, const void* C, int64_t C_stride, const void* z,
                             int64_t z_stride, const void* dt, int64_t dt_stride, int32_t io_dtype, void* y,
                             int64_t y_stride, int32_t y_dtype, void* stream);

/* Workspace bytes mamba1_prefill needs for num_seqs sequences of total_tokens
 * rows (chunk_size as in mamba1_prefill; max_ckpt is the width of the
 * checkpoint table).  The size also serves any call with the same num_seqs,
 * chunk_size and max_ckpt and at most total_tokens rows.
 * Errors: M2_ERR_ARG (NULL, negative counts), M2_ERR_UNSUPPORTED (a Mamba2
 * pool, chunk_size neither 0 nor in 16..4096, d_state outside {8, 16, 32, 64,
 * 128, 256}), M2_ERR_SHAPE (size overflow). */
m2_status mamba1_prefill_workspace_size(const m2_pool* pool, int32_t num_seqs, int32_t total_tokens,
                                        int32_t chunk_size, int32_t max_ckpt, uint64_t* bytes);

/* Mamba1 prefill of packed sequences on a Mamba1 pool: the recurrence of
 * mamba1_decode_step ([notes] "Mamba" equations, Mamba1 shapes of the same
 * page's state-shape table) over each sequence's rows, with the prefill and
 * checkpoint behaviour [SSM-hybrids] describes for hybrid models (the
 * chunked-prefill handoff and SGLang checkpoint passages).  The state is kept
 * in fp32 between tokens and rounded only into the final slot and the
 * checkpoint slots (the Mamba2 prefill's rules: cu_seqlens, slots, has_initial_state, start_pos,
 * ckpt_interval, ckpt_slots [num_seqs][max_ckpt] -- any interval and start
 * position).  Rows: x, z, dt [T][D] (x raw, before the conv), B, C [T][N]
 * (16-byte aligned with 16-byte multiple row strides), y [T][D].  The work
 * runs in chunks of chunk_size rows (16..4096): each chunk's end state from
 * zero, a pass through each sequence's chunks, then every chunk again from its
 * entering state (a sequence's last chunk runs once).  chunk_size 0 lets the
 * library choose from the shapes alone (D, d_state, num_seqs, total rows):
 * about total/num_seqs rows per chunk, so sequences stay whole, when the batch
 * has at least 512 / ceil(D / (1024 / d_state)) sequences; else shorter
 * chunks, enough for 1024 workgroups (chunk lengths change the fp32 rounding
 * order only).  workspace: at least mamba1_prefill_workspace_size(...)
 * bytes, 256-byte aligned.  The launch tables travel in the arguments of small
 * upload launches (no allocation, no host-to-device copy, no host wait).
 * Errors: as mamba2_prefill_chunked (slot range, repeats and aliasing
 * M2_ERR_SLOT; cu_seqlens M2_ERR_SHAPE; alignment M2_ERR_ALIGN; workspace
 * M2_ERR_WORKSPACE), plus M2_ERR_UNSUPPORTED for a Mamba2 pool, d_state
 * outside {8, 16, 32, 64, 128, 256} or more than 65535 chunks or sequences.
 * On any error nothing is enqueued. */
m2_status mamba1_prefill(m2_pool* pool, int32_t layer, const m2_layer_params* params, int32_t num_seqs,
                         const int32_t* cu_seqlens, const int32_t* slots, const uint8_t* has_initial_state,
                         const int32_t* start_pos, const void* x, int64_t x_stride, const void* B,
                         int64_t B_stride, const void* C, int64_t C_stride, const void* z, int64_t z_stride,
                         const void* dt, int64_t dt_stride, int32_t io_dtype, void* y, int64_t y_stride,
                         int32_t y_dtype, int32_t chunk_size, int32_t ckpt_interval,
                         const int32_t* ckpt_slots, int32_t max_ckpt, void* workspace,
                         uint64_t workspace_bytes, void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* mamba2_last_error(void);

/* ABI version of this header (incremented on any signature change). */
int32_t mamba2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA2_POOL_H */
