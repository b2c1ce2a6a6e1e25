// Host side of the C ABI in include/mamba2_pool.h: validation, pool handles,
// prefill chunk tables, and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_set>
#include <vector>

#include "int8_store.h"
#include "kernels.h"
#include "mamba1.h"
#include "prefill.h"
#include "spec_decode.h"
#include "mamba2_pool.h"

struct m2_pool {
  m2_pool_desc d;
  m2::LayerShape sh;
  uint64_t ssm_slot_bytes;   // one slot, one layer
  uint64_t conv_slot_bytes;
};

namespace {

thread_local std::string g_err;

m2_status fail(m2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

m2_status ok() {
  g_err.clear();
  return M2_OK;
}

int esize(int32_t dt) { return dt == M2_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dt) { return dt == M2_F32 || dt == M2_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a*b with overflow detection
bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
  if (a != 0 && b > UINT64_MAX / a) return false;
  *out = a * b;
  return true;
}

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

struct IoCheck {
  const char* name;
  const void* p;
  int64_t stride;
  int64_t width;
  int es;
  bool need16;
};

m2_status check_io(const IoCheck* io, int n) {
  for (int i = 0; i < n; ++i) {
    const IoCheck& c = io[i];
    if (!c.p) return fail(M2_ERR_ARG, "%s is NULL", c.name);
    if (c.stride < c.width)
      return fail(M2_ERR_SHAPE, "%s row stride %lld is smaller than the row width %lld", c.name,
                  (long long)c.stride, (long long)c.width);
    if (c.need16 && (!aligned16(c.p) || (c.stride * c.es) % 16 != 0))
      return fail(M2_ERR_ALIGN, "%s must be 16-byte aligned with a 16-byte multiple row stride", c.name);
  }
  return M2_OK;
}

m2_status check_params(const m2_pool* pool, const m2_layer_params* w) {
  if (!w) return fail(M2_ERR_ARG, "params is NULL");
  if (!w->A || !w->D || !w->dt_bias || !w->conv_w || !w->conv_b)
    return fail(M2_ERR_ARG, "a layer parameter pointer is NULL");
  if (!aligned16(w->conv_w)) return fail(M2_ERR_ALIGN, "conv_w must be 16-byte aligned");
  (void)pool;
  return M2_OK;
}

m2::LayerShape make_shape(const m2_pool_desc& d) {
  m2::LayerShape s;
  s.H = d.nheads;
  s.P = d.head_dim;
  s.N = d.d_state;
  s.G = d.n_groups;
  s.W = d.conv_kernel;
  s.I = d.nheads * d.head_dim;
  // Mamba1: the conv runs over x only
  s.Cd = d.family == M2_FAMILY_MAMBA1 ? s.I : s.I + 2 * d.n_groups * d.d_state;
  return s;
}

const char* family_name(int family) {
  switch (family) {
    case M2_FAMILY_MAMBA2: return "Mamba2";
    case M2_FAMILY_MAMBA1: return "Mamba1";
    case M2_FAMILY_GDN: return "GDN";
    case M2_FAMILY_KDA: return "KDA";
    default: return "unknown";
  }
}

m2_status require_family(const m2_pool* pool, int family, const char* what) {
  if (pool->d.family != family)
    return fail(M2_ERR_UNSUPPORTED, "%s needs a %s pool, not a %s pool", what, family_name(family),
                family_name(pool->d.family));
  return M2_OK;
}

m2_status hip_fail(hipError_t e, const char* what) {
  return fail(M2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Prefill tables and workspace carving.
struct PrefillLayout {
  uint64_t meta_bytes;   // the packed tables (sequences, chunks) at the start
  uint64_t QC, NP, planes;
  uint64_t off_delta, off_dA, off_Cf, off_Btf, off_Gf, plane_Cf, plane_Btf, total;
};

// Workspace regions for nc chunks of at most Q tokens over T packed tokens.
bool prefill_layout(const m2::LayerShape& sh, bool split, int64_t num_seqs, int64_t T, int64_t Q, uint64_t nc,
                    PrefillLayout* L) {
  L->planes = split ? 2 : 1;
  L->QC = (uint64_t)(Q + 31) / 32 * 32;
  L->NP = sh.N < 32 ? 32 : (uint64_t)sh.N;
  L->meta_bytes = align_up(align_up(num_seqs * sizeof(m2::SeqEntry), 16) + nc * sizeof(m2::ChunkEntry), 256);
  uint64_t v, cg;
  if (!mul_ok(nc, (uint64_t)sh.G, &cg)) return false;
  if (!mul_ok((uint64_t)T, (uint64_t)sh.H * 4, &v)) return false;
  L->off_delta = L->meta_bytes;
  L->off_dA = align_up(L->off_delta + v, 256);
  L->off_Cf = align_up(L->off_dA + v, 256);
  if (!mul_ok(cg, L->QC * L->NP, &L->plane_Cf)) return false;
  if (!mul_ok(L->plane_Cf, 2 * L->planes, &v)) return false;
  L->off_Btf = align_up(L->off_Cf + v, 256);
  if (!mul_ok(cg, L->QC * (uint64_t)sh.N, &L->plane_Btf)) return false;
  if (!mul_ok(L->plane_Btf, 2 * L->planes, &v)) return false;
  L->off_Gf = align_up(L->off_Btf + v, 256);
  if (!mul_ok(cg, (uint64_t)m2::kGPairs * 64 * 8 * (split ? 4 : 2), &v)) return false;
  L->total = align_up(L->off_Gf + v, 256);
  return true;
}

// Checks of the per-sequence host arguments shared by the prefill and its workspace query.
m2_status check_prefill_seqs(int32_t num_seqs, const int32_t* cu_seqlens, const int32_t* start_pos,
                             int32_t chunk_size, int32_t ckpt_interval, const int32_t* ckpt_slots, int32_t max_ckpt) {
  if (num_seqs < 0) return fail(M2_ERR_ARG, "num_seqs is negative");
  if (chunk_size < 16 || chunk_size > 256 || chunk_size % 16 != 0)
    return fail(M2_ERR_UNSUPPORTED, "chunk_size must be a multiple of 16 in [16, 256], got %d", chunk_size);
  if (ckpt_interval < 0 || max_ckpt < 0) return fail(M2_ERR_ARG, "negative checkpoint interval or count");
  if (num_seqs == 0) return M2_OK;
  if (!cu_seqlens) return fail(M2_ERR_ARG, "cu_seqlens is required");
  if (cu_seqlens[0] != 0) return fail(M2_ERR_SHAPE, "cu_seqlens[0] must be 0");
  for (int s = 0; s < num_seqs; ++s) {
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return fail(M2_ERR_SHAPE, "cu_seqlens decreases at %d", s);
    if (start_pos && start_pos[s] < 0) return fail(M2_ERR_ARG, "start_pos of sequence %d is negative", s);
  }
  if (ckpt_interval > 0 && max_ckpt > 0 && !ckpt_slots) return fail(M2_ERR_ARG, "ckpt_slots is NULL");
  return M2_OK;
}

// The launch tables of a prefill call.  Chunks run chunk_size rows from each sequence's first row; a
// checkpoint position inside a chunk ends that chunk early, so every checkpoint falls on a chunk end.
// slots and has_init may be NULL (a size query): the entries then hold -1 and 0.
struct PrefillTables {
  std::vector<m2::SeqEntry> seqs;
  std::vector<m2::ChunkEntry> chunks;
};

void build_prefill_tables(int num_seqs, const int32_t* cu_seqlens, const int32_t* slots, const uint8_t* has_init,
                          const int32_t* start_pos, int chunk_size, int ckpt_interval, const int32_t* ckpt_slots,
                          int max_ckpt, PrefillTables* t) {
  const bool ckpt_on = ckpt_interval > 0 && max_ckpt > 0;
  t->seqs.assign(num_seqs, m2::SeqEntry{});
  t->chunks.clear();
  t->chunks.reserve((size_t)(cu_seqlens[num_seqs] / chunk_size) + (size_t)num_seqs);
  std::vector<std::pair<int, int>> ends;   // (rows into the sequence, checkpoint slot or -1)
  for (int s = 0; s < num_seqs; ++s) {
    const int t0 = cu_seqlens[s], len = cu_seqlens[s + 1] - cu_seqlens[s];
    const int64_t sp = start_pos ? start_pos[s] : 0;
    m2::SeqEntry& e = t->seqs[s];
    e.t0 = t0;
    e.len = len;
    e.slot = slots ? slots[s] : -1;
    e.has_init = has_init && has_init[s] ? 1 : 0;
    e.chunk0 = (int32_t)t->chunks.size();
    e.nchunk = 0;
    e.pad0 = e.pad1 = 0;
    ends.clear();
    for (int c0 = 0; c0 < len; c0 += chunk_size) ends.push_back({c0 + chunk_size < len ? c0 + chunk_size : len, -1});
    if (ckpt_on) {
      // entry k: the k-th multiple p of the interval with start_pos < p <= start_pos + len
      for (int k = 0; k < max_ckpt; ++k) {
        const int ck = ckpt_slots[(int64_t)s * max_ckpt + k];
        const int64_t off = (sp / ckpt_interval + 1 + k) * (int64_t)ckpt_interval - sp;
        if (ck >= 0 && off <= len) ends.push_back({(int)off, ck});
      }
    }
    std::sort(ends.begin(), ends.end(), [](const std::pair<int, int>& a, const std::pair<int, int>& b) {
      return a.first != b.first ? a.first < b.first : a.second > b.second;   // a checkpoint first
    });
    int prev = 0;
    for (const auto& en : ends) {
      if (en.first == prev) continue;   // the same end again (a grid end under a checkpoint)
      m2::ChunkEntry c;
      c.seq = s;
      c.t0 = t0 + prev;
      c.len = en.first - prev;
      c.tau0 = prev;
      c.ckpt_slot = en.second;
      c.is_last = en.first == len;
      c.pad0 = c.pad1 = 0;
      t->chunks.push_back(c);
      ++e.nchunk;
      prev = en.first;
    }
  }
  // The walk launch takes the sequences in table order: longest first, so the long walks start
  // early and the short ones fill in behind them.  (Chunks keep their order; each names its entry.)
  std::vector<int> order(num_seqs);
  for (int s = 0; s < num_seqs; ++s) order[s] = s;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return t->seqs[x].nchunk > t->seqs[y].nchunk; });
  std::vector<int> where(num_seqs);
  std::vector<m2::SeqEntry> sorted(num_seqs);
  for (int k = 0; k < num_seqs; ++k) {
    sorted[k] = t->seqs[order[k]];
    where[order[k]] = k;
  }
  t->seqs.swap(sorted);
  for (m2::ChunkEntry& c : t->chunks) c.seq = where[c.seq];
}

// Dense sizes of an int8 store of num_entries entries for this pool.
bool int8_store_sizes(const m2_pool* pool, int64_t num_entries, uint64_t* codes, uint64_t* scales, uint64_t* conv) {
  const m2::LayerShape& sh = pool->sh;
  uint64_t el;
  if (!mul_ok((uint64_t)num_entries, (uint64_t)pool->d.num_layers, &el)) return false;
  return mul_ok(el, (uint64_t)sh.H * sh.P * sh.N, codes) && mul_ok(el, (uint64_t)sh.H * sh.N * 4, scales) &&
         mul_ok(el, pool->conv_slot_bytes, conv);
}

// Shared checks and launch of the int8 store's two directions.
m2_status int8_store_call(m2_pool* pool, const m2_int8_store* store, int32_t layer, int32_t n, const int32_t* slots,
                          const int32_t* entries, const int32_t* slots_host, const int32_t* entries_host, bool put,
                          void* stream) {
  if (!pool || !store) return fail(M2_ERR_ARG, "pool and store must not be NULL");
  if (layer < -1 || layer >= pool->d.num_layers) return fail(M2_ERR_ARG, "layer %d out of range", layer);
  if (n < 0) return fail(M2_ERR_ARG, "n is negative");
  if (store->num_entries < 0) return fail(M2_ERR_ARG, "num_entries is negative");
  uint64_t cb, sb, vb;
  if (!int8_store_sizes(pool, store->num_entries, &cb, &sb, &vb)) return fail(M2_ERR_SHAPE, "store size overflows");
  if (store->codes_bytes != cb || store->scales_bytes != sb || store->conv_bytes != vb)
    return fail(M2_ERR_SHAPE, "store sizes (%llu, %llu, %llu) differ from the dense sizes (%llu, %llu, %llu)",
                (unsigned long long)store->codes_bytes, (unsigned long long)store->scales_bytes,
                (unsigned long long)store->conv_bytes, (unsigned long long)cb, (unsigned long long)sb,
                (unsigned long long)vb);
  if (n == 0) return ok();
  if (!slots || !entries) return fail(M2_ERR_ARG, "slots and entries must not be NULL");
  if (!store->codes || !store->scales || !store->conv) return fail(M2_ERR_ARG, "a store array is NULL");
  if (!aligned16(store->codes) || !aligned16(store->scales) || !aligned16(store->conv))
    return fail(M2_ERR_ALIGN, "store arrays must be 16-byte aligned");
  if (n > 65535) return fail(M2_ERR_UNSUPPORTED, "at most 65535 pairs per call");
  if (pool->sh.N / 8 > 256) return fail(M2_ERR_UNSUPPORTED, "d_state above 2048 is not supported by the int8 store");
  if (slots_host && entries_host) {
    const int S = pool->d.num_slots, E = store->num_entries;
    std::vector<uint8_t> seen(put ? E : S, 0);
    for (int i = 0; i < n; ++i) {
      const int sl = slots_host[i], en = entries_host[i];
      if (sl < 0 || sl >= S) return fail(M2_ERR_SLOT, "pair %d: slot %d out of range", i, sl);
      if (en < 0 || en >= E) return fail(M2_ERR_SLOT, "pair %d: entry %d out of range", i, en);
      const int d = put ? en : sl;
      if (seen[d]) return fail(M2_ERR_SLOT, "destination %s %d appears twice", put ? "entry" : "slot", d);
      seen[d] = 1;
    }
  }
  m2::Int8StoreArgs a;
  a.ssm = static_cast<char*>(pool->d.ssm_base);
  a.conv = static_cast<char*>(pool->d.conv_base);
  a.codes = static_cast<int8_t*>(store->codes);
  a.scales = static_cast<float*>(store->scales);
  a.store_conv = static_cast<char*>(store->conv);
  a.conv_bytes = pool->conv_slot_bytes;
  a.H = pool->sh.H;
  a.P = pool->sh.P;
  a.N = pool->sh.N;
  a.ssm_bf16 = pool->d.ssm_dtype == M2_BF16;
  a.num_layers = pool->d.num_layers;
  a.num_slots = pool->d.num_slots;
  a.num_entries = store->num_entries;
  a.l0 = layer < 0 ? 0 : layer;
  a.slots = slots;
  a.entries = entries;
  const int nl = layer < 0 ? pool->d.num_layers : 1;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = put ? m2::launch_int8_put(a, n, nl, hs) : m2::launch_int8_get(a, n, nl, hs);
  if (e != hipSuccess) return hip_fail(e, put ? "int8 store put launch" : "int8 store get launch");
  return ok();
}

// Mamba1 prefill workspace: tables, then each chunk's end state and sum of Delta, the state
// entering each chunk, and each sequence's initial window.
struct M1Layout {
  uint64_t off_chunks, off_ck, tab_bytes, off_S, off_SD, off_Hin, off_W0, total;
};

bool m1_layout(const m2::LayerShape& sh, int64_t num_seqs, int64_t nc, int64_t nck, M1Layout* L) {
  uint64_t v, dn;
  L->off_chunks = align_up((uint64_t)num_seqs * sizeof(m2::M1Seq), 16);
  L->off_ck = align_up(L->off_chunks + (uint64_t)nc * sizeof(m2::M1Chunk), 16);
  L->tab_bytes = align_up(L->off_ck + (uint64_t)nck * 4, 16);
  if (!mul_ok((uint64_t)sh.H, (uint64_t)sh.N, &dn)) return false;
  L->off_S = align_up(L->tab_bytes, 256);
  if (!mul_ok((uint64_t)nc, dn * 4, &v)) return false;
  L->off_SD = align_up(L->off_S + v, 256);
  L->off_Hin = align_up(L->off_SD + (uint64_t)nc * sh.H * 4, 256);
  L->off_W0 = align_up(L->off_Hin + v, 256);
  L->total = align_up(L->off_W0 + (uint64_t)num_seqs * sh.H * (sh.W - 1) * 4, 256);
  return true;
}

}  // namespace

extern "C" {

int32_t mamba2_abi_version(void) { return 3; }

const char* mamba2_last_error(void) { return g_err.c_str(); }

m2_status mamba2_pool_create(const m2_pool_desc* desc, m2_pool** out) {
  if (!desc || !out) return fail(M2_ERR_ARG, "desc and out must not be NULL");
  *out = nullptr;
  const m2_pool_desc& d = *desc;
  if (d.num_layers < 1 || d.num_slots < 1 || d.nheads < 1 || d.head_dim < 1 || d.d_state < 1 ||
      d.n_groups < 1)
    return fail(M2_ERR_ARG, "layer, slot, head, head_dim, d_state and group counts must be positive");
  if (d.conv_kernel < 2 || d.conv_kernel > 4)
    return fail(M2_ERR_UNSUPPORTED, "conv_kernel %d outside the supported range 2..4", d.conv_kernel);
  if (d.family < M2_FAMILY_MAMBA2 || d.family > M2_FAMILY_KDA)
    return fail(M2_ERR_ARG, "family %d is none of Mamba2 (0), Mamba1 (1), GDN (2), KDA (3)", d.family);
  if (d.family == M2_FAMILY_MAMBA1) {
    if (d.head_dim != 1 || d.n_groups != 1)
      return fail(M2_ERR_SHAPE, "a Mamba1 pool has head_dim 1 and n_groups 1 (nheads = D channels)");
    if (d.nheads % 8 != 0 || d.d_state % 8 != 0)
      return fail(M2_ERR_SHAPE, "a Mamba1 pool needs D and d_state multiples of 8");
  } else {
    if (d.nheads % d.n_groups != 0)
      return fail(M2_ERR_SHAPE, "nheads %d is not a multiple of n_groups %d", d.nheads, d.n_groups);
    if (d.head_dim % 8 != 0 || d.d_state % 8 != 0)
      return fail(M2_ERR_SHAPE, "head_dim and d_state must be multiples of 8");
  }
  if (d.family == M2_FAMILY_KDA && (d.head_dim != d.d_state || d.n_groups != d.nheads))
    return fail(M2_ERR_SHAPE, "a KDA pool has a square (head_dim, head_dim) state per head and n_groups = nheads "
                "(got head_dim %d, d_state %d, n_groups %d, nheads %d)", d.head_dim, d.d_state, d.n_groups, d.nheads);
  if (!dtype_ok(d.ssm_dtype) || !dtype_ok(d.conv_dtype)) return fail(M2_ERR_DTYPE, "ssm/conv dtype must be F32 or BF16");
  if (d.family == M2_FAMILY_GDN && (d.ssm_dtype != M2_BF16 || d.conv_dtype != M2_BF16))
    return fail(M2_ERR_DTYPE, "a GDN pool keeps both objects in bf16");
  if (d.family == M2_FAMILY_KDA && (d.ssm_dtype != M2_F32 || d.conv_dtype != M2_BF16))
    return fail(M2_ERR_DTYPE, "a KDA pool keeps its conv window in bf16 and its state in fp32");
  if (!d.ssm_base || !d.conv_base) return fail(M2_ERR_ARG, "ssm_base and conv_base must not be NULL");
  if (!aligned16(d.ssm_base) || !aligned16(d.conv_base))
    return fail(M2_ERR_ALIGN, "pool bases must be 16-byte aligned");
  const m2::LayerShape sh = make_shape(d);
  uint64_t ssm_slot, conv_slot, tmp, ssm_total, conv_total;
  if (!mul_ok((uint64_t)sh.H * sh.P, (uint64_t)sh.N * esize(d.ssm_dtype), &ssm_slot) ||
      !mul_ok((uint64_t)sh.Cd, (uint64_t)(sh.W - 1) * esize(d.conv_dtype), &conv_slot) ||
      !mul_ok((uint64_t)d.num_layers, (uint64_t)d.num_slots, &tmp) || !mul_ok(tmp, ssm_slot, &ssm_total) ||
      !mul_ok(tmp, conv_slot, &conv_total))
    return fail(M2_ERR_SHAPE, "pool size overflows 64 bits");
  if (d.ssm_bytes != ssm_total)
    return fail(M2_ERR_SHAPE, "ssm_bytes %llu != layers*slots*H*P*N*size = %llu", (unsigned long long)d.ssm_bytes,
                (unsigned long long)ssm_total);
  if (d.conv_bytes != conv_total)
    return fail(M2_ERR_SHAPE, "conv_bytes %llu != layers*slots*d_conv*(W-1)*size = %llu",
                (unsigned long long)d.conv_bytes, (unsigned long long)conv_total);
  m2_pool* p = new (std::nothrow) m2_pool();
  if (!p) return fail(M2_ERR_ARG, "out of host memory");
  p->d = d;
  p->sh = sh;
  p->ssm_slot_bytes = ssm_slot;
  p->conv_slot_bytes = conv_slot;
  *out = p;
  return ok();
}

void mamba2_pool_destroy(m2_pool* pool) { delete pool; }

m2_status mamba2_pool_info(const m2_pool* pool, uint64_t* ssm_bytes, uint64_t* conv_bytes) {
  if (!pool || !ssm_bytes || !conv_bytes) return fail(M2_ERR_ARG, "NULL argument");
  *ssm_bytes = pool->ssm_slot_bytes;
  *conv_bytes = pool->conv_slot_bytes;
  return ok();
}

m2_status mamba2_decode_step(m2_pool* pool, int32_t layer, const m2_layer_params* params, int32_t batch,
                             const int32_t* slots, const int32_t* slots_host, const void* x, int64_t x_stride,
                             const void* B, int64_t B_stride, const void* C, int64_t C_stride, const void* z,
                             int64_t z_stride, const void* dt, int64_t dt_stride, int32_t io_dtype, void* y,
                             int64_t y_stride, int32_t y_dtype, void* stream) {
  if (!pool) return fail(M2_ERR_ARG, "pool is NULL");
  if (m2_status st = require_family(pool, M2_FAMILY_MAMBA2, "mamba2_decode_step")) return st;
  const m2::LayerShape& sh = pool->sh;
  if (layer < 0 || layer >= pool->d.num_layers) return fail(M2_ERR_ARG, "layer %d out of range", layer);
  if (batch < 0) return fail(M2_ERR_ARG, "batch %d is negative", batch);
  if (m2_status st = check_params(pool, params)) return st;
  if (!dtype_ok(io_dtype) || !dtype_ok(y_dtype)) return fail(M2_ERR_DTYPE, "io/y dtype must be F32 or BF16");
  if (batch == 0) return ok();
  if (!slots) return fail(M2_ERR_ARG, "slots is NULL");
  const int ies = esize(io_dtype);
  const int GN = sh.G * sh.N;
  const IoCheck io[] = {{"x", x, x_stride, sh.I, ies, true},        {"B", B, B_stride, GN, ies, true},
                        {"C", C, C_stride, GN, ies, true},          {"z", z, z_stride, sh.I, ies, false},
                        {"dt", dt, dt_stride, sh.H, ies, false},    {"y", y, y_stride, sh.I, esize(y_dtype), false}};
  if (m2_status st = check_io(io, 6)) return st;
  if (!m2::decode_supported(pool->d.ssm_dtype == M2_BF16, sh.N, sh.W))
    return fail(M2_ERR_UNSUPPORTED, "decode supports d_state in {16,32,64,128,256}, got %d", sh.N);
  if (m2::decode_lds_bytes(sh.H / sh.G, sh.P, sh.N) > m2::kMaxLdsBytes)
    return fail(M2_ERR_UNSUPPORTED, "decode: a group of %d heads x %d rows needs more LDS per workgroup than %zu bytes",
                sh.H / sh.G, sh.P, m2::kMaxLdsBytes);
  if (slots_host) {
    std::vector<uint8_t> seen(pool->d.num_slots, 0);
    for (int i = 0; i < batch; ++i) {
      const int s = slots_host[i];
      if (s == -1) continue;
      if (s < 0 || s >= pool->d.num_slots) return fail(M2_ERR_SLOT, "slot %d of row %d out of range", s, i);
      if (seen[s]) return fail(M2_ERR_SLOT, "slot %d appears twice", s);
      seen[s] = 1;
    }
  }
  m2::DecodeParams p;
  p.ssm = static_cast<char*>(pool->d.ssm_base) + (uint64_t)layer * pool->d.num_slots * pool->ssm_slot_bytes;
  p.conv = static_cast<char*>(pool->d.conv_base) + (uint64_t)layer * pool->d.num_slots * pool->conv_slot_bytes;
  p.num_slots = pool->d.num_slots;
  p.ssm_bf16 = pool->d.ssm_dtype == M2_BF16;
  p.conv_bf16 = pool->d.conv_dtype == M2_BF16;
  p.io_bf16 = io_dtype == M2_BF16;
  p.y_bf16 = y_dtype == M2_BF16;
  p.H = sh.H;
  p.P = sh.P;
  p.G = sh.G;
  p.I = sh.I;
  p.x_stride = x_stride;
  p.B_stride = B_stride;
  p.C_stride = C_stride;
  p.z_stride = z_stride;
  p.dt_stride = dt_stride;
  p.y_stride = y_stride;
  p.A = params->A;
  p.D = params->D;
  p.dt_bias = params->dt_bias;
  p.conv_w = params->conv_w;
  p.conv_b = params->conv_b;
  const int kMaxRows = 65535;   // rows per launch
  for (int r0 = 0; r0 < batch; r0 += kMaxRows) {
    const int nb = batch - r0 < kMaxRows ? batch - r0 : kMaxRows;
    p.slots = slots + r0;
    p.x = static_cast<const char*>(x) + (int64_t)r0 * x_stride * ies;
    p.B = static_cast<const char*>(B) + (int64_t)r0 * B_stride * ies;
    p.C = static_cast<const char*>(C) + (int64_t)r0 * C_stride * ies;
    p.z = static_cast<const char*>(z) + (int64_t)r0 * z_stride * ies;
    p.dt = static_cast<const char*>(dt) + (int64_t)r0 * dt_stride * ies;
    p.y = static_cast<char*>(y) + (int64_t)r0 * y_stride * esize(y_dtype);
    const hipError_t e = m2::launch_decode(p, sh.N, sh.W, nb, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  return ok();
}

m2_status mamba2_prefill_workspace_size(const m2_pool* pool, int32_t num_seqs, const int32_t* cu_seqlens,
                                        const int32_t* start_pos, int32_t chunk_size, int32_t ckpt_interval,
                                        const int32_t* ckpt_slots, int32_t max_ckpt, uint64_t* bytes) {
  if (!pool || !bytes) return fail(M2_ERR_ARG, "NULL argument");
  if (m2_status st = require_family(pool, M2_FAMILY_MAMBA2, "mamba2_prefill_workspace_size")) return st;
  if (m2_status st = check_prefill_seqs(num_seqs, cu_seqlens, start_pos, chunk_size, ckpt_interval, ckpt_slots,
                                        max_ckpt))
    return st;
  *bytes = 0;
  if (num_seqs == 0 || cu_seqlens[num_seqs] == 0) return ok();
  PrefillTables t;
  build_prefill_tables(num_seqs, cu_seqlens, nullptr, nullptr, start_pos, chunk_size, ckpt_interval, ckpt_slots,
                       max_ckpt, &t);
  PrefillLayout L;
  if (!prefill_layout(pool->sh, pool->d.ssm_dtype == M2_F32, num_seqs, cu_seqlens[num_seqs], chunk_size,
                      t.chunks.size(), &L))
    return fail(M2_ERR_SHAPE, "workspace size overflows 64 bits");
  *bytes = L.total;
  return ok();
}

m2_status mamba2_prefill_chunked(m2_pool* pool, int32_t layer, const m2_layer_params* params, int32_t num_seqs,
                                 const int32_t* cu_seqlens, const int32_t* slots, const uint8_t* has_init,
                                 const int32_t* start_pos, const void* x, int64_t x_stride, const void* B,
                                 int64_t B_stride, const void* C, int64_t C_stride, const void* z, int64_t z_stride,
                                 const void* dt, int64_t dt_stride, int32_t io_dtype, void* y, int64_t y_stride,
                                 int32_t y_dtype, int32_t chunk_size, int32_t ckpt_interval,
                                 const int32_t* ckpt_slots, int32_t max_ckpt, void* workspace,
                                 uint64_t workspace_bytes, void* stream) {
  if (!pool) return fail(M2_ERR_ARG, "pool is NULL");
  if (m2_status st = require_family(pool, M2_FAMILY_MAMBA2, "mamba2_prefill_chunked")) return st;
  const m2::LayerShape& sh = pool->sh;
  if (layer < 0 || layer >= pool->d.num_layers) return fail(M2_ERR_ARG, "layer %d out of range", layer);
  if (num_seqs < 0) return fail(M2_ERR_ARG, "num_seqs is negative");
  if (m2_status st = check_params(pool, params)) return st;
  if (!dtype_ok(io_dtype) || !dtype_ok(y_dtype)) return fail(M2_ERR_DTYPE, "io/y dtype must be F32 or BF16");
  if (m2_status st = check_prefill_seqs(num_seqs, cu_seqlens, start_pos, chunk_size, ckpt_interval, ckpt_slots,
                                        max_ckpt))
    return st;
  if (num_seqs == 0) return ok();
  if (!slots || !has_init) return fail(M2_ERR_ARG, "slots and has_initial_state are required");
  const int64_t T = cu_seqlens[num_seqs];
  const bool ckpt_on = ckpt_interval > 0 && max_ckpt > 0;
  const int S = pool->d.num_slots;
  std::vector<uint8_t> used(S, 0);
  for (int s = 0; s < num_seqs; ++s) {
    const int sl = slots[s];
    if (sl < 0 || sl >= S) return fail(M2_ERR_SLOT, "slot %d of sequence %d out of range", sl, s);
    if (used[sl]) return fail(M2_ERR_SLOT, "slot %d appears twice", sl);
    used[sl] = 1;
  }
  if (ckpt_on) {
    for (int64_t i = 0; i < (int64_t)num_seqs * max_ckpt; ++i) {
      const int sl = ckpt_slots[i];
      if (sl == -1) continue;
      if (sl < 0 || sl >= S) return fail(M2_ERR_SLOT, "checkpoint slot %d out of range", sl);
      if (used[sl]) return fail(M2_ERR_SLOT, "checkpoint slot %d repeats or aliases a sequence slot", sl);
      used[sl] = 1;
    }
  }
  if (T == 0) return ok();
  const int ies = esize(io_dtype);
  const int GN = sh.G * sh.N;
  const IoCheck io[] = {{"x", x, x_stride, sh.I, ies, true},        {"B", B, B_stride, GN, ies, true},
                        {"C", C, C_stride, GN, ies, true},          {"z", z, z_stride, sh.I, ies, false},
                        {"dt", dt, dt_stride, sh.H, ies, false},    {"y", y, y_stride, sh.I, esize(y_dtype), false}};
  if (m2_status st = check_io(io, 6)) return st;
  // the walk addresses the rows of a chunk with 32-bit byte offsets from the chunk's first row
  if (x_stride * ies >= (int64_t)1 << 24 || z_stride * ies >= (int64_t)1 << 24 ||
      y_stride * esize(y_dtype) >= (int64_t)1 << 24)
    return fail(M2_ERR_SHAPE, "prefill row strides of x, z and y must be below 16 MiB");
  if (!m2::prefill_supported(sh.P, sh.N, sh.W))
    return fail(M2_ERR_UNSUPPORTED, "prefill supports head_dim in {16,32,64,128} and d_state in {16,32,64,128}");

  PrefillTables t;
  build_prefill_tables(num_seqs, cu_seqlens, slots, has_init, start_pos, chunk_size, ckpt_interval, ckpt_slots,
                       max_ckpt, &t);
  const std::vector<m2::SeqEntry>& seqs = t.seqs;
  const std::vector<m2::ChunkEntry>& chunks = t.chunks;
  PrefillLayout L;
  if (!prefill_layout(sh, pool->d.ssm_dtype == M2_F32, num_seqs, T, chunk_size, chunks.size(), &L))
    return fail(M2_ERR_SHAPE, "workspace size overflows");
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(M2_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(M2_ERR_WORKSPACE, "workspace has %llu bytes, needs %llu", (unsigned long long)workspace_bytes,
                (unsigned long long)L.total);
  if (chunks.empty()) return ok();
  if ((int64_t)num_seqs * sh.H * (sh.P / m2::prefill_part(sh.P, pool->d.ssm_dtype == M2_F32)) > INT32_MAX || (int64_t)chunks.size() * sh.G > INT32_MAX)
    return fail(M2_ERR_UNSUPPORTED, "too many sequences or chunks for one launch");

  // ---- pack the tables; small ones travel in the first launch's arguments, larger ones in the
  // arguments of upload launches ahead of it (no host-to-device copy, no host wait)
  const size_t tab_chunks = align_up(seqs.size() * sizeof(m2::SeqEntry), 16);
  const size_t tab_bytes = align_up(tab_chunks + chunks.size() * sizeof(m2::ChunkEntry), 16);
  if (tab_bytes > L.meta_bytes) return fail(M2_ERR_WORKSPACE, "table packing exceeds its workspace region");
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool tab_inline = tab_bytes <= (size_t)m2::kInlineTableBytes;
  std::vector<char> packed(tab_bytes, 0);
  memcpy(packed.data(), seqs.data(), seqs.size() * sizeof(m2::SeqEntry));
  memcpy(packed.data() + tab_chunks, chunks.data(), chunks.size() * sizeof(m2::ChunkEntry));
  m2::InlineTables inl;
  if (tab_inline) {
    memcpy(inl.w, packed.data(), tab_bytes);
  } else {
    const hipError_t eu = m2::launch_table_upload(ws, packed.data(), tab_bytes, hs);
    if (eu != hipSuccess) return hip_fail(eu, "table upload");
  }

  const int yes = esize(y_dtype);
  m2::PrefillParams p;
  p.ssm = static_cast<char*>(pool->d.ssm_base) + (uint64_t)layer * pool->d.num_slots * pool->ssm_slot_bytes;
  p.conv = static_cast<char*>(pool->d.conv_base) + (uint64_t)layer * pool->d.num_slots * pool->conv_slot_bytes;
  p.ssm_bf16 = pool->d.ssm_dtype == M2_BF16;
  p.conv_bf16 = pool->d.conv_dtype == M2_BF16;
  p.io_bf16 = io_dtype == M2_BF16;
  p.y_bf16 = y_dtype == M2_BF16;
  // z and y in vector pieces of up to 8 elements: bases and row pitches aligned to 8 elements
  p.zy_vec = (reinterpret_cast<uintptr_t>(z) % (8 * ies)) == 0 && (reinterpret_cast<uintptr_t>(y) % (8 * yes)) == 0 &&
             z_stride % 8 == 0 && y_stride % 8 == 0;
  p.sh = sh;
  p.Q = chunk_size;
  p.QC = (int)L.QC;
  p.nparts = sh.P / m2::prefill_part(sh.P, pool->d.ssm_dtype == M2_F32);
  p.num_seqs = num_seqs;
  p.num_chunks = (int)chunks.size();
  p.total_tokens = (int)T;
  p.seqs = reinterpret_cast<const m2::SeqEntry*>(ws);
  p.chunks = reinterpret_cast<const m2::ChunkEntry*>(ws + tab_chunks);
  p.tab_chunks = (int)tab_chunks;
  p.tab_inline = tab_inline ? (int)tab_bytes : 0;
  p.x = x;
  p.B = B;
  p.C = C;
  p.z = z;
  p.dt = dt;
  p.x_stride = x_stride;
  p.B_stride = B_stride;
  p.C_stride = C_stride;
  p.z_stride = z_stride;
  p.dt_stride = dt_stride;
  p.y = y;
  p.y_stride = y_stride;
  p.A = params->A;
  p.D = params->D;
  p.dt_bias = params->dt_bias;
  p.conv_w = params->conv_w;
  p.conv_b = params->conv_b;
  p.delta = reinterpret_cast<float*>(ws + L.off_delta);
  p.dA = reinterpret_cast<float*>(ws + L.off_dA);
  p.Cf = reinterpret_cast<uint16_t*>(ws + L.off_Cf);
  p.Btf = reinterpret_cast<uint16_t*>(ws + L.off_Btf);
  p.Gf = ws + L.off_Gf;
  p.Cf_plane = (int64_t)L.plane_Cf;
  p.Btf_plane = (int64_t)L.plane_Btf;
  const hipError_t e = m2::launch_prefill(p, tab_inline ? &inl : nullptr, hs);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

m2_status mamba2_prefill_chunked_noalloc(m2_pool* pool, int32_t layer, const m2_layer_params* params,
                                         int32_t num_seqs, const int32_t* cu_seqlens, const int32_t* slots,
                                         const uint8_t* has_init, const int32_t* start_pos, const void* x,
                                         int64_t x_stride, const void* B, int64_t B_stride, const void* C,
                                         int64_t C_stride, const void* z, int64_t z_stride, const void* dt,
                                         int64_t dt_stride, int32_t io_dtype, void* y, int64_t y_stride,
                                         int32_t y_dtype, int32_t chunk_size, int32_t ckpt_interval,
                                         const int32_t* ckpt_slots, int32_t max_ckpt, void* stream) {
  if (!pool) return fail(M2_ERR_ARG, "pool is NULL");
  uint64_t need = 0;
  if (m2_status st = mamba2_prefill_workspace_size(pool, num_seqs, cu_seqlens, start_pos, chunk_size, ckpt_interval,
                                                   ckpt_slots, max_ckpt, &need))
    return st;
  if (need > m2::kNoAllocScratchBytes)
    return fail(M2_ERR_WORKSPACE, "the call needs %llu bytes of scratch; the static scratch holds %llu",
                (unsigned long long)need, (unsigned long long)m2::kNoAllocScratchBytes);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = m2::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
  }
  return mamba2_prefill_chunked(pool, layer, params, num_seqs, cu_seqlens, slots, has_init, start_pos, x, x_stride,
                                B, B_stride, C, C_stride, z, z_stride, dt, dt_stride, io_dtype, y, y_stride, y_dtype,
                                chunk_size, ckpt_interval, ckpt_slots, max_ckpt, scratch,
                                need > 0 ? m2::kNoAllocScratchBytes : 0, stream);
}

m2_status mamba2_checkpoint_states(m2_pool* pool, int32_t layer, int32_t n, const int32_t* src, const int32_t* dst,
                                   const int32_t* src_host, const int32_t* dst_host, void* stream) {
  if (!pool) return fail(M2_ERR_ARG, "pool is NULL");
  if (layer < -1 || layer >= pool->d.num_layers) return fail(M2_ERR_ARG, "layer %d out of range", layer);
  if (n < 0) return fail(M2_ERR_ARG, "n is negative");
  if (n == 0) return ok();
  if (!src || !dst) return fail(M2_ERR_ARG, "src and dst must not be NULL");
  if (n > 65535) return fail(M2_ERR_UNSUPPORTED, "at most 65535 pairs per call");
  if (src_host && dst_host) {
    const int S = pool->d.num_slots;
    std::vector<uint8_t> is_dst(S, 0), is_src(S, 0);
    for (int i = 0; i < n; ++i) {
      const int s = src_host[i], d = dst_host[i];
      if (s < 0 || s >= S || d < 0 || d >= S) return fail(M2_ERR_SLOT, "pair %d (%d -> %d) out of range", i, s, d);
      if (s == d) return fail(M2_ERR_SLOT, "pair %d copies slot %d onto itself", i, s);
      if (is_dst[d]) return fail(M2_ERR_SLOT, "destination slot %d appears twice", d);
      is_dst[d] = 1;
      is_src[s] = 1;
    }
    for (int i = 0; i < n; ++i)
      if (is_src[dst_host[i]]) return fail(M2_ERR_SLOT, "destination slot %d is also a source", dst_host[i]);
  }
  const int l0 = layer < 0 ? 0 : layer;
  const int nl = layer < 0 ? pool->d.num_layers : 1;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int S = pool->d.num_slots;
  const hipError_t e = m2::launch_slot_copy(pool->d.ssm_base, pool->ssm_slot_bytes, pool->d.conv_base,
                                            pool->conv_slot_bytes, (uint64_t)S, l0, nl, n, src, dst, hs);
  if (e != hipSuccess) return hip_fail(e, "checkpoint copy launch");
  return ok();
}

m2_status mamba2_int8_store_size(const m2_pool* pool, int32_t num_entries, uint64_t* codes_bytes,
                                 uint64_t* scales_bytes, uint64_t* conv_bytes) {
  if (!pool || !codes_bytes || !scales_bytes || !conv_bytes) return fail(M2_ERR_ARG, "NULL argument");
  if (num_entries < 0) return fail(M2_ERR_ARG, "num_entries is negative");
  if (!int8_store_sizes(pool, num_entries, codes_bytes, scales_bytes, conv_bytes))
    return fail(M2_ERR_SHAPE, "store size overflows");
  return ok();
}

m2_status mamba2_int8_store_put(m2_pool* pool, const m2_int8_store* store, int32_t layer, int32_t n,
                                const int32_t* slots, const int32_t* entries, const int32_t* slots_host,
                                const int32_t* entries_host, void* stream) {
  return int8_store_call(pool, store, layer, n, slots, entries, slots_host, entries_host, true, stream);
}

m2_status mamba2_int8_store_get(m2_pool* pool, const m2_int8_store* store, int32_t layer, int32_t n,
                                const int32_t* entries, const int32_t* slots, const int32_t* entries_host,
                                const int32_t* slots_host, void* stream) {
  return int8_store_call(pool, store, layer, n, slots, entries, slots_host, entries_host, false, stream);
}

m2_status mamba2_decode_multi(m2_pool* pool, int32_t layer, const m2_layer_params* params, int32_t batch,
                              int32_t num_tokens, const int32_t* slots_in, const int32_t* slots_out,
                              const int32_t* slots_in_host, const int32_t* slots_out_host, const void* x,
                              int64_t x_stride, const void* B, int64_t B_stride, const void* C, int64_t C_stride,
                              const void* z, int64_t z_stride, const void* dt, int64_t dt_stride, int32_t io_dtype,
                              void* y, int64_t y_stride, int32_t y_dtype, void* stream) {
  if (!pool) return fail(M2_ERR_ARG, "pool is NULL");
  if (m2_status st = require_family(pool, M2_FAMILY_MAMBA2, "mamba2_decode_multi")) return st;
  const m2::LayerShape& sh = pool->sh;
  if (layer < 0 || layer >= pool->d.num_layers) return fail(M2_ERR_ARG, "layer %d out of range", layer);
  if (batch < 0) return fail(M2_ERR_ARG, "batch %d is negative", batch);
  if (num_tokens < 1 || num_tokens > m2::kMaxDecodeTokens)
    return fail(M2_ERR_UNSUPPORTED, "num_tokens must be in [1, %d], got %d", m2::kMaxDecodeTokens, num_tokens);
  if (m2::multi_decode_lds_bytes(pool->sh.H / pool->sh.G, pool->sh.P, pool->sh.N, num_tokens) > m2::kMaxLdsBytes)
    return fail(M2_ERR_UNSUPPORTED, "multi-token decode: %d tokens of a %d-head x %d-row group need more LDS per "
                "workgroup than %zu bytes", num_tokens, pool->sh.H / pool->sh.G, pool->sh.P, m2::kMaxLdsBytes);
  if (m2_status st = check_params(pool, params)) return st;
  if (!dtype_ok(io_dtype) || !dtype_ok(y_dtype)) return fail(M2_ERR_DTYPE, "io/y dtype must be F32 or BF16");
  if (batch == 0) return ok();
  if (!slots_in || !slots_out) return fail(M2_ERR_ARG, "slots_in and slots_out must not be NULL");
  const int ies = esize(io_dtype);
  const int GN = sh.G * sh.N;
  const IoCheck io[] = {{"x", x, x_stride, sh.I, ies, true},        {"B", B, B_stride, GN, ies, true},
                        {"C", C, C_stride, GN, ies, true},          {"z", z, z_stride, sh.I, ies, false},
                        {"dt", dt, dt_stride, sh.H, ies, false},    {"y", y, y_stride, sh.I, esize(y_dtype), false}};
  if (m2_status st = check_io(io, 6)) return st;
  if (!m2::decode_supported(pool->d.ssm_dtype == M2_BF16, sh.N, sh.W))
    return fail(M2_ERR_UNSUPPORTED, "decode supports d_state in {16,32,64,128,256}, got %d", sh.N);
  if ((int64_t)batch > 65535) return fail(M2_ERR_UNSUPPORTED, "at most 65535 sequences per multi-token call");
  if (slots_in_host && slots_out_host) {
    const int S = pool->d.num_slots;
    std::vector<int> in_row(S, -1);   // the row that reads each slot
    for (int i = 0; i < batch; ++i) {
      const int s = slots_in_host[i];
      if (s == -1) continue;
      if (s < 0 || s >= S) return fail(M2_ERR_SLOT, "input slot %d of row %d out of range", s, i);
      if (in_row[s] >= 0) return fail(M2_ERR_SLOT, "input slot %d appears twice", s);
      in_row[s] = i;
    }
    std::vector<uint8_t> written(S, 0);
    for (int64_t i = 0; i < (int64_t)batch * num_tokens; ++i) {
      const int o = slots_out_host[i];
      if (o == -1) continue;
      const int row = (int)(i / num_tokens);
      if (o < 0 || o >= S) return fail(M2_ERR_SLOT, "output slot %d of row %d out of range", o, row);
      if (written[o]) return fail(M2_ERR_SLOT, "output slot %d appears twice", o);
      if (in_row[o] >= 0 && in_row[o] != row)
        return fail(M2_ERR_SLOT, "output slot %d of row %d is the input slot of row %d", o, row, in_row[o]);
      written[o] = 1;
    }
  }
  m2::MultiDecodeParams m;
  m2::DecodeParams& p = m.d;
  p.ssm = static_cast<char*>(pool->d.ssm_base) + (uint64_t)layer * pool->d.num_slots * pool->ssm_slot_bytes;
  p.conv = static_cast<char*>(pool->d.conv_base) + (uint64_t)layer * pool->d.num_slots * pool->conv_slot_bytes;
  p.num_slots = pool->d.num_slots;
  p.ssm_bf16 = pool->d.ssm_dtype == M2_BF16;
  p.conv_bf16 = pool->d.conv_dtype == M2_BF16;
  p.io_bf16 = io_dtype == M2_BF16;
  p.y_bf16 = y_dtype == M2_BF16;
  p.H = sh.H;
  p.P = sh.P;
  p.G = sh.G;
  p.I = sh.I;
  p.slots = slots_in;
  p.x = x;
  p.B = B;
  p.C = C;
  p.z = z;
  p.dt = dt;
  p.x_stride = x_stride;
  p.B_stride = B_stride;
  p.C_stride = C_stride;
  p.z_stride = z_stride;
  p.dt_stride = dt_stride;
  p.y = y;
  p.y_stride = y_stride;
  p.A = params->A;
  p.D = params->D;
  p.dt_bias = params->dt_bias;
  p.conv_w = params->conv_w;
  p.conv_b = params->conv_b;
  m.slots_out = slots_out;
  m.K = num_tokens;
  const hipError_t e = m2::launch_decode_multi(m, sh.N, sh.W, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "multi-token decode launch");
  return ok();
}

m2_status mamba1_decode_step(m2_pool* pool, int32_t layer, const m2_layer_params* params, int32_t batch,
                             const int32_t* slots, const int32_t* slots_host, const void* x, int64_t x_stride,
                             const void* B, int64_t B_stride, const void* C, int64_t C_stride, const void* z,
                             int64_t z_stride, const void* dt, int64_t dt_stride, int32_t io_dtype, void* y,
                             int64_t y_stride, int32_t y_dtype, void* stream) {
  if (!pool) return fail(M2_ERR_ARG, "pool is NULL");
  if (m2_status st = require_family(pool, M2_FAMILY_MAMBA1, "mamba1_decode_step")) return st;
  const m2::LayerShape& sh = pool->sh;
  if (layer < 0 || layer >= pool->d.num_layers) return fail(M2_ERR_ARG, "layer %d out of range", layer);
  if (batch < 0) return fail(M2_ERR_ARG, "batch %d is negative", batch);
  if (m2_status st = check_params(pool, params)) return st;
  if (!dtype_ok(io_dtype) || !dtype_ok(y_dtype)) return fail(M2_ERR_DTYPE, "io/y dtype must be F32 or BF16");
  if (batch == 0) return ok();
  if (!slots) return fail(M2_ERR_ARG, "slots is NULL");
  const int ies = esize(io_dtype);
  const int D = sh.H;
  const IoCheck io[] = {{"x", x, x_stride, D, ies, false},      {"B", B, B_stride, sh.N, ies, false},
                        {"C", C, C_stride, sh.N, ies, false},   {"z", z, z_stride, D, ies, false},
                        {"dt", dt, dt_stride, D, ies, false},   {"y", y, y_stride, D, esize(y_dtype), false}};
  if (m2_status st = check_io(io, 6)) return st;
  if (!m2::mamba1_supported(sh.N, sh.W))
    return fail(M2_ERR_UNSUPPORTED, "Mamba1 decode supports d_state in {8,16,32,64,128,256}, got %d", sh.N);
  if (slots_host) {
    std::vector<uint8_t> seen(pool->d.num_slots, 0);
    for (int i = 0; i < batch; ++i) {
      const int s = slots_host[i];
      if (s == -1) continue;
      if (s < 0 || s >= pool->d.num_slots) return fail(M2_ERR_SLOT, "slot %d of row %d out of range", s, i);
      if (seen[s]) return fail(M2_ERR_SLOT, "slot %d appears twice", s);
      seen[s] = 1;
    }
  }
  m2::Mamba1Params p;
  p.ssm = static_cast<char*>(pool->d.ssm_base) + (uint64_t)layer * pool->d.num_slots * pool->ssm_slot_bytes;
  p.conv = static_cast<char*>(pool->d.conv_base) + (uint64_t)layer * pool->d.num_slots * pool->conv_slot_bytes;
  p.num_slots = pool->d.num_slots;
  p.ssm_bf16 = pool->d.ssm_dtype == M2_BF16;
  p.conv_bf16 = pool->d.conv_dtype == M2_BF16;
  p.io_bf16 = io_dtype == M2_BF16;
  p.y_bf16 = y_dtype == M2_BF16;
  p.D = D;
  p.x_stride = x_stride;
  p.B_stride = B_stride;
  p.C_stride = C_stride;
  p.z_stride = z_stride;
  p.dt_stride = dt_stride;
  p.y_stride = y_stride;
  p.A = params->A;
  p.Dk = params->D;
  p.dt_bias = params->dt_bias;
  p.conv_w = params->conv_w;
  p.conv_b = params->conv_b;
  const int kMaxRows = 65535;   // grid.y limit
  for (int r0 = 0; r0 < batch; r0 += kMaxRows) {
    const int nb = batch - r0 < kMaxRows ? batch - r0 : kMaxRows;
    p.slots = slots + r0;
    p.x = static_cast<const char*>(x) + (int64_t)r0 * x_stride * ies;
    p.B = static_cast<const char*>(B) + (int64_t)r0 * B_stride * ies;
    p.C = static_cast<const char*>(C) + (int64_t)r0 * C_stride * ies;
    p.z = static_cast<const char*>(z) + (int64_t)r0 * z_stride * ies;
    p.dt = static_cast<const char*>(dt) + (int64_t)r0 * dt_stride * ies;
    p.y = static_cast<char*>(y) + (int64_t)r0 * y_stride * esize(y_dtype);
    const hipError_t e = m2::launch_mamba1_decode(p, sh.N, sh.W, nb, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "Mamba1 decode launch");
  }
  return ok();
}

// Rows per chunk when the caller leaves the choice to the library (chunk_size 0).  A chunk costs
// its rows once more in launch (1) unless it is its sequence's last, so sequences stay whole
// (about total/num_seqs rows per chunk, which also splits the longest ones of a ragged batch) as
// long as they give the chunk kernels kM1MinWgs workgroups; fewer sequences are cut into chunks
// until the chunks give kM1FillWgs.  Workgroups per chunk: ceil(D / channels per workgroup), 256
// threads over channels of N/4 lanes.  The rule depends on the shapes only, not on the device, so
// a batch is chunked (and rounded) the same way everywhere.
constexpr int64_t kM1MinWgs = 512, kM1FillWgs = 1024;
int64_t m1_auto_target(const m2::LayerShape& sh, int64_t num_seqs) {   // chunks aimed at
  const int64_t cpw = 256 / (sh.N / 4);
  const int64_t wgs = (sh.H + cpw - 1) / cpw;
  const int64_t chunks = num_seqs * wgs < kM1MinWgs ? (kM1FillWgs + wgs - 1) / wgs : num_seqs;
  return chunks < 1 ? 1 : chunks;
}
int64_t m1_auto_chunk(const m2::LayerShape& sh, int64_t num_seqs, int64_t total_tokens) {
  const int64_t chunks = m1_auto_target(sh, num_seqs);
  int64_t q = (total_tokens + chunks - 1) / chunks;
  q = (q + 15) / 16 * 16;
  return q < 16 ? 16 : q;
}

m2_status mamba1_prefill_workspace_size(const m2_pool* pool, int32_t num_seqs, int32_t total_tokens,
                                        int32_t chunk_size, int32_t max_ckpt, uint64_t* bytes) {
  if (!pool || !bytes) return fail(M2_ERR_ARG, "NULL argument");
  if (m2_status st = require_family(pool, M2_FAMILY_MAMBA1, "mamba1_prefill_workspace_size")) return st;
  if (num_seqs < 0 || total_tokens < 0 || max_ckpt < 0) return fail(M2_ERR_ARG, "negative count");
  if (chunk_size != 0 && (chunk_size < 16 || chunk_size > 4096))
    return fail(M2_ERR_UNSUPPORTED, "chunk_size must be 0 or in [16, 4096]");
  if (!m2::mamba1_supported(pool->sh.N, pool->sh.W))
    return fail(M2_ERR_UNSUPPORTED, "Mamba1 prefill supports d_state in {8,16,32,64,128,256}, got %d", pool->sh.N);
  // chunks: sum over sequences of ceil(len / q) <= floor(total / q) + num_seqs.  With the library's
  // choice floor(T / q) <= min(T / 16, target) for every T <= total_tokens, so a workspace sized
  // for a bound on the rows also serves any smaller batch of the same sequence count.
  const int64_t nfull = chunk_size ? (int64_t)total_tokens / chunk_size
                                   : std::min<int64_t>((int64_t)total_tokens / 16, m1_auto_target(pool->sh, num_seqs));
  M1Layout L;
  if (!m1_layout(pool->sh, num_seqs, nfull + num_seqs, (int64_t)num_seqs * max_ckpt, &L))
    return fail(M2_ERR_SHAPE, "workspace size overflows 64 bits");
  *bytes = L.total;
  return ok();
}

m2_status mamba1_prefill(m2_pool* pool, int32_t layer, const m2_layer_params* params, int32_t num_seqs,
                         const int32_t* cu_seqlens, const int32_t* slots, const uint8_t* has_init,
                         const int32_t* start_pos, const void* x, int64_t x_stride, const void* B, int64_t B_stride,
                         const void* C, int64_t C_stride, const void* z, int64_t z_stride, const void* dt,
                         int64_t dt_stride, int32_t io_dtype, void* y, int64_t y_stride, int32_t y_dtype,
                         int32_t chunk_size, int32_t ckpt_interval, const int32_t* ckpt_slots, int32_t max_ckpt,
                         void* workspace, uint64_t workspace_bytes, void* stream) {
  if (!pool) return fail(M2_ERR_ARG, "pool is NULL");
  if (m2_status st = require_family(pool, M2_FAMILY_MAMBA1, "mamba1_prefill")) return st;
  const m2::LayerShape& sh = pool->sh;
  if (layer < 0 || layer >= pool->d.num_layers) return fail(M2_ERR_ARG, "layer %d out of range", layer);
  if (num_seqs < 0) return fail(M2_ERR_ARG, "num_seqs is negative");
  if (m2_status st = check_params(pool, params)) return st;
  if (!dtype_ok(io_dtype) || !dtype_ok(y_dtype)) return fail(M2_ERR_DTYPE, "io/y dtype must be F32 or BF16");
  if (chunk_size != 0 && (chunk_size < 16 || chunk_size > 4096))
    return fail(M2_ERR_UNSUPPORTED, "chunk_size must be 0 or in [16, 4096]");
  if (ckpt_interval < 0 || max_ckpt < 0) return fail(M2_ERR_ARG, "negative checkpoint interval or count");
  if (num_seqs == 0) return ok();
  if (!cu_seqlens || !slots || !has_init) return fail(M2_ERR_ARG, "cu_seqlens, slots and has_initial_state are required");
  if (cu_seqlens[0] != 0) return fail(M2_ERR_SHAPE, "cu_seqlens[0] must be 0");
  for (int s = 0; s < num_seqs; ++s)
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return fail(M2_ERR_SHAPE, "cu_seqlens decreases at %d", s);
  const int64_t T = cu_seqlens[num_seqs];
  const bool ckpt_on = ckpt_interval > 0 && max_ckpt > 0;
  if (ckpt_on && !ckpt_slots) return fail(M2_ERR_ARG, "ckpt_slots is NULL");
  const int S = pool->d.num_slots;
  std::vector<uint8_t> used(S, 0);
  for (int s = 0; s < num_seqs; ++s) {
    const int sl = slots[s];
    if (sl < 0 || sl >= S) return fail(M2_ERR_SLOT, "slot %d of sequence %d out of range", sl, s);
    if (used[sl]) return fail(M2_ERR_SLOT, "slot %d appears twice", sl);
    used[sl] = 1;
    if (start_pos && start_pos[s] < 0) return fail(M2_ERR_ARG, "start_pos of sequence %d is negative", s);
  }
  if (ckpt_on) {
    for (int64_t i = 0; i < (int64_t)num_seqs * max_ckpt; ++i) {
      const int sl = ckpt_slots[i];
      if (sl == -1) continue;
      if (sl < 0 || sl >= S) return fail(M2_ERR_SLOT, "checkpoint slot %d out of range", sl);
      if (used[sl]) return fail(M2_ERR_SLOT, "checkpoint slot %d repeats or aliases a sequence slot", sl);
      used[sl] = 1;
    }
  }
  if (T == 0) return ok();
  const int ies = esize(io_dtype);
  const int D = sh.H;
  const IoCheck io[] = {{"x", x, x_stride, D, ies, false},      {"B", B, B_stride, sh.N, ies, true},
                        {"C", C, C_stride, sh.N, ies, true},    {"z", z, z_stride, D, ies, false},
                        {"dt", dt, dt_stride, D, ies, false},   {"y", y, y_stride, D, esize(y_dtype), false}};
  if (m2_status st = check_io(io, 6)) return st;
  if (!m2::mamba1_supported(sh.N, sh.W))
    return fail(M2_ERR_UNSUPPORTED, "Mamba1 prefill supports d_state in {8,16,32,64,128,256}, got %d", sh.N);
  // tables: chunks of q rows from each sequence's first row
  const int64_t q = chunk_size ? chunk_size : m1_auto_chunk(sh, num_seqs, T);
  std::vector<m2::M1Seq> seqs(num_seqs);
  std::vector<m2::M1Chunk> chunks;
  for (int s = 0; s < num_seqs; ++s) {
    const int t0 = cu_seqlens[s], len = cu_seqlens[s + 1] - t0;
    seqs[s] = m2::M1Seq{t0, len, slots[s], has_init[s] ? 1 : 0, start_pos ? start_pos[s] : 0,
                        s * (ckpt_on ? max_ckpt : 0), ckpt_on ? max_ckpt : 0, (int32_t)chunks.size()};
    for (int64_t c0 = 0; c0 < len; c0 += q)
      chunks.push_back(m2::M1Chunk{s, t0 + (int)c0, (int)(len - c0 < q ? len - c0 : q), (int)c0});
  }
  if (chunks.size() > 65535 || num_seqs > 65535)
    return fail(M2_ERR_UNSUPPORTED, "%zu chunks and %d sequences: at most 65535 of each (raise chunk_size)",
                chunks.size(), num_seqs);
  const int64_t nck = ckpt_on ? (int64_t)num_seqs * max_ckpt : 0;
  M1Layout L;
  if (!m1_layout(sh, num_seqs, (int64_t)chunks.size(), nck, &L)) return fail(M2_ERR_SHAPE, "workspace size overflows");
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(M2_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(M2_ERR_WORKSPACE, "workspace has %llu bytes, needs %llu", (unsigned long long)workspace_bytes,
                (unsigned long long)L.total);
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  {
    std::vector<char> t(L.tab_bytes, 0);
    memcpy(t.data(), seqs.data(), seqs.size() * sizeof(m2::M1Seq));
    memcpy(t.data() + L.off_chunks, chunks.data(), chunks.size() * sizeof(m2::M1Chunk));
    if (nck) memcpy(t.data() + L.off_ck, ckpt_slots, (size_t)nck * 4);
    const hipError_t eu = m2::launch_table_upload(ws, t.data(), L.tab_bytes, hs);
    if (eu != hipSuccess) return hip_fail(eu, "table upload");
  }
  m2::Mamba1PrefillParams p;
  p.ssm = static_cast<char*>(pool->d.ssm_base) + (uint64_t)layer * pool->d.num_slots * pool->ssm_slot_bytes;
  p.conv = static_cast<char*>(pool->d.conv_base) + (uint64_t)layer * pool->d.num_slots * pool->conv_slot_bytes;
  p.num_slots = S;
  p.ssm_bf16 = pool->d.ssm_dtype == M2_BF16;
  p.conv_bf16 = pool->d.conv_dtype == M2_BF16;
  p.io_bf16 = io_dtype == M2_BF16;
  p.y_bf16 = y_dtype == M2_BF16;
  p.D = D;
  p.x = x;
  p.B = B;
  p.C = C;
  p.z = z;
  p.dt = dt;
  p.x_stride = x_stride;
  p.B_stride = B_stride;
  p.C_stride = C_stride;
  p.z_stride = z_stride;
  p.dt_stride = dt_stride;
  p.y = y;
  p.y_stride = y_stride;
  p.A = params->A;
  p.Dk = params->D;
  p.dt_bias = params->dt_bias;
  p.conv_w = params->conv_w;
  p.conv_b = params->conv_b;
  p.num_seqs = num_seqs;
  p.num_chunks = (int)chunks.size();
  p.ckpt_interval = ckpt_on ? ckpt_interval : 0;
  int nonempty = 0;
  for (int s = 0; s < num_seqs; ++s) nonempty += seqs[s].len > 0;
  p.whole_seqs = (int)chunks.size() == nonempty;
  p.seqs = reinterpret_cast<const m2::M1Seq*>(ws);
  p.chunks = reinterpret_cast<const m2::M1Chunk*>(ws + L.off_chunks);
  p.ck = reinterpret_cast<const int32_t*>(ws + L.off_ck);
  p.S = reinterpret_cast<float*>(ws + L.off_S);
  p.SD = reinterpret_cast<float*>(ws + L.off_SD);
  p.Hin = reinterpret_cast<float*>(ws + L.off_Hin);
  p.Win0 = reinterpret_cast<float*>(ws + L.off_W0);
  const hipError_t e = m2::launch_mamba1_prefill(p, sh.N, sh.W, hs);
  if (e != hipSuccess) return hip_fail(e, "Mamba1 prefill launch");
  return ok();
}

}  // extern "C"
