// C ABI of libattn: argument checks, workspace sizing, launch planning and the kernel
// launches, all on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/attn.h"
#include "kernel_args.h"

namespace {

thread_local int g_last_hip_error = 0;

// Debug mode (attn_debug(1), or ATTN_DEBUG=1 in the environment at the first call): calls with
// device-resident metadata check it first, synchronously, and return ATTN_ERR_INVALID_ARG
// instead of launching anything when it is inconsistent.
std::atomic<int> g_debug{-1};

bool debug_on() {
  int d = g_debug.load(std::memory_order_relaxed);
  if (d < 0) {
    const char* e = std::getenv("ATTN_DEBUG");
    d = (e != nullptr && e[0] != '\0' && e[0] != '0') ? 1 : 0;
    int expect = -1;
    g_debug.compare_exchange_strong(expect, d);
    d = g_debug.load(std::memory_order_relaxed);
  }
  return d > 0;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool stride_ok(int64_t s) { return s >= 0 && s % 8 == 0; }

attn_status check_tensor(const attn_tensor& t, bool packed) {
  if (t.ptr == nullptr || !aligned16(t.ptr)) return ATTN_ERR_INVALID_ARG;
  if (!stride_ok(t.stride_s) || !stride_ok(t.stride_h)) return ATTN_ERR_INVALID_ARG;
  if (!packed && !stride_ok(t.stride_b)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// 16-bit tensor types
bool dtype16_ok(int dt) { return dt == ATTN_DTYPE_BF16 || dt == ATTN_DTYPE_F16; }

// varlen: 0 dense, 1 pad_mask, 2 cu_seqlens
attn_status check_shape(const attn_shape* s, int varlen) {
  if (s == nullptr) return ATTN_ERR_INVALID_ARG;
  if (s->B < 0 || s->S < 0 || s->Hq <= 0 || s->Hkv <= 0 || s->total < 0) return ATTN_ERR_INVALID_ARG;
  if (s->Hq % s->Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (s->D != 256 && s->D != 512) return ATTN_ERR_UNSUPPORTED;
  if (!dtype16_ok(s->dtype)) return ATTN_ERR_UNSUPPORTED;
  // every row index handled as a 32-bit int inside the kernels
  const int64_t rows = varlen == 2 ? (int64_t)s->total : (int64_t)s->B * s->S;
  if (rows * s->Hq >= INT_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// varlen metadata: per-sequence offset, length, and the batch order by decreasing length
size_t meta_bytes(int B, int varlen) { return varlen ? round_up(3 * sizeof(int32_t) * (size_t)B) : 0; }

// Workgroups per XCD for `total` items of W per unit: with a batch order (see xcd_item) each
// XCD takes whole units, ceil(units / 8) of them.  Fewer than 8 units would leave XCDs idle
// either that way or dealt by units, so they take the dense mapping instead: each XCD a
// contiguous run of items, a unit split over neighbouring XCDs.
int per_xcd_for(attn::AttnArgs& a, int total, int W) {
  if (a.balanced && total / W < 8) {
    a.order = nullptr;
    a.balanced = 0;
  }
  return a.order != nullptr ? ((total / W + 7) / 8) * W : (total + 7) / 8;
}

int varlen_kind(const int32_t* cu, const uint8_t* mask) { return cu ? 2 : (mask ? 1 : 0); }

attn_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  g_last_hip_error = (int)e;
  return ATTN_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Optional per-kernel timing (attn_profile): HIP event pairs around each launch.
// ---------------------------------------------------------------------------
struct TimedLaunch {
  const char* name;
  hipEvent_t start, stop;
};
struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> pool;   // created lazily, reused
  size_t used = 0;
  std::vector<TimedLaunch> launches;
};
thread_local Profiler g_prof;

// attn_count_restarts: device counter the forward kernels add their key-loop restarts to.
thread_local int* g_restarts = nullptr;
constexpr size_t kMaxTimed = 4096;

hipEvent_t prof_event() {
  if (g_prof.used == g_prof.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_prof.pool.push_back(e);
  }
  return g_prof.pool[g_prof.used++];
}

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_prof.on || g_prof.launches.size() >= kMaxTimed) return launch();
  hipEvent_t a = prof_event(), b = prof_event();
  if (!a || !b) return launch();
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  g_prof.launches.push_back({name, a, b});
  return hipSuccess;
}

// Query heads packed per workgroup: the largest power of two dividing r, capped so a
// tile still spans at least 16 positions.
int heads_per_tile(int r, int rows) {
  int hpt = 1;
  while (hpt * 2 <= 8 && r % (hpt * 2) == 0 && rows / (hpt * 2) >= 16) hpt *= 2;
  return hpt;
}

void plan_rows(attn::AttnArgs& a, int rows) {
  a.hpt = heads_per_tile(a.r, rows);
  a.mpos = rows / a.hpt;
  a.nhb = a.r / a.hpt;
  a.nqt = (a.S + a.mpos - 1) / a.mpos;
  a.total_items = a.B * a.Hkv * a.nhb * a.nqt;
  a.per_xcd = per_xcd_for(a, a.total_items, a.nqt);
}

// One forward or backward call, whole sequences or a chunk pair, after argument checks.
struct Call {
  int B, S, Sk, total, Hq, Hkv, D;
  int varlen;          // 0 dense, 1 pad_mask, 2 cu_seqlens
  int f16;             // 16-bit tensors are IEEE half
  int causal, window;  // window normalised (see normalise_offsets)
  int shift;           // query position offset of the chunk pair; 0 for whole sequences
  int empty_lse_ninf;  // chunk pairs: a row with no visible key has LSE = -inf
  float softcap;       // tanh cap of the scaled scores; 0: none
};

// Visibility of (query i, key j) depends only on d = i + delta - j, the distance of their
// positions, over i < S and j < Sk: visible when d >= 0 (causal) and d < window (window > 0).
// This rewrites (delta, window) into an equivalent pair with delta in [-S, Sk] and window in
// [0, S + Sk - 1], so that every position sum inside the kernels fits in 32 bits.
void normalise_offsets(Call& c, int64_t delta) {
  if (!c.causal) {  // every pair is visible; positions do not matter
    c.shift = 0;
    c.window = 0;
    return;
  }
  const int64_t dmax = delta + c.S - 1, dmin = delta - (c.Sk - 1);
  int64_t w = c.window;
  if (dmax < 0 || (w > 0 && dmin >= w)) {  // no visible pair: every query sits before every key
    c.shift = -c.S;
    c.window = 0;
    return;
  }
  if (w > dmax) w = 0;  // the window never binds
  if (w == 0) {
    c.shift = (int)std::min<int64_t>(delta, c.Sk);  // delta >= 1 - S here
    c.window = 0;
  } else if (delta >= c.Sk - 1) {
    // the causal bound never binds; only delta - window matters
    const int64_t e = delta - w;  // in [1 - S, Sk - 2]
    c.shift = c.Sk;
    c.window = (int)(c.Sk - e);
  } else {
    c.shift = (int)delta;  // in [1 - S, Sk - 2]
    c.window = (int)w;     // at most dmax < S + Sk
  }
}

void fill_common(attn::AttnArgs& a, const Call& c, float scale, const int32_t* meta) {
  a.B = c.B;
  a.S = c.S;
  a.Sk = c.Sk;
  a.q_shift = c.shift;
  a.empty_lse_ninf = c.empty_lse_ninf;
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.r = c.Hq / c.Hkv;
  a.packed = c.varlen == 2;
  a.f16 = c.f16;
  a.causal = c.causal;
  a.window = c.window;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  a.softcap = c.softcap;
  a.sc_in = c.softcap > 0.f ? scale / c.softcap : 0.f;
  a.sc_out = c.softcap > 0.f ? c.softcap / scale : 0.f;
  a.seq_off = c.varlen ? meta : nullptr;
  a.seq_len = c.varlen ? meta + c.B : nullptr;
  a.balanced = c.varlen != 0;  // sequences of different lengths: see xcd_item
  a.order = (c.varlen && c.B <= attn::kOrderMaxBatch) ? meta + 2 * c.B : nullptr;
  if (a.packed) {
    a.st_sb = 0;
    a.st_sh = c.total;
  } else {
    a.st_sh = c.S;
    a.st_sb = (int64_t)c.Hq * c.S;
  }
}

void set_tensor(const attn_tensor& t, bool packed, int64_t& sb, int64_t& ss, int64_t& sh) {
  sb = packed ? 0 : t.stride_b;
  ss = t.stride_s;
  sh = t.stride_h;
}

attn_status check_common(const attn_shape* shape, float scale, int causal, int window, const int32_t* cu,
                         const uint8_t* mask, size_t ws_bytes, size_t need, const void* ws) {
  if (cu && mask) return ATTN_ERR_INVALID_ARG;
  attn_status st = check_shape(shape, varlen_kind(cu, mask));
  if (st != ATTN_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (window < 0) return ATTN_ERR_INVALID_ARG;
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (need > 0 && (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))))
    return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

// dS block layout of the backward (see ds_block_index): triangular for causal attention
// of whole sequences without a window, else a fixed number of blocks per 128-row query tile
// (every key block for a chunk pair without a window).
struct DsLayout {
  int tri, cnt;
  int64_t per_head;  // blocks per (batch, query head)
};

DsLayout ds_layout(const Call& c) {
  const int nqt = (c.S + attn::kDsRows - 1) / attn::kDsRows;
  const int nkb = (c.Sk + attn::kDsKeys - 1) / attn::kDsKeys;
  DsLayout L;
  if (c.causal && c.shift <= -c.S) {  // no visible pair (see normalise_offsets)
    L.tri = 0;
    L.cnt = 0;
    L.per_head = 0;
  } else if (c.causal && c.window <= 0 && c.shift == 0 && c.Sk == c.S) {
    L.tri = 1;
    L.cnt = 0;
    L.per_head = 2LL * nqt * (nqt + 1);
  } else {
    // a tile's visible key blocks span at most (window + 254) / 32 + 2 <= (window + 127) / 32 + 6 blocks
    L.tri = 0;
    L.cnt = (c.causal && c.window > 0) ? std::min(nkb, (c.window + attn::kDsRows - 1) / attn::kDsKeys + 6) : nkb;
    L.per_head = (int64_t)nqt * L.cnt;
  }
  return L;
}

// Packed rows (cu_seqlens) give each sequence a dS region sized by its own length
// (ds_head_blocks), placed by a prefix sum on the device; batches past kOrderMaxBatch keep one
// region of the longest sequence's size per (sequence, head).
bool ds_per_sequence(const Call& c) { return c.varlen == 2 && c.B <= attn::kOrderMaxBatch; }

size_t ds_seq_bytes(const Call& c) { return ds_per_sequence(c) ? round_up(sizeof(int64_t) * (size_t)c.B) : 0; }

// dS blocks of the whole call.  Per sequence: with n_b = ceil(len_b / 128) query tiles,
// sum_b n_b <= min(B nqt, floor(total / 128) + B) =: N and n_b <= nqt, so the triangular layout
// needs at most 2 N (nqt + 1) blocks per head and the others N cnt.
int64_t ds_blocks(const Call& c) {
  const DsLayout L = ds_layout(c);
  if (!ds_per_sequence(c)) return (int64_t)c.B * c.Hq * L.per_head;
  const int64_t nqt = (c.S + attn::kDsRows - 1) / attn::kDsRows;
  const int64_t N = std::min<int64_t>((int64_t)c.B * nqt, c.total / attn::kDsRows + c.B);
  return (int64_t)c.Hq * (L.tri ? 2 * N * (nqt + 1) : N * L.cnt);
}

size_t ds_bytes(const Call& c) {
  return round_up((size_t)ds_blocks(c) * attn::kDsBlockElems * sizeof(__bf16));
}

// Largest backward workspace: the dS blocks grow with the square of the sequence length (about
// B Hq S^2 bytes for causal attention).  Past this a whole-sequence backward is refused
// (ATTN_ERR_UNSUPPORTED); chunk pairs (attn_bwd_chunk) bound the workspace by the chunk sizes.
constexpr size_t kMaxBwdWorkspace = size_t(1) << 37;  // 128 GiB of the GPU's 288 GB

size_t stat_bytes(const Call& c) {
  return round_up(sizeof(float) * (size_t)c.Hq * (c.varlen == 2 ? (size_t)c.total : (size_t)c.B * c.S));
}

// The dK/dV pass has one workgroup per 64-key tile of each (batch, kv head); with fewer tiles
// than compute units (short dense sequences, chunk pairs of a ring) each tile's query heads are
// split over 2 or 4 workgroups, whose fp32 partial sums a reduction adds in a fixed order.
constexpr int kComputeUnits = 256;  // MI355X

int kv_split_for(const Call& c) {
  if (c.varlen != 0) return 1;
  const int64_t items = (int64_t)c.B * c.Hkv * ((c.Sk + attn::kDkdvKeys - 1) / attn::kDkdvKeys);
  const int r = c.Hq / c.Hkv;
  int split = 1;
  while (split < 4 && items * split < kComputeUnits && r % (2 * split) == 0) split *= 2;
  return split;
}

size_t kv_part_bytes(const Call& c) {
  const int split = kv_split_for(c);
  return split > 1 ? round_up(sizeof(float) * 2 * split * (size_t)c.B * c.Sk * c.Hkv * c.D) : 0;
}

size_t bwd_bytes(const Call& c) {
  return meta_bytes(c.B, c.varlen) + ds_seq_bytes(c) + stat_bytes(c) + ds_bytes(c) + kv_part_bytes(c);
}

Call whole_call(const attn_shape* s, int varlen, int causal, int window) {
  Call c = {};
  c.B = s->B;
  c.S = s->S;
  c.Sk = s->S;
  c.total = s->total;
  c.Hq = s->Hq;
  c.Hkv = s->Hkv;
  c.D = s->D;
  c.varlen = varlen;
  c.f16 = s->dtype == ATTN_DTYPE_F16;
  c.causal = causal ? 1 : 0;
  c.window = window;
  normalise_offsets(c, 0);
  return c;
}

// Chunk pairs: dense (B, Sq | Sk, H, D) tensors.
attn_status check_chunk(const attn_chunk_shape* s, int causal, int window, int64_t q_pos0, int64_t k_pos0) {
  if (s == nullptr) return ATTN_ERR_INVALID_ARG;
  if (s->B < 0 || s->Sq < 0 || s->Sk < 0 || s->Hq <= 0 || s->Hkv <= 0) return ATTN_ERR_INVALID_ARG;
  if (s->Hq % s->Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (window < 0 || q_pos0 < 0 || k_pos0 < 0 || q_pos0 > (INT64_MAX >> 2) || k_pos0 > (INT64_MAX >> 2))
    return ATTN_ERR_INVALID_ARG;
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (s->D != 256 && s->D != 512) return ATTN_ERR_UNSUPPORTED;
  if (!dtype16_ok(s->dtype)) return ATTN_ERR_UNSUPPORTED;
  if (s->Sq >= (1 << 28) || s->Sk >= (1 << 28)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)s->B * s->Sq * s->Hq >= INT_MAX / 2 || (int64_t)s->B * s->Sk * s->Hkv >= INT_MAX / 2)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

Call chunk_call(const attn_chunk_shape* s, int causal, int window, int64_t q_pos0, int64_t k_pos0) {
  Call c = {};
  c.B = s->B;
  c.S = s->Sq;
  c.Sk = s->Sk;
  c.total = 0;
  c.Hq = s->Hq;
  c.Hkv = s->Hkv;
  c.D = s->D;
  c.varlen = 0;
  c.f16 = s->dtype == ATTN_DTYPE_F16;
  c.causal = causal ? 1 : 0;
  c.window = window;
  c.empty_lse_ninf = 1;
  normalise_offsets(c, q_pos0 - k_pos0);
  return c;
}

// Launches one kernel unless its grid is empty.
template <class F>
attn_status launch(const char* name, hipStream_t s, int items, F&& f) {
  if (items <= 0) return ATTN_OK;
  return hip_status(timed(name, s, f));
}

struct Tensors {
  attn_tensor q, k, v, o, dout, dq, dk, dv;
};

void set_tensors(attn::AttnArgs& a, const Tensors& t, bool packed, bool bwd) {
  a.q = static_cast<const __bf16*>(t.q.ptr);
  a.k = static_cast<const __bf16*>(t.k.ptr);
  a.v = static_cast<const __bf16*>(t.v.ptr);
  set_tensor(t.q, packed, a.q_sb, a.q_ss, a.q_sh);
  set_tensor(t.k, packed, a.k_sb, a.k_ss, a.k_sh);
  set_tensor(t.v, packed, a.v_sb, a.v_ss, a.v_sh);
  set_tensor(t.o, packed, a.o_sb, a.o_ss, a.o_sh);
  if (!bwd) {
    a.out = static_cast<__bf16*>(t.o.ptr);
    return;
  }
  a.o = static_cast<const __bf16*>(t.o.ptr);
  a.dout = static_cast<const __bf16*>(t.dout.ptr);
  a.out = static_cast<__bf16*>(t.dq.ptr);
  a.dk = static_cast<__bf16*>(t.dk.ptr);
  a.dv = static_cast<__bf16*>(t.dv.ptr);
  set_tensor(t.dout, packed, a.do_sb, a.do_ss, a.do_sh);
  set_tensor(t.dq, packed, a.dq_sb, a.dq_ss, a.dq_sh);
  set_tensor(t.dk, packed, a.dk_sb, a.dk_ss, a.dk_sh);
  set_tensor(t.dv, packed, a.dv_sb, a.dv_ss, a.dv_sh);
}

attn_status debug_check_varlen(const Call& c, const int32_t* cu_seqlens, const uint8_t* pad_mask, hipStream_t s) {
  if (!c.varlen || !debug_on()) return ATTN_OK;
  bool bad = false;
  attn_status st = hip_status(attn::check_varlen_meta(pad_mask, cu_seqlens, c.B, c.S, c.total, s, bad));
  if (st != ATTN_OK) return st;
  return bad ? ATTN_ERR_INVALID_ARG : ATTN_OK;
}

attn_status debug_check_pages(const attn_decode_shape& sh, const int32_t* table, const int32_t* ctx, hipStream_t s,
                              int contiguous = 0) {
  if (!debug_on()) return ATTN_OK;
  bool bad = false;
  attn_status st = hip_status(attn::check_pages_meta(table, contiguous, ctx, sh.B, sh.max_pages_per_seq, sh.page_size,
                                                     sh.num_pages, s, bad));
  if (st != ATTN_OK) return st;
  return bad ? ATTN_ERR_INVALID_ARG : ATTN_OK;
}

// Per-sequence offsets and lengths, then the batch order the work items are dealt by.
attn_status varlen_meta(const Call& c, const int32_t* cu_seqlens, const uint8_t* pad_mask, int32_t* meta,
                        hipStream_t s) {
  if (!c.varlen) return ATTN_OK;
  attn_status st = launch("varlen_prep", s, c.B, [&] {
    return attn::launch_varlen_prep(pad_mask, cu_seqlens, c.B, c.S, c.total, meta, meta + c.B, s);
  });
  if (st || c.B > attn::kOrderMaxBatch) return st;
  return launch("varlen_order", s, c.B,
                [&] { return attn::launch_varlen_order(meta + c.B, c.B, meta + 2 * c.B, s); });
}

// Where the forward puts its result: O in the inputs' 16-bit type, O in fp32 (a chunk partial),
// or merged into a running fp32 (O, LSE) with an optional 16-bit copy of the merged O.
enum class FwdOut { half, f32, merge };

// K and V of a paged forward: the caches' page strides and the table that places each
// sequence's pages (the tensors' own pointers, slot and head strides are in Tensors).
struct PagedKV {
  const int32_t* table;
  const int32_t* kv_len;
  int64_t k_page, v_page;
  int max_pages, num_pages;
};

attn_status run_fwd(const Call& c, const Tensors& t, float scale, float* lse, const int32_t* cu_seqlens,
                    const uint8_t* pad_mask, void* workspace, hipStream_t s, FwdOut mode = FwdOut::half,
                    attn_tensor final16 = {}, const PagedKV* paged = nullptr, float* split_ws = nullptr) {
  int32_t* meta = static_cast<int32_t*>(workspace);
  attn_status st;
  if ((st = debug_check_varlen(c, cu_seqlens, pad_mask, s))) return st;
  // the paged forward reads its query offsets (cu_seqlens) directly
  if (paged == nullptr && (st = varlen_meta(c, cu_seqlens, pad_mask, meta, s))) return st;
  attn::AttnArgs a = {};
  fill_common(a, c, scale, meta);
  set_tensors(a, t, c.varlen == 2, false);
  if (mode != FwdOut::half) {
    a.out = nullptr;
    a.out_f32 = static_cast<float*>(t.o.ptr);
  }
  if (mode == FwdOut::merge) {
    a.merge = 1;
    a.out = static_cast<__bf16*>(final16.ptr);
    set_tensor(final16, false, a.r_sb, a.r_ss, a.r_sh);
  }
  if (paged != nullptr) {
    a.seq_off = cu_seqlens;
    a.seq_len = nullptr;
    a.total = c.total;
    // A sequence's cost grows with its cached keys, not its query rows, so its items are dealt
    // round-robin over all units rather than in a batch order by length (see xcd_item).
    a.order = nullptr;
    a.paged = 1;
    a.table = paged->table;
    a.kv_len = paged->kv_len;
    a.k_sb = paged->k_page;
    a.v_sb = paged->v_page;
    a.max_pages = paged->max_pages;
    a.num_pages = paged->num_pages;
  }
  a.lse = lse;
  a.restarts = g_restarts;
  plan_rows(a, attn::kFwdRows);
  // Decode rows are split only while the batch's units leave compute units without a workgroup
  // (with one per compute unit a row's single workgroup already streams its keys at the memory's
  // pace, and its pieces would add their start-up and a merge), and only when a sequence can have
  // one new token (it cannot when every sequence has max_q > 1 of them).
  if (split_ws != nullptr && ((int64_t)a.B * a.Hkv * a.nhb >= kComputeUnits ||
                              (c.S > 1 && c.total == c.B * c.S)))
    split_ws = nullptr;
  if (paged != nullptr && split_ws != nullptr) {
    // split decode rows: kSplitMax more items per unit, after every query tile's, hold the pieces;
    // the sequences are ranked by work on the device for the deal (paged_split_item)
    const int U = a.B * a.Hkv * a.nhb;
    a.split_slot0 = a.nqt;
    a.nqt += attn::kSplitMax;
    a.total_items = U * a.nqt;
    a.split_o = split_ws;
    a.split_lse = split_ws + (int64_t)a.B * a.Hq * attn::kSplitMax * c.D;
    int32_t* order = reinterpret_cast<int32_t*>(split_ws + (int64_t)a.B * a.Hq * attn::kSplitMax * (c.D + 1));
    const int blocks = U * ((a.split_slot0 + 31) / 32);
    a.split_nA = 8 * ((blocks + 7) / 8) * 32;
    a.per_xcd = (a.split_nA + U * attn::kSplitMax) / 8;
    a.balanced = 0;
    a.order = order;
    attn_status st1 = launch("paged_rank", s, a.B, [&] {
      return attn::launch_paged_rank(cu_seqlens, paged->kv_len, a.B, a.total, c.S, paged->max_pages * 16, order, s);
    });
    if (st1 != ATTN_OK) return st1;
  }
  attn_status st2 = launch(paged ? "attn_fwd_paged" : mode == FwdOut::merge ? "attn_fwd_merge" : "attn_fwd", s,
                           a.total_items, [&] { return attn::launch_fwd(a, c.D, s); });
  if (st2 != ATTN_OK || a.split_o == nullptr) return st2;
  return launch("attn_fwd_split_merge", s, a.B * a.Hq, [&] { return attn::launch_fwd_split_merge(a, c.D, s); });
}

attn_status run_bwd(const Call& c, const Tensors& t, float scale, const float* lse, const int32_t* cu_seqlens,
                    const uint8_t* pad_mask, void* workspace, hipStream_t s, bool grad_f32 = false) {
  // adding the parts of a pair that has no visible (query, key) pair changes nothing
  if (grad_f32 && c.causal && c.shift <= -c.S) return ATTN_OK;
  int32_t* meta = static_cast<int32_t*>(workspace);
  int64_t* ds_seq = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + meta_bytes(c.B, c.varlen));
  float* delta = reinterpret_cast<float*>(reinterpret_cast<char*>(ds_seq) + ds_seq_bytes(c));
  attn_status st;
  if ((st = debug_check_varlen(c, cu_seqlens, pad_mask, s))) return st;
  if ((st = varlen_meta(c, cu_seqlens, pad_mask, meta, s))) return st;
  const DsLayout L = ds_layout(c);
  if (ds_per_sequence(c) &&
      (st = launch("ds_seq_base", s, c.B, [&] {
         return attn::launch_ds_seq_base(meta + c.B, c.B, c.Hq, L.tri, L.cnt, ds_blocks(c), ds_seq, s);
       })))
    return st;
  attn::AttnArgs a = {};
  fill_common(a, c, scale, meta);
  set_tensors(a, t, c.varlen == 2, true);
  if (grad_f32) {
    a.out = a.dk = a.dv = nullptr;
    a.dq_f32 = static_cast<float*>(t.dq.ptr);
    a.dk_f32 = static_cast<float*>(t.dk.ptr);
    a.dv_f32 = static_cast<float*>(t.dv.ptr);
  }
  a.lse = const_cast<float*>(lse);
  a.delta = delta;
  {
    a.ds_seq = ds_per_sequence(c) ? ds_seq : nullptr;
    a.dsb = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(delta) + stat_bytes(c));
    a.ds_head = L.per_head;
    a.ds_tri = L.tri;
    a.ds_cnt = L.cnt;
  }

  const int rows = (c.varlen == 2 ? c.total : c.B * c.S) * c.Hq;
  if ((st = launch("bwd_pre", s, rows, [&] { return attn::launch_bwd_pre(a, c.D, rows, s); }))) return st;

  attn::AttnArgs kv = a;
  kv.nkt = (c.Sk + attn::kDkdvKeys - 1) / attn::kDkdvKeys;
  kv.kv_split = kv_split_for(c);
  kv.kv_part = kv.kv_split > 1 ? reinterpret_cast<float*>(reinterpret_cast<char*>(a.dsb) + ds_bytes(c)) : nullptr;
  kv.total_items = c.B * c.Hkv * kv.nkt * kv.kv_split;
  kv.per_xcd = per_xcd_for(kv, kv.total_items, kv.nkt * kv.kv_split);
  if ((st = launch("bwd_dkdv", s, kv.total_items, [&] { return attn::launch_bwd_dkdv(kv, c.D, s); }))) return st;
  if (kv.kv_split > 1 &&
      (st = launch("bwd_kv_reduce", s, c.B * c.Sk, [&] { return attn::launch_bwd_kv_reduce(kv, c.D, s); })))
    return st;

  attn::AttnArgs qa = a;
  qa.nqt = (c.S + attn::kDsRows - 1) / attn::kDsRows;
  qa.total_items = c.B * c.Hkv * qa.nqt * qa.r * (c.D == 512 ? attn::kDqSplit512 : 1);
  qa.per_xcd = per_xcd_for(qa, qa.total_items, qa.nqt * qa.r * (c.D == 512 ? attn::kDqSplit512 : 1));
  return launch("bwd_dq", s, qa.total_items, [&] { return attn::launch_bwd_dq(qa, c.D, s); });
}

bool lse_ok(const float* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// softcap: 0 (none) or a finite positive cap
bool softcap_ok(float x) { return std::isfinite(x) && x >= 0.f; }

Call with_softcap(Call c, float softcap) {
  c.softcap = softcap;
  return c;
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_bytes(const attn_shape* shape, int varlen, int causal, int window) {
  if (varlen < 0 || varlen > 2 || check_shape(shape, varlen) != ATTN_OK) return 0;
  if ((causal != 0 && causal != 1) || window < 0 || (window > 0 && !causal)) return 0;
  const size_t n = bwd_bytes(whole_call(shape, varlen, causal, window));
  return n > kMaxBwdWorkspace ? 0 : n;
}

size_t attn_fwd_workspace_bytes(const attn_shape* shape, int varlen) {
  if (varlen < 0 || varlen > 2 || check_shape(shape, varlen) != ATTN_OK) return 0;
  return meta_bytes(shape->B, varlen);
}

attn_status attn_fwd(const attn_shape* shape, attn_tensor q, attn_tensor k, attn_tensor v, float scale, int causal,
                     int window, float softcap, const int32_t* cu_seqlens, const uint8_t* pad_mask, attn_tensor o,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  const int varlen = varlen_kind(cu_seqlens, pad_mask);
  attn_status st = check_common(shape, scale, causal, window, cu_seqlens, pad_mask, workspace_bytes,
                                shape ? attn_fwd_workspace_bytes(shape, varlen) : 0, workspace);
  if (st != ATTN_OK) return st;
  if (!softcap_ok(softcap)) return ATTN_ERR_INVALID_ARG;
  const bool packed = varlen == 2;
  if ((st = check_tensor(q, packed)) || (st = check_tensor(k, packed)) || (st = check_tensor(v, packed)) ||
      (st = check_tensor(o, packed)))
    return st;
  if (!lse_ok(lse)) return ATTN_ERR_INVALID_ARG;
  if (shape->B == 0 || shape->S == 0 || (packed && shape->total == 0)) return ATTN_OK;
  const Tensors t = {q, k, v, o, {}, {}, {}, {}};
  return run_fwd(with_softcap(whole_call(shape, varlen, causal, window), softcap), t, scale, lse, cu_seqlens,
                 pad_mask, workspace, static_cast<hipStream_t>(stream));
}

attn_status attn_bwd(const attn_shape* shape, attn_tensor q, attn_tensor k, attn_tensor v, attn_tensor o,
                     const float* lse, attn_tensor dout, float scale, int causal, int window, float softcap,
                     const int32_t* cu_seqlens, const uint8_t* pad_mask, attn_tensor dq, attn_tensor dk,
                     attn_tensor dv, void* workspace, size_t workspace_bytes, void* stream) {
  const int varlen = varlen_kind(cu_seqlens, pad_mask);
  attn_status st = check_common(shape, scale, causal, window, cu_seqlens, pad_mask, workspace_bytes,
                                shape ? attn_bwd_workspace_bytes(shape, varlen, causal, window) : 0, workspace);
  if (st != ATTN_OK) return st;
  if (bwd_bytes(whole_call(shape, varlen, causal, window)) > kMaxBwdWorkspace) return ATTN_ERR_UNSUPPORTED;
  if (!softcap_ok(softcap)) return ATTN_ERR_INVALID_ARG;
  const bool packed = varlen == 2;
  if ((st = check_tensor(q, packed)) || (st = check_tensor(k, packed)) || (st = check_tensor(v, packed)) ||
      (st = check_tensor(o, packed)) || (st = check_tensor(dout, packed)) || (st = check_tensor(dq, packed)) ||
      (st = check_tensor(dk, packed)) || (st = check_tensor(dv, packed)))
    return st;
  if (!lse_ok(lse)) return ATTN_ERR_INVALID_ARG;
  if (shape->B == 0 || shape->S == 0 || (packed && shape->total == 0)) return ATTN_OK;
  const Tensors t = {q, k, v, o, dout, dq, dk, dv};
  return run_bwd(with_softcap(whole_call(shape, varlen, causal, window), softcap), t, scale, lse, cu_seqlens,
                 pad_mask, workspace, static_cast<hipStream_t>(stream));
}

size_t attn_bwd_chunk_workspace_bytes(const attn_chunk_shape* shape, int causal, int window, int64_t q_pos0,
                                      int64_t k_pos0) {
  if (check_chunk(shape, causal, window, q_pos0, k_pos0) != ATTN_OK) return 0;
  const size_t n = bwd_bytes(chunk_call(shape, causal, window, q_pos0, k_pos0));
  return n > kMaxBwdWorkspace ? 0 : n;
}

attn_status attn_fwd_chunk(const attn_chunk_shape* shape, attn_tensor q, attn_tensor k, attn_tensor v, float scale,
                           int causal, int window, float softcap, int64_t q_pos0, int64_t k_pos0, attn_tensor o,
                           int o_dtype, float* lse, void* stream) {
  attn_status st = check_chunk(shape, causal, window, q_pos0, k_pos0);
  if (st != ATTN_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f) || !softcap_ok(softcap)) return ATTN_ERR_INVALID_ARG;
  if (o_dtype != shape->dtype && o_dtype != ATTN_DTYPE_F32) return ATTN_ERR_INVALID_ARG;
  if ((st = check_tensor(q, false)) || (st = check_tensor(k, false)) || (st = check_tensor(v, false)) ||
      (st = check_tensor(o, false)))
    return st;
  if (!lse_ok(lse)) return ATTN_ERR_INVALID_ARG;
  if (shape->B == 0 || shape->Sq == 0) return ATTN_OK;
  const Tensors t = {q, k, v, o, {}, {}, {}, {}};
  return run_fwd(with_softcap(chunk_call(shape, causal, window, q_pos0, k_pos0), softcap), t, scale, lse, nullptr,
                 nullptr, nullptr, static_cast<hipStream_t>(stream),
                 o_dtype == ATTN_DTYPE_F32 ? FwdOut::f32 : FwdOut::half);
}

attn_status attn_fwd_chunk_merge(const attn_chunk_shape* shape, attn_tensor q, attn_tensor k, attn_tensor v,
                                 float scale, int causal, int window, float softcap, int64_t q_pos0, int64_t k_pos0,
                                 attn_tensor o, float* lse, attn_tensor out, void* stream) {
  attn_status st = check_chunk(shape, causal, window, q_pos0, k_pos0);
  if (st != ATTN_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f) || !softcap_ok(softcap)) return ATTN_ERR_INVALID_ARG;
  if ((st = check_tensor(q, false)) || (st = check_tensor(k, false)) || (st = check_tensor(v, false)) ||
      (st = check_tensor(o, false)))
    return st;
  if (out.ptr != nullptr && (st = check_tensor(out, false))) return st;
  if (!lse_ok(lse)) return ATTN_ERR_INVALID_ARG;
  if (shape->B == 0 || shape->Sq == 0) return ATTN_OK;
  const Tensors t = {q, k, v, o, {}, {}, {}, {}};
  return run_fwd(with_softcap(chunk_call(shape, causal, window, q_pos0, k_pos0), softcap), t, scale, lse, nullptr,
                 nullptr, nullptr, static_cast<hipStream_t>(stream), FwdOut::merge, out);
}

attn_status attn_bwd_chunk(const attn_chunk_shape* shape, attn_tensor q, attn_tensor k, attn_tensor v, attn_tensor o,
                           const float* lse, attn_tensor dout, float scale, int causal, int window, float softcap,
                           int64_t q_pos0, int64_t k_pos0, attn_tensor dq, attn_tensor dk, attn_tensor dv,
                           int grad_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = check_chunk(shape, causal, window, q_pos0, k_pos0);
  if (st != ATTN_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f) || !softcap_ok(softcap)) return ATTN_ERR_INVALID_ARG;
  if (grad_dtype != shape->dtype && grad_dtype != ATTN_DTYPE_F32) return ATTN_ERR_INVALID_ARG;
  if (bwd_bytes(chunk_call(shape, causal, window, q_pos0, k_pos0)) > kMaxBwdWorkspace) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_bwd_chunk_workspace_bytes(shape, causal, window, q_pos0, k_pos0);
  if (need > 0 &&
      (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))))
    return ATTN_ERR_WORKSPACE;
  if ((st = check_tensor(q, false)) || (st = check_tensor(k, false)) || (st = check_tensor(v, false)) ||
      (st = check_tensor(o, false)) || (st = check_tensor(dout, false)) || (st = check_tensor(dq, false)) ||
      (st = check_tensor(dk, false)) || (st = check_tensor(dv, false)))
    return st;
  if (!lse_ok(lse)) return ATTN_ERR_INVALID_ARG;
  if (shape->B == 0 || (shape->Sq == 0 && shape->Sk == 0)) return ATTN_OK;
  const Tensors t = {q, k, v, o, dout, dq, dk, dv};
  return run_bwd(with_softcap(chunk_call(shape, causal, window, q_pos0, k_pos0), softcap), t, scale, lse, nullptr,
                 nullptr, workspace, static_cast<hipStream_t>(stream), grad_dtype == ATTN_DTYPE_F32);
}

attn_status attn_lse_merge(int32_t B, int32_t S, int32_t H, int32_t D, attn_tensor o, float* lse,
                           attn_tensor o_part, const float* lse_part, attn_tensor out, int out_dtype, void* stream) {
  if (B < 0 || S < 0 || H <= 0) return ATTN_ERR_INVALID_ARG;
  if (D != 128 && D != 256 && D != 512) return ATTN_ERR_UNSUPPORTED;
  if (!dtype16_ok(out_dtype)) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * S * H >= INT_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  attn_status st;
  if ((st = check_tensor(o, false)) || (st = check_tensor(o_part, false))) return st;
  if (out.ptr != nullptr && (st = check_tensor(out, false))) return st;
  if (!lse_ok(lse) || !lse_ok(lse_part)) return ATTN_ERR_INVALID_ARG;
  if (B == 0 || S == 0) return ATTN_OK;
  attn::MergeArgs a = {};
  a.o = static_cast<float*>(o.ptr);
  a.lse = lse;
  a.o_part = static_cast<const float*>(o_part.ptr);
  a.lse_part = lse_part;
  a.out = static_cast<__bf16*>(out.ptr);
  a.o_sb = o.stride_b;
  a.o_ss = o.stride_s;
  a.o_sh = o.stride_h;
  a.p_sb = o_part.stride_b;
  a.p_ss = o_part.stride_s;
  a.p_sh = o_part.stride_h;
  a.r_sb = out.stride_b;
  a.r_ss = out.stride_s;
  a.r_sh = out.stride_h;
  a.B = B;
  a.S = S;
  a.H = H;
  a.rows = B * S * H;
  a.out_f16 = out_dtype == ATTN_DTYPE_F16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch("lse_merge", s, a.rows, [&] { return attn::launch_lse_merge(a, D, s); });
}

// Shared checks and arguments of paged_kv_append and paged_kv_gather.
static attn_status paged_copy(const attn_decode_shape* shape, int32_t n, attn_tensor k_tok, attn_tensor v_tok,
                              attn_tensor k_cache, attn_tensor v_cache, const int32_t* block_table,
                              const int32_t* ctx_lens, int gather, const char* name, void* stream,
                              bool meta_check = true) {
  if (shape == nullptr) return ATTN_ERR_INVALID_ARG;
  const attn_decode_shape& sh = *shape;
  if (sh.B < 0 || n < 0 || sh.Hkv <= 0 || sh.num_pages <= 0 || sh.max_pages_per_seq <= 0 || sh.page_size <= 0)
    return ATTN_ERR_INVALID_ARG;
  if ((sh.D != 128 && sh.D != 256 && sh.D != 512) || !dtype16_ok(sh.dtype)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)sh.max_pages_per_seq * sh.page_size > INT_MAX / 2 || (int64_t)sh.B * n * sh.Hkv >= INT_MAX / 4)
    return ATTN_ERR_UNSUPPORTED;
  if (block_table == nullptr || ctx_lens == nullptr) return ATTN_ERR_INVALID_ARG;
  attn_status st;
  if ((st = check_tensor(k_tok, false)) || (st = check_tensor(v_tok, false)) || (st = check_tensor(k_cache, false)) ||
      (st = check_tensor(v_cache, false)))
    return st;
  if (sh.B == 0 || n == 0) return ATTN_OK;
  if (meta_check && (st = debug_check_pages(sh, block_table, ctx_lens, static_cast<hipStream_t>(stream)))) return st;
  attn::PagedCopyArgs a = {};
  a.tk = static_cast<__bf16*>(k_tok.ptr);
  a.tv = static_cast<__bf16*>(v_tok.ptr);
  a.kc = static_cast<__bf16*>(k_cache.ptr);
  a.vc = static_cast<__bf16*>(v_cache.ptr);
  a.table = block_table;
  a.ctx = ctx_lens;
  a.tk_sb = k_tok.stride_b;
  a.tk_ss = k_tok.stride_s;
  a.tk_sh = k_tok.stride_h;
  a.tv_sb = v_tok.stride_b;
  a.tv_ss = v_tok.stride_s;
  a.tv_sh = v_tok.stride_h;
  a.kc_sp = k_cache.stride_b;
  a.kc_ss = k_cache.stride_s;
  a.kc_sh = k_cache.stride_h;
  a.vc_sp = v_cache.stride_b;
  a.vc_ss = v_cache.stride_s;
  a.vc_sh = v_cache.stride_h;
  a.B = sh.B;
  a.n = n;
  a.Hkv = sh.Hkv;
  a.D = sh.D;
  a.page_size = sh.page_size;
  a.num_pages = sh.num_pages;
  a.max_pages = sh.max_pages_per_seq;
  a.gather = gather;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch(name, s, 1, [&] { return attn::launch_paged_kv_copy(a, s); });
}

size_t paged_decode_workspace_bytes(const attn_decode_shape* s) {
  if (s == nullptr || s->B < 0 || s->Hq <= 0 || s->Hkv <= 0 || s->D != 128 || s->page_size != 16 ||
      s->max_pages_per_seq <= 0 || !dtype16_ok(s->dtype))
    return 0;
  const size_t chunks = ((size_t)s->max_pages_per_seq * s->page_size + attn::kDecodeChunk - 1) / attn::kDecodeChunk;
  return round_up(sizeof(float) * (size_t)s->B * s->Hq * chunks * (s->D + 2));
}

// Argument checks of paged_decode and paged_decode_noalloc, before the workspace.
static attn_status check_decode(const attn_decode_shape* shape, const void* q, int64_t q_stride_b,
                                int64_t q_stride_h, attn_tensor k_cache, attn_tensor v_cache,
                                const int32_t* block_table, const int32_t* ctx_lens, float scale, float softcap,
                                void* o, int64_t o_stride_b, int64_t o_stride_h) {
  if (shape == nullptr) return ATTN_ERR_INVALID_ARG;
  const attn_decode_shape& sh = *shape;
  if (sh.B < 0 || sh.Hq <= 0 || sh.Hkv <= 0 || sh.num_pages <= 0 || sh.max_pages_per_seq <= 0 || sh.page_size <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (sh.Hq % sh.Hkv != 0) return ATTN_ERR_INVALID_ARG;
  const int r = sh.Hq / sh.Hkv;
  if (sh.D != 128 || sh.page_size != 16 || (r != 1 && r != 2 && r != 4 && r != 8)) return ATTN_ERR_UNSUPPORTED;
  if (!dtype16_ok(sh.dtype)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)sh.max_pages_per_seq * sh.page_size > INT_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  if (!(std::isfinite(scale) && scale > 0.f) || !softcap_ok(softcap)) return ATTN_ERR_INVALID_ARG;
  if (q == nullptr || o == nullptr || !aligned16(q) || !aligned16(o) || block_table == nullptr || ctx_lens == nullptr)
    return ATTN_ERR_INVALID_ARG;
  if (!stride_ok(q_stride_b) || !stride_ok(q_stride_h) || !stride_ok(o_stride_b) || !stride_ok(o_stride_h))
    return ATTN_ERR_INVALID_ARG;
  attn_status st;
  if ((st = check_tensor(k_cache, false)) || (st = check_tensor(v_cache, false))) return st;
  // offsets inside one page are 32-bit byte offsets
  if (k_cache.stride_s > (INT_MAX / 2) / 16 || v_cache.stride_s > (INT_MAX / 2) / 16) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Which decode runs: one 8-wave workgroup per (sequence, kv head) over the whole context when
// the batch alone gives every compute unit a workgroup and no context can exceed 8192 tokens;
// otherwise 512-token chunks over (kv head, chunk, sequence) and a merge of their partials.
// Measured on the head_dim-128 decode workload's lengths (Hkv 8): whole against chunked 2.8
// against 3.3 TB/s at 8 sequences, 3.0 / 3.6 at 16, 4.15 / 4.0 at 32, 4.9 / 4.3 at 48.
static bool decode_whole(const attn_decode_shape& sh) {
  return (int64_t)sh.B * sh.Hkv >= kComputeUnits && (int64_t)sh.max_pages_per_seq * sh.page_size <= 8192;
}

// The decode's launches, after every check; `workspace` holds the chunk partials (split path).
static attn_status run_decode(const attn_decode_shape& sh, const void* q, int64_t q_stride_b, int64_t q_stride_h,
                              attn_tensor k_cache, attn_tensor v_cache, const int32_t* block_table,
                              const int32_t* ctx_lens, float scale, float softcap, void* o, int64_t o_stride_b,
                              int64_t o_stride_h, void* workspace, void* stream, int contiguous = 0,
                              bool meta_check = true) {
  attn_status st;
  if (meta_check &&
      (st = debug_check_pages(sh, block_table, ctx_lens, static_cast<hipStream_t>(stream), contiguous)))
    return st;
  const int r = sh.Hq / sh.Hkv;

  attn::DecodeArgs a = {};
  a.q = static_cast<const __bf16*>(q);
  a.kc = static_cast<const __bf16*>(k_cache.ptr);
  a.vc = static_cast<const __bf16*>(v_cache.ptr);
  a.table = block_table;
  a.ctx = ctx_lens;
  a.o = static_cast<__bf16*>(o);
  a.part = static_cast<float*>(workspace);
  a.f16 = sh.dtype == ATTN_DTYPE_F16;
  a.contiguous = contiguous;
  a.q_sb = q_stride_b;
  a.q_sh = q_stride_h;
  a.o_sb = o_stride_b;
  a.o_sh = o_stride_h;
  a.kc_sp = k_cache.stride_b;
  a.kc_ss = k_cache.stride_s;
  a.kc_sh = k_cache.stride_h;
  a.vc_sp = v_cache.stride_b;
  a.vc_ss = v_cache.stride_s;
  a.vc_sh = v_cache.stride_h;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.r = r;
  a.page_size = sh.page_size;
  a.num_pages = sh.num_pages;
  a.max_pages = sh.max_pages_per_seq;
  a.max_chunks = (sh.max_pages_per_seq * sh.page_size + attn::kDecodeChunk - 1) / attn::kDecodeChunk;
  a.c = scale * 1.4426950408889634f;
  a.sc_in = softcap > 0.f ? scale / softcap : 0.f;
  a.sc_out = softcap > 0.f ? softcap / scale : 0.f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (decode_whole(sh))
    return hip_status(timed("decode_whole", s, [&] { return attn::launch_decode_whole(a, sh.D, s); }));
  hipError_t e = timed("decode_split", s, [&] { return attn::launch_decode_split(a, sh.D, s); });
  if (e != hipSuccess) return hip_status(e);
  return hip_status(timed("decode_merge", s, [&] { return attn::launch_decode_merge(a, sh.D, s); }));
}

attn_status paged_decode(const attn_decode_shape* shape, const void* q, int64_t q_stride_b, int64_t q_stride_h,
                         attn_tensor k_cache, attn_tensor v_cache, const int32_t* block_table,
                         const int32_t* ctx_lens, float scale, float softcap, void* o, int64_t o_stride_b,
                         int64_t o_stride_h, void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = check_decode(shape, q, q_stride_b, q_stride_h, k_cache, v_cache, block_table, ctx_lens, scale,
                                softcap, o, o_stride_b, o_stride_h);
  if (st != ATTN_OK) return st;
  const size_t need = paged_decode_workspace_bytes(shape);
  if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  if (shape->B == 0) return ATTN_OK;
  return run_decode(*shape, q, q_stride_b, q_stride_h, k_cache, v_cache, block_table, ctx_lens, scale, softcap, o,
                    o_stride_b, o_stride_h, workspace, stream);
}

attn_status paged_decode_contiguous(const attn_decode_shape* shape, const void* q, int64_t q_stride_b,
                                    int64_t q_stride_h, attn_tensor k_cache, attn_tensor v_cache,
                                    const int32_t* first_page, const int32_t* ctx_lens, float scale, float softcap,
                                    void* o, int64_t o_stride_b, int64_t o_stride_h, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  attn_status st = check_decode(shape, q, q_stride_b, q_stride_h, k_cache, v_cache, first_page, ctx_lens, scale,
                                softcap, o, o_stride_b, o_stride_h);
  if (st != ATTN_OK) return st;
  const size_t need = paged_decode_workspace_bytes(shape);
  if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  if (shape->B == 0) return ATTN_OK;
  return run_decode(*shape, q, q_stride_b, q_stride_h, k_cache, v_cache, first_page, ctx_lens, scale, softcap, o,
                    o_stride_b, o_stride_h, workspace, stream, 1);
}

size_t paged_decode_noalloc_max_bytes(void) { return attn::kDecodeScratchBytes; }

attn_status paged_decode_noalloc(const attn_decode_shape* shape, const void* q, int64_t q_stride_b,
                                 int64_t q_stride_h, attn_tensor k_cache, attn_tensor v_cache,
                                 const int32_t* block_table, const int32_t* ctx_lens, float scale, float softcap,
                                 void* o, int64_t o_stride_b, int64_t o_stride_h, void* stream) {
  attn_status st = check_decode(shape, q, q_stride_b, q_stride_h, k_cache, v_cache, block_table, ctx_lens, scale,
                                softcap, o, o_stride_b, o_stride_h);
  if (st != ATTN_OK) return st;
  if (paged_decode_workspace_bytes(shape) > attn::kDecodeScratchBytes) return ATTN_ERR_WORKSPACE;
  if (shape->B == 0) return ATTN_OK;
  void* scratch = nullptr;
  if ((st = hip_status(attn::decode_scratch(&scratch)))) return st;
  return run_decode(*shape, q, q_stride_b, q_stride_h, k_cache, v_cache, block_table, ctx_lens, scale, softcap, o,
                    o_stride_b, o_stride_h, scratch, stream);
}

}  // extern "C"

// One captured decode step per batch bucket (paged_decode_graphs_*).
struct attn_decode_graphs {
  std::vector<int32_t> buckets;
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
};

namespace {

void destroy_graphs(attn_decode_graphs* g) {
  for (hipGraphExec_t e : g->execs) (void)hipGraphExecDestroy(e);
  for (hipGraph_t gr : g->graphs) (void)hipGraphDestroy(gr);
  delete g;
}

}  // namespace

extern "C" {

attn_status paged_decode_graphs_create(const attn_decode_shape* shape, const int32_t* buckets, int32_t n_buckets,
                                       const void* q, int64_t q_stride_b, int64_t q_stride_h, attn_tensor k_new,
                                       attn_tensor v_new, attn_tensor k_cache, attn_tensor v_cache,
                                       const int32_t* block_table, const int32_t* ctx_lens, float scale, float softcap,
                                       void* o, int64_t o_stride_b, int64_t o_stride_h, void* workspace,
                                       size_t workspace_bytes, void* stream, attn_decode_graphs** out) {
  if (out == nullptr) return ATTN_ERR_INVALID_ARG;
  *out = nullptr;
  attn_status st = check_decode(shape, q, q_stride_b, q_stride_h, k_cache, v_cache, block_table, ctx_lens, scale,
                                softcap, o, o_stride_b, o_stride_h);
  if (st != ATTN_OK) return st;
  if (stream == nullptr || buckets == nullptr || n_buckets <= 0 || shape->B <= 0) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < n_buckets; ++i)
    if (buckets[i] < 1 || buckets[i] > shape->B || (i > 0 && buckets[i] <= buckets[i - 1])) return ATTN_ERR_INVALID_ARG;
  const bool append = k_new.ptr != nullptr || v_new.ptr != nullptr;
  if (append && ((st = check_tensor(k_new, false)) || (st = check_tensor(v_new, false)))) return st;
  const size_t need = paged_decode_workspace_bytes(shape);
  if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // metadata is checked once, here (a check synchronises, which a capture cannot)
  if ((st = debug_check_pages(*shape, block_table, ctx_lens, s))) return st;

  attn_decode_graphs* g = new attn_decode_graphs();
  const bool prof = g_prof.on;
  g_prof.on = false;  // no timing events inside the graphs
  for (int i = 0; i < n_buckets && st == ATTN_OK; ++i) {
    attn_decode_shape sb = *shape;
    sb.B = buckets[i];
    hipGraph_t graph = nullptr;
    st = hip_status(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    if (st != ATTN_OK) break;
    attn_status run = ATTN_OK;
    if (append)
      run = paged_copy(&sb, 1, k_new, v_new, k_cache, v_cache, block_table, ctx_lens, 0, "paged_kv_append", stream,
                       false);
    if (run == ATTN_OK)
      run = run_decode(sb, q, q_stride_b, q_stride_h, k_cache, v_cache, block_table, ctx_lens, scale, softcap, o,
                       o_stride_b, o_stride_h, workspace, stream, 0, false);
    const hipError_t end = hipStreamEndCapture(s, &graph);
    st = run != ATTN_OK ? run : hip_status(end);
    if (graph != nullptr) g->graphs.push_back(graph);
    if (st != ATTN_OK) break;
    hipGraphExec_t exec = nullptr;
    st = hip_status(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
    if (st == ATTN_OK) {
      g->execs.push_back(exec);
      g->buckets.push_back(buckets[i]);
    }
  }
  g_prof.on = prof;
  if (st != ATTN_OK) {
    destroy_graphs(g);
    return st;
  }
  *out = g;
  return ATTN_OK;
}

attn_status paged_decode_graphs_launch(const attn_decode_graphs* graphs, int32_t B, void* stream,
                                       int32_t* bucket) {
  if (graphs == nullptr || B < 0 || B > graphs->buckets.back()) return ATTN_ERR_INVALID_ARG;
  if (bucket != nullptr) *bucket = 0;
  if (B == 0) return ATTN_OK;
  size_t i = 0;
  while (graphs->buckets[i] < B) ++i;
  if (bucket != nullptr) *bucket = graphs->buckets[i];
  return hip_status(hipGraphLaunch(graphs->execs[i], static_cast<hipStream_t>(stream)));
}

void paged_decode_graphs_destroy(attn_decode_graphs* graphs) {
  if (graphs != nullptr) destroy_graphs(graphs);
}

attn_status paged_kv_append(const attn_decode_shape* shape, int32_t n_tokens, attn_tensor k_new, attn_tensor v_new,
                            attn_tensor k_cache, attn_tensor v_cache, const int32_t* block_table,
                            const int32_t* ctx_lens, void* stream) {
  return paged_copy(shape, n_tokens, k_new, v_new, k_cache, v_cache, block_table, ctx_lens, 0, "paged_kv_append",
                    stream);
}

attn_status paged_kv_gather(const attn_decode_shape* shape, int32_t n_tokens, attn_tensor k_cache,
                            attn_tensor v_cache, const int32_t* block_table, const int32_t* ctx_lens,
                            attn_tensor k_out, attn_tensor v_out, void* stream) {
  return paged_copy(shape, n_tokens, k_out, v_out, k_cache, v_cache, block_table, ctx_lens, 1, "paged_kv_gather",
                    stream);
}

// Paged prefill: packed new query rows (cu_q) against each sequence's paged cache.
static attn_status check_paged_shape(const attn_paged_shape* s) {
  if (s == nullptr) return ATTN_ERR_INVALID_ARG;
  if (s->B < 0 || s->max_q < 0 || s->total_q < 0 || s->Hq <= 0 || s->Hkv <= 0 || s->num_pages <= 0 ||
      s->max_pages_per_seq <= 0 || s->page_size <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (s->Hq % s->Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if ((s->D != 256 && s->D != 512) || s->page_size != 16 || !dtype16_ok(s->dtype)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)s->max_pages_per_seq * s->page_size > INT_MAX / 2 || (int64_t)s->total_q * s->Hq >= INT_MAX / 2 ||
      s->max_q >= (1 << 28))
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // extern "C"

namespace {

// Workspace of the split paged forward: per (sequence, query head) kSplitMax pieces of an fp32
// O row and an LSE.
size_t paged_split_bytes(const attn_paged_shape& sh) {
  return round_up((size_t)sh.B * sh.Hq * attn::kSplitMax * (sh.D + 1) * sizeof(float) + sizeof(int32_t) * sh.B);
}

attn_status fwd_paged(const attn_paged_shape* shape, attn_tensor q, attn_tensor k_cache, attn_tensor v_cache,
                      const int32_t* block_table, const int32_t* cu_q, const int32_t* ctx_lens, float scale,
                      int window, float softcap, attn_tensor o, float* lse, float* split_ws, void* stream) {
  attn_status st = check_paged_shape(shape);
  if (st != ATTN_OK) return st;
  const attn_paged_shape& sh = *shape;
  if (!(std::isfinite(scale) && scale > 0.f) || !softcap_ok(softcap) || window < 0) return ATTN_ERR_INVALID_ARG;
  if (block_table == nullptr || cu_q == nullptr || ctx_lens == nullptr) return ATTN_ERR_INVALID_ARG;
  if ((st = check_tensor(q, true)) || (st = check_tensor(o, true)) || (st = check_tensor(k_cache, false)) ||
      (st = check_tensor(v_cache, false)))
    return st;
  if (!lse_ok(lse)) return ATTN_ERR_INVALID_ARG;
  // offsets inside one page are 32-bit byte offsets
  if (k_cache.stride_s > (INT_MAX / 2) / 16 || v_cache.stride_s > (INT_MAX / 2) / 16) return ATTN_ERR_UNSUPPORTED;
  if (sh.B == 0 || sh.max_q == 0 || sh.total_q == 0) return ATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const attn_decode_shape pages = {sh.B, sh.Hq, sh.Hkv, sh.D, sh.page_size, sh.num_pages, sh.max_pages_per_seq,
                                   sh.dtype};
  if ((st = debug_check_pages(pages, block_table, ctx_lens, s))) return st;

  Call c = {};
  c.B = sh.B;
  c.S = sh.max_q;
  c.Sk = sh.max_pages_per_seq * sh.page_size;
  c.total = sh.total_q;
  c.Hq = sh.Hq;
  c.Hkv = sh.Hkv;
  c.D = sh.D;
  c.varlen = 2;
  c.f16 = sh.dtype == ATTN_DTYPE_F16;
  c.causal = 1;
  // a query's position is below Sk, so a window of Sk or more never binds; a smaller one keeps
  // every position difference inside 32 bits
  c.window = window >= c.Sk ? 0 : window;
  c.shift = 0;
  c.softcap = softcap;
  const Tensors t = {q, k_cache, v_cache, o, {}, {}, {}, {}};
  const PagedKV pg = {block_table, ctx_lens, k_cache.stride_b, v_cache.stride_b, sh.max_pages_per_seq, sh.num_pages};
  return run_fwd(c, t, scale, lse, cu_q, nullptr, nullptr, s, FwdOut::half, {}, &pg, split_ws);
}

}  // namespace

extern "C" {

attn_status attn_fwd_paged(const attn_paged_shape* shape, attn_tensor q, attn_tensor k_cache, attn_tensor v_cache,
                           const int32_t* block_table, const int32_t* cu_q, const int32_t* ctx_lens, float scale,
                           int window, float softcap, attn_tensor o, float* lse, void* stream) {
  return fwd_paged(shape, q, k_cache, v_cache, block_table, cu_q, ctx_lens, scale, window, softcap, o, lse, nullptr,
                   stream);
}

size_t attn_fwd_paged_workspace_bytes(const attn_paged_shape* shape) {
  if (check_paged_shape(shape) != ATTN_OK) return 0;
  return paged_split_bytes(*shape);
}

attn_status attn_fwd_paged_split(const attn_paged_shape* shape, attn_tensor q, attn_tensor k_cache,
                                 attn_tensor v_cache, const int32_t* block_table, const int32_t* cu_q,
                                 const int32_t* ctx_lens, float scale, int window, float softcap, attn_tensor o,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = check_paged_shape(shape);
  if (st != ATTN_OK) return st;
  const size_t need = paged_split_bytes(*shape);
  if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return ATTN_ERR_WORKSPACE;
  return fwd_paged(shape, q, k_cache, v_cache, block_table, cu_q, ctx_lens, scale, window, softcap, o, lse,
                   static_cast<float*>(workspace), stream);
}

int attn_debug(int on) {
  debug_on();  // the environment's setting is read first, so that this call overrides it
  const int prev = g_debug.exchange(on ? 1 : 0);
  return prev > 0;
}

const char* attn_status_str(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument (null pointer, shape, stride or alignment)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration (head_dim, window without causal, sizes)";
    case ATTN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int attn_last_hip_error(void) { return g_last_hip_error; }

int attn_count_restarts(int32_t* device_counter) {
  g_restarts = reinterpret_cast<int*>(device_counter);
  return 0;
}

int attn_profile(int on) {
  g_prof.on = on != 0;
  return 0;
}

int attn_profile_read(attn_kernel_time* out, int max_entries) {
  int n = 0;
  bool failed = false;
  for (const TimedLaunch& t : g_prof.launches) {
    float ms = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) {
      failed = true;
      break;
    }
    int i = 0;
    while (i < n && std::strcmp(out[i].kernel, t.name) != 0) ++i;
    if (i == n) {
      if (n == max_entries) continue;
      out[n++] = {t.name, 0, 0.0};
    }
    out[i].launches += 1;
    out[i].total_ms += ms;
  }
  g_prof.launches.clear();
  g_prof.used = 0;
  return failed ? -1 : n;
}

attn_status attn_peak_probe(int kind, void* buf, size_t bytes, int reps, void* stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e);
  if (buf == nullptr || !aligned16(buf) || cus <= 0) return ATTN_ERR_INVALID_ARG;
  if (kind == 0 && (reps <= 0 || bytes < (size_t)cus * 4 * 256 * sizeof(float))) return ATTN_ERR_INVALID_ARG;
  if ((kind == 1 || kind == 2) && (bytes < 4096 || bytes % 32 != 0)) return ATTN_ERR_INVALID_ARG;
  if (kind < 0 || kind > 2) return ATTN_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(attn::launch_peak_probe(kind, buf, bytes, reps, cus, s));
}

const char* attn_version(void) { return "0.1.0"; }

}  // extern "C"
