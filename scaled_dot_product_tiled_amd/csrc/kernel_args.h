// Kernel argument blocks and launch entry points shared by the HIP kernels and the
// C-ABI layer.  All strides are in elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// One fused-attention call (forward or backward).  Row (b, pos, h) of a tensor X
// lives at X + b * X_sb + (seq_off[b] + pos) * X_ss + h * X_sh; packed inputs pass
// X_sb = 0 and seq_off from cu_seqlens, dense inputs pass seq_off = seq_len = NULL.
// Row statistics (LSE, delta) of (b, h, pos) live at st + b * st_sb + h * st_sh +
// seq_off[b] + pos.
//
// Query row i sits at position i + q_shift and key row j at position j, so query i sees
// key j when j <= i + q_shift (causal) and j > i + q_shift - window (window > 0).  Whole
// sequences have q_shift = 0 and Sk = S; a chunk pair of a sequence split into chunks has
// S query rows, Sk key rows and q_shift = (position of its first query) - (position of its
// first key).  The host keeps q_shift in [-S, Sk] and window in [0, S + Sk].
struct AttnArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  __bf16* out;  // forward: O; backward: dQ
  float* out_f32;  // forward: O in fp32 instead of out (chunk partials); NULL otherwise
  __bf16* dk;
  __bf16* dv;
  // backward of a chunk pair: when set, the pair's dQ, dK, dV are added to these fp32
  // accumulators (same strides as dq, dk, dv) instead of written in bf16
  float* dq_f32;
  float* dk_f32;
  float* dv_f32;
  float* lse;   // forward writes, backward reads
  float* delta;  // backward: rowsum(dO * O)
  __bf16* dsb;   // backward: dS blocks (see ds_block_index)
  int64_t ds_head;  // dS blocks per (batch, query head)
  int ds_tri, ds_cnt;  // block layout: triangular, or ds_cnt blocks per query tile
  // packed (cu_seqlens) rows: first dS block of each sequence's region, whose heads hold
  // ds_head_blocks(len) blocks each (sized by the sequence's own length, not the longest);
  // -1: the sequence does not fit the workspace (inconsistent offsets) and is skipped.
  // NULL: every (batch, head) holds ds_head blocks.
  const int64_t* ds_seq;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;    // O (forward output / backward input)
  int64_t do_sb, do_ss, do_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  int64_t st_sb, st_sh;
  const int32_t* seq_off;  // NULL: 0
  const int32_t* seq_len;  // NULL: S
  int B, S, Hq, Hkv, r;
  int Sk;                   // key rows (dense); S for whole sequences
  int q_shift;              // query position offset (see above)
  int empty_lse_ninf;       // a query row with no visible key stores LSE = -inf (else 0)
  int hpt, mpos, nhb, nqt;  // heads per tile, positions per tile, head blocks, q tiles
  int nkt;                  // key tiles (dK/dV kernel)
  int kv_split;             // dK/dV: workgroups sharing one key tile's query heads (1, 2 or 4)
  float* kv_part;           // kv_split > 1: fp32 partial dK, dV, [part][dK|dV][B][Sk][Hkv][D]
  int f16;                  // 16-bit tensors are IEEE half (else bfloat16)
  int packed;               // rows past a sequence's length do not exist
  int causal, window;
  float scale;
  // tanh softcap of the scaled scores s -> cap tanh(s / cap) (cap = softcap > 0), applied to
  // raw scores x (s = scale x) as x -> sc_out tanh(sc_in x) with sc_in = scale / cap and
  // sc_out = cap / scale, so the rest of the arithmetic is unchanged
  float softcap, sc_in, sc_out;              // multiplies Q K^T
  float c;                  // scale * log2(e)
  int per_xcd, total_items;
  int balanced;             // deal work items in rounds (see xcd_item)
  const int32_t* order;     // batch indices by decreasing length (varlen), or null
  // forward, merge: out_f32 and lse hold a running result that the row's O and LSE are
  // merged into; out (strides r_*), if not NULL, receives the merged O in 16 bits
  int merge;
  int64_t r_sb, r_ss, r_sh;
  // forward: when not NULL, every restart of a workgroup's key loop (head_dim 512 softmax
  // reference raised) adds 1 here
  int* restarts;
  // forward over a paged cache (paged): K, V are (num_pages, 16, Hkv, D) with k_sb / v_sb the
  // page stride, k_ss / v_ss the slot stride and k_sh / v_sh the head stride; sequence b's key
  // j lives in page table[b * max_pages + j / 16], slot j % 16; it holds kv_len[b] keys (its
  // cached tokens, the new ones included) and its len query rows sit at positions
  // kv_len[b] - len .. kv_len[b] - 1.  seq_off is then the B + 1 query row offsets (cu_q),
  // read directly, and total the packed row count
  int paged;
  int total;
  const int32_t* table;
  const int32_t* kv_len;
  int max_pages, num_pages;
  // paged forward with split decode rows (split_o not NULL): a sequence with one new token
  // whose keys span more than kSplitMinTiles tiles is cut into pieces (decode_pieces), each a
  // workgroup (the unit's item split_slot0 + piece) that writes its normalised fp32 O to split_o[((unit * kSplitMax + piece) * hpt +
  // head in the tile) * D ..] and its LSE to split_lse[(unit * kSplitMax + piece) * hpt + head
  // in the tile]; fwd_split_merge combines them
  float* split_o;
  float* split_lse;
  int split_slot0;  // a unit's items split_slot0 .. split_slot0 + kSplitMax - 1 hold the pieces
  // workgroups of the split deal's first phase (paged_split_item), 0 for the other deals
  int split_nA;
};

// Split decode rows of the paged forward: at most kSplitMax pieces of at least kSplitMinTiles
// 32-key tiles each.
constexpr int kSplitMax = 16;
constexpr int kSplitMinTiles = 8;

// Pieces of the decode row of a paged sequence with lenk cached keys (its one query sits at
// position lenk - 1): its key tiles t_lo .. t_lo + n - 1 are cut into pieces of ch tiles (the
// last one shorter), every piece holding at least one visible key.  Returns the piece count;
// 1 means the row is not split.
__host__ __device__ inline int decode_pieces(int lenk, int window, int& t_lo, int& ch) {
  const int jlo = window > 0 ? (lenk - window > 0 ? lenk - window : 0) : 0;
  t_lo = jlo / 32;
  const int n = lenk > jlo ? (lenk + 31) / 32 - t_lo : 0;
  int ns = (n + kSplitMinTiles - 1) / kSplitMinTiles;
  ns = ns < kSplitMax ? ns : kSplitMax;
  ch = n;
  if (ns <= 1) return 1;
  ch = (n + ns - 1) / ns;
  return (n + ch - 1) / ch;
}

struct DecodeArgs {
  const __bf16* q;
  const __bf16* kc;
  const __bf16* vc;
  const int32_t* table;
  const int32_t* ctx;
  __bf16* o;
  float* part;        // per (b, h, chunk): m, l, o[D]
  int64_t q_sb, q_sh, o_sb, o_sh;
  int64_t kc_sp, kc_ss, kc_sh, vc_sp, vc_ss, vc_sh;
  int B, Hq, Hkv, r, page_size, num_pages, max_pages, max_chunks;
  float c;            // scale * log2(e)
  float sc_in, sc_out;  // softcap (see AttnArgs); unused without a cap
  int f16;            // 16-bit tensors are IEEE half (else bfloat16)
  int contiguous;     // table holds one first page per sequence: logical page p of b is table[b] + p
};

// Paged KV copies (append: token tensor -> cache pages; gather: cache pages -> token tensor).
// Token tensors are (B, n, Hkv, D) with element strides; caches (num_pages, page_size, Hkv, D).
struct PagedCopyArgs {
  __bf16* tk;  // keys of the n tokens per sequence (read by append, written by gather)
  __bf16* tv;
  __bf16* kc;  // caches (written by append, read by gather)
  __bf16* vc;
  const int32_t* table;
  const int32_t* ctx;  // tokens per sequence, the appended ones included
  int64_t tk_sb, tk_ss, tk_sh, tv_sb, tv_ss, tv_sh;
  int64_t kc_sp, kc_ss, kc_sh, vc_sp, vc_ss, vc_sh;
  int B, n, Hkv, D, page_size, num_pages, max_pages;
  int gather;
};

// In-place log-sum-exp merge of a partial result (o_part, lse_part) into (o, lse), rows
// (b, s, h) of fp32 O (B, S, H, D) with element strides and fp32 LSE (B, H, S) contiguous;
// optionally also the merged O rounded to bf16 into out (strides r_*).
struct MergeArgs {
  float* o;
  float* lse;
  const float* o_part;
  const float* lse_part;
  __bf16* out;  // NULL: not written
  int64_t o_sb, o_ss, o_sh;
  int64_t p_sb, p_ss, p_sh;
  int64_t r_sb, r_ss, r_sh;
  int B, S, H, rows;
  int out_f16;  // out is IEEE half (else bfloat16)
};

// The backward stores dS = P * (dP - delta) (bf16) once, for the dQ product.  It is kept in
// blocks of kDsKeys keys x kDsRows query rows of one (batch, query head), 8 KB each, stored
// transposed in four quarters of 32 query rows: quarter, then key, then the 32 rows (64
// bytes per key), so the dK/dV step that produces 32 rows of a block writes whole 16-byte
// pieces (ds_elem gives the element offset of (row, key) in a block).  Query tile qt
// (rows 128 qt ..) keeps key blocks ds_kb_lo(qt) .. ds_kb_hi(qt), the only ones that can
// hold a visible pair, packed tile after tile: 4 (qt + 1) blocks for causal attention of a
// whole sequence (tri), else a fixed count cnt per tile.
constexpr int kDsRows = 128;
constexpr int kDsKeys = 32;
constexpr int kDsBlockElems = kDsRows * kDsKeys;

__host__ __device__ constexpr int ds_elem(int row, int key) {
  return (row >> 5) * (32 * kDsKeys) + key * 32 + (row & 31);
}

__host__ __device__ inline int ds_kb_lo(int qt, int causal, int window, int delta) {
  if (!causal || window <= 0) return 0;
  const int lo = qt * kDsRows + delta - window - (kDsRows - 1);  // no visible key below this one
  return lo <= 0 ? 0 : lo / kDsKeys;
}
__host__ __device__ inline int ds_kb_hi(int qt, int causal, int Sk, int delta) {
  const int nkb = (Sk + kDsKeys - 1) / kDsKeys;
  if (!causal) return nkb - 1;
  const int last = qt * kDsRows + (kDsRows - 1) + delta;  // the tile's largest visible key
  const int hi = last < 0 ? -1 : last / kDsKeys;
  return hi < nkb - 1 ? hi : nkb - 1;
}
// dS blocks of one query head of a sequence of len rows in the packed layout.
__host__ __device__ inline int64_t ds_head_blocks(int len, int tri, int cnt) {
  const int64_t n = (len + kDsRows - 1) / kDsRows;
  return tri ? 2 * n * (n + 1) : n * cnt;
}
// Index of block (qt, kb) among the blocks of one (batch, head); -1 if it is not stored.
__host__ __device__ inline int64_t ds_block_index(int qt, int kb, int causal, int window, int delta, int Sk,
                                                  int tri, int cnt) {
  const int lo = ds_kb_lo(qt, causal, window, delta);
  if (kb < lo || kb > ds_kb_hi(qt, causal, Sk, delta) || (!tri && kb - lo >= cnt)) return -1;
  const int64_t first = tri ? 2LL * qt * (qt + 1) : (int64_t)qt * cnt;
  return first + (kb - lo);
}

// Launchers (return the HIP launch status).
hipError_t launch_varlen_prep(const uint8_t* pad_mask, const int32_t* cu_seqlens, int B, int S, int total,
                              int32_t* seq_off, int32_t* seq_len, hipStream_t stream);
// Batch indices by decreasing length (ties by index), from the lengths varlen_prep wrote.
constexpr int kOrderMaxBatch = 4096;  // larger batches keep the plain round order
hipError_t launch_varlen_order(const int32_t* seq_len, int B, int32_t* order, hipStream_t stream);
// First dS block of each packed sequence (prefix sums of Hq * ds_head_blocks(len)); a sequence
// whose region would end past `capacity` blocks gets -1.
hipError_t launch_ds_seq_base(const int32_t* seq_len, int B, int Hq, int tri, int cnt, int64_t capacity,
                              int64_t* ds_seq, hipStream_t stream);
// Debug-mode metadata checks: synchronise the stream and set bad when the metadata is invalid.
hipError_t check_varlen_meta(const uint8_t* pad_mask, const int32_t* cu_seqlens, int B, int S, int total,
                             hipStream_t stream, bool& bad);
hipError_t check_pages_meta(const int32_t* table, int contiguous, const int32_t* ctx, int B, int max_pages,
                            int page_size, int num_pages, hipStream_t stream, bool& bad);
hipError_t launch_fwd(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_fwd_split_merge(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_paged_rank(const int32_t* cu_q, const int32_t* kv_len, int B, int total, int max_q, int max_keys,
                             int32_t* order, hipStream_t stream);
hipError_t launch_bwd_pre(const AttnArgs& a, int D, int rows, hipStream_t stream);
hipError_t launch_bwd_dkdv(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_dq(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_kv_reduce(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_decode_split(const DecodeArgs& a, int D, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, int D, hipStream_t stream);
hipError_t launch_decode_whole(const DecodeArgs& a, int D, hipStream_t stream);
// Device address of the fixed decode scratch on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_lse_merge(const MergeArgs& a, int D, hipStream_t stream);
hipError_t launch_paged_kv_copy(const PagedCopyArgs& a, hipStream_t stream);
// Roofline probes (not on the attention path): 0 matrix rate, 1 streaming read, 2 streaming copy.
hipError_t launch_peak_probe(int kind, void* buf, size_t bytes, int reps, int cus, hipStream_t stream);

// Tile geometry used by the host planner.
constexpr int kFwdRows = 128;   // query rows per forward workgroup
constexpr int kFwdKeys = 32;    // keys per forward step
constexpr int kDqSplit512 = 2;  // head_dim slices of a dQ query tile at head_dim 512
constexpr int kDkdvKeys = 64;   // keys per dK/dV workgroup
constexpr int kDecodeChunk = 512;  // tokens per decode workgroup

}  // namespace attn
