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
struct AttnArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  __bf16* out;  // forward: O; backward: dQ
  __bf16* dk;
  __bf16* dv;
  float* lse;   // forward writes, backward reads
  float* delta;  // backward: rowsum(dO * O)
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
  int hpt, mpos, nhb, nqt;  // heads per tile, positions per tile, head blocks, q tiles
  int nkt;                  // key tiles (dK/dV kernel)
  int packed;               // rows past a sequence's length do not exist
  int causal, window;
  float scale;              // multiplies Q K^T
  float c;                  // scale * log2(e)
  int per_xcd, total_items;
};

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
};

// Launchers (return the HIP launch status).
hipError_t launch_varlen_prep(const uint8_t* pad_mask, const int32_t* cu_seqlens, int B, int S,
                              int32_t* seq_off, int32_t* seq_len, hipStream_t stream);
hipError_t launch_fwd(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_pre(const AttnArgs& a, int D, int rows, hipStream_t stream);
hipError_t launch_bwd_dkdv(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_dq(const AttnArgs& a, int D, hipStream_t stream);
hipError_t launch_decode_split(const DecodeArgs& a, int D, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, int D, hipStream_t stream);

// Tile geometry used by the host planner.
constexpr int kFwdRows = 128;   // query rows per forward workgroup
constexpr int kFwdKeys = 32;    // keys per forward step
constexpr int kDkdvKeys = 64;   // keys per dK/dV workgroup
constexpr int kDkdvRows = 32;   // query rows per dK/dV step
constexpr int kDqRows = 64;     // query rows per dQ workgroup
constexpr int kDqKeys = 32;     // keys per dQ step
constexpr int kDecodeChunk = 512;  // tokens per decode workgroup

}  // namespace attn
