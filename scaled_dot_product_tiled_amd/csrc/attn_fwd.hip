// Fused causal grouped-query attention, forward: O = softmax(scale Q K^T + mask) V and
// the row log-sum-exp, without materialising the score matrix.
//
// The computation is the one the page "Gemma4 FFPA attention backend support for
// accelerating Gemma4-family training" routes head_dim=512 full-attention layers to
// (section Integration) instead of the unfused path that builds the S x S matrix
// (operator table, Debugging notes).
//
// Workgroup = 4 waves = 128 query rows of one kv-head group: `hpt` query heads of the
// group times `mpos` consecutive positions, so one K/V tile in LDS serves every head
// that shares it (grouped-query sharing; the repeat-KV mapping of that page's
// Debugging notes).  Each wave owns 32 rows:
//   S^T (N keys x 32 rows) = K Q^T : A = K rows from LDS, B = the wave's Q rows held
//                                   in registers for the whole key loop;
//   O^T (D x 32 rows) += V^T P^T   : A = V read transposed from LDS, B = P^T straight
//                                   from the S^T accumulator registers.
// Queries sit in lanes, keys and head_dim in registers, so the row max and row sum are
// in-register reductions plus one swap between the two wave halves.  K and V tiles are
// copied memory -> LDS asynchronously; the next K tile loads while P V runs and the
// next V tile while the next Q K^T runs.  Tiles wholly outside the causal / window /
// length range are never visited; tiles that straddle an edge are masked.
//
// Softmax reference.  Exponentials are 2^(s - m) for a per-row reference m (log2
// units) and the output is normalised by the sum of the same exponentials, which is
// exact in real arithmetic for any m.  Two policies:
//  * exact running maximum (head_dim 256): m is the maximum seen so far; when it grows,
//    the accumulators are scaled by 2^(m_old - m_new).  The largest probability of the
//    tile holding the row maximum is then exactly 1, so peaked rows (one key dominating)
//    keep their dominant term exact in bf16.
//  * fixed reference (head_dim 512): m is fixed from the first tile in which the row
//    sees a key.  A tile whose row maximum exceeds m by more than kRefSlack would push
//    the exponentials past 2^kRefSlack; then the whole workgroup raises its references
//    to the maxima seen so far and restarts its key loop from the first tile.  The
//    accumulators are never rescaled: at head_dim 512 they fill the matrix-core
//    accumulator registers and are only ever written by MFMA or cleared.  The dominant
//    probability 2^(s_max - m) is then rounded to the 16-bit type (2^-9 relative in
//    bf16); the normaliser sums the rounded probabilities, so that rounding divides out
//    of a row one key dominates.
// A row that has seen no key yet uses m = 0 (its exponentials are all 2^-inf = 0).
#include "device_common.h"
#include "kernel_args.h"

namespace attn {

// Largest exponent (log2 units) an exponential may reach above the fixed reference: P is
// rounded to the 16-bit type before the P V product, and IEEE half ends at 65504 < 2^16.
constexpr float kRefSlack = 32.0f;
constexpr float kRefSlackF16 = 15.0f;

// Deal of the split paged forward.  Phase A (the first split_nA workgroups) holds every unit's
// query-tile items in blocks of 32, the blocks of the units ranked by decreasing work (order: the
// sequences by new rows x cached keys) dealt to the XCDs in a snake order (workgroup k runs on XCD
// k mod 8), so that a long prompt's tiles fill whole XCDs first and each XCD's L2 serves few
// units' keys; phase B holds the pieces of split decode rows, round-robin over the units, dealt
// after every tile.  Returns the item (unit * nqt + slot) or -1.
__device__ __forceinline__ int paged_split_item(const AttnArgs& a) {
  const int W = a.nqt, W0 = a.split_slot0, U = a.total_items / W;
  const int k = blockIdx.x;
  if (k >= a.split_nA) {
    const int kb = k - a.split_nA;
    if (kb >= U * kSplitMax) return -1;
    const int round = kb / U;
    return ((kb + round) % U) * W + W0 + round;
  }
  const int NB = (W0 + 31) / 32;  // blocks per unit
  const int x = k & 7, p = k >> 3, j = p >> 5, s = p & 31;
  const int rho = 8 * j + ((j & 1) ? 7 - x : x);
  if (rho >= U * NB) return -1;
  const int ur = rho / NB, slot = (rho - ur * NB) * 32 + s;
  if (slot >= W0) return -1;
  const int upb = a.Hkv * a.nhb;
  return (a.order[ur / upb] * upb + ur % upb) * W + slot;
}

// MERGE: instead of storing the row's O and LSE, merge them into a running result (fp32 O
// in out_f32, LSE in lse) by log-sum-exp weighting and optionally round the merged O to the
// 16-bit out: the chunk-pair forward and the merge of its partial in one pass.
// PAGED: K and V come from a paged cache through the page table (see AttnArgs::paged).
template <int D, int N, bool EXACT, bool SOFTCAP, bool F16, bool MERGE, bool PAGED>
__device__ __forceinline__ void fwd_body(AttnArgs a) {
  constexpr int NKB = N / 32;  // 32-key blocks per tile
  constexpr int NS = N / 16;   // 16-key steps per tile
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NDMA = dma_rows_per_wave<D, N, 4>();
  __shared__ __attribute__((aligned(1024))) bf16 Ks[N * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[N * D];
  __shared__ int restart_flag[2][4];

  const int item = (PAGED && a.split_nA > 0) ? paged_split_item(a)
                                             : xcd_item(a.per_xcd, a.total_items, a.nqt, a.balanced, a.order,
                                                        a.Hkv * a.nhb);
  if (item < 0) return;
  const int unit = item / a.nqt;
  int qt = a.nqt - 1 - (item - unit * a.nqt);  // longest causal rows first
  const int hb = unit % a.nhb;
  const int g = (unit / a.nhb) % a.Hkv;
  const int b = unit / (a.nhb * a.Hkv);
  int len, off;
  if constexpr (PAGED) {
    // query rows straight from the offsets: sequence b owns rows cu[b] .. cu[b+1]-1, clamped into
    // the packed rows (cu is a.seq_off, B + 1 entries)
    off = min(max(a.seq_off[b], 0), a.total);
    len = min(max(a.seq_off[b + 1] - off, 0), a.total - off);
  } else {
    len = a.seq_len ? a.seq_len[b] : a.S;
    off = a.seq_off ? a.seq_off[b] : 0;
  }
  len = min(max(len, 0), a.S);
  // key rows; a paged sequence's are its cached keys, clamped to its table row, and its
  // queries are the newest of them
  const int lenk = PAGED ? min(max(a.kv_len[b], 0), a.max_pages * 16) : a.seq_len ? len : a.Sk;
  const int dlt = PAGED ? lenk - len : a.q_shift;
  [[maybe_unused]] int piece = -1, piece_t0 = 0, piece_ch = 0;  // split decode row: its key tiles
  if constexpr (PAGED) {
    // The unit's r-th item takes the r-th tile counted back from the sequence's last row, so
    // that every sequence's heaviest tile (its newest queries see the most keys) comes in the
    // first round of the deal, decode rows included; items past the sequence's rows exit.  The
    // pieces of a split decode row take the unit's items split_slot0 + p, past every sequence's
    // query tiles, so that they are dealt after the long tiles of the prompt chunks and fill the
    // compute units those leave.
    const int slot = a.nqt - 1 - qt;
    qt = (len + a.mpos - 1) / a.mpos - 1 - slot;
    if (a.split_o != nullptr && len == 1) {
      const int np = decode_pieces(lenk, a.window, piece_t0, piece_ch);
      if (np > 1) {
        piece = slot - a.split_slot0;
        if (piece < 0 || piece >= np) return;
        qt = 0;
      }
    }
    if (qt < 0) return;
  }

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g2 = lane >> 5, ln = lane & 31;
  const int R = wave * 32 + ln;
  const int hh = R / a.mpos;
  const int p0 = qt * a.mpos;
  const int pos = p0 + (R - hh * a.mpos);
  const int h = g * a.r + hb * a.hpt + hh;

  bf16x8 qreg[KS];
  {
    // Rows past the length read a valid row (never past the tensor) and are zeroed.
    const int prow = min(pos, max(len - 1, 0));
    const bf16* qp = a.q + b * a.q_sb + (int64_t)(off + prow) * a.q_ss + h * a.q_sh + 8 * g2;
    const bool ok = pos < len;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const bf16x8 x = ldg8(qp + 16 * t);
      qreg[t] = ok ? x : zero_bf16x8();
    }
  }

  const int plast = min(p0 + a.mpos, len) - 1;
  const int jhi = (plast < p0) ? 0 : (a.causal ? min(plast + dlt + 1, lenk) : lenk);
  const int jlo = a.window > 0 ? max(0, p0 + dlt - a.window + 1) : 0;
  int t_lo = jlo / N;
  int t_hi = jhi > jlo ? (jhi + N - 1) / N : t_lo;
  if constexpr (PAGED) {
    if (piece >= 0) {  // the same tiles decode_pieces cut (N = 32)
      t_lo = piece_t0 + piece * piece_ch;
      t_hi = min(t_hi, t_lo + piece_ch);
    }
  }

  const bf16* kbase = a.k + (PAGED ? 0 : b * a.k_sb + (int64_t)off * a.k_ss) + g * a.k_sh;
  const bf16* vbase = a.v + (PAGED ? 0 : b * a.v_sb + (int64_t)off * a.v_ss) + g * a.v_sh;
  [[maybe_unused]] const int32_t* trow = PAGED ? a.table + (int64_t)b * a.max_pages : nullptr;
  static_assert(!PAGED || N == 32, "a paged tile spans two pages");
  [[maybe_unused]] int phys[2] = {0, 0};  // physical pages of the tile being copied (paged)
  const RowFrags<D> rowf(lane);
  const TrFrags<D> trf(lane);
  const float c = a.c;

  f32x16 oacc[DB];
  float m_ref = -INFINITY, l_run = 0.f;
  bool restart = true;
  while (restart) {
    restart = false;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    l_run = 0.f;
    if (t_lo < t_hi) {
      if constexpr (PAGED) {
        table_pages2(phys, trow, t_lo * N, lenk - t_lo * N);
        dma_rows_paged<D, N, 4>(Ks, paged_tile_src<N>(kbase, a.k_sb, a.k_ss, phys, a.num_pages, lenk - t_lo * N),
                                wave, lane);
        dma_rows_paged<D, N, 4>(Vs, paged_tile_src<N>(vbase, a.v_sb, a.v_ss, phys, a.num_pages, lenk - t_lo * N),
                                wave, lane);
      } else {
        dma_rows<D, N, 4>(Ks, tile_src<N>(kbase, a.k_ss, t_lo * N, lenk - t_lo * N), wave, lane);
        dma_rows<D, N, 4>(Vs, tile_src<N>(vbase, a.v_ss, t_lo * N, lenk - t_lo * N), wave, lane);
      }
    }
    // Copies after the first tile's (non-paged, head_dim 512): the next K tile's row copies are
    // spread over this tile's P V products and this tile's V copies over its Q K^T products, one
    // per two matrix instructions, so that the four waves do not queue their copies on the load
    // path all at once (issued back to back, a wave's eight copies took about 650 cycles to
    // leave it; spread: 1.22 -> 1.19 ms on B2 S4096).  The first tile's K and V are copied above,
    // back to back.  At head_dim 256 the spread copies' registers spill and two workgroups per
    // compute unit already overlap each other's copies: it stays with the bursts.
    constexpr bool SPREAD = !PAGED && D == 512;
    for (int jt = t_lo; jt < t_hi; ++jt) {
      const int j0 = jt * N;
      const bool has_next = jt + 1 < t_hi;
      if (SPREAD && jt != t_lo)
        wait_vmcnt<0>();  // K(jt) has landed (V(jt) is copied below)
      else
        wait_vmcnt<NDMA>();  // K(jt) has landed; V(jt) may still be in flight
      barrier_lds();
      TileSrc vsrc{};
      if constexpr (SPREAD) vsrc = tile_src<N>(vbase, a.v_ss, j0, lenk - j0);
      const bool copy_v = SPREAD && jt != t_lo;

      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      {
        // K fragments are read KPF steps ahead of the matrix core (three at head_dim 512, where
        // one wave per SIMD must hide the LDS latency alone: 5-6% faster than two; two at 256,
        // where a third spills); the schedule barrier keeps the compiler from hoisting every
        // read (and its registers) to the top.
        constexpr int KPF = D == 512 ? 3 : 2;
        bf16x8 kf[KPF + 1][NKB];
#pragma unroll
        for (int t = 0; t < KPF; ++t)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) kf[t][kb] = rowf.read(Ks, kb * 32, t);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          if (t + KPF < KS) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kf[(t + KPF) % (KPF + 1)][kb] = rowf.read(Ks, kb * 32, t + KPF);
          }
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) sacc[kb] = E16<F16>::mma32(kf[t % (KPF + 1)][kb], qreg[t], sacc[kb]);
          if (copy_v && (t & 1) == 0 && t / 2 < NDMA) dma_rows_one<D, N, 4>(Vs, vsrc, wave, lane, t / 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // The next K tile is copied once every wave is past the barrier below (which every wave
      // reaches after its S reads of Ks), so that one barrier per tile serves both.
      auto copy_next_k = [&]() __attribute__((always_inline)) {
        if constexpr (PAGED) {
          if (has_next) {
            table_pages2(phys, trow, j0 + N, lenk - j0 - N);  // the next tile's pages, for K and V
            dma_rows_paged<D, N, 4>(Ks, paged_tile_src<N>(kbase, a.k_sb, a.k_ss, phys, a.num_pages, lenk - j0 - N),
                                    wave, lane);
          }
        } else {
          if (!SPREAD && has_next) dma_rows<D, N, 4>(Ks, tile_src<N>(kbase, a.k_ss, j0 + N, lenk - j0 - N), wave, lane);
        }  // (SPREAD: copied during the P V products below)
      };

      if constexpr (SOFTCAP) {
        // the cap applies to every score before the mask (masked entries become -inf below)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] = a.sc_out * tanh_from_exp(sacc[kb][r] * a.sc_in);
      }
      const bool need_mask = (j0 + N > lenk) || (p0 + a.mpos > len) || (a.causal && j0 + N - 1 > p0 + dlt) ||
                             (a.window > 0 && j0 <= plast + dlt - a.window);
      if (need_mask) {
        // the row's visible keys are one interval [lo, hi]; per 32-key block it becomes a 32-bit
        // mask (bit t: key j0 + 32 kb + t), and register r tests bit 8 (r/4) + 4 g2 + r%4
        const int ip = pos + dlt;
        const int hi = a.causal ? min(lenk - 1, ip) : lenk - 1;
        const int lo = a.window > 0 ? ip - a.window + 1 : 0;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int jb = j0 + 32 * kb;
          const int nh = min(max(hi - jb + 1, 0), 32), nl = min(max(lo - jb, 0), 32);
          const uint32_t mh = (uint32_t)((1ull << nh) - 1), ml = (uint32_t)((1ull << nl) - 1);
          const uint32_t vis = (pos < len ? (mh & ~ml) : 0u) >> (4 * g2);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((vis >> (8 * (r >> 2) + (r & 3))) & 1u)) sacc[kb][r] = -INFINITY;
        }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = half_swap_max(mt) * c;
      if constexpr (EXACT) {
        const float mnew = fmaxf(m_ref, mt);
        const bool need = mnew > m_ref;
        if (__any(need)) {
          const float alpha = need ? fast_exp2(m_ref - mnew) : 1.0f;  // 2^-inf = 0 for a first key
          m_ref = mnew;
          l_run *= alpha;
#pragma unroll
          for (int d = 0; d < DB; ++d) oacc[d] *= alpha;
        }
        wait_vmcnt<0>();  // V(jt) has landed (K(jt+1) is not issued yet)
        barrier_lds();     // V(jt) visible to every wave; every wave is done with Ks
        copy_next_k();
      } else {
        // A row's first visible keys fix its reference (its accumulators are still zero).
        if (m_ref == -INFINITY) m_ref = mt;
        const bool need = mt > m_ref + (F16 ? kRefSlackF16 : kRefSlack);
        const bool wave_need = __any(need);
        if (lane == 0) restart_flag[jt & 1][wave] = wave_need ? 1 : 0;

        wait_vmcnt<0>();  // V(jt) has landed (K(jt+1) is not issued yet)
        barrier_lds();     // the flags and V(jt) visible to every wave; every wave is done with Ks
        if (restart_flag[jt & 1][0] | restart_flag[jt & 1][1] | restart_flag[jt & 1][2] |
            restart_flag[jt & 1][3]) {
          m_ref = fmaxf(m_ref, mt);
          restart = true;
          if (a.restarts != nullptr && threadIdx.x == 0) atomicAdd(a.restarts, 1);
          wait_vmcnt<0>();
          barrier_lds();  // no wave still reads Ks / Vs before they are refilled
          break;
        }
        copy_next_k();
      }

      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      // P is rounded to the 16-bit type for the P V product, and the normaliser sums the same
      // rounded values, so that the weights applied to V sum to exactly one: a dominant term
      // far above the reference then divides out instead of carrying its rounding into O.
      float rs = 0.f;
      bf16x8 pb[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + e], c, -m_use));  // masked: 2^-inf = 0
          pb[s][e] = E16<F16>::from_float(p);
          rs += E16<F16>::to_float(pb[s][e]);
        }
      l_run += half_swap_sum(rs);
      {
        // V^T fragments in (d block, key step) order, read VPF ahead of the matrix core.
        constexpr int NF = DB * NS;
        constexpr int VPF = D == 512 ? 3 : 2;
        bf16x8 vf[VPF + 1];
        TileSrc ksrc{};  // the next K tile
        if constexpr (SPREAD) ksrc = tile_src<N>(kbase, a.k_ss, j0 + N, lenk - j0 - N);
        const bool copy_k = SPREAD && has_next;
        static_assert(2 * NDMA <= NF && 2 * NDMA <= KS, "every copy needs a slot in the matrix loops");
#pragma unroll
        for (int f = 0; f < VPF; ++f) vf[f] = trf.read(Vs, 16 * (f % NS), f / NS);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f + VPF < NF) vf[(f + VPF) % (VPF + 1)] = trf.read(Vs, 16 * ((f + VPF) % NS), (f + VPF) / NS);
          oacc[f / NS] = E16<F16>::mma32(vf[f % (VPF + 1)], pb[f % NS], oacc[f / NS]);
          if (copy_k && (f & 1) == 0 && f / 2 < NDMA) dma_rows_one<D, N, 4>(Ks, ksrc, wave, lane, f / 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // Every wave is done with Vs before V(jt+1) is copied: with the copies spread, V(jt+1) is
      // copied after the next tile's first barrier, which every wave reaches after these reads.
      if constexpr (!SPREAD) barrier_lds();
      if constexpr (PAGED) {
        if (has_next)
          dma_rows_paged<D, N, 4>(Vs, paged_tile_src<N>(vbase, a.v_sb, a.v_ss, phys, a.num_pages, lenk - j0 - N),
                                  wave, lane);
      } else {
        if (!SPREAD && has_next) dma_rows<D, N, 4>(Vs, tile_src<N>(vbase, a.v_ss, j0 + N, lenk - j0 - N), wave, lane);
      }
    }
  }

  const bool wrow = a.packed ? (pos < len) : (pos < a.S);
  if (wrow) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    const int64_t oo = b * a.o_sb + (int64_t)(off + pos) * a.o_ss + h * a.o_sh + 4 * g2;
    if constexpr (MERGE) {
      const int64_t li = b * a.st_sb + h * a.st_sh + off + pos;
      // Both lanes of the row read its running LSE before the first one stores the merged
      // value (one wave, loads before the store in program order).  The running O is read
      // only where it has weight, so the first merge may start from LSE = -inf and any O.
      const float lp = l_run > 0.f ? kLn2 * (m_ref + __log2f(l_run)) : -INFINITY;
      const MergeWeights w = lse_merge_weights(a.lse[li], lp);
      float* ro = a.out_f32 + oo;
      bf16* r16 = a.out ? a.out + b * a.r_sb + (int64_t)(off + pos) * a.r_ss + h * a.r_sh + 4 * g2 : nullptr;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int qa = 0; qa < 4; ++qa) {
          float* p = ro + 32 * d + 8 * qa;
          float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
          if (w.w1 > 0.f) x = *reinterpret_cast<const float4*>(p);
          const float y0 = lse_merge_value(w, x.x, oacc[d][4 * qa] * inv);
          const float y1 = lse_merge_value(w, x.y, oacc[d][4 * qa + 1] * inv);
          const float y2 = lse_merge_value(w, x.z, oacc[d][4 * qa + 2] * inv);
          const float y3 = lse_merge_value(w, x.w, oacc[d][4 * qa + 3] * inv);
          stg4(p, y0, y1, y2, y3);
          if (r16) stg4e<F16>(r16 + 32 * d + 8 * qa, y0, y1, y2, y3);
        }
      if (g2 == 0) a.lse[li] = w.lse;
    } else {
      auto store = [&](auto* op) {
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int qa = 0; qa < 4; ++qa)
            st4<F16>(op + 32 * d + 8 * qa, oacc[d][4 * qa] * inv, oacc[d][4 * qa + 1] * inv,
                     oacc[d][4 * qa + 2] * inv, oacc[d][4 * qa + 3] * inv);
      };
      float* o32 = a.out_f32 ? a.out_f32 + oo : nullptr;
      float* lp = a.lse + (b * a.st_sb + h * a.st_sh + off + pos);
      bool ninf = a.empty_lse_ninf;
      if constexpr (PAGED) {
        if (piece >= 0) {
          // a piece of a split decode row: its normalised O in fp32 and its LSE (-inf without a
          // visible key), for fwd_split_merge
          const int64_t pi = ((int64_t)unit * kSplitMax + piece) * a.hpt + hh;
          o32 = a.split_o + pi * D + 4 * g2;
          lp = a.split_lse + pi;
          ninf = true;
        }
      }
      if (o32)
        store(o32);  // a partial over one key chunk: rounded once, when the partials are merged
      else
        store(a.out + oo);
      if (g2 == 0) *lp = l_run > 0.f ? kLn2 * (m_ref + __log2f(l_run)) : (ninf ? -INFINITY : 0.f);
    }
  }
}

// At head_dim 256 a wave fits in 256 registers, so two workgroups share a compute unit and
// one's softmax and barriers overlap the other's matrix work; at 512 the accumulators alone
// take 256 registers.
template <int D, int N, bool EXACT, bool SOFTCAP, bool F16>
__global__ __launch_bounds__(256, D == 256 ? 2 : 1) void fwd_kernel(AttnArgs a) {
  fwd_body<D, N, EXACT, SOFTCAP, F16, false, false>(a);
}

template <int D, int N, bool EXACT, bool SOFTCAP, bool F16>
__global__ __launch_bounds__(256, D == 256 ? 2 : 1) void fwd_merge_kernel(AttnArgs a) {
  fwd_body<D, N, EXACT, SOFTCAP, F16, true, false>(a);
}

template <int D, int N, bool EXACT, bool SOFTCAP, bool F16>
__global__ __launch_bounds__(256, D == 256 ? 2 : 1) void fwd_paged_kernel(AttnArgs a) {
  fwd_body<D, N, EXACT, SOFTCAP, F16, false, true>(a);
}

// Merge of the pieces of split decode rows (paged forward).  One wave per (sequence, query head);
// a row that was not split exits.  Over the row's pieces p, in piece order:
//   L = ln sum_p e^LSE_p,  O = sum_p e^(LSE_p - L) O_p,
// the log-sum-exp combination of partial results over disjoint key sets; O is rounded to the
// 16-bit type.  Every piece holds a visible key, so L is finite for finite scores.
template <int D, bool F16>
__global__ __launch_bounds__(256) void fwd_split_merge_kernel(AttnArgs a) {
  constexpr int E = D / 64;  // elements per lane
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= a.B * a.Hq) return;
  const int b = w / a.Hq, h = w - b * a.Hq;
  const int off = min(max(a.seq_off[b], 0), a.total);
  const int len = min(min(max(a.seq_off[b + 1] - off, 0), a.total - off), a.S);
  if (len != 1) return;
  const int lenk = min(max(a.kv_len[b], 0), a.max_pages * 16);
  int t0, ch;
  const int np = decode_pieces(lenk, a.window, t0, ch);
  if (np <= 1) return;
  const int g = h / a.r, hg = h - g * a.r;
  const int unit = (b * a.Hkv + g) * a.nhb + hg / a.hpt;
  const int64_t i0 = (int64_t)unit * kSplitMax * a.hpt + hg % a.hpt;  // piece p: i0 + p hpt
  // lane p < np holds piece p's LSE and then its weight
  const float lp = lane < np ? a.split_lse[i0 + lane * a.hpt] : -INFINITY;
  float m = lp;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
  const float wl = (lane < np && m > -INFINITY) ? expf(lp - m) : 0.f;
  float sum = 0.f;
  for (int p = 0; p < np; ++p) sum += __shfl(wl, p);  // piece order
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const float* src = a.split_o + i0 * D + E * lane;
#pragma unroll 4
  for (int p = 0; p < np; ++p) {
    const float wt = __shfl(wl, p);
#pragma unroll
    for (int e = 0; e < E / 4; ++e) {
      const float4 x = reinterpret_cast<const float4*>(src + (int64_t)p * a.hpt * D)[e];
      acc[4 * e] += wt * x.x;
      acc[4 * e + 1] += wt * x.y;
      acc[4 * e + 2] += wt * x.z;
      acc[4 * e + 3] += wt * x.w;
    }
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  auto* op = a.out + b * a.o_sb + (int64_t)off * a.o_ss + h * a.o_sh + E * lane;
#pragma unroll
  for (int e = 0; e < E / 4; ++e)
    st4<F16>(op + 4 * e, acc[4 * e] * inv, acc[4 * e + 1] * inv, acc[4 * e + 2] * inv, acc[4 * e + 3] * inv);
  if (lane == 0) a.lse[b * a.st_sb + h * a.st_sh + off] = sum > 0.f ? m + logf(sum) : 0.f;
}

hipError_t launch_fwd_split_merge(const AttnArgs& a, int D, hipStream_t stream) {
  const dim3 grid((a.B * a.Hq + 3) / 4), block(256);
  if (D == 512 && a.f16)
    hipLaunchKernelGGL((fwd_split_merge_kernel<512, true>), grid, block, 0, stream, a);
  else if (D == 512)
    hipLaunchKernelGGL((fwd_split_merge_kernel<512, false>), grid, block, 0, stream, a);
  else if (D == 256 && a.f16)
    hipLaunchKernelGGL((fwd_split_merge_kernel<256, true>), grid, block, 0, stream, a);
  else if (D == 256)
    hipLaunchKernelGGL((fwd_split_merge_kernel<256, false>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D, bool EXACT, bool SOFTCAP, bool F16>
void launch_fwd_one(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(8 * a.per_xcd), block(256);
  if (a.paged)
    hipLaunchKernelGGL((fwd_paged_kernel<D, kFwdKeys, EXACT, SOFTCAP, F16>), grid, block, 0, stream, a);
  else if (a.merge)
    hipLaunchKernelGGL((fwd_merge_kernel<D, kFwdKeys, EXACT, SOFTCAP, F16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_kernel<D, kFwdKeys, EXACT, SOFTCAP, F16>), grid, block, 0, stream, a);
}

template <bool F16>
hipError_t launch_fwd_t(const AttnArgs& a, int D, hipStream_t stream) {
  const bool sc = a.softcap > 0.f;
  if (D == 512 && !sc)
    launch_fwd_one<512, false, false, F16>(a, stream);
  else if (D == 512)
    launch_fwd_one<512, false, true, F16>(a, stream);
  else if (D == 256 && !sc)
    launch_fwd_one<256, true, false, F16>(a, stream);
  else if (D == 256)
    launch_fwd_one<256, true, true, F16>(a, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, int D, hipStream_t stream) {
  return a.f16 ? launch_fwd_t<true>(a, D, stream) : launch_fwd_t<false>(a, D, stream);
}

}  // namespace attn
