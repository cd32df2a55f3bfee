// Fused causal grouped-query attention, backward: gradients of sum(O * dO) with
// respect to Q, K and V, from the forward's saved O and LSE (the page "Gemma4 FFPA
// attention backend support for accelerating Gemma4-family training", section Results,
// keeps the forward's outputs for the backward instead of replaying it).
//
// With P = exp(scale Q K^T - LSE) (masked entries 0), dP = dO V^T, delta = rowsum(dO * O)
// and dS = P * (dP - delta):  dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
// Three kernels run in stream order:
//   bwd_pre   delta per (query row, head), fp32;
//   bwd_dkdv  one workgroup per (batch, kv head, 64-key tile): K and V of the tile stay
//             in registers, every visible query tile (32 rows; 64 at head_dim 256) of
//             every query head of the group streams through LDS, and dK, dV accumulate
//             in registers (no atomics,
//             one pass over the group's heads, so the grouped-query sum is exact).  It
//             also stores dS (bf16) in blocks, so that dQ needs no second pass over
//             Q K^T and dO V^T;
//   bwd_dq    one workgroup per (batch, query head, 128 query rows): dQ = scale dS K as
//             a plain product over the stored dS blocks and 32-key blocks of K.
// Masked entries become exact zeros by selection, never by multiplication, so a
// non-finite value outside the visible region cannot reach a gradient (the page "Root
// cause analysis: Gemma4 sliding-window BF16 cuDNN SDPA NaN on H100" traces non-finite
// dQ/dK/dV from finite dO in a masked sliding-window backward).
//
// Inside the dK/dV kernel the four waves split by role: two "score" waves compute
// S = Q K^T for one 32-key block each and two "dP" waves compute dO V^T for the same
// blocks; dP crosses to the score wave through LDS, the score wave forms P and dS, and
// every wave then owns a quarter of head_dim for the two gradient products.
#include "device_common.h"
#include "kernel_args.h"

namespace attn {

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <int D, bool F16>
__global__ __launch_bounds__(256) void bwd_pre_kernel(AttnArgs a, int rows) {
  // A quarter wave per row, 16-byte loads: 16 (head_dim 256) or 32 (512) elements per lane.
  constexpr int LPR = 16;
  constexpr int NV = D / (8 * LPR);  // 16-byte vectors per lane and tensor
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= rows) return;
  const int lane = threadIdx.x & (LPR - 1);
  int b, pos, h, len;
  if (a.packed) {
    // packed rows: batch stride and per-sequence offset are folded into the row index
    const int t = row / a.Hq;
    h = row - t * a.Hq;
    b = 0;
    pos = t;
    len = t + 1;
  } else {
    h = row % a.Hq;
    const int bp = row / a.Hq;
    pos = bp % a.S;
    b = bp / a.S;
    len = a.seq_len ? min(max(a.seq_len[b], 0), a.S) : a.S;
  }
  float acc = 0.f;
  if (pos < len) {
    const bf16* op = a.o + b * a.o_sb + (int64_t)pos * a.o_ss + h * a.o_sh + lane * 8 * NV;
    const bf16* dp = a.dout + b * a.do_sb + (int64_t)pos * a.do_ss + h * a.do_sh + lane * 8 * NV;
    bf16x8 ov[NV], dv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      ov[v] = ldg8(op + 8 * v);
      dv[v] = ldg8(dp + 8 * v);
    }
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += E16<F16>::to_float(ov[v][e]) * E16<F16>::to_float(dv[v][e]);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);  // within the row's 16 lanes
  if (lane == 0) a.delta[b * a.st_sb + h * a.st_sh + pos] = acc;
}

template <bool F16>
hipError_t launch_bwd_pre_t(const AttnArgs& a, int D, int rows, hipStream_t stream) {
  const dim3 grid((rows + 15) / 16), block(256);
  if (D == 512)
    hipLaunchKernelGGL((bwd_pre_kernel<512, F16>), grid, block, 0, stream, a, rows);
  else if (D == 256)
    hipLaunchKernelGGL((bwd_pre_kernel<256, F16>), grid, block, 0, stream, a, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const AttnArgs& a, int D, int rows, hipStream_t stream) {
  return a.f16 ? launch_bwd_pre_t<true>(a, D, rows, stream) : launch_bwd_pre_t<false>(a, D, rows, stream);
}

// Row statistics (LSE * log2 e and delta) of query rows i0 .. i0+31 of head h into LDS:
// 32 floats of LSE then 32 of delta, one 4-byte DMA lane each.
__device__ __forceinline__ void dma_stats(float* dst, const float* lse_row0, const float* delta_row0, int i0,
                                          int imax, int lane) {
  const int i = min(i0 + (lane & 31), imax);
  const float* src = (lane < 32 ? lse_row0 : delta_row0) + i;
  lds_dma4(dst, src);
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D, bool SOFTCAP, bool F16>
__global__ __launch_bounds__(256, D == 256 ? 2 : 1) void bwd_dkdv_kernel(AttnArgs a) {
  constexpr int NK = kDkdvKeys;   // 64 keys per workgroup
  // query rows per step: one block of 32.  At head_dim 256 two workgroups share a compute unit
  // (LOWREG: 256 registers and 74 KB of LDS each), so that one's softmax, exchange and barriers
  // overlap the other's matrix work.
  constexpr int RB = 1;
  constexpr bool LOWREG = D == 256;
  constexpr bool DMA_EARLY = false;
  constexpr int MQ = 32 * RB;
  constexpr int KS = D / 16;
  constexpr int DBW = D / 128;    // 32-wide d blocks owned by each wave
  constexpr int NDMA = dma_rows_per_wave<D, MQ, 4>();
  static_assert(NK == 64, "role split assumes 2 key blocks");
  __shared__ __attribute__((aligned(1024))) bf16 Qs[2][MQ * D];
  __shared__ __attribute__((aligned(1024))) bf16 dOs[2][MQ * D];
  __shared__ __attribute__((aligned(16))) float stat[2][64 * RB];         // per 32-row block: LSE, delta
  // S / dP exchange, [rb][kb][0: dP of registers 0..7 for the score wave, 1: S of registers
  // 8..15 for the dP wave][reg/4 (mod 2)][lane].  Once a wave has read its half it writes its
  // P and dS fragments over it (P at [0], dS at [1]): only that wave reads that half.
  __shared__ __attribute__((aligned(16))) f32x4 xch[RB][2][2][2][64];

  const int item = xcd_item(a.per_xcd, a.total_items, a.nkt * a.kv_split, a.balanced, a.order, a.Hkv);
  if (item < 0) return;
  const int unit = item / (a.nkt * a.kv_split);
  const int rem = item - unit * (a.nkt * a.kv_split);
  const int kt = rem / a.kv_split;  // low key tiles see the most query rows: first
  const int part = rem - kt * a.kv_split;
  const int g = unit % a.Hkv;
  // the query heads of the group this workgroup visits: all of them, or one of kv_split
  // equal parts (then its dK, dV are partial sums, added by a separate reduction)
  const int rs = a.r / a.kv_split;
  const int hb0 = g * a.r + part * rs;
  const int b = unit / a.Hkv;
  int len = a.seq_len ? a.seq_len[b] : a.S;
  len = min(max(len, 0), a.S);
  // packed rows: this sequence's dS region (a sequence that does not fit is skipped)
  const int64_t ds_b = a.ds_seq ? a.ds_seq[b] : 0;
  if (ds_b < 0) len = 0;
  const int lenk = a.seq_len ? len : a.Sk;  // key rows
  const int dlt = a.q_shift;
  const int off = a.seq_off ? a.seq_off[b] : 0;
  const int j0 = kt * NK;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g2 = lane >> 5, ln = lane & 31;
  const bool score_wave = wave < 2;
  const int kb = wave & 1;            // key block of this wave's score / dP product
  const int dsl = wave * DBW;         // first d block of this wave's gradient slice

  f32x16 dvacc[2][DBW], dkacc[2][DBW];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int d = 0; d < DBW; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) dvacc[x][d][r] = dkacc[x][d][r] = 0.f;

  // query range that sees any key of the tile
  const int qlo = a.causal ? max(j0 - dlt, 0) : 0;
  int qhi = len;
  if (a.window > 0) qhi = min(qhi, j0 + NK - 1 + a.window - dlt);
  const int tq0 = qlo / MQ;
  const int nq = (j0 < lenk && qhi > qlo) ? (qhi + MQ - 1) / MQ - tq0 : 0;
  const int nsteps = rs * nq;

  if (nsteps > 0) {
    // this wave's 32 keys of K (score waves) or V (dP waves) as B operands
    bf16x8 kv[KS];
    {
      const int key = j0 + 32 * kb + ln;
      const bool ok = key < lenk;
      const int krow = min(key, lenk - 1);
      const bf16* src = score_wave ? a.k + b * a.k_sb + (int64_t)(off + krow) * a.k_ss + g * a.k_sh
                                   : a.v + b * a.v_sb + (int64_t)(off + krow) * a.v_ss + g * a.v_sh;
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const bf16x8 x = ldg8(src + 16 * t + 8 * g2);
        kv[t] = ok ? x : zero_bf16x8();
      }
    }
    const float c = a.c;

    // Step k = (query tile, head), query tiles from the last one down and heads innermost:
    // every workgroup of this (batch, kv head) starts at the same tile and advances at the
    // same pace, so the workgroups sharing an XCD read each Q / dO tile while it is in L2.
    // The copies of step k+1 (Q and dO tiles: NDMA row copies each per wave) are spread
    // over the matrix loop of step k, one every two matrix instructions, so the load path
    // is busy while the matrix cores are, and so is the small row-statistics copy.
    const int tq_last = tq0 + nq - 1;
    static_assert(2 * NDMA <= KS * RB / 2, "every copy needs a slot in the S / dP loop");
    // Row tiles are visited from the last one down (heads innermost).  With a window every key
    // tile sees the same number nq of row tiles, each key tile's range two tiles above its
    // neighbour's, so a plain top-down visit would have the workgroups of a unit read tiles
    // spread over the whole sequence at every step.  Instead the visit starts at a rotated tile
    // and wraps from the first tile to the last: step k then reads an absolute tile congruent to
    // -k/rs modulo nq in every workgroup, a handful of distinct tiles that the XCD's L2 serves.
    // Without a window every key tile's range ends at the same last tile and the plain visit
    // already keeps the workgroups together.
    const int phase = a.window > 0 ? tq_last % nq : 0;
    int tcur = tq_last - phase;  // row tile of step k
    int hi = 0;                  // head of step k
    // Addresses of step k: Q and dO at (row i0, head hb0 + hi), the row statistics and the dS
    // blocks of that head.  A step advances one head, or after the group's last head returns
    // to head hb0 one query tile lower (or, at the wrap, to the last tile).
    const int i00 = tcur * MQ;
    const bf16* qrow = a.q + b * a.q_sb + (int64_t)(off + i00) * a.q_ss + hb0 * a.q_sh;
    const bf16* drow = a.dout + b * a.do_sb + (int64_t)(off + i00) * a.do_ss + hb0 * a.do_sh;
    int64_t so = b * a.st_sb + hb0 * a.st_sh + off;
    const int64_t ds_hb = a.ds_seq ? ds_head_blocks(len, a.ds_tri, a.ds_cnt) : a.ds_head;
    bf16* dshead = a.dsb + ((a.ds_seq ? ds_b : (int64_t)b * a.Hq * ds_hb) + (int64_t)hb0 * ds_hb) * kDsBlockElems;
    const int64_t q_back = -(int64_t)(rs - 1) * a.q_sh;  // from the last head back to the first
    const int64_t d_back = -(int64_t)(rs - 1) * a.do_sh;
    const int64_t s_wrap = -(int64_t)(rs - 1) * a.st_sh;
    const int64_t ds_step = ds_hb * kDsBlockElems;
    int ds_qt = -1;  // query tile of the dS block index ds_bi (of this wave's key block)
    int64_t ds_bi = -1;
    auto stats = [&](int64_t sofs, int i0s, int buf) {
      if (wave == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          dma_stats(stat[buf] + 64 * rb, a.lse + sofs, a.delta + sofs, i0s + 32 * rb, len - 1, lane);
      }
    };
    dma_rows<D, MQ, 4>(Qs[0], tile_src_rows<MQ>(qrow, a.q_ss, len - i00), wave, lane);
    dma_rows<D, MQ, 4>(dOs[0], tile_src_rows<MQ>(drow, a.do_ss, len - i00), wave, lane);
    stats(so, i00, 0);
    // dS for the dQ product, this lane's key.  At head_dim 512 the dS of step k is stored at the
    // top of step k+1, after its wait, so that the wait there is for the tile copies alone and
    // the store has a whole step to complete.  ds_pend holds query rows 8 xh + 4 g2 + (0..3)
    // and 8 xh + 8 + 4 g2 + (0..3) of the block; lanes l and l + 32 trade four of them so that
    // each holds 8 consecutive rows (8 xh + 8 g2 ..) and writes them with one 16-byte store.
    static_assert(RB == 1, "one 32-row block per step");
    bf16x8 ds_pend = zero_bf16x8();
    int pend_i0 = 0;
    bf16* pend_dsh = dshead;
    auto store_pending = [&]() {
      const int xh = score_wave ? 0 : 2;
      if (pend_i0 / kDsRows != ds_qt) {
        ds_qt = pend_i0 / kDsRows;
        ds_bi = ds_block_index(ds_qt, (j0 / kDsKeys) + kb, a.causal, a.window, dlt, lenk, a.ds_tri, a.ds_cnt);
      }
      const int64_t bi = ds_bi;
      if (bi < 0) return;
      uint32_t w[4];
      __builtin_memcpy(w, &ds_pend, 16);
      const uint32_t give0 = g2 ? w[0] : w[2], give1 = g2 ? w[1] : w[3];
      const auto r0 = __builtin_amdgcn_permlane32_swap(give0, give0, false, false);
      const auto r1 = __builtin_amdgcn_permlane32_swap(give1, give1, false, false);
      // r[0] carries the lower half's value to every lane, r[1] the upper half's
      const uint32_t got0 = g2 ? r0[0] : r0[1], got1 = g2 ? r1[0] : r1[1];
      const uint32_t o[4] = {g2 ? got0 : w[0], g2 ? got1 : w[1], g2 ? w[2] : got0, g2 ? w[3] : got1};
      bf16* dst = pend_dsh + bi * kDsBlockElems + ds_elem(pend_i0 & (kDsRows - 1), ln) + 8 * xh + 8 * g2;
      uint4 v;
      __builtin_memcpy(&v, o, 16);
      *reinterpret_cast<uint4*>(dst) = v;
    };
    for (int k = 0; k < nsteps; ++k) {
      const int buf = k & 1;
      const int i0 = tcur * MQ;
      const bool wrap = hi + 1 == rs;                    // step k+1
      const int hn = wrap ? 0 : hi + 1;
      const int tn = wrap ? (tcur == tq0 ? tq_last : tcur - 1) : tcur;
      const int i0n = tn * MQ;
      const int64_t rmove = (int64_t)(i0n - i0);         // rows moved at a wrap
      const bool has_next = k + 1 < nsteps;
      const bf16* qrn = qrow + (wrap ? q_back + rmove * a.q_ss : a.q_sh);
      const bf16* drn = drow + (wrap ? d_back + rmove * a.do_ss : a.do_sh);
      const int64_t son = so + (wrap ? s_wrap : a.st_sh);
      // the last step copies nothing real: an empty range reads zeros into the idle buffers
      const TileSrc qn = tile_src_rows<MQ>(qrn, a.q_ss, has_next ? len - i0n : 0);
      const TileSrc dn = tile_src_rows<MQ>(drn, a.do_ss, has_next ? len - i0n : 0);
      wait_vmcnt<0>();
      barrier_lds();  // step k is in LDS; every wave is done with step k-1
      if constexpr (!LOWREG) {
        if (k > 0) store_pending();
      }

      f32x16 sacc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.f;
      // At head_dim 256 the lane index is re-read each step (an opaque copy), so that the LDS
      // fragment bases and the copies' lane offsets are recomputed in the loop instead of being
      // kept live across it.
      int dlane = lane;
      if constexpr (LOWREG) asm volatile("v_mov_b32 %0, %1" : "=v"(dlane) : "v"(lane));
      const RowFrags<D> rowf(dlane);
      const TrFrags<D> trf(dlane);
      // the transposing-read bases of this wave's d blocks dsl .. dsl + DBW - 1
      int tlo[DBW], thi[DBW];
#pragma unroll
      for (int d = 0; d < DBW; ++d) trf.pick(dsl + d, tlo[d], thi[d]);
      {
        const bf16* src = score_wave ? Qs[buf] : dOs[buf];
        // fragments read PF steps ahead: three at head_dim 512; two at 256, whose two workgroups
        // per compute unit hide part of each other's LDS latency within half the registers (one
        // ahead measured 3.5% slower there, three spilled)
        constexpr int PF = LOWREG ? 2 : 3;
        bf16x8 f[RB][PF + 1];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int t = 0; t < PF; ++t) f[rb][t] = rowf.read(src, 32 * rb, t);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            if (t + PF < KS) f[rb][(t + PF) % (PF + 1)] = rowf.read(src, 32 * rb, t + PF);
            sacc[rb] = E16<F16>::mma32(f[rb][t % (PF + 1)], kv[t], sacc[rb]);
            // copy slots: one every two matrix instructions, or (DMA_EARLY) all at the first ones
            const int slot = t * RB + rb;
            if (t == 1 && rb == 0 && has_next) stats(son, i0n, buf ^ 1);
            if (DMA_EARLY ? slot < 2 * NDMA : ((slot & 1) == 0 && slot / 2 < 2 * NDMA)) {
              const int j = DMA_EARLY ? slot : slot / 2;
              if (j < NDMA)
                dma_rows_one<D, MQ, 4>(Qs[buf ^ 1], qn, wave, dlane, j);
              else
                dma_rows_one<D, MQ, 4>(dOs[buf ^ 1], dn, wave, dlane, j - NDMA);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // sacc[rb]: lane = key j0 + 32 kb + ln, register r = query row i0 + 32 rb + 8 (r/4) + 4 g2 + r%4
      // P and dS are formed by all four waves: the score wave of key block kb takes
      // registers 0..7 (query rows 4 g2 + 0..3 and 8 + 4 g2 + 0..3) and receives their dP, the
      // dP wave takes registers 8..15 and receives their S.
      const int xh = score_wave ? 0 : 2;  // this wave's registers: 4 xh .. 4 xh + 7
      // register 4 x + e holds query row i0 + 8 x + 4 g2 + e; the statistics are read before the
      // exchange so that their latency overlaps it
      f32x4 lse4[RB][2], dl4[RB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const f32x4* st4 = reinterpret_cast<const f32x4*>(stat[buf] + 64 * rb);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          lse4[rb][u] = st4[2 * (xh + u) + g2] * kLog2e;
          dl4[rb][u] = st4[8 + 2 * (xh + u) + g2];
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (score_wave) {
#pragma unroll
          for (int x = 2; x < 4; ++x)
            xch[rb][kb][1][x - 2][lane] =
                f32x4{sacc[rb][4 * x], sacc[rb][4 * x + 1], sacc[rb][4 * x + 2], sacc[rb][4 * x + 3]};
        } else {
#pragma unroll
          for (int x = 0; x < 2; ++x)
            xch[rb][kb][0][x][lane] =
                f32x4{sacc[rb][4 * x], sacc[rb][4 * x + 1], sacc[rb][4 * x + 2], sacc[rb][4 * x + 3]};
        }
      }
      barrier_lds();
      bf16x8 ds_out[RB];  // this lane's dS values of the step, stored during the gradient products
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 sv[2], dpv[2];
        if (score_wave) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            sv[u] = f32x4{sacc[rb][4 * u], sacc[rb][4 * u + 1], sacc[rb][4 * u + 2], sacc[rb][4 * u + 3]};
            dpv[u] = xch[rb][kb][0][u][lane];
          }
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            sv[u] = xch[rb][kb][1][u][lane];
            dpv[u] = f32x4{sacc[rb][8 + 4 * u], sacc[rb][9 + 4 * u], sacc[rb][10 + 4 * u], sacc[rb][11 + 4 * u]};
          }
        }
        const int ir = i0 + 32 * rb;  // first query row of this block
        const bool full = (ir + 32 <= len) && (j0 + NK <= lenk) && (!a.causal || j0 + NK - 1 <= ir + dlt) &&
                          (a.window <= 0 || j0 > ir + 31 + dlt - a.window);
        bf16x8 pb, db;
        // under a softcap the score is capped before the exponential and dS takes the cap's
        // derivative 1 - tanh^2 (the stored dS is then the gradient of the uncapped score)
        auto capped = [&](float x, float& der) {
          if constexpr (SOFTCAP) {
            const float t = tanh_from_exp(x * a.sc_in);
            der = 1.0f - t * t;
            return a.sc_out * t;
          } else {
            der = 1.0f;
            return x;
          }
        };
        if (full) {
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            float der;
            const float sx = capped(sv[r >> 2][r & 3], der);
            const float p = fast_exp2(fmaf(sx, c, -lse4[rb][r >> 2][r & 3]));
            pb[r] = E16<F16>::from_float(p);
            db[r] = E16<F16>::from_float(p * (dpv[r >> 2][r & 3] - dl4[rb][r >> 2][r & 3]) * der);
          }
        } else {
          // this lane's key is visible from query rows rlo .. rhi-1
          const int key = j0 + 32 * kb + ln;
          const int rlo = a.causal ? key - dlt : 0;
          int rhi = key < lenk ? len : 0;
          if (a.window > 0) rhi = min(rhi, key + a.window - dlt);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int row = ir + 8 * (xh + (r >> 2)) + 4 * g2 + (r & 3);
            const bool vis = (row >= rlo) & (row < rhi);
            float der;
            const float sx = capped(sv[r >> 2][r & 3], der);
            const float e = fast_exp2(fmaf(sx, c, -lse4[rb][r >> 2][r & 3]));
            const float p = vis ? e : 0.f;
            const float ds = vis ? p * (dpv[r >> 2][r & 3] - dl4[rb][r >> 2][r & 3]) * der : 0.f;  // +0 when masked
            pb[r] = E16<F16>::from_float(p);
            db[r] = E16<F16>::from_float(ds);
          }
        }
        // 16-row half 2 rb + (xh / 2) of P and dS, over the exchange half this wave has read
        bf16x8* mine = reinterpret_cast<bf16x8*>(&xch[rb][kb][xh >> 1][0][0]);
        mine[lane] = pb;
        mine[64 + lane] = db;
        ds_out[rb] = db;
      }
      // the dS of the step: stored now at head_dim 256 (there are no registers to carry it across
      // the barrier), at the top of the next step at 512
      ds_pend = ds_out[0];
      pend_i0 = i0;
      pend_dsh = dshead;
      if constexpr (LOWREG) store_pending();
      barrier_lds();
      if constexpr (LOWREG) {
        // one 16-row half at a time: its P and dS fragments, then per d block the four products;
        // the transposed dO and Q fragments are read one (half, d block) step ahead
        bf16x8 ado = trf.read_with(dOs[buf], 0, dsl, tlo[0], thi[0]), aq = trf.read_with(Qs[buf], 0, dsl, tlo[0], thi[0]);
#pragma unroll
        for (int s = 0; s < 2 * RB; ++s) {
          bf16x8 pfr[4];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const bf16x8* src = reinterpret_cast<const bf16x8*>(&xch[s >> 1][x][s & 1][0][0]);
            pfr[x] = src[lane];           // P, key block x
            pfr[2 + x] = src[64 + lane];  // dS, key block x
          }
#pragma unroll
          for (int d = 0; d < DBW; ++d) {
            const int ns = d + 1 == DBW ? s + 1 : s, nd = d + 1 == DBW ? 0 : d + 1;
            bf16x8 ado_n = ado, aq_n = aq;
            if (ns < 2 * RB) {
              ado_n = trf.read_with(dOs[buf], 16 * ns, dsl + nd, tlo[nd], thi[nd]);
              aq_n = trf.read_with(Qs[buf], 16 * ns, dsl + nd, tlo[nd], thi[nd]);
            }
            dvacc[0][d] = E16<F16>::mma32(ado, pfr[0], dvacc[0][d]);
            dvacc[1][d] = E16<F16>::mma32(ado, pfr[1], dvacc[1][d]);
            dkacc[0][d] = E16<F16>::mma32(aq, pfr[2], dkacc[0][d]);
            dkacc[1][d] = E16<F16>::mma32(aq, pfr[3], dkacc[1][d]);
            ado = ado_n;
            aq = aq_n;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
        // the transposed fragments of (s, d) are read one (s, d) step ahead of their products
        bf16x8 ado = trf.read_with(dOs[buf], 0, dsl, tlo[0], thi[0]), aq = trf.read_with(Qs[buf], 0, dsl, tlo[0], thi[0]);
        // every 16-row half's P and dS fragments are read before the first products
        bf16x8 pfr[2 * RB][4];
#pragma unroll
        for (int s = 0; s < 2 * RB; ++s) {
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const bf16x8* src = reinterpret_cast<const bf16x8*>(&xch[s >> 1][x][s & 1][0][0]);
            pfr[s][x] = src[lane];           // P, key block x
            pfr[s][2 + x] = src[64 + lane];  // dS, key block x
          }
        }
#pragma unroll
        for (int s = 0; s < 2 * RB; ++s) {
          const bf16x8 p0 = pfr[s][0], p1 = pfr[s][1];
          const bf16x8 s0 = pfr[s][2], s1 = pfr[s][3];
#pragma unroll
          for (int d = 0; d < DBW; ++d) {
            const int ns = d + 1 == DBW ? s + 1 : s, nd = d + 1 == DBW ? 0 : d + 1;
            bf16x8 ado_n = ado, aq_n = aq;
            if (ns < 2 * RB) {
              ado_n = trf.read_with(dOs[buf], 16 * ns, dsl + nd, tlo[nd], thi[nd]);
              aq_n = trf.read_with(Qs[buf], 16 * ns, dsl + nd, tlo[nd], thi[nd]);
            }
            dvacc[0][d] = E16<F16>::mma32(ado, p0, dvacc[0][d]);
            dvacc[1][d] = E16<F16>::mma32(ado, p1, dvacc[1][d]);
            dkacc[0][d] = E16<F16>::mma32(aq, s0, dkacc[0][d]);
            dkacc[1][d] = E16<F16>::mma32(aq, s1, dkacc[1][d]);
            ado = ado_n;
            aq = aq_n;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      tcur = tn;
      hi = hn;
      qrow = qrn;
      drow = drn;
      so = son;
      dshead += wrap ? -(rs - 1) * ds_step : ds_step;
    }
    if constexpr (!LOWREG) store_pending();
    wait_vmcnt<0>();  // no copy into LDS may be in flight when the workgroup ends
  }

  // dV^T / dK^T blocks: lane = key j0 + 32 x + ln, register r = d 32 (dsl + d) + 8 (r/4) + 4 g2 + r%4
  if (a.kv_split > 1) {
    // partial sums over this workgroup's heads, every key of the tile (zeros where no row
    // of these heads sees it), reduced by bwd_kv_reduce in part order
    const int64_t plane = (int64_t)a.B * a.Sk * a.Hkv * D;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int key = j0 + 32 * x + ln;
      if (key >= a.Sk) continue;
      const int64_t row = (((int64_t)b * a.Sk + key) * a.Hkv + g) * D + 4 * g2;
      float* pk = a.kv_part + (2 * part) * plane + row;
      float* pv = a.kv_part + (2 * part + 1) * plane + row;
      const float sc = a.scale;
#pragma unroll
      for (int d = 0; d < DBW; ++d)
#pragma unroll
        for (int qa = 0; qa < 4; ++qa) {
          const int col = 32 * (dsl + d) + 8 * qa;
          stg4(pk + col, dkacc[x][d][4 * qa] * sc, dkacc[x][d][4 * qa + 1] * sc, dkacc[x][d][4 * qa + 2] * sc,
               dkacc[x][d][4 * qa + 3] * sc);
          stg4(pv + col, dvacc[x][d][4 * qa], dvacc[x][d][4 * qa + 1], dvacc[x][d][4 * qa + 2],
               dvacc[x][d][4 * qa + 3]);
        }
    }
    return;
  }
  if (a.dk_f32 != nullptr) {
    // accumulate a chunk pair's parts; a tile that no query row of the pair sees adds nothing
    if (nsteps == 0) return;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int key = j0 + 32 * x + ln;
      if (key >= a.Sk) continue;
      float* pk = a.dk_f32 + b * a.dk_sb + (int64_t)key * a.dk_ss + g * a.dk_sh + 4 * g2;
      float* pv = a.dv_f32 + b * a.dv_sb + (int64_t)key * a.dv_ss + g * a.dv_sh + 4 * g2;
      const float sc = a.scale;
#pragma unroll
      for (int d = 0; d < DBW; ++d)
#pragma unroll
        for (int qa = 0; qa < 4; ++qa) {
          const int col = 32 * (dsl + d) + 8 * qa;
          add4(pk + col, dkacc[x][d][4 * qa] * sc, dkacc[x][d][4 * qa + 1] * sc, dkacc[x][d][4 * qa + 2] * sc,
               dkacc[x][d][4 * qa + 3] * sc);
          add4(pv + col, dvacc[x][d][4 * qa], dvacc[x][d][4 * qa + 1], dvacc[x][d][4 * qa + 2],
               dvacc[x][d][4 * qa + 3]);
        }
    }
    return;
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int key = j0 + 32 * x + ln;
    const bool wr = a.packed ? key < len : key < a.Sk;
    if (!wr) continue;
    bf16* pk = a.dk + b * a.dk_sb + (int64_t)(off + key) * a.dk_ss + g * a.dk_sh + 4 * g2;
    bf16* pv = a.dv + b * a.dv_sb + (int64_t)(off + key) * a.dv_ss + g * a.dv_sh + 4 * g2;
    const float sc = a.scale;
#pragma unroll
    for (int d = 0; d < DBW; ++d)
#pragma unroll
      for (int qa = 0; qa < 4; ++qa) {
        const int col = 32 * (dsl + d) + 8 * qa;
        stg4e<F16>(pk + col, dkacc[x][d][4 * qa] * sc, dkacc[x][d][4 * qa + 1] * sc, dkacc[x][d][4 * qa + 2] * sc,
                   dkacc[x][d][4 * qa + 3] * sc);
        stg4e<F16>(pv + col, dvacc[x][d][4 * qa], dvacc[x][d][4 * qa + 1], dvacc[x][d][4 * qa + 2],
                   dvacc[x][d][4 * qa + 3]);
      }
  }
}

// dK, dV of workgroups that split a group's query heads: the sum of the parts in part order
// (deterministic), written in bf16 or added to the fp32 accumulators.  Elementwise: 8
// consecutive head_dim elements per thread.
template <int D, bool F16>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(AttnArgs a) {
  constexpr int TPR = D / 8;
  const int64_t rows = (int64_t)a.B * a.Sk * a.Hkv;
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gi / TPR;
  if (row >= rows) return;
  const int c0 = 8 * (int)(gi - row * TPR);
  const int g = (int)(row % a.Hkv);
  const int64_t bk = row / a.Hkv;
  const int key = (int)(bk % a.Sk);
  const int b = (int)(bk / a.Sk);
  const int64_t plane = rows * D;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    for (int p = 0; p < a.kv_split; ++p) {
      const float* src = a.kv_part + (2 * p + which) * plane + row * D + c0;
      const float4 x0 = *reinterpret_cast<const float4*>(src);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
      v[0] += x0.x; v[1] += x0.y; v[2] += x0.z; v[3] += x0.w;
      v[4] += x1.x; v[5] += x1.y; v[6] += x1.z; v[7] += x1.w;
    }
    if (a.dk_f32 != nullptr) {
      float* acc = (which ? a.dv_f32 + b * a.dv_sb + (int64_t)key * a.dv_ss + g * a.dv_sh
                          : a.dk_f32 + b * a.dk_sb + (int64_t)key * a.dk_ss + g * a.dk_sh) + c0;
      add4(acc, v[0], v[1], v[2], v[3]);
      add4(acc + 4, v[4], v[5], v[6], v[7]);
    } else {
      bf16* out = (which ? a.dv + b * a.dv_sb + (int64_t)key * a.dv_ss + g * a.dv_sh
                         : a.dk + b * a.dk_sb + (int64_t)key * a.dk_ss + g * a.dk_sh) + c0;
      stg4e<F16>(out, v[0], v[1], v[2], v[3]);
      stg4e<F16>(out + 4, v[4], v[5], v[6], v[7]);
    }
  }
}

template <bool F16>
hipError_t launch_bwd_kv_reduce_t(const AttnArgs& a, int D, hipStream_t stream) {
  const int64_t threads = (int64_t)a.B * a.Sk * a.Hkv * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (D == 512)
    hipLaunchKernelGGL((bwd_kv_reduce_kernel<512, F16>), grid, block, 0, stream, a);
  else if (D == 256)
    hipLaunchKernelGGL((bwd_kv_reduce_kernel<256, F16>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_kv_reduce(const AttnArgs& a, int D, hipStream_t stream) {
  return a.f16 ? launch_bwd_kv_reduce_t<true>(a, D, stream) : launch_bwd_kv_reduce_t<false>(a, D, stream);
}

template <bool F16>
hipError_t launch_bwd_dkdv_t(const AttnArgs& a, int D, hipStream_t stream) {
  const dim3 grid(8 * a.per_xcd), block(256);
  const bool sc = a.softcap > 0.f;
  if (D == 512 && !sc)
    hipLaunchKernelGGL((bwd_dkdv_kernel<512, false, F16>), grid, block, 0, stream, a);
  else if (D == 512)
    hipLaunchKernelGGL((bwd_dkdv_kernel<512, true, F16>), grid, block, 0, stream, a);
  else if (D == 256 && !sc)
    hipLaunchKernelGGL((bwd_dkdv_kernel<256, false, F16>), grid, block, 0, stream, a);
  else if (D == 256)
    hipLaunchKernelGGL((bwd_dkdv_kernel<256, true, F16>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const AttnArgs& a, int D, hipStream_t stream) {
  return a.f16 ? launch_bwd_dkdv_t<true>(a, D, stream) : launch_bwd_dkdv_t<false>(a, D, stream);
}

// Copy of one stored dS block into a swizzled LDS tile of kDsKeys rows (keys) x kDsRows
// columns (query rows), as dma_rows does for a row-major tile: LDS chunk p of key row r
// receives the block's chunk p ^ h(r) of that key, found at its place in the quartered
// layout (ds_elem).
template <int NW>
__device__ __forceinline__ void dma_ds_block(bf16* tile, const TileSrc& src, int wave, int lane) {
  constexpr int CH = kDsRows / 8;   // 16-byte chunks per key row
  constexpr int RPI = 64 / CH;      // key rows per wave-instruction
  constexpr int NI = kDsKeys / RPI;
  static_assert(NI % NW == 0, "the block must split evenly over the waves");
#pragma unroll
  for (int k = 0; k < NI / NW; ++k) {
    const int i = wave + k * NW;
    const int key = i * RPI + lane / CH;
    const int c = (lane % CH) ^ swz_h(key);
    const uint32_t voff = (uint32_t)(2 * ds_elem(8 * c, key));
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + i * RPI * kDsRows));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff),
                 "s"(src.rsrc)
                 : "memory");
  }
}

// ---------------------------------------------------------------------------
// dQ = scale dS K, from the stored dS blocks
// ---------------------------------------------------------------------------
// One workgroup per (batch, query head, 128-row query tile, head_dim slice of D columns):
// at head_dim 512 the columns are split in NSPLIT = 2 halves, so that a wave needs only
// 128 accumulator registers and two workgroups share a compute unit; one's copies and
// barriers then overlap the other's matrix work (the same dS block is read by both halves,
// from L2).  Each step brings one 32-key block of K (the workgroup's columns) and the
// matching dS^T block into LDS; wave w owns columns 32 DBW w .. of the slice for all 128
// rows, so every K fragment it reads serves four products and every dS fragment DBW.
// dQ^T accumulates in registers: A operand K^T and B operand dS^T, both read with
// transposing LDS reads.  Pairs that are not visible are zeroed by selection (blocks on the
// diagonal or the window edge may hold stale values there).
template <int D, int NW, int NSPLIT, bool F16>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bwd_dq_kernel(AttnArgs a) {
  // D: head_dim columns of this workgroup (the full head_dim is D * NSPLIT)
  constexpr int M = kDsRows;          // 128 query rows
  constexpr int NK = kDsKeys;         // 32 keys per step
  constexpr int DBW = D / (32 * NW);  // 32-wide d blocks per wave
  constexpr int RB = M / 32;          // 32-row blocks
  static_assert(DBW >= 1 && DBW * 32 * NW == D, "head_dim must split evenly over the waves");
  // A step's two blocks are copied NBUF - 1 steps ahead: its own matrix work is short against
  // the memory latency of a dS block (written by the dK/dV pass, read once here).
  constexpr int NBUF = 3;
  constexpr int NCOPY = NK * D / 512 / NW + (NK / (64 / (M / 8))) / NW;  // copies per wave and block
  __shared__ __attribute__((aligned(1024))) bf16 Ks[NBUF][NK * D];
  __shared__ __attribute__((aligned(1024))) bf16 Ss[NBUF][NK * M];

  const int item = xcd_item(a.per_xcd, a.total_items, a.nqt * a.r * NSPLIT, a.balanced, a.order, a.Hkv);
  if (item < 0) return;
  // items: (batch, kv head) units, query tiles from the last one down, then the group's
  // heads and the column slices, so that the workgroups sharing an XCD read the same K
  // and dS blocks
  const int per_unit = a.nqt * a.r * NSPLIT;
  const int unit = item / per_unit;
  const int rem0 = item - unit * per_unit;
  const int dh = rem0 % NSPLIT;
  const int rem = rem0 / NSPLIT;
  const int qt = a.nqt - 1 - rem / a.r;
  const int g = unit % a.Hkv;
  const int b = unit / a.Hkv;
  const int h = g * a.r + rem % a.r;
  int len = a.seq_len ? a.seq_len[b] : a.S;
  len = min(max(len, 0), a.S);
  const int64_t ds_b = a.ds_seq ? a.ds_seq[b] : 0;
  if (ds_b < 0) len = 0;  // a sequence that did not fit the workspace (see bwd_dkdv)
  const int lenk = a.seq_len ? len : a.Sk;  // key rows
  const int dlt = a.q_shift;
  const int off = a.seq_off ? a.seq_off[b] : 0;
  const int p0 = qt * M;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g2 = lane >> 5, ln = lane & 31;
  const int dsl = wave * DBW;

  f32x16 acc[RB][DBW];
#pragma unroll
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int d = 0; d < DBW; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][d][r] = 0.f;

  // visible key blocks of the tile's rows
  const int plast = min(p0 + M, len) - 1;
  const int kb_first =
      max(ds_kb_lo(qt, a.causal, a.window, dlt), a.window > 0 ? max(0, p0 + dlt - a.window + 1) / NK : 0);
  const int jmax = a.causal ? min(plast + dlt, lenk - 1) : lenk - 1;  // the tile's largest visible key
  const int kb_last = (plast < p0 || jmax < 0) ? -1 : jmax / NK;

  if (kb_first <= kb_last) {
    const bf16* kbase = a.k + b * a.k_sb + (int64_t)off * a.k_ss + g * a.k_sh + dh * D;
    const int64_t ds_hb = a.ds_seq ? ds_head_blocks(len, a.ds_tri, a.ds_cnt) : a.ds_head;
    const bf16* sbase = a.dsb + ((a.ds_seq ? ds_b : (int64_t)b * a.Hq * ds_hb) + (int64_t)h * ds_hb) * kDsBlockElems;
    // Every block in kb_first .. kb_last holds a visible pair, so it is stored, and the stored
    // blocks of a query tile are consecutive: block kb sits (kb - kb_first) blocks after the
    // first.  The copies walk K and dS with two pointers, one block per copy.
    const int64_t bi0 = ds_block_index(qt, kb_first, a.causal, a.window, dlt, lenk, a.ds_tri, a.ds_cnt);
    const bf16* scopy = sbase + (bi0 < 0 ? 0 : bi0) * kDsBlockElems;
    const bf16* kcopy = kbase + (int64_t)kb_first * NK * a.k_ss;
    int kbcopy = kb_first;  // block of the next copy
    const TrFrags<D> trk(lane);
    const TrFrags<M> trs(lane);
    int klo[DBW], khi[DBW];  // bases of this wave's d blocks
#pragma unroll
    for (int d = 0; d < DBW; ++d) trk.pick(dsl + d, klo[d], khi[d]);

    auto copy_block = [&](int buf) {
      dma_rows<D, NK, NW>(Ks[buf], tile_src<NK>(kcopy, a.k_ss, 0, lenk - kbcopy * NK), wave, lane);
      dma_ds_block<NW>(Ss[buf], tile_src<NK>(scopy, M, 0, NK), wave, lane);
      kcopy += (int64_t)NK * a.k_ss;
      scopy += kDsBlockElems;
      ++kbcopy;
    };
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
      if (kb_first + i <= kb_last) copy_block(i);
    int buf = 0;
    for (int kb = kb_first; kb <= kb_last; ++kb) {
      const int j0 = kb * NK;
      // block kb has landed; the later blocks already issued may still be in flight
      static_assert(NBUF == 3, "the waits below assume one block in flight beyond the current one");
      if (kb + 1 <= kb_last)
        wait_vmcnt<NCOPY>();
      else
        wait_vmcnt<0>();
      barrier_lds();  // block kb is in LDS; every wave is done with block kb-1 (buffer of kb + 2)
      if (kb + NBUF - 1 <= kb_last) copy_block(buf == 0 ? NBUF - 1 : buf - 1);  // block kb + NBUF - 1
      const bool full = (p0 + M <= len) && (j0 + NK <= lenk) && (!a.causal || j0 + NK - 1 <= p0 + dlt) &&
                        (a.window <= 0 || j0 > p0 + M - 1 + dlt - a.window);
      // dS fragments of key step s are read one step ahead and masked when used; the K
      // fragment of (s, d) is read one (s, d) step ahead of its products.  On a block that
      // straddles an edge, a row's visible keys are one interval [lo, hi], held as a 32-bit mask
      // over the block's keys (bit t: key j0 + t), from which each fragment takes its 8 bits.
      uint32_t vis[RB];
      if (!full) {
#pragma unroll
        for (int x = 0; x < RB; ++x) {
          const int row = p0 + 32 * x + ln;
          const int ip = row + dlt;
          const int hi = a.causal ? min(lenk - 1, ip) : lenk - 1;
          const int lo = a.window > 0 ? ip - a.window + 1 : 0;
          const int nh = min(max(hi - j0 + 1, 0), 32), nl = min(max(lo - j0, 0), 32);
          const uint32_t mh = (uint32_t)((1ull << nh) - 1), ml = (uint32_t)((1ull << nl) - 1);
          vis[x] = row < len ? (mh & ~ml) : 0u;
        }
      }
      auto mask = [&](bf16x8& v, int s, int x) {
        // element e holds key j0 + 16 s + 4 g2 + e (e < 4) or j0 + 16 s + 8 + 4 g2 + e - 4;
        // 16-bit halves of dword i hold elements 2 i and 2 i + 1
        const uint32_t ba = vis[x] >> (16 * s + 4 * g2), bb = ba >> 8;
        auto halves = [](uint32_t t) { return ((t & 1u) * 0xffffu) | ((t & 2u) * 0x7fff8000u); };
        uint32_t w[4];
        __builtin_memcpy(w, &v, 16);
        w[0] &= halves(ba);
        w[1] &= halves(ba >> 2);
        w[2] &= halves(bb);
        w[3] &= halves(bb >> 2);
        __builtin_memcpy(&v, w, 16);
      };
      bf16x8 bs[RB], bsn[RB];
#pragma unroll
      for (int x = 0; x < RB; ++x) bs[x] = trs.read(Ss[buf], 0, x);
      bf16x8 ak = trk.read_with(Ks[buf], 0, dsl, klo[0], khi[0]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (!full) {
#pragma unroll
          for (int x = 0; x < RB; ++x) mask(bs[x], s, x);
        }
#pragma unroll
        for (int d = 0; d < DBW; ++d) {
          const bool last_d = d + 1 == DBW;
          if (last_d && s == 0) {
#pragma unroll
            for (int x = 0; x < RB; ++x) bsn[x] = trs.read(Ss[buf], 16, x);
          }
          bf16x8 akn = ak;
          if (!(last_d && s == 1)) {
            const int ns = last_d ? s + 1 : s, nd = last_d ? 0 : d + 1;
            akn = trk.read_with(Ks[buf], 16 * ns, dsl + nd, klo[nd], khi[nd]);
          }
#pragma unroll
          for (int x = 0; x < RB; ++x) acc[x][d] = E16<F16>::mma32(ak, bs[x], acc[x][d]);
          ak = akn;
          __builtin_amdgcn_sched_barrier(0);
        }
        if (s == 0) {
#pragma unroll
          for (int x = 0; x < RB; ++x) bs[x] = bsn[x];
        }
      }
      buf = buf + 1 == NBUF ? 0 : buf + 1;
    }
  }

  // dQ^T blocks: lane = row p0 + 32 x + ln, register r = d 32 (dsl + d) + 8 (r/4) + 4 g2 + r%4
  if (a.dq_f32 != nullptr) {
    // accumulate a chunk pair's part; rows that see no key of the pair add nothing
    if (kb_first > kb_last) return;
#pragma unroll
    for (int x = 0; x < RB; ++x) {
      const int px = p0 + 32 * x + ln;
      if (px >= a.S) continue;
      float* pq = a.dq_f32 + b * a.dq_sb + (int64_t)px * a.dq_ss + h * a.dq_sh + dh * D + 4 * g2;
      const float sc = a.scale;
#pragma unroll
      for (int d = 0; d < DBW; ++d)
#pragma unroll
        for (int qa = 0; qa < 4; ++qa)
          add4(pq + 32 * (dsl + d) + 8 * qa, acc[x][d][4 * qa] * sc, acc[x][d][4 * qa + 1] * sc,
               acc[x][d][4 * qa + 2] * sc, acc[x][d][4 * qa + 3] * sc);
    }
    return;
  }
#pragma unroll
  for (int x = 0; x < RB; ++x) {
    const int px = p0 + 32 * x + ln;
    const bool wr = a.packed ? px < len : px < a.S;
    if (!wr) continue;
    bf16* pq = a.out + b * a.dq_sb + (int64_t)(off + px) * a.dq_ss + h * a.dq_sh + dh * D + 4 * g2;
    const float sc = a.scale;
#pragma unroll
    for (int d = 0; d < DBW; ++d)
#pragma unroll
      for (int qa = 0; qa < 4; ++qa)
        stg4e<F16>(pq + 32 * (dsl + d) + 8 * qa, acc[x][d][4 * qa] * sc, acc[x][d][4 * qa + 1] * sc,
             acc[x][d][4 * qa + 2] * sc, acc[x][d][4 * qa + 3] * sc);
  }
}

template <bool F16>
hipError_t launch_bwd_dq_t(const AttnArgs& a, int D, hipStream_t stream) {
  const dim3 grid(8 * a.per_xcd);
  if (D == 512)
    hipLaunchKernelGGL((bwd_dq_kernel<512 / kDqSplit512, 4, kDqSplit512, F16>), grid, dim3(256), 0, stream, a);
  else if (D == 256)
    hipLaunchKernelGGL((bwd_dq_kernel<256, 4, 1, F16>), grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const AttnArgs& a, int D, hipStream_t stream) {
  return a.f16 ? launch_bwd_dq_t<true>(a, D, stream) : launch_bwd_dq_t<false>(a, D, stream);
}

}  // namespace attn
