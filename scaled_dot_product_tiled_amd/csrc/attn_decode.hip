// Paged-KV single-token decode: one query token per sequence against a KV cache stored
// in fixed-size pages, located through a per-sequence page table (the paged cache and
// page table of the page "flex_attention + paged KV + CUDA graphs vs vLLM", Architecture
// notes).  Pages sit anywhere in the pool, so every page costs one table lookup (that
// page's section "What each option did" measures what skipping the lookup saves when
// pages happen to be contiguous; here they are not).
//
// The work is bound by reading K and V once from HBM.  The arithmetic per byte is small,
// but on the vector ALUs alone it would not keep up with the memory (two multiply-adds
// per K and V element and query head, plus the reductions), so the two contractions run
// on the matrix cores, which leaves the vector units only the softmax:
//   split  one workgroup per (kv head, 512-token chunk, sequence), four independent waves;
//          a wave takes steps of two 16-token pages.  The step's K and V rows go straight
//          from memory to the wave's own LDS area (16 lanes move one 256-byte row, so
//          every copy reads whole rows), then
//            S^T (16 tokens x 16 heads) = K_page (16 x 128) . Q^T        (per page)
//          with the query heads of the kv head as the columns of Q^T (columns past
//          Hq/Hkv are zero), and
//            O^T (128 x 16 heads) += V^T (128 x 32 tokens) . P^T (32 tokens x 16 heads)
//          where P^T is the score accumulator itself (its layout is the operand layout)
//          and V^T is read with transposing LDS reads.  An online softmax per query head
//          gives a partial (max, sum, unnormalised output) per chunk and head; the four
//          waves' partials are combined in LDS.
//   merge  one workgroup per (sequence, query head) combines the chunk partials.
// Tokens at or past ctx_len are masked; their loads are redirected to a valid slot of
// the same step, so no unused slot or page is ever read.
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "kernel_args.h"

namespace attn {

// Chunk partials of paged_decode_noalloc: a fixed array in device memory instead of a
// caller-provided workspace, for callers that cannot allocate.  Every GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not the device address: the address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to the kernels.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

constexpr int kDecD = 128;

// Value of this lane's partner at lane ^ 16, combined.
__device__ __forceinline__ float row_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int R, bool F16, bool SOFTCAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_kernel(DecodeArgs a) {
  constexpr int D = kDecD;
  constexpr int CH = kDecodeChunk;      // tokens per workgroup
  constexpr int SPW = CH / 32 / 4;      // steps per wave
  static_assert(SPW >= 1 && CH % 128 == 0, "chunk must hold whole steps of every wave");
  constexpr int PAGE_B = 16 * D * 2;    // bytes of one staged K or V page (16 rows of 256 bytes)
  // per wave: V page 0, V page 1, K page 0, K page 1
  __shared__ __attribute__((aligned(16))) char stage[4][4 * PAGE_B];
  __shared__ float s_m[4][R], s_l[4][R];
  static_assert(4 * R * (D + 4) * 4 <= (int)sizeof(stage), "wave partials reuse the staging area");
  auto s_o = reinterpret_cast<float(*)[R][D + 4]>(&stage[0][0]);

  // kv head fastest: the workgroups of one page range start together
  const int g = blockIdx.x % a.Hkv;
  const int bc = blockIdx.x / a.Hkv;
  const int c = bc % a.max_chunks;
  const int b = bc / a.max_chunks;
  int ctx = a.ctx[b];
  ctx = min(max(ctx, 0), a.max_pages * 16);
  if (c * CH >= ctx) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, li = lane & 15;
  const float cs = a.c;

  // B operand Q^T: column li is query head g*R + li, k = 32 kk + 8 grp + e.
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qf[kk] = zero_bf16x8();
    if (li < R) qf[kk] = ldg8(a.q + b * a.q_sb + (g * R + li) * a.q_sh + 32 * kk + 8 * grp);
  }

  const int32_t* trow = a.table + (int64_t)b * a.max_pages;
  const uint32_t kss = (uint32_t)a.kc_ss * 2u, vss = (uint32_t)a.vc_ss * 2u;  // slot strides in bytes
  const int rem = ctx - c * CH - wave * 32;
  const int nst = rem <= 0 ? 0 : min(SPW, (rem + 127) / 128);  // steps of this wave

  // Physical pages of this wave's steps, fetched once: lane 2 s + pg holds page pg of step s.
  // A page past the context is replaced by the step's first page (its tokens are masked).
  // Contiguous pages need no table row: page lp is the sequence's first page + lp.
  int tbl = 0;
  if (lane < 2 * nst) {
    const int tok0 = c * CH + (4 * (lane >> 1) + wave) * 32;
    const int lp = (tok0 + 16 * (lane & 1) < ctx) ? (tok0 >> 4) + (lane & 1) : (tok0 >> 4);
    const int64_t id = a.contiguous ? (int64_t)a.table[b] + lp : (int64_t)trow[lp];
    tbl = (int)min<int64_t>(max<int64_t>(id, 0), a.num_pages - 1);
  }

  // Staged rows are 256 bytes.  K: chunk ch of row r sits at chunk position ch ^ r, so the
  // fragment reads (16 rows at one chunk per 16 lanes) hit 16 different positions.
  // V: chunk ch of row r sits at ch ^ 2 (r & 7), so the transposing reads (8 rows x 32
  // bytes per half-wave) hit all 64 banks once.  Copy j of a page moves rows 4 j .. 4 j + 3:
  // lane i fills row 4 j + i / 16 at position i % 16 and so fetches the chunk the swizzle
  // puts there.
  char* vb = stage[wave];
  char* kb = stage[wave] + 2 * PAGE_B;
  int nv[2];
  auto load = [&](int s) {
    const int tok0 = c * CH + (4 * s + wave) * 32;  // first token of the step (< ctx)
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      nv[pg] = min(max(ctx - tok0 - 16 * pg, 0), 16);
      const int last = nv[pg] > 0 ? nv[pg] - 1 : 0;
      const int phys = __builtin_amdgcn_readlane(tbl, 2 * s + pg);
      const char* kp = reinterpret_cast<const char*>(a.kc + (int64_t)phys * a.kc_sp + (int64_t)g * a.kc_sh);
      const char* vp = reinterpret_cast<const char*>(a.vc + (int64_t)phys * a.vc_sp + (int64_t)g * a.vc_sh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + grp;
        const uint32_t slot = (uint32_t)min(r, last);
        __builtin_amdgcn_global_load_lds(kp + (slot * kss + 16u * (li ^ r)),
                                         (lds_void_t*)(kb + pg * PAGE_B + 1024 * j), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp + (slot * vss + 16u * (li ^ (2 * (r & 7)))),
                                         (lds_void_t*)(vb + pg * PAGE_B + 1024 * j), 16, 0, 0);
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int rrd = 4 * grp + (li >> 2);  // V row of this lane's transposing read
  const int rd_base = rrd * 256 + 16 * ((li >> 1) & 1) + 8 * (li & 1);
  const int rd_x = rrd & 7;

  auto compute = [&]() {
    f32x4 st[2];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      st[pg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + pg * PAGE_B + li * 256 + 16 * ((4 * kk + grp) ^ li));
        st[pg] = E16<F16>::mma16(kf, qf[kk], st[pg]);
      }
    }
    // lane: head li, tokens 4 grp + i of each page
    float t[2][4];
    float lm = -INFINITY;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = st[pg][i];
        if constexpr (SOFTCAP) x = a.sc_out * tanh_from_exp(x * a.sc_in);  // cap before the mask
        t[pg][i] = (4 * grp + i < nv[pg]) ? x * cs : -INFINITY;
        lm = fmaxf(lm, t[pg][i]);
      }
    lm = row_swap_max(lm);
    lm = half_swap_max(lm);
    if (lm > m + kRescaleSlack) {  // same decision in the four lanes of a head
      const float alpha = fast_exp2(m - lm);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
      m = lm;
    }
    bf16x8 pb;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the normaliser sums the rounded probabilities that multiply V
        pb[4 * pg + i] = E16<F16>::from_float(fast_exp2(t[pg][i] - m));
        l += E16<F16>::to_float(pb[4 * pg + i]);
      }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int off = rd_base + 32 * (blk ^ rd_x);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vb + off));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vb + PAGE_B + off));
      acc[blk] = E16<F16>::mma16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, acc[blk]);
    }
  };

  // Each wave runs its steps one after the other; the copies of other waves (two workgroups
  // per compute unit) cover the memory latency of a step.  The compiler tracks the copies
  // (no inline assembly here): it waits for them before the first LDS read of a step, and
  // the copies of the next step are issued after this step's LDS reads have returned.
#pragma unroll 1
  for (int s = 0; s < nst; ++s) {
    load(s);
    __builtin_amdgcn_sched_barrier(0);  // every copy of the step is issued before its first wait
    compute();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this step's LDS reads are done
    __builtin_amdgcn_sched_barrier(0);
  }

  l = row_swap_sum(l);
  l = half_swap_sum(l);
  __syncthreads();  // every wave is done with its staging area
  if (li < R) {
    if (grp == 0) {
      s_m[wave][li] = m;
      s_l[wave][li] = l;
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
      *reinterpret_cast<f32x4*>(&s_o[wave][li][16 * blk + 4 * grp]) = acc[blk];
  }
  __syncthreads();
  // combine the four waves: thread t handles (head, d) pairs t, t + 256, ...
  for (int idx = threadIdx.x; idx < R * D; idx += 256) {
    const int hh = idx / D, d = idx - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][hh]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float o = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = fast_exp2(s_m[w][hh] - Mu);
      o = fmaf(wt, s_o[w][hh][d], o);
      den = fmaf(wt, s_l[w][hh], den);
    }
    float* part = a.part + ((int64_t)(b * a.Hq + g * R + hh) * a.max_chunks + c) * (D + 2);
    if (d == 0) {
      part[0] = Mu;
      part[1] = den;
    }
    part[2 + d] = o;
  }
}

// One pass over the chunk partials of a (sequence, query head): the loads of up to U
// chunks are issued together, and a running maximum rescales what was summed before.
template <bool F16>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a) {
  constexpr int D = kDecD;
  constexpr int U = 8;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  int ctx = a.ctx[b];
  ctx = min(max(ctx, 0), a.max_pages * a.page_size);
  const int nch = (ctx + kDecodeChunk - 1) / kDecodeChunk;
  const int d = threadIdx.x;
  const float* part = a.part + (int64_t)bh * a.max_chunks * (D + 2);
  float M = -INFINITY, acc = 0.f, den = 0.f;
  for (int c0 = 0; c0 < nch; c0 += U) {
    float mv[U], lv[U], ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = c0 + u < nch;
      const float* pc = part + (int64_t)min(c0 + u, nch - 1) * (D + 2);
      mv[u] = ok ? pc[0] : -INFINITY;
      lv[u] = pc[1];
      ov[u] = pc[2 + d];
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < U; ++u) Mn = fmaxf(Mn, mv[u]);
    const float alpha = fast_exp2(M - Mn);  // M = -inf on the first pass: alpha = 0
    acc *= alpha;
    den *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = fast_exp2(mv[u] - Mn);  // 0 for chunks past nch
      den = fmaf(w, lv[u], den);
      acc = fmaf(w, ov[u], acc);
    }
    M = Mn;
  }
  const float out = den > 0.f ? acc / den : 0.f;
  a.o[b * a.o_sb + h * a.o_sh + d] = E16<F16>::from_float(out);
}

// Whole-sequence decode: one workgroup of NWV = 8 waves per (sequence, kv head) reads the
// sequence's whole context, wave w taking the 32-token steps w, w + 8, ... with the split
// kernel's per-step code; the waves' partials are combined in LDS and O is written directly, so
// nothing goes through memory and no merge kernel runs.  The workgroups are dealt to the
// sequences by decreasing context (ranked in the kernel for B <= 64), so the longest start first
// and the short ones fill in behind them.  Used when the batch alone fills the chip.
template <int R, bool F16, bool SOFTCAP>
__global__ __launch_bounds__(512) void decode_whole_kernel(DecodeArgs a) {
  constexpr int D = kDecD;
  constexpr int NWV = 8;
  constexpr int PAGE_B = 16 * D * 2;
  constexpr int GRP = 32;  // steps whose page ids one fetch puts in the lanes
  __shared__ __attribute__((aligned(16))) char stage[NWV][4 * PAGE_B];
  __shared__ float s_m[NWV][R], s_l[NWV][R];
  __shared__ int s_b;
  static_assert(NWV * R * (D + 4) * 4 <= (int)sizeof(stage), "wave partials reuse the staging area");
  auto s_o = reinterpret_cast<float(*)[R][D + 4]>(&stage[0][0]);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, li = lane & 15;
  const int cmax = a.max_pages * 16;
  // kv head fastest: the workgroups of one sequence run together
  const int g = blockIdx.x % a.Hkv;
  const int rk = blockIdx.x / a.Hkv;  // the sequence's rank by decreasing context
  int b = rk;
  if (a.B <= 64) {
    if (wave == 0) {
      const int cl = lane < a.B ? min(max(a.ctx[lane], 0), cmax) : -1;
      int rank = 0;
      for (int o = 0; o < a.B; ++o) {
        const int co = __shfl(cl, o);
        rank += (co > cl) | ((co == cl) & (o < lane));
      }
      const unsigned long long hit = __ballot(lane < a.B && rank == rk);
      if (lane == 0) s_b = hit ? (int)__ffsll((long long)hit) - 1 : rk;
    }
    __syncthreads();
    b = s_b;
  }
  const int ctx = min(max(a.ctx[b], 0), cmax);
  const float cs = a.c;

  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qf[kk] = zero_bf16x8();
    if (li < R) qf[kk] = ldg8(a.q + b * a.q_sb + (g * R + li) * a.q_sh + 32 * kk + 8 * grp);
  }
  const int32_t* trow = a.table + (int64_t)b * a.max_pages;
  const uint32_t kss = (uint32_t)a.kc_ss * 2u, vss = (uint32_t)a.vc_ss * 2u;
  const int steps = (ctx + 31) / 32;
  const int nst = steps > wave ? (steps - wave + NWV - 1) / NWV : 0;  // steps of this wave

  char* vb = stage[wave];
  char* kb = stage[wave] + 2 * PAGE_B;
  int nv[2];
  int tbl = 0;
  int k0 = 0;  // first step of the fetched group
  auto load = [&](int s) {
    const int tok0 = (wave + NWV * s) * 32;  // first token of the step (< ctx)
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      nv[pg] = min(max(ctx - tok0 - 16 * pg, 0), 16);
      const int last = nv[pg] > 0 ? nv[pg] - 1 : 0;
      // a page past the context is replaced by the step's first page (its tokens are masked)
      const int phys = __builtin_amdgcn_readlane(tbl, 2 * (s - k0) + (nv[pg] > 0 ? pg : 0));
      const char* kp = reinterpret_cast<const char*>(a.kc + (int64_t)phys * a.kc_sp + (int64_t)g * a.kc_sh);
      const char* vp = reinterpret_cast<const char*>(a.vc + (int64_t)phys * a.vc_sp + (int64_t)g * a.vc_sh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + grp;
        const uint32_t slot = (uint32_t)min(r, last);
        __builtin_amdgcn_global_load_lds(kp + (slot * kss + 16u * (li ^ r)),
                                         (lds_void_t*)(kb + pg * PAGE_B + 1024 * j), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp + (slot * vss + 16u * (li ^ (2 * (r & 7)))),
                                         (lds_void_t*)(vb + pg * PAGE_B + 1024 * j), 16, 0, 0);
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int rrd = 4 * grp + (li >> 2);
  const int rd_base = rrd * 256 + 16 * ((li >> 1) & 1) + 8 * (li & 1);
  const int rd_x = rrd & 7;

  auto compute = [&]() {
    f32x4 st[2];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      st[pg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + pg * PAGE_B + li * 256 + 16 * ((4 * kk + grp) ^ li));
        st[pg] = E16<F16>::mma16(kf, qf[kk], st[pg]);
      }
    }
    float t[2][4];
    float lm = -INFINITY;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = st[pg][i];
        if constexpr (SOFTCAP) x = a.sc_out * tanh_from_exp(x * a.sc_in);  // cap before the mask
        t[pg][i] = (4 * grp + i < nv[pg]) ? x * cs : -INFINITY;
        lm = fmaxf(lm, t[pg][i]);
      }
    lm = row_swap_max(lm);
    lm = half_swap_max(lm);
    if (lm > m + kRescaleSlack) {
      const float alpha = fast_exp2(m - lm);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
      m = lm;
    }
    bf16x8 pb;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[4 * pg + i] = E16<F16>::from_float(fast_exp2(t[pg][i] - m));
        l += E16<F16>::to_float(pb[4 * pg + i]);
      }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int off = rd_base + 32 * (blk ^ rd_x);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vb + off));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vb + PAGE_B + off));
      acc[blk] = E16<F16>::mma16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, acc[blk]);
    }
  };

#pragma unroll 1
  for (k0 = 0; k0 < nst; k0 += GRP) {
    // page ids of steps k0 .. k0 + GRP - 1 of this wave: lane 2 (s - k0) + pg holds page pg of s
    if (lane < 2 * min(GRP, nst - k0)) {
      const int tok = (wave + NWV * (k0 + (lane >> 1))) * 32 + 16 * (lane & 1);
      const int lp = (tok < ctx ? tok : tok - 16) >> 4;  // a page past the context: the step's first
      const int64_t id = a.contiguous ? (int64_t)a.table[b] + lp : (int64_t)trow[lp];
      tbl = (int)min<int64_t>(max<int64_t>(id, 0), a.num_pages - 1);
    }
    const int send = min(nst, k0 + GRP);
#pragma unroll 1
    for (int s = k0; s < send; ++s) {
      load(s);
      __builtin_amdgcn_sched_barrier(0);
      compute();
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this step's LDS reads are done
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  l = row_swap_sum(l);
  l = half_swap_sum(l);
  __syncthreads();  // every wave is done with its staging area
  if (li < R) {
    if (grp == 0) {
      s_m[wave][li] = m;
      s_l[wave][li] = l;
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
      *reinterpret_cast<f32x4*>(&s_o[wave][li][16 * blk + 4 * grp]) = acc[blk];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * D; idx += 64 * NWV) {
    const int hh = idx / D, d = idx - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, s_m[w][hh]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float o = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float wt = fast_exp2(s_m[w][hh] - Mu);
      o = fmaf(wt, s_o[w][hh][d], o);
      den = fmaf(wt, s_l[w][hh], den);
    }
    a.o[b * a.o_sb + (g * R + hh) * a.o_sh + d] = E16<F16>::from_float(den > 0.f ? o / den : 0.f);
  }
}

template <bool F16, bool SC>
hipError_t launch_decode_whole_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 g1(a.B * a.Hkv), b1(512);
  switch (a.r) {
    case 1: hipLaunchKernelGGL((decode_whole_kernel<1, F16, SC>), g1, b1, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_whole_kernel<2, F16, SC>), g1, b1, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_whole_kernel<4, F16, SC>), g1, b1, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_whole_kernel<8, F16, SC>), g1, b1, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_whole(const DecodeArgs& a, int D, hipStream_t stream) {
  if (D != kDecD) return hipErrorInvalidValue;
  const bool sc = a.sc_in > 0.f;
  if (a.f16) return sc ? launch_decode_whole_t<true, true>(a, stream) : launch_decode_whole_t<true, false>(a, stream);
  return sc ? launch_decode_whole_t<false, true>(a, stream) : launch_decode_whole_t<false, false>(a, stream);
}

template <bool F16, bool SC>
hipError_t launch_decode_split_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 g1(a.B * a.Hkv * a.max_chunks), b1(256);
  switch (a.r) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<1, F16, SC>), g1, b1, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<2, F16, SC>), g1, b1, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<4, F16, SC>), g1, b1, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<8, F16, SC>), g1, b1, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, int D, hipStream_t stream) {
  if (D != kDecD) return hipErrorInvalidValue;
  const bool sc = a.sc_in > 0.f;
  if (a.f16) return sc ? launch_decode_split_t<true, true>(a, stream) : launch_decode_split_t<true, false>(a, stream);
  return sc ? launch_decode_split_t<false, true>(a, stream) : launch_decode_split_t<false, false>(a, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& a, int D, hipStream_t stream) {
  if (D != kDecD) return hipErrorInvalidValue;
  if (a.f16)
    hipLaunchKernelGGL(decode_merge_kernel<true>, dim3(a.B * a.Hq), dim3(kDecD), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<false>, dim3(a.B * a.Hq), dim3(kDecD), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
