// Paged-KV single-token decode: one query token per sequence against a KV cache stored
// in fixed-size pages, located through a per-sequence page table (the paged cache and
// page table of the page "flex_attention + paged KV + CUDA graphs vs vLLM", Architecture
// notes).  Pages sit anywhere in the pool, so every page costs one table lookup (that
// page's section "What each option did" measures what skipping the lookup saves when
// pages happen to be contiguous; here they are not).
//
// The work is bound by reading K and V once from HBM, so the kernel is built around
// the loads, not the matrix cores:
//   split  one workgroup per (sequence, kv head, 256-token chunk); each wave walks 4
//          pages; each 16-lane row of a wave takes one token, each lane 8 of the 128
//          head_dim values (16-byte loads, a 256-byte K or V row per row of lanes).
//          All Hq/Hkv query heads of the kv head are scored against the same loaded
//          row; the row sum runs over the 16 lanes.  An online softmax per lane row
//          gives a partial (max, sum, unnormalised output) per chunk and head.
//   merge  one workgroup per (sequence, query head) combines the chunk partials.
// Tokens at or past ctx_len are never loaded; pages are read through clamped ids.
#include "device_common.h"
#include "kernel_args.h"

namespace attn {

constexpr int kDecD = 128;
constexpr float kDecSlack = 16.0f;

template <int R>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int D = kDecD;
  constexpr int CH = kDecodeChunk;      // tokens per workgroup
  constexpr int PPW = CH / 16 / 4;      // pages per wave (16-token pages)
  __shared__ float s_m[16][R], s_l[16][R];
  __shared__ __attribute__((aligned(16))) float s_o[16][R][D];

  const int c = blockIdx.x % a.max_chunks;
  const int bg = blockIdx.x / a.max_chunks;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  int ctx = a.ctx[b];
  ctx = min(max(ctx, 0), a.max_pages * a.page_size);
  if (c * CH >= ctx) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tr = lane >> 4;       // token row within a group of 4
  const int dc = lane & 15;       // 8-wide head_dim chunk
  const float cs = a.c;

  float q[R][8];
#pragma unroll
  for (int hh = 0; hh < R; ++hh) {
    const bf16x8 x = ldg8(a.q + b * a.q_sb + (g * R + hh) * a.q_sh + 8 * dc);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[hh][e] = (float)x[e] * cs;
  }
  float m[R], l[R], o[R][8];
#pragma unroll
  for (int hh = 0; hh < R; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }

  const int ps = a.page_size;  // 16 (checked on the host)
  const int32_t* trow = a.table + (int64_t)b * a.max_pages;
#pragma unroll 1
  for (int p = 0; p < PPW; ++p) {
    const int lp = (c * CH) / 16 + wave * PPW + p;  // logical page
    if (lp * 16 >= ctx) break;
    int phys = trow[lp];
    phys = min(max(phys, 0), a.num_pages - 1);
    const bf16* kp = a.kc + (int64_t)phys * a.kc_sp + g * a.kc_sh + 8 * dc;
    const bf16* vp = a.vc + (int64_t)phys * a.vc_sp + g * a.vc_sh + 8 * dc;
    bf16x8 kx[4], vx[4];
    const int nvalid = min(16, ctx - lp * 16);
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int slot = 4 * gq + tr;
      const int sl = min(slot, nvalid - 1);  // never read past the context
      kx[gq] = ldg8(kp + (int64_t)sl * a.kc_ss);
      vx[gq] = ldg8(vp + (int64_t)sl * a.vc_ss);
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const bool valid = 4 * gq + tr < nvalid;
      float kf[8], vf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kf[e] = (float)kx[gq][e];
        vf[e] = (float)vx[gq][e];
      }
#pragma unroll
      for (int hh = 0; hh < R; ++hh) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(q[hh][e], kf[e], s);
        s += __shfl_xor(s, 8, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 1, 16);
        s = valid ? s : -INFINITY;
        if (s > m[hh] + kDecSlack) {  // raise the reference (uniform across the 16-lane row)
          const float alpha = fast_exp2(m[hh] - s);
          l[hh] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[hh][e] *= alpha;
          m[hh] = s;
        }
        const float pr = valid ? fast_exp2(s - m[hh]) : 0.f;
        l[hh] += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pr, vf[e], o[hh][e]);
      }
    }
  }

  const int row = wave * 4 + tr;
#pragma unroll
  for (int hh = 0; hh < R; ++hh) {
    if (dc == 0) {
      s_m[row][hh] = m[hh];
      s_l[row][hh] = l[hh];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_o[row][hh][8 * dc + e] = o[hh][e];
  }
  __syncthreads();
  // combine the 16 lane rows: thread t handles (head, d) pairs t and t + 256
  for (int idx = threadIdx.x; idx < R * D; idx += 256) {
    const int hh = idx / D, d = idx - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) M = fmaxf(M, s_m[i][hh]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float acc = 0.f, den = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float w = fast_exp2(s_m[i][hh] - Mu);
      acc = fmaf(w, s_o[i][hh][d], acc);
      den = fmaf(w, s_l[i][hh], den);
    }
    float* part = a.part + ((int64_t)(b * a.Hq + g * R + hh) * a.max_chunks + c) * (D + 2);
    if (d == 0) {
      part[0] = Mu;
      part[1] = den;
    }
    part[2 + d] = acc;
  }
}

__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a) {
  constexpr int D = kDecD;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  int ctx = a.ctx[b];
  ctx = min(max(ctx, 0), a.max_pages * a.page_size);
  const int nch = (ctx + kDecodeChunk - 1) / kDecodeChunk;
  const int d = threadIdx.x;
  const float* part = a.part + (int64_t)bh * a.max_chunks * (D + 2);
  float M = -INFINITY;
  for (int ch = 0; ch < nch; ++ch) M = fmaxf(M, part[ch * (D + 2)]);
  float acc = 0.f, den = 0.f;
  for (int ch = 0; ch < nch; ++ch) {
    const float w = fast_exp2(part[ch * (D + 2)] - M);
    den = fmaf(w, part[ch * (D + 2) + 1], den);
    acc = fmaf(w, part[ch * (D + 2) + 2 + d], acc);
  }
  const float out = den > 0.f ? acc / den : 0.f;
  a.o[b * a.o_sb + h * a.o_sh + d] = (bf16)out;
}

hipError_t launch_decode(const DecodeArgs& a, int D, hipStream_t stream) {
  if (D != kDecD) return hipErrorInvalidValue;
  const dim3 g1(a.B * a.Hkv * a.max_chunks), b1(256);
  switch (a.r) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, g1, b1, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, g1, b1, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, g1, b1, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(decode_split_kernel<8>, g1, b1, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(a.B * a.Hq), dim3(kDecD), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
