// Log-sum-exp merge of two partial attention results of the same query rows over disjoint
// key sets.  A row's attention over keys K1 u K2 is the LSE-weighted mix of its attention
// over K1 and over K2: with L = ln(e^L1 + e^L2), O = e^(L1 - L) O1 + e^(L2 - L) O2.  This is
// how the ring path of the page "Gemma4 FFPA attention backend support for accelerating
// Gemma4-family training" (section Integration) combines the full-attention chunks that
// one rank computes as the key/value chunks pass around the ring; the forward returns LSE
// for exactly this purpose.
//
// Partials and the running result are fp32, so a row's output is rounded to bf16 once,
// when the last partial has been merged (the optional bf16 output), however many ring
// steps it took.
//
// Memory-bound and elementwise: one row (head_dim D) is D/8 lanes of one wave, each
// owning 8 contiguous floats of O; the two weights are computed in fp32 from the row's
// two LSE values, the larger of which is the reference, so the weights are e^0 = 1 and
// e^-(|L1 - L2|) before normalising and never overflow.  A partial with LSE = -inf (a row
// that saw no key of that chunk) has weight 0 and its O is not read into the result; two
// of them give O = 0 and LSE = -inf.  The result is written over the first partial, in
// place: every lane of a row reads the row's LSE before the row's first lane stores it,
// since the row is one wave and the store follows the loads in program order.
#include "device_common.h"
#include "kernel_args.h"

namespace attn {

template <int D, bool F16>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 8;      // lanes per row
  constexpr int RPB = 256 / TPR;  // rows per workgroup
  static_assert(TPR <= 64, "a row must stay inside one wave");
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= a.rows) return;
  const int t = threadIdx.x % TPR;
  // row = (b * S + s) * H + h
  const int h = row % a.H;
  const int bs = row / a.H;
  const int s = bs % a.S;
  const int b = bs / a.S;
  const int64_t li = ((int64_t)b * a.H + h) * a.S + s;
  const MergeWeights w = lse_merge_weights(a.lse[li], a.lse_part[li]);
  float* o1 = a.o + b * a.o_sb + (int64_t)s * a.o_ss + h * a.o_sh + 8 * t;
  const float* o2 = a.o_part + b * a.p_sb + (int64_t)s * a.p_ss + h * a.p_sh + 8 * t;
  float y[8];
#pragma unroll
  for (int hv = 0; hv < 2; ++hv) {
    const float4 x1 = *reinterpret_cast<const float4*>(o1 + 4 * hv);
    const float4 x2 = *reinterpret_cast<const float4*>(o2 + 4 * hv);
    const float a1[4] = {x1.x, x1.y, x1.z, x1.w}, a2[4] = {x2.x, x2.y, x2.z, x2.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) y[4 * hv + e] = lse_merge_value(w, a1[e], a2[e]);
  }
  stg4(o1, y[0], y[1], y[2], y[3]);
  stg4(o1 + 4, y[4], y[5], y[6], y[7]);
  if (a.out) {
    bf16* r = a.out + b * a.r_sb + (int64_t)s * a.r_ss + h * a.r_sh + 8 * t;
    stg4e<F16>(r, y[0], y[1], y[2], y[3]);
    stg4e<F16>(r + 4, y[4], y[5], y[6], y[7]);
  }
  if (t == 0) a.lse[li] = w.lse;
}

template <bool F16>
hipError_t launch_lse_merge_t(const MergeArgs& a, int D, hipStream_t stream) {
  const int rpb = 256 / (D / 8);
  const dim3 grid((a.rows + rpb - 1) / rpb), block(256);
  if (D == 512)
    hipLaunchKernelGGL((lse_merge_kernel<512, F16>), grid, block, 0, stream, a);
  else if (D == 256)
    hipLaunchKernelGGL((lse_merge_kernel<256, F16>), grid, block, 0, stream, a);
  else if (D == 128)
    hipLaunchKernelGGL((lse_merge_kernel<128, F16>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeArgs& a, int D, hipStream_t stream) {
  return a.out_f16 ? launch_lse_merge_t<true>(a, D, stream) : launch_lse_merge_t<false>(a, D, stream);
}

}  // namespace attn
