// Variable-length metadata: per-sequence (offset, length) from either a right-padded 2D
// bool mask or cumulative sequence offsets.  A 2D bool padding mask selects the
// variable-length path on the page "Gemma4 FFPA attention backend support for
// accelerating Gemma4-family training" (section Integration); for a right-padded mask
// the length of row b is the number of valid entries.  Lengths are clamped to [0, S].
#include "device_common.h"
#include "kernel_args.h"

namespace attn {

__global__ __launch_bounds__(256) void varlen_prep_kernel(const uint8_t* pad_mask, const int32_t* cu_seqlens, int S,
                                                           int32_t* seq_off, int32_t* seq_len) {
  const int b = blockIdx.x;
  if (cu_seqlens) {
    if (threadIdx.x == 0) {
      const int lo = cu_seqlens[b], hi = cu_seqlens[b + 1];
      seq_off[b] = lo;
      seq_len[b] = min(max(hi - lo, 0), S);
    }
    return;
  }
  __shared__ int partial[4];
  const uint8_t* row = pad_mask + (int64_t)b * S;
  int count = 0;
  for (int i = threadIdx.x; i < S; i += 256) count += row[i] != 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) count += __shfl_xor(count, m);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = count;
  __syncthreads();
  if (threadIdx.x == 0) {
    seq_off[b] = 0;
    seq_len[b] = min(partial[0] + partial[1] + partial[2] + partial[3], S);
  }
}

hipError_t launch_varlen_prep(const uint8_t* pad_mask, const int32_t* cu_seqlens, int B, int S, int32_t* seq_off,
                              int32_t* seq_len, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_prep_kernel, dim3(B), dim3(256), 0, stream, pad_mask, cu_seqlens, S, seq_off, seq_len);
  return hipGetLastError();
}

}  // namespace attn
