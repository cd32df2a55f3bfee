// Measurement kernels for the benchmark's roofline peaks on the device itself: the rate of
// bf16 32x32x16 matrix instructions with independent accumulators, a streaming HBM read and
// a streaming copy.  The published MI355X figures (2.5 PFLOP/s dense bf16, 8 TB/s) assume the
// peak engine clock and ideal memory efficiency; these kernels show what a plain kernel gets
// on the box, so the benchmark can quote both.  They are not on the attention path.
#include "device_common.h"
#include "kernel_args.h"

namespace attn {

// Every wave runs `reps` rounds of 8 independent matrix instructions (8 accumulators, so
// the matrix pipe never waits for a result); one float per thread is stored so nothing is
// optimised away.
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* out, int reps) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(float)((lane + e) & 7);
    b[e] = (bf16)(float)((lane * 3 + e) & 7);
  }
  f32x16 c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[i][r] = 0.f;
  for (int it = 0; it < reps; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = mfma32(a, b, c[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[i][r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid-stride read of n 16-byte vectors; the sum is stored only if it equals a value no
// finite input produces, so the loads stay but nothing is written in practice.
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ in, int64_t n, uint4* sink) {
  uint32_t x = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const uint4 v = in[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x7fc00001u) sink[threadIdx.x] = make_uint4(x, x, x, x);
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const uint4* __restrict__ in, uint4* __restrict__ out,
                                                         int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) out[i] = in[i];
}

hipError_t launch_peak_probe(int kind, void* buf, size_t bytes, int reps, int cus, hipStream_t stream) {
  if (kind == 0) {
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(4 * cus), dim3(256), 0, stream, static_cast<float*>(buf), reps);
  } else if (kind == 1) {
    const int64_t n = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(probe_read_kernel, dim3(8 * cus), dim3(256), 0, stream, static_cast<const uint4*>(buf), n,
                       static_cast<uint4*>(buf));
  } else if (kind == 2) {
    const int64_t n = (int64_t)(bytes / 32);
    const uint4* in = static_cast<const uint4*>(buf);
    hipLaunchKernelGGL(probe_copy_kernel, dim3(8 * cus), dim3(256), 0, stream, in,
                       const_cast<uint4*>(in) + n, n);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
