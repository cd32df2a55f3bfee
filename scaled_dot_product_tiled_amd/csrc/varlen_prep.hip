// Variable-length metadata: per-sequence (offset, length) from either a right-padded 2D
// bool mask or cumulative sequence offsets.  A 2D bool padding mask selects the
// variable-length path on the page "Gemma4 FFPA attention backend support for
// accelerating Gemma4-family training" (section Integration); for a right-padded mask
// the length of row b is the number of valid entries.  Lengths are clamped to [0, S], and
// packed offsets to the packed rows, so no later access leaves the caller's buffers even when
// the metadata is wrong.
//
// The metadata's own consistency (a prefix mask, non-decreasing offsets that end at the row
// count, page ids inside the pool) is checked only on request, by the check kernels below: they
// raise a device-side error word that the host reads after synchronising.
#include "device_common.h"
#include "kernel_args.h"

namespace attn {

__global__ __launch_bounds__(256) void varlen_prep_kernel(const uint8_t* pad_mask, const int32_t* cu_seqlens, int S,
                                                           int total, int32_t* seq_off, int32_t* seq_len) {
  const int b = blockIdx.x;
  if (cu_seqlens) {
    if (threadIdx.x == 0) {
      const int lo = min(max(cu_seqlens[b], 0), total), hi = cu_seqlens[b + 1];
      seq_off[b] = lo;
      seq_len[b] = min(min(max(hi - lo, 0), S), total - lo);
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

hipError_t launch_varlen_prep(const uint8_t* pad_mask, const int32_t* cu_seqlens, int B, int S, int total,
                              int32_t* seq_off, int32_t* seq_len, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_prep_kernel, dim3(B), dim3(256), 0, stream, pad_mask, cu_seqlens, S, total, seq_off,
                     seq_len);
  return hipGetLastError();
}

// Rank of sequence b among all B by decreasing length, ties by index: the number of sequences
// that come before it.  O(B^2) reads of B lengths, all from cache; used for B <= kOrderMaxBatch.
__global__ __launch_bounds__(256) void varlen_order_kernel(const int32_t* seq_len, int B, int32_t* order) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int lb = seq_len[b];
  int rank = 0;
  for (int o = 0; o < B; ++o) {
    const int lo = seq_len[o];
    rank += (lo > lb) | ((lo == lb) & (o < b));
  }
  order[rank] = b;
}

hipError_t launch_varlen_order(const int32_t* seq_len, int B, int32_t* order, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_order_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, seq_len, B, order);
  return hipGetLastError();
}

// Rank of paged sequence b by decreasing work, the product of its new query rows and its cached
// keys (both clamped as the forward clamps them), ties by index: order[rank] = b.  Used for the
// deal of the split paged forward (B below the compute-unit count there).
__global__ __launch_bounds__(256) void paged_rank_kernel(const int32_t* cu_q, const int32_t* kv_len, int B, int total,
                                                          int max_q, int max_keys, int32_t* order) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  auto work = [&](int s) {
    const int off = min(max(cu_q[s], 0), total);
    const int n = min(min(max(cu_q[s + 1] - off, 0), total - off), max_q);
    return (int64_t)n * min(max(kv_len[s], 0), max_keys);
  };
  const int64_t wb = work(b);
  int rank = 0;
  for (int o = 0; o < B; ++o) {
    const int64_t wo = work(o);
    rank += (wo > wb) | ((wo == wb) & (o < b));
  }
  order[rank] = b;
}

hipError_t launch_paged_rank(const int32_t* cu_q, const int32_t* kv_len, int B, int total, int max_q, int max_keys,
                             int32_t* order, hipStream_t stream) {
  hipLaunchKernelGGL(paged_rank_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, cu_q, kv_len, B, total, max_q,
                     max_keys, order);
  return hipGetLastError();
}

// Thread b sums the dS blocks of sequences 0 .. b-1 (O(B^2) reads of B lengths, all from cache;
// used for B <= kOrderMaxBatch).  With consistent offsets the host's capacity bound holds; with
// overlapping ones the lengths can sum past the packed rows, and a sequence that would not fit
// is marked -1 so that the backward skips it instead of writing past the workspace.
__global__ __launch_bounds__(256) void ds_seq_base_kernel(const int32_t* seq_len, int B, int Hq, int tri, int cnt,
                                                           int64_t capacity, int64_t* ds_seq) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  int64_t base = 0;
  for (int o = 0; o < b; ++o) base += (int64_t)Hq * ds_head_blocks(seq_len[o], tri, cnt);
  const int64_t need = (int64_t)Hq * ds_head_blocks(seq_len[b], tri, cnt);
  ds_seq[b] = base + need <= capacity ? base : -1;
}

hipError_t launch_ds_seq_base(const int32_t* seq_len, int B, int Hq, int tri, int cnt, int64_t capacity,
                              int64_t* ds_seq, hipStream_t stream) {
  hipLaunchKernelGGL(ds_seq_base_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, seq_len, B, Hq, tri, cnt,
                     capacity, ds_seq);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Metadata checks (debug mode).  Any thread that finds a violation stores 1 to the error word.
// ---------------------------------------------------------------------------
__device__ int g_meta_error;

__global__ __launch_bounds__(256) void varlen_check_kernel(const uint8_t* pad_mask, const int32_t* cu_seqlens, int B,
                                                            int S, int total) {
  const int b = blockIdx.x;
  if (cu_seqlens) {
    if (threadIdx.x == 0) {
      const int lo = cu_seqlens[b], hi = cu_seqlens[b + 1];
      const bool bad = (b == 0 && lo != 0) || hi < lo || hi - lo > S || hi > total || (b == B - 1 && hi != total);
      if (bad) g_meta_error = 1;
    }
    return;
  }
  // a right-padded prefix: entry i is valid exactly when i < (number of valid entries)
  __shared__ int partial[4];
  const uint8_t* row = pad_mask + (int64_t)b * S;
  int count = 0;
  for (int i = threadIdx.x; i < S; i += 256) count += row[i] != 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) count += __shfl_xor(count, m);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = count;
  __syncthreads();
  const int n = partial[0] + partial[1] + partial[2] + partial[3];
  bool bad = false;
  for (int i = threadIdx.x; i < S; i += 256) bad |= (row[i] != 0) != (i < n);
  if (bad) g_meta_error = 1;
}

// contiguous: table holds one first page per sequence, whose pages must lie inside the pool.
__global__ __launch_bounds__(256) void pages_check_kernel(const int32_t* table, int contiguous, const int32_t* ctx,
                                                           int max_pages, int page_size, int num_pages) {
  const int b = blockIdx.x;
  const int n = ctx[b];
  if (n < 0 || (int64_t)n > (int64_t)max_pages * page_size) {
    if (threadIdx.x == 0) g_meta_error = 1;
    return;
  }
  const int pages = (n + page_size - 1) / page_size;
  if (contiguous) {
    if (threadIdx.x == 0 && pages > 0 && (table[b] < 0 || (int64_t)table[b] + pages > num_pages)) g_meta_error = 1;
    return;
  }
  bool bad = false;
  for (int p = threadIdx.x; p < pages; p += 256) {
    const int id = table[(int64_t)b * max_pages + p];
    bad |= id < 0 || id >= num_pages;
  }
  if (bad) g_meta_error = 1;
}

// Runs one check kernel on the stream, waits for it and reports whether it found a violation.
template <class L>
static hipError_t run_check(hipStream_t stream, bool& bad, L&& launch) {
  const int zero = 0;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_meta_error), &zero, sizeof(int), 0, hipMemcpyHostToDevice,
                                        stream);
  if (e != hipSuccess) return e;
  launch();
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int flag = 0;
  if ((e = hipMemcpyFromSymbolAsync(&flag, HIP_SYMBOL(g_meta_error), sizeof(int), 0, hipMemcpyDeviceToHost,
                                    stream)) != hipSuccess)
    return e;
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
  bad = flag != 0;
  return hipSuccess;
}

hipError_t check_varlen_meta(const uint8_t* pad_mask, const int32_t* cu_seqlens, int B, int S, int total,
                             hipStream_t stream, bool& bad) {
  return run_check(stream, bad, [&] {
    hipLaunchKernelGGL(varlen_check_kernel, dim3(B), dim3(256), 0, stream, pad_mask, cu_seqlens, B, S, total);
  });
}

hipError_t check_pages_meta(const int32_t* table, int contiguous, const int32_t* ctx, int B, int max_pages,
                            int page_size, int num_pages, hipStream_t stream, bool& bad) {
  return run_check(stream, bad, [&] {
    hipLaunchKernelGGL(pages_check_kernel, dim3(B), dim3(256), 0, stream, table, contiguous, ctx, max_pages,
                       page_size, num_pages);
  });
}

}  // namespace attn
