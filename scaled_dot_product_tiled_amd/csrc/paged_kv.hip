// Paged KV cache maintenance around the paged decode: appending the newest tokens of each
// sequence to its pages, and gathering a sequence's cached tokens into a contiguous tensor
// (the key/value side of a paged prefill, run as a chunk-pair forward).  The page table maps
// logical page p of sequence b to physical page table[b][p] (the PagedKVCache + PageTable
// arrangement of the page "flex_attention + paged KV + CUDA graphs vs vLLM", Architecture
// notes); token t of sequence b lives in slot t % page_size of logical page t / page_size.
//
// HBM-bound copies: one thread moves 16 bytes (8 elements) of one token row of one kv head,
// a row being D/8 consecutive threads, so every access is a whole, aligned 16-byte vector.
// Positions whose page id falls outside [0, num_pages) are never touched (append) or read as
// zeros (gather), so a bad table entry cannot move data outside the pool.
#include "device_common.h"
#include "kernel_args.h"

namespace attn {

__global__ __launch_bounds__(256) void paged_kv_copy_kernel(PagedCopyArgs a) {
  const int tpr = a.D / 8;  // threads per token row
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.n * a.Hkv;
  const int64_t row = gi / tpr;
  if (row >= 2 * rows) return;  // K rows, then V rows
  const int which = row >= rows;
  const int64_t rr = which ? row - rows : row;
  const int c0 = 8 * (int)(gi - row * tpr);
  const int g = (int)(rr % a.Hkv);
  const int64_t bi = rr / a.Hkv;
  const int i = (int)(bi % a.n);
  const int b = (int)(bi / a.n);

  int ctx = a.ctx[b];
  ctx = min(max(ctx, 0), a.max_pages * a.page_size);
  // append: token i is the (n - i)-th newest, at position ctx - n + i; gather: position i
  const int pos = a.gather ? i : ctx - a.n + i;
  const bool live = pos >= 0 && pos < ctx;
  int page = -1;
  if (live) {
    page = a.table[(int64_t)b * a.max_pages + pos / a.page_size];
    if (page >= a.num_pages) page = -1;
  }
  const int slot = pos - (pos / a.page_size) * a.page_size;
  bf16* cache = which ? a.vc : a.kc;
  const int64_t cp = which ? a.vc_sp : a.kc_sp, cs = which ? a.vc_ss : a.kc_ss, ch = which ? a.vc_sh : a.kc_sh;
  bf16* tok = which ? a.tv : a.tk;
  const int64_t ts_b = which ? a.tv_sb : a.tk_sb, ts_s = which ? a.tv_ss : a.tk_ss, ts_h = which ? a.tv_sh : a.tk_sh;
  bf16* t = tok + b * ts_b + (int64_t)i * ts_s + g * ts_h + c0;
  if (a.gather) {
    bf16x8 x = zero_bf16x8();
    if (page >= 0) x = *reinterpret_cast<const bf16x8*>(cache + page * cp + slot * cs + g * ch + c0);
    *reinterpret_cast<bf16x8*>(t) = x;
  } else if (page >= 0) {
    *reinterpret_cast<bf16x8*>(cache + page * cp + slot * cs + g * ch + c0) = *reinterpret_cast<const bf16x8*>(t);
  }
}

hipError_t launch_paged_kv_copy(const PagedCopyArgs& a, hipStream_t stream) {
  const int64_t threads = 2 * (int64_t)a.B * a.n * a.Hkv * (a.D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  hipLaunchKernelGGL(paged_kv_copy_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
