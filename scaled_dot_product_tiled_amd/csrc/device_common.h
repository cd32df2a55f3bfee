// Device-side building blocks shared by the libattn kernels (gfx950 / CDNA4).
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, one wave of 64 lanes):
//   A operand (32 x 16): lane l holds row (l % 32), 8 consecutive k of group (l / 32)
//   B operand (16 x 32): lane l holds column (l % 32), the same 8 k of group (l / 32)
//   C/D (32 x 32, 16 fp32 per lane): register r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
//   column l % 32.
// Only the C layout matters for correctness below: A and B always take the same
// (lane group, element) -> k assignment, so any such assignment sums the same products.
//
// LDS tiles hold rows of D bf16 with no padding.  The 16-byte chunk c of row r is stored
// at chunk position c ^ h(r), h(r) = 4 (r & 3) + ((r >> 2) & 3).  With 64 four-byte
// banks, one pass of a 16-byte-per-lane read serves 16 lanes and one pass of an
// 8-byte-per-lane read serves 32 lanes; h makes both access patterns used here
// conflict-free: 16 consecutive rows at one chunk (row fragments), and 4 consecutive
// rows x 4 consecutive chunks (transposing reads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
// A running row maximum is only raised when a new score exceeds it by more than
// this many powers of two; exponentials then stay below 2^8, exact in fp32 and
// rounded relative to their own size in bf16.  The normaliser uses the same
// reference value, so the result is unchanged in exact arithmetic.
constexpr float kRescaleSlack = 8.0f;

// 16-bit element types: bfloat16 (F16 = false) or IEEE half (F16 = true).  Tensors, LDS
// tiles and matrix operands are moved as 16-bit patterns in the bf16 storage type; only the
// matrix instruction and the conversions to and from fp32 (round to nearest even) depend on
// the type.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <bool F16>
struct E16;

template <>
struct E16<false> {
  static __device__ __forceinline__ bf16 from_float(float x) { return (bf16)x; }
  static __device__ __forceinline__ float to_float(bf16 x) { return (float)x; }
  static __device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct E16<true> {
  static __device__ __forceinline__ bf16 from_float(float x) { return __builtin_bit_cast(bf16, (_Float16)x); }
  static __device__ __forceinline__ float to_float(bf16 x) { return (float)__builtin_bit_cast(_Float16, x); }
  static __device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  }
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) { return E16<false>::mma32(a, b, c); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh(x).  For |x| >= 1/8 from the exponential, tanh(x) = sign(x) (1 - 2 / (e^(2|x|) + 1))
// with e^(2|x|) = 2^(2 log2(e) |x|) (for large |x| the exponential overflows to inf and the
// result is +-1 exactly).  Below 1/8 that difference would cancel to a few ulps of 1, so the
// Taylor series x (1 - x^2/3 + 2x^4/15 - 17x^6/315) is used instead (next term 62x^9/2835:
// relative error below 2e-9).
__device__ __forceinline__ float tanh_from_exp(float x) {
  const float ax = fabsf(x);
  const float e = fast_exp2(2.8853900817779268f * ax);
  const float big = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  const float x2 = ax * ax;
  const float small = ax * fmaf(x2, fmaf(x2, fmaf(x2, -0.053968253968253971f, 0.13333333333333333f),
                                         -0.33333333333333333f), 1.0f);
  return copysignf(ax < 0.125f ? small : big, x);
}

// Value of this lane's partner in the other half of the wave (lane ^ 32), combined.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles
// ---------------------------------------------------------------------------
__device__ __forceinline__ constexpr int swz_h(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Element offset of (row, col) in a swizzled tile of D columns.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + (((col >> 3) ^ swz_h(row)) << 3) + (col & 7);
}

// Row fragments for the MFMA operand "row (lane % 32), k chunk 2t + (lane / 32)" of a
// tile whose row block starts at a multiple of 16: the byte offset is one of eight
// lane-dependent bases (t & 7) plus a constant, so a fully unrolled loop needs eight
// address registers and immediate offsets.
template <int D>
struct RowFrags {
  int base[8];
  __device__ __forceinline__ explicit RowFrags(int lane) {
    const int ln = lane & 31, g2 = lane >> 5;
#pragma unroll
    for (int q = 0; q < 8; ++q) base[q] = ln * D * 2 + 16 * ((2 * q + g2) ^ swz_h(ln));
  }
  // rows rblk + lane % 32 (rblk a multiple of 16), k step t (columns 16t .. 16t+15)
  __device__ __forceinline__ bf16x8 read(const bf16* tile, int rblk, int t) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + base[t & 7] +
                                            rblk * D * 2 + 256 * (t >> 3));
  }
};

// Transposing fragments of a row-major tile T (rows = contraction index k): read(kbase,
// db) returns, for lane l with g = l / 32, T[kbase + 4g + e][32 db + l%32] for e = 0..3
// and T[kbase + 8 + 4g + e - 4][32 db + l%32] for e = 4..7.  This is the k order in
// which a C-layout accumulator over the same 16 rows feeds a B operand.  kbase is a
// multiple of 16.
template <int D>
struct TrFrags {
  int base[8];  // [half][db & 3]
  __device__ __forceinline__ explicit TrFrags(int lane) {
    const int G = lane >> 4, i = lane & 15;
    const int rl = 4 * (G >> 1) + (i >> 2);
    const int u = 2 * (G & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int x = 0; x < 4; ++x)
        base[4 * hf + x] = (rl + 8 * hf) * D * 2 + 16 * ((4 * x + u) ^ swz_h(rl + 8 * hf)) + 8 * (i & 1);
  }
  __device__ __forceinline__ bf16x8 read(const bf16* tile, int kbase, int db) const {
    return read_with(tile, kbase, db, base[db & 3], base[4 + (db & 3)]);
  }
  // The two bases of column block db, chosen without indexing the array by a run-time
  // value (which would put it in scratch memory).
  __device__ __forceinline__ void pick(int db, int& lo, int& hi) const {
    const int x = db & 3;
    lo = x == 0 ? base[0] : x == 1 ? base[1] : x == 2 ? base[2] : base[3];
    hi = x == 0 ? base[4] : x == 1 ? base[5] : x == 2 ? base[6] : base[7];
  }
  __device__ __forceinline__ bf16x8 read_with(const bf16* tile, int kbase, int db, int lo, int hi) const {
    const char* t = reinterpret_cast<const char*>(tile) + kbase * D * 2 + 256 * (db >> 2);
    bf16x4 l = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(t + lo));
    bf16x4 h = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(t + hi));
    return __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// Memory -> LDS copies (global_load_lds / buffer_load ... lds).  They are issued from inline
// assembly rather than the compiler builtins: with the builtin, the compiler waits for
// every outstanding LDS read before each later LDS read, which exposes the LDS latency in
// front of every matrix-core instruction.  Completion is tracked here by hand (wait_vmcnt +
// barrier).  The instructions take their LDS base from M0, written here just before each
// with one wait state between the write and the use.  Nothing else in these kernels uses
// M0 (no LDS DMA builtin, no dynamically indexed register arrays), so no value is lost.
// 4 bytes per lane: lane l writes lds_base + 4 l; its source is the per-lane address src.
__device__ __forceinline__ void lds_dma4(void* lds_base, const void* src) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(src)
               : "memory");
}

// Asynchronous copy of a tile of ROWS rows into a swizzled LDS tile, straight from memory
// to LDS with buffer loads (buffer_load_dwordx4 ... lds).  The source is described once per
// tile (TileSrc: a buffer resource based at the tile's first row whose range covers only its
// first `nvalid` rows); rows past them read as zeros through the buffer range check, so
// ragged tiles need no clamping.  Each wave-instruction moves 1 KB (64 lanes x 16 bytes) to
// consecutive LDS; wave `wave` of NW issues instructions wave, wave+NW, ...; dma_rows_one
// issues this wave's k-th one, so callers can spread a copy over a loop of matrix
// instructions.  Per instruction this costs one M0 write and a couple of address
// instructions, where a global-address copy needed a 64-bit row address computation.
// Nothing is waited for here: the caller waits with wait_vmcnt and a barrier.  `wave` must
// be wave-uniform.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

struct TileSrc {
  i32x4 rsrc;
  uint32_t row_bytes;
};

template <int ROWS>
__device__ __forceinline__ TileSrc tile_src(const bf16* g, int64_t stride, int row0, int nvalid) {
  nvalid = min(max(nvalid, 0), ROWS);
  const uint64_t p = (uint64_t)(uintptr_t)(g + (int64_t)row0 * stride);
  TileSrc t;
  t.row_bytes = (uint32_t)(stride * 2);
  t.rsrc[0] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  t.rsrc[1] = (int32_t)(__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xffffu);  // stride field 0
  t.rsrc[2] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)nvalid * t.row_bytes);  // bytes in range
  t.rsrc[3] = 0x00020000;                                                                // raw 32-bit data
  return t;
}

// The same for a tile whose first row is at `row0` (rows `stride` elements apart).
template <int ROWS>
__device__ __forceinline__ TileSrc tile_src_rows(const bf16* row0, int64_t stride, int nvalid) {
  return tile_src<ROWS>(row0, stride, 0, nvalid);
}

template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_rows_one(bf16* tile, const TileSrc& src, int wave, int lane, int k) {
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int RPI = 64 / CH;   // rows per wave-instruction
  constexpr int NI = ROWS / RPI;
  static_assert(CH >= 16 && 64 % CH == 0, "row must be 256..1024 bytes");
  static_assert(NI % NW == 0, "tile must split evenly over the waves");
  const int i = wave + k * NW;
  const int trow = i * RPI + lane / CH;  // row within the tile
  const uint32_t voff = (uint32_t)trow * src.row_bytes + (uint32_t)(16 * ((lane % CH) ^ swz_h(trow)));
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + i * RPI * D));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff),
               "s"(src.rsrc)
               : "memory");
}

// All of this wave's instructions of one tile copy, back to back.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_rows(bf16* tile, const TileSrc& src, int wave, int lane) {
  constexpr int NK = ROWS * D / 512 / NW;
#pragma unroll
  for (int k = 0; k < NK; ++k) dma_rows_one<D, ROWS, NW>(tile, src, wave, lane, k);
}

template <int D, int ROWS, int NW>
constexpr int dma_rows_per_wave() { return ROWS * D / 512 / NW; }

// A tile of ROWS key / value rows of a paged cache: 16-token pages, rows of one page at a fixed
// slot stride, the pages anywhere in the pool.  One buffer resource per page; rows past `nvalid`
// read as zeros.  row0 is a multiple of 16.
template <int ROWS>
struct PagedTileSrc {
  static_assert(ROWS % 16 == 0, "whole pages");
  TileSrc pg[ROWS / 16];
};

// The physical page ids of the two pages of a 32-row tile starting at row0 (a multiple of 16),
// of which nvalid >= 1 rows are valid, from the sequence's page-table row `trow`.  They are read
// with scalar loads and one wait for those loads alone: the compiler would otherwise emit a
// vector load whose wait also drains the tile copies still in flight.  The second entry is only
// read when the second page holds a valid row (else the first entry is read again and the id
// goes unused).
__device__ __forceinline__ void table_pages2(int (&phys)[2], const int32_t* trow, int row0, int nvalid) {
  const uint64_t base = (uint64_t)(uintptr_t)trow;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const uint64_t ub = ((uint64_t)hi << 32) | lo;
  const uint32_t o0 = __builtin_amdgcn_readfirstlane((uint32_t)(row0 >> 4) * 4u);
  const uint32_t o1 = __builtin_amdgcn_readfirstlane(o0 + (nvalid > 16 ? 4u : 0u));
  int p0, p1;
  asm volatile("s_load_dword %0, %2, %3\n\ts_load_dword %1, %2, %4\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(p0), "=&s"(p1)
               : "s"(ub), "s"(o0), "s"(o1)
               : "memory");
  phys[0] = p0;
  phys[1] = p1;
}

template <int ROWS>
__device__ __forceinline__ PagedTileSrc<ROWS> paged_tile_src(const bf16* cache, int64_t page_stride,
                                                             int64_t slot_stride, const int (&phys)[ROWS / 16],
                                                             int num_pages, int nvalid) {
  PagedTileSrc<ROWS> t;
#pragma unroll
  for (int p = 0; p < ROWS / 16; ++p) {
    const int id = min(max(phys[p], 0), num_pages - 1);  // out-of-pool ids are clamped, never followed
    t.pg[p] = tile_src<16>(cache + (int64_t)id * page_stride, slot_stride, 0, nvalid - 16 * p);
  }
  return t;
}

// dma_rows for a paged tile: wave-instruction i moves tile rows i * RPI .. (all in one page)
// from that page's resource into the same swizzled LDS positions dma_rows uses.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_rows_paged(bf16* tile, const PagedTileSrc<ROWS>& src, int wave, int lane) {
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  constexpr int NI = ROWS / RPI;
  static_assert(16 % RPI == 0 && NI % NW == 0, "an instruction's rows lie in one page");
#pragma unroll
  for (int k = 0; k < NI / NW; ++k) {
    const int i = wave + k * NW;
    const int page = (i * RPI) >> 4;  // wave-uniform
    const int trow = i * RPI + lane / CH;
    // the page's resource, selected without indexing the array by a run-time value and kept
    // in scalar registers (the instruction takes it from there)
    i32x4 rs = src.pg[0].rsrc;
    uint32_t rb = src.pg[0].row_bytes;
#pragma unroll
    for (int p = 1; p < ROWS / 16; ++p)
      if (page == p) {
        rs = src.pg[p].rsrc;
        rb = src.pg[p].row_bytes;
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) rs[e] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)rs[e]);
    const uint32_t voff = (uint32_t)(trow & 15) * rb + (uint32_t)(16 * ((lane % CH) ^ swz_h(trow)));
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + i * RPI * D));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff),
                 "s"(rs)
                 : "memory");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that first retires this wave's outstanding LDS reads, so that a
// buffer may be refilled by any wave once every wave has passed it.  Global loads in
// flight are not waited for.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
  return z;
}

__device__ __forceinline__ bf16x8 ldg8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ void stg4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}

// Four fp32 values rounded to the 16-bit type F16 selects.
template <bool F16>
__device__ __forceinline__ void stg4e(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = E16<F16>::from_float(a);
  v[1] = E16<F16>::from_float(b);
  v[2] = E16<F16>::from_float(c);
  v[3] = E16<F16>::from_float(d);
  *reinterpret_cast<bf16x4*>(p) = v;
}

__device__ __forceinline__ void stg4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Store to an output that is either the 16-bit type F16 selects or fp32.
template <bool F16>
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) { stg4e<F16>(p, a, b, c, d); }
template <bool F16>
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) { stg4(p, a, b, c, d); }

// Log-sum-exp merge of two partial results of one query row over disjoint key sets:
// L = ln(e^l1 + e^l2) and O = e^(l1 - L) O1 + e^(l2 - L) O2.  The larger LSE is the
// reference, so the two exponentials are 1 and e^-|l1 - l2| and never overflow; a partial
// with LSE = -inf gets weight 0, and two of them give L = -inf.  The standalone merge
// kernel and the forward's merging epilogue both use these two functions, with
// contraction off, so the fused and the two-step paths round identically.
struct MergeWeights {
  float w1, w2, lse;
};

__device__ __forceinline__ MergeWeights lse_merge_weights(float l1, float l2) {
  MergeWeights w = {0.f, 0.f, -INFINITY};
  const float m = fmaxf(l1, l2);
  if (m > -INFINITY) {
    const float e1 = expf(l1 - m), e2 = expf(l2 - m);  // the larger is exactly 1; e^-inf = 0
    const float tot = e1 + e2;
    w.w1 = e1 / tot;
    w.w2 = e2 / tot;
    w.lse = m + log1pf(fminf(e1, e2));
  }
  return w;
}

// One merged element.  A zero weight selects, so a non-finite value in a partial that does
// not contribute cannot leak in.
__device__ __forceinline__ float lse_merge_value(const MergeWeights& w, float a1, float a2) {
#pragma clang fp contract(off)
  const float v1 = w.w1 > 0.f ? w.w1 * a1 : 0.f;
  const float v2 = w.w2 > 0.f ? w.w2 * a2 : 0.f;
  return v1 + v2;
}

// p[0..3] += (a, b, c, d) in fp32; p is owned by this lane alone.
__device__ __forceinline__ void add4(float* p, float a, float b, float c, float d) {
  float4 v = *reinterpret_cast<const float4*>(p);
  v.x += a;
  v.y += b;
  v.z += c;
  v.w += d;
  *reinterpret_cast<float4*>(p) = v;
}

// Work-item order.  Items are (unit, w) with W items per unit, w = 0 the heaviest.
// Consecutive workgroup ids land on consecutive XCDs (id % 8).  When every unit carries the
// same work (dense inputs), the items of one XCD are taken from one contiguous range of the
// item list, heaviest first within each unit: the workgroups of a unit then share K/V in
// that XCD's L2.  When units differ (variable lengths), whole units still stay on one XCD,
// but they are dealt to the XCDs by decreasing length in a snake order (XCD 0..7, then
// 7..0, ...), `upb` consecutive units per sequence, which evens out the XCDs' totals; an XCD
// takes its units one after the other, each unit's items heaviest first, so that the
// workgroups running together on it stream the same tiles (taking its units' items in rounds
// instead thrashed its L2).  The grid then holds 8 x ceil(units / 8) x W workgroups.  Without
// an order (very large batches), items are dealt in rounds over all units, the unit order
// rotated by one each round so that every unit visits every XCD.
__device__ __forceinline__ int xcd_item(int per_xcd, int total, int W, int balanced, const int32_t* order,
                                        int upb) {
  if (balanced && order != nullptr) {
    const int U = total / W;
    const int upx = (U + 7) / 8;  // units per XCD
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int j = slot / W, r = slot - j * W;  // unit-major within the XCD
    if (j >= upx) return -1;
    const int rho = 8 * j + ((j & 1) ? 7 - xcd : xcd);  // rank of the unit by decreasing length
    if (rho >= U) return -1;
    const int unit = order[rho / upb] * upb + rho % upb;
    return unit * W + r;
  }
  if (balanced) {
    const int k = blockIdx.x;
    if (k >= total) return -1;
    const int U = total / W;
    const int round = k / U;
    return ((k + round) % U) * W + round;
  }
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int item = xcd * per_xcd + slot;
  return (slot < per_xcd && item < total) ? item : -1;
}

// Query row i (of lenq) sees key row j (of lenk); query i sits at position i + delta.
__device__ __forceinline__ bool key_visible(int i, int j, int lenq, int lenk, int delta, int causal, int window) {
  const int ip = i + delta;
  return (i < lenq) & (j < lenk) & ((!causal) | (j <= ip)) & ((window <= 0) | (j > ip - window));
}

}  // namespace attn
