"""Seeded synthetic inputs for fused causal grouped-query attention and paged decode.

This module is shared by the tests, the smoke check and the benchmark, and by
both sides of every parity comparison.  It holds no attention arithmetic: only
random draws, their rounding to bfloat16, sequence lengths, padding masks and
page tables.  Every random stream is derived from
``numpy.random.SeedSequence([seed, workload_id, stream_id])`` so that a stream
does not change when another one is added.

The workloads mirror the shapes the pages run (Gemma4 head_dim=512
full-attention layers and head_dim=256 sliding-window layers in "Gemma4 FFPA
attention backend support for accelerating Gemma4-family training", section
Results; the batch-64 paged-KV decode rollout in "flex_attention + paged KV +
CUDA graphs vs vLLM", section Batch-size sweep) with random values in place of
the pages' datasets and trained weights, which are not used.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "AttnWorkload", "DecodeWorkload", "ATTN_WORKLOADS", "DECODE_WORKLOADS",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "bf16_bits_to_f64", "f32_to_f16_bits", "f16_bits_to_f64",
    "bits_to_f64", "NAN_BITS", "stream", "normal_bf16", "normal_16", "make_attention_inputs", "make_decode_inputs",
    "lengths_to_pad_mask", "lengths_to_cu_seqlens", "pack_rows", "draw_lengths", "STREAM",
    "PrefillWorkload", "PREFILL_WORKLOADS", "make_prefill_inputs",
]

# Stream ids inside one workload.
STREAM = {"q": 0, "k": 1, "v": 2, "do": 3, "lengths": 4, "pages": 5, "fill": 6, "new": 7}


# ----------------------------------------------------------------------------
# bfloat16 bit handling (round to nearest, ties to even)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    NaN stays a quiet NaN with its sign; values past the largest bfloat16 round to +-inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)).astype(np.uint16) & np.uint16(0x8000)) | np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


# ----------------------------------------------------------------------------
# IEEE half bit handling (numpy's float32 -> float16 conversion rounds to nearest, ties to even)
# ----------------------------------------------------------------------------
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half (nearest, ties to even); returns uint16 bit patterns."""
    with np.errstate(over="ignore"):  # past the largest half: +-inf, as rounding defines
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of IEEE half bit patterns to float64."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def bits_to_f64(b: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Exact widening of 16-bit patterns of the given type ("bf16" or "f16") to float64."""
    return f16_bits_to_f64(b) if dtype == "f16" else bf16_bits_to_f64(b)


# quiet NaN bit pattern of each 16-bit type
NAN_BITS = {"bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}


def stream(seed: int, workload_id: int, stream_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, workload_id, stream_id]))


def normal_16(rng: np.random.Generator, shape, std: float = 1.0, dtype: str = "bf16",
              chunk: int = 1 << 26) -> np.ndarray:
    """N(0, std^2) draws in float32, rounded to 16-bit patterns ("bf16" or "f16"), drawn in
    bounded chunks."""
    conv = f32_to_f16_bits if dtype == "f16" else f32_to_bf16_bits
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = conv(x)
    return out.reshape(shape)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0, chunk: int = 1 << 26) -> np.ndarray:
    """N(0, std^2) draws in float32, rounded to bfloat16 bit patterns, drawn in bounded chunks."""
    return normal_16(rng, shape, std, "bf16", chunk)


# ----------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class AttnWorkload:
    """One fused-attention forward+backward workload (layout B, S, H, D, bfloat16)."""
    wid: int
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    causal: bool = True
    window: int = 0              # 0: none; W > 0: key j visible from query i iff i - W < j <= i
    qk_std: float = 1.0          # std of the Q and K draws
    vdo_std: float = 1.0         # std of the V and dO draws
    varlen: Optional[str] = None  # None, "pad_mask" (right padded to S) or "cu_seqlens" (packed rows)
    len_range: Optional[tuple] = None  # inclusive uniform range of valid lengths
    dtype: str = "bf16"          # 16-bit element type of every tensor: "bf16" or "f16"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def r(self) -> int:
        return self.Hq // self.Hkv

    def scaled(self, **kw) -> "AttnWorkload":
        """A copy with some fields replaced (used for reduced-size parity cases)."""
        d = dict(self.__dict__)
        d.update(kw)
        return AttnWorkload(**d)


@dataclass(frozen=True)
class DecodeWorkload:
    """Single-token decode against a paged KV cache (bfloat16)."""
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    page_size: int = 16
    ctx_range: tuple = (512, 4096)   # inclusive uniform range of context lengths
    pool_factor: float = 1.5         # page pool = ceil(pool_factor * pages actually used)
    dtype: str = "bf16"              # 16-bit element type of q, caches and o: "bf16" or "f16"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.ctx_range[1] // self.page_size)

    def scaled(self, **kw) -> "DecodeWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return DecodeWorkload(**d)


ATTN_WORKLOADS = {
    "tiny_d512": AttnWorkload(1, "tiny causal GQA d512 (B1 S128 Hq2 Hkv1)", 1, 128, 2, 1, 512),
    "full_d512": AttnWorkload(2, "causal GQA d512 full attention (B2 S4096 Hq32 Hkv4)", 2, 4096, 32, 4, 512),
    "window_d256": AttnWorkload(3, "causal sliding window 1024 d256 (B2 S4096 Hq32 Hkv16)", 2, 4096, 32, 16, 256,
                                window=1024, qk_std=3.0),
    "varlen_d512": AttnWorkload(4, "padded varlen causal GQA d512 (B8 Smax8192 Hq32 Hkv4)", 8, 8192, 32, 4, 512,
                                varlen="pad_mask", len_range=(512, 8192)),
}

DECODE_WORKLOADS = {
    "decode_d128": DecodeWorkload(5, "paged decode d128 (B64 Hq32 Hkv8, 16-token pages)", 64, 32, 8, 128),
}


@dataclass(frozen=True)
class PrefillWorkload:
    """New query tokens of several sequences against their paged KV caches in one call: each
    sequence holds ctx tokens (its new ones included) and has n of them new; n = 1 is a decode
    row, n = ctx a whole prompt, anything between a prompt chunk after a cached prefix."""
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    ctx: tuple                       # per sequence: tokens in the cache after the step
    new: tuple                       # per sequence: how many of them are new query rows
    page_size: int = 16
    pool_factor: float = 1.5
    dtype: str = "bf16"
    window: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def scaled(self, **kw) -> "PrefillWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return PrefillWorkload(**d)


PREFILL_WORKLOADS = {
    # a 2048-token prompt chunk after 6144 cached tokens at the full-attention layer's shape
    "paged_prefill_d512": PrefillWorkload(6, "paged prefill d512: 2048 new tokens after 6144 cached "
                                             "(Hq32 Hkv4, 16-token pages)", 1, 32, 4, 512, (8192,), (2048,)),
    # a serving step mixing one prompt chunk with 31 decode rows of 512..4096-token contexts
    "mixed_step_d512": PrefillWorkload(7, "mixed step d512: a 1024-token chunk after 3072 cached plus 31 decode "
                                          "rows (Hq32 Hkv4, 16-token pages)", 32, 32, 4, 512,
                                       (4096,) + tuple(512 + (3584 * i) // 30 for i in range(31)),
                                       (1024,) + (1,) * 31),
}


def make_prefill_inputs(w: PrefillWorkload, seed: int = 0, poison_unused: bool = False) -> dict:
    """Seeded paged prefill inputs: the caches and block table of make_decode_inputs for the
    contexts w.ctx (pages permuted over the pool), plus the packed new query rows q (T, Hq, D)
    with their offsets cu_q (B+1) and max_q."""
    dw = DecodeWorkload(w.wid, w.name, w.B, w.Hq, w.Hkv, w.D, w.page_size,
                        (min(w.ctx), max(w.ctx)), w.pool_factor, w.dtype)
    out = make_decode_inputs(dw, seed, poison_unused, ctx_lens=np.asarray(w.ctx, dtype=np.int32))
    n = np.asarray(w.new, dtype=np.int64)
    cu = lengths_to_cu_seqlens(n)
    out["q"] = normal_16(stream(seed, w.wid, STREAM["new"]), (int(cu[-1]), w.Hq, w.D), 1.0, w.dtype)
    out["cu_q"] = cu
    out["max_q"] = int(n.max()) if len(n) else 0
    return out


# ----------------------------------------------------------------------------
# Varlen helpers
# ----------------------------------------------------------------------------
def lengths_to_pad_mask(lengths: np.ndarray, S: int) -> np.ndarray:
    """(B,) lengths -> (B, S) uint8 right-padded validity mask."""
    lengths = np.asarray(lengths)
    return (np.arange(S)[None, :] < lengths[:, None]).astype(np.uint8)


def lengths_to_cu_seqlens(lengths: np.ndarray) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


def pack_rows(x: np.ndarray, lengths: np.ndarray) -> np.ndarray:
    """(B, S, ...) padded rows -> (sum(lengths), ...) packed rows."""
    return np.concatenate([x[b, :int(n)] for b, n in enumerate(lengths)], axis=0)


def draw_lengths(w, seed):
    """The workload's seeded sequence lengths (the ones make_attention_inputs uses), or None."""
    if w.len_range is None:
        return None
    lo, hi = w.len_range
    return stream(seed, w.wid, STREAM["lengths"]).integers(lo, hi + 1, size=w.B).astype(np.int32)


def make_attention_inputs(w: AttnWorkload, seed: int = 0, poison_padding: bool = False) -> dict:
    """Seeded 16-bit Q, K, V, dO (uint16 bit patterns of w.dtype, shape (B, S, H, D)) plus varlen
    metadata.

    Padding positions hold ordinary draws; with ``poison_padding`` they hold NaN, which a correct
    varlen path must never let reach a valid output.
    """
    q = normal_16(stream(seed, w.wid, STREAM["q"]), (w.B, w.S, w.Hq, w.D), w.qk_std, w.dtype)
    k = normal_16(stream(seed, w.wid, STREAM["k"]), (w.B, w.S, w.Hkv, w.D), w.qk_std, w.dtype)
    v = normal_16(stream(seed, w.wid, STREAM["v"]), (w.B, w.S, w.Hkv, w.D), w.vdo_std, w.dtype)
    do = normal_16(stream(seed, w.wid, STREAM["do"]), (w.B, w.S, w.Hq, w.D), w.vdo_std, w.dtype)
    lengths = draw_lengths(w, seed)
    out = {"q": q, "k": k, "v": v, "do": do, "lengths": lengths}
    if lengths is not None:
        out["pad_mask"] = lengths_to_pad_mask(lengths, w.S)
        out["cu_seqlens"] = lengths_to_cu_seqlens(lengths)
        if poison_padding:
            nan = NAN_BITS[w.dtype]
            for b, n in enumerate(lengths):
                for t in (q, k, v, do):
                    t[b, n:] = nan
    return out


def make_decode_inputs(w: DecodeWorkload, seed: int = 0, poison_unused: bool = False,
                       ctx_lens: Optional[np.ndarray] = None) -> dict:
    """Seeded paged-KV decode inputs.

    Pages per sequence = ceil(ctx / page_size); the pool holds ceil(pool_factor * total pages)
    pages and the block table assigns a random permutation of pool ids in sequence order.
    Unused table entries are -1.  Unassigned pages and the tail slots past each context hold
    ordinary draws, or NaN with ``poison_unused``.
    """
    if ctx_lens is None:
        lo, hi = w.ctx_range
        ctx_lens = stream(seed, w.wid, STREAM["lengths"]).integers(lo, hi + 1, size=w.B).astype(np.int32)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    ps = w.page_size
    pages = -(-ctx_lens.astype(np.int64) // ps)
    total = int(pages.sum())
    pool = max(1, int(np.ceil(w.pool_factor * total)))
    perm = stream(seed, w.wid, STREAM["pages"]).permutation(pool).astype(np.int32)
    maxp = max(w.max_pages_per_seq, int(pages.max()) if len(pages) else 0)
    table = np.full((w.B, maxp), -1, dtype=np.int32)
    off = 0
    for b in range(w.B):
        n = int(pages[b])
        table[b, :n] = perm[off:off + n]
        off += n
    q = normal_16(stream(seed, w.wid, STREAM["q"]), (w.B, w.Hq, w.D), 1.0, w.dtype)
    kc = normal_16(stream(seed, w.wid, STREAM["k"]), (pool, ps, w.Hkv, w.D), 1.0, w.dtype)
    vc = normal_16(stream(seed, w.wid, STREAM["v"]), (pool, ps, w.Hkv, w.D), 1.0, w.dtype)
    if poison_unused:
        nan = NAN_BITS[w.dtype]
        used = np.zeros(pool, dtype=bool)
        for b in range(w.B):
            n = int(pages[b])
            used[table[b, :n]] = True
            tail = int(ctx_lens[b]) - (n - 1) * ps
            if n > 0 and tail < ps:
                kc[table[b, n - 1], tail:] = nan
                vc[table[b, n - 1], tail:] = nan
        kc[~used] = nan
        vc[~used] = nan
    return {"q": q, "k_cache": kc, "v_cache": vc, "block_table": table, "ctx_lens": ctx_lens,
            "num_pages": pool, "page_size": ps}
