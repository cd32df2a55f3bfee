"""The C-ABI library without a GPU: it loads, exports every function include/attn.h declares,
sizes workspaces, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

from scaled_dot_product_tiled_amd.binding import (AttnChunkShape, AttnDecodeShape, AttnPagedShape, AttnShape,
                                                  AttnTensor, load_library)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_function_is_exported():
    lib = load_library()
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd", "paged_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    lib = load_library()
    for s in range(5):
        assert lib.attn_status_str(s)
    assert lib.attn_version() == b"0.1.0"
    assert lib.attn_last_hip_error() == 0


def test_workspace_sizes():
    lib = load_library()
    s = AttnShape(2, 4096, 0, 32, 4, 512)
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(s), 0) == 0
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(s), 1) == 256       # 2 x B int32, rounded to 256 bytes
    # backward: delta (one fp32 per (row, head)), then dS in 8 KB blocks of 32 keys x 128 rows:
    # causal keeps key blocks 0 .. 4 qt + 3 of query tile qt (2 nqt (nqt + 1) per head),
    # non-causal all of them, a window a fixed (window + 127) / 32 + 6 per query tile
    delta = 2 * 4096 * 32 * 4
    blk = 32 * 128 * 2
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(s), 0, 1, 0) == delta + 64 * (2 * 32 * 33) * blk
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(s), 0, 0, 0) == delta + 64 * (32 * 128) * blk
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(s), 0, 1, 1024) == delta + 64 * (32 * 41) * blk
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(s), 0, 0, 1024) == 0     # window needs causal
    # packed rows: metadata, one int64 dS offset per sequence, delta, and dS regions sized by each
    # sequence's own length, bounded from the row count: with n_b = ceil(len_b / 128) query tiles,
    # sum n_b <= min(B nqt, total // 128 + B) =: N, and 2 N (nqt + 1) triangular blocks per head
    p = AttnShape(3, 100, 250, 8, 2, 256)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(p), 2, 1, 0) == (256 + 256 + ((250 * 8 * 4 + 255) // 256) * 256
                                                                       + 3 * 8 * 4 * blk)
    # 64 documents of at most 8192 tokens packed into 65536 rows (32 query heads): N = 512 + 64
    # tiles, against 64 x 64 if every document were given the longest one's triangle
    pk = AttnShape(64, 8192, 65536, 32, 4, 512)
    N = 65536 // 128 + 64
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(pk), 2, 1, 0) == (
        256 * 3 + 512 + 65536 * 32 * 4 + 32 * 2 * N * 65 * blk)
    # a padded mask: the lengths are only known on the device, so every row gets the longest
    # triangle; for 64 rows of 8192 that is 139.7 GB, past the cap below
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(pk), 1, 1, 0) == 0
    pm = AttnShape(16, 8192, 0, 32, 4, 512)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(pm), 1, 1, 0) == (
        256 + 16 * 8192 * 32 * 4 + 16 * 32 * 2 * 64 * 65 * blk)
    # past 128 GiB (one dense 65536-token sequence, 32 heads: 137.7 GB of dS) the whole-sequence
    # backward is refused; chunk pairs bound the workspace instead
    long = AttnShape(1, 65536, 0, 32, 4, 512)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(long), 0, 1, 0) == 0
    st = lib.attn_bwd(ctypes.byref(long), _t(), _t(), _t(), _t(), 0x20000, _t(), 0.05, 1, 0, 0.0, None, None,
                      _t(), _t(), _t(), 0x100000, 1 << 40, None)
    assert st == UNSUPPORTED
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(AttnShape(1, 49152, 0, 32, 4, 512)), 0, 1, 0) > 0
    bad = AttnShape(1, 10, 0, 6, 4, 512)      # 6 % 4 != 0
    assert lib.attn_fwd_workspace_bytes(ctypes.byref(bad), 0) == 0
    d = AttnDecodeShape(64, 32, 8, 128, 16, 1000, 256)
    assert lib.paged_decode_workspace_bytes(ctypes.byref(d)) == 64 * 32 * 8 * 130 * 4   # 512-token chunks


def _t(ptr=0x10000, sb=4096 * 32 * 512, ss=32 * 512, sh=512):
    return AttnTensor(ptr, sb, ss, sh)


def _fwd(lib, shape, q=None, scale=0.05, causal=1, window=0, cu=None, pm=None, lse=0x20000, ws=None, wsb=0,
         softcap=0.0):
    q = q or _t()
    return lib.attn_fwd(ctypes.byref(shape) if shape is not None else None, q, _t(), _t(), scale, causal, window,
                        softcap, cu, pm, _t(), lse, ws, wsb, None)


def test_argument_checks_happen_before_any_launch():
    lib = load_library()
    s = AttnShape(2, 64, 0, 8, 2, 512)
    assert _fwd(lib, None) == INVALID
    assert _fwd(lib, s, q=_t(ptr=0)) == INVALID                    # null pointer
    assert _fwd(lib, s, q=_t(ptr=0x10008)) == INVALID              # not 16-byte aligned
    assert _fwd(lib, s, q=_t(ss=100)) == INVALID                   # stride not a multiple of 8
    assert _fwd(lib, s, lse=0) == INVALID
    assert _fwd(lib, s, scale=0.0) == INVALID
    assert _fwd(lib, s, scale=float("nan")) == INVALID
    assert _fwd(lib, s, causal=0, window=16) == UNSUPPORTED       # window requires causal
    assert _fwd(lib, s, window=-1) == INVALID
    assert _fwd(lib, s, softcap=-1.0) == INVALID                   # softcap: 0 (none) or a positive cap
    assert _fwd(lib, s, softcap=float("inf")) == INVALID
    assert _fwd(lib, s, softcap=float("nan")) == INVALID
    assert _fwd(lib, AttnShape(2, 64, 0, 8, 2, 128)) == UNSUPPORTED   # head_dim 128 is decode-only
    assert _fwd(lib, AttnShape(2, 64, 0, 8, 3, 512)) == INVALID       # Hq % Hkv
    assert _fwd(lib, AttnShape(2, 64, 0, 8, 2, 512, 1)) == UNSUPPORTED  # tensors are bf16 or fp16, not fp32
    assert _fwd(lib, AttnShape(0, 64, 0, 8, 2, 512, 2)) == OK            # fp16
    assert _fwd(lib, s, cu=0x30000, pm=0x40000) == INVALID            # both varlen forms
    assert _fwd(lib, s, pm=0x40000) == WORKSPACE                      # varlen needs metadata workspace
    assert _fwd(lib, s, pm=0x40000, ws=0x50010, wsb=4096) == WORKSPACE  # misaligned workspace
    assert _fwd(lib, AttnShape(0, 64, 0, 8, 2, 512)) == OK            # empty batch: nothing to do
    assert lib.attn_last_hip_error() == 0


def test_backward_and_decode_checks():
    lib = load_library()
    s = AttnShape(2, 64, 0, 8, 2, 512)
    st = lib.attn_bwd(ctypes.byref(s), _t(), _t(), _t(), _t(), 0x20000, _t(), 0.05, 1, 0, 0.0, None, None,
                      _t(), _t(), _t(), None, 0, None)
    assert st == WORKSPACE
    st = lib.attn_bwd(ctypes.byref(s), _t(), _t(), _t(), _t(), 0x20000, _t(ptr=0), 0.05, 1, 0, 0.0, None, None,
                      _t(), _t(), _t(), 0x100000, 1 << 24, None)
    assert st == INVALID
    d = AttnDecodeShape(4, 32, 8, 128, 16, 100, 8)
    kc = AttnTensor(0x10000, 16 * 8 * 128, 8 * 128, 128)

    def dec(shape, q=0x1000, table=0x2000, ws=0x100000, wsb=1 << 20, cap=0.0):
        return lib.paged_decode(ctypes.byref(shape), q, 32 * 128, 128, kc, kc, table, 0x3000, 0.1, cap, 0x4000,
                                32 * 128, 128, ws, wsb, None)
    assert dec(AttnDecodeShape(4, 32, 8, 64, 16, 100, 8)) == UNSUPPORTED     # head_dim
    assert dec(AttnDecodeShape(4, 32, 8, 128, 32, 100, 8)) == UNSUPPORTED    # page size
    assert dec(AttnDecodeShape(4, 24, 8, 128, 16, 100, 8)) == UNSUPPORTED    # group ratio 3
    assert dec(d, q=0) == INVALID
    assert dec(d, table=0) == INVALID
    assert dec(d, wsb=16) == WORKSPACE
    assert dec(d, cap=-1.0) == INVALID
    assert dec(AttnDecodeShape(0, 32, 8, 128, 16, 100, 8)) == OK

    # the allocation-free decode: the same checks, and a shape whose chunk partials exceed the
    # library's fixed array is refused before anything is launched
    def dec_na(shape, q=0x1000, table=0x2000):
        return lib.paged_decode_noalloc(ctypes.byref(shape), q, 32 * 128, 128, kc, kc, table, 0x3000, 0.1, 0.0,
                                        0x4000, 32 * 128, 128, None)
    assert lib.paged_decode_noalloc_max_bytes() == 16 << 20
    assert dec_na(AttnDecodeShape(4, 32, 8, 64, 16, 100, 8)) == UNSUPPORTED
    assert dec_na(d, q=0) == INVALID
    assert dec_na(AttnDecodeShape(4, 32, 8, 128, 16, 100, 1 << 16)) == WORKSPACE   # 136 MB of partials
    assert dec_na(AttnDecodeShape(0, 32, 8, 128, 16, 100, 8)) == OK
    assert lib.attn_last_hip_error() == 0


def test_chunk_workspace_sizes():
    """Chunk pairs of a sequence cut into 2048-row chunks (head_dim 512, 32 query heads): the
    diagonal pair keeps the triangular dS layout, a pair wholly in the past keeps every key block,
    a pair wholly in the future stores nothing, and a window keeps (window + 128) / 32 + 6 blocks
    per 128-row query tile.  128 key tiles (4 kv heads x 32) are fewer than the 256 compute
    units, so each tile's 8 query heads are split over 2 workgroups whose fp32 partial dK, dV
    (2 parts x 2 tensors x 2048 x 4 x 512) take space too."""
    lib = load_library()
    c = AttnChunkShape(1, 2048, 2048, 32, 4, 512)
    kvp = 2 * 2 * 2048 * 4 * 512 * 4
    delta = 2048 * 32 * 4 + kvp
    blk = 32 * 128 * 2

    def ws(causal, window, qp, kp, shape=c):
        return lib.attn_bwd_chunk_workspace_bytes(ctypes.byref(shape), causal, window, qp, kp)
    assert ws(1, 0, 2048, 2048) == delta + 32 * (2 * 16 * 17) * blk
    assert ws(1, 0, 4096, 0) == delta + 32 * (16 * 64) * blk
    assert ws(0, 0, 0, 4096) == delta + 32 * (16 * 64) * blk      # non-causal: positions do not matter
    assert ws(1, 0, 0, 2048) == delta                               # every key after every query
    assert ws(1, 1024, 2048, 2048) == delta + 32 * (16 * 41) * blk
    assert ws(1, 1024, 8192, 0) == delta                            # every key beyond the window
    assert ws(1, 0, -1, 0) == 0                                     # positions are >= 0
    assert ws(0, 16, 0, 0) == 0                                     # window needs causal
    assert ws(1, 0, 0, 0, AttnChunkShape(1, 64, 64, 8, 2, 128)) == 0   # head_dim
    assert ws(1, 0, 0, 0, AttnChunkShape(1, 1 << 28, 64, 8, 2, 512)) == 0


def test_chunk_and_merge_checks():
    lib = load_library()
    c = AttnChunkShape(2, 64, 96, 8, 2, 512)

    def fwd(shape=c, causal=1, window=0, qp=0, kp=0, lse=0x20000, q=None, odt=1, cap=0.0):
        return lib.attn_fwd_chunk(ctypes.byref(shape), q or _t(), _t(), _t(), 0.05, causal, window, cap, qp, kp,
                                  _t(), odt, lse, None)
    assert fwd(causal=0, window=8) == UNSUPPORTED
    assert fwd(qp=-5) == INVALID
    assert fwd(lse=0) == INVALID
    assert fwd(q=_t(ptr=0x10008)) == INVALID
    assert fwd(shape=AttnChunkShape(2, 64, 96, 8, 3, 512)) == INVALID
    assert fwd(odt=2) == INVALID                                        # O is fp32 or the inputs' type (bf16)
    assert fwd(odt=3) == INVALID
    assert fwd(cap=-2.0) == INVALID
    assert fwd(shape=AttnChunkShape(0, 64, 96, 8, 2, 512)) == OK       # empty batch
    assert fwd(shape=AttnChunkShape(0, 64, 96, 8, 2, 512), odt=0) == OK
    assert fwd(shape=AttnChunkShape(2, 0, 96, 8, 2, 512)) == OK        # no query rows
    def bwd(gdt=0, ws=None, wsb=0):
        return lib.attn_bwd_chunk(ctypes.byref(c), _t(), _t(), _t(), _t(), 0x20000, _t(), 0.05, 1, 0, 0.0, 64, 0,
                                  _t(), _t(), _t(), gdt, ws, wsb, None)
    assert bwd() == WORKSPACE
    assert bwd(gdt=1) == WORKSPACE
    assert bwd(gdt=3, ws=0x100000, wsb=1 << 30) == INVALID             # parts are bf16 or fp32

    def merge(B=2, S=64, H=8, D=512, lse=0x20000, part=0x30000, o=None, out=None, odt=0):
        return lib.attn_lse_merge(B, S, H, D, o or _t(), lse, _t(), part, out or AttnTensor(None, 0, 0, 0), odt,
                                  None)
    assert merge(D=64) == UNSUPPORTED
    assert merge(H=0) == INVALID
    assert merge(lse=0) == INVALID
    assert merge(part=0x30002) == INVALID                               # fp32 alignment
    assert merge(o=_t(ptr=0)) == INVALID
    assert merge(out=_t(ptr=0x10008)) == INVALID                        # the bf16 output is optional, but aligned
    assert merge(B=0) == OK
    assert merge(B=0, odt=2) == OK
    assert merge(B=0, odt=1) == INVALID                                 # the final output is 16-bit
    assert merge(B=0, out=_t()) == OK

    def fmerge(shape=c, causal=1, window=0, qp=0, kp=0, lse=0x20000, o=None, out=None, cap=0.0, scale=0.05):
        return lib.attn_fwd_chunk_merge(ctypes.byref(shape), _t(), _t(), _t(), scale, causal, window, cap, qp, kp,
                                        o or _t(), lse, out or AttnTensor(None, 0, 0, 0), None)
    assert fmerge(causal=0, window=8) == UNSUPPORTED
    assert fmerge(qp=-5) == INVALID
    assert fmerge(lse=0) == INVALID and fmerge(lse=0x20002) == INVALID
    assert fmerge(o=_t(ptr=0)) == INVALID                               # the running O is required
    assert fmerge(out=_t(ptr=0x10008)) == INVALID                       # the 16-bit copy is optional, but aligned
    assert fmerge(scale=0.0) == INVALID and fmerge(cap=-1.0) == INVALID
    assert fmerge(shape=AttnChunkShape(2, 64, 96, 8, 3, 512)) == INVALID
    assert fmerge(shape=AttnChunkShape(0, 64, 96, 8, 2, 512)) == OK    # empty batch: no launch
    assert fmerge(shape=AttnChunkShape(2, 0, 96, 8, 2, 512), out=_t()) == OK
    assert lib.attn_last_hip_error() == 0


def test_paged_cache_call_checks():
    lib = load_library()
    d = AttnDecodeShape(4, 32, 8, 128, 16, 100, 8)
    kc = AttnTensor(0x10000, 16 * 8 * 128, 8 * 128, 128)
    tok = AttnTensor(0x20000, 8 * 128, 8 * 128, 128)

    def app(shape=d, n=1, table=0x3000, ctx=0x4000, k=None):
        return lib.paged_kv_append(ctypes.byref(shape), n, k or tok, tok, kc, kc, table, ctx, None)

    def gat(shape=d, n=8, table=0x3000, ctx=0x4000):
        return lib.paged_kv_gather(ctypes.byref(shape), n, kc, kc, table, ctx, tok, tok, None)
    assert app(n=-1) == INVALID
    assert app(table=0) == INVALID and gat(ctx=0) == INVALID
    assert app(k=AttnTensor(0x20008, 1024, 1024, 128)) == INVALID                  # misaligned
    assert app(AttnDecodeShape(4, 32, 8, 64, 16, 100, 8)) == UNSUPPORTED           # head_dim
    assert gat(AttnDecodeShape(4, 32, 8, 128, 16, 100, 8, 1)) == UNSUPPORTED       # fp32 cache
    assert app(n=0) == OK and gat(AttnDecodeShape(0, 32, 8, 512, 16, 100, 8)) == OK  # nothing to move
    assert lib.attn_last_hip_error() == 0


def test_paged_prefill_checks():
    """attn_fwd_paged takes no workspace; bad arguments are refused before any launch."""
    lib = load_library()
    sh = AttnPagedShape(32, 1024, 1055, 32, 4, 512, 0, 16, 7000, 256)
    q = AttnTensor(0x10000, 0, 32 * 512, 512)
    kc = AttnTensor(0x20000, 16 * 4 * 512, 4 * 512, 512)

    def call(shape=sh, q=q, k=kc, table=0x3000, cu=0x3100, ctx=0x3200, scale=0.05, window=0, softcap=0.0,
             lse=0x5000):
        return lib.attn_fwd_paged(ctypes.byref(shape), q, k, k, table, cu, ctx, scale, window, softcap, q, lse, None)
    assert call(table=0) == INVALID and call(cu=0) == INVALID and call(ctx=0) == INVALID
    assert call(scale=0.0) == INVALID and call(window=-1) == INVALID and call(softcap=-1.0) == INVALID
    assert call(lse=0x5002) == INVALID                                   # misaligned lse
    assert call(q=AttnTensor(0x10008, 0, 32 * 512, 512)) == INVALID      # misaligned rows
    for bad, st in ((AttnPagedShape(2, 8, 16, 32, 4, 128, 0, 16, 10, 4), UNSUPPORTED),   # head_dim
                    (AttnPagedShape(2, 8, 16, 32, 4, 512, 0, 32, 10, 4), UNSUPPORTED),   # page size
                    (AttnPagedShape(2, 8, 16, 32, 4, 512, 1, 16, 10, 4), UNSUPPORTED),   # fp32
                    (AttnPagedShape(2, 8, 16, 30, 4, 512, 0, 16, 10, 4), INVALID),       # Hq % Hkv
                    (AttnPagedShape(2, 8, 16, 32, 4, 512, 0, 16, 0, 4), INVALID)):       # empty pool
        assert call(shape=bad) == st
    assert call(k=AttnTensor(0x20000, 1 << 31, 1 << 27, 512)) == UNSUPPORTED   # slot stride past 2^26
    assert call(shape=AttnPagedShape(0, 0, 0, 32, 4, 512, 0, 16, 1, 1)) == OK   # nothing to do
    assert lib.attn_last_hip_error() == 0


def test_paged_prefill_split_workspace():
    """attn_fwd_paged_split: fp32 O and LSE for 16 pieces per (sequence, query head) and one int32
    per sequence, rounded up to 256 bytes; a missing, small or misaligned workspace is refused before any launch, and so are
    the arguments attn_fwd_paged refuses."""
    lib = load_library()
    sh = AttnPagedShape(32, 1024, 1055, 32, 4, 512, 0, 16, 7000, 256)
    need = lib.attn_fwd_paged_workspace_bytes(ctypes.byref(sh))
    assert need == -(-(32 * 32 * 16 * 513 * 4 + 4 * 32) // 256) * 256   # pieces, then the deal's sequence order
    assert lib.attn_fwd_paged_workspace_bytes(ctypes.byref(AttnPagedShape(2, 8, 16, 32, 4, 128, 0, 16, 10, 4))) == 0
    q = AttnTensor(0x10000, 0, 32 * 512, 512)
    kc = AttnTensor(0x20000, 16 * 4 * 512, 4 * 512, 512)

    def call(ws=0x100000, nbytes=need, scale=0.05, shape=sh):
        return lib.attn_fwd_paged_split(ctypes.byref(shape), q, kc, kc, 0x3000, 0x3100, 0x3200, scale, 0, 0.0, q,
                                        0x5000, ws, nbytes, None)
    assert call(ws=0) == WORKSPACE and call(nbytes=need - 1) == WORKSPACE and call(ws=0x100010) == WORKSPACE
    assert call(scale=0.0) == INVALID
    assert call(shape=AttnPagedShape(2, 8, 16, 30, 4, 512, 0, 16, 10, 4)) == INVALID
    assert lib.attn_last_hip_error() == 0


def test_decode_graph_checks():
    """paged_decode_graphs_create refuses bad buckets, a NULL stream and a small workspace before
    any capture; launch refuses a missing graph set."""
    lib = load_library()
    d = AttnDecodeShape(8, 32, 8, 128, 16, 100, 8)
    kc = AttnTensor(0x10000, 16 * 8 * 128, 8 * 128, 128)
    none = AttnTensor(None, 0, 0, 0)
    need = lib.paged_decode_workspace_bytes(ctypes.byref(d))

    def create(buckets=(1, 2, 4, 8), stream=0x1234, ws=0x40000, nbytes=need, out=True):
        arr = (ctypes.c_int32 * len(buckets))(*buckets)
        h = ctypes.c_void_p()
        return lib.paged_decode_graphs_create(ctypes.byref(d), arr, len(buckets), 0x20000, 32 * 128, 128, none, none,
                                              kc, kc, 0x3000, 0x4000, 0.1, 0.0, 0x50000, 32 * 128, 128, ws, nbytes,
                                              stream, ctypes.byref(h) if out else None)
    assert create(out=False) == INVALID
    assert create(buckets=(2, 1)) == INVALID and create(buckets=(0, 4)) == INVALID and create(buckets=(4, 9)) == INVALID
    assert create(stream=0) == INVALID
    assert create(ws=0) == WORKSPACE and create(nbytes=need - 1) == WORKSPACE
    b = ctypes.c_int32(-1)
    assert lib.paged_decode_graphs_launch(None, 1, None, ctypes.byref(b)) == INVALID
    lib.paged_decode_graphs_destroy(None)
    assert lib.attn_last_hip_error() == 0


def test_debug_mode_switch():
    """attn_debug sets the process-wide metadata-check mode and returns the previous one (no GPU
    call is made by the switch itself)."""
    lib = load_library()
    first = lib.attn_debug(1)
    assert first in (0, 1)
    assert lib.attn_debug(0) == 1
    assert lib.attn_debug(0) == 0
    lib.attn_debug(first)
