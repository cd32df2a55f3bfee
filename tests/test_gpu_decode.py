"""GPU parity of the paged decode against the float64 oracle, through the C ABI, plus the
bit-exact page-gather properties: the same logical tokens in different pool pages give the same
bytes, and unassigned pages or slots past the context (filled with NaN) are never read."""
import numpy as np
import pytest
import torch

import oracle
from synth import DECODE_WORKLOADS, bf16_bits_to_f64, bits_to_f64, f32_to_bf16_bits, make_decode_inputs
from tests.gpu_util import O_MAX_ABS, all_finite, dev, host, host_bits, max_abs

pytestmark = pytest.mark.gpu

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402


def run(inp, scale):
    q, kc, vc = dev(inp["q"]), dev(inp["k_cache"]), dev(inp["v_cache"])
    table = torch.from_numpy(inp["block_table"]).to("cuda:0")
    ctx = torch.from_numpy(inp["ctx_lens"]).to("cuda:0")
    o = sdpt.paged_decode(q, kc, vc, table, ctx, scale=scale)
    torch.cuda.synchronize()
    return o


def ref(inp, scale):
    return oracle.paged_decode(bf16_bits_to_f64(inp["q"]), bf16_bits_to_f64(inp["k_cache"]),
                               bf16_bits_to_f64(inp["v_cache"]), inp["block_table"], inp["ctx_lens"], scale)


def test_full_size_decode_matches_oracle():
    w = DECODE_WORKLOADS["decode_d128"]
    inp = make_decode_inputs(w, seed=0)
    print(f"[decode full] B={w.B} pages={inp['num_pages']}", flush=True)
    o = run(inp, w.scale)
    assert all_finite(o)
    assert max_abs(host(o), ref(inp, w.scale)) <= O_MAX_ABS


@pytest.mark.parametrize("ctx", [[1, 15, 16, 17], [255, 256, 257, 4096], [0, 3, 511, 1000]])
def test_ragged_contexts_match_oracle(ctx):
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=len(ctx))
    inp = make_decode_inputs(w, seed=1, ctx_lens=np.array(ctx, dtype=np.int32))
    print(f"[decode ctx {ctx}]", flush=True)
    o = run(inp, w.scale)
    r = ref(inp, w.scale)
    assert all_finite(o)
    assert max_abs(host(o), r) <= O_MAX_ABS
    for b, n in enumerate(ctx):
        if n == 0:
            assert not host_bits(o[b]).any()


def test_page_placement_and_unused_pages_do_not_change_bytes():
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=16)
    inp = make_decode_inputs(w, seed=2)
    pois = make_decode_inputs(w, seed=2, poison_unused=True)
    o1 = host_bits(run(inp, w.scale))
    o2 = host_bits(run(pois, w.scale))
    assert np.array_equal(o1, o2)
    # move every page to another pool slot and rewrite the table accordingly
    perm = np.random.default_rng(3).permutation(inp["num_pages"])
    moved = dict(inp)
    inv = np.argsort(perm)
    moved["k_cache"] = inp["k_cache"][inv]
    moved["v_cache"] = inp["v_cache"][inv]
    t = inp["block_table"]
    moved["block_table"] = np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32)
    o3 = host_bits(run(moved, w.scale))
    assert np.array_equal(o1, o3)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (64, 8)])
def test_other_group_ratios(Hq, Hkv):
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=5, Hq=Hq, Hkv=Hkv, ctx_range=(1, 700))
    inp = make_decode_inputs(w, seed=4)
    o = run(inp, w.scale)
    assert max_abs(host(o), ref(inp, w.scale)) <= O_MAX_ABS


@pytest.mark.parametrize("cap", [1.5, 30.0])
def test_decode_softcap_matches_oracle(cap):
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=6, ctx_range=(1, 1200))
    inp = make_decode_inputs(w, seed=13)
    inp["q"] = f32_to_bf16_bits(3.0 * bf16_bits_to_f64(inp["q"]).astype(np.float32))   # scores of a few units
    print(f"[decode softcap {cap}] ctx {inp['ctx_lens'].tolist()}", flush=True)
    q, kc, vc = dev(inp["q"]), dev(inp["k_cache"]), dev(inp["v_cache"])
    table = torch.from_numpy(inp["block_table"]).to("cuda:0")
    ctx = torch.from_numpy(inp["ctx_lens"]).to("cuda:0")
    o = sdpt.paged_decode(q, kc, vc, table, ctx, scale=w.scale, softcap=cap)
    torch.cuda.synchronize()
    r = oracle.paged_decode(bf16_bits_to_f64(inp["q"]), bf16_bits_to_f64(inp["k_cache"]),
                            bf16_bits_to_f64(inp["v_cache"]), inp["block_table"], inp["ctx_lens"], w.scale,
                            w.page_size, cap)
    assert all_finite(o)
    assert max_abs(host(o), r) <= O_MAX_ABS


def test_one_workspace_serves_calls_of_different_sizes():
    """One workspace sized for the largest call serves smaller and larger calls in any order: each
    result equals the one a fresh workspace gives, bit for bit."""
    import ctypes
    from scaled_dot_product_tiled_amd.binding import AttnDecodeShape
    big = DECODE_WORKLOADS["decode_d128"].scaled(B=12, ctx_range=(1, 2000))
    small = DECODE_WORKLOADS["decode_d128"].scaled(B=5, ctx_range=(600, 1500))
    shape = AttnDecodeShape(big.B, big.Hq, big.Hkv, big.D, big.page_size, 1, big.max_pages_per_seq, 0)
    ws = torch.full((sdpt.load_library().paged_decode_workspace_bytes(ctypes.byref(shape)),), 0x5A,
                    device="cuda:0", dtype=torch.uint8)
    for w, seed in ((big, 3), (small, 4), (big, 5)):
        inp = make_decode_inputs(w, seed=seed)
        q, kc, vc = dev(inp["q"]), dev(inp["k_cache"]), dev(inp["v_cache"])
        table = torch.from_numpy(inp["block_table"]).to("cuda:0")
        ctx = torch.from_numpy(inp["ctx_lens"]).to("cuda:0")
        fresh = sdpt.paged_decode(q, kc, vc, table, ctx, scale=w.scale)
        reused = sdpt.paged_decode(q, kc, vc, table, ctx, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(reused), host_bits(fresh))
        assert max_abs(host(reused), ref(inp, w.scale)) <= O_MAX_ABS


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 2), (24, 6)])
def test_chunks_merged_across_xcds(Hq, Hkv):
    """Long contexts (up to 16 chunks of 512 tokens) with kv-head counts that spread a sequence's
    chunks over different XCDs, merged in chunk order: repeated calls give the same bytes and every
    result is within the oracle's tolerance."""
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=24, Hq=Hq, Hkv=Hkv, ctx_range=(1, 8192))
    inp = make_decode_inputs(w, seed=9)
    print(f"[decode xcd] Hq={Hq} Hkv={Hkv} ctx {inp['ctx_lens'].tolist()}", flush=True)
    first = run(inp, w.scale)
    assert all_finite(first)
    assert max_abs(host(first), ref(inp, w.scale)) <= O_MAX_ABS
    for _ in range(3):
        assert np.array_equal(host_bits(run(inp, w.scale)), host_bits(first))


def _in_order(inp, w):
    """The same logical tokens moved so that every sequence's pages are consecutive in a new pool
    (sequence after sequence, unused pages after them): caches, consecutive table, first pages."""
    table, ctx = inp["block_table"], inp["ctx_lens"]
    order, first = [], np.zeros(w.B, dtype=np.int32)
    t2 = np.full_like(table, -1)
    for b in range(w.B):
        n = -(-int(ctx[b]) // w.page_size)
        first[b] = len(order)
        t2[b, :n] = np.arange(len(order), len(order) + n)
        order += [int(p) for p in table[b, :n]]
    used = set(order)
    rest = [p for p in range(inp["k_cache"].shape[0]) if p not in used]
    perm = np.array(order + rest)
    return dict(inp, k_cache=inp["k_cache"][perm], v_cache=inp["v_cache"][perm], block_table=t2), first


@pytest.mark.parametrize("B,ctx_range,softcap", [(64, (512, 4096), 0.0), (7, (1, 300), 0.0), (9, (0, 700), 15.0)])
def test_contiguous_pages_equal_the_table_path_bit_for_bit(B, ctx_range, softcap):
    """paged_decode_contiguous on consecutive pages gives the bytes paged_decode gives on the same
    logical tokens through a permuted table (and through a consecutive one)."""
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=B, ctx_range=ctx_range)
    inp = make_decode_inputs(w, seed=40)
    cont, first = _in_order(inp, w)
    print(f"[decode contiguous] B={B} ctx={ctx_range} softcap={softcap}", flush=True)
    q = dev(inp["q"])
    ctx = torch.from_numpy(inp["ctx_lens"]).to("cuda:0")
    o_perm = sdpt.paged_decode(q, dev(inp["k_cache"]), dev(inp["v_cache"]),
                               torch.from_numpy(inp["block_table"]).to("cuda:0"), ctx, scale=w.scale, softcap=softcap)
    kc, vc = dev(cont["k_cache"]), dev(cont["v_cache"])
    o_tab = sdpt.paged_decode(q, kc, vc, torch.from_numpy(cont["block_table"]).to("cuda:0"), ctx, scale=w.scale,
                              softcap=softcap)
    o_con = sdpt.paged_decode_contiguous(q, kc, vc, torch.from_numpy(first).to("cuda:0"), ctx,
                                         inp["block_table"].shape[1], scale=w.scale, softcap=softcap)
    torch.cuda.synchronize()
    assert all_finite(o_con)
    assert np.array_equal(host_bits(o_con), host_bits(o_perm))
    assert np.array_equal(host_bits(o_con), host_bits(o_tab))
    if B == 64:
        assert max_abs(host(o_con), ref(inp, w.scale)) <= O_MAX_ABS


# ---------------------------------------------------------------------------
# The two decode strategies: one workgroup per (sequence, kv head) over the whole context when
# the batch gives every compute unit a workgroup (B * Hkv >= 256 and contexts of at most 8192
# tokens), otherwise 512-token chunks and a merge
# ---------------------------------------------------------------------------
def _pad_table(inp, cols):
    """The same inputs with the block table widened to `cols` columns (unused entries -1): the
    table's capacity then passes 8192 tokens and the chunked path runs."""
    t = np.full((inp["block_table"].shape[0], cols), -1, dtype=np.int32)
    t[:, :inp["block_table"].shape[1]] = inp["block_table"]
    return dict(inp, block_table=t)


def test_whole_and_chunked_decode_agree_with_the_oracle():
    w = DECODE_WORKLOADS["decode_d128"]
    ctx = make_decode_inputs(w, seed=41)["ctx_lens"].copy()
    ctx[[3, 40]] = 0                                   # sequences with no context: O = 0
    ctx[7] = 1
    inp = make_decode_inputs(w, seed=41, ctx_lens=ctx)
    wide = _pad_table(inp, 520)
    print("[decode whole vs chunked]", flush=True)
    o_whole, o_chunk = run(inp, w.scale), run(wide, w.scale)
    r = ref(inp, w.scale)
    assert all_finite(o_whole, o_chunk)
    assert max_abs(host(o_whole), r) <= O_MAX_ABS and max_abs(host(o_chunk), r) <= O_MAX_ABS
    for b in (3, 40):
        assert not host_bits(o_whole[b]).any() and not host_bits(o_chunk[b]).any()


@pytest.mark.parametrize("B,Hq,dtype,cap", [(64, 8, "bf16", 0.0), (64, 16, "bf16", 0.0), (64, 64, "f16", 0.0),
                                            (80, 32, "bf16", 0.0), (64, 32, "bf16", 20.0)])
def test_whole_sequence_decode_variants(B, Hq, dtype, cap):
    """The whole-sequence kernel at group sizes 1, 2, 8 and 4, in fp16, with a softcap, and for a
    batch above 64 sequences (dealt in index order instead of by decreasing context).  Unused
    pages and the slots past each context hold NaN, so a read of any of them shows in O."""
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=B, Hq=Hq, ctx_range=(0, 900), dtype=dtype)
    inp = make_decode_inputs(w, seed=42, poison_unused=True)
    print(f"[decode whole] B={B} Hq={Hq} {dtype} cap={cap}", flush=True)
    q, kc, vc = dev(inp["q"], dtype), dev(inp["k_cache"], dtype), dev(inp["v_cache"], dtype)
    o = sdpt.paged_decode(q, kc, vc, torch.from_numpy(inp["block_table"]).to("cuda:0"),
                          torch.from_numpy(inp["ctx_lens"]).to("cuda:0"), scale=w.scale, softcap=cap)
    torch.cuda.synchronize()
    f = lambda x: bits_to_f64(x, dtype)  # noqa: E731
    r = oracle.paged_decode(f(inp["q"]), f(inp["k_cache"]), f(inp["v_cache"]), inp["block_table"], inp["ctx_lens"],
                            w.scale, w.page_size, cap)
    assert all_finite(o)
    assert max_abs(host(o), r) <= O_MAX_ABS
