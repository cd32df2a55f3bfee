"""GPU checks of the paged cache calls (paged_kv_append, paged_kv_gather) through the C ABI,
a decode step captured in a HIP graph and replayed, a paged prefill (gather + chunk-pair
forward) against the float64 oracle, and the in-kernel paged forward attn_fwd_paged (prompt
chunks, whole prompts and decode rows in one call) against the oracle and, bit for bit,
against the gather + chunk-pair path.

Append and gather move bits, so they are compared bit for bit with the oracle's scatter and
gather.  The graph replays are compared bit for bit with the same calls made eagerly (same
kernels, same inputs) and with the oracle within the usual tolerance.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import (DECODE_WORKLOADS, PREFILL_WORKLOADS, bits_to_f64, make_decode_inputs, make_prefill_inputs,
                   normal_16, stream)
from tests.gpu_util import LSE_MAX_ABS, O_MAX_ABS, all_finite, dev, host, host_bits, max_abs

pytestmark = pytest.mark.gpu

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _with_room(inp, w, n):
    """The decode inputs with every table row extended so that n more tokens fit (fresh pool
    pages appended at the end of the caches)."""
    ctx0 = inp["ctx_lens"].astype(np.int64)
    ctx1 = ctx0 + n
    table = np.concatenate([inp["block_table"], np.full((w.B, -(-n // w.page_size) + 1), -1, np.int32)], axis=1)
    kc, vc = inp["k_cache"], inp["v_cache"]
    pool = kc.shape[0]
    extra = 0
    for b in range(w.B):
        for p in range(int(-(-ctx1[b] // w.page_size))):
            if table[b, p] < 0:
                table[b, p] = pool + extra
                extra += 1
    fill = normal_16(stream(9, w.wid, 7), (extra,) + kc.shape[1:], 1.0, w.dtype)
    kc = np.concatenate([kc, fill])
    vc = np.concatenate([vc, fill[::-1].copy()])
    return table, kc, vc, ctx1.astype(np.int32)


@pytest.mark.parametrize("n,dtype,D", [(1, "bf16", 128), (5, "bf16", 128), (3, "f16", 256), (20, "bf16", 512)])
def test_append_and_gather_move_exact_bits(n, dtype, D):
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=6, Hkv=2, D=D, ctx_range=(0, 70), dtype=dtype)
    inp = make_decode_inputs(w, seed=3)
    table, kc, vc, ctx1 = _with_room(inp, w, n)
    table[1, :] = -1                                   # a sequence without pages: skipped / zeros
    table[2, 0] = kc.shape[0] + 5                      # out-of-range page id: skipped / zeros
    new_k = normal_16(stream(4, w.wid, 0), (w.B, n, w.Hkv, w.D), 1.0, dtype)
    new_v = normal_16(stream(4, w.wid, 1), (w.B, n, w.Hkv, w.D), 1.0, dtype)
    say(f"[paged append] n={n} dtype={dtype} D={D} ctx={ctx1.tolist()}")
    k_d, v_d = dev(kc, dtype), dev(vc, dtype)
    t_d = torch.from_numpy(table).to("cuda:0")
    c_d = torch.from_numpy(ctx1).to("cuda:0")
    sdpt.paged_kv_append(dev(new_k, dtype), dev(new_v, dtype), k_d, v_d, t_d, c_d)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(k_d), oracle.paged_append(kc, table, ctx1, new_k, w.page_size))
    assert np.array_equal(host_bits(v_d), oracle.paged_append(vc, table, ctx1, new_v, w.page_size))
    # gather the first m tokens back: cached tokens where the page exists, zeros elsewhere
    m = int(ctx1.max()) + 3
    gk, gv = sdpt.paged_kv_gather(k_d, v_d, t_d, c_d, m)
    torch.cuda.synchronize()
    kk, vv = host_bits(k_d), host_bits(v_d)
    gkb, gvb = host_bits(gk), host_bits(gv)
    for b in range(w.B):
        for t in range(m):
            page = table[b, t // w.page_size] if t < ctx1[b] else -1
            ok = 0 <= page < kk.shape[0]
            ek = kk[page, t % w.page_size] if ok else 0
            ev = vv[page, t % w.page_size] if ok else 0
            assert np.array_equal(gkb[b, t], np.broadcast_to(ek, (w.Hkv, w.D))), (b, t)
            assert np.array_equal(gvb[b, t], np.broadcast_to(ev, (w.Hkv, w.D))), (b, t)


def test_decode_step_captured_in_a_graph_replays_like_eager_calls():
    """One decode step = append the current token's K/V, then paged_decode; captured once in a
    HIP graph (no allocation, no memset inside) and replayed for three steps with new inputs
    copied into the captured buffers; every replay equals the eager calls bit for bit and the
    oracle within tolerance."""
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=8, ctx_range=(40, 300))
    inp = make_decode_inputs(w, seed=8)
    steps = 3
    table, kc, vc, _ = _with_room(inp, w, steps)
    ctx0 = inp["ctx_lens"].astype(np.int32)
    k_d, v_d = dev(kc), dev(vc)
    k_eager, v_eager = k_d.clone(), v_d.clone()
    t_d = torch.from_numpy(table).to("cuda:0")
    q_s = torch.empty((w.B, w.Hq, w.D), device="cuda:0", dtype=torch.bfloat16)
    kn_s = torch.empty((w.B, 1, w.Hkv, w.D), device="cuda:0", dtype=torch.bfloat16)
    vn_s = torch.empty_like(kn_s)
    ctx_s = torch.empty(w.B, device="cuda:0", dtype=torch.int32)
    out_s = torch.empty_like(q_s)
    ws = torch.empty(max(1 << 20, 4 * w.B * w.Hq * 64 * (w.D + 2)), device="cuda:0", dtype=torch.uint8)

    def step(kcache, vcache, out):
        sdpt.paged_kv_append(kn_s, vn_s, kcache, vcache, t_d, ctx_s)
        sdpt.paged_decode(q_s, kcache, vcache, t_d, ctx_s, scale=w.scale, out=out, workspace=ws)

    def load(i):
        q_s.copy_(dev(normal_16(stream(20 + i, w.wid, 0), (w.B, w.Hq, w.D))))
        kn_s.copy_(dev(normal_16(stream(20 + i, w.wid, 1), (w.B, 1, w.Hkv, w.D))))
        vn_s.copy_(dev(normal_16(stream(20 + i, w.wid, 2), (w.B, 1, w.Hkv, w.D))))
        ctx_s.copy_(torch.from_numpy(ctx0 + i + 1).to("cuda:0"))

    load(0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):             # warm-up outside the graph (first launches load code)
        step(k_d.clone(), v_d.clone(), torch.empty_like(q_s))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(k_d, v_d, out_s)
    torch.cuda.synchronize()
    # the capture ran nothing: restore the caches and replay step by step
    k_d.copy_(dev(kc))
    v_d.copy_(dev(vc))
    kc_ref, vc_ref = bits_to_f64(kc, "bf16"), bits_to_f64(vc, "bf16")
    for i in range(steps):
        say(f"[graph decode] replay {i}")
        load(i)
        g.replay()
        torch.cuda.synchronize()
        got = out_s.clone()
        eager = torch.empty_like(q_s)
        step(k_eager, v_eager, eager)      # the same step made with eager calls on other caches
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(got), host_bits(eager)), i
        assert np.array_equal(host_bits(k_d), host_bits(k_eager)) and np.array_equal(host_bits(v_d),
                                                                                     host_bits(v_eager))
        ctx = ctx0 + i + 1
        kc_ref = oracle.paged_append(kc_ref, table, ctx, host(kn_s), w.page_size)
        vc_ref = oracle.paged_append(vc_ref, table, ctx, host(vn_s), w.page_size)
        ref = oracle.paged_decode(host(q_s), kc_ref, vc_ref, table, ctx, w.scale, w.page_size)
        assert all_finite(got)
        assert max_abs(host(got), ref) <= O_MAX_ABS, i


@pytest.mark.parametrize("D,prev,n", [(256, 300, 77), (512, 0, 130), (512, 513, 64)])
def test_paged_prefill_matches_oracle(D, prev, n):
    """A chunk of n new query tokens after prev cached ones: append the chunk's K/V to the pages,
    gather the prev + n tokens, run attn_fwd_chunk at q_pos0 = prev against them; rows equal the
    last n rows of causal attention over the whole sequence."""
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=1, Hq=8, Hkv=2, D=D, ctx_range=(max(prev, 1), max(prev, 1)))
    inp = make_decode_inputs(w, seed=10, ctx_lens=np.array([prev], dtype=np.int32))
    table, kc, vc, ctx1 = _with_room(inp, w, n)
    q_new = normal_16(stream(11, w.wid, 0), (1, n, w.Hq, D))
    new_k = normal_16(stream(11, w.wid, 1), (1, n, w.Hkv, D))
    new_v = normal_16(stream(11, w.wid, 2), (1, n, w.Hkv, D))
    say(f"[paged prefill] D={D} prev={prev} n={n}")
    k_d, v_d = dev(kc), dev(vc)
    t_d = torch.from_numpy(table).to("cuda:0")
    c_d = torch.from_numpy(ctx1).to("cuda:0")
    sdpt.paged_kv_append(dev(new_k), dev(new_v), k_d, v_d, t_d, c_d)
    L = prev + n
    kg, vg = sdpt.paged_kv_gather(k_d, v_d, t_d, c_d, L)
    o, lse = sdpt.attn_fwd_chunk(dev(q_new), kg, vg, prev, 0, scale=1.0 / np.sqrt(D), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert all_finite(o, lse)
    kf = np.concatenate([oracle.gather_pages(bits_to_f64(kc), table[0], prev, w.page_size),
                         bits_to_f64(new_k)[0]])[None]
    vf = np.concatenate([oracle.gather_pages(bits_to_f64(vc), table[0], prev, w.page_size),
                         bits_to_f64(new_v)[0]])[None]
    qf = np.zeros((1, L, w.Hq, D))
    qf[0, prev:] = bits_to_f64(q_new)[0]
    ro, rl = oracle.attention_forward(qf, kf, vf, 1.0 / np.sqrt(D), True, 0)
    assert max_abs(host(o), ro[:, prev:]) <= O_MAX_ABS
    assert max_abs(host(lse), rl[:, :, prev:]) <= LSE_MAX_ABS


# ---------------------------------------------------------------------------
# attn_fwd_paged: K/V read through the block table inside the forward kernel
# ---------------------------------------------------------------------------
def _prefill_dev(inp, dtype):
    return dict(q=dev(inp["q"], dtype), kc=dev(inp["k_cache"], dtype), vc=dev(inp["v_cache"], dtype),
                table=torch.from_numpy(inp["block_table"]).to("cuda:0"),
                cu=torch.from_numpy(inp["cu_q"].astype(np.int32)).to("cuda:0"),
                ctx=torch.from_numpy(inp["ctx_lens"]).to("cuda:0"))


def _prefill_oracle(inp, w, softcap=0.0):
    f = lambda x: bits_to_f64(x, w.dtype)  # noqa: E731
    return oracle.paged_prefill(f(inp["q"]), f(inp["k_cache"]), f(inp["v_cache"]), inp["block_table"], inp["cu_q"],
                                inp["ctx_lens"], w.scale, w.window, w.page_size, softcap)


MIXED = PREFILL_WORKLOADS["mixed_step_d512"]
# (D, dtype, window, softcap, contexts, new rows): a prompt chunk after a cached prefix, whole
# prompts, decode rows (n = 1) with one-token, page-edge and long contexts, a sequence with no
# new row, and rows before position 0 (more new rows than cached tokens)
PREFILL_CASES = [
    (512, "bf16", 0, 0.0, (300, 1, 17, 130, 520, 40, 64), (77, 1, 1, 130, 1, 40, 0)),
    (256, "bf16", 100, 0.0, (700, 33, 1, 260), (190, 1, 1, 260)),
    (512, "f16", 0, 0.0, (96, 2, 400), (96, 1, 33)),
    (256, "bf16", 0, 20.0, (129, 64, 3), (129, 1, 3)),
    (512, "bf16", 0, 0.0, (3, 10, 0), (40, 40, 5)),
]


@pytest.mark.parametrize("D,dtype,window,softcap,ctx,new", PREFILL_CASES)
def test_fwd_paged_matches_oracle(D, dtype, window, softcap, ctx, new):
    w = MIXED.scaled(B=len(ctx), Hq=8, Hkv=2, D=D, dtype=dtype, window=window, ctx=ctx, new=new,
                     name=f"paged fwd d{D}")
    inp = make_prefill_inputs(w, seed=31)
    say(f"[fwd paged] D={D} dtype={dtype} window={window} softcap={softcap} ctx={ctx} new={new}")
    d = _prefill_dev(inp, dtype)
    o, lse = sdpt.attn_fwd_paged(d["q"], d["kc"], d["vc"], d["table"], d["cu"], d["ctx"], inp["max_q"],
                                 scale=w.scale, window=window, softcap=softcap)
    torch.cuda.synchronize()
    assert all_finite(o, lse)
    ro, rl = _prefill_oracle(inp, w, softcap)
    assert max_abs(host(o), ro) <= O_MAX_ABS
    assert max_abs(host(lse), rl) <= LSE_MAX_ABS
    # rows before position 0 and sequences without keys: exact zeros
    cu, c = inp["cu_q"], inp["ctx_lens"]
    for b in range(w.B):
        neg = min(max(int(new[b]) - int(c[b]), 0), int(new[b])) if c[b] > 0 else int(new[b])
        if neg:
            assert not host(o)[cu[b]:cu[b] + neg].any() and not host(lse)[:, cu[b]:cu[b] + neg].any()


@pytest.mark.parametrize("D,dtype,window", [(512, "bf16", 0), (256, "f16", 48)])
def test_fwd_paged_equals_gather_then_chunk_bit_for_bit(D, dtype, window):
    """The same kernel arithmetic reads the keys through the table instead of a gathered copy:
    per sequence, O and LSE equal paged_kv_gather + attn_fwd_chunk at q_pos0 = ctx - n exactly."""
    ctx, new = (600, 1, 250, 45), (200, 1, 250, 1)
    w = MIXED.scaled(B=len(ctx), Hq=8, Hkv=2, D=D, dtype=dtype, window=window, ctx=ctx, new=new)
    inp = make_prefill_inputs(w, seed=32)
    say(f"[fwd paged vs gather] D={D} dtype={dtype} window={window}")
    d = _prefill_dev(inp, dtype)
    o, lse = sdpt.attn_fwd_paged(d["q"], d["kc"], d["vc"], d["table"], d["cu"], d["ctx"], inp["max_q"],
                                 scale=w.scale, window=window)
    torch.cuda.synchronize()
    ob, lb = host_bits(o), lse.cpu().numpy()
    cu = inp["cu_q"]
    for b in range(w.B):
        L, n = int(ctx[b]), int(new[b])
        tb = d["table"][b:b + 1].contiguous()
        cb = d["ctx"][b:b + 1].contiguous()
        kg, vg = sdpt.paged_kv_gather(d["kc"], d["vc"], tb, cb, L)
        qb = d["q"][cu[b]:cu[b + 1]].unsqueeze(0).contiguous()
        oc, lc = sdpt.attn_fwd_chunk(qb, kg, vg, L - n, 0, scale=w.scale, window=window, out_dtype=qb.dtype)
        torch.cuda.synchronize()
        assert np.array_equal(ob[cu[b]:cu[b + 1]], host_bits(oc)[0]), b
        assert np.array_equal(lb[:, cu[b]:cu[b + 1]], lc.cpu().numpy()[0]), b


def test_fwd_paged_never_reads_unused_pages_or_slots():
    """Pool pages no sequence uses, the slots past each context and the table entries past each
    sequence's pages hold NaN / out-of-pool ids: the result is finite and equals the clean run's
    bit for bit."""
    w = MIXED.scaled(B=4, Hq=8, Hkv=2, D=512, ctx=(70, 1, 33, 300), new=(20, 1, 1, 64))
    clean = make_prefill_inputs(w, seed=33)
    pois = make_prefill_inputs(w, seed=33, poison_unused=True)
    table = pois["block_table"].copy()
    for b in range(w.B):
        table[b, -(-int(w.ctx[b]) // 16):] = 1 << 30
    pois["block_table"] = table
    say("[fwd paged poisoned]")
    outs = []
    for inp in (clean, pois):
        d = _prefill_dev(inp, "bf16")
        o, lse = sdpt.attn_fwd_paged(d["q"], d["kc"], d["vc"], d["table"], d["cu"], d["ctx"], inp["max_q"],
                                     scale=w.scale)
        torch.cuda.synchronize()
        outs.append((host_bits(o), lse.cpu().numpy()))
    assert np.isfinite(outs[1][1]).all() and all_finite(torch.from_numpy(outs[1][1]))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


# (D, dtype, window, softcap, contexts, new rows) for the split paged forward: decode rows whose
# keys span 9, 10, 66 and 128 tiles (2, 2, 9 and 16 pieces) beside a prompt chunk; a window that
# leaves 16 tiles (2 pieces) beside a short prompt; a batch of decode rows only (one item slot per
# unit without the split) in fp16 with a softcap; decode rows at or under 8 tiles (not split)
SPLIT_CASES = [
    (512, "bf16", 0, 0.0, (1000, 4096, 257, 300, 2100, 256), (300, 1, 1, 1, 1, 1)),
    (256, "bf16", 500, 0.0, (3000, 1200, 40), (1, 64, 1)),
    (512, "f16", 0, 30.0, (1500, 800, 4000), (1, 1, 1)),
    (256, "bf16", 0, 0.0, (1030, 33, 700), (1, 1, 20)),
]


@pytest.mark.parametrize("D,dtype,window,softcap,ctx,new", SPLIT_CASES)
def test_fwd_paged_split_matches_oracle(D, dtype, window, softcap, ctx, new):
    """attn_fwd_paged_split: every row against the oracle; rows that are not split (every row of a
    sequence with more than one new token, decode rows of at most 8 key tiles) bit for bit equal to
    attn_fwd_paged's; split decode rows within the tolerance of attn_fwd_paged's."""
    w = MIXED.scaled(B=len(ctx), Hq=8, Hkv=2, D=D, dtype=dtype, window=window, ctx=ctx, new=new,
                     name=f"paged fwd split d{D}")
    inp = make_prefill_inputs(w, seed=33)
    say(f"[fwd paged split] D={D} dtype={dtype} window={window} softcap={softcap} ctx={ctx} new={new}")
    d = _prefill_dev(inp, dtype)
    kw = dict(scale=w.scale, window=window, softcap=softcap)
    o, lse = sdpt.attn_fwd_paged_split(d["q"], d["kc"], d["vc"], d["table"], d["cu"], d["ctx"], inp["max_q"], **kw)
    o1, lse1 = sdpt.attn_fwd_paged(d["q"], d["kc"], d["vc"], d["table"], d["cu"], d["ctx"], inp["max_q"], **kw)
    torch.cuda.synchronize()
    assert all_finite(o, lse)
    ro, rl = _prefill_oracle(inp, w, softcap)
    assert max_abs(host(o), ro) <= O_MAX_ABS
    assert max_abs(host(lse), rl) <= LSE_MAX_ABS
    ob, ob1, lb, lb1 = host_bits(o), host_bits(o1), lse.cpu().numpy(), lse1.cpu().numpy()
    cu = inp["cu_q"]
    n_split = 0
    for b in range(w.B):
        L, n = int(ctx[b]), int(new[b])
        rows = slice(int(cu[b]), int(cu[b + 1]))
        lo = max(0, L - window) if window > 0 else 0
        tiles = (L + 31) // 32 - lo // 32 if L > lo else 0
        if n == 1 and tiles > 8:
            n_split += 1
            assert max_abs(host(o)[rows], host(o1)[rows]) <= O_MAX_ABS, b
            assert max_abs(lb[:, rows], lb1[:, rows]) <= LSE_MAX_ABS, b
        else:
            assert np.array_equal(ob[rows], ob1[rows]), b
            assert np.array_equal(lb[:, rows], lb1[:, rows]), b
    assert n_split > 0
    say(f"[fwd paged split] {n_split} of {w.B} sequences split")


def test_fwd_paged_split_captured_in_a_graph():
    """attn_fwd_paged_split (rank, forward, merge) captured once in a HIP graph over fixed buffers
    and one workspace, then replayed with new query values and new context lengths of the decode
    rows written into the captured buffers: the pieces a row is cut into are decided on the device
    at each replay, and every replay equals an eager call on the same inputs bit for bit (and the
    oracle within tolerance)."""
    ctx, new = (600, 2000, 300, 1200), (100, 1, 1, 1)
    w = MIXED.scaled(B=len(ctx), Hq=8, Hkv=2, D=512, dtype="bf16", window=0, ctx=ctx, new=new,
                     name="paged fwd split graph")
    inp = make_prefill_inputs(w, seed=34)
    d = _prefill_dev(inp, "bf16")
    maxq = inp["max_q"]
    ws = torch.empty(sdpt.binding.attn_fwd_paged_workspace_bytes(d["q"], d["kc"], d["table"], d["cu"], maxq),
                     device="cuda:0", dtype=torch.uint8)
    o, lse = torch.empty_like(d["q"]), torch.empty((w.Hq, d["q"].shape[0]), device="cuda:0", dtype=torch.float32)

    def call(out, l):
        sdpt.attn_fwd_paged_split(d["q"], d["kc"], d["vc"], d["table"], d["cu"], d["ctx"], maxq, scale=w.scale,
                                  out=out, lse=l, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the graph
        call(torch.empty_like(o), torch.empty_like(lse))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(o, lse)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(35)
    # decode rows' contexts per replay, never above the pages their table rows hold (the prompt's
    # stays): 8..63 tiles, so 2..8 pieces, or one decode row not split
    ctxs = [(600, 2000, 300, 1200), (600, 1500, 257, 256), (600, 290, 299, 1199)]
    for i, c in enumerate(ctxs):
        say(f"[paged split graph] replay {i} contexts {c}")
        d["q"].copy_(torch.randn(d["q"].shape, generator=gen, device="cuda:0").to(torch.bfloat16))
        d["ctx"].copy_(torch.tensor(c, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        eo, el = torch.empty_like(o), torch.empty_like(lse)
        call(eo, el)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(o), host_bits(eo)), i
        assert np.array_equal(lse.cpu().numpy(), el.cpu().numpy()), i
        assert all_finite(o, lse)
    inp2 = dict(inp, q=host_bits(d["q"]), ctx_lens=np.array(ctxs[-1], dtype=np.int32))
    w2 = MIXED.scaled(B=len(ctx), Hq=8, Hkv=2, D=512, dtype="bf16", window=0, ctx=ctxs[-1], new=new,
                      name="paged fwd split graph")
    ro, rl = _prefill_oracle(inp2, w2)
    assert max_abs(host(o), ro) <= O_MAX_ABS
    assert max_abs(host(lse), rl) <= LSE_MAX_ABS


@pytest.mark.parametrize("name,split", [("mixed_step_d512", False), ("mixed_step_d512", True),
                                        ("paged_prefill_d512", False)])
def test_paged_forward_full_size_sampled_rows(name, split):
    """The benchmark's paged-forward workloads at their full sizes (a 1024-token chunk after 3072
    cached plus 31 decode rows; a 2048-token chunk after 6144 cached; 32 query heads, D = 512):
    every decode row, the chunk's first, last and tile-edge rows and seeded random rows, every
    head, against the oracle row by row; the mixed step also through attn_fwd_paged_split."""
    w = PREFILL_WORKLOADS[name]
    inp = make_prefill_inputs(w, seed=0)
    say(f"[{name} full size] split={split}")
    d = _prefill_dev(inp, "bf16")
    fwd = sdpt.attn_fwd_paged_split if split else sdpt.attn_fwd_paged
    o, lse = fwd(d["q"], d["kc"], d["vc"], d["table"], d["cu"], d["ctx"], inp["max_q"], scale=w.scale)
    torch.cuda.synchronize()
    assert all_finite(o, lse)
    oh, lh = host(o), lse.cpu().numpy()
    cu = inp["cu_q"]
    n0 = int(w.new[0])
    pick = np.random.default_rng(7).choice(n0, size=min(24, n0), replace=False).tolist()
    rows = sorted(set([0, 1, 15, 16, 127, 128, n0 // 2, n0 - 2, n0 - 1] + pick + list(range(n0, int(cu[-1])))))
    f = lambda x: bits_to_f64(x, "bf16")  # noqa: E731
    q, kc, vc = f(inp["q"]), f(inp["k_cache"]), f(inp["v_cache"])
    worst_o = worst_l = 0.0
    gathered = {}
    for t in rows:
        b = int(np.searchsorted(cu, t, side="right") - 1)
        L, n = int(w.ctx[b]), int(w.new[b])
        pos = L - n + (t - int(cu[b]))
        if b not in gathered:
            gathered = {b: (oracle.gather_pages(kc, inp["block_table"][b], L, w.page_size)[None],
                            oracle.gather_pages(vc, inp["block_table"][b], L, w.page_size)[None])}
        kk, vv = gathered[b]
        ro, rl = oracle.attention_forward_chunk(q[None, t:t + 1], kk, vv, w.scale, True, 0, pos, 0)
        worst_o = max(worst_o, max_abs(oh[t], ro[0, 0]))
        worst_l = max(worst_l, max_abs(lh[:, t], rl[0, :, 0]))
    say(f"[{name} full size] rows={len(rows)} O max-abs {worst_o:.3g} LSE max-abs {worst_l:.3g}")
    assert worst_o <= O_MAX_ABS and worst_l <= LSE_MAX_ABS


def test_decode_graphs_per_bucket_replay_like_eager_calls():
    """One captured decode step (append the current token's K/V, then decode) per bucket [1, 2, 4,
    ..., 64], over one set of buffers and one shared workspace (DecodeGraphs).  For a sequence of
    batch sizes, the smallest bucket >= B is replayed with rows B .. bucket-1 as padding (context
    0); each replay equals the same step made with eager calls on the bucket's rows bit for bit
    (output and caches: the graph of bucket n is the step on rows 0 .. n-1, and the decode's
    schedule, hence its rounding, depends on the row count), its padding rows are exact zeros,
    and the B rows are within tolerance of the oracle."""
    w = DECODE_WORKLOADS["decode_d128"].scaled(ctx_range=(20, 700))    # B = 64 rows, shorter contexts
    inp = make_decode_inputs(w, seed=50)
    sizes = [1, 3, 8, 17, 64, 40, 3, 64]
    table, kc, vc, _ = _with_room(inp, w, len(sizes))
    cur = inp["ctx_lens"].astype(np.int32).copy()
    k_d, v_d = dev(kc), dev(vc)
    k_e, v_e = k_d.clone(), v_d.clone()
    t_d = torch.from_numpy(table).to("cuda:0")
    q_s = torch.zeros((w.B, w.Hq, w.D), device="cuda:0", dtype=torch.bfloat16)
    kn_s = torch.zeros((w.B, 1, w.Hkv, w.D), device="cuda:0", dtype=torch.bfloat16)
    vn_s = torch.zeros_like(kn_s)
    ctx_s = torch.zeros(w.B, device="cuda:0", dtype=torch.int32)
    out_s = torch.zeros_like(q_s)
    buckets = [1, 2, 4, 8, 16, 32, 64]
    g = sdpt.DecodeGraphs(q_s, k_d, v_d, t_d, ctx_s, out_s, buckets, scale=w.scale, k_new=kn_s, v_new=vn_s)
    torch.cuda.synchronize()
    kc_ref, vc_ref = bits_to_f64(kc, "bf16"), bits_to_f64(vc, "bf16")
    ws = torch.empty(1 << 24, device="cuda:0", dtype=torch.uint8)
    for i, B in enumerate(sizes):
        cur[:B] += 1
        ctx = np.where(np.arange(w.B) < B, cur, 0).astype(np.int32)
        q_s.copy_(dev(normal_16(stream(60 + i, w.wid, 0), (w.B, w.Hq, w.D))))
        kn_s.copy_(dev(normal_16(stream(60 + i, w.wid, 1), (w.B, 1, w.Hkv, w.D))))
        vn_s.copy_(dev(normal_16(stream(60 + i, w.wid, 2), (w.B, 1, w.Hkv, w.D))))
        ctx_s.copy_(torch.from_numpy(ctx).to("cuda:0"))
        out_s.fill_(1.0)
        torch.cuda.synchronize()
        say(f"[decode graphs] step {i} B={B}")
        bucket = g.launch(B)
        assert bucket == min(b for b in buckets if b >= B)
        torch.cuda.synchronize()
        got = out_s.clone()
        # the same step with eager calls on the bucket's rows (padding included) and other caches
        tb, cb = t_d[:bucket].contiguous(), ctx_s[:bucket].contiguous()
        sdpt.paged_kv_append(kn_s[:bucket].contiguous(), vn_s[:bucket].contiguous(), k_e, v_e, tb, cb)
        eager = sdpt.paged_decode(q_s[:bucket].contiguous(), k_e, v_e, tb, cb, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(got[:bucket]), host_bits(eager)), i
        assert not host_bits(got[B:bucket]).any(), i                      # padding rows: O = 0
        assert np.array_equal(host_bits(k_d), host_bits(k_e)) and np.array_equal(host_bits(v_d), host_bits(v_e)), i
        kc_ref = oracle.paged_append(kc_ref, table[:B], ctx[:B], host(kn_s[:B]), w.page_size)
        vc_ref = oracle.paged_append(vc_ref, table[:B], ctx[:B], host(vn_s[:B]), w.page_size)
        ref = oracle.paged_decode(host(q_s[:B]), kc_ref, vc_ref, table[:B], ctx[:B], w.scale, w.page_size)
        assert all_finite(got[:B])
        assert max_abs(host(got[:B]), ref) <= O_MAX_ABS, i
    g.close()


@pytest.mark.parametrize("Hq,Hkv,split", [(4, 4, False), (16, 1, False), (4, 4, True), (16, 1, True)])
def test_fwd_paged_strided_views_and_group_sizes(Hq, Hkv, split):
    """Queries and outputs as strided views (every other head of a wider tensor) and K/V caches as
    the two halves of one combined (num_pages, 16, 2, Hkv, D) cache, at group sizes 1 and 16, through
    attn_fwd_paged and attn_fwd_paged_split (whose decode row of 700 keys is cut into 3 pieces): the
    kernels read every tensor through its own strides; results as the oracle's."""
    ctx, new = (200, 700, 77), (64, 1, 77)
    w = MIXED.scaled(B=3, Hq=Hq, Hkv=Hkv, D=256, ctx=ctx, new=new)
    inp = make_prefill_inputs(w, seed=34)
    say(f"[fwd paged strided] Hq={Hq} Hkv={Hkv} split={split}")
    T = int(inp["cu_q"][-1])
    qw = torch.zeros((T, 2 * Hq, w.D), device="cuda:0", dtype=torch.bfloat16)
    qw[:, ::2] = dev(inp["q"])
    q = qw[:, ::2]                                     # head stride 2 D
    kv = torch.zeros((inp["k_cache"].shape[0], 16, 2, Hkv, w.D), device="cuda:0", dtype=torch.bfloat16)
    kv[:, :, 0] = dev(inp["k_cache"])
    kv[:, :, 1] = dev(inp["v_cache"])
    ow = torch.full((T, 2 * Hq, w.D), 7.0, device="cuda:0", dtype=torch.bfloat16)
    o = ow[:, 1::2]
    d = _prefill_dev(inp, "bf16")
    fwd = sdpt.attn_fwd_paged_split if split else sdpt.attn_fwd_paged
    _, lse = fwd(q, kv[:, :, 0], kv[:, :, 1], d["table"], d["cu"], d["ctx"], inp["max_q"], scale=w.scale, out=o)
    torch.cuda.synchronize()
    ro, rl = _prefill_oracle(inp, w)
    assert max_abs(host(o), ro) <= O_MAX_ABS and max_abs(host(lse), rl) <= LSE_MAX_ABS
    assert (ow[:, ::2] == 7.0).all()                   # the interleaved heads are untouched
