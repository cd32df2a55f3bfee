"""GPU parity of the chunk-pair calls (attn_fwd_chunk, attn_bwd_chunk, attn_lse_merge,
attn_fwd_chunk_merge) against the float64 oracle, through the C ABI.

A sequence is cut into chunks, as a ring of context-parallel ranks would hold it; every query chunk
meets every key/value chunk (fully masked pairs included) at its true positions.  Checked:
  * each pair's partial O and LSE against the oracle's chunk forward (rows that see no key of the
    pair: O exactly zero, LSE exactly -inf);
  * the partials merged with attn_lse_merge against the oracle's whole-sequence forward, and the
    fused forward-and-merge call bit for bit against the two-step one;
  * a rank's forward steps captured in a HIP graph and replayed, bit for bit against eager calls;
  * each pair's gradient parts against the oracle's chunk backward (fed the oracle's own final O
    and LSE), and the parts summed in fp32 against the oracle's whole-sequence backward.
Tolerances as for the whole-sequence path: O max-abs 2e-2, LSE max-abs 1e-2, gradients relative
L2 5e-2.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import AttnWorkload, bf16_bits_to_f64, bits_to_f64, make_attention_inputs, normal_16, stream
from tests.gpu_util import GRAD_REL_L2, LSE_MAX_ABS, O_MAX_ABS, all_finite, dev, host, host_bits, max_abs, rel_l2

pytestmark = pytest.mark.gpu

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def ring_forward(q, k, v, bounds, scale, causal, window, softcap=0.0):
    """Partials (fp32 O) of every (query chunk, key chunk) pair, and per query chunk their merge:
    the bf16 O written by the last merge and the merged LSE."""
    parts, merged = {}, []
    n = len(bounds) - 1
    for a in range(n):
        q0, q1 = bounds[a], bounds[a + 1]
        acc_o = acc_l = None
        out = torch.empty_like(q[:, q0:q1])
        for c in range(n):
            k0, k1 = bounds[c], bounds[c + 1]
            o, lse = sdpt.attn_fwd_chunk(q[:, q0:q1], k[:, k0:k1], v[:, k0:k1], q0, k0, scale=scale, causal=causal,
                                         window=window, softcap=softcap)
            parts[a, c] = (o.clone(), lse.clone())
            if acc_o is None:
                acc_o, acc_l = o, lse
            else:
                sdpt.attn_lse_merge(acc_o, acc_l, o, lse, out=out if c == n - 1 else None)
        merged.append((out, acc_l))
    torch.cuda.synchronize()
    return parts, merged


def ring_backward(q, k, v, do, merged, bounds, scale, causal, window, softcap=0.0):
    """Per query chunk and key chunk: the pair's gradient parts written in bf16, and the same
    parts added by the kernels into fp32 accumulators dQ, dK, dV (the ring's running sums)."""
    dq = torch.zeros(q.shape, device=q.device, dtype=torch.float32)
    dk = torch.zeros(k.shape, device=q.device, dtype=torch.float32)
    dv = torch.zeros(v.shape, device=q.device, dtype=torch.float32)
    parts = {}
    for a in range(len(bounds) - 1):
        q0, q1 = bounds[a], bounds[a + 1]
        o, lse = merged[a]
        for c in range(len(bounds) - 1):
            k0, k1 = bounds[c], bounds[c + 1]
            args = (q[:, q0:q1], k[:, k0:k1], v[:, k0:k1], o, lse, do[:, q0:q1], q0, k0)
            kw = dict(scale=scale, causal=causal, window=window, softcap=softcap)
            parts[a, c] = sdpt.attn_bwd_chunk(*args, **kw)
            sdpt.attn_bwd_chunk(*args, dq=dq[:, q0:q1], dk=dk[:, k0:k1], dv=dv[:, k0:k1], accumulate=True, **kw)
    torch.cuda.synchronize()
    return parts, (dq, dk, dv)


def check_grad_part(got, ref, name):
    if not np.any(ref):
        assert not host_bits(got).any(), f"{name}: a part with no visible pair must be exact zeros"
    else:
        err = rel_l2(host(got), ref)
        assert err <= GRAD_REL_L2, (name, err)


RING = [
    # name, workload, chunk bounds[, softcap]
    ("d512_gqa_ragged", AttnWorkload(201, "ring d512 gqa", 2, 600, 8, 2, 512), [0, 256, 512, 600]),
    ("d512_unaligned", AttnWorkload(202, "ring d512 unaligned", 1, 500, 4, 1, 512), [0, 130, 390, 500]),
    ("d256_window", AttnWorkload(203, "ring d256 window 200", 2, 700, 4, 2, 256, window=200, qk_std=3.0),
     [0, 300, 420, 700]),
    ("d256_window_wide", AttnWorkload(204, "ring d256 window 500", 1, 900, 4, 1, 256, window=500, qk_std=3.0),
     [0, 200, 450, 700, 900]),
    ("d512_noncausal", AttnWorkload(205, "ring d512 non-causal", 1, 300, 4, 2, 512, causal=False), [0, 100, 300]),
    ("d512_softcap", AttnWorkload(210, "ring d512 softcap", 1, 520, 8, 2, 512, qk_std=2.0), [0, 200, 520], 2.5),
]


@pytest.mark.parametrize("case", RING, ids=[c[0] for c in RING])
def test_ring_chunks_match_oracle(case):
    name, w, bounds = case[:3]
    cap = case[3] if len(case) > 3 else 0.0
    say(f"[ring {name}] B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} causal={w.causal} W={w.window} "
        f"chunks={bounds} cap={cap}")
    inp = make_attention_inputs(w, seed=0)
    q, k, v, do = (dev(inp[x]) for x in ("q", "k", "v", "do"))
    f = {x: bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "do")}
    parts, merged = ring_forward(q, k, v, bounds, w.scale, w.causal, w.window, cap)

    # pair partials against the oracle's chunk forward
    for (a, c), (o, lse) in parts.items():
        q0, q1, k0, k1 = bounds[a], bounds[a + 1], bounds[c], bounds[c + 1]
        ro, rl = oracle.attention_forward_chunk(f["q"][:, q0:q1], f["k"][:, k0:k1], f["v"][:, k0:k1], w.scale,
                                                w.causal, w.window, q0, k0, cap)
        go, gl = host(o), host(lse)
        live = np.isfinite(rl)                               # (B, Hq, Sq)
        assert np.array_equal(np.isfinite(gl), live), (a, c)
        assert np.all(gl[~live] == -np.inf)
        assert not go.view(np.uint64)[np.transpose(~live, (0, 2, 1))].any(), (a, c)   # +0.0 exactly
        assert all_finite(go)
        if live.any():
            assert max_abs(gl[live], rl[live]) <= LSE_MAX_ABS, (a, c)
            lrow = np.transpose(live, (0, 2, 1))
            assert max_abs(go[lrow], ro[lrow]) <= O_MAX_ABS, (a, c)

    # merged partials against the whole-sequence oracle
    ro, rl = oracle.attention_forward(f["q"], f["k"], f["v"], w.scale, w.causal, w.window, None, cap)
    for a, (o, lse) in enumerate(merged):
        q0, q1 = bounds[a], bounds[a + 1]
        assert all_finite(o, lse)
        assert max_abs(host(o), ro[:, q0:q1]) <= O_MAX_ABS, a
        assert max_abs(host(lse), rl[:, :, q0:q1]) <= LSE_MAX_ABS, a

    # gradients: parts against the oracle's chunk backward, the kernels' fp32 sums against the
    # whole backward
    gparts, (dq, dk, dv) = ring_backward(q, k, v, do, merged, bounds, w.scale, w.causal, w.window, cap)
    for (a, c), (gq, gk, gv) in gparts.items():
        q0, q1, k0, k1 = bounds[a], bounds[a + 1], bounds[c], bounds[c + 1]
        rq, rk, rv = oracle.attention_backward_chunk(f["q"][:, q0:q1], f["k"][:, k0:k1], f["v"][:, k0:k1],
                                                     ro[:, q0:q1], rl[:, :, q0:q1], f["do"][:, q0:q1], w.scale,
                                                     w.causal, w.window, q0, k0, cap)
        assert all_finite(gq, gk, gv)
        check_grad_part(gq, rq, f"dq{a}{c}")
        check_grad_part(gk, rk, f"dk{a}{c}")
        check_grad_part(gv, rv, f"dv{a}{c}")
    rq, rk, rv = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], w.scale, w.causal, w.window, None, cap)
    for name_, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = rel_l2(host(got), ref)
        assert err <= GRAD_REL_L2, (name_, err)


FUSED = RING + [("f16_d512_ragged", AttnWorkload(211, "ring f16 d512", 1, 600, 8, 2, 512, dtype="f16"),
                  [0, 256, 512, 600])]


@pytest.mark.parametrize("case", FUSED, ids=[c[0] for c in FUSED])
def test_fused_merge_matches_chunk_then_merge(case):
    """attn_fwd_chunk_merge, started from LSE = -inf and a NaN-filled running O, against
    attn_fwd_chunk into an fp32 partial followed by attn_lse_merge, pair by pair in a ring's
    order (the rank's own chunk first, then the chunks before it, wrapping): the running fp32 O,
    the LSE and the final 16-bit O equal bit for bit after every pair; the final result also
    against the whole-sequence oracle."""
    name, w, bounds = case[:3]
    cap = case[3] if len(case) > 3 else 0.0
    say(f"[fused merge {name}] B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} causal={w.causal} W={w.window} "
        f"chunks={bounds} cap={cap} dtype={w.dtype}")
    inp = make_attention_inputs(w, seed=0)
    q, k, v = (dev(inp[x], w.dtype) for x in ("q", "k", "v"))
    n = len(bounds) - 1
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, softcap=cap)
    f = {x: bits_to_f64(inp[x], w.dtype) for x in ("q", "k", "v")}
    ro, rl = oracle.attention_forward(f["q"], f["k"], f["v"], w.scale, w.causal, w.window, None, cap)
    for a in range(n):
        q0, q1 = bounds[a], bounds[a + 1]
        qa = q[:, q0:q1]
        f_o = torch.full((w.B, q1 - q0, w.Hq, w.D), float("nan"), device="cuda:0")
        f_l = torch.full((w.B, w.Hq, q1 - q0), -float("inf"), device="cuda:0")
        f_out, s_out = torch.empty_like(qa), torch.empty_like(qa)
        s_o = s_l = None
        order = [(a - i) % n for i in range(n)]
        for i, c in enumerate(order):
            k0, k1 = bounds[c], bounds[c + 1]
            last = i == n - 1
            sdpt.attn_fwd_chunk_merge(qa, k[:, k0:k1], v[:, k0:k1], q0, k0, f_o, f_l, out=f_out if last else None,
                                      **kw)
            po, pl = sdpt.attn_fwd_chunk(qa, k[:, k0:k1], v[:, k0:k1], q0, k0, **kw)
            if s_o is None:
                s_o, s_l = po, pl
            else:
                sdpt.attn_lse_merge(s_o, s_l, po, pl, out=s_out if last else None)
            torch.cuda.synchronize()
            assert np.array_equal(host_bits(f_o), host_bits(s_o)), (a, c)
            assert np.array_equal(host_bits(f_l), host_bits(s_l)), (a, c)
        assert np.array_equal(host_bits(f_out), host_bits(s_out)), a
        assert all_finite(f_out, f_l)
        assert max_abs(host(f_out), ro[:, q0:q1]) <= O_MAX_ABS, a
        assert max_abs(host(f_l), rl[:, :, q0:q1]) <= LSE_MAX_ABS, a


def test_pairs_without_visible_keys_and_far_positions():
    """A key chunk wholly after the query chunk, and one wholly beyond the window, leave O = 0,
    LSE = -inf and zero gradient parts; positions far above 2^31 give the same bytes as the same
    distances near zero."""
    w = AttnWorkload(206, "ring far", 1, 256, 4, 2, 256)
    inp = make_attention_inputs(w, seed=1)
    q, k, v, do = (dev(inp[x]) for x in ("q", "k", "v", "do"))
    qc, kc, vc, dc = q[:, :128], k[:, 128:], v[:, 128:], do[:, :128]
    say("[ring far] future and beyond-window pairs")
    # the query rows' final O and LSE: their own diagonal chunk at positions 0..127
    o_ref, l_ref = sdpt.attn_fwd_chunk(qc, k[:, :128], v[:, :128], 0, 0, scale=w.scale, out_dtype=torch.bfloat16)
    for (qp, kp, win) in ((0, 128, 0), (1000, 0, 200), (5000, 3000, 1000)):
        o, lse = sdpt.attn_fwd_chunk(qc, kc, vc, qp, kp, scale=w.scale, window=win)
        torch.cuda.synchronize()
        assert not host_bits(o).any(), (qp, kp, win)
        assert np.all(host(lse) == -np.inf), (qp, kp, win)
        gq, gk, gv = sdpt.attn_bwd_chunk(qc, kc, vc, o_ref, l_ref, dc, qp, kp, scale=w.scale, window=win)
        torch.cuda.synchronize()
        for t in (gq, gk, gv):
            assert not host_bits(t).any(), (qp, kp, win)
    # accumulating the parts of a pair without visible keys leaves the accumulators as they were
    acc = [torch.full(t.shape, 1.5, device="cuda:0", dtype=torch.float32) for t in (qc, kc, vc)]
    sdpt.attn_bwd_chunk(qc, kc, vc, o_ref, l_ref, dc, 0, 128, scale=w.scale, dq=acc[0], dk=acc[1], dv=acc[2],
                        accumulate=True)
    torch.cuda.synchronize()
    assert all(bool((t == 1.5).all()) for t in acc)
    # distances decide visibility: shifting both chunks by 2^40 changes no byte
    big = 1 << 40
    for (qp, kp, win) in ((512, 0, 0), (300, 256, 0), (700, 600, 150), (128, 128, 64)):
        o1, l1 = sdpt.attn_fwd_chunk(qc, kc, vc, qp, kp, scale=w.scale, window=win)
        o2, l2 = sdpt.attn_fwd_chunk(qc, kc, vc, qp + big, kp + big, scale=w.scale, window=win)
        g1 = sdpt.attn_bwd_chunk(qc, kc, vc, o_ref, l_ref, dc, qp, kp, scale=w.scale, window=win)
        g2 = sdpt.attn_bwd_chunk(qc, kc, vc, o_ref, l_ref, dc, qp + big, kp + big, scale=w.scale, window=win)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(o1), host_bits(o2)), (qp, kp, win)
        assert np.array_equal(host(l1), host(l2)), (qp, kp, win)
        for x, y in zip(g1, g2):
            assert np.array_equal(host_bits(x), host_bits(y)), (qp, kp, win)


def test_chunk_at_whole_sequence_positions_equals_whole_call():
    """A single chunk pair covering the whole sequence at equal positions is the whole-sequence
    call: the same O and LSE bytes (forward) and the same gradient bytes (backward)."""
    for w in (AttnWorkload(207, "ring whole d512", 2, 300, 8, 2, 512),
              AttnWorkload(208, "ring whole d256 window", 1, 400, 4, 1, 256, window=90, qk_std=3.0)):
        say(f"[ring whole] {w.name}")
        inp = make_attention_inputs(w, seed=2)
        q, k, v, do = (dev(inp[x]) for x in ("q", "k", "v", "do"))
        o, lse = sdpt.attn_fwd(q, k, v, scale=w.scale, causal=True, window=w.window)
        co, cl = sdpt.attn_fwd_chunk(q, k, v, 77, 77, scale=w.scale, window=w.window, out_dtype=torch.bfloat16)
        co32, cl32 = sdpt.attn_fwd_chunk(q, k, v, 77, 77, scale=w.scale, window=w.window)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(o), host_bits(co))
        assert np.array_equal(host(lse), host(cl))
        assert np.array_equal(host(lse), host(cl32))
        # the fp32 partial is the bf16 output before its rounding (both round to nearest even)
        assert np.array_equal(host_bits(o), host_bits(co32.to(torch.bfloat16)))
        g = sdpt.attn_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True, window=w.window)
        cg = sdpt.attn_bwd_chunk(q, k, v, o, lse, do, 77, 77, scale=w.scale, window=w.window)
        torch.cuda.synchronize()
        for x, y in zip(g, cg):
            assert np.array_equal(host_bits(x), host_bits(y))


def test_lse_merge_identity_symmetry_and_poison():
    B, S, H = 2, 70, 4
    gen = torch.Generator(device="cpu")
    gen.manual_seed(9)
    for D in (128, 256, 512):
        say(f"[merge] D={D}")
        oa = torch.randn((B, S, H, D), generator=gen).cuda()
        ob = torch.randn((B, S, H, D), generator=gen).cuda()
        la = (torch.randn((B, H, S), generator=gen) * 4).cuda()
        lb = (torch.randn((B, H, S), generator=gen) * 4).cuda()
        lb[:, :, :10] = -float("inf")          # rows where the second partial saw no key
        la[:, :, 5:10] = -float("inf")         # rows 5..9: neither saw a key
        ob_p = ob.clone()
        ob_p[:, :10] = float("nan")            # never read where its LSE is -inf
        # symmetry: merging (a, b) and (b, a) gives the same bytes
        x_o, x_l, x_r = oa.clone(), la.clone(), torch.empty((B, S, H, D), device="cuda:0", dtype=torch.bfloat16)
        sdpt.attn_lse_merge(x_o, x_l, ob_p, lb, out=x_r)
        y_o, y_l = ob_p.clone(), lb.clone()
        sdpt.attn_lse_merge(y_o, y_l, oa, la)
        torch.cuda.synchronize()
        xb, yb = host_bits(x_o), host_bits(y_o)
        assert np.array_equal(xb[:, 10:], yb[:, 10:])
        assert np.array_equal(host(x_l), host(y_l))
        # the bf16 output is the merged fp32 result rounded to nearest even
        assert np.array_equal(host_bits(x_r), host_bits(x_o.to(torch.bfloat16)))
        # rows 0..4: the -inf partial adds nothing, the result is the other partial's bytes
        assert np.array_equal(xb[:, :5], host_bits(oa)[:, :5])
        assert np.array_equal(host(x_l)[:, :, :5], host(la)[:, :, :5])
        # rows 5..9: nothing seen at all
        assert not xb[:, 5:10].any() and np.all(host(x_l)[:, :, 5:10] == -np.inf)
        # the oracle's merge
        ro, rl = oracle.lse_merge(host(oa), host(la), np.nan_to_num(host(ob_p)), host(lb))
        assert max_abs(host(x_o), ro) <= 1e-5
        live = np.isfinite(rl)
        assert np.array_equal(np.isfinite(host(x_l)), live)
        assert max_abs(host(x_l)[live], rl[live]) <= 1e-5


def test_full_size_ring_d512_two_chunks():
    """Causal GQA d512 (B=1, S=4096, Hq=32, Hkv=4) cut into two 2048-row chunks: the per-rank
    share of context parallelism at its real shape.  Sampled rows of O, LSE and dQ against the
    oracle row by row; dK and dV of one kv head in full.  The fused forward-and-merge path (first
    pair by attn_fwd_chunk, the second by attn_fwd_chunk_merge, as the ring benchmark runs it)
    gives the same bytes as the two-step one."""
    w = AttnWorkload(209, "ring full d512", 1, 4096, 32, 4, 512)
    bounds = [0, 2048, 4096]
    inp = make_attention_inputs(w, seed=0)
    q, k, v, do = (dev(inp[x]) for x in ("q", "k", "v", "do"))
    say("[ring full] GPU")
    _, merged = ring_forward(q, k, v, bounds, w.scale, True, 0)
    _, (dq, dk, dv) = ring_backward(q, k, v, do, merged, bounds, w.scale, True, 0)
    o = torch.cat([m[0] for m in merged], dim=1)
    lse = torch.cat([m[1] for m in merged], dim=2)
    assert all_finite(o, lse, dq, dk, dv)
    for a in range(2):                    # own chunk first, then the other one
        qa = q[:, bounds[a]:bounds[a + 1]]
        own, other = (bounds[a], bounds[a + 1]), (bounds[1 - a], bounds[2 - a])
        kv = lambda c: (k[:, c[0]:c[1]], v[:, c[0]:c[1]])  # noqa: E731
        run_o, run_l = sdpt.attn_fwd_chunk(qa, *kv(own), bounds[a], own[0], scale=w.scale)
        fused = torch.empty_like(qa)
        sdpt.attn_fwd_chunk_merge(qa, *kv(other), bounds[a], other[0], run_o, run_l, scale=w.scale, out=fused)
        acc_o, acc_l = sdpt.attn_fwd_chunk(qa, *kv(own), bounds[a], own[0], scale=w.scale)
        part_o, part_l = sdpt.attn_fwd_chunk(qa, *kv(other), bounds[a], other[0], scale=w.scale)
        two_step = torch.empty_like(qa)
        sdpt.attn_lse_merge(acc_o, acc_l, part_o, part_l, out=two_step)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(fused), host_bits(two_step)), a
        assert np.array_equal(host_bits(run_o), host_bits(acc_o)), a
        assert np.array_equal(host_bits(run_l), host_bits(acc_l)), a
    f = {x: bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "do")}
    rng = np.random.default_rng(3)
    for h in (0, 13, 31):
        rows = np.unique(np.concatenate([[0, 2047, 2048, 4095], rng.integers(0, 4096, size=28)]))
        say(f"[ring full] oracle rows h={h}")
        ro, rl, rq = oracle.attention_rows(f["q"], f["k"], f["v"], f["do"], 0, h, rows, w.scale, True, 0, None)
        assert max_abs(host(o[0, rows, h]), ro) <= O_MAX_ABS
        assert max_abs(host(lse[0, h, rows]), rl) <= LSE_MAX_ABS
        assert rel_l2(host(dq[0, rows, h]), rq) <= GRAD_REL_L2
    say("[ring full] oracle unit g=1")
    rq, rk, rv = oracle.attention_backward_group(f["q"], f["k"], f["v"], f["do"], 0, 1, w.scale, True, 0, None)
    assert rel_l2(host(dq[0, :, 8:16]), rq) <= GRAD_REL_L2
    assert rel_l2(host(dk[0, :, 1]), rk) <= GRAD_REL_L2
    assert rel_l2(host(dv[0, :, 1]), rv) <= GRAD_REL_L2


def test_ring_forward_step_captured_in_a_graph():
    """One rank's forward over three key chunks (attn_fwd_chunk, then attn_fwd_chunk_merge twice,
    the last writing the bf16 O) captured once in a HIP graph and replayed with new queries copied
    into the captured buffer: every replay equals the same calls made eagerly, bit for bit, so
    the chunk calls allocate nothing and do not synchronise."""
    w = AttnWorkload(212, "ring graph", 1, 384, 8, 2, 512)
    bounds = [0, 128, 256, 384]
    inp = make_attention_inputs(w, seed=2)
    k, v = dev(inp["k"]), dev(inp["v"])
    q0 = bounds[2]
    q_s = torch.empty((1, 128, w.Hq, w.D), device="cuda:0", dtype=torch.bfloat16)
    run_o = torch.empty((1, 128, w.Hq, w.D), device="cuda:0")
    run_l = torch.empty((1, w.Hq, 128), device="cuda:0")
    out_s = torch.empty_like(q_s)

    def rank_forward(qq, ro, rl, out):
        for i, c in enumerate((2, 1, 0)):
            k0, k1 = bounds[c], bounds[c + 1]
            if i == 0:
                sdpt.attn_fwd_chunk(qq, k[:, k0:k1], v[:, k0:k1], q0, k0, scale=w.scale, out=ro, lse=rl)
            else:
                sdpt.attn_fwd_chunk_merge(qq, k[:, k0:k1], v[:, k0:k1], q0, k0, ro, rl, scale=w.scale,
                                          out=out if i == 2 else None)

    def load(i):
        q_s.copy_(dev(normal_16(stream(30 + i, w.wid, 0), (1, 128, w.Hq, w.D))))

    load(0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):              # warm-up outside the graph
        rank_forward(q_s, torch.empty_like(run_o), torch.empty_like(run_l), torch.empty_like(out_s))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rank_forward(q_s, run_o, run_l, out_s)
    torch.cuda.synchronize()
    for i in range(3):
        say(f"[ring graph] replay {i}")
        load(i)
        g.replay()
        torch.cuda.synchronize()
        e_o, e_l, e_out = torch.empty_like(run_o), torch.empty_like(run_l), torch.empty_like(out_s)
        rank_forward(q_s, e_o, e_l, e_out)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out_s), host_bits(e_out)), i
        assert np.array_equal(host_bits(run_l), host_bits(e_l)), i
        assert np.array_equal(host_bits(run_o), host_bits(e_o)), i
        assert all_finite(out_s, run_l)
