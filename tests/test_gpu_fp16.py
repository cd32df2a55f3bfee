"""GPU parity of IEEE-half (fp16) inputs against the float64 oracle, through the C ABI.

The first page's eligibility gate admits fp16 as well as bf16 (section Integration).  The same
kernels run with the half-precision matrix instructions and conversions; the oracle sees the
exact values of the fp16 draws.  Cases: the whole-sequence forward and backward (GQA d512 with
a ragged tail, d256 sliding window, padded varlen, non-causal, a softcap), a ring of chunk pairs
merged into an fp16 output, the paged decode, and a full-size d512 workload on sampled rows.
Tolerances as for bf16 (O max-abs 2e-2, LSE 1e-2, gradients relative L2 5e-2).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import (ATTN_WORKLOADS, DECODE_WORKLOADS, AttnWorkload, bits_to_f64, lengths_to_pad_mask,
                   make_attention_inputs, make_decode_inputs)
from tests.gpu_util import GRAD_REL_L2, LSE_MAX_ABS, O_MAX_ABS, all_finite, dev, host, host_bits, max_abs, rel_l2

pytestmark = pytest.mark.gpu

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(inp, x):
    return bits_to_f64(inp[x], "f16")


CASES = [
    # name, workload, lengths, softcap
    ("d512_gqa_ragged", AttnWorkload(301, "f16 d512 gqa", 2, 300, 16, 2, 512, dtype="f16"), None, 0.0),
    ("d256_window", AttnWorkload(302, "f16 d256 window", 2, 700, 4, 2, 256, window=200, qk_std=3.0,
                                 dtype="f16"), None, 0.0),
    ("d512_varlen", AttnWorkload(303, "f16 d512 varlen", 3, 333, 8, 2, 512, varlen="pad_mask", dtype="f16"),
     [333, 1, 150], 0.0),
    ("d512_noncausal", AttnWorkload(304, "f16 d512 non-causal", 1, 257, 4, 1, 512, causal=False, dtype="f16"),
     None, 0.0),
    ("d512_softcap", AttnWorkload(305, "f16 d512 softcap", 1, 400, 8, 2, 512, qk_std=2.0, dtype="f16"), None,
     3.0),
]


@pytest.mark.parametrize("name,w,lengths,cap", CASES, ids=[c[0] for c in CASES])
def test_fp16_matches_oracle(name, w, lengths, cap):
    say(f"[fp16 {name}] B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} W={w.window} cap={cap}")
    inp = make_attention_inputs(w, seed=0)
    q, k, v, do = (dev(inp[x], "f16") for x in ("q", "k", "v", "do"))
    assert q.dtype == torch.float16
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, softcap=cap)
    L = [w.S] * w.B if lengths is None else lengths
    if lengths is not None:
        kw["pad_mask"] = torch.from_numpy(lengths_to_pad_mask(np.array(lengths), w.S)).to("cuda:0")
    o, lse = sdpt.attn_fwd(q, k, v, **kw)
    dq, dk, dv = sdpt.attn_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert t.dtype == torch.float16
    assert all_finite(o, lse, dq, dk, dv)
    ro, rl = oracle.attention_forward(f64(inp, "q"), f64(inp, "k"), f64(inp, "v"), w.scale, w.causal, w.window,
                                      lengths, cap)
    rq, rk, rv = oracle.attention_backward(f64(inp, "q"), f64(inp, "k"), f64(inp, "v"), f64(inp, "do"), w.scale,
                                           w.causal, w.window, lengths, cap)
    go, gl = host(o), host(lse)
    cat = lambda x: np.concatenate([x[b, :L[b]] for b in range(w.B)])  # noqa: E731
    assert max_abs(cat(go), cat(ro)) <= O_MAX_ABS
    assert max(max_abs(gl[b, :, :L[b]], rl[b, :, :L[b]]) for b in range(w.B)) <= LSE_MAX_ABS
    for nm, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = rel_l2(cat(host(g)), cat(r))
        assert err <= GRAD_REL_L2, (nm, err)
    for b in range(w.B):   # padded rows and keys: exact zeros
        for t in (o, dq, dk, dv):
            assert not host_bits(t[b, L[b]:]).any()


def test_fp16_ring_of_chunks_matches_oracle():
    """Three chunk pairs per query chunk: fp32 partials merged with an fp16 final output, and the
    gradient parts added into fp32 accumulators."""
    w = AttnWorkload(306, "f16 ring", 1, 520, 8, 2, 512, dtype="f16")
    bounds = [0, 200, 400, 520]
    inp = make_attention_inputs(w, seed=1)
    q, k, v, do = (dev(inp[x], "f16") for x in ("q", "k", "v", "do"))
    say("[fp16 ring]")
    n = len(bounds) - 1
    outs, lses = [], []
    for a in range(n):
        q0, q1 = bounds[a], bounds[a + 1]
        out = torch.empty_like(q[:, q0:q1])
        acc_o = acc_l = None
        for c in range(n):
            k0, k1 = bounds[c], bounds[c + 1]
            po, pl = sdpt.attn_fwd_chunk(q[:, q0:q1], k[:, k0:k1], v[:, k0:k1], q0, k0, scale=w.scale)
            if acc_o is None:
                acc_o, acc_l = po, pl
            else:
                sdpt.attn_lse_merge(acc_o, acc_l, po, pl, out=out if c == n - 1 else None)
        outs.append(out)
        lses.append(acc_l)
    dq = torch.zeros(q.shape, device="cuda:0")
    dk = torch.zeros(k.shape, device="cuda:0")
    dv = torch.zeros(v.shape, device="cuda:0")
    for a in range(n):
        q0, q1 = bounds[a], bounds[a + 1]
        for c in range(n):
            k0, k1 = bounds[c], bounds[c + 1]
            sdpt.attn_bwd_chunk(q[:, q0:q1], k[:, k0:k1], v[:, k0:k1], outs[a], lses[a], do[:, q0:q1], q0, k0,
                                scale=w.scale, dq=dq[:, q0:q1], dk=dk[:, k0:k1], dv=dv[:, k0:k1], accumulate=True)
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1)
    assert o.dtype == torch.float16 and all_finite(o, dq, dk, dv)
    ro, rl = oracle.attention_forward(f64(inp, "q"), f64(inp, "k"), f64(inp, "v"), w.scale, True, 0)
    rq, rk, rv = oracle.attention_backward(f64(inp, "q"), f64(inp, "k"), f64(inp, "v"), f64(inp, "do"), w.scale,
                                           True, 0)
    assert max_abs(host(o), ro) <= O_MAX_ABS
    assert max_abs(host(torch.cat(lses, dim=2)), rl) <= LSE_MAX_ABS
    for nm, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert rel_l2(host(g), r) <= GRAD_REL_L2, nm


def test_fp16_paged_decode_matches_oracle():
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=6, ctx_range=(1, 1500), dtype="f16")
    inp = make_decode_inputs(w, seed=5)
    say(f"[fp16 decode] ctx {inp['ctx_lens'].tolist()}")
    qd, kc, vc = (dev(inp[x], "f16") for x in ("q", "k_cache", "v_cache"))
    table = torch.from_numpy(inp["block_table"]).to("cuda:0")
    ctx = torch.from_numpy(inp["ctx_lens"]).to("cuda:0")
    o = sdpt.paged_decode(qd, kc, vc, table, ctx, scale=w.scale)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16 and all_finite(o)
    r = oracle.paged_decode(f64(inp, "q"), f64(inp, "k_cache"), f64(inp, "v_cache"), inp["block_table"],
                            inp["ctx_lens"], w.scale)
    assert max_abs(host(o), r) <= O_MAX_ABS


def test_fp16_full_size_d512_sampled_rows():
    w = ATTN_WORKLOADS["full_d512"].scaled(dtype="f16")
    inp = make_attention_inputs(w, seed=0)
    q, k, v, do = (dev(inp[x], "f16") for x in ("q", "k", "v", "do"))
    say("[fp16 full] GPU")
    o, lse = sdpt.attn_fwd(q, k, v, scale=w.scale)
    dq, dk, dv = sdpt.attn_bwd(q, k, v, o, lse, do, scale=w.scale)
    torch.cuda.synchronize()
    assert all_finite(o, lse, dq, dk, dv)
    f = {x: f64(inp, x) for x in ("q", "k", "v", "do")}
    rng = np.random.default_rng(4)
    for (b, h) in ((0, 3), (1, 30)):
        rows = np.unique(np.concatenate([[0, 1, w.S - 1], rng.integers(0, w.S, size=29)]))
        say(f"[fp16 full] oracle rows b={b} h={h}")
        ro, rl, rq = oracle.attention_rows(f["q"], f["k"], f["v"], f["do"], b, h, rows, w.scale, True, 0, None)
        assert max_abs(host(o[b, rows, h]), ro) <= O_MAX_ABS
        assert max_abs(host(lse[b, h, rows]), rl) <= LSE_MAX_ABS
        assert rel_l2(host(dq[b, rows, h]), rq) <= GRAD_REL_L2
