"""The head_dim-512 forward's softmax reference: forced restarts and peaked rows.

At head_dim 512 the forward fixes each row's softmax reference from the first keys the row sees
and, when a later score exceeds it by more than the 16-bit probability range allows (32 powers
of two in bf16, 15 in IEEE half), restarts the workgroup's key loop with raised references.  N(0,1)
scores never get there, so these tests build inputs that must: every query row of a kv group is
one vector u plus small noise, keys are small noise, and a few "spike" keys are multiples of u
whose scores sit tens of nats above everything else.  A row that sees a spike restarts once per
spike that raises its maximum past the slack; the restart counter (attn_count_restarts) shows
that the branch ran.  Two neighbouring spikes of equal height along u but different directions
keep the softmax after the restart non-trivial (weights near one half, varying by row).  O, LSE, dQ, dK and dV are
compared element by element with the float64 oracle at the usual tolerances.

The peaked case without a softcap (Q and K with standard deviation 3, head_dim 512: scaled
scores with standard deviation 9) puts one key far above the rest in most rows without any
restart; the forward's normaliser sums the rounded probabilities, so the dominant term's
rounding divides out of O.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import AttnWorkload, bits_to_f64, f32_to_bf16_bits, f32_to_f16_bits, make_attention_inputs
from tests.gpu_util import GRAD_REL_L2, LSE_MAX_ABS, O_MAX_ABS, all_finite, dev, host, max_abs, rel_l2

pytestmark = pytest.mark.gpu

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def spike_inputs(w, seed, spikes, q_noise=0.1, k_noise=0.25):
    """Inputs whose query rows of kv group g are u_g + q_noise * N(0,1) (u_g a N(0,1) row), keys
    k_noise * N(0,1), except key j of every sequence and kv head set to beta * (u_g + mix * w_g)
    for each (j, beta, mix) in spikes, w_g a N(0,1) row made orthogonal to u_g.  Against a query
    row the w_g part only meets the noise, so two spikes of one height with mix 0 and 1 score
    within a fraction of a nat of each other while their keys stay far apart (nearly equal keys
    would make dQ the small difference of two large bf16-rounded terms).  Rounded to the
    workload's 16-bit type; the same bytes go to both sides."""
    inp = make_attention_inputs(w, seed=seed)
    q = bits_to_f64(inp["q"], w.dtype)
    k = bits_to_f64(inp["k"], w.dtype)
    v = bits_to_f64(inp["v"], w.dtype)
    r = w.r
    for g in range(w.Hkv):
        u = q[0, 0, g * r].copy()
        wv = v[0, 0, g].copy()
        wv -= (wv @ u) / (u @ u) * u
        q[:, :, g * r:(g + 1) * r] = u + q_noise * q[:, :, g * r:(g + 1) * r]
        k[:, :, g] *= k_noise
        for j, beta, mix in spikes:
            k[:, j, g] = beta * (u + mix * wv)
    conv = f32_to_f16_bits if w.dtype == "f16" else f32_to_bf16_bits
    inp["q"] = conv(q.astype(np.float32))
    inp["k"] = conv(k.astype(np.float32))
    return inp


def run_and_compare(w, inp):
    """GPU forward + backward with the restart counter on; compares everything with the oracle
    and returns the number of workgroup restarts."""
    q, k, v, do = (dev(inp[x], w.dtype) for x in ("q", "k", "v", "do"))
    counter = torch.zeros(1, device="cuda:0", dtype=torch.int32)
    kw = dict(scale=w.scale, causal=w.causal, window=w.window)
    sdpt.binding.count_restarts(counter)
    try:
        o, lse = sdpt.attn_fwd(q, k, v, **kw)
    finally:
        sdpt.binding.count_restarts(None)
    dq, dk, dv = sdpt.attn_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    restarts = int(counter.item())
    assert all_finite(o, lse, dq, dk, dv)
    f = {x: bits_to_f64(inp[x], w.dtype) for x in ("q", "k", "v", "do")}
    ro, rl = oracle.attention_forward(f["q"], f["k"], f["v"], w.scale, w.causal, w.window)
    rq, rk, rv = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], w.scale, w.causal, w.window)
    e_o, e_l = max_abs(host(o), ro), max_abs(host(lse), rl)
    e_g = [rel_l2(host(a), r) for a, r in ((dq, rq), (dk, rk), (dv, rv))]
    say(f"[{w.name}] workgroup restarts {restarts}; O max-abs {e_o:.3e}, LSE max-abs {e_l:.3e}, "
        f"rel-L2 dQ {e_g[0]:.3e} dK {e_g[1]:.3e} dV {e_g[2]:.3e}")
    assert e_o <= O_MAX_ABS, e_o
    assert e_l <= LSE_MAX_ABS, e_l
    for name, e in zip(("dq", "dk", "dv"), e_g):
        assert e <= GRAD_REL_L2, (name, e)
    return restarts


# scaled score of a spike beta * u against a row u + noise: about beta * |u|^2 / sqrt(512), i.e.
# beta * 22.6 nats = beta * 32.6 powers of two above the noise keys' scores (about 0)
RESTART_CASES = [
    # name, dtype, spikes (key, beta, mix): the first pair of spikes lies beyond the first key
    # tile and more than the slack above it; the last spike exceeds the raised reference again
    ("bf16", "bf16", [(150, 2.0, 0.0), (151, 2.0, 1.0), (420, 4.0, 0.0)]),
    ("f16", "f16", [(100, 0.8, 0.0), (101, 0.8, 1.0), (333, 1.6, 0.0)]),
]


@pytest.mark.parametrize("name,dtype,spikes", RESTART_CASES, ids=[c[0] for c in RESTART_CASES])
def test_d512_reference_restart_matches_oracle(name, dtype, spikes):
    w = AttnWorkload(140 if dtype == "bf16" else 141, f"d512 forced restarts {dtype}", 2, 600, 8, 2, 512,
                     dtype=dtype)
    inp = spike_inputs(w, 0, spikes)
    restarts = run_and_compare(w, inp)
    # every workgroup holding a row past the first spike restarts at least once
    assert restarts > 0, "the restart branch did not run"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_d512_peaked_without_softcap_matches_oracle(dtype):
    # in IEEE half the slack is 15 powers of two, so these rows also restart
    w = AttnWorkload(142, f"d512 peaked (Q, K std 3), no softcap, {dtype}", 1, 2048, 16, 2, 512, qk_std=3.0,
                     dtype=dtype)
    inp = make_attention_inputs(w, seed=0)
    run_and_compare(w, inp)
