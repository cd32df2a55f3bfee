"""Full-size parity: every valid row and head of O, LSE and dQ, and every kv head of dK and dV,
of the causal GQA head_dim-512 workload (B2 S4096 Hq32 Hkv4), the head_dim-256 sliding-window
workload (B2 S4096 Hq32 Hkv16, W 1024, Q and K with standard deviation 3) and the padded varlen
workload (B8, lengths U{512..8192} right-padded to 8192, Hq32 Hkv4, head_dim 512), against the
float64 oracle on the same seeded bf16 inputs.

The GPU runs each workload once (a module fixture, in the launch configuration the benchmark
times) and keeps the outputs on the host; each test then compares one sequence against the
oracle, (batch, kv head) unit by unit.  Tolerances: O max-abs 2e-2 and LSE max-abs 1e-2 over
valid rows; dQ, dK, dV relative L2 5e-2 per sequence (which bounds the per-tensor figure);
padded rows of O, dQ, LSE and padded keys of dK, dV exact zeros; no non-finite value anywhere.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from synth import ATTN_WORKLOADS, bits_to_f64, make_attention_inputs
from tests.gpu_util import GRAD_REL_L2, LSE_MAX_ABS, O_MAX_ABS, dev, first_nonfinite, host, host_bits

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_finite(*ts) -> bool:
    ok = all(bool(torch.isfinite(t).all().item()) for t in ts)
    if not ok:
        nf = first_nonfinite(*ts)
        say(f"first non-finite: tensor #{nf[0]} flat index {nf[1]} value {nf[2]}")
    return ok


class FullRun:
    """One GPU forward + backward of a workload; outputs copied to the host as raw bits."""

    def __init__(self, name, seed=0):
        w = ATTN_WORKLOADS[name]
        self.w = w
        say(f"[full {name}] inputs")
        self.inp = make_attention_inputs(w, seed=seed)
        L = self.inp["lengths"]
        self.lengths = [w.S] * w.B if L is None else [int(x) for x in L]
        say(f"[full {name}] GPU forward + backward, lengths {self.lengths}")
        q, k, v, do = (dev(self.inp[x], w.dtype) for x in ("q", "k", "v", "do"))
        kw = dict(scale=w.scale, causal=w.causal, window=w.window)
        if w.varlen == "pad_mask":
            kw["pad_mask"] = torch.from_numpy(self.inp["pad_mask"]).to("cuda:0")
        o, lse = sdpt.attn_fwd(q, k, v, **kw)
        dq, dk, dv = sdpt.attn_bwd(q, k, v, o, lse, do, **kw)
        torch.cuda.synchronize()
        self.finite = device_finite(o, lse, dq, dk, dv)
        self.bits = {n: host_bits(t) for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
        self.lse = host(lse)
        del q, k, v, do, o, lse, dq, dk, dv
        torch.cuda.empty_cache()

    def check_sequence(self, b):
        w, n = self.w, self.lengths[b]
        assert self.finite, "non-finite output"
        t0 = time.perf_counter()
        f = {x: bits_to_f64(self.inp[x][b:b + 1], w.dtype) for x in ("q", "k", "v", "do")}
        r = w.r
        o_err = lse_err = 0.0
        num = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
        den = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
        for g in range(w.Hkv):
            ro, rl, rq, rk, rv = oracle.attention_group(f["q"], f["k"], f["v"], f["do"], 0, g, w.scale, w.causal,
                                                        w.window, [n])
            hs = slice(g * r, (g + 1) * r)
            go = bits_to_f64(self.bits["o"][b, :n, hs], w.dtype)
            o_err = max(o_err, float(np.max(np.abs(go - ro[:n]))))
            lse_err = max(lse_err, float(np.max(np.abs(self.lse[b, hs, :n] - rl[:, :n]))))
            for name, got, ref in (("dq", self.bits["dq"][b, :n, hs], rq[:n]),
                                   ("dk", self.bits["dk"][b, :n, g], rk[:n]),
                                   ("dv", self.bits["dv"][b, :n, g], rv[:n])):
                x = bits_to_f64(got, w.dtype)
                num[name] += float(np.sum((x - ref) ** 2))
                den[name] += float(np.sum(ref ** 2))
        rel = {x: (num[x] / den[x]) ** 0.5 if den[x] > 0 else num[x] ** 0.5 for x in num}
        say(f"[full {w.name}] b={b} len={n}: O max-abs {o_err:.3e}, LSE max-abs {lse_err:.3e}, "
            f"rel-L2 dQ {rel['dq']:.3e} dK {rel['dk']:.3e} dV {rel['dv']:.3e} "
            f"({w.Hkv} units, {time.perf_counter() - t0:.1f} s of oracle)")
        assert o_err <= O_MAX_ABS, o_err
        assert lse_err <= LSE_MAX_ABS, lse_err
        for x in rel:
            assert rel[x] <= GRAD_REL_L2, (x, rel[x])
        # padded rows and keys are exact zeros
        for x in ("o", "dq", "dk", "dv"):
            assert not self.bits[x][b, n:].any(), x
        assert not np.any(self.lse[b, :, n:])


@pytest.fixture(scope="module")
def full_d512():
    return FullRun("full_d512")


@pytest.fixture(scope="module")
def window_d256():
    return FullRun("window_d256")


@pytest.fixture(scope="module")
def varlen_d512():
    return FullRun("varlen_d512")


@pytest.mark.parametrize("b", [0, 1])
def test_full_size_d512_causal_gqa(full_d512, b):
    full_d512.check_sequence(b)


@pytest.mark.parametrize("b", [0, 1])
def test_full_size_d256_sliding_window(window_d256, b):
    window_d256.check_sequence(b)


@pytest.mark.parametrize("b", list(range(8)))
def test_full_size_d512_varlen_pad_mask(varlen_d512, b):
    varlen_d512.check_sequence(b)
