"""Pins the oracle to facts that do not come from the oracle itself.

* a causal two-position example worked by hand (tests/golden/hand_worked_two_keys.json);
* closed forms: K = 0 makes every visible score 0, so LSE_i = ln(count_i) and O_i is the mean
  of the visible V rows; a single visible key returns that V row exactly; equal keys give the
  mean of the visible V rows for any Q;
* invariants: softmax rows sum to 1, grouped-query heads equal multi-head attention on
  repeated K/V (the repeat-KV path of the page "Gemma4 FFPA attention backend support for
  accelerating Gemma4-family training", Debugging notes), packed rows equal padded rows;
* central finite differences of L = sum(O * dO) for every gradient coordinate on tiny shapes;
* an independent library routine: torch's float64 CPU scaled_dot_product_attention with an
  explicit boolean mask and autograd, which shares nothing with the oracle;
* the paged decode equals causal attention's last row on the gathered tokens, and does not
  depend on which pool pages hold them;
* chunk pairs (ring context parallelism) merge, by log-sum-exp, to the full attention, and
  their gradient parts sum to the full gradients;
* the tanh softcap: central differences, torch autograd through explicit tanh / softmax
  tensor ops, and its limits (a huge cap is no cap; equal scores stay equal).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import (ATTN_WORKLOADS, DECODE_WORKLOADS, bf16_bits_to_f64,
                   lengths_to_cu_seqlens, lengths_to_pad_mask, make_attention_inputs,
                   make_decode_inputs, pack_rows)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        table = {"ln3": math.log(3), "2ln3": 2 * math.log(3), "ln4": math.log(4),
                 "-1.125ln3": -1.125 * math.log(3), "1.125ln3": 1.125 * math.log(3)}
        return table[x]
    return float(x)


def _arr(rows):
    return np.array([[_num(x) for x in r] if isinstance(r, list) else _num(r) for r in rows])


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# Worked by hand
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", [0, 1])
def test_hand_worked_two_keys(case):
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_two_keys.json")))
    c = g["cases"][case]
    q = _arr(c["q"])[None, :, None, :]
    k = _arr(g["k"])[None, :, None, :]
    v = _arr(g["v"])[None, :, None, :]
    do = _arr(g["do"])[None, :, None, :]
    e = g["expect"]
    o, lse = oracle.attention_forward(q, k, v, c["scale"], causal=True)
    np.testing.assert_allclose(o[0, :, 0], _arr(e["o"]), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], _arr(e["lse"]), atol=1e-14)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, c["scale"], causal=True)
    np.testing.assert_allclose(dq[0, :, 0], _arr(e["dq_scale1" if case == 0 else "dq_scale_half"]), atol=1e-14)
    np.testing.assert_allclose(dk[0, :, 0], _arr(e["dk"]), atol=1e-14)
    np.testing.assert_allclose(dv[0, :, 0], _arr(e["dv"]), atol=1e-14)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------
def _visible_count(i, n, causal, window):
    if i >= n:
        return 0
    lo = 0
    hi = i + 1 if causal else n
    if window > 0:
        lo = max(lo, i - window + 1)
    return hi - lo


@pytest.mark.parametrize("causal,window,lengths", [
    (True, 0, None), (True, 5, None), (False, 0, None), (True, 0, [11, 4]), (True, 3, [7, 11]),
])
def test_zero_keys_give_log_count(causal, window, lengths):
    rng = np.random.default_rng(1)
    B, S, Hq, Hkv, D = 2, 11, 4, 2, 8
    q = _rand(rng, B, S, Hq, D)
    k = np.zeros((B, S, Hkv, D))
    v = _rand(rng, B, S, Hkv, D)
    o, lse = oracle.attention_forward(q, k, v, 0.3, causal, window, lengths)
    L = [S] * B if lengths is None else lengths
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                cnt = _visible_count(i, L[b], causal, window)
                if cnt == 0:
                    assert lse[b, h, i] == 0.0 and not o[b, i, h].any()
                    continue
                assert abs(lse[b, h, i] - math.log(cnt)) < 1e-13
                hi = i + 1 if causal else L[b]
                lo = hi - cnt
                np.testing.assert_allclose(o[b, i, h], v[b, lo:hi, h // 2].mean(axis=0), atol=1e-13)


def test_equal_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(2)
    B, S, H, D = 1, 9, 2, 6
    q = _rand(rng, B, S, H, D) * 3
    k = np.broadcast_to(_rand(rng, 1, 1, H, D), (B, S, H, D)).copy()
    v = _rand(rng, B, S, H, D)
    o, _ = oracle.attention_forward(q, k, v, 0.7, causal=True, window=4)
    for i in range(S):
        lo = max(0, i - 3)
        np.testing.assert_allclose(o[0, i], v[0, lo:i + 1].mean(axis=0), atol=1e-13)


def test_single_visible_key_returns_value_row_exactly():
    rng = np.random.default_rng(3)
    q = _rand(rng, 1, 6, 2, 4)
    k = _rand(rng, 1, 6, 1, 4)
    v = _rand(rng, 1, 6, 1, 4)
    o, _ = oracle.attention_forward(q, k, v, 0.5, causal=True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0]) and np.array_equal(o[0, 0, 1], v[0, 0, 0])
    o, _ = oracle.attention_forward(q, k, v, 0.5, causal=True, window=1)   # window 1: only the diagonal
    assert np.array_equal(o[0, :, 0], v[0, :, 0])


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------
def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(4)
    n = 33
    for causal, window in [(True, 0), (True, 7), (False, 0)]:
        _, _, p = oracle.unit_forward(_rand(rng, n, 16) * 3, _rand(rng, n, 16) * 3, _rand(rng, n, 16), 0.25,
                                      oracle.visibility(n, causal, window))
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
        assert (p >= 0).all()
        assert not p[~oracle.visibility(n, causal, window)].any()


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(5)
    B, S, Hq, Hkv, D = 2, 10, 6, 2, 8
    q, do = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hq, D)
    k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    kr, vr = np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2)
    lengths = [10, 6]
    o1, l1 = oracle.attention_forward(q, k, v, 0.3, True, 4, lengths)
    o2, l2 = oracle.attention_forward(q, kr, vr, 0.3, True, 4, lengths)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    g1 = oracle.attention_backward(q, k, v, do, 0.3, True, 4, lengths)
    g2 = oracle.attention_backward(q, kr, vr, do, 0.3, True, 4, lengths)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-12)
    for a, b in ((g1[1], g2[1]), (g1[2], g2[2])):
        np.testing.assert_allclose(a, b.reshape(B, S, Hkv, Hq // Hkv, D).sum(axis=3), atol=1e-12)


def test_packed_rows_equal_padded_rows():
    rng = np.random.default_rng(6)
    B, S, Hq, Hkv, D = 3, 12, 4, 2, 8
    lengths = np.array([12, 5, 9])
    q, do = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hq, D)
    k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    cu = lengths_to_cu_seqlens(lengths)
    o, lse = oracle.attention_forward(q, k, v, 0.4, True, 0, lengths)
    op, lsep = oracle.attention_forward_packed(pack_rows(q, lengths), pack_rows(k, lengths),
                                               pack_rows(v, lengths), cu, 0.4, True, 0)
    np.testing.assert_allclose(op, pack_rows(o, lengths), atol=1e-13)
    np.testing.assert_allclose(lsep, pack_rows(lse.transpose(0, 2, 1), lengths).T, atol=1e-13)
    g = oracle.attention_backward(q, k, v, do, 0.4, True, 0, lengths)
    gp = oracle.attention_backward_packed(pack_rows(q, lengths), pack_rows(k, lengths), pack_rows(v, lengths),
                                          pack_rows(do, lengths), cu, 0.4, True, 0)
    for a, b in zip(gp, g):
        np.testing.assert_allclose(a, pack_rows(b, lengths), atol=1e-12)
    # padded rows and keys are exactly zero
    for t in (o, *g):
        for b in range(B):
            assert not t[b, lengths[b]:].any()


def test_padding_values_never_reach_valid_outputs():
    rng = np.random.default_rng(7)
    B, S, Hq, Hkv, D = 2, 9, 2, 1, 4
    lengths = [9, 5]
    q, do = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hq, D)
    k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    ref = oracle.attention_forward(q, k, v, 0.5, True, 0, lengths), \
        oracle.attention_backward(q, k, v, do, 0.5, True, 0, lengths)
    for t in (q, k, v, do):
        t[1, 5:] = np.nan
    got = oracle.attention_forward(q, k, v, 0.5, True, 0, lengths), \
        oracle.attention_backward(q, k, v, do, 0.5, True, 0, lengths)
    for a, b in zip(ref[0] + ref[1], got[0] + got[1]):
        assert np.array_equal(a, b)


def test_pad_mask_lengths_and_rejection():
    m = lengths_to_pad_mask(np.array([3, 0, 5]), 5)
    assert list(oracle.lengths_from_pad_mask(m)) == [3, 0, 5]
    bad = m.copy()
    bad[0, 4] = 1
    with pytest.raises(ValueError):
        oracle.lengths_from_pad_mask(bad)
    assert list(oracle.lengths_from_cu_seqlens(np.array([0, 3, 3, 8]))) == [3, 0, 5]


# ---------------------------------------------------------------------------
# Finite differences: every coordinate of dQ, dK, dV
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("softcap", [0.0, 1.3])
def test_gradients_match_central_differences(softcap):
    rng = np.random.default_rng(8)
    B, S, Hq, Hkv, D = 2, 9, 4, 2, 8
    lengths = [9, 5]
    scale, causal, window = 0.37, True, 3
    q, do = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hq, D)
    k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    if softcap:
        q *= 2.0                            # scores of a few units: the cap bends them

    def loss(q_, k_, v_):
        o, _ = oracle.attention_forward(q_, k_, v_, scale, causal, window, lengths, softcap)
        return float((o * do).sum())

    grads = oracle.attention_backward(q, k, v, do, scale, causal, window, lengths, softcap)
    eps = 1e-6
    for which, g in enumerate(grads):
        base = [q, k, v]
        num = np.zeros_like(g)
        t = base[which]
        for idx in np.ndindex(*t.shape):
            keep = t[idx]
            t[idx] = keep + eps
            lp = loss(*base)
            t[idx] = keep - eps
            lm = loss(*base)
            t[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-6, (which, err)


# ---------------------------------------------------------------------------
# Independent library routine: torch float64 CPU SDPA + autograd
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal,window,lengths,Hq,Hkv,D", [
    (True, 0, None, 4, 1, 64),
    (True, 16, None, 4, 2, 32),
    (True, 0, [40, 17, 1], 8, 2, 16),
    (False, 0, [40, 23, 8], 2, 2, 16),
])
def test_matches_torch_float64_sdpa(causal, window, lengths, Hq, Hkv, D):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(9)
    B, S = (3 if lengths else 2), 40
    scale = 1.0 / math.sqrt(D)
    q, do = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hq, D)
    k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    L = [S] * B if lengths is None else lengths
    o, lse = oracle.attention_forward(q, k, v, scale, causal, window, lengths)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal, window, lengths)

    mask = np.zeros((B, 1, S, S), dtype=bool)
    dmask = do.copy()
    for b in range(B):
        n = L[b]
        mask[b, 0, :n, :n] = oracle_free_visibility(n, causal, window)
        mask[b, 0, n:, 0] = True           # padded query rows: any finite row, then zero its dO
        dmask[b, n:] = 0.0
    tq = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)
    r = Hq // Hkv
    tk = torch.tensor(np.repeat(k, r, axis=2).transpose(0, 2, 1, 3), requires_grad=True)
    tv = torch.tensor(np.repeat(v, r, axis=2).transpose(0, 2, 1, 3), requires_grad=True)
    to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(mask), scale=scale)
    to.backward(torch.tensor(dmask.transpose(0, 2, 1, 3)))
    t_o = to.detach().numpy().transpose(0, 2, 1, 3)
    t_dq = tq.grad.numpy().transpose(0, 2, 1, 3)
    t_dk = tk.grad.numpy().transpose(0, 2, 1, 3).reshape(B, S, Hkv, r, D).sum(axis=3)
    t_dv = tv.grad.numpy().transpose(0, 2, 1, 3).reshape(B, S, Hkv, r, D).sum(axis=3)
    for b in range(B):
        n = L[b]
        np.testing.assert_allclose(o[b, :n], t_o[b, :n], atol=1e-12)
        np.testing.assert_allclose(dq[b, :n], t_dq[b, :n], atol=1e-12)
        np.testing.assert_allclose(dk[b, :n], t_dk[b, :n], atol=1e-12)
        np.testing.assert_allclose(dv[b, :n], t_dv[b, :n], atol=1e-12)
        # LSE against a direct log-sum-exp of torch-computed scores
        s = torch.einsum("hid,hjd->hij", torch.tensor(q[b, :n].transpose(1, 0, 2)),
                         torch.tensor(np.repeat(k[b, :n], r, axis=1).transpose(1, 0, 2))) * scale
        s = s.masked_fill(~torch.tensor(mask[b, 0, :n, :n]), float("-inf"))
        np.testing.assert_allclose(lse[b, :, :n], torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal,window,lengths,softcap", [
    (True, 0, None, 2.0),
    (True, 9, [40, 13], 0.7),
    (False, 0, [40, 31], 5.0),
])
def test_softcap_matches_torch_autograd(causal, window, lengths, softcap):
    """Soft-capped attention written with torch's float64 CPU tensor ops (tanh, masked softmax,
    matmul) and differentiated by torch's autograd: a second, independent route to the same
    numbers.  Masked entries are excluded after the cap, so tanh never sees -inf."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    B, S, Hq, Hkv, D = 2, 40, 4, 2, 16
    scale = 1.0 / math.sqrt(D)
    q, do = 3.0 * _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hq, D)
    k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    L = [S] * B if lengths is None else lengths
    o, lse = oracle.attention_forward(q, k, v, scale, causal, window, lengths, softcap)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal, window, lengths, softcap)
    r = Hq // Hkv
    for b in range(B):
        n = L[b]
        vis = torch.tensor(oracle_free_visibility(n, causal, window))
        tq = torch.tensor(q[b, :n].transpose(1, 0, 2), requires_grad=True)
        tk = torch.tensor(k[b, :n].transpose(1, 0, 2), requires_grad=True)
        tv = torch.tensor(v[b, :n].transpose(1, 0, 2), requires_grad=True)
        kk = tk.repeat_interleave(r, dim=0)
        vv = tv.repeat_interleave(r, dim=0)
        sc = softcap * torch.tanh(scale * torch.matmul(tq, kk.transpose(1, 2)) / softcap)
        sc = sc.masked_fill(~vis, float("-inf"))
        to = torch.matmul(torch.softmax(sc, dim=-1), vv)
        to.backward(torch.tensor(do[b, :n].transpose(1, 0, 2)))
        np.testing.assert_allclose(o[b, :n], to.detach().numpy().transpose(1, 0, 2), atol=1e-12)
        np.testing.assert_allclose(lse[b, :, :n], torch.logsumexp(sc, dim=-1).detach().numpy(), atol=1e-12)
        np.testing.assert_allclose(dq[b, :n], tq.grad.numpy().transpose(1, 0, 2), atol=1e-12)
        np.testing.assert_allclose(dk[b, :n], tk.grad.numpy().transpose(1, 0, 2), atol=1e-12)
        np.testing.assert_allclose(dv[b, :n], tv.grad.numpy().transpose(1, 0, 2), atol=1e-12)


def test_softcap_limits():
    """A cap far above every score changes nothing (tanh(x) = x + O(x^3)); equal scores stay
    equal under the cap, so K = 0 still gives LSE = ln(visible count)."""
    rng = np.random.default_rng(22)
    B, S, Hq, Hkv, D = 1, 17, 2, 1, 8
    q, k, v, do = (_rand(rng, B, S, h, D) for h in (Hq, Hkv, Hkv, Hq))
    plain = oracle.attention_forward(q, k, v, 0.4, True, 5) + oracle.attention_backward(q, k, v, do, 0.4, True, 5)
    capped = (oracle.attention_forward(q, k, v, 0.4, True, 5, None, 1e7)
              + oracle.attention_backward(q, k, v, do, 0.4, True, 5, None, 1e7))
    for a, b in zip(plain, capped):
        np.testing.assert_allclose(a, b, atol=1e-10)
    _, lse = oracle.attention_forward(q, np.zeros_like(k), v, 0.4, True, 5, None, 0.3)
    cnt = np.minimum(np.arange(S) + 1, 5)
    np.testing.assert_allclose(lse[0], np.broadcast_to(np.log(cnt), (Hq, S)), atol=1e-14)


def oracle_free_visibility(n, causal, window):
    """The mask for the torch cross-check, built without the oracle."""
    m = np.ones((n, n), dtype=bool)
    if causal:
        m = np.tril(m)
    if window > 0:
        m &= ~np.tril(np.ones((n, n), dtype=bool), -window)
    return m


# ---------------------------------------------------------------------------
# Paged decode
# ---------------------------------------------------------------------------
def test_decode_is_last_row_of_causal_attention_and_table_independent():
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=4, ctx_range=(1, 70))
    inp = make_decode_inputs(w, seed=3, ctx_lens=np.array([1, 16, 17, 70], dtype=np.int32))
    q = bf16_bits_to_f64(inp["q"])
    kc, vc = bf16_bits_to_f64(inp["k_cache"]), bf16_bits_to_f64(inp["v_cache"])
    table, ctx = inp["block_table"], inp["ctx_lens"]
    o = oracle.paged_decode(q, kc, vc, table, ctx, w.scale, w.page_size)
    for b in range(w.B):
        n = int(ctx[b])
        kk = np.stack([kc[table[b, t // 16], t % 16] for t in range(n)])[None]
        vv = np.stack([vc[table[b, t // 16], t % 16] for t in range(n)])[None]
        qq = np.zeros((1, n, w.Hq, w.D))
        qq[0, n - 1] = q[b]
        od, _ = oracle.attention_forward(qq, kk, vv, w.scale, causal=True)
        np.testing.assert_allclose(o[b], od[0, n - 1], atol=1e-13)
    # a different physical placement of the same logical tokens gives identical bytes
    perm = np.random.default_rng(0).permutation(inp["num_pages"])
    inv = np.argsort(perm)
    kc2, vc2 = kc[inv], vc[inv]                 # page p moves to slot perm[p]
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2 = oracle.paged_decode(q, kc2, vc2, table2, ctx, w.scale, w.page_size)
    assert np.array_equal(o, o2)


def test_decode_matches_torch_sdpa_and_ignores_unused_pages():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=3, ctx_range=(20, 90))
    inp = make_decode_inputs(w, seed=5)
    pois = make_decode_inputs(w, seed=5, poison_unused=True)
    args = [bf16_bits_to_f64(inp[x]) for x in ("q", "k_cache", "v_cache")]
    o = oracle.paged_decode(*args, inp["block_table"], inp["ctx_lens"], w.scale)
    argsp = [bf16_bits_to_f64(pois[x]) for x in ("q", "k_cache", "v_cache")]
    op = oracle.paged_decode(*argsp, pois["block_table"], pois["ctx_lens"], w.scale)
    assert np.array_equal(o, op) and np.isfinite(o).all()
    r = w.Hq // w.Hkv
    for b in range(w.B):
        n = int(inp["ctx_lens"][b])
        tok = np.arange(n)
        kk = args[1][inp["block_table"][b][tok // 16], tok % 16]
        vv = args[2][inp["block_table"][b][tok // 16], tok % 16]
        tq = torch.tensor(args[0][b][:, None, :])                        # (Hq, 1, D)
        tk = torch.tensor(np.repeat(kk, r, axis=1).transpose(1, 0, 2))   # (Hq, n, D)
        tv = torch.tensor(np.repeat(vv, r, axis=1).transpose(1, 0, 2))
        ref = F.scaled_dot_product_attention(tq, tk, tv, scale=w.scale).numpy()[:, 0]
        np.testing.assert_allclose(o[b], ref, atol=1e-12)
    ctx0 = oracle.paged_decode(*args, inp["block_table"], np.zeros(w.B, dtype=np.int32), w.scale)
    assert not ctx0.any()


# ---------------------------------------------------------------------------
# Oracle on the generated workloads (small slices): finite everywhere
# ---------------------------------------------------------------------------
def test_oracle_finite_on_peaked_window_workload_slice():
    w = ATTN_WORKLOADS["window_d256"].scaled(B=1, S=300, Hq=2, Hkv=1, window=64)
    inp = make_attention_inputs(w, seed=0)
    q, k, v, do = (bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    o, lse = oracle.attention_forward(q, k, v, w.scale, True, w.window)
    g = oracle.attention_backward(q, k, v, do, w.scale, True, w.window)
    for t in (o, lse, *g):
        assert np.isfinite(t).all()


def test_row_sampled_oracle_equals_full_unit():
    rng = np.random.default_rng(10)
    B, S, Hq, Hkv, D = 2, 30, 4, 2, 8
    q, do = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hq, D)
    k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    lengths = [30, 17]
    o, lse = oracle.attention_forward(q, k, v, 0.4, True, 5, lengths)
    dq, _, _ = oracle.attention_backward(q, k, v, do, 0.4, True, 5, lengths)
    rows = [0, 3, 16, 17, 29]
    for b in range(B):
        for h in range(Hq):
            ro, rl, rdq = oracle.attention_rows(q, k, v, do, b, h, rows, 0.4, True, 5, lengths)
            np.testing.assert_allclose(ro, o[b, rows, h], atol=1e-13)
            np.testing.assert_allclose(rl, lse[b, h, rows], atol=1e-13)
            np.testing.assert_allclose(rdq, dq[b, rows, h], atol=1e-13)


def test_group_evaluation_equals_forward_and_backward():
    """attention_group (one softmax evaluation per head for the forward and the backward of a
    (batch, kv head) unit, used by the full-size GPU comparisons) returns exactly what the pinned
    attention_forward and attention_backward return for that unit."""
    rng = np.random.default_rng(11)
    B, S, Hq, Hkv, D = 2, 30, 6, 2, 8
    q, do = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hq, D)
    k, v = _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    lengths = [30, 17]
    o, lse = oracle.attention_forward(q, k, v, 0.4, True, 5, lengths)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.4, True, 5, lengths)
    r = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            go, gl, gq, gk, gv = oracle.attention_group(q, k, v, do, b, g, 0.4, True, 5, lengths)
            hs = slice(g * r, (g + 1) * r)
            np.testing.assert_array_equal(go, o[b, :, hs])
            np.testing.assert_array_equal(gl, lse[b, hs])
            np.testing.assert_array_equal(gq, dq[b, :, hs])
            np.testing.assert_array_equal(gk, dk[b, :, g])
            np.testing.assert_array_equal(gv, dv[b, :, g])


# ---------------------------------------------------------------------------
# Chunks of a sequence (ring context parallelism): pinned to the full oracle by the
# decomposition identity -- a row's attention over all keys is the log-sum-exp merge of its
# attention over disjoint key chunks, and the gradients are sums of per-chunk-pair parts.
# ---------------------------------------------------------------------------
def _chunk_inputs(seed, B=2, S=24, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, S, H, D)) for H in (Hq, Hkv, Hkv, Hq))
    return q, k, v, do


@pytest.mark.parametrize("causal,window,C", [(True, 0, 8), (True, 5, 8), (False, 0, 6), (True, 11, 6)])
def test_chunked_forward_merges_to_full_attention(causal, window, C):
    q, k, v, _ = _chunk_inputs(1)
    S = q.shape[1]
    scale = 0.37
    fo, fl = oracle.attention_forward(q, k, v, scale, causal, window)
    for q0 in range(0, S, C):
        o = np.zeros_like(q[:, q0:q0 + C])
        lse = np.full((q.shape[0], q.shape[2], C), -np.inf)
        for k0 in range(0, S, C):   # every key chunk, fully masked ones included
            po, pl = oracle.attention_forward_chunk(q[:, q0:q0 + C], k[:, k0:k0 + C], v[:, k0:k0 + C], scale,
                                                    causal, window, q0, k0)
            o, lse = oracle.lse_merge(o, lse, po, pl)
        np.testing.assert_allclose(o, fo[:, q0:q0 + C], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, fl[:, :, q0:q0 + C], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,window,C", [(True, 0, 8), (True, 7, 12), (False, 0, 8)])
def test_chunked_backward_sums_to_full_gradients(causal, window, C):
    q, k, v, do = _chunk_inputs(2)
    S = q.shape[1]
    scale = 0.29
    fo, fl = oracle.attention_forward(q, k, v, scale, causal, window)
    fq, fk, fv = oracle.attention_backward(q, k, v, do, scale, causal, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for q0 in range(0, S, C):
        for k0 in range(0, S, C):
            a, b_, c_ = oracle.attention_backward_chunk(q[:, q0:q0 + C], k[:, k0:k0 + C], v[:, k0:k0 + C],
                                                        fo[:, q0:q0 + C], fl[:, :, q0:q0 + C], do[:, q0:q0 + C],
                                                        scale, causal, window, q0, k0)
            dq[:, q0:q0 + C] += a
            dk[:, k0:k0 + C] += b_
            dv[:, k0:k0 + C] += c_
    for got, ref in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


def test_chunk_rows_without_keys_and_merge_identity():
    q, k, v, _ = _chunk_inputs(3, S=8)
    # a key chunk entirely after the query chunk: causal rows see nothing of it
    o, lse = oracle.attention_forward_chunk(q, k, v, 0.5, True, 0, 0, 8)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    # merging with that empty partial returns the other partial unchanged
    po, pl = oracle.attention_forward_chunk(q, k, v, 0.5, True, 0, 0, 0)
    mo, ml = oracle.lse_merge(po, pl, o, lse)
    np.testing.assert_array_equal(mo, po)
    np.testing.assert_array_equal(ml, pl)
    # the merge is symmetric and agrees with the closed form for two keys, one per chunk
    s1, s2 = 0.3, -1.1
    oa = np.full((1, 1, 1, 1), 2.0)
    ob = np.full((1, 1, 1, 1), -5.0)
    mo, ml = oracle.lse_merge(oa, np.full((1, 1, 1), s1), ob, np.full((1, 1, 1), s2))
    mo2, ml2 = oracle.lse_merge(ob, np.full((1, 1, 1), s2), oa, np.full((1, 1, 1), s1))
    w1 = math.exp(s1) / (math.exp(s1) + math.exp(s2))
    assert abs(float(mo[0, 0, 0, 0]) - (2.0 * w1 - 5.0 * (1 - w1))) < 1e-14
    assert abs(float(ml[0, 0, 0]) - math.log(math.exp(s1) + math.exp(s2))) < 1e-14
    assert np.array_equal(mo, mo2) and np.array_equal(ml, ml2)


# ---------------------------------------------------------------------------
# Paged cache append: a hand-placed example and the gather round trip
# ---------------------------------------------------------------------------
def test_paged_append_hand_example():
    # page_size 2; sequence 0 uses pages 3, 1 and holds 3 tokens after the append (its new
    # token lands at position 2: page 1, slot 0); sequence 1 uses pages 0, 2 and holds 1 token
    # (position 0: page 0, slot 0); a third sequence with a -1 entry is skipped
    cache = np.zeros((4, 2, 1, 1))
    table = np.array([[3, 1], [0, 2], [-1, -1]], dtype=np.int32)
    new = np.array([[[[7.0]]], [[[9.0]]], [[[5.0]]]])
    out = oracle.paged_append(cache, table, np.array([3, 1, 1]), new, page_size=2)
    expect = np.zeros((4, 2, 1, 1))
    expect[1, 0] = 7.0
    expect[0, 0] = 9.0
    assert np.array_equal(out, expect)
    assert not cache.any()                       # the input is not modified


def test_paged_append_then_gather_round_trip():
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=5, ctx_range=(3, 90), Hkv=2)
    inp = make_decode_inputs(w, seed=6)
    ctx0 = inp["ctx_lens"]
    n = 3
    ctx1 = ctx0 + n
    table = inp["block_table"]
    rng = np.random.default_rng(7)
    new = rng.standard_normal((w.B, n, w.Hkv, w.D))
    kc = bf16_bits_to_f64(inp["k_cache"])
    # room for the appended tokens: extend each table row with fresh pool pages where needed
    pages_needed = -(-ctx1 // w.page_size)
    used = set(table[table >= 0].tolist())
    free = [p for p in range(kc.shape[0]) if p not in used]
    table = np.concatenate([table, np.full((w.B, 2), -1, dtype=np.int32)], axis=1)
    for b in range(w.B):
        for p in range(int(pages_needed[b])):
            if table[b, p] < 0:
                if not free:
                    kc = np.concatenate([kc, np.zeros((1,) + kc.shape[1:])])
                    free.append(kc.shape[0] - 1)
                table[b, p] = free.pop()
    out = oracle.paged_append(kc, table, ctx1, new, w.page_size)
    for b in range(w.B):
        g = oracle.gather_pages(out, table[b], ctx1[b], w.page_size)
        assert np.array_equal(g[ctx0[b]:], new[b])                       # the appended tokens
        assert np.array_equal(g[:ctx0[b]], oracle.gather_pages(kc, table[b], ctx0[b], w.page_size))
    touched = np.zeros(kc.shape[:2], dtype=bool)
    for b in range(w.B):
        for t in range(int(ctx0[b]), int(ctx1[b])):
            touched[table[b, t // w.page_size], t % w.page_size] = True
    assert np.array_equal(out[~touched], kc[~touched])                    # nothing else changed


def test_decode_softcap_is_last_row_of_capped_causal_attention():
    """The capped decode equals the last row of capped causal attention over the gathered tokens
    (the same pin as the uncapped decode, with the cap)."""
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=3, Hq=4, Hkv=2, ctx_range=(1, 40))
    inp = make_decode_inputs(w, seed=12)
    q = 3.0 * bf16_bits_to_f64(inp["q"])
    kc, vc = bf16_bits_to_f64(inp["k_cache"]), bf16_bits_to_f64(inp["v_cache"])
    o = oracle.paged_decode(q, kc, vc, inp["block_table"], inp["ctx_lens"], w.scale, w.page_size, 2.0)
    for b in range(w.B):
        n = int(inp["ctx_lens"][b])
        kk = oracle.gather_pages(kc, inp["block_table"][b], n, w.page_size)[None]
        vv = oracle.gather_pages(vc, inp["block_table"][b], n, w.page_size)[None]
        qq = np.zeros((1, n, w.Hq, w.D))
        qq[0, n - 1] = q[b]
        full, _ = oracle.attention_forward(qq, kk, vv, w.scale, True, 0, None, 2.0)
        np.testing.assert_allclose(o[b], full[0, n - 1], atol=1e-13)


# ---------------------------------------------------------------------------
# Paged prefill: the new rows of several sequences against their paged caches
# ---------------------------------------------------------------------------
def _paged_sequences(rng, ctx, Hkv, D, ps, pool, maxp):
    """Each sequence's tokens written into pages of a permuted pool with paged_append (pinned by
    its hand example); returns the caches, the table and the dense tokens."""
    B = len(ctx)
    perm = rng.permutation(pool)
    table = np.full((B, maxp), -1, np.int32)
    off = 0
    for b in range(B):
        n = -(-int(ctx[b]) // ps)
        table[b, :n] = perm[off:off + n]
        off += n
    kc = rng.standard_normal((pool, ps, Hkv, D))         # unused slots hold other values
    vc = rng.standard_normal((pool, ps, Hkv, D))
    toks_k = [rng.standard_normal((int(c), Hkv, D)) for c in ctx]
    toks_v = [rng.standard_normal((int(c), Hkv, D)) for c in ctx]
    for b in range(B):
        if ctx[b] > 0:
            kc = oracle.paged_append(kc, table[b:b + 1], ctx[b:b + 1], toks_k[b][None], ps)
            vc = oracle.paged_append(vc, table[b:b + 1], ctx[b:b + 1], toks_v[b][None], ps)
    return kc, vc, table, toks_k, toks_v


@pytest.mark.parametrize("window,softcap", [(0, 0.0), (7, 0.0), (0, 2.0)])
def test_paged_prefill_rows_are_last_rows_of_causal_attention(window, softcap):
    """A sequence's n new rows equal the last n rows of whole-sequence causal attention
    (attention_forward, pinned against torch's float64 SDPA) over its ctx tokens, whatever the
    page placement; decode rows (n = 1) equal paged_decode; rows at negative positions (n > ctx)
    see nothing and the others are the sequence's causal rows."""
    rng = np.random.default_rng(21)
    Hq, Hkv, D, ps, pool, maxp = 4, 2, 8, 4, 40, 5
    ctx = np.array([9, 1, 12, 5, 6, 2, 0], dtype=np.int32)
    new = np.array([3, 1, 12, 1, 0, 4, 2])
    kc, vc, table, tk, tv = _paged_sequences(rng, ctx, Hkv, D, ps, pool, maxp)
    cu = np.concatenate([[0], np.cumsum(new)])
    q = 2.0 * rng.standard_normal((int(cu[-1]), Hq, D))
    scale = 0.4
    o, lse = oracle.paged_prefill(q, kc, vc, table, cu, ctx, scale, window, ps, softcap)
    for b in range(len(ctx)):
        lo, hi, n, c = int(cu[b]), int(cu[b + 1]), int(new[b]), int(ctx[b])
        if n == 0:
            continue
        neg = max(n - c, 0)                       # rows before position 0
        assert not o[lo:lo + neg].any() and not lse[:, lo:lo + neg].any()
        if c == 0:
            continue
        qf = np.zeros((1, c, Hq, D))
        qf[0, c - (n - neg):] = q[lo + neg:hi]
        full, fl = oracle.attention_forward(qf, tk[b][None], tv[b][None], scale, True, window, None, softcap)
        np.testing.assert_allclose(o[lo + neg:hi], full[0, c - (n - neg):], atol=1e-13)
        np.testing.assert_allclose(lse[:, lo + neg:hi], fl[0, :, c - (n - neg):], atol=1e-13)
        if n == 1 and window == 0:
            qd = np.zeros((len(ctx), Hq, D))
            qd[b] = q[lo]
            od = oracle.paged_decode_one(qd, kc, vc, table, ctx, scale, b, ps, softcap)
            np.testing.assert_allclose(o[lo], od, atol=1e-13)
    # another placement of the same tokens gives the same bytes
    kc2, vc2, table2, _, _ = _paged_sequences(np.random.default_rng(21), ctx, Hkv, D, ps, pool, maxp)
    perm = np.random.default_rng(5).permutation(pool)
    inv = np.argsort(perm)
    table3 = np.where(table2 >= 0, perm[np.maximum(table2, 0)], -1)
    o3, lse3 = oracle.paged_prefill(q, kc2[inv], vc2[inv], table3, cu, ctx, scale, window, ps, softcap)
    assert np.array_equal(o3, o) and np.array_equal(lse3, lse)
