"""GPU checks of debug mode (attn_debug): with it on, calls that take device-resident metadata
check it first and fail with an invalid-argument status, before launching their kernels, when
it is inconsistent; consistent metadata gives the same bits as with the checks off.

Every inconsistent case is one the kernels also survive with the checks off (lengths and
offsets are clamped, out-of-pool page ids skipped), so no case here can fault the GPU.
"""
import sys

import numpy as np
import pytest
import torch

from synth import (DECODE_WORKLOADS, PREFILL_WORKLOADS, AttnWorkload, lengths_to_pad_mask, make_attention_inputs,
                   make_decode_inputs, make_prefill_inputs)
from tests.gpu_util import dev, host_bits

pytestmark = pytest.mark.gpu

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture
def debug_on():
    prev = sdpt.debug(True)
    yield
    sdpt.debug(prev)


def _packed_inputs():
    w = AttnWorkload(401, "debug packed", 1, 300, 4, 2, 256)
    inp = make_attention_inputs(w, seed=0)
    q, k, v = (dev(inp[x])[0] for x in ("q", "k", "v"))   # (total, H, D)
    return w, q, k, v


GOOD_CU = [0, 100, 100, 300]
BAD_CU = {
    "decreasing": [0, 150, 100, 300],
    "short_total": [0, 100, 200, 290],
    "nonzero_start": [5, 100, 200, 300],
    "too_long": [0, 10, 20, 300],          # 280 rows > max_seqlen 200
}


def test_good_packed_metadata_passes_and_matches_unchecked(debug_on):
    w, q, k, v = _packed_inputs()
    cu = torch.tensor(GOOD_CU, dtype=torch.int32, device="cuda:0")
    say("[debug] good cu_seqlens")
    o1, l1 = sdpt.attn_fwd(q, k, v, scale=w.scale, cu_seqlens=cu, max_seqlen=200)
    sdpt.debug(False)
    o2, l2 = sdpt.attn_fwd(q, k, v, scale=w.scale, cu_seqlens=cu, max_seqlen=200)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert torch.equal(l1.cpu(), l2.cpu())


@pytest.mark.parametrize("name", list(BAD_CU))
def test_bad_cu_seqlens_is_rejected(debug_on, name):
    w, q, k, v = _packed_inputs()
    cu = torch.tensor(BAD_CU[name], dtype=torch.int32, device="cuda:0")
    say(f"[debug] cu_seqlens {name}")
    with pytest.raises(RuntimeError, match="status 1"):
        sdpt.attn_fwd(q, k, v, scale=w.scale, cu_seqlens=cu, max_seqlen=200)
    o, lse = sdpt.attn_fwd(q, k, v, scale=w.scale, cu_seqlens=torch.tensor(GOOD_CU, dtype=torch.int32,
                                                                              device="cuda:0"), max_seqlen=200)
    do = torch.ones_like(o)
    with pytest.raises(RuntimeError, match="status 1"):
        sdpt.attn_bwd(q, k, v, o, lse, do, scale=w.scale, cu_seqlens=cu, max_seqlen=200)
    torch.cuda.synchronize()


def test_non_prefix_pad_mask_is_rejected(debug_on):
    w = AttnWorkload(402, "debug mask", 2, 200, 4, 2, 256, varlen="pad_mask")
    inp = make_attention_inputs(w, seed=1)
    q, k, v = (dev(inp[x]) for x in ("q", "k", "v"))
    good = lengths_to_pad_mask(np.array([200, 77]), w.S)
    say("[debug] pad mask")
    sdpt.attn_fwd(q, k, v, scale=w.scale, pad_mask=torch.from_numpy(good).to("cuda:0"))
    bad = good.copy()
    bad[1, 100] = True                      # a valid entry after the padding starts
    with pytest.raises(RuntimeError, match="status 1"):
        sdpt.attn_fwd(q, k, v, scale=w.scale, pad_mask=torch.from_numpy(bad).to("cuda:0"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("fault", ["page_id", "negative_page", "ctx_too_long", "negative_ctx"])
def test_bad_page_metadata_is_rejected(debug_on, fault):
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=4, ctx_range=(10, 200))
    inp = make_decode_inputs(w, seed=2)
    q, kc, vc = (dev(inp[x]) for x in ("q", "k_cache", "v_cache"))
    table = inp["block_table"].copy()
    ctx = inp["ctx_lens"].copy()
    say(f"[debug] pages {fault}")
    t_d = torch.from_numpy(table).to("cuda:0")
    c_d = torch.from_numpy(ctx).to("cuda:0")
    ref = sdpt.paged_decode(q, kc, vc, t_d, c_d, scale=w.scale)
    if fault == "page_id":
        table[1, 0] = kc.shape[0]
    elif fault == "negative_page":
        table[2, (ctx[2] - 1) // w.page_size] = -1
    elif fault == "ctx_too_long":
        ctx[0] = table.shape[1] * w.page_size + 1
    else:
        ctx[3] = -1
    bt, bc = torch.from_numpy(table).to("cuda:0"), torch.from_numpy(ctx).to("cuda:0")
    out = ref.clone()
    with pytest.raises(RuntimeError, match="status 1"):
        sdpt.paged_decode(q, kc, vc, bt, bc, scale=w.scale, out=out)
    new = torch.zeros((w.B, 1, w.Hkv, w.D), device="cuda:0", dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="status 1"):
        sdpt.paged_kv_append(new, new, kc, vc, bt, bc)
    with pytest.raises(RuntimeError, match="status 1"):
        sdpt.paged_kv_gather(kc, vc, bt, bc, 8)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), host_bits(ref))   # nothing was launched


@pytest.mark.parametrize("fault", ["cu_decreasing", "cu_short_total", "page_id", "ctx_too_long"])
def test_bad_paged_forward_metadata_is_rejected(debug_on, fault):
    """attn_fwd_paged checks its query offsets and its pages before its one launch."""
    w = PREFILL_WORKLOADS["mixed_step_d512"].scaled(B=3, Hq=4, Hkv=2, D=256, ctx=(40, 20, 70), new=(10, 1, 30))
    inp = make_prefill_inputs(w, seed=3)
    q, kc, vc = (dev(inp[x]) for x in ("q", "k_cache", "v_cache"))
    table, ctx, cu = inp["block_table"].copy(), inp["ctx_lens"].copy(), inp["cu_q"].astype(np.int32)
    say(f"[debug] paged forward {fault}")

    def run(table, ctx, cu, out=None):
        return sdpt.attn_fwd_paged(q, kc, vc, torch.from_numpy(table).to("cuda:0"), torch.from_numpy(cu).to("cuda:0"),
                                   torch.from_numpy(ctx).to("cuda:0"), inp["max_q"], scale=w.scale, out=out)
    ref, _ = run(table, ctx, cu)
    if fault == "cu_decreasing":
        cu = cu.copy()
        cu[1], cu[2] = cu[2], cu[1]
    elif fault == "cu_short_total":
        cu = cu.copy()
        cu[-1] -= 1
    elif fault == "page_id":
        table[2, 1] = kc.shape[0]
    else:
        ctx[0] = table.shape[1] * w.page_size + 1
    out = ref.clone()
    with pytest.raises(RuntimeError, match="status 1"):
        run(table, ctx, cu, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), host_bits(ref))   # nothing was launched


def test_contiguous_pages_leaving_the_pool_are_rejected(debug_on):
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=3, ctx_range=(10, 60))
    inp = make_decode_inputs(w, seed=4)
    q, kc, vc = (dev(inp[x]) for x in ("q", "k_cache", "v_cache"))
    ctx = torch.from_numpy(inp["ctx_lens"]).to("cuda:0")
    pages = -(-inp["ctx_lens"].astype(np.int64) // 16)
    first = np.concatenate([[0], np.cumsum(pages)[:-1]]).astype(np.int32)
    say("[debug] contiguous first pages")
    mp = inp["block_table"].shape[1]
    ref = sdpt.paged_decode_contiguous(q, kc, vc, torch.from_numpy(first).to("cuda:0"), ctx, mp, scale=w.scale)
    bad = first.copy()
    bad[2] = kc.shape[0] - int(pages[2]) + 1          # its last page is past the pool
    out = ref.clone()
    with pytest.raises(RuntimeError, match="status 1"):
        sdpt.paged_decode_contiguous(q, kc, vc, torch.from_numpy(bad).to("cuda:0"), ctx, mp, scale=w.scale, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), host_bits(ref))
