"""paged_decode_noalloc (the decode for callers that cannot allocate: the chunk partials live in
the library's fixed device array) against paged_decode with a caller workspace, through the C
ABI: the same bytes on two calls in a row, the second with a smaller batch and shorter contexts
(the array keeps the first call's partials, which the second must not read), and both within the
decode tolerance of the float64 oracle.  Runs alone in a fresh process or after the other tests."""
import numpy as np
import pytest
import torch

import oracle
from synth import DECODE_WORKLOADS, bf16_bits_to_f64, make_decode_inputs
from tests.gpu_util import O_MAX_ABS, all_finite, dev, host, host_bits, max_abs

pytestmark = pytest.mark.gpu

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402


def _inputs(w, seed):
    inp = make_decode_inputs(w, seed=seed)
    d = dict(q=dev(inp["q"]), kc=dev(inp["k_cache"]), vc=dev(inp["v_cache"]),
             table=torch.from_numpy(inp["block_table"]).to("cuda:0"),
             ctx=torch.from_numpy(inp["ctx_lens"]).to("cuda:0"))
    return inp, d


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    w = DECODE_WORKLOADS["decode_d128"]
    cases = [(w, 0), (w.scaled(B=5, ctx_range=(1, 700)), 1)]   # the second call is smaller
    for cw, seed in cases:
        print(f"[noalloc decode] B={cw.B} ctx {cw.ctx_range} seed {seed}", flush=True)
        inp, d = _inputs(cw, seed)
        ws_out = sdpt.paged_decode(d["q"], d["kc"], d["vc"], d["table"], d["ctx"], scale=cw.scale)
        na_out = torch.empty_like(d["q"])
        sdpt.binding.paged_decode_noalloc(d["q"], d["kc"], d["vc"], d["table"], d["ctx"], out=na_out,
                                          scale=cw.scale)
        torch.cuda.synchronize()
        assert all_finite(na_out)
        assert np.array_equal(host_bits(na_out), host_bits(ws_out))
        ref = oracle.paged_decode(bf16_bits_to_f64(inp["q"]), bf16_bits_to_f64(inp["k_cache"]),
                                  bf16_bits_to_f64(inp["v_cache"]), inp["block_table"], inp["ctx_lens"], cw.scale)
        assert max_abs(host(na_out), ref) <= O_MAX_ABS


def test_noalloc_decode_rejects_shapes_beyond_its_array():
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=4, ctx_range=(1, 64))
    _, d = _inputs(w, 2)
    big_table = torch.zeros((4, 1 << 16), device="cuda:0", dtype=torch.int32)   # 1M-token capacity
    out = torch.empty_like(d["q"])
    with pytest.raises(RuntimeError, match="status 3"):
        sdpt.binding.paged_decode_noalloc(d["q"], d["kc"], d["vc"], big_table, d["ctx"], out=out, scale=w.scale)
