"""Output canaries: every output of the C ABI written through views into larger buffers whose
remaining elements hold a sentinel bit pattern (guard bands before and after, and the gaps of
padded head and row strides), and workspaces followed by a sentinel region.  After each call
every sentinel must be unchanged (an out-of-bounds or wrongly strided write shows up here) and
the results must equal, bit for bit, those of the same call with plain contiguous outputs."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from synth import DECODE_WORKLOADS, AttnWorkload, lengths_to_pad_mask, make_attention_inputs, make_decode_inputs
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

import scaled_dot_product_tiled_amd as sdpt  # noqa: E402
from scaled_dot_product_tiled_amd.binding import AttnDecodeShape  # noqa: E402

SENT16 = 0x5A5A          # sentinel of 16-bit buffers
SENT32 = 0x7F5A5A5A      # sentinel of fp32 buffers (a NaN pattern: a write of any value changes it)
GUARD = 4096             # elements before and after each view


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Guarded:
    """A (rows..., D) view with a padded last stride and guard bands, in one sentinel buffer."""

    def __init__(self, shape, dtype, pad=0):
        *outer, d = shape
        self.full_shape = (*outer, d + pad)
        n = int(np.prod(self.full_shape))
        self.buf = torch.empty(n + 2 * GUARD, device="cuda:0", dtype=dtype)
        self.int_view().fill_(SENT32 if dtype == torch.float32 else SENT16)
        self.view = self.buf[GUARD:GUARD + n].view(self.full_shape)[..., :d]
        self.d, self.pad = d, pad

    def int_view(self):
        return self.buf.view(torch.int32 if self.buf.dtype == torch.float32 else torch.int16)

    def sentinels_intact(self) -> bool:
        a = self.int_view().cpu().numpy()
        want = SENT32 if self.buf.dtype == torch.float32 else SENT16
        n = a.size - 2 * GUARD
        ok = (a[:GUARD] == want).all() and (a[GUARD + n:] == want).all()
        if self.pad:
            mid = a[GUARD:GUARD + n].reshape(self.full_shape)
            ok = ok and (mid[..., self.d:] == want).all()
        return bool(ok)


def bits(t):
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


CASES = [
    ("d512_varlen_gqa", AttnWorkload(141, "canary d512 varlen", 2, 300, 8, 2, 512, varlen="pad_mask"), [300, 123]),
    ("d256_window", AttnWorkload(142, "canary d256 window", 1, 333, 4, 2, 256, window=100, qk_std=3.0), None),
]


@pytest.mark.parametrize("name,w,lengths", CASES, ids=[c[0] for c in CASES])
def test_fwd_bwd_outputs_stay_in_bounds(name, w, lengths):
    say(f"[canary {name}]")
    inp = make_attention_inputs(w, seed=0)
    q, k, v, do = (dev(inp[x]) for x in ("q", "k", "v", "do"))
    kw = dict(scale=w.scale, causal=w.causal, window=w.window)
    if lengths is not None:
        kw["pad_mask"] = torch.from_numpy(lengths_to_pad_mask(np.array(lengths), w.S)).to("cuda:0")
    o_ref, lse_ref = sdpt.attn_fwd(q, k, v, **kw)
    dq_ref, dk_ref, dv_ref = sdpt.attn_bwd(q, k, v, o_ref, lse_ref, do, **kw)
    o = Guarded(tuple(q.shape), torch.bfloat16, pad=64)
    lse = Guarded((w.B * w.Hq * w.S,), torch.float32)
    dq = Guarded(tuple(q.shape), torch.bfloat16, pad=32)
    dk = Guarded(tuple(k.shape), torch.bfloat16, pad=8)
    dv = Guarded(tuple(v.shape), torch.bfloat16)
    lse_v = lse.view.view(w.B, w.Hq, w.S)
    sdpt.attn_fwd(q, k, v, out=o.view, lse=lse_v, **kw)
    sdpt.attn_bwd(q, k, v, o.view, lse_v, do, dq=dq.view, dk=dk.view, dv=dv.view, **kw)
    torch.cuda.synchronize()
    for g, n in ((o, "o"), (lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert g.sentinels_intact(), n
    assert np.array_equal(bits(o.view), bits(o_ref)) and np.array_equal(bits(lse_v), bits(lse_ref))
    for g, r in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        assert np.array_equal(bits(g.view), bits(r))


def test_decode_and_chunk_workspaces_and_outputs_stay_in_bounds():
    w = DECODE_WORKLOADS["decode_d128"].scaled(B=6, ctx_range=(1, 1300))
    inp = make_decode_inputs(w, seed=4)
    say(f"[canary decode] ctx {inp['ctx_lens'].tolist()}")
    q, kc, vc = (dev(inp[x]) for x in ("q", "k_cache", "v_cache"))
    table = torch.from_numpy(inp["block_table"]).to("cuda:0")
    ctx = torch.from_numpy(inp["ctx_lens"]).to("cuda:0")
    ref = sdpt.paged_decode(q, kc, vc, table, ctx, scale=w.scale)
    out = Guarded(tuple(q.shape), torch.bfloat16, pad=16)
    ws = torch.full((1 << 22,), 0x5A, device="cuda:0", dtype=torch.uint8)  # larger than the call needs
    sdpt.paged_decode(q, kc, vc, table, ctx, scale=w.scale, out=out.view, workspace=ws)
    torch.cuda.synchronize()
    assert out.sentinels_intact()
    assert np.array_equal(bits(out.view), bits(ref))
    # the library is given (and may write) exactly the bytes it asked for
    shape = AttnDecodeShape(w.B, w.Hq, w.Hkv, w.D, w.page_size, kc.shape[0], table.shape[1], 0)
    nbytes = sdpt.load_library().paged_decode_workspace_bytes(ctypes.byref(shape))
    assert nbytes < ws.numel() and bool((ws[nbytes:] == 0x5A).all())

    # a chunk pair's backward with its workspace followed by sentinels
    cw = AttnWorkload(143, "canary chunk", 1, 400, 8, 2, 512)
    ci = make_attention_inputs(cw, seed=1)
    cq, ck, cv, cdo = (dev(ci[x]) for x in ("q", "k", "v", "do"))
    qs, ks = cq[:, 200:], ck[:, :200]
    vs, dos = cv[:, :200], cdo[:, 200:]
    o_p, l_p = sdpt.attn_fwd_chunk(qs, ks, vs, 200, 0, scale=cw.scale, out_dtype=torch.bfloat16)
    need = sdpt.attn_bwd_chunk_workspace_bytes(qs, ks, 200, 0)
    wsb = torch.full((need + (1 << 16),), 0x5A, device="cuda:0", dtype=torch.uint8)
    g = sdpt.attn_bwd_chunk(qs, ks, vs, o_p, l_p, dos, 200, 0, scale=cw.scale, workspace=wsb)
    torch.cuda.synchronize()
    assert bool((wsb[need:] == 0x5A).all())
    g_ref = sdpt.attn_bwd_chunk(qs, ks, vs, o_p, l_p, dos, 200, 0, scale=cw.scale)
    torch.cuda.synchronize()
    for a, b in zip(g, g_ref):
        assert np.array_equal(bits(a), bits(b))
