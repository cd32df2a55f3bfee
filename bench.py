"""Benchmark of the fused attention hot path on one MI355X.

A step is one forward + backward of causal grouped-query attention, head_dim 512 (B=2, S=4096,
Hq=32, Hkv=4, bf16, seeded N(0,1) inputs already resident in HBM): attn_fwd then attn_bwd through
the C ABI.  Reported:
  value     causal-counted TFLOP/s of the step: forward 4 D pairs, backward 2.5x that, where pairs =
            visible (query, key) pairs summed over batch and heads (exact, not S^2/2);
  roofline  for the dominant kernel, timed with HIP events on the stream it runs on;
  decode    paged single-token decode (B=64, Hq=32, Hkv=8, D=128, 16-token pages, contexts
            U{512..4096}, pages permuted over a 1.5x pool) as achieved HBM GB/s of the algorithmic
            bytes, rotating over two KV pools so the 256 MB last-level cache cannot serve repeats;
            pages_in_order is the same decode with each sequence's pages consecutive in the pool;
  other_workloads  (median of per-call HIP-event timings) forward / backward TFLOP/s of the sliding-window (D=256, W=1024) and padded
            varlen (B=8, lengths U{512..8192}, D=512) workloads, of one context-parallel rank's
            chunk pairs (16k tokens in 8 chunks, D=512) and of the step's workload in IEEE half,
            not part of the timed step;
  cpu_baseline  the float64 oracle on a bounded sample of the same workload on the host cores.
Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E

# HBM traffic records (rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch, scaled by a plain copy)
# of each kernel on this workload; a record counts only while its kernel source is unchanged.
TRAFFIC = {
    "attn_fwd": ("profiles/attn_fwd_d512_B2_S4096_traffic.txt", "fwd_kernel<512,32,false,false,false>"),
    "bwd_dkdv": ("profiles/bwd_dkdv_d512_B2_S4096_traffic.txt", "bwd_dkdv_kernel<512,false,false>"),
    "bwd_dq": ("profiles/bwd_dq_d512_B2_S4096_traffic.txt", "bwd_dq_kernel<256,4,2,false>"),
    "decode_split": ("profiles/decode_split_d128_B64_traffic.txt", "decode_split_kernel<4,false,false>"),
}


def traffic_bytes(kernel):
    from scaled_dot_product_tiled_amd.profiling import read_traffic
    if kernel not in TRAFFIC:
        return None
    path, name = TRAFFIC[kernel]
    rec = read_traffic(os.path.join(ROOT, path), name)
    return None if rec is None else rec["bytes"]


def causal_pairs(S, window=0):
    i = np.arange(S, dtype=np.int64)
    cnt = i + 1 if window <= 0 else np.minimum(i + 1, window)
    return int(cnt.sum())


def other_workload(name, steps, stream, softcap=0.0, **changes):
    """Forward and backward times of the sliding-window and padded-varlen workloads, or of a workload
    with some fields changed (device-side seeded draws of the same shapes and distributions;
    lengths and masks from synth)."""
    import torch
    import scaled_dot_product_tiled_amd as sdpt
    from synth import ATTN_WORKLOADS
    from synth import draw_lengths, lengths_to_pad_mask
    w = ATTN_WORKLOADS[name].scaled(**changes)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(1234 + w.wid)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]

    def draw(shape, std):
        return (torch.randn(shape, generator=gen, device="cuda:0", dtype=torch.float32) * std).to(dt)

    q = draw((w.B, w.S, w.Hq, w.D), w.qk_std)
    k = draw((w.B, w.S, w.Hkv, w.D), w.qk_std)
    v = draw((w.B, w.S, w.Hkv, w.D), 1.0)
    do = draw((w.B, w.S, w.Hq, w.D), 1.0)
    lengths = draw_lengths(w, 0)
    pm = None
    if lengths is not None:
        pm = torch.from_numpy(lengths_to_pad_mask(lengths, w.S).astype(np.uint8)).to("cuda:0")
        pairs = sum(int(n) * (int(n) + 1) // 2 for n in lengths) * w.Hq
    else:
        pairs = causal_pairs(w.S, w.window) * w.B * w.Hq
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), device="cuda:0", dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = dict(scale=w.scale, causal=True, window=w.window, pad_mask=pm, softcap=softcap)

    def fwd():
        sdpt.attn_fwd(q, k, v, out=o, lse=lse, **kw)

    def bwd():
        sdpt.attn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, **kw)

    fwd()
    bwd()
    torch.cuda.synchronize()
    ms_f = time_median(fwd, steps, stream)
    ms_b = time_median(bwd, steps, stream)
    ff = 4.0 * w.D * pairs
    res = {"workload": w.name + ("" if w.dtype == "bf16" else f" {w.dtype}") + (f" softcap {softcap}" if softcap else ""),
           "pairs": pairs, "fwd_ms": round(ms_f, 4), "bwd_ms": round(ms_b, 4),
           "fwd_tflops": round(ff / ms_f / 1e9, 2), "bwd_tflops": round(2.5 * ff / ms_b / 1e9, 2),
           "step_tflops": round(3.5 * ff / (ms_f + ms_b) / 1e9, 2)}
    res["step_frac"] = round(res["step_tflops"] / PEAK_BF16_TFLOPS, 4)
    del q, k, v, do, o, lse, dq, dk, dv
    return res


def ring_workload(steps, stream, n_chunks=8, chunk=2048, Hq=32, Hkv=4, D=512):
    """One context-parallel rank's share of causal attention at 16k tokens (8 chunks of 2048
    positions, D=512, GQA 32/4): the last rank's query chunk against every key/value chunk
    that it sees (7 whole chunks and its own diagonal one).  Forward = attn_fwd_chunk for the
    first pair into the fp32 running O and LSE, then one attn_fwd_chunk_merge per further pair
    (the last one writes bf16 O); the two-step form (attn_fwd_chunk into an fp32 partial, then
    attn_lse_merge) is timed beside it.  Backward = one attn_bwd_chunk per pair adding into fp32
    dQ, dK, dV.  Device-side N(0,1) draws."""
    import torch
    import scaled_dot_product_tiled_amd as sdpt
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(4321)

    def draw(shape):
        return torch.randn(shape, generator=gen, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)

    rank = n_chunks - 1
    q, do = draw((1, chunk, Hq, D)), draw((1, chunk, Hq, D))
    k, v = draw((1, n_chunks * chunk, Hkv, D)), draw((1, n_chunks * chunk, Hkv, D))
    q0 = rank * chunk
    scale = 1.0 / math.sqrt(D)
    acc_o = torch.empty((1, chunk, Hq, D), device="cuda:0", dtype=torch.float32)
    part = torch.empty_like(acc_o)
    acc_l = torch.empty((1, Hq, chunk), device="cuda:0", dtype=torch.float32)
    part_l = torch.empty_like(acc_l)
    o = torch.empty_like(q)
    dq = torch.zeros((1, chunk, Hq, D), device="cuda:0", dtype=torch.float32)
    dk = torch.zeros((1, n_chunks * chunk, Hkv, D), device="cuda:0", dtype=torch.float32)
    dv = torch.zeros_like(dk)
    ks = [(c * chunk, (c + 1) * chunk) for c in range(rank + 1)]
    nws = max(sdpt.binding.attn_bwd_chunk_workspace_bytes(q, k[:, k0:k1], q0, k0) for k0, k1 in ks)
    ws = torch.empty(nws, device="cuda:0", dtype=torch.uint8)

    def fwd():
        for i, (k0, k1) in enumerate(ks):
            if i == 0:
                sdpt.attn_fwd_chunk(q, k[:, k0:k1], v[:, k0:k1], q0, k0, scale=scale, out=acc_o, lse=acc_l)
            else:
                sdpt.attn_fwd_chunk_merge(q, k[:, k0:k1], v[:, k0:k1], q0, k0, acc_o, acc_l, scale=scale,
                                          out=o if i == len(ks) - 1 else None)

    def fwd_two_step():
        for i, (k0, k1) in enumerate(ks):
            dst = (acc_o, acc_l) if i == 0 else (part, part_l)
            sdpt.attn_fwd_chunk(q, k[:, k0:k1], v[:, k0:k1], q0, k0, scale=scale, out=dst[0], lse=dst[1])
            if i > 0:
                sdpt.attn_lse_merge(acc_o, acc_l, part, part_l, out=o if i == len(ks) - 1 else None)

    def bwd():
        for k0, k1 in ks:
            sdpt.attn_bwd_chunk(q, k[:, k0:k1], v[:, k0:k1], o, acc_l, do, q0, k0, scale=scale, dq=dq,
                                dk=dk[:, k0:k1], dv=dv[:, k0:k1], accumulate=True, workspace=ws)

    fwd()
    bwd()
    torch.cuda.synchronize()
    ms_f2 = time_median(fwd_two_step, steps, stream)
    ms_f = time_median(fwd, steps, stream)
    ms_b = time_median(bwd, steps, stream)
    sdpt.binding.profile(True)
    for _ in range(steps):
        fwd()
        bwd()
    sdpt.binding.profile(False)
    kern = {n: {"launches": c, "ms_avg": round(t / c, 4)} for n, (c, t) in sdpt.binding.profile_read().items()}
    pairs = (rank * chunk * chunk + chunk * (chunk + 1) // 2) * Hq
    ff = 4.0 * D * pairs
    res = {"workload": f"ring context-parallel rank share, causal GQA d{D} (chunk {chunk} of {n_chunks}, "
                       f"Hq{Hq} Hkv{Hkv}, last rank: {rank + 1} chunk pairs)",
           "pairs": pairs, "fwd_ms": round(ms_f, 4), "fwd_ms_two_step": round(ms_f2, 4), "bwd_ms": round(ms_b, 4),
           "fwd_tflops": round(ff / ms_f / 1e9, 2), "bwd_tflops": round(2.5 * ff / ms_b / 1e9, 2),
           "step_tflops": round(3.5 * ff / (ms_f + ms_b) / 1e9, 2), "kernels": kern}
    res["step_frac"] = round(res["step_tflops"] / PEAK_BF16_TFLOPS, 4)
    del q, do, k, v, acc_o, part, acc_l, part_l, o, dq, dk, dv, ws
    return res


def paged_prefill_workload(steps, stream, B=1, prev=6144, n=2048, Hq=32, Hkv=4, D=512):
    """A 2048-token chunk of new queries after 6144 cached tokens (D=512, GQA 32/4, 16-token pages
    permuted over the pool): append the chunk's K/V to the pages, gather the 8192 tokens, run the
    chunk-pair forward at q_pos0 = 6144.  TFLOP/s of the attention (causal-counted pairs) over the
    time of the three calls."""
    import torch
    import scaled_dot_product_tiled_amd as sdpt
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(99)
    L = prev + n
    pages = -(-L // 16)
    pool = int(1.5 * pages)
    kc = torch.randn((pool, 16, Hkv, D), generator=gen, device="cuda:0").to(torch.bfloat16)
    vc = torch.randn((pool, 16, Hkv, D), generator=gen, device="cuda:0").to(torch.bfloat16)
    perm = torch.randperm(pool, generator=gen, device="cuda:0")[:pages].to(torch.int32)
    table = perm.reshape(1, pages).repeat(B, 1).contiguous()
    ctx = torch.full((B,), L, device="cuda:0", dtype=torch.int32)
    q = torch.randn((B, n, Hq, D), generator=gen, device="cuda:0").to(torch.bfloat16)
    kn = torch.randn((B, n, Hkv, D), generator=gen, device="cuda:0").to(torch.bfloat16)
    vn = torch.randn((B, n, Hkv, D), generator=gen, device="cuda:0").to(torch.bfloat16)
    kg = torch.empty((B, L, Hkv, D), device="cuda:0", dtype=torch.bfloat16)
    vg = torch.empty_like(kg)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, n), device="cuda:0", dtype=torch.float32)
    scale = 1.0 / math.sqrt(D)

    def run():
        sdpt.paged_kv_append(kn, vn, kc, vc, table, ctx)
        sdpt.paged_kv_gather(kc, vc, table, ctx, L, k_out=kg, v_out=vg)
        sdpt.attn_fwd_chunk(q, kg, vg, prev, 0, scale=scale, out=o, lse=lse)

    run()
    torch.cuda.synchronize()
    ms = time_median(run, steps, stream)
    sdpt.binding.profile(True)
    for _ in range(steps):
        run()
    sdpt.binding.profile(False)
    kern = {k: {"launches": c, "ms_avg": round(t / c, 4)} for k, (c, t) in sdpt.binding.profile_read().items()}
    pairs = (n * prev + n * (n + 1) // 2) * Hq * B
    ff = 4.0 * D * pairs
    return {"workload": f"paged prefill d{D}: {n} new tokens after {prev} cached (Hq{Hq} Hkv{Hkv}, 16-token pages)",
            "pairs": pairs, "ms": round(ms, 4), "tflops": round(ff / ms / 1e9, 2),
            "frac": round(ff / ms / 1e9 / PEAK_BF16_TFLOPS, 4), "kernels": kern}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--decode-steps", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-units", type=int, default=8, help="(batch, kv head) units the oracle times (of 8)")
    p.add_argument("--no-other", action="store_true", help="skip the sliding-window and varlen workloads")
    return p.parse_args()


def dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def time_events(fn, iters, stream):
    """Average milliseconds of fn() over iters calls, timed with HIP events on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def time_median(fn, iters, stream):
    """Median milliseconds of one fn() call over iters calls, each timed with its own pair of HIP
    events on `stream` (robust to a rare stall of the device that one long window would absorb)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    evs[-1][1].synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def cpu_baseline(units):
    """Times the float64 oracle (forward + backward of whole (batch, kv head) units) on the host."""
    import oracle
    from synth import ATTN_WORKLOADS, bf16_bits_to_f64, make_attention_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    w = ATTN_WORKLOADS["full_d512"]
    inp = make_attention_inputs(w, seed=0)
    q, k, v, do = (bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    for u in range(units):                 # (batch, kv head) units in order
        b, g = divmod(u, w.Hkv)
        for hi in range(w.r):
            oracle.attention_forward_head(q, k, v, b, g * w.r + hi, w.scale, True)
        oracle.attention_backward_group(q, k, v, do, b, g, w.scale, True)
    dt = time.perf_counter() - t0
    flops = 3.5 * 4 * w.D * causal_pairs(w.S) * w.r * units
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} of {w.B * w.Hkv} (batch, kv-head) units of the workload (forward + backward of "
                      f"{w.r} query heads each, causal-counted flops), {dt:.1f} s wall, float64 NumPy/BLAS",
            "seconds": dt, "cpu_count": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; the attention kernels shard by "
                                   "(batch, kv head) with no exchange, and multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import scaled_dot_product_tiled_amd as sdpt
    from synth import ATTN_WORKLOADS, DECODE_WORKLOADS, make_attention_inputs, make_decode_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    w = ATTN_WORKLOADS["full_d512"]
    inp = make_attention_inputs(w, seed=0)
    q, k, v, do = (dev(inp[x]) for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), device="cuda:0", dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = dict(scale=w.scale, causal=True, window=0)

    def fwd():
        sdpt.attn_fwd(q, k, v, out=o, lse=lse, **kw)

    def bwd():
        sdpt.attn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, **kw)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    pairs = causal_pairs(w.S) * w.B * w.Hq
    fwd_flops = 4.0 * w.D * pairs
    bwd_flops = 2.5 * fwd_flops

    # timed region: exactly `steps` steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = time_events(step, args.steps, stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps * 1e3
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12

    # per-call times (HIP events on the launch stream)
    ms_fwd = time_events(fwd, args.steps, stream)
    ms_bwd = time_events(bwd, args.steps, stream)
    fwd_tf = fwd_flops / (ms_fwd * 1e-3) / 1e12
    bwd_tf = bwd_flops / (ms_bwd * 1e-3) / 1e12

    # per-kernel times: the library records HIP event pairs around each of its launches
    sdpt.binding.profile(True)
    for _ in range(args.steps):
        step()
    sdpt.binding.profile(False)
    kt = sdpt.binding.profile_read()
    per_kernel = {n: {"launches": c, "ms_avg": round(t / c, 4)} for n, (c, t) in kt.items()}
    # algorithmic flops of each kernel: a contraction is 2 D flops per visible pair; the forward
    # does two (S, PV), dK/dV four (S, dP, dV, dK), dQ the one the definition adds (dQ)
    unit = 2.0 * w.D * pairs
    algo = {"attn_fwd": 2 * unit, "bwd_dkdv": 4 * unit, "bwd_dq": 1 * unit}
    dom = max(per_kernel, key=lambda n: per_kernel[n]["ms_avg"] * per_kernel[n]["launches"])
    dom_ms = per_kernel[dom]["ms_avg"]
    dom_tf = algo.get(dom, 0.0) / (dom_ms * 1e-3) / 1e12

    # paged decode, rotating over two independent KV pools
    dw = DECODE_WORKLOADS["decode_d128"]
    pools = []
    for s in (0, 1):
        di = make_decode_inputs(dw, seed=s)
        pools.append(dict(q=dev(di["q"]), kc=dev(di["k_cache"]), vc=dev(di["v_cache"]),
                          table=torch.from_numpy(di["block_table"]).to("cuda:0"),
                          ctx=torch.from_numpy(di["ctx_lens"]).to("cuda:0"), ctx_host=di["ctx_lens"]))
    outs = [torch.empty_like(p["q"]) for p in pools]
    ws = torch.empty(1 << 25, device="cuda:0", dtype=torch.uint8)

    def dbytes(ctx):
        tok = int(np.sum(ctx))
        pages = int(np.sum(-(-ctx.astype(np.int64) // dw.page_size)))
        return tok * dw.Hkv * dw.D * 2 * 2 + 2 * dw.B * dw.Hq * dw.D * 2 + 4 * pages + 4 * dw.B

    it = [0]

    def dec():
        p = pools[it[0] & 1]
        sdpt.paged_decode(p["q"], p["kc"], p["vc"], p["table"], p["ctx"], scale=dw.scale, out=outs[it[0] & 1],
                          workspace=ws)
        it[0] += 1

    for _ in range(4):
        dec()
    torch.cuda.synchronize()
    n_dec = args.decode_steps - (args.decode_steps % 2)
    ms_dec = time_events(dec, n_dec, stream)
    dec_bytes = 0.5 * (dbytes(pools[0]["ctx_host"]) + dbytes(pools[1]["ctx_host"]))
    dec_gbs = dec_bytes / (ms_dec * 1e-3) / 1e9
    sdpt.binding.profile(True)
    for _ in range(n_dec):
        dec()
    sdpt.binding.profile(False)
    dec_kernels = {n: {"launches": c, "ms_avg": round(t / c, 4)} for n, (c, t) in sdpt.binding.profile_read().items()}

    # the same decode with every sequence's pages laid out in order (page table = consecutive
    # ids): what the per-page table lookup costs against the permuted pool above
    def in_order(p):
        tbl = p["table"].cpu().numpy()
        ctx = p["ctx_host"]
        order = [int(tbl[b, j]) for b in range(dw.B) for j in range(-(-int(ctx[b]) // dw.page_size))]
        idx = torch.tensor(order, dtype=torch.long, device="cuda:0")
        t2 = np.full_like(tbl, -1)
        k = 0
        for b in range(dw.B):
            n = -(-int(ctx[b]) // dw.page_size)
            t2[b, :n] = np.arange(k, k + n)
            k += n
        return dict(q=p["q"], kc=p["kc"][idx].contiguous(), vc=p["vc"][idx].contiguous(),
                    table=torch.from_numpy(t2).to("cuda:0"), ctx=p["ctx"])

    cpools = [in_order(p) for p in pools]
    itc = [0]

    def dec_in_order():
        p = cpools[itc[0] & 1]
        sdpt.paged_decode(p["q"], p["kc"], p["vc"], p["table"], p["ctx"], scale=dw.scale, out=outs[itc[0] & 1],
                          workspace=ws)
        itc[0] += 1

    for _ in range(4):
        dec_in_order()
    torch.cuda.synchronize()
    ms_dec_in_order = time_events(dec_in_order, n_dec, stream)
    del cpools

    roof = {"kernel": dom, "bound": "mfma", "achieved": round(dom_tf, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic_bytes(dom),
            "ms_per_launch": dom_ms, "flop_per_launch": algo.get(dom, 0.0)}

    others = {}
    if not args.no_other:
        # the largest workload last: after its 20 GB of buffers the smaller ones timed slower
        others["ring_cp8_d512"] = ring_workload(5, stream)
        others["window_d256"] = other_workload("window_d256", 5, stream)
        others["full_d512_f16"] = other_workload("full_d512", 5, stream, dtype="f16")
        others["full_d512_softcap"] = other_workload("full_d512", 5, stream, softcap=30.0)
        others["paged_prefill_d512"] = paged_prefill_workload(5, stream)
        others["varlen_d512"] = other_workload("varlen_d512", 5, stream)

    out = {
        "metric": "causal attn fwd+bwd TFLOP/s @d=512 (% bf16 MFMA peak); decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "seq_len": w.S, "heads_q": w.Hq, "heads_kv": w.Hkv,
                   "head_dim": w.D, "causal": True, "parallelism": "single GPU"},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"ms": round(ms_fwd, 4), "tflops": round(fwd_tf, 2), "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(ms_bwd, 4), "tflops": round(bwd_tf, 2), "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4)},
        "wall_ms_per_step": round(wall, 4),
        "kernels": per_kernel,
        "roofline": roof,
        "decode": {"workload": dw.name, "ms": round(ms_dec, 4), "GB/s": round(dec_gbs, 1), "kernels": dec_kernels,
                   "pages_in_order": {"ms": round(ms_dec_in_order, 4),
                                      "GB/s": round(dec_bytes / (ms_dec_in_order * 1e-3) / 1e9, 1)},
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                                "bytes_per_launch": dec_bytes, "traffic": traffic_bytes("decode_split")}},
        "other_workloads": others,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_units)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
