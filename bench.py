"""Benchmark of the fused attention hot path on one MI355X.

A step is one forward + backward of causal grouped-query attention, head_dim 512 (B=2, S=4096,
Hq=32, Hkv=4, bf16, seeded N(0,1) inputs already resident in HBM): attn_fwd then attn_bwd through
the C ABI.  Reported:
  value     causal-counted TFLOP/s of the step over the timed region (exactly --steps steps between
            two synchronisations, a HIP event between consecutive steps): forward 4 D pairs, backward
            2.5x that, where pairs = visible (query, key) pairs summed over batch and heads (exact,
            not S^2/2); step_ms gives the median and best of the per-step event times;
  roofline  for the dominant kernel, timed with HIP event pairs around each of its launches on the
            stream it runs on (attn_profile), beside the rocprofv3 kernel-trace average of the
            committed profile of the same workload and their difference;
  decode    paged single-token decode (B=64, Hq=32, Hkv=8, D=128, 16-token pages, contexts
            U{512..4096}, pages permuted over a 1.5x pool) as achieved HBM GB/s of the algorithmic
            bytes, rotating over two KV pools so the 256 MB last-level cache cannot serve repeats;
            pages_in_order is the same decode with each sequence's pages consecutive in the pool,
            through the table and through paged_decode_contiguous (first page per sequence, no table);
            graph_replay replays the decode captured per batch bucket (DecodeGraphs) and gives the host
            time per launch beside that of an eager call;
  other_workloads  (median and best of per-call HIP-event timings) forward / backward TFLOP/s of the
            tiny (B=1 S=128 D=512), sliding-window (D=256, W=1024) and padded varlen (B=8, lengths
            U{512..8192}, D=512) workloads, of one context-parallel rank's chunk pairs (16k tokens in
            8 chunks, D=512), of the step's workload in IEEE half and with a softcap, and of two
            paged forwards (attn_fwd_paged): a 2048-token prompt chunk after 6144 cached tokens (beside
            the gather + chunk-pair path it replaces) and a serving step mixing a 1024-token chunk
            with 31 decode rows (attn_fwd_paged_split, which splits the decode rows, beside
            attn_fwd_paged); not part of the timed step;
  measured_peaks  what plain kernels reach on this device (attn_peak_probe): independent bf16
            32x32x16 matrix instructions, a streaming read and a streaming copy;
  cpu_baseline  the float64 oracle on a bounded sample of the same workload on the host cores, and
            per_config samples of the other workloads.
Prints one JSON line.

    python bench.py --workload NAME   (NAME: tiny_d512, full_d512, window_d256, varlen_d512,
                                        decode_d128, paged_prefill_d512, mixed_step_d512) runs only
                                        that workload's forward + backward (or decode, or paged
                                        forward) steps and prints its per-kernel times; the
                                        rocprofv3 summaries in profiles/ are taken from such runs.
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
    "attn_fwd": ("profiles/full_d512_traffic.txt", "fwd_kernel<512,32,false,false,false>"),
    "bwd_dkdv": ("profiles/full_d512_traffic.txt", "bwd_dkdv_kernel<512,false,false>"),
    "bwd_dq": ("profiles/full_d512_traffic.txt", "bwd_dq_kernel<256,4,2,false>"),
    "decode_whole": ("profiles/decode_d128_traffic.txt", "decode_whole_kernel<4,false,false>"),
}


# rocprofv3 --kernel-trace --stats summaries of each workload (committed profiles)
STATS = {
    "full_d512": "profiles/full_d512_kernel_stats.txt",
    "tiny_d512": "profiles/tiny_d512_kernel_stats.txt",
    "window_d256": "profiles/window_d256_kernel_stats.txt",
    "varlen_d512": "profiles/varlen_d512_kernel_stats.txt",
    "decode_d128": "profiles/decode_d128_kernel_stats.txt",
}
KERNEL_OF = {"attn_fwd": "fwd_kernel<", "bwd_dkdv": "bwd_dkdv_kernel<", "bwd_dq": "bwd_dq_kernel<",
             "bwd_pre": "bwd_pre_kernel<", "decode_split": "decode_split_kernel<",
             "decode_merge": "decode_merge_kernel<", "decode_whole": "decode_whole_kernel<"}


def rocprof_ms(workload, kernel):
    """(median, mean) duration in ms of `kernel`'s dispatches in the committed rocprofv3 summary of
    `workload` (its kernel trace, warm-up launches included), or None."""
    path = os.path.join(ROOT, STATS.get(workload, ""))
    if not os.path.isfile(path) or kernel not in KERNEL_OF:
        return None
    for line in open(path):
        parts = line.split()
        if len(parts) > 6 and parts[0].isdigit() and KERNEL_OF[kernel] in line.replace(" ", ""):
            return float(parts[2]) / 1e3, float(parts[1]) / 1e3
    return None


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


def time_calls(fn, n, stream):
    """n calls of fn() on `stream` with a HIP event before the first and after each call: the
    per-call times (ms) and their median, best and mean (the mean is the whole window / n)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record(stream)
    for i in range(n):
        fn()
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    return {"median": float(np.median(per)), "best": float(min(per)), "mean": evs[0].elapsed_time(evs[-1]) / n,
            "reps": n}


def rounded(t, nd=4):
    return {k: (round(v, nd) if isinstance(v, float) else v) for k, v in t.items()}


def kernel_times(fn, n):
    """Per-kernel HIP-event times (attn_profile: an event pair around every launch, on its stream)
    over n calls of fn()."""
    import scaled_dot_product_tiled_amd as sdpt
    sdpt.binding.profile(True)
    for _ in range(n):
        fn()
    sdpt.binding.profile(False)
    return {k: {"launches": c, "ms_avg": round(t / c, 4)} for k, (c, t) in sdpt.binding.profile_read().items()}


def attn_case(name, softcap=0.0, host_inputs=False, **changes):
    """Device buffers and fwd / bwd closures of one attention workload.  host_inputs: the seeded
    CPU draws the tests use (synth.make_attention_inputs); otherwise device-side seeded draws of
    the same shapes and distributions (lengths and masks from synth)."""
    import torch
    import scaled_dot_product_tiled_amd as sdpt
    from synth import ATTN_WORKLOADS, draw_lengths, lengths_to_pad_mask, make_attention_inputs
    w = ATTN_WORKLOADS[name].scaled(**changes)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    if host_inputs:
        inp = make_attention_inputs(w, seed=0)
        q, k, v, do = (torch.from_numpy(np.ascontiguousarray(inp[x]).view(np.int16)).to("cuda:0").view(dt)
                       for x in ("q", "k", "v", "do"))
        lengths = inp["lengths"]
    else:
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(1234 + w.wid)

        def draw(shape, std):
            return (torch.randn(shape, generator=gen, device="cuda:0", dtype=torch.float32) * std).to(dt)

        q = draw((w.B, w.S, w.Hq, w.D), w.qk_std)
        k = draw((w.B, w.S, w.Hkv, w.D), w.qk_std)
        v = draw((w.B, w.S, w.Hkv, w.D), w.vdo_std)
        do = draw((w.B, w.S, w.Hq, w.D), w.vdo_std)
        lengths = draw_lengths(w, 0)
    pm = None
    if lengths is not None:
        pm = torch.from_numpy(lengths_to_pad_mask(lengths, w.S).astype(np.uint8)).to("cuda:0")
        pairs = sum(int(n) * (int(n) + 1) // 2 for n in lengths) * w.Hq
    else:
        pairs = causal_pairs(w.S, w.window) * w.B * w.Hq if w.causal else w.S * w.S * w.B * w.Hq
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), device="cuda:0", dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, pad_mask=pm, softcap=softcap)
    bufs = [q, k, v, do, o, lse, dq, dk, dv, pm]

    def fwd():
        sdpt.attn_fwd(q, k, v, out=o, lse=lse, **kw)

    def bwd():
        sdpt.attn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, **kw)

    label = w.name + ("" if w.dtype == "bf16" else f" {w.dtype}") + (f" softcap {softcap}" if softcap else "")
    return {"w": w, "fwd": fwd, "bwd": bwd, "pairs": pairs, "fwd_flops": 4.0 * w.D * pairs, "label": label,
            "lengths": None if lengths is None else [int(x) for x in lengths], "bufs": bufs}


def other_workload(name, steps, stream, softcap=0.0, **changes):
    """Forward and backward per-call times (median and best of `steps` calls) of a workload."""
    import torch
    c = attn_case(name, softcap, **changes)
    c["fwd"]()
    c["bwd"]()
    torch.cuda.synchronize()
    tf = time_calls(c["fwd"], steps, stream)
    tb = time_calls(c["bwd"], steps, stream)
    ff = c["fwd_flops"]
    res = {"workload": c["label"], "pairs": c["pairs"], "reps": steps,
           "fwd_ms": round(tf["median"], 4), "fwd_ms_best": round(tf["best"], 4),
           "bwd_ms": round(tb["median"], 4), "bwd_ms_best": round(tb["best"], 4),
           "fwd_tflops": round(ff / tf["median"] / 1e9, 2), "bwd_tflops": round(2.5 * ff / tb["median"] / 1e9, 2),
           "step_tflops": round(3.5 * ff / (tf["median"] + tb["median"]) / 1e9, 2)}
    res["step_frac"] = round(res["step_tflops"] / PEAK_BF16_TFLOPS, 4)
    del c
    torch.cuda.empty_cache()
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
    ms_f2 = time_calls(fwd_two_step, steps, stream)["median"]
    ms_f = time_calls(fwd, steps, stream)["median"]
    ms_b = time_calls(bwd, steps, stream)["median"]
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


def prefill_workload(name, steps, stream, compare=True):
    """A PREFILL_WORKLOADS step: each sequence's new query rows against its paged cache (16-token
    pages permuted over a pool 1.5x the pages used), K/V read through the table inside
    attn_fwd_paged.  Times the attention call alone and with the step's paged_kv_append of the new
    tokens' K/V; for a single sequence also the gathered path it replaces (append, paged_kv_gather
    of the whole context, attn_fwd_chunk).  TFLOP/s count the causal-visible (query, key) pairs.
    Values are drawn on the device (torch's generator, seeded) to keep set-up short.  compare=False
    (--workload, the profiled runs) skips the unsplit call, whose forward kernel has the split
    call's name."""
    import torch
    import scaled_dot_product_tiled_amd as sdpt
    from synth import PREFILL_WORKLOADS
    w = PREFILL_WORKLOADS[name]
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(99)
    ctx = [int(c) for c in w.ctx]
    new = [int(n) for n in w.new]
    npages = [-(-c // 16) for c in ctx]
    pool = int(1.5 * sum(npages))
    maxp = max(npages)

    def randn(shape):
        return torch.randn(shape, generator=gen, device="cuda:0").to(torch.bfloat16)
    kc, vc = randn((pool, 16, w.Hkv, w.D)), randn((pool, 16, w.Hkv, w.D))
    perm = torch.randperm(pool, generator=gen, device="cuda:0").to(torch.int32)
    table = torch.full((w.B, maxp), -1, dtype=torch.int32, device="cuda:0")
    off = 0
    for b in range(w.B):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += npages[b]
    ctx_d = torch.tensor(ctx, dtype=torch.int32, device="cuda:0")
    cu = torch.tensor([0] + list(np.cumsum(new)), dtype=torch.int32, device="cuda:0")
    T, maxq = sum(new), max(new)
    q = randn((T, w.Hq, w.D))
    # the step's append: each sequence's new tokens, one paged_kv_append per distinct count
    groups = []
    for n in sorted(set(new)):
        idx = torch.tensor([b for b in range(w.B) if new[b] == n], device="cuda:0")
        groups.append((table[idx].contiguous(), ctx_d[idx].contiguous(), randn((len(idx), n, w.Hkv, w.D)),
                       randn((len(idx), n, w.Hkv, w.D))))
    o = torch.empty_like(q)
    lse = torch.empty((w.Hq, T), device="cuda:0", dtype=torch.float32)
    # with decode rows beside the chunk, the step runs attn_fwd_paged_split (decode rows split over
    # several workgroups, one workspace for every call); attn_fwd_paged is timed beside it
    split = 1 in new
    ws = torch.empty(sdpt.binding.attn_fwd_paged_workspace_bytes(q, kc, table, cu, maxq), device="cuda:0",
                     dtype=torch.uint8) if split else None

    def unsplit():
        sdpt.attn_fwd_paged(q, kc, vc, table, cu, ctx_d, maxq, scale=w.scale, out=o, lse=lse)

    def attn():
        if split:
            sdpt.attn_fwd_paged_split(q, kc, vc, table, cu, ctx_d, maxq, scale=w.scale, out=o, lse=lse, workspace=ws)
        else:
            unsplit()

    def append():
        for tg, cg, kn, vn in groups:
            sdpt.paged_kv_append(kn, vn, kc, vc, tg, cg)

    def step():
        append()
        attn()

    for f in (attn, step):
        f()
    torch.cuda.synchronize()
    ta = time_calls(attn, steps, stream)
    tst = time_calls(step, steps, stream)
    kern = kernel_times(step, steps)
    pairs = sum(n * (c - n) + n * (n + 1) // 2 for c, n in zip(ctx, new)) * w.Hq
    ff = 4.0 * w.D * pairs
    res = {"workload": w.name, "pairs": pairs, "ms": round(ta["median"], 4), "ms_best": round(ta["best"], 4),
           "tflops": round(ff / ta["median"] / 1e9, 2), "frac": round(ff / ta["median"] / 1e9 / PEAK_BF16_TFLOPS, 4),
           "step_ms_with_append": round(tst["median"], 4),
           "step_tflops_with_append": round(ff / tst["median"] / 1e9, 2), "kernels": kern}
    if split and compare:
        unsplit()
        torch.cuda.synchronize()
        tu = time_calls(unsplit, steps, stream)
        res["call"] = "attn_fwd_paged_split"
        res["unsplit"] = {"call": "attn_fwd_paged", "ms": round(tu["median"], 4), "ms_best": round(tu["best"], 4),
                          "tflops": round(ff / tu["median"] / 1e9, 2)}
    if w.B == 1:
        L, n = ctx[0], new[0]
        kg = torch.empty((1, L, w.Hkv, w.D), device="cuda:0", dtype=torch.bfloat16)
        vg = torch.empty_like(kg)
        q4 = q.view(1, n, w.Hq, w.D)
        o4 = torch.empty_like(q4)
        l4 = torch.empty((1, w.Hq, n), device="cuda:0", dtype=torch.float32)

        def gathered():
            append()
            sdpt.paged_kv_gather(kc, vc, table, ctx_d, L, k_out=kg, v_out=vg)
            sdpt.attn_fwd_chunk(q4, kg, vg, L - n, 0, scale=w.scale, out=o4, lse=l4, out_dtype=torch.bfloat16)

        gathered()
        torch.cuda.synchronize()
        tg = time_calls(gathered, steps, stream)
        res["gathered_path"] = {"ms": round(tg["median"], 4), "tflops": round(ff / tg["median"] / 1e9, 2),
                                "kernels": kernel_times(gathered, steps)}
        del kg, vg, o4, l4
    del kc, vc, q, groups, o, ws
    return res


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--decode-steps", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-units", type=int, default=8, help="(batch, kv head) units the oracle times (of 8)")
    p.add_argument("--no-other", action="store_true", help="skip the other workloads")
    p.add_argument("--workload", default=None,
                   help="profile one workload only: tiny_d512, full_d512, window_d256, varlen_d512, decode_d128, "
                        "paged_prefill_d512, mixed_step_d512")
    return p.parse_args()


def dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def cpu_info():
    """Host cores, BLAS library and threads, CPU model."""
    info = {"cpu_count": len(os.sched_getaffinity(0)), "cpu_model": None, "blas": None, "blas_threads": 1}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                info["blas"] = f"{i.get('internal_api')} {i.get('version')}"
                info["blas_threads"] = int(i.get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return info


def cpu_baseline(units):
    """Times the float64 oracle on the host: forward + backward of whole (batch, kv head) units of
    the step's workload (one process, BLAS threads as the library sets them), and bounded samples
    of the other workloads."""
    import oracle
    from synth import (ATTN_WORKLOADS, DECODE_WORKLOADS, bf16_bits_to_f64, draw_lengths, make_attention_inputs,
                       make_decode_inputs)
    info = cpu_info()

    def attn_units(name, picks):
        """picks: (batch, kv head) units; the oracle's inputs are the workload's seeded draws, except
        for the padded varlen workload, whose units are timed on draws of one sequence of the
        unit's length (the oracle's cost depends on the shapes only)."""
        w = ATTN_WORKLOADS[name]
        L = draw_lengths(w, 0)
        inp = make_attention_inputs(w, seed=0) if L is None else None
        flops = 0.0
        t0 = time.perf_counter()
        for b, g in picks:
            n = w.S if L is None else int(L[b])
            src = inp if L is None else make_attention_inputs(w.scaled(B=1, S=n, varlen=None, len_range=None), 0)
            bb = b if L is None else 0
            f = {x: bf16_bits_to_f64(src[x][bb:bb + 1]) for x in ("q", "k", "v", "do")}
            oracle.attention_group(f["q"], f["k"], f["v"], f["do"], 0, g, w.scale, w.causal, w.window, [n])
            flops += 3.5 * 4 * w.D * causal_pairs(n, w.window) * w.r
        dt = time.perf_counter() - t0
        lens = "" if L is None else f" (sequence lengths {[int(L[b]) for b, _ in picks]})"
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "seconds": round(dt, 2),
                "sample": f"{len(picks)} of {w.B * w.Hkv} (batch, kv-head) units {picks}{lens} of {w.name}, "
                          f"forward + backward of {w.r} query heads each (causal-counted flops)"}

    w = ATTN_WORKLOADS["full_d512"]
    main = attn_units("full_d512", [divmod(u, w.Hkv) for u in range(units)])
    per = {"tiny_d512": attn_units("tiny_d512", [(0, 0)]),
           "window_d256": attn_units("window_d256", [(0, 0), (1, 15)]),
           "varlen_d512": attn_units("varlen_d512", [(4, 0), (7, 3)])}
    dw = DECODE_WORKLOADS["decode_d128"]
    di = make_decode_inputs(dw, seed=0)
    q, kc, vc = (bf16_bits_to_f64(di[x]) for x in ("q", "k_cache", "v_cache"))
    nb = 16
    t0 = time.perf_counter()
    for b in range(nb):
        oracle.paged_decode_one(q, kc, vc, di["block_table"], di["ctx_lens"], dw.scale, b)
    dt = time.perf_counter() - t0
    tok = int(np.sum(di["ctx_lens"][:nb]))
    per["decode_d128"] = {"value": tok * dw.Hkv * dw.D * 4 / dt / 1e9, "unit": "GB/s", "seconds": round(dt, 2),
                          "sample": f"{nb} of {dw.B} sequences of {dw.name} (algorithmic K/V bytes)"}
    for v in per.values():
        v["value"] = round(v["value"], 5)
    return {"value": round(main["value"], 5), "unit": "TFLOP/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": main["sample"] + f", {main['seconds']} s wall, float64 NumPy",
            "seconds": main["seconds"], "workers": 1, "blas": info["blas"], "blas_threads": info["blas_threads"],
            "cpu_count": info["cpu_count"], "cpu_model": info["cpu_model"], "per_config": per}


def measured_peaks(stream):
    """Matrix rate, streaming read and copy of plain kernels on this device (attn_peak_probe)."""
    import torch
    import scaled_dot_product_tiled_amd as sdpt
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    buf = torch.zeros(cus * 4096, device="cuda:0", dtype=torch.uint8)
    reps = 4096
    sdpt.binding.peak_probe(0, buf, reps)
    t = time_calls(lambda: sdpt.binding.peak_probe(0, buf, reps), 5, stream)
    flops = 4 * cus * 4 * reps * 8 * 32768.0
    out["mfma_bf16_tflops"] = round(flops / t["best"] / 1e9, 1)
    big = torch.zeros(4 << 30, device="cuda:0", dtype=torch.uint8)
    sdpt.binding.peak_probe(1, big)
    t = time_calls(lambda: sdpt.binding.peak_probe(1, big), 5, stream)
    out["hbm_read_gbs"] = round(big.numel() / t["best"] / 1e6, 1)
    sdpt.binding.peak_probe(2, big)
    t = time_calls(lambda: sdpt.binding.peak_probe(2, big), 5, stream)
    out["hbm_copy_gbs"] = round(big.numel() / t["best"] / 1e6, 1)   # bytes read + written
    out["note"] = ("best of 5 launches: independent bf16 32x32x16 matrix instructions (4 workgroups x 4 waves per "
                   "CU), a 4 GiB streaming read, a 2 GiB -> 2 GiB streaming copy (read + written bytes)")
    del buf, big
    torch.cuda.empty_cache()
    return out


def decode_setup(seeds=(0, 1)):
    """Device copies of the decode workload's seeded pools, one per seed."""
    import torch
    from synth import DECODE_WORKLOADS, make_decode_inputs
    dw = DECODE_WORKLOADS["decode_d128"]
    pools = []
    for s in seeds:
        di = make_decode_inputs(dw, seed=s)
        pools.append(dict(q=dev(di["q"]), kc=dev(di["k_cache"]), vc=dev(di["v_cache"]),
                          table=torch.from_numpy(di["block_table"]).to("cuda:0"),
                          ctx=torch.from_numpy(di["ctx_lens"]).to("cuda:0"), ctx_host=di["ctx_lens"]))
    return dw, pools


def decode_bytes(dw, ctx):
    tok = int(np.sum(ctx))
    pages = int(np.sum(-(-ctx.astype(np.int64) // dw.page_size)))
    return tok * dw.Hkv * dw.D * 2 * 2 + 2 * dw.B * dw.Hq * dw.D * 2 + 4 * pages + 4 * dw.B


def profile_workload(args):
    """--workload: only that workload's steps (for rocprofv3), with its per-kernel event times."""
    import torch
    import scaled_dot_product_tiled_amd as sdpt
    stream = torch.cuda.current_stream()
    if args.workload in ("paged_prefill_d512", "mixed_step_d512"):
        res = prefill_workload(args.workload, args.steps, stream, compare=False)
    elif args.workload == "decode_d128":
        dw, pools = decode_setup()
        outs = [torch.empty_like(p["q"]) for p in pools]
        ws = torch.empty(1 << 25, device="cuda:0", dtype=torch.uint8)
        it = [0]

        def dec():
            p = pools[it[0] & 1]
            sdpt.paged_decode(p["q"], p["kc"], p["vc"], p["table"], p["ctx"], scale=dw.scale, out=outs[it[0] & 1],
                              workspace=ws)
            it[0] += 1
        for _ in range(args.warmup):
            dec()
        torch.cuda.synchronize()
        t = time_calls(dec, args.steps, stream)
        res = {"workload": dw.name, "ms": rounded(t), "kernels": kernel_times(dec, args.steps)}
    else:
        c = attn_case(args.workload, host_inputs=args.workload == "full_d512")
        for _ in range(args.warmup):
            c["fwd"]()
            c["bwd"]()
        torch.cuda.synchronize()
        tf = time_calls(c["fwd"], args.steps, stream)
        tb = time_calls(c["bwd"], args.steps, stream)
        ff = c["fwd_flops"]
        res = {"workload": c["label"], "pairs": c["pairs"], "fwd_ms": rounded(tf), "bwd_ms": rounded(tb),
               "fwd_tflops": round(ff / tf["median"] / 1e9, 2), "bwd_tflops": round(2.5 * ff / tb["median"] / 1e9, 2),
               "kernels": kernel_times(lambda: (c["fwd"](), c["bwd"]()), args.steps)}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; the attention kernels shard by "
                                   "(batch, kv head) with no exchange, and multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import scaled_dot_product_tiled_amd as sdpt

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.workload is not None:
        profile_workload(args)
        return

    c = attn_case("full_d512", host_inputs=True)
    w = c["w"]
    fwd, bwd = c["fwd"], c["bwd"]

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    fwd_flops = c["fwd_flops"]
    bwd_flops = 2.5 * fwd_flops

    # timed region: exactly `steps` steps between two synchronisations, an event after each
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ts = time_calls(step, args.steps, stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps * 1e3
    ms_step = ts["mean"]
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12

    # per-call times (HIP events on the launch stream)
    tf = time_calls(fwd, args.steps, stream)
    tb = time_calls(bwd, args.steps, stream)
    fwd_tf = fwd_flops / (tf["median"] * 1e-3) / 1e12
    bwd_tf = bwd_flops / (tb["median"] * 1e-3) / 1e12

    # per-kernel times: the library records HIP event pairs around each of its launches
    per_kernel = kernel_times(step, args.steps)
    # algorithmic flops of each kernel: a contraction is 2 D flops per visible pair; the forward
    # does two (S, PV), dK/dV four (S, dP, dV, dK), dQ the one the definition adds (dQ)
    unit = 2.0 * w.D * c["pairs"]
    algo = {"attn_fwd": 2 * unit, "bwd_dkdv": 4 * unit, "bwd_dq": 1 * unit}
    dom = max(per_kernel, key=lambda n: per_kernel[n]["ms_avg"] * per_kernel[n]["launches"])
    dom_ms = per_kernel[dom]["ms_avg"]
    dom_tf = algo.get(dom, 0.0) / (dom_ms * 1e-3) / 1e12
    rp = rocprof_ms("full_d512", dom)

    # paged decode, rotating over two independent KV pools
    dw, pools = decode_setup()
    outs = [torch.empty_like(p["q"]) for p in pools]
    ws = torch.empty(1 << 25, device="cuda:0", dtype=torch.uint8)
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
    td = time_calls(dec, n_dec, stream)
    dec_bytes = 0.5 * (decode_bytes(dw, pools[0]["ctx_host"]) + decode_bytes(dw, pools[1]["ctx_host"]))
    dec_gbs = dec_bytes / (td["mean"] * 1e-3) / 1e9
    dec_kernels = kernel_times(dec, n_dec)

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
                    table=torch.from_numpy(t2).to("cuda:0"), ctx=p["ctx"],
                    first=torch.from_numpy(np.ascontiguousarray(t2[:, 0])).to("cuda:0"), max_pages=tbl.shape[1])

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
    tdo = time_calls(dec_in_order, n_dec, stream)

    # the same in-order pools through paged_decode_contiguous: no table, one first page per sequence
    def dec_contiguous():
        p = cpools[itc[0] & 1]
        sdpt.paged_decode_contiguous(p["q"], p["kc"], p["vc"], p["first"], p["ctx"], p["max_pages"], scale=dw.scale,
                                     out=outs[itc[0] & 1], workspace=ws)
        itc[0] += 1

    for _ in range(4):
        dec_contiguous()
    torch.cuda.synchronize()
    tdc = time_calls(dec_contiguous, n_dec, stream)
    del cpools

    # the decode replayed from captured graphs (one per batch bucket, DecodeGraphs) against eager
    # calls: GPU time per step, and host time per launch
    p0 = pools[0]
    gr = sdpt.DecodeGraphs(p0["q"], p0["kc"], p0["vc"], p0["table"], p0["ctx"], outs[0], [1, 2, 4, 8, 16, 32, 64],
                           scale=dw.scale)
    torch.cuda.synchronize()
    tgr = time_calls(lambda: gr.launch(dw.B), n_dec, stream)

    def host_us(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        return (t1 - t0) / n * 1e6
    graph_host = host_us(lambda: gr.launch(dw.B), n_dec)
    eager_host = host_us(lambda: sdpt.paged_decode(p0["q"], p0["kc"], p0["vc"], p0["table"], p0["ctx"],
                                                    scale=dw.scale, out=outs[0], workspace=ws), n_dec)
    gr.close()

    # smaller batches of the same pools (their first B sequences): below one workgroup per compute
    # unit (B * Hkv < 256) the call takes the chunked schedule
    sweep = {}
    for bs in (8, 16, 32, 48):
        its = [0]

        def dec_b():
            p = pools[its[0] & 1]
            sdpt.paged_decode(p["q"][:bs], p["kc"], p["vc"], p["table"][:bs], p["ctx"][:bs], scale=dw.scale,
                              out=outs[its[0] & 1][:bs], workspace=ws)
            its[0] += 1

        for _ in range(4):
            dec_b()
        torch.cuda.synchronize()
        tb_ = time_calls(dec_b, 20, stream)
        kb_ = kernel_times(dec_b, 4)
        dwb = dw.scaled(B=bs)
        byt = 0.5 * (decode_bytes(dwb, pools[0]["ctx_host"][:bs]) + decode_bytes(dwb, pools[1]["ctx_host"][:bs]))
        sweep[str(bs)] = {"ms": round(tb_["mean"], 4), "GB/s": round(byt / (tb_["mean"] * 1e-3) / 1e9, 1),
                          "kernels": sorted(kb_)}
    # the decode workload's batch fills the chip: one launch of the whole-sequence kernel
    dec_kernel = "decode_whole" if "decode_whole" in dec_kernels else "decode_split"
    rpd = rocprof_ms("decode_d128", dec_kernel)

    roof = {"kernel": dom, "bound": "mfma", "achieved": round(dom_tf, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic_bytes(dom),
            "ms_per_launch": dom_ms, "flop_per_launch": algo.get(dom, 0.0),
            "timing": "HIP event pair around each launch on its stream, averaged over the run's launches",
            "rocprof_ms_median": None if rp is None else rp[0], "rocprof_ms_mean": None if rp is None else rp[1],
            "rocprof_source": STATS["full_d512"] if rp is not None else None,
            "event_vs_rocprof_median": None if rp is None else round(dom_ms / rp[0] - 1.0, 4),
            "rocprof_frac": None if rp is None else round(algo.get(dom, 0.0) / (rp[0] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                                          4)}

    peaks = measured_peaks(stream)

    others = {}
    if not args.no_other:
        others["tiny_d512"] = other_workload("tiny_d512", 50, stream)
        # the largest workload last: after its 20 GB of buffers the smaller ones timed slower
        others["ring_cp8_d512"] = ring_workload(5, stream)
        others["window_d256"] = other_workload("window_d256", 20, stream)
        others["full_d512_f16"] = other_workload("full_d512", 5, stream, dtype="f16")
        others["full_d512_softcap"] = other_workload("full_d512", 5, stream, softcap=30.0)
        others["paged_prefill_d512"] = prefill_workload("paged_prefill_d512", 10, stream)
        others["mixed_step_d512"] = prefill_workload("mixed_step_d512", 10, stream)
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
        "step_ms": rounded(ts),
        "step_tflops_median": round((fwd_flops + bwd_flops) / (ts["median"] * 1e-3) / 1e12, 2),
        "step_tflops_best": round((fwd_flops + bwd_flops) / (ts["best"] * 1e-3) / 1e12, 2),
        "fwd": {"ms": round(tf["median"], 4), "ms_best": round(tf["best"], 4), "tflops": round(fwd_tf, 2),
                "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(tb["median"], 4), "ms_best": round(tb["best"], 4), "tflops": round(bwd_tf, 2),
                "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4)},
        "wall_ms_per_step": round(wall, 4),
        "kernels": per_kernel,
        "roofline": roof,
        "measured_peaks": peaks,
        "decode": {"workload": dw.name, "ms": round(td["mean"], 4), "ms_median": round(td["median"], 4),
                   "ms_best": round(td["best"], 4), "reps": n_dec, "GB/s": round(dec_gbs, 1),
                   "kernels": dec_kernels,
                   "pages_in_order": {"ms": round(tdo["mean"], 4), "ms_best": round(tdo["best"], 4),
                                      "GB/s": round(dec_bytes / (tdo["mean"] * 1e-3) / 1e9, 1),
                                      "contiguous_call": {"ms": round(tdc["mean"], 4), "ms_best": round(tdc["best"], 4),
                                                          "GB/s": round(dec_bytes / (tdc["mean"] * 1e-3) / 1e9, 1)}},
                   "batch_sweep": sweep,
                   "graph_replay": {"ms": round(tgr["mean"], 4), "ms_best": round(tgr["best"], 4),
                                    "host_us_per_launch": round(graph_host, 1),
                                    "eager_host_us_per_call": round(eager_host, 1)},
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                                "bytes_per_launch": dec_bytes, "traffic": traffic_bytes(dec_kernel),
                                "kernel": dec_kernel,
                                "timing": "HIP events around each call (every launch of the call and the gaps)",
                                "rocprof_ms_median": None if rpd is None else rpd[0]}},
        "other_workloads": others,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_units)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
