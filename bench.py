#!/usr/bin/env python3
"""Benchmark of the Grok-1 attention core on one MI355X.

Default run (N=1): the headline workload is the 8k causal prefill
(B=1, T=8192, 48 query heads on 8 KV heads, head size 128, bf16): one step is
RoPE of Q and K plus the causal GQA attention, and ``value`` is its
algorithmic TFLOP/s (4*D*Hq*B*T(T+1)/2 flop per step: QK^T and P.V over the
causal lower triangle, diagonal included). The same JSON line carries the
decode workloads (single-token decode on a full 8192-slot cache; 32 ragged
sequences) as KV GB/s, the full sub-layer as TFLOP/s, the roofline of the
dominant kernel, and the fp64 CPU oracle timed on a bounded sample.

Inputs are synthetic, seeded, and resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GQA attn prefill TFLOP/s + decode KV GB/s (48q/8kv/d128), % of roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--only", default="", help="comma list of prefill,decode_b1,decode_ragged,sublayer,"
                    "decode_sublayer_b1,decode_sublayer_b32,chunk,moe (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device-to-device copy (HBM counter calibration)")
    return ap.parse_args()


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gqa_attention_grok_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if the
    kernel sources are unchanged since the counters were taken; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def steps_per_graph(steps):
    """Steps captured per graph: 8 (or the largest of 4, 2, 1 dividing `steps`),
    so that exactly `steps` steps are timed and the host's graph launches do
    not pace a step of a few tens of microseconds."""
    for k in (8, 4, 2, 1):
        if steps % k == 0:
            return k
    return 1


def time_steps(torch, pipe, fns, steps, warmup):
    """Capture consecutive steps (cycling over `fns`, e.g. one per replica of the
    inputs) into HIP graphs of steps_per_graph(steps) steps each, warm up, then
    time exactly `steps` steps between two device synchronisations; returns
    seconds per step."""
    k = steps_per_graph(steps)
    R = len(fns)
    ngraphs = R // math.gcd(R, k)  # graphs until the replica cycle repeats
    graphs = []
    for gi_ in range(ngraphs):
        idx = [(gi_ * k + j) % R for j in range(k)]
        graphs.append(pipe.capture(lambda idx=idx: [fns[i]() for i in idx]))
    nrep = steps // k
    for i in range(max(1, warmup // k)):
        graphs[i % ngraphs].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(nrep):
        graphs[i % ngraphs].replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / (nrep * k)
    del graphs
    return sec


def time_kernel(torch, fn, reps):
    """Mean duration of the kernel(s) `fn` launches, from HIP events recorded on
    the stream they are launched on (torch's current stream)."""
    fn(0)
    ev = []
    for i in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def bench_prefill(torch, grok, pipe, U, gi, steps, warmup):
    w = gi.WORKLOADS["prefill_b1_t8192"]
    p = gi.make_workload(w.name)
    st = pipe.PrefillStep(U.dev_bf16(p["q"]), U.dev_bf16(p["k"]), U.dev_bf16(p["v"]), w.attn_mult,
                          w.softcap)
    del p
    flop = 4 * w.D * w.Hq * w.B * w.T * (w.T + 1) // 2
    sec = time_steps(torch, pipe, [st], steps, warmup)
    kern_ms = time_kernel(torch, lambda i: st.attend(), max(steps, 5))
    return {
        "workload": w.name, "ms_per_step": sec * 1e3, "value": flop / sec / 1e12, "unit": "TFLOP/s",
        "flop_per_step": flop, "kernel": "prefill_mfma_kernel", "kernel_ms": kern_ms,
        "kernel_tflops": flop / (kern_ms * 1e-3) / 1e12,
    }


def bench_decode(torch, grok, pipe, U, gi, name, steps, warmup, replicas):
    """One step = RoPE + append of the new token and split-K decode attention (the
    append runs inside the split kernel), then the combine.
    `replicas` copies of the cache are cycled so the working set exceeds the
    256 MB last-level cache and each step streams K/V from HBM."""
    w = gi.WORKLOADS[name]
    p = gi.make_workload(name)
    kc0, vc0 = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
    reps = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(replicas - 1)]
    q, kn, vn, stp = U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]), U.dev(p["step"])
    steps_obj = [pipe.DecodeStep(kc, vc, q, kn, vn, stp, w.attn_mult, w.softcap) for kc, vc in reps]
    L = p["kv_len"].astype(np.int64)
    D, Hq, Hkv = w.D, w.Hq, w.Hkv
    # algorithmic bytes: valid K and V rows once, q, the new k/v row, the output
    kv_bytes = int(L.sum()) * Hkv * D * 2 * 2
    io_bytes = w.B * (Hq * D * 2 + 2 * Hkv * D * 2 + Hq * D * 2)
    nbytes = kv_bytes + io_bytes
    sec = time_steps(torch, pipe, steps_obj, steps, warmup)

    def attend(i):  # the step's launches, eager (split with the append fused, combine)
        steps_obj[i % len(steps_obj)]()

    kern_ms = time_kernel(torch, attend, max(steps, 2 * len(steps_obj)))
    return {
        "workload": name, "ms_per_step": sec * 1e3, "value": nbytes / sec / 1e9, "unit": "GB/s",
        "bytes_per_step": nbytes, "kernel": "decode_split_kernel(append fused)+decode_combine_kernel",
        "kernel_ms": kern_ms, "kernel_gbs": nbytes / (kern_ms * 1e-3) / 1e9,
        "kernel_frac_of_hbm_peak": nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "cache_replicas": replicas,
    }


def bench_sublayer(torch, grok, pipe, U, gi, steps, warmup):
    w = gi.WORKLOADS["sublayer_b4_t2048"]
    p = gi.make_workload(w.name)
    dv = {k: (U.dev_bf16(v) if k == "x" else U.dev(v)) for k, v in p.items()}
    del p
    st = pipe.SublayerStep(dv["x"], dv["wq"], dv["sq"], dv["wk"], dv["sk"], dv["wv"], dv["sv"], dv["wo"],
                           dv["so"], w.Hq, w.Hkv, w.D, w.attn_mult, w.softcap, w.eps)
    M, d = w.B * w.T, w.d_model
    proj = 2 * M * d * (w.Hq * w.D + 2 * w.Hkv * w.D) + 2 * M * (w.Hq * w.D) * d
    attn = 4 * w.D * w.Hq * w.B * w.T * (w.T + 1) // 2
    flop = proj + attn
    sec = time_steps(torch, pipe, [st], steps, warmup)
    return {"workload": w.name, "ms_per_step": sec * 1e3, "value": flop / sec / 1e12,
            "unit": "TFLOP/s", "flop_per_step": flop}


def bench_decode_sublayer(torch, grok, pipe, U, gi, name, steps, warmup, replicas):
    """One step = the attention sub-layer for one new token per sequence: pre-norm,
    Q|K|V projection (one launch), RoPE + append, decode attention, output
    projection, post-norm + residual. `replicas` copies of the weights and caches
    are cycled so that each step streams them from HBM, not from the last-level
    cache."""
    w = gi.WORKLOADS[name]
    p = gi.make_workload(name)
    x, stp = U.dev_bf16(p["x"]), U.dev(p["step"])
    wnames = ("wq", "sq", "wk", "sk", "wv", "sv", "wo", "so")
    steps_obj = []
    for _ in range(replicas):
        kc, vc = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
        ww = [U.dev(p[k]) for k in wnames]
        steps_obj.append(pipe.DecodeSublayerStep(x, kc, vc, stp, *ww, w.Hq, w.Hkv, w.D, w.attn_mult,
                                                 w.softcap, w.eps))
    B, d, D, Hq, Hkv = w.B, w.d_model, w.D, w.Hq, w.Hkv
    L = p["kv_len"].astype(np.int64)
    del p
    cols = Hq * D + 2 * Hkv * D
    w_bytes = d * cols + Hq * D * d + 4 * (cols + d)       # int8 weights + fp32 scales
    kv_bytes = int(L.sum()) * Hkv * D * 2 * 2               # valid K and V slots, once
    io_bytes = B * (2 * d * 2 + 2 * Hkv * D * 2)            # x in, y out, new k/v written
    nbytes = w_bytes + kv_bytes + io_bytes
    sec = time_steps(torch, pipe, steps_obj, steps, warmup)

    # the weight-streaming kernels of one step (norm + Q|K|V + RoPE + append;
    # the output projection with the post-norm and residual), replayed from
    # graphs (no host work)
    proj_ms = time_steps(torch, pipe, [lambda s_=s_: (s_.front(), s_.back()) for s_ in steps_obj],
                         steps, warmup) * 1e3
    # weights and scales once; x in, q and the k/v rows out; attn and x in, y out
    pbytes = d * cols + Hq * D * d + 4 * (cols + d) + B * 2 * (d + cols + Hq * D + 2 * d)
    # the same step with the back half as the separate projection and norm
    ref_obj = [pipe.DecodeSublayerStep(s_.x, s_.k_cache, s_.v_cache, s_.step, *s_.w_args, s_.Hq, s_.Hkv, s_.D,
                                       s_.attn_mult, s_.softcap, s_.eps, fused_back=False) for s_ in steps_obj]
    sec_unfused_back = time_steps(torch, pipe, ref_obj, steps, warmup)
    del ref_obj
    return {
        "workload": name, "ms_per_step": sec * 1e3, "value": nbytes / sec / 1e9, "unit": "GB/s",
        "ms_per_step_back_half_unfused": sec_unfused_back * 1e3,
        "bytes_per_step": nbytes,
        "kernel": "decode_qkv_kernel + gemv_out_norm_kernel (Q|K|V with norm/RoPE/append; O with norm and residual)",
        "kernel_ms": proj_ms, "kernel_gbs": pbytes / (proj_ms * 1e-3) / 1e9,
        "kernel_frac_of_hbm_peak": pbytes / (proj_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "replicas": replicas,
    }


def bench_chunk(torch, grok, pipe, U, gi, steps, warmup, replicas=2):
    """One step = RoPE + append of a 512-token chunk per sequence, then its
    causal attention over the cached prefix and itself."""
    w = gi.WORKLOADS["prefill_chunk_b4_t512"]
    p = gi.make_workload(w.name)
    q, kn, vn, stp = U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]), U.dev(p["step"])
    steps_obj = [pipe.ChunkStep(U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"]), q, kn, vn, stp, w.attn_mult,
                                w.softcap) for _ in range(replicas)]
    offs = p["step"].astype(np.int64)
    del p
    flop = int(sum(4 * w.D * w.Hq * (w.T * (o + 1) + w.T * (w.T - 1) // 2) for o in offs))
    sec = time_steps(torch, pipe, steps_obj, steps, warmup)
    kern_ms = time_kernel(torch, lambda i: steps_obj[i % replicas].attend(), max(steps, 2 * replicas))
    return {"workload": w.name, "ms_per_step": sec * 1e3, "value": flop / sec / 1e12, "unit": "TFLOP/s",
            "flop_per_step": flop, "offsets": [int(o) for o in offs], "kernel": "prefill_mfma_kernel (offset)",
            "kernel_ms": kern_ms, "kernel_tflops": flop / (kern_ms * 1e-3) / 1e12}


def bench_moe(torch, grok, pipe, U, gi, steps, warmup):
    """One step = the MoE FFN sub-layer over 8192 token rows: norm, router,
    routing plan, the two grouped int8 expert products (GeGLU up projection of
    the gathered rows, down projection), gate-weighted combine, norm, residual.
    Counted work: the expert products, 6 * T * k * d * F flop."""
    w = gi.WORKLOADS["moe_b4_t2048"]
    p = gi.make_workload(w.name)
    T, d, F = w.B * w.T, w.d_model, w.d_ffn
    x = U.dev_bf16(p["x"].reshape(T, d))
    experts = [tuple(U.dev(a) for a in ex) for ex in p["experts"]]
    wr = U.dev(p["w_router"])
    del p
    step = pipe.MoeStep(x, wr, experts, k=w.top_k)
    del experts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    flop = 6 * T * w.top_k * d * F
    sec = time_steps(torch, pipe, [step], steps, warmup)
    kern_ms = time_kernel(torch, lambda i: step(), max(2, steps // 2))
    counts = np.bincount(step.idx.cpu().numpy().ravel(), minlength=w.n_experts)
    return {"workload": w.name, "ms_per_step": sec * 1e3, "value": flop / sec / 1e12, "unit": "TFLOP/s",
            "flop_per_step": flop, "rows_per_expert": counts.tolist(), "kernel": "moe_ffn (all kernels)",
            "kernel_ms": kern_ms, "kernel_tflops": flop / (kern_ms * 1e-3) / 1e12}


# ---------------------------------------------------------------------------
# The fp64 oracle timed on the host's cores (a reported baseline, not a target).
# Runs in worker processes started with "spawn" before this process touches
# the GPU; the workers import only the oracle and the input generator.
# ---------------------------------------------------------------------------
_W = {}


def _oracle_init(name, k_bits=None, v_bits=None):
    """Worker set-up (untimed): for the 8k prefill, the keys rotated at
    positions 0..T-1 and the values in float64."""
    import gqa_inputs as gi
    import oracle as orc
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)  # one core per worker process
    w = gi.WORKLOADS[name]
    _W.update(w=w, orc=orc)
    if k_bits is not None:
        _W["k"] = orc.rope(orc.bf16_bits_to_f64(k_bits), np.arange(w.T)[None], out="bf16")
        _W["v"] = orc.bf16_bits_to_f64(v_bits)


def _oracle_prefill_rows(task):
    """Causal softcapped attention of the given query rows (all heads)."""
    rows, q_bits = task
    w, orc = _W["w"], _W["orc"]
    q = orc.rope(orc.bf16_bits_to_f64(q_bits), rows[None], out="bf16")
    mask = orc.attention_mask(rows[None], w.T)
    for c in range(0, len(rows), 8):  # bounded memory: 8 rows at a time
        orc.attention(q[:, c:c + 8], _W["k"], _W["v"], mask[:, c:c + 8], w.attn_mult, w.softcap, out="bf16")
    return len(rows)


def _oracle_decode_seq(task):
    """One sequence of a decode workload: RoPE of q and the new k, the append,
    attention over the valid slots of its whole cache."""
    kc, vc, q, kn, vn, step = task
    w, orc = _W["w"], _W["orc"]
    f = orc.bf16_bits_to_f64
    orc.decode_step(f(kc), f(vc), f(q), f(kn), f(vn), step, w.attn_mult, w.softcap)
    return 0


def _noop(i):
    time.sleep(0.2)  # keeps each worker busy long enough that all of them start
    return i


def _timed_pool(name, fn, tasks, workers, initargs=()):
    """Wall time of fn over tasks on `workers` spawned processes (set-up excluded)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                             initializer=_oracle_init, initargs=(name, *initargs)) as ex:
        list(ex.map(_noop, range(workers)))  # every worker has run its set-up
        t0 = time.perf_counter()
        list(ex.map(fn, tasks))
        return time.perf_counter() - t0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    """The fp64 oracle (NumPy, one thread per worker process) on the host cores:
    a bounded sample of the 8k prefill (all 48 heads of 96 query rows per
    worker, spread over the sequence), and the tiny fp32 prefill, the
    one-sequence decode and the 32-sequence ragged decode in full."""
    import gqa_inputs as gi
    import oracle as orc
    workers = max(1, min(16, os.cpu_count() or 1))
    w = gi.WORKLOADS["prefill_b1_t8192"]
    p = gi.make_workload(w.name)
    T = w.T
    rows = np.linspace(0, T - 1, 96 * workers).astype(np.int64)
    # one task per worker, rows interleaved so that each holds short and long rows
    tasks = [(rows[i::workers], p["q"][:, rows[i::workers]]) for i in range(workers)]
    sec = _timed_pool(w.name, _oracle_prefill_rows, tasks, workers, (p["k"], p["v"]))
    del p, tasks
    flop = int(sum(4 * w.D * w.Hq * (int(t) + 1) for t in rows))
    extra = {}
    wt = gi.WORKLOADS["prefill_f32_t16"]
    pt = gi.make_workload(wt.name)
    pos = np.arange(wt.T)[None]
    t0 = time.perf_counter()
    for _ in range(5):
        qt = orc.rope(pt["q"].astype(np.float64), pos, out="f32")
        kt = orc.rope(pt["k"].astype(np.float64), pos, out="f32")
        orc.attention(qt, kt, pt["v"].astype(np.float64), orc.attention_mask(pos, wt.T), wt.attn_mult, wt.softcap)
    t1 = (time.perf_counter() - t0) / 5
    extra[wt.name] = {"ms": round(t1 * 1e3, 3), "cores": 1, "full": True, "unit": "TFLOP/s",
                      "value": 4 * wt.D * wt.Hq * wt.T * (wt.T + 1) // 2 / t1 / 1e12}
    for name in ("decode_b1_t8192", "decode_ragged_b32_t8192"):
        wd = gi.WORKLOADS[name]
        pd = gi.make_workload(name)
        dtasks = [(pd["k_cache"][b:b + 1], pd["v_cache"][b:b + 1], pd["q"][b:b + 1], pd["k_new"][b:b + 1],
                   pd["v_new"][b:b + 1], pd["step"][b:b + 1]) for b in range(wd.B)]
        nw = min(workers, wd.B)
        s = _timed_pool(name, _oracle_decode_seq, dtasks, nw)
        L = pd["kv_len"].astype(np.int64)
        del pd, dtasks
        nbytes = int(L.sum()) * wd.Hkv * wd.D * 4 + wd.B * (2 * wd.Hq * wd.D * 2 + 2 * wd.Hkv * wd.D * 2)
        extra[name] = {"ms": round(s * 1e3, 1), "cores": nw, "full": True, "value": nbytes / s / 1e9,
                       "unit": "GB/s"}
    return {"value": flop / sec / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{len(rows)} of {T} query rows (all 48 heads) of the 8k prefill, RoPE of q included "
                      f"(keys rotated once per worker, untimed); {flop} flop in {sec:.1f} s on {workers} "
                      f"single-threaded NumPy worker processes",
            "other_workloads": extra}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention core shards with no exchange over KV heads: see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    cpu = None
    if not args.no_cpu_baseline:  # before this process initialises the GPU
        cpu = cpu_baseline()
        print(f"# cpu baseline done: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} cores", file=sys.stderr,
              flush=True)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gqa_attention_grok_amd as grok
    import gqa_attention_grok_amd.pipeline as pipe
    import gqa_inputs as gi
    import gqa_inputs.device as U

    only = set(args.only.split(",")) if args.only else {"prefill", "decode_b1", "decode_ragged", "sublayer",
                                                        "decode_sublayer_b1", "decode_sublayer_b32", "chunk", "moe"}
    res = {}
    if args.copy_calibration:
        # a plain copy of known size: reads and writes exactly 256 MiB
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("# copy calibration done: 268435456 bytes read and written", file=sys.stderr, flush=True)
    if "prefill" in only:
        res["prefill"] = bench_prefill(torch, grok, pipe, U, gi, args.steps, args.warmup)
        print(f"# prefill done: {res['prefill']['value']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if "decode_b1" in only:
        res["decode_b1"] = bench_decode(torch, grok, pipe, U, gi, "decode_b1_t8192", args.steps, args.warmup, 16)
        print(f"# decode_b1 done: {res['decode_b1']['value']:.1f} GB/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if "decode_ragged" in only:
        res["decode_ragged"] = bench_decode(torch, grok, pipe, U, gi, "decode_ragged_b32_t8192", args.steps,
                                 args.warmup, 2)
        print(f"# decode_ragged done: {res['decode_ragged']['value']:.1f} GB/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if "sublayer" in only:
        res["sublayer"] = bench_sublayer(torch, grok, pipe, U, gi, max(1, args.steps // 4), min(args.warmup, 2))
        print(f"# sublayer done: {res['sublayer']['value']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    for key, name, reps in (("decode_sublayer_b1", "decode_sublayer_b1_t8192", 4),
                            ("decode_sublayer_b32", "decode_sublayer_b32_t8192", 2)):
        if key in only:
            res[key] = bench_decode_sublayer(torch, grok, pipe, U, gi, name, args.steps, args.warmup, reps)
            print(f"# {key} done: {res[key]['value']:.1f} GB/s, {res[key]['ms_per_step'] * 1e3:.1f} us/step",
                  file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
    if "chunk" in only:
        res["chunk"] = bench_chunk(torch, grok, pipe, U, gi, args.steps, args.warmup)
        print(f"# chunk done: {res['chunk']['value']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if "moe" in only:
        res["moe"] = bench_moe(torch, grok, pipe, U, gi, max(2, args.steps // 10), min(args.warmup, 4))
        print(f"# moe done: {res['moe']['value']:.1f} TFLOP/s", file=sys.stderr, flush=True)

    head = res.get("prefill") or next(iter(res.values()))
    line = {
        "metric": METRIC,
        "value": round(head["value"], 3),
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"] + (
            ": causal GQA prefill B=1 T=8192 Hq=48 Hkv=8 D=128 bf16, step = RoPE(Q,K) + attention"
            if head is res.get("prefill") else "")},
    }
    if head is res.get("prefill"):
        tr = traffic_for(head["kernel"])
        line["roofline"] = {
            "kernel": head["kernel"], "bound": "mfma", "achieved": round(head["kernel_tflops"], 3),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(head["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": tr, "kernel_ms": round(head["kernel_ms"], 4),
        }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    line["secondary"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                         for k, r in res.items() if r is not head}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
