"""Throughput of the DSA forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]
                    [--prefill-workload p128k]

A step is one dsa_forward call (indexer scores -> top-k -> sparse attention)
over one batch of synthetic inputs already resident in HBM.  The metric has
two halves, both at 128K context with k = 2048:
  * decode steps/s (the headline `value`): the default workload is 8
    sequences of 131072 cached tokens, one new query each, fp8 e4m3 indexer
    keys, MLA latent 576/512 bf16; inputs rotate over several replicas so
    consecutive steps do not find the key cache in the last-level cache;
  * prefill tokens/s (the `prefill` sub-record): one 131072-token sequence,
    bf16 indexer, MLA latent, the forward pass running its query rows in
    1 GiB score chunks.
Prints one JSON line.  Besides the step throughput it carries:
  * roofline: the dominant kernel's algorithmic bytes (or flops) per launch
    over its average duration, timed with HIP events on the library's stream,
    as a fraction of the vendor peak and of the peak measured on this device
    (`measured_peaks`: a streaming-read kernel and MFMA issue loops);
  * spread: p10 / p50 / p90 of the step time over blocks of steps;
  * cpu_baseline: the CPU oracle timed on a bounded sample of the same
    workload on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer+sparse-attn tokens/s (prefill) & decode steps/s at 128K ctx, k=2048"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA
FP8_PEAK_TFLOPS = 5000.0
FP32_VECTOR_TFLOPS = 157.3
# the forward pass's score block (capi.hip): query rows per chunk = 1 GiB / (B * S * 4)
SCORE_CHUNK_BYTES = 1 << 30
WORKLOADS = ["c1", "c2", "c2-fp8", "c3", "c4", "p128k", "short2k"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=WORKLOADS)
    ap.add_argument("--prefill-workload", default="p128k", choices=WORKLOADS + ["none"],
                    help="with a decode --workload: the prefill half of the metric")
    ap.add_argument("--prefill-steps", type=int, default=3)
    ap.add_argument("--kl", type=int, default=0,
                    help="prefill: also time the indexer distillation loss (forward) per chunk")
    ap.add_argument("--include-current", type=int, default=0,
                    help="always keep the current token (dsa_forward_ex flag)")
    ap.add_argument("--replicas", type=int, default=0, help="input replicas (0 = auto)")
    ap.add_argument("--graph", type=int, default=1, help="replay the step as a HIP graph")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--stages", type=int, default=1,
                    help="also time each entry point alone (per-stage times, rooflines)")
    ap.add_argument("--peaks", type=int, default=1, help="measure the device's achievable peaks")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES between two device buffers (counter calibration)")
    return ap.parse_args()


def copy_calibration(nbytes: int):
    """A plain device copy of a known size: reads and writes exactly nbytes, so
    the FETCH_SIZE / WRITE_SIZE counters it produces calibrate their units."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "dispatches": 3}))


def algorithmic(w):
    """Algorithmic work of one step and of each stage (what the method must
    read, write or compute; dense work a masked kernel might add is not
    counted)."""
    from learned_sparse_attention_lightning_amd.configs import causal_pairs, selected_entries
    eb = {"f32": 4, "bf16": 2, "fp8": 1}
    B, T, S, H, D, k = w.B, w.T, w.S, w.index_n_heads, w.index_head_dim, w.index_topk
    pairs = B * causal_pairs(T, S)
    entries = B * selected_entries(T, S, k)
    ib = eb[w.idx_dtype]
    idx_bytes = B * S * D * ib + B * T * H * D * ib + B * T * H * 4
    idx_flops = pairs * 2 * H * D
    if S <= k:  # the dense limit: no scores are needed to select everything
        idx_bytes = idx_flops = 0
    attn_flops = entries * 2 * w.num_heads * (w.d_qk + w.d_v)
    io_bytes = B * T * w.num_heads * (w.d_qk * 2 + w.d_v * 2)
    if w.form == "mla":
        attn_bytes = entries * w.d_qk * 2 + io_bytes
    else:
        # every selected key/value row is read at least once: the union of the
        # selections, at most the whole cache of each sequence
        attn_bytes = min(entries, B * S) * w.num_heads * (w.d_qk + w.d_v) * 2 + io_bytes
    sel_bytes = B * T * k * 4
    return {"indexer_bytes": idx_bytes, "indexer_flops": idx_flops, "attn_bytes": attn_bytes,
            "attn_flops": attn_flops, "step_bytes": idx_bytes + attn_bytes + sel_bytes,
            "pairs": pairs, "entries": entries}


def kernel_source_hash(name: str) -> str:
    p = os.path.join(ROOT, "learned_sparse_attention_lightning_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_record(workload: str, kernel_file: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the summary is missing or the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha256_16") != kernel_source_hash(kernel_file):
        return None
    v = rec.get("hbm_bytes_per_launch")
    return None if v is None else int(round(v))


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 5), "p50": round(float(np.median(a)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "n": int(a.size)}


# ------------------------------------------------------------------ peaks --

def measure_peaks(read_bytes: int):
    """Achievable peaks of this device: a streaming read (16-byte nontemporal
    loads, four in flight a thread) of `read_bytes` and of 1 GiB, and MFMA
    issue loops (bf16 32x32x16, fp8 32x32x64) on register operands."""
    import torch
    from learned_sparse_attention_lightning_amd import build as hb
    if not os.path.exists(hb.PROBE_LIB):
        raise RuntimeError(f"{hb.PROBE_LIB} is missing: build with __graft_entry__.build()")
    lib = ctypes.CDLL(hb.PROBE_LIB)
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    for f in (lib.probe_mfma_bf16, lib.probe_mfma_fp8):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    for nbytes in sorted({read_bytes // 16 * 16, 1 << 30}):
        # 4 buffers rotated, so a launch never finds its data in the 256 MB cache;
        # the best of a few launch shapes is the device's achievable read rate
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(4)]
        for bb in bufs:
            bb.fill_(1)
        it = [0]
        best, shapes = 0.0, {}
        for blocks in (1024, 2048, 4096, 8192):
            for inflight in (4, 8):
                def rd():
                    bb = bufs[it[0] % 4]
                    it[0] += 1
                    rc = lib.probe_stream_read(ctypes.c_void_p(bb.data_ptr()), nbytes,
                                               ctypes.c_void_p(sink.data_ptr()), blocks,
                                               inflight, stream)
                    assert rc == 0, rc
                ms = timed(rd, 20)
                gbs = nbytes / (ms * 1e-3) / 1e9
                shapes[f"{blocks}x{inflight}"] = round(gbs, 1)
                best = max(best, gbs)
        out[f"stream_read_{nbytes}"] = round(best, 1)
        out[f"stream_read_{nbytes}_shapes"] = shapes
        del bufs
    iters, blocks = 4000, 512
    for name, fn, flop in (("mfma_bf16", lib.probe_mfma_bf16, 32768),
                           ("mfma_fp8", lib.probe_mfma_fp8, 131072)):
        ms = timed(lambda: fn(ctypes.c_void_p(sink.data_ptr()), iters, blocks, stream), 5)
        out[f"{name}_tflops"] = round(blocks * 4 * iters * 4 * flop / (ms * 1e-3) / 1e12, 1)
    return out


# ------------------------------------------------------------ cpu baseline --

def cpu_baseline(w, x, budget_s: float):
    """The oracle, untuned, on a bounded sample of the workload: whole decode
    steps (all sequences in one call, so OpenMP spreads them over the
    threads), or batches of random query rows of a prefill, as many as fit
    in the time budget."""
    import numpy as np

    import oracle
    oracle.build()
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    t0 = time.perf_counter()
    if w.decode:
        done = 0
        while True:
            sc = oracle.indexer_scores(x["q_idx"], x["k_idx"], x["w"])
            sel = oracle.topk(sc, w.index_topk)
            oracle.sparse_attention(w.form, x["q"], x["kv"], x["v"], sel, w.scale, d_v=w.d_v)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        el = time.perf_counter() - t0
        return {"value": done / el, "unit": "steps/s", "cores": min(threads, w.B * w.num_heads),
                "kind": "oracle",
                "sample": f"{done} whole step(s): indexer over {w.B} x {w.S} keys and top-"
                          f"{w.index_topk} ({min(threads, w.B)} threads, one a sequence), "
                          f"{w.num_heads}-head attention ({threads} threads); {el:.1f} s"}
    rows = []
    rng = np.random.default_rng(0)
    cand = [int(r) for r in rng.permutation(w.T)]
    batch = max(1, threads)
    while cand:
        rb, cand = cand[:batch], cand[batch:]
        rows += rb
        pos = np.array([rb])
        sc = oracle.indexer_scores(x["q_idx"][:, rb], x["k_idx"], x["w"][:, rb], q_pos=pos)
        sel = oracle.topk(sc, w.index_topk, q_pos=pos)
        oracle.sparse_attention(w.form, x["q"][:, rb], x["kv"], x["v"], sel, w.scale,
                                d_v=w.d_v)
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    # scale the sampled rows to whole-sequence work by their causal length
    frac = sum(r + 1 for r in rows) / sum(t + 1 for t in range(w.T))
    return {"value": w.T * w.B / (el / frac), "unit": "tokens/s", "cores": min(threads, batch),
            "kind": "oracle", "sample": f"{len(rows)} random query rows of {w.T} in batches of "
                                        f"{batch} (one thread a row), {el:.1f} s, scaled to the "
                                        "whole sequence by causal length"}


# ------------------------------------------------------------------ runs --

def setup(w, dev, replicas, include_current):
    import torch

    from learned_sparse_attention_lightning_amd import dsa, synth
    reps = [synth.make_inputs(w, device=dev, seed=synth.default_seed(w) + r)
            for r in range(replicas)]
    desc = dsa.desc_for(w)
    out = torch.empty((w.B, w.T, w.num_heads, w.d_v),
                      dtype=synth.TORCH_DTYPES[w.out_dtype], device=dev)
    idx = torch.empty((w.B, w.T, w.index_topk), dtype=torch.int32, device=dev)
    nws = dsa.workspace_bytes(dsa.DSA_OP_FORWARD, desc, w.B, w.T, w.S, w.index_n_heads,
                              w.index_head_dim, w.index_topk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def step(r):
        x = reps[r]
        dsa.dsa_forward(desc, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], x["v"],
                        w.index_topk, out=out, idx_out=idx, workspace=ws,
                        include_current=include_current)
    return reps, desc, out, idx, ws, step


def time_steps(step, R, steps, warmup, use_graph):
    """W untimed steps, then exactly K timed steps between two events (HIP
    graph replays when use_graph); returns (ms per step, host ms per step,
    graphs)."""
    import torch
    for s in range(warmup):
        step(s % R)
    torch.cuda.synchronize()
    graphs = None
    if use_graph:
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        for r in range(R):
            graphs[r].replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        if graphs:
            graphs[s % R].replay()
        else:
            step(s % R)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall_ms, graphs


def step_spread(step, graphs, R, blocks, per_block):
    """Step time of `blocks` blocks of `per_block` back-to-back steps each
    (one event pair a block): p10 / p50 / p90 over the blocks."""
    import torch
    times = []
    for blk in range(blocks):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for s in range(per_block):
            if graphs:
                graphs[(blk * per_block + s) % R].replay()
            else:
                step((blk * per_block + s) % R)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / per_block)
    return percentiles(times)


def decode_stage_ms(w, reps, desc, out, idx, R, nst, include_current, dev):
    """Average duration of each stage's launches: the three entry points issue
    exactly dsa_forward's launches for decode; each runs nst times back to back
    over the replicas between one pair of HIP events on the launch stream."""
    import torch

    from learned_sparse_attention_lightning_amd import dsa
    sc = torch.empty((w.B, w.T, w.S), dtype=torch.float32, device=dev)
    stages = [
        lambda x: dsa.dsa_indexer_scores(x["q_idx"], x["k_idx"], x["w"], scores=sc,
                                         causal_only=True),
        lambda x: dsa.dsa_topk(sc, w.index_topk, idx=idx, include_current=include_current),
        lambda x: dsa.dsa_sparse_attention(desc, x["q"], x["kv"], x["v"], idx, out=out,
                                           causal_prefix=True),
    ]
    for f in stages:  # inputs for the later stages, and warm launches
        for r in range(R):
            f(reps[r])
    torch.cuda.synchronize()
    res = []
    for f in stages:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for s in range(nst):
            f(reps[s % R])
        b.record()
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) / nst)
    return res


def prefill_stages(w, x, desc, out, idx, include_current, dev, kl=False):
    """Each stage with the forward pass's own launches: query rows in chunks of
    the forward's 1 GiB score block; the indexer writes only s <= t (the
    forward's flag) and sees the cache up to the chunk's last position, so
    every launch has the forward's grid and work; two timed passes after a
    warm one.  Returns (stage ms, chunk rows, launches, kl record or None)."""
    import torch

    from learned_sparse_attention_lightning_amd import dsa
    assert w.B == 1, "prefill stage timing takes one sequence"
    dense = w.S <= w.index_topk
    ch = max(1, min(w.T, SCORE_CHUNK_BYTES // (w.B * w.S * 4)))
    flat = torch.empty(w.B * ch * w.S, dtype=torch.float32, device=dev)
    chunks = []
    for r0 in range(0, w.T, ch):
        r1 = min(w.T, r0 + ch)
        s1 = w.S - w.T + r1   # the chunk's last position + 1
        chunks.append((r0, r1, s1, flat[: (r1 - r0) * s1].view(1, r1 - r0, s1)))

    def st_indexer():
        for r0, r1, s1, sc in chunks:
            dsa.dsa_indexer_scores(x["q_idx"][:, r0:r1], x["k_idx"][:, :s1], x["w"][:, r0:r1],
                                   scores=sc, causal_only=True)

    def st_topk():
        for r0, r1, s1, sc in chunks:
            dsa.dsa_topk(sc, w.index_topk, idx=idx[:, r0:r1], include_current=include_current)

    def st_attention():
        for r0, r1, s1, sc in chunks:
            dsa.dsa_sparse_attention(desc, x["q"][:, r0:r1], x["kv"][:, :s1],
                                     None if x["v"] is None else x["v"][:, :s1],
                                     idx[:, r0:r1], out=out[:, r0:r1], causal_prefix=True)

    stage_ms = []
    for f in (st_indexer, st_topk, st_attention):
        if dense and f is not st_attention:
            stage_ms.append(0.0)  # skipped by the forward pass
            continue
        f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(2):
            f()
        b.record()
        torch.cuda.synchronize()
        stage_ms.append(a.elapsed_time(b) / 2)
    kl_rec = None
    if kl and not dense:
        kl_rec = time_kl(w, x, desc, out, idx, chunks, dev)
    del flat
    return stage_ms, ch, len(chunks), kl_rec


def time_kl(w, x, desc, out, idx, chunks, dev):
    """The distillation-loss kernel per chunk: the chunk's scores and the
    attention's log-sum-exp are computed untimed, then the loss launch is
    timed (second pass kept)."""
    import torch

    from learned_sparse_attention_lightning_amd import dsa
    ch = max(r1 - r0 for r0, r1, _, _ in chunks)
    sc = torch.empty((w.B, ch, w.S), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, ch, w.num_heads), dtype=torch.float32, device=dev)
    loss = torch.empty((w.B, ch), dtype=torch.float32, device=dev)
    kl_ms = 0.0
    for rep in range(2):
        tot = 0.0
        for r0, r1, _, _ in chunks:
            n = r1 - r0
            pos = torch.arange(w.S - w.T + r0, w.S - w.T + r1, dtype=torch.int32,
                               device=dev).view(1, -1)
            dsa.dsa_indexer_scores(x["q_idx"][:, r0:r1], x["k_idx"], x["w"][:, r0:r1],
                                   q_pos=pos, scores=sc[:, :n])
            dsa.dsa_sparse_attention(desc, x["q"][:, r0:r1], x["kv"], x["v"], idx[:, r0:r1],
                                     out=out[:, r0:r1], lse=lse[:, :n])
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dsa.dsa_indexer_kl(desc, x["q"][:, r0:r1], x["kv"], idx[:, r0:r1], lse[:, :n],
                               sc[:, :n], loss=loss[:, :n])
            b.record()
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        kl_ms = tot
    alg = algorithmic(w)
    kl_flops = alg["entries"] * 2 * w.num_heads * w.d_qk
    kl_tf = kl_flops / (kl_ms * 1e-3) / 1e12
    # MLA and the MHA masked-dense form (bf16, k >= S/4): matrix-core
    # products; other MHA shapes: per-head dot products on the vector ALUs
    dense = dsa.workspace_bytes(dsa.DSA_OP_KL, desc, w.B, ch, w.S, 1, 1, w.index_topk) > 0
    if w.form == "mla":
        kpk, kb, kname = BF16_PEAK_TFLOPS, "mfma", "mla_indexer_kl_kernel"
    elif dense:
        kpk, kb = BF16_PEAK_TFLOPS, "mfma"
        kname = "mha_bitmap_kernel+mha_kl_dense_kernel+kl_split_merge_kernel"
    else:
        kpk, kb, kname = FP32_VECTOR_TFLOPS, "alu", "mha_indexer_kl_kernel"
    return {"bound": kb, "achieved": round(kl_tf, 2), "peak": kpk, "unit": "TFLOP/s",
            "frac": round(kl_tf / kpk, 4), "ms": round(kl_ms, 4),
            "kernel": kname, "algorithmic_flops": kl_flops}


def mfma_roof(flops, ms, peak, measured, kernel, launches):
    tf = flops / (ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
         "frac": round(tf / peak, 4), "kernel": kernel, "algorithmic_flops": flops,
         "ms": round(ms, 4), "launches": launches}
    if measured:
        r["measured_peak"] = measured
        r["frac_of_measured"] = round(tf / measured, 4)
    return r


def run_prefill(w, args, dev, peaks, with_cpu):
    """One prefill workload: throughput of whole forward steps, the stages
    with the forward's launches, their rooflines."""
    import torch
    cur = bool(args.include_current)
    reps, desc, out, idx, ws, step = setup(w, dev, 1, cur)
    steps = args.prefill_steps if args.workload != w.name else args.steps
    warm = 1 if args.workload != w.name else args.warmup
    ms, wall_ms, graphs = time_steps(step, 1, steps, warm, use_graph=False)
    per_step = []
    for _ in range(max(3, min(steps, 5))):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step(0)
        b.record()
        torch.cuda.synchronize()
        per_step.append(a.elapsed_time(b))
    alg = algorithmic(w)
    stage_ms, ch, nl, kl_rec = ([float("nan")] * 3, None, None, None)
    if args.stages:
        stage_ms, ch, nl, kl_rec = prefill_stages(w, reps[0], desc, out, idx, cur, dev,
                                                  kl=bool(args.kl))
    dense = w.S <= w.index_topk
    ipk = FP8_PEAK_TFLOPS if w.idx_dtype == "fp8" else BF16_PEAK_TFLOPS
    ipk_meas = peaks.get("mfma_fp8_tflops" if w.idx_dtype == "fp8" else "mfma_bf16_tflops")
    apk = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_VECTOR_TFLOPS
    apk_meas = peaks.get("mfma_bf16_tflops") if w.dtype == "bf16" else None
    # the stage time covers every launch of one attention call (for the MHA
    # masked-dense form: the selection bitmap, then the attention; inside the
    # forward the top-k writes that bitmap and only the attention runs)
    att_kernel = ("mla_attention_kernel" if w.form == "mla" else
                  "mha_bitmap_kernel+mha_fa_kernel" if w.dtype == "bf16" else
                  "attention_gather_kernel")
    rec = {
        "workload": f"{w.name}: {w.description}",
        "value": round(w.B * w.T / (ms * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": round(ms, 4), "steps": steps, "warmup": warm, "launch": "eager",
        "spread_ms": percentiles(per_step),
        "stage_ms": {"indexer": round(stage_ms[0], 4), "topk": round(stage_ms[1], 4),
                     "attention": round(stage_ms[2], 4)},
        "score_chunk_rows": ch, "chunks": nl,
        "attention_roofline": (mfma_roof(alg["attn_flops"], stage_ms[2], apk, apk_meas,
                                         att_kernel, nl) if args.stages else None),
        "indexer_roofline": (None if dense or not args.stages else
                             mfma_roof(alg["indexer_flops"], stage_ms[0], ipk, ipk_meas,
                                       f"indexer_prefill_kernel<{w.idx_dtype}>", nl)),
    }
    if kl_rec is not None:
        rec["indexer_kl_roofline"] = kl_rec
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, reps[0], args.cpu_seconds)
    host_ms = wall_ms
    del reps, out, idx, ws
    torch.cuda.empty_cache()
    return rec, ms, host_ms, alg


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path shards by "
              "sequence or query rows and is not built for several GPUs here.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from learned_sparse_attention_lightning_amd import configs

    w = configs.get(args.workload)
    dev = torch.device("cuda:0")
    cur = bool(args.include_current)
    dtype_name = "fp8+bf16" if w.idx_dtype == "fp8" else w.dtype

    if not w.decode:
        # a prefill workload as the headline
        peaks = measure_peaks(1 << 27) if args.peaks else {}
        rec, ms, host_ms, alg = run_prefill(w, args, dev, peaks, bool(args.cpu_baseline))
        res = {
            "metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype_name, "data": "synthetic",
            "config": {"workload": rec["workload"], "batch": w.B, "ctx": w.S,
                       "query_rows": w.T, "index_n_heads": w.index_n_heads,
                       "index_head_dim": w.index_head_dim, "index_topk": w.index_topk,
                       "form": w.form, "heads": w.num_heads, "d_qk": w.d_qk, "d_v": w.d_v,
                       "launch": "eager", "include_current": cur,
                       "dense_limit": w.S <= w.index_topk, "parallelism": "single-gpu"},
            "roofline": rec["attention_roofline"],
            "indexer_roofline": rec["indexer_roofline"],
            "host_ms_per_step": round(host_ms, 5),
            "stage_ms": rec["stage_ms"], "spread_ms": rec["spread_ms"],
            "score_chunk_rows": rec["score_chunk_rows"],
            "measured_peaks": peaks or None,
            "cpu_baseline": rec.get("cpu_baseline"),
        }
        if "indexer_kl_roofline" in rec:
            res["indexer_kl_roofline"] = rec["indexer_kl_roofline"]
        print(json.dumps(res), flush=True)
        return

    # ---- decode headline
    R = args.replicas or 4
    reps, desc, out, idx, ws, step = setup(w, dev, R, cur)
    ms, wall_ms, graphs = time_steps(step, R, args.steps, args.warmup, bool(args.graph))
    spread = step_spread(step, graphs, R, blocks=20, per_block=10)
    alg = algorithmic(w)
    stage_ms = [float("nan")] * 3
    if args.stages:
        stage_ms = decode_stage_ms(w, reps, desc, out, idx, R, max(20, args.steps), cur, dev)
    peaks = measure_peaks(alg["indexer_bytes"]) if args.peaks else {}
    kern_ms = stage_ms[0]
    achieved = alg["indexer_bytes"] / (kern_ms * 1e-3) / 1e9
    meas_bw = peaks.get(f"stream_read_{alg['indexer_bytes'] // 16 * 16}")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_record(w.name, "indexer.hip"),
            "kernel": f"indexer_stream_kernel<{w.idx_dtype}>",
            "algorithmic_bytes_per_launch": alg["indexer_bytes"],
            "avg_launch_ms": round(kern_ms, 5)}
    if meas_bw:
        roof["measured_peak"] = meas_bw
        roof["frac_of_measured"] = round(achieved / meas_bw, 4)
    value = 1e3 / ms
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_name, "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "batch": w.B, "ctx": w.S,
                   "query_rows": w.T, "index_n_heads": w.index_n_heads,
                   "index_head_dim": w.index_head_dim, "index_topk": w.index_topk,
                   "form": w.form, "heads": w.num_heads, "d_qk": w.d_qk, "d_v": w.d_v,
                   "input_replicas": R, "launch": "hip-graph" if graphs else "eager",
                   "include_current": cur, "parallelism": "single-gpu"},
        "roofline": roof,
        "host_ms_per_step": round(wall_ms, 5),
        "spread_ms": spread,
        "tokens_per_s": round(value * w.B, 1),
        "step_algorithmic_bytes": alg["step_bytes"],
        "step_hbm_frac": round(alg["step_bytes"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "stage_ms": {"indexer": round(stage_ms[0], 5), "topk": round(stage_ms[1], 5),
                     "attention": round(stage_ms[2], 5)},
        "measured_peaks": peaks or None,
    }
    if args.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, reps[0], args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    del reps, out, idx, ws, graphs
    torch.cuda.empty_cache()
    # ---- the prefill half of the metric
    if args.prefill_workload != "none":
        pw = configs.get(args.prefill_workload)
        if pw.decode:
            raise SystemExit("--prefill-workload must be a prefill workload")
        rec, _, _, _ = run_prefill(pw, args, dev, peaks, bool(args.cpu_baseline))
        res["prefill"] = rec
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
