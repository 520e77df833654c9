"""Throughput of the DSA forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

A step is one dsa_forward call (indexer scores -> top-k -> sparse attention)
over one batch of synthetic inputs already resident in HBM.  The default
workload is the 128K-context decode: 8 sequences of 131072 cached tokens, one
new query each, k = 2048, fp8 e4m3 indexer keys, MLA latent 576/512 bf16.
Decode inputs are rotated over several replicas so that consecutive steps do
not find the key cache in the last-level cache.

Prints one JSON line.  Besides the step throughput it carries:
  * roofline: the dominant kernel's algorithmic bytes (or flops) per launch
    over its average duration, timed with HIP events on the library's stream;
  * cpu_baseline: the CPU oracle timed on a bounded sample of the same
    workload on this host's cores.
"""
from __future__ import annotations

import argparse
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=["c1", "c2", "c2-fp8", "c3", "c4", "p128k", "short2k"])
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
    if w.form == "mla":
        attn_flops = entries * 2 * w.num_heads * (w.d_qk + w.d_v)
        attn_bytes = entries * w.d_qk * 2 + B * T * w.num_heads * (w.d_qk * 2 + w.d_v * 2)
    else:
        attn_flops = entries * 2 * w.num_heads * (w.d_qk + w.d_v)
        attn_bytes = entries * w.num_heads * (w.d_qk + w.d_v) * 2 + B * T * w.num_heads * (
            w.d_qk * 2 + w.d_v * 2)
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


def cpu_baseline(w, x, budget_s: float):
    """The oracle, untuned, on a bounded sample: whole sequences (decode) or
    whole query rows (prefill), as many as fit in the time budget."""
    import numpy as np

    import oracle
    oracle.build()
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    t0 = time.perf_counter()
    done = 0
    if w.decode:
        for b in range(w.B):
            sc = oracle.indexer_scores(x["q_idx"][b:b + 1], x["k_idx"][b:b + 1], x["w"][b:b + 1])
            sel = oracle.topk(sc, w.index_topk)
            oracle.sparse_attention(w.form, x["q"][b:b + 1], x["kv"][b:b + 1],
                                    None if x["v"] is None else x["v"][b:b + 1], sel, w.scale,
                                    d_v=w.d_v)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        el = time.perf_counter() - t0
        return {"value": done / w.B / el, "unit": "steps/s", "cores": cores, "kind": "oracle",
                "sample": f"{done} of {w.B} sequences of one step (indexer over {w.S} keys, "
                          f"top-{w.index_topk}, {w.num_heads}-head attention), {el:.1f} s"}
    rows = []
    rng = np.random.default_rng(0)
    cand = rng.permutation(w.T)
    for r in cand:
        rows.append(int(r))
        pos = np.array([[r]])
        sc = oracle.indexer_scores(x["q_idx"][:, [r]], x["k_idx"], x["w"][:, [r]], q_pos=pos)
        sel = oracle.topk(sc, w.index_topk, q_pos=pos)
        oracle.sparse_attention(w.form, x["q"][:, [r]], x["kv"], x["v"], sel, w.scale,
                                d_v=w.d_v)
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    # scale the sampled rows to whole-sequence work by their causal length
    frac = sum(r + 1 for r in rows) / sum(t + 1 for t in range(w.T))
    return {"value": w.T * w.B / (el / frac), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "sample": f"{len(rows)} random query rows of {w.T}, "
                                        f"{el:.1f} s, scaled by causal length"}


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

    from learned_sparse_attention_lightning_amd import configs, dsa, synth

    w = configs.get(args.workload)
    dev = torch.device("cuda:0")
    R = args.replicas or (4 if w.decode else 1)
    reps = [synth.make_inputs(w, device=dev, seed=synth.default_seed(w) + r) for r in range(R)]
    desc = dsa.desc_for(w)
    out = torch.empty((w.B, w.T, w.num_heads, w.d_v),
                      dtype=synth.TORCH_DTYPES[w.out_dtype], device=dev)
    idx = torch.empty((w.B, w.T, w.index_topk), dtype=torch.int32, device=dev)
    nws = dsa.workspace_bytes(dsa.DSA_OP_FORWARD, desc, w.B, w.T, w.S, w.index_n_heads,
                              w.index_head_dim, w.index_topk)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    cur = bool(args.include_current)
    # a context no longer than the budget selects everything: the forward pass
    # runs only the selection fill and the attention
    dense = w.S <= w.index_topk

    def step(r):
        x = reps[r]
        dsa.dsa_forward(desc, x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], x["v"],
                        w.index_topk, out=out, idx_out=idx, workspace=ws, include_current=cur)

    for s in range(args.warmup):
        step(s % R)
    torch.cuda.synchronize()

    graphs = None
    if args.graph:
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
    for s in range(args.steps):
        if graphs:
            graphs[s % R].replay()
        else:
            step(s % R)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps

    # ---- per-stage kernel durations (same kernels and launch shapes as the
    # step: for decode the three entry points issue exactly dsa_forward's
    # launches).  Each stage runs `nst` times back to back between one pair of
    # HIP events on the launch stream, so the average is the kernels' own
    # duration (plus the launch gaps), not the cost of an event pair.
    alg = algorithmic(w)
    stage_ms = None
    kl_roof = None
    if not args.stages:
        stage_ms = [float("nan")] * 3
    elif w.decode:
        sc = torch.empty((w.B, w.T, w.S), dtype=torch.float32, device=dev)
        nst = max(20, args.steps)
        stages = [
            lambda x: dsa.dsa_indexer_scores(x["q_idx"], x["k_idx"], x["w"], scores=sc),
            lambda x: dsa.dsa_topk(sc, w.index_topk, idx=idx, include_current=cur),
            lambda x: dsa.dsa_sparse_attention(desc, x["q"], x["kv"], x["v"], idx, out=out,
                                               causal_prefix=True),
        ]
        for f in stages:  # inputs for the later stages, and warm launches
            for r in range(R):
                f(reps[r])
        torch.cuda.synchronize()
        stage_ms = []
        for f in stages:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for s in range(nst):
                f(reps[s % R])
            b.record()
            torch.cuda.synchronize()
            stage_ms.append(a.elapsed_time(b) / nst)

    else:
        # prefill: each entry point over all query rows (the step runs the same
        # kernels on row chunks), in row chunks of at most 4 GiB of scores with
        # explicit positions; two timed runs after a warm one
        ch = max(1, min(w.T, (4 << 30) // (w.B * w.S * 4)))
        sc = torch.empty((w.B, ch, w.S), dtype=torch.float32, device=dev)
        x = reps[0]
        chunks = []
        for r0 in range(0, w.T, ch):
            r1 = min(w.T, r0 + ch)
            pos = None if ch == w.T else (torch.arange(w.S - w.T + r0, w.S - w.T + r1,
                                                       dtype=torch.int32, device=dev)
                                          .view(1, -1).repeat(w.B, 1))
            chunks.append((r0, r1, pos))

        def st_indexer():
            for r0, r1, pos in chunks:
                dsa.dsa_indexer_scores(x["q_idx"][:, r0:r1], x["k_idx"], x["w"][:, r0:r1],
                                       q_pos=pos, scores=sc[:, : r1 - r0])

        def st_topk():
            for r0, r1, pos in chunks:
                dsa.dsa_topk(sc[:, : r1 - r0], w.index_topk, q_pos=pos, idx=idx[:, r0:r1],
                             include_current=cur)

        def st_attention():
            for r0, r1, pos in chunks:
                # the forward pass's attention stops at each row's selected count
                dsa.dsa_sparse_attention(desc, x["q"][:, r0:r1], x["kv"], x["v"],
                                         idx[:, r0:r1], out=out[:, r0:r1], causal_prefix=True,
                                         q_pos=(pos if pos is not None else
                                                torch.arange(w.S - w.T + r0, w.S - w.T + r1,
                                                             dtype=torch.int32, device=dev)
                                                .view(1, -1).repeat(w.B, 1)))

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
        if args.kl:
            # the loss kernel needs each chunk's scores and the attention's
            # log-sum-exp: both computed untimed, then the loss launch timed
            lse = torch.empty((w.B, ch, w.num_heads), dtype=torch.float32, device=dev)
            loss = torch.empty((w.B, ch), dtype=torch.float32, device=dev)
            kl_ms = 0.0
            for rep in range(2):
                tot = 0.0
                for r0, r1, pos in chunks:
                    n = r1 - r0
                    dsa.dsa_indexer_scores(x["q_idx"][:, r0:r1], x["k_idx"], x["w"][:, r0:r1],
                                           q_pos=pos, scores=sc[:, :n])
                    dsa.dsa_sparse_attention(desc, x["q"][:, r0:r1], x["kv"], x["v"],
                                             idx[:, r0:r1], out=out[:, r0:r1], lse=lse[:, :n])
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    dsa.dsa_indexer_kl(desc, x["q"][:, r0:r1], x["kv"], idx[:, r0:r1],
                                       lse[:, :n], sc[:, :n], loss=loss[:, :n])
                    b.record()
                    torch.cuda.synchronize()
                    tot += a.elapsed_time(b)
                kl_ms = tot  # the second pass (warm) is kept
            kl_flops = alg["entries"] * 2 * w.num_heads * w.d_qk
            kl_tf = kl_flops / (kl_ms * 1e-3) / 1e12
            # MLA: matrix-core products; MHA: per-head dot products on the
            # vector ALUs (fp32 FMA peak)
            kpk, kb = (BF16_PEAK_TFLOPS, "mfma") if w.form == "mla" else (157.3, "alu")
            kl_roof = {"bound": kb, "achieved": round(kl_tf, 2), "peak": kpk,
                       "unit": "TFLOP/s", "frac": round(kl_tf / kpk, 4),
                       "ms": round(kl_ms, 4),
                       "kernel": f"{w.form}_indexer_kl_kernel",
                       "algorithmic_flops": kl_flops}
        del sc

    if w.decode:
        kern_ms = stage_ms[0]
        achieved = alg["indexer_bytes"] / (kern_ms * 1e-3) / 1e9
        tr = traffic_record(w.name, "indexer.hip")
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": tr,
                "kernel": f"indexer_stream_kernel<{w.idx_dtype}>",
                "algorithmic_bytes_per_launch": alg["indexer_bytes"],
                "avg_launch_ms": round(kern_ms, 5)}
        value = 1e3 / ms
        unit = "steps/s"
    else:
        value = w.B * w.T / (ms * 1e-3)
        unit = "tokens/s"
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else 157.3  # fp32: vector peak
        # dominant kernel: the attention (MFMA for MLA); the indexer's MFMA
        # fraction is reported beside it
        att = alg["attn_flops"] / (stage_ms[2] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(att, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(att / peak, 4), "traffic": None,
                "kernel": "mla_attention_kernel" if w.form == "mla" else "mha attention",
                "algorithmic_flops_per_launch": alg["attn_flops"],
                "avg_launch_ms": round(stage_ms[2], 4)}
        ipk = FP8_PEAK_TFLOPS if w.idx_dtype == "fp8" else BF16_PEAK_TFLOPS
        if dense or not stage_ms[0] > 0:
            indexer_roof = None
        else:
            ind = alg["indexer_flops"] / (stage_ms[0] * 1e-3) / 1e12
            indexer_roof = {"bound": "mfma", "achieved": round(ind, 2), "peak": ipk,
                            "unit": "TFLOP/s", "frac": round(ind / ipk, 4),
                            "avg_launch_ms": round(stage_ms[0], 4)}

    res = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16" if w.idx_dtype == "fp8" else w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "batch": w.B, "ctx": w.S,
                   "query_rows": w.T, "index_n_heads": w.index_n_heads,
                   "index_head_dim": w.index_head_dim, "index_topk": w.index_topk,
                   "form": w.form, "heads": w.num_heads, "d_qk": w.d_qk, "d_v": w.d_v,
                   "input_replicas": R, "launch": "hip-graph" if graphs else "eager",
                   "include_current": cur, "dense_limit": dense,
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "host_ms_per_step": round(wall_ms, 5),
        "step_algorithmic_bytes": alg["step_bytes"],
        "step_hbm_frac": round(alg["step_bytes"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
    }
    res["stage_ms"] = {"indexer": round(stage_ms[0], 5), "topk": round(stage_ms[1], 5),
                       "attention": round(stage_ms[2], 5)}
    if w.decode:
        res["tokens_per_s"] = round(value * w.B, 1)
    else:
        res["indexer_roofline"] = indexer_roof
    if kl_roof is not None:
        res["indexer_kl_roofline"] = kl_roof
    if args.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, reps[0], args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
