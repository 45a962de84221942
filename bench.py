"""Benchmark of one DSA decode step on one MI355X.

A step is one pass of the whole hot path over one batch: dsa_index_score ->
dsa_topk -> dsa_sparse_mla_attn on the batched-decode workload (32 sequences x
32768 cached rows, 32 indexer heads x 128, top-k 2048, 64 MLA heads over a 576-wide
bf16 latent cache), inputs resident in HBM. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode graph|eager]

value = decode tokens/s (sequences per step / step time). The roofline object is for
the dominant kernel (the indexer-score kernel, HBM-bound): algorithmic bytes per launch
/ its average duration measured with HIP events on the launch stream over the timed
region. cpu_baseline is the CPU oracle timed on a bounded sample of the same workload.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
DEFAULT_WORKLOAD = "batched_decode_b32_32k"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_index_score.json")


def algorithmic_bytes(wl):
    """Bytes the method itself must move per step (not the full cache it avoids)."""
    isz = 4 if wl.idx_dtype == 0 else 2
    msz = 4 if wl.mla_dtype == 0 else 2
    rows = wl.B * wl.n_q
    keys = wl.B * wl.n_kv * wl.D * isz
    q = rows * wl.H * wl.D * isz
    w = rows * wl.H * 4
    scores = rows * wl.n_kv * 4
    idx = rows * wl.top_k * 4
    qa = rows * wl.Hm * wl.Dc * msz
    gather = rows * wl.top_k * wl.Dc * msz
    out = rows * wl.Hm * wl.d_latent * 4
    lse = rows * wl.Hm * 4
    return {
        "index_score": keys + q + w + scores,
        "topk": scores + idx,
        "sparse_mla": idx + qa + gather + out + lse,
        "step": keys + q + w + 2 * scores + 2 * idx + qa + gather + out + lse,
    }


def prep_bytes(wl):
    """Bytes of the indexer-input preparation of the step's new tokens: fp32 q and k in, q
    out and the k row in the indexer dtype, the latent row in and out, the positions."""
    isz = 4 if wl.idx_dtype == 0 else 2
    msz = 4 if wl.mla_dtype == 0 else 2
    tok = wl.B * wl.n_q
    return tok * (wl.H * wl.D * (4 + isz) + wl.D * (4 + isz) + 2 * wl.Dc * msz + 4)


def score_flops(wl, causal=True):
    """Indexer contraction flops (2 * H * D per scored (query, key) pair)."""
    import numpy as np
    pos = wl.q_pos()[0].astype(np.int64)
    pairs = int(np.minimum(pos + 1, wl.n_kv).sum()) * wl.B if causal else wl.B * wl.n_q * wl.n_kv
    return 2 * wl.H * wl.D * pairs


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("index_score.hip", "common.h"):
        with open(os.path.join(ROOT, "sparse_attention_10_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(wl_name):
    """HBM bytes per launch of the score kernel from rocprofv3 counters, if they were taken
    on the current kernel source for this workload (else None)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_source_hash() or t.get("workload") != wl_name:
        return None
    return t.get("bytes_per_launch")


def _counter_rows(path, counter):
    """(dispatch id, kernel name, value in KiB) of one counter from a counter_collection.csv."""
    import csv
    rows = []
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def write_traffic(wl_name, fetch_csv, write_csv, copy_mib):
    """HBM bytes per launch of the score kernel: its mean FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each divided by the factor the same counter reads for the calibration copy
    (the last three copy-kernel dispatches, copy_mib MiB read and written)."""
    if copy_mib <= 0:
        sys.exit("--traffic-from needs --copy-calibration-mib (the size the counted runs copied)")
    copy_bytes = copy_mib * 1024 * 1024
    out = {"workload": wl_name, "kernel_sha": kernel_source_hash(), "copy_bytes": copy_bytes}
    total = 0.0
    for tag, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _counter_rows(path, counter)
        copies = [v for _, name, v in rows if "copyBuffer" in name][-3:]
        score = [v for _, name, v in rows if "index_score_" in name]
        if len(copies) < 3 or not score:
            sys.exit(f"{path}: no calibration copies or score dispatches with {counter}")
        factor = sum(copies) / len(copies) * 1024 / copy_bytes
        per = sum(score) / len(score) * 1024 / factor
        out[tag] = {"counter": counter, "copy_kib": sum(copies) / len(copies), "factor": round(factor, 4),
                    "kernel_kib": sum(score) / len(score), "dispatches": len(score), "bytes_per_launch": round(per)}
        total += per
    out["bytes_per_launch"] = round(total)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def kpool_bytes(wl, width):
    """Algorithmic bytes of one pooled-indexer decode step: pool keys, q, w, the pool scores
    written and read, pool indices written and read, the valid entries of the selected tokens,
    token indices written and read, the absorbed query, the selected latent rows, out, lse."""
    rows = wl.B * wl.n_q
    n_pool, kp = wl.n_kv // wl.kpool, wl.top_k // wl.kpool
    isz, msz = 2, 2
    score = wl.B * n_pool * wl.D * isz + rows * wl.H * (wl.D * isz + 4) + rows * n_pool * 4
    topk = rows * n_pool * 4 + rows * kp * 4
    expand = rows * kp * 4 + rows * width * (isz + 4)
    mla = rows * width * 4 + rows * wl.Hm * wl.Dc * msz + rows * width * wl.Dc * msz + rows * wl.Hm * (wl.d_latent + 1) * 4
    # the fused call reads the pool indices and the valid entries and never writes token indices
    fused = rows * kp * 4 + rows * width * isz + mla - rows * width * 4
    return {"index_score": score, "topk": topk, "expand": expand, "sparse_mla": mla,
            "step": score + topk + expand + mla, "fused_sparse_mla": fused, "fused_step": score + topk + fused}


def kpool_leg(dsa, dev, steps, warmup, seed):
    """The pooled-indexer (kpool) decode step at the batched 32K decode shape, timed like the main
    step: compress the cache's complete pools once (the prefill-time cost), then K steps of
    pool scores -> top-k over pools -> sparse MLA (no rope) that expands the pools to tokens
    itself, replayed from a graph (and the same step with the expansion as a call of its own);
    per-call times from HIP events in an eager pass. Inputs are drawn on the device
    from torch's seeded generator with the distributions of workloads.gen_kpool."""
    import torch
    import workloads
    wl = workloads.KPOOL_DECODE_32K
    g = torch.Generator(device=dev).manual_seed(seed + 5)
    B, n_kv, D, kpool = wl.B, wl.n_kv, wl.D, wl.kpool
    n_pool, kp = n_kv // kpool, wl.top_k // kpool
    width = kpool * kp + kpool - 1
    kv_len = torch.tensor([n_kv - (b % kpool) for b in range(B)], dtype=torch.int32, device=dev)
    packed = torch.empty((B, n_kv, 2 * D + 1), dtype=torch.float16, device=dev)
    packed[:, :, :D] = torch.randn((B, n_kv, D), generator=g, device=dev) / D ** 0.5
    packed[:, :, D:2 * D] = torch.randn((B, n_kv, D), generator=g, device=dev)
    packed[:, :, 2 * D] = (torch.arange(n_kv, device=dev)[None] < kv_len[:, None].long()).half()
    ape = torch.randn((kpool, D), generator=g, device=dev)
    q = (torch.randn((B, 1, wl.H, D), generator=g, device=dev) / D ** 0.5).half()
    w = torch.rand((B, 1, wl.H), generator=g, device=dev) * wl.w_scale
    qa = torch.randn((B, 1, wl.Hm, wl.Dc), generator=g, device=dev).bfloat16()
    lat = (torch.randn((B, n_kv, wl.Dc), generator=g, device=dev) * wl.latent_std).bfloat16()
    pooled = torch.empty((B, n_pool, D), dtype=torch.float16, device=dev)
    scores = torch.empty((B, 1, n_pool), dtype=torch.float32, device=dev)
    pidx = torch.empty((B, 1, kp), dtype=torch.int32, device=dev)
    tok = torch.empty((B, 1, width), dtype=torch.int32, device=dev)
    out = torch.empty((B, 1, wl.Hm, wl.d_latent), dtype=torch.float32, device=dev)
    lse = torch.empty((B, 1, wl.Hm), dtype=torch.float32, device=dev)
    ns = dsa.dsa_sparse_mla_num_splits(B, 1, width)
    ws_t = torch.empty(max(1, dsa.dsa_topk_workspace_size(B, n_pool, kp)), dtype=torch.uint8, device=dev)
    ws_m = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(B, 1, wl.Hm, width, wl.d_latent, ns)),
                       dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def compress_all():
        dsa.dsa_kpool_compress(packed, ape, pooled, D, kpool)

    score_call = lambda: dsa.dsa_kpool_index_score(q, pooled, w, scores, kpool, kv_len=kv_len, scale=wl.scale)  # noqa: E731
    topk_call = lambda: dsa.dsa_topk(scores, pidx, kp, workspace=ws_t)  # noqa: E731
    # the step: pool scores, top-k over pools, and the attention call that expands the pools itself
    calls = {
        "index_score": score_call,
        "topk": topk_call,
        "sparse_mla": lambda: dsa.dsa_kpool_sparse_mla_attn(qa, lat, pidx, packed, D, kpool, out, wl.d_latent,
                                                            wl.sm_scale, lse=lse, kv_len=kv_len, n_split=ns,
                                                            workspace=ws_m),
    }
    # the same step with the expansion as a call of its own
    two_calls = {
        "index_score": score_call,
        "topk": topk_call,
        "expand": lambda: dsa.dsa_kpool_expand(pidx, packed, D, tok, kpool, kv_len=kv_len),
        "sparse_mla": lambda: dsa.dsa_sparse_mla_attn(qa, lat, tok, out, wl.d_latent, wl.sm_scale, lse=lse,
                                                      kv_len=kv_len, n_split=ns, workspace=ws_m),
    }

    def kstep():
        for f in calls.values():
            f()

    def kstep_two():
        for f in two_calls.values():
            f()

    for _ in range(3):
        compress_all()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        compress_all()
    e1.record(stream)
    torch.cuda.synchronize()
    compress_ms = e0.elapsed_time(e1) / 10
    compress_b = B * n_kv * (2 * D + 1) * 2 + B * n_pool * D * 2 + kpool * D * 4
    for _ in range(max(1, warmup)):
        kstep()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    for s_ in range(steps):
        ev[s_][0].record(stream)
        for j, f in enumerate(calls.values()):
            f()
            ev[s_][j + 1].record(stream)
    torch.cuda.synchronize()
    per = {name: sum(ev[s_][j].elapsed_time(ev[s_][j + 1]) for s_ in range(steps)) / steps
           for j, name in enumerate(calls)}
    def graph_time(fn):
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        for _ in range(max(1, warmup)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    step_s = graph_time(kstep)
    two_s = graph_time(kstep_two)
    ab = kpool_bytes(wl, width)
    ab["sparse_mla"] = ab["fused_sparse_mla"]
    return {"workload": wl.name, "B": B, "n_kv": n_kv, "kpool": kpool, "top_k_tokens": wl.top_k,
            "pools_selected": kp, "attended_width": width, "d_rope": wl.d_rope, "indexer_dtype": "f16",
            "ms_per_step": round(step_s * 1e3, 4), "tokens_per_s": round(B / step_s, 1),
            "step_algorithmic_bytes": ab["fused_step"], "step_hbm_gbs": round(ab["fused_step"] / step_s / 1e9, 1),
            "step_hbm_frac": round(ab["fused_step"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
            "expansion_as_own_call_ms_per_step": round(two_s * 1e3, 4),
            "kernels_ms": {k_: round(v, 4) for k_, v in per.items()},
            "kernels_gbs": {k_: round(ab[k_] / (per[k_] * 1e-3) / 1e9, 1) for k_ in per},
            "compress_all_pools": {"ms": round(compress_ms, 4), "bytes": compress_b,
                                   "gbs": round(compress_b / (compress_ms * 1e-3) / 1e9, 1),
                                   "frac": round(compress_b / (compress_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def cpu_baseline(wl, inp, seconds_target=15.0):
    """The oracle chain on whole sequences of the workload, cycling over the batch, until about
    seconds_target of work."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        cores = max(int(i.get("num_threads", 1)) for i in threadpoolctl.threadpool_info()) \
            if threadpoolctl.threadpool_info() else 1
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    done = 0
    t0 = time.perf_counter()
    while True:
        b = done % wl.B
        sl = slice(b, b + 1)
        sub = {k: v[sl] for k, v in inp.items() if k != "kv_len"}
        sub["kv_len"] = inp["kv_len"][sl]
        S = oracle.index_score(sub["q"], sub["k"], sub["w"], sub["kv_len"], sub["q_pos"] if wl.q_pos_start is not None else None,
                               wl.scale, wl.idx_dtype, wl.idx_dtype)
        idx = oracle.topk(S.reshape(-1, wl.n_kv), wl.top_k).reshape(1, wl.n_q, wl.top_k)
        oracle.sparse_mla(sub["qa"], sub["latent"], idx, wl.sm_scale, wl.d_latent, wl.mla_dtype, sub["kv_len"])
        done += 1
        if time.perf_counter() - t0 > seconds_target:
            break
    dt = time.perf_counter() - t0
    tokens = done * wl.n_q
    seqs = f"sequences 0..{done - 1}" if done <= wl.B else f"{done} sequences ({done / wl.B:.1f} passes over the {wl.B})"
    return {"value": tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle chain (score, top-k, sparse MLA) on {seqs} of {wl.name} "
                      f"({tokens} tokens, {dt:.1f} s, float64 numpy with {cores} BLAS threads)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tune", action="append", default=[], metavar="KEY=VALUE",
                    help="dsa_set_tuning before the run (repeatable)")
    ap.add_argument("--pipelines", type=int, default=1,
                    help="run the step as this many chains over equal slices of the batch, each on its "
                         "own stream, so one slice's latency-bound stages overlap another's streaming")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kpool", action="store_true",
                    help="skip the pooled-indexer (kpool) decode leg of the bench line")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--scrub-mib", type=int, default=0,
                    help="also time eager steps with a buffer of this many MiB written between them "
                         "(steps that start with cold caches)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the bench, run 3 device-to-device copies of this many MiB (the known-size "
                         "copy that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="read two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE run, WRITE_SIZE "
                         "run of this script with --copy-calibration-mib) and write the score kernel's "
                         "HBM bytes per launch to profiles/traffic_index_score.json; no GPU work")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(args.workload, args.traffic_from[0], args.traffic_from[1], args.copy_calibration_mib)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path is run and reported per GPU only (--gpus 1); "
              "a run over several GPUs is not part of this library.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    from sparse_attention_10_amd import dsa

    for kv_ in args.tune:
        key_, val_ = kv_.split("=")
        dsa.dsa_set_tuning(key_, int(val_))
    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    inp = workloads.gen_all(wl, args.seed)
    print(f"[bench] generated {wl.name} inputs in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def to_dev(a, code=None):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16 if code == workloads.BF16 else torch.float16)
        else:
            t = torch.from_numpy(a)
        return t.to(dev)

    q = to_dev(inp["q"], wl.idx_dtype)
    k = to_dev(inp["k"], wl.idx_dtype)
    w = to_dev(inp["w"])
    qa = to_dev(inp["qa"], wl.mla_dtype)
    lat = to_dev(inp["latent"], wl.mla_dtype)
    kv_len = to_dev(inp["kv_len"])
    q_pos = to_dev(inp["q_pos"]) if wl.q_pos_start is not None else None
    rows = wl.B * wl.n_q
    scores = torch.empty((wl.B, wl.n_q, wl.n_kv), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.B, wl.n_q, wl.top_k), dtype=torch.int32, device=dev)
    out = torch.empty((wl.B, wl.n_q, wl.Hm, wl.d_latent), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.B, wl.n_q, wl.Hm), dtype=torch.float32, device=dev)
    n_split = dsa.dsa_sparse_mla_num_splits(wl.B, wl.n_q, wl.top_k)
    ws_t = torch.empty(max(1, dsa.dsa_topk_workspace_size(rows, wl.n_kv, wl.top_k)), dtype=torch.uint8, device=dev)
    ws_m = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(wl.B, wl.n_q, wl.Hm, wl.top_k, wl.d_latent, n_split)),
                       dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def call_score():
        dsa.dsa_index_score(q, k, w, scores, kv_len=kv_len, q_pos=q_pos, scale=wl.scale)

    def call_topk():
        dsa.dsa_topk(scores, idx, wl.top_k, workspace=ws_t)

    def call_mla():
        dsa.dsa_sparse_mla_attn(qa, lat, idx, out, wl.d_latent, wl.sm_scale, lse=lse, kv_len=kv_len,
                                n_split=n_split, workspace=ws_m)

    def step():
        call_score()
        call_topk()
        call_mla()

    # the step as P chains over batch slices on P streams (default priority), joined at the end
    P = args.pipelines
    if P < 1 or wl.B % P != 0:
        print(f"--pipelines must divide B={wl.B}", file=sys.stderr)
        sys.exit(2)
    parts = []
    if P > 1:
        hb = wl.B // P
        for p_ in range(P):
            sl = slice(p_ * hb, (p_ + 1) * hb)
            ns_p = dsa.dsa_sparse_mla_num_splits(hb, wl.n_q, wl.top_k)
            parts.append({
                "sl": sl, "ns": ns_p, "stream": torch.cuda.Stream(),
                "ws_t": torch.empty(max(1, dsa.dsa_topk_workspace_size(hb * wl.n_q, wl.n_kv, wl.top_k)),
                                    dtype=torch.uint8, device=dev),
                "ws_m": torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(hb, wl.n_q, wl.Hm, wl.top_k,
                                                                             wl.d_latent, ns_p)),
                                    dtype=torch.uint8, device=dev)})

    def pstep():
        if P == 1:
            step()
            return
        cur = torch.cuda.current_stream()
        for part in parts:
            sl, st = part["sl"], part["stream"]
            st.wait_stream(cur)
            with torch.cuda.stream(st):
                dsa.dsa_index_score(q[sl], k[sl], w[sl], scores[sl], kv_len=kv_len[sl],
                                    q_pos=q_pos[sl] if q_pos is not None else None, scale=wl.scale)
                dsa.dsa_topk(scores[sl], idx[sl], wl.top_k, workspace=part["ws_t"])
                dsa.dsa_sparse_mla_attn(qa[sl], lat[sl], idx[sl], out[sl], wl.d_latent, wl.sm_scale, lse=lse[sl],
                                        kv_len=kv_len[sl], n_split=part["ns"], workspace=part["ws_m"])
        for part in parts:
            cur.wait_stream(part["stream"])

    # warmup (also the eager reference of one step)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    # per-call durations: HIP events on the launch stream around each call, eager, K steps
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        call_score()
        ev[s][1].record(stream)
        call_topk()
        ev[s][2].record(stream)
        call_mla()
        ev[s][3].record(stream)
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t0) / args.steps
    per = {"index_score": 0.0, "topk": 0.0, "sparse_mla": 0.0}
    for s in range(args.steps):
        per["index_score"] += ev[s][0].elapsed_time(ev[s][1])
        per["topk"] += ev[s][1].elapsed_time(ev[s][2])
        per["sparse_mla"] += ev[s][2].elapsed_time(ev[s][3])
    per = {k_: v / args.steps for k_, v in per.items()}  # ms

    # the timed region: K steps, graph replay (launch overhead captured once) or eager
    if args.mode == "graph":
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            pstep()  # first call outside capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            pstep()
        for _ in range(max(1, args.warmup)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        step_s = (time.perf_counter() - t0) / args.steps
        # a layer that shares the previous full layer's indices runs the attention only
        gm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gm):
            call_mla()
        for _ in range(max(1, args.warmup)):
            gm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            gm.replay()
        torch.cuda.synchronize()
        shared_s = (time.perf_counter() - t0) / args.steps
    else:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            pstep()
        torch.cuda.synchronize()
        step_s = (time.perf_counter() - t0) / args.steps
        t0 = time.perf_counter()
        for _ in range(args.steps):
            call_mla()
        torch.cuda.synchronize()
        shared_s = (time.perf_counter() - t0) / args.steps

    # indexer-input preparation of the step's new tokens (the stage upstream of the scores):
    # timed on its own with HIP events, after the timed region, writing the same cache rows
    prep_in = workloads.gen_prep(wl, args.seed)
    p_q = to_dev(prep_in["q_in"])
    p_k = to_dev(prep_in["k_in"])
    p_lat = to_dev(prep_in["latent_in"], wl.mla_dtype)
    p_pos = to_dev(prep_in["pos"])
    p_qout = torch.empty(q.shape, dtype=q.dtype, device=dev)

    def call_prep():
        dsa.dsa_indexer_prep(p_pos, q_in=p_q, q_out=p_qout, k_in=p_k, k_cache=k, latent_in=p_lat,
                             latent_cache=lat)

    for _ in range(5):
        call_prep()
    torch.cuda.synchronize()
    # a few microseconds of GPU work per call: the host cannot queue single calls fast enough,
    # so a graph of 20 calls is replayed and the time per call taken from that
    pg = torch.cuda.CUDAGraph()
    pside = torch.cuda.Stream()
    pside.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(pside):
        call_prep()
    torch.cuda.current_stream().wait_stream(pside)
    torch.cuda.synchronize()
    with torch.cuda.graph(pg):
        for _ in range(20):
            call_prep()
    pg.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // 20)
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record(stream)
    for _ in range(reps):
        pg.replay()
    pe1.record(stream)
    torch.cuda.synchronize()
    prep_ms = pe0.elapsed_time(pe1) / (reps * 20)

    kpool = None
    if not args.no_kpool and wl.n_q == 1:
        kpool = kpool_leg(dsa, dev, args.steps, args.warmup, args.seed)

    # a plain device-to-device copy of 1 GiB: the bandwidth a streaming kernel reaches here
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record(stream)
    for _ in range(3):
        cdst.copy_(csrc)
    ce1.record(stream)
    ce1.synchronize()
    copy_gbs = 3 * 2 * (1 << 30) / (ce0.elapsed_time(ce1) * 1e-3) / 1e9
    del csrc, cdst

    scrub = None
    if args.scrub_mib > 0:
        buf = torch.empty(args.scrub_mib << 20, dtype=torch.uint8, device=dev)
        se = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):  # the fill runs between the event pairs, outside them
            buf.fill_(i & 255)
            se[i][0].record(stream)
            step()
            se[i][1].record(stream)
        torch.cuda.synchronize()
        tot = sum(a.elapsed_time(b) for a, b in se)
        scrub = {"scrub_mib": args.scrub_mib, "ms_per_step": round(tot / args.steps, 4)}
        del buf

    ab = algorithmic_bytes(wl)
    tokens = rows
    # IndexShare over GLM-5.2's 78 DSA layers: full layers run the whole step, shared layers
    # reuse the last full layer's indices and run the attention only
    n_full = sum(dsa.dsa_layer_computes_topk(l) for l in range(78))
    per_layer_s = (n_full * step_s + (78 - n_full) * shared_s) / 78
    value = tokens / step_s
    score_ms = per["index_score"]
    achieved = ab["index_score"] / (score_ms * 1e-3) / 1e9
    traffic = load_traffic(wl.name)
    prefill = wl.n_q > 1
    if prefill:
        fl = score_flops(wl)
        tfl = fl / (score_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tfl, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": "index_score_prefill_mfma", "flops_per_launch": fl,
                "dense_frac": round(score_flops(wl, causal=False) / (score_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "index_score_decode_mfma", "bytes_per_launch": ab["index_score"]}
    result = {
        "metric": "DSA decode tokens/s at 32K ctx (batch 32) + achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "n_q": wl.n_q, "n_kv": wl.n_kv, "H": wl.H, "D": wl.D,
                   "top_k": wl.top_k, "Hm": wl.Hm, "d_latent": wl.d_latent, "d_rope": wl.d_rope,
                   "indexer_dtype": workloads.DTYPE_NAMES[wl.idx_dtype],
                   "latent_dtype": workloads.DTYPE_NAMES[wl.mla_dtype], "mode": args.mode,
                   "mla_splits": n_split, "pipelines": P, "tuning": args.tune, "parallelism": "single GPU"},
        "step_hbm_gbs": round(ab["step"] / step_s / 1e9, 1),
        "step_hbm_frac": round(ab["step"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": ab["step"],
        "eager_ms_per_step": round(eager_s * 1e3, 4),
        "kernels_ms": {k_: round(v, 4) for k_, v in per.items()},
        "kernels_gbs": {k_: round(ab[k_] / (per[k_] * 1e-3) / 1e9, 1) for k_ in per},
        "roofline": roof,
        "indexshare": {"full_layers": n_full, "shared_layers": 78 - n_full,
                       "shared_layer_ms": round(shared_s * 1e3, 4),
                       "ms_per_layer": round(per_layer_s * 1e3, 4),
                       "tokens_per_s_per_layer": round(tokens / per_layer_s, 1)},
        "copy_gbs": round(copy_gbs, 1),
        "score_frac_of_copy": round(achieved / copy_gbs, 4) if not prefill else None,
        "indexer_prep": {"ms": round(prep_ms, 4), "bytes": prep_bytes(wl),
                         "gbs": round(prep_bytes(wl) / (prep_ms * 1e-3) / 1e9, 1),
                         "frac": round(prep_bytes(wl) / (prep_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "tokens": rows},
        "context": "whole-model figures on other hardware (not comparable): GLM-5.2 IQ2_XXS greedy decode "
                   "~0.3-0.4 tokens/s and 200-token prefill ~3.2 tokens/s on an RTX 4060 Ti 16GB with SSD "
                   "expert streaming",
    }
    if kpool is not None:
        result["kpool"] = kpool
    if scrub is not None:
        result["cold_cache_eager"] = scrub
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
        # the same oracle on one thread (BLAS limited to 1), a shorter sample
        try:
            import threadpoolctl
            with threadpoolctl.threadpool_limits(limits=1):
                one = cpu_baseline(wl, inp, max(1.0, args.cpu_seconds / 3))
            result["cpu_baseline"]["single_thread"] = {"value": one["value"], "unit": one["unit"],
                                                       "cores": one["cores"], "sample": one["sample"]}
        except ImportError:
            pass
    print(json.dumps(result), flush=True)
    if args.copy_calibration_mib > 0:
        del q, k, w, qa, lat, scores, idx, out, lse, ws_t, ws_m, p_q, p_k, p_lat, p_qout
        n = args.copy_calibration_mib * 1024 * 1024
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration: 3 copies of {args.copy_calibration_mib} MiB", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
