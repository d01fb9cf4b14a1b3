#!/usr/bin/env python3
"""Benchmark of the MIS hot path on one MI355X.

One step = the whole hot path over one batch already resident in HBM:
``mis_build_segments`` (host checks, metadata upload, builder kernels),
``mis_attention_prefill`` (bf16 MFMA MIS attention) and ``mis_score_labels``
(readout gather, LM head, split-vocab logsumexp, label log-probs).

Default workload: the long-prefix batch, the largest single-GPU workload
(4 requests of a 16384-token prefix and 256 items of 48 tokens plus a closing
delimiter; GQA 64 query / 8 KV heads, head_dim 128, bf16; label scoring with
hidden 8192, vocabulary 128256, 3 labels). ``--config 2`` and ``--config 3``
select the single-request and profile-labeling workloads. Inputs are seeded
synthetic data shaped like the pages' workloads (one long shared prefix,
tens to hundreds of short items).

Prints one JSON line. ``value`` is the unmasked attention rate: 4*D*Hq
times the number of (query, key) pairs the MIS mask lets through, divided by
the attention kernel's mean duration over the timed steps (HIP events on the
launch stream around every call). ``item_scores_per_s`` is items divided by
the whole step time.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MIS prefill attention TFLOP/s (unmasked) + item scores/sec, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4 SIMD x 1024 bf16 FLOP/clk x 2.4 GHz (dense MFMA)
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def visible_pairs(wl, items_only: bool = False) -> int:
    """(query, key) pairs the MIS mask allows, summed over requests (one head);
    with ``items_only`` the item rows' pairs only (appending items to a cached
    prefix)."""
    total = 0
    lens = wl.item_lengths()
    for r in range(wl.num_requests):
        lq = int(wl.prefix_lens[r])
        s = lens[int(wl.cu_items[r]) : int(wl.cu_items[r + 1])].astype(np.int64)
        if not items_only:
            total += lq * (lq + 1) // 2
        total += int((s * lq + s * (s + 1) // 2).sum())
    return total


def attention_flops(wl, items_only: bool = False) -> int:
    return 4 * wl.d * wl.hq * visible_pairs(wl, items_only)


def lm_head_cost(wl, rows=None):
    """FLOPs and algorithmic bytes of scoring ``rows`` readout rows (default:
    one per item) against the whole vocabulary."""
    rows = wl.total_items if rows is None else rows
    flops = 2 * rows * wl.hidden * wl.vocab
    nbytes = 2 * (wl.vocab * wl.hidden + rows * wl.hidden) + 4 * rows * wl.num_labels
    return flops, nbytes


def lm_head_bound_s(flops, nbytes):
    return max(nbytes / (PEAK_HBM_GBS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12))


ATTN_SOURCES = ("attn_bf16.hip", "attn_bf16_pipe.hip", "attn_loop.inc")


def attention_source_sha() -> str:
    """First 16 hex digits of the SHA-256 of the bf16 attention sources (both kernels)."""
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "item_scoring_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from a committed counter summary, if it matches the kernel sources."""
    path = os.path.join(PROFILES, f"traffic_attention_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                key, val = ln.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_sha256") != attention_source_sha():
        return None
    try:
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu() -> dict:
    """CPU model, usable cores and BLAS library of this host (for the oracle timing)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = [], 1
    try:
        from threadpoolctl import threadpool_info

        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas.append(f"{p.get('internal_api')} {p.get('version')} ({p.get('architecture')})")
                threads = max(threads, int(p.get("num_threads") or 1))
    except Exception:  # pragma: no cover - threadpoolctl is part of the image
        pass
    return {"cpu_model": model, "usable_cores": len(os.sched_getaffinity(0)), "blas": "; ".join(blas) or "unknown",
            "blas_threads": threads}


def cpu_baseline(wl, q, k, v, hid, W, labels, budget_s: float, flops: float):
    """Time the fp64 oracle on a bounded sample of the same workload (host cores).

    Segments are timed whole. Attention: every dense explicit-mask row of a
    request costs the same, so random query rows (all heads) are timed until
    half the budget is spent and the time is scaled by T / rows. Scoring: the
    oracle's time is a fixed part (the LM head converted to fp64 chunk by
    chunk) plus a part per item, so two item counts are timed and the line
    through them is read off at N (all items are timed when N <= 64).
    """
    import oracle

    info = host_cpu()
    workers = oracle.mis._workers(None)
    t0 = time.perf_counter()
    so = oracle.build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts)
    t_seg = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    T = wl.total_tokens
    n_rows = 32
    rows_done = 0
    t_attn = 0.0
    while rows_done < T:
        rows = np.sort(rng.choice(T, size=min(n_rows, T), replace=False))
        t1 = time.perf_counter()
        oracle.attention(q, k, v, wl.cu_seqlens, so["item_id"], rows=rows)
        t_attn += time.perf_counter() - t1
        rows_done += len(rows)
        if t_attn > budget_s * 0.5:
            break
        n_rows = min(T - rows_done, n_rows * 2) or 1
    attn_full = t_attn * T / rows_done
    N = wl.total_items
    readout = so["readout_pos"]

    def time_items(n):
        t1 = time.perf_counter()
        oracle.label_scores(hid, readout[:n], W, labels)
        return time.perf_counter() - t1

    if N <= 64:
        score_full = time_items(N)
        score_note = f"all {N} items' full-vocab label scores timed whole"
    else:
        n1, n2 = 16, 64
        t_1, t_2 = time_items(n1), time_items(n2)
        per_item = max(t_2 - t_1, 0.0) / (n2 - n1)
        score_full = t_2 + per_item * (N - n2)
        score_note = (f"label scores timed on {n1} and {n2} items ({t_1:.2f} s, {t_2:.2f} s) and "
                      f"extrapolated along that line to all {N} items")
    total = t_seg + attn_full + score_full
    return {
        "value": flops / attn_full / 1e12,
        "unit": "TFLOP/s",
        "cores": int(max(workers, info["blas_threads"])),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle (dense explicit-mask rows): segments timed whole; attention timed on "
                   f"{rows_done} of {T} query rows (all heads, {workers} threads) and scaled by T/rows; "
                   f"{score_note}"),
        "item_scores_per_s": N / total,
        "seconds_per_step": total,
        "host": info,
    }


def layout(wl, requests):
    """Row map and metadata of a packed batch built from a member batch's rows.

    ``requests`` lists (member, item indices) pairs; each becomes one request
    made of the member's query rows followed by those items' rows. Returns
    (rows, cu_seqlens, prefix_lens, cu_items, item_starts) with ``rows`` the
    source row of every packed token."""
    lens = wl.item_lengths()
    rows, cu, pl, ci, st = [], [0], [], [0], []
    for r, items in requests:
        base, lq = int(wl.cu_seqlens[r]), int(wl.prefix_lens[r])
        rows.append(np.arange(base, base + lq))
        off = lq
        for i in items:
            g = int(wl.cu_items[r]) + int(i)
            s0 = base + int(wl.item_starts[g])
            rows.append(np.arange(s0, s0 + int(lens[g])))
            st.append(off)
            off += int(lens[g])
        cu.append(cu[-1] + off)
        pl.append(lq)
        ci.append(ci[-1] + len(items))
    return (np.concatenate(rows), np.asarray(cu, np.int32), np.asarray(pl, np.int32), np.asarray(ci, np.int32),
            np.asarray(st, np.int32))


def paper(args) -> int:
    """MIS against single-item scoring on the profile-labeling benchmark's shape.

    From Generation to Scoring, §6.1: members' queries of mean 744 tokens
    (median 543, p95 2,047), items of about 28 tokens (chat layout; 24 in the
    compact layout of §3.1), 200 candidates per member; §6.4 sweeps the items
    per request N from 1 to 200 and splits 200 candidates into two requests of
    100. Here a batch of members (one seeded draw) is scored, whole step each
    (segments, attention, label scores), as
      mis:    one request per member holding its N items behind its query;
      split:  two requests per member of N/2 items, the query in each (N = 200);
      single: one request [q; c_i] per item (no prefix reuse across requests).
    Every layout is gathered on the GPU from the same rows, so all score the
    same values. Reported beside each measured speedup: the prefill-token
    ratio of the batch and Eq. 5's R(N) with the workload ratio 744 / 28.
    """
    import torch

    import item_scoring_attention_amd as mis
    import workloads

    torch.cuda.set_device(0)
    nmax = 200
    wl = workloads.paper_batch(args.members, nmax, args.item_tokens)
    print(f"[paper] {wl.description}: T={wl.total_tokens}", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = workloads.qkv(wl)
    qd, kd, vd = dev(q), dev(k), dev(v)
    seg = mis.mis_build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, 64, 64)
    hid = np.zeros((wl.total_tokens, wl.hidden), dtype=np.uint16)
    hid[seg.array("readout_pos").cpu().numpy()] = workloads.readout_values(wl)
    hidd, Wd = dev(hid), dev(workloads.lm_head(wl))
    labels = workloads.label_ids(wl)
    del q, k, v, hid
    bm, bn = mis.mis_attention_tile_shape(mis.MIS_BF16, wl.hq, wl.hkv, wl.d)
    rho = workloads.PAPER_QUERY_MEAN / args.item_tokens

    def run(requests):
        rows, cu, pl, ci, st = layout(wl, requests)
        idx = torch.from_numpy(rows).cuda()
        qx, kx, vx, hx = qd[idx], kd[idx], vd[idx], hidd[idx]
        ox = torch.empty_like(qx)
        T, N = int(cu[-1]), int(ci[-1])
        seg_buf = torch.empty(mis.mis_segments_bytes(cu, N, bm, bn), dtype=torch.uint8, device="cuda")
        scores = torch.empty((N, wl.num_labels), dtype=torch.float32, device="cuda")
        ws = torch.empty(mis.mis_score_workspace_bytes(N, wl.vocab, wl.num_labels, wl.hidden, mis.MIS_BF16),
                         dtype=torch.uint8, device="cuda")

        def step():
            s = mis.mis_build_segments(cu, pl, ci, st, bm, bn, dev_buf=seg_buf, stream=stream)
            mis.mis_attention_prefill(s, qx, kx, vx, o=ox, stream=stream)
            mis.mis_score_labels(s, hx, Wd, labels, scores=scores, ws=ws, stream=stream)

        # warm-up: at least 3 steps and 50 ms, so that the clocks have left
        # idle before the first layout is timed; then at least 30 ms timed
        tw, nw = time.perf_counter(), 0
        while nw < 3 or time.perf_counter() - tw < 0.05:
            step()
            nw += 1
            if nw % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        nsteps = max(args.steps, int(0.03 * nw / (time.perf_counter() - tw)) + 1)
        gc.collect()
        gc.disable()
        t0 = time.perf_counter()
        for _ in range(nsteps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / nsteps
        gc.enable()
        lens = np.diff(cu)
        pairs = int(sum(int(a) * (int(a) + 1) // 2 for a in pl))
        for r in range(len(pl)):
            s_items = np.diff(np.append(st[ci[r]:ci[r + 1]], lens[r])).astype(np.int64)
            pairs += int((s_items * int(pl[r]) + s_items * (s_items + 1) // 2).sum())
        return {"requests": len(pl), "tokens": T, "items": N, "ms_per_step": round(ms, 4), "timed_steps": nsteps,
                "item_scores_per_s": round(N / (ms * 1e-3), 1),
                "prefill_tokens_per_label": round(T / N, 2),
                "attention_tflop": round(4 * wl.d * wl.hq * pairs / 1e12, 4)}

    members = range(wl.num_requests)
    rows = []
    for n in args.paper_n:
        line = {"items_per_member": n}
        line["mis"] = run([(r, range(n)) for r in members])
        line["single"] = run([(r, [i]) for r in members for i in range(n)])
        if n == nmax:
            line["split_2x100"] = run([(r, range(h * n // 2, (h + 1) * n // 2)) for r in members for h in (0, 1)])
            line["split_vs_mis"] = round(line["mis"]["ms_per_step"] / line["split_2x100"]["ms_per_step"], 3)
        line["speedup_vs_single"] = round(line["single"]["ms_per_step"] / line["mis"]["ms_per_step"], 3)
        line["prefill_token_ratio"] = round(line["single"]["tokens"] / line["mis"]["tokens"], 3)
        line["R_eq5_workload"] = round(n * (1 + rho) / (n + rho), 3)
        rows.append(line)
        print(json.dumps(line), file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "MIS vs single-item scoring on the profile-labeling shape, whole step, 1 GPU",
        "unit": "item scores/s", "steps": args.steps, "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "members": wl.num_requests,
                   "item_tokens": args.item_tokens, "seed": wl.seed,
                   "query_lengths": {"mean": float(np.mean(wl.prefix_lens)),
                                     "median": float(np.median(wl.prefix_lens)),
                                     "p95": float(np.percentile(wl.prefix_lens, 95))},
                   "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.d, "hidden": wl.hidden, "vocab": wl.vocab,
                   "labels": wl.num_labels},
        "sweep": rows}), flush=True)
    return 0


def percentiles(xs) -> dict:
    """mean, median, p10 and p90 of per-launch durations (ms)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": round(float(a.mean()), 4), "median": round(float(np.median(a)), 4),
            "p10": round(float(np.percentile(a, 10)), 4), "p90": round(float(np.percentile(a, 90)), 4),
            "n": int(a.size)}


def mfma_peak_tflops(stream) -> dict:
    """Best bf16 MFMA rate of four launches of the probe kernel (TFLOP/s), with
    small repeating operands and with random N(0, 1)-like operands."""
    import ctypes

    import torch

    from item_scoring_attention_amd import build as B

    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.mis_probe_mfma_bf16.restype = ctypes.c_int
    lib.mis_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mis_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.mis_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    blocks, iters = 2048, 4096
    sink = torch.empty(blocks, dtype=torch.float32, device="cuda")
    out = {}
    for mode, name in ((0, "repeating_operands"), (1, "random_operands")):
        best = 0.0
        for _ in range(4):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = lib.mis_probe_mfma_bf16(blocks, iters, mode, ctypes.c_void_p(sink.data_ptr()),
                                         ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"MFMA probe launch failed: hip error {rc}")
            b.record(stream)
            b.synchronize()
            best = max(best, lib.mis_probe_mfma_bf16_flops(blocks, iters) / (a.elapsed_time(b) * 1e-3) / 1e12)
        out[name] = round(best, 1)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, help="workload 2, 3 or 5 (default 5, the largest)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle attention work")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed after a 512 MB write between steps (cold caches); 0 skips them")
    ap.add_argument("--paper", "--sweep", action="store_true", dest="paper",
                    help="the profile-labeling benchmark's shape: MIS against single-item scoring and the 2 x 100 "
                         "split for N = 1 .. 200 items per member")
    ap.add_argument("--members", type=int, default=32, help="members in the --paper batch")
    ap.add_argument("--item-tokens", type=int, default=28, help="item length in --paper (28 chat, 24 compact)")
    ap.add_argument("--paper-n", type=lambda x: [int(t) for t in x.split(",")], default=[1, 5, 20, 50, 100, 200],
                    help="items per member in --paper")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the timings beside the step (rotary, cached-prefix append, scores at several rows "
                         "per item), which launch the step's kernels again on other shapes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        return 2

    import torch

    import item_scoring_attention_amd as mis
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.paper:
        return paper(args)
    torch.cuda.set_device(0)
    wl = workloads.config(args.config)
    if wl.dtype != "bf16" or not wl.has_scoring:
        print("bench.py times the bf16 path with label scoring; pick workload 2, 3 or 5", file=sys.stderr)
        return 2
    print(f"[bench] {wl.name}: generating inputs", file=sys.stderr, flush=True)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = workloads.qkv(wl)
    qd, kd, vd = dev(q), dev(k), dev(v)
    od = torch.empty_like(qd)
    bm, bn = mis.mis_attention_tile_shape(mis.MIS_BF16, wl.hq, wl.hkv, wl.d)
    seg_bytes = mis.mis_segments_bytes(wl.cu_seqlens, wl.total_items, bm, bn)
    seg_buf = torch.empty(seg_bytes, dtype=torch.uint8, device="cuda")
    seg = mis.mis_build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, bm, bn,
                                 dev_buf=seg_buf)
    readout = seg.array("readout_pos").cpu().numpy()
    hid = np.full((wl.total_tokens, wl.hidden), workloads.NAN_BF16, dtype=np.uint16)
    hid[readout] = workloads.readout_values(wl)
    hidd = dev(hid)
    W = workloads.lm_head(wl)
    Wd = dev(W)
    labels = workloads.label_ids(wl)
    scores = torch.empty((wl.total_items, wl.num_labels), dtype=torch.float32, device="cuda")
    ws = torch.empty(mis.mis_score_workspace_bytes(wl.total_items, wl.vocab, wl.num_labels, wl.hidden,
                                                   mis.MIS_BF16), dtype=torch.uint8, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")  # larger than the 256 MB MALL
    torch.cuda.synchronize()
    attn_kernel = mis.attention_kernel_name(seg, mis.MIS_BF16, wl.hq, wl.hkv, wl.d)
    score_kernel = mis.score_kernel_name(wl.total_items, wl.hidden, mis.MIS_BF16)

    stream = torch.cuda.current_stream()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(marks=None):
        if marks is not None:
            marks.append([ev()])
        s = mis.mis_build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, bm, bn,
                                   dev_buf=seg_buf, stream=stream)
        if marks is not None:
            marks[-1].append(ev())
        mis.mis_attention_prefill(s, qd, kd, vd, o=od, stream=stream)
        if marks is not None:
            marks[-1].append(ev())
        mis.mis_score_labels(s, hidd, Wd, labels, scores=scores, ws=ws, stream=stream)
        if marks is not None:
            marks[-1].append(ev())

    print(f"[bench] {wl.name}: {args.warmup} warm-up + {args.steps} timed steps ({attn_kernel}, "
          f"{score_kernel})", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: K steps back to back, HIP events on the launch stream
    # around every call (each event adds a few microseconds of queue time to
    # the step, negligible against the long-prefix step's ~40 ms).
    # (the Python garbage collector is held off meanwhile: a collection pass
    # on the host can stall the launches of one step by milliseconds)
    warm = []
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(warm)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    ms_step = (t1 - t0) * 1e3 / args.steps

    def split(marks):
        return {"segments": [m[0].elapsed_time(m[1]) for m in marks],
                "attention": [m[1].elapsed_time(m[2]) for m in marks],
                "score": [m[2].elapsed_time(m[3]) for m in marks]}

    warm_ms = split(warm)
    # Cold caches: a 512 MB write between steps evicts L2 and the MALL.
    cold_ms = None
    if args.cold_steps > 0:
        cold = []
        for _ in range(args.cold_steps):
            flush.fill_(1)
            step(cold)
        torch.cuda.synchronize()
        cold_ms = split(cold)
    print("[bench] timed; measuring the MFMA probe" + ("" if args.no_extras else " and the calls beside the step"),
          file=sys.stderr, flush=True)
    t_att_warm = float(np.mean(warm_ms["attention"]))
    rope_tab = torch.empty((seg.max_seqlen, wl.d), dtype=torch.float32, device="cuda")
    mfma_peak = mfma_peak_tflops(stream)

    if not args.no_extras:
        # Rotary embedding at the reused positions (in place on q and k; not in
        # the step, timed last since it changes q and k).
        def back_to_back(fn, n):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            fn()
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
            b.synchronize()
            return a.elapsed_time(b) / n

        t_rope = back_to_back(lambda: mis.mis_apply_rope(seg, qd, kd, 1e6, stream=stream), 10)
        rope_bytes = 2 * wl.total_tokens * (wl.hq + wl.hkv) * wl.d * 2  # read and write q, k (bf16)
        # The same rotation with Q turned inside the attention kernel: K alone in
        # the pass, Q from the cos/sin table as it is loaded (outputs bit-identical
        # to pass + attention). The table depends on theta, D and the longest
        # request only (built once, for every layer and batch).
        n_att = max(2, min(20, int(200.0 / max(t_att_warm, 1e-3))))
        # Items against a cached prefix: item rows only, the prefix K/V read as
        # cached (query tiles of prefix rows only exit at once).
        t_append = back_to_back(lambda: mis.mis_attention_append(seg, qd, kd, vd, od, stream=stream), n_att)
        # Label scores at several marker rows per item (the last m rows of each
        # item, m = 3 where every item is that long), host row list included.
        m_at = int(min(3, int(wl.item_lengths().min())))
        markers = (readout[:, None] - np.arange(m_at - 1, -1, -1)[None, :]).reshape(-1).astype(np.int64)
        hidd[torch.from_numpy(markers).cuda()] = hidd[torch.from_numpy(np.repeat(readout, m_at).astype(np.int64)).cuda()]
        sc_at = torch.empty((markers.size, wl.num_labels), dtype=torch.float32, device="cuda")
        ws_at = torch.empty(mis.mis_score_workspace_bytes(markers.size, wl.vocab, wl.num_labels, wl.hidden,
                                                          mis.MIS_BF16), dtype=torch.uint8, device="cuda")
        t_sco_warm = float(np.mean(warm_ms["score"]))
        n_at = max(3, min(50, int(100.0 / max(m_at * t_sco_warm, 1e-3))))
        t_at = back_to_back(lambda: mis.mis_score_labels_at(markers, hidd, Wd, labels, scores=sc_at, ws=ws_at,
                                                            stream=stream), n_at)
        at_kernel = mis.score_kernel_name(int(markers.size), wl.hidden, mis.MIS_BF16)
        t_table = back_to_back(lambda: mis.mis_rope_table(seg.max_seqlen, wl.d, 1e6, table=rope_tab, stream=stream), 3)
        t_rope_k = back_to_back(lambda: mis.mis_apply_rope(seg, None, kd, 1e6, stream=stream), 10)
        t_att_plain = back_to_back(lambda: mis.mis_attention_prefill(seg, qd, kd, vd, o=od, stream=stream), n_att)
        t_att_fused = back_to_back(lambda: mis.mis_attention_prefill_rope(seg, qd, kd, vd, rope_tab, o=od,
                                                                          stream=stream), n_att)
        rope_k_bytes = 2 * wl.total_tokens * wl.hkv * wl.d * 2

    flops = attention_flops(wl)
    t_att = float(np.mean(warm_ms["attention"]))
    t_sco = float(np.mean(warm_ms["score"]))
    tflops = flops / (t_att * 1e-3) / 1e12
    traffic = read_traffic(wl.name)
    kernel_stats = {"warm": {key: percentiles(val) for key, val in warm_ms.items()}}
    if cold_ms:
        kernel_stats["cold"] = {key: percentiles(val) for key, val in cold_ms.items()}
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "item_scores_per_s": round(wl.total_items / (ms_step * 1e-3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "requests": wl.num_requests,
            "tokens": wl.total_tokens,
            "items": wl.total_items,
            "hq": wl.hq,
            "hkv": wl.hkv,
            "head_dim": wl.d,
            "hidden": wl.hidden,
            "vocab": wl.vocab,
            "labels": wl.num_labels,
            "tile": [bm, bn],
            "seed": wl.seed,
        },
        "call_ms": kernel_stats,
        "kernels": {"attention": attn_kernel, "score": f"{score_kernel} + combine_kernel"},
        "roofline": {
            "kernel": f"{attn_kernel} (MIS prefill attention)",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops,
            "measured_mfma_peak": mfma_peak,
            "frac_of_measured_peak": {k: round(tflops / p, 4) for k, p in mfma_peak.items()},
            "duration_ms": {"mean": round(t_att, 4), "median": kernel_stats["warm"]["attention"]["median"]},
        },
    }
    f_lm, b_lm = lm_head_cost(wl)
    t_bound = lm_head_bound_s(f_lm, b_lm)
    out["roofline_score"] = {
        "kernel": f"{score_kernel} + combine_kernel (LM head, split-vocab logsumexp)",
        "bound": "hbm" if b_lm / (PEAK_HBM_GBS * 1e9) >= f_lm / (PEAK_BF16_TFLOPS * 1e12) else "mfma",
        "achieved_gbs": round(b_lm / (t_sco * 1e-3) / 1e9, 1),
        "achieved_tflops": round(f_lm / (t_sco * 1e-3) / 1e12, 2),
        "frac": round(t_bound / (t_sco * 1e-3), 4),
        "algorithmic_bytes_per_launch": b_lm,
        "algorithmic_flops_per_launch": f_lm,
    }
    if cold_ms:
        t_cold = float(np.mean(cold_ms["score"]))
        out["roofline_score"]["frac_cold"] = round(t_bound / (t_cold * 1e-3), 4)
    if not args.no_extras:
        out["roofline_rope"] = {
            "kernel": "rope_kernel (rotary embedding of q and k at the reused positions, not in the step)",
            "bound": "hbm",
            "ms": round(t_rope, 4),
            "achieved_gbs": round(rope_bytes / (t_rope * 1e-3) / 1e9, 1),
            "peak_gbs": PEAK_HBM_GBS,
            "frac": round(rope_bytes / (t_rope * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes_per_launch": rope_bytes,
            "k_only": {"ms": round(t_rope_k, 4), "algorithmic_bytes_per_launch": rope_k_bytes,
                       "achieved_gbs": round(rope_k_bytes / (t_rope_k * 1e-3) / 1e9, 1)},
        }
        f_app = attention_flops(wl, items_only=True)
        out["append"] = {
            "kernel": f"{attn_kernel} (items against a cached prefix, not in the step)",
            "bound": "mfma",
            "ms": round(t_append, 4),
            "achieved_tflops": round(f_app / (t_append * 1e-3) / 1e12, 2),
            "frac": round(f_app / (t_append * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flops_per_launch": f_app,
            "full_prefill_ms": round(t_att_plain, 4),
        }
        f_at, b_at = lm_head_cost(wl, rows=int(markers.size))
        out["score_at"] = {
            "kernel": f"{at_kernel} + combine_kernel (label scores at {m_at} marker rows per item, not in the step)",
            "rows": int(markers.size),
            "ms": round(t_at, 4),
            "achieved_gbs": round(b_at / (t_at * 1e-3) / 1e9, 1),
            "achieved_tflops": round(f_at / (t_at * 1e-3) / 1e12, 2),
            "frac": round(lm_head_bound_s(f_at, b_at) / (t_at * 1e-3), 4),
            "algorithmic_bytes_per_launch": b_at,
            "algorithmic_flops_per_launch": f_at,
        }
        # attention with the rotation, both ways (back-to-back launches, same state)
        out["rope_step_ms"] = {
            "separate": round(t_rope + t_att_plain, 4),
            "fused": round(t_rope_k + t_att_fused, 4),
            "rotation_pass_q_and_k": round(t_rope, 4),
            "rotation_pass_k": round(t_rope_k, 4),
            "attention": round(t_att_plain, 4),
            "attention_rotating_q": round(t_att_fused, 4),
            "table_once": round(t_table, 4),
            "table_positions": int(seg.max_seqlen),
        }
    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda")  # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": a.numel() * 2, "write": a.numel() * 2, "launches": 3}
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, q, k, v, hid, W, labels, args.cpu_budget, flops)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
