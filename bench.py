#!/usr/bin/env python3
"""Benchmark of the wave-index hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input: build the index
of the Llama-shaped 128K layer (segmented spherical k-means, finalise, permuted K/V) and run
the workload's 64 decode steps against it (score, select, exact + estimate, merge). Inputs
are resident in HBM before timing starts. Before each decode call a 512 MiB buffer is read (a
reduction) so that the call finds its data in HBM rather than in the 256 MB Infinity Cache, as
it would after the other layers of a model; the per-kernel figures come from HIP events that
the library records between its kernels (the flush lies outside them).

The timed steps run the plain entry points with HIP events around each call (call time =
first kernel start to last kernel end, as the stream sees it); one more step runs the traced
entry points, whose per-kernel start / end events give the kernel breakdown and rooflines
(those events add a few microseconds around each kernel, so they are not used for the call
time). A 256 MiB device-to-device copy runs once before the warmup: its FETCH_SIZE /
WRITE_SIZE counters calibrate the HBM-traffic figures taken from rocprofv3 runs of this
script.

Prints one JSON line. `value` is decode-attention tokens/s of the 128K layer (batch / median
time of one decode call); the index-build rate and achieved HBM bandwidth are extra fields,
with p10 / p90 of the call time. Further legs in the same line:
  * extend: the extension of an index built for one segment fewer tokens, against a full
    build, with decode calls before and after it;
  * prefill_fused_build: the index built chunk by chunk (one segment of new tokens at a time)
    on a second stream beside a prefill stand-in, serial against overlapped;
  * stack_b8: the 32-layer Llama-shaped stack at batch 8 and 122 880 tokens, every layer's
    cache and index resident: the build over the stack, decode steps of one call per layer,
    and dense flash-decode steps over the same caches (the speedup);
  * stack_1m: the 32-layer stack at 1M tokens (about 150 GB resident): the build over the
    whole context, decode steps;
  * sweep: the 28-layer Qwen-shaped stack at batch 4 and 256K over cluster sizes 8/16/32 and
    budgets 0.5/1/1.8/4 %: step throughput and the error against exact attention per point;
  * anns: the same layer's decode steps through the attention-aware vector search (a graph
    over the keys built from 4096 training queries; beam search; attention over the steady
    zone and the retrieved tokens): build time, call time with its kernels, the recall of the
    exact top-k, nodes scored, and the error against dense attention beside the wave
    index's;
  * tier: the same layer's decode steps with the cache in pinned host memory behind a device
    block cache of a fraction of the layer's blocks (the wave buffer): call time against the
    resident call, the share of retrieved rows found in the block cache, bytes over the bus;
  * cpu_baseline: the CPU oracle on the host cores, one thread and all cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama128k")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="decode calls per step (default: the workload's)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-decode-steps", type=int, default=64)
    ap.add_argument("--extend", default="llama128k",
                    help="time the extension of this workload's index by one segment of new "
                         "tokens against a full build ('none': skip)")
    ap.add_argument("--prefill", default="llama128k",
                    help="prefill-fused build of this workload's index, chunk by chunk on a "
                         "second stream beside a prefill stand-in ('none': skip)")
    ap.add_argument("--stack8", default="llama122k_b8",
                    help="resident multi-layer stack with dense flash-decode beside it: layer "
                         "loops of wave and dense decode calls ('none': skip)")
    ap.add_argument("--stack1m", default="llama1m",
                    help="resident multi-layer stack at a long context: the build over the "
                         "whole stack and layer loops of decode calls ('none': skip)")
    ap.add_argument("--sweep", default="qwen256k",
                    help="resident stack over cluster sizes x retrieval budgets: throughput "
                         "and error against exact attention at each point ('none': skip)")
    ap.add_argument("--stack-steps", type=int, default=8)
    ap.add_argument("--anns", default="llama128k",
                    help="workload of the vector-search leg ('none' to skip)")
    ap.add_argument("--tier", default="1,0.05,0.01",
                    help="device block-cache sizes of the host-memory tier leg, as fractions "
                         "of the layer's 32-row blocks ('none' to skip)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): the wave index path here runs on one GPU (it would shard by (batch, "
              "KV head), each GPU holding its heads' cache and index).", file=sys.stderr,
              flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_vector_index_amd as wi
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wi.library()
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    nds = args.decode_steps or w.steps
    w = w.with_(steps=nds)
    B, H, Hq, G, d = w.batch, w.n_kv_heads, w.n_q_heads, w.group, 128
    L0, C, nr, T = w.context, w.n_clusters, w.n_retrieve, w.n_iters
    print(f"[bench] workload {w.name}: B={B} Hq={Hq} Hkv={H} L0={L0} S={w.segment_size} "
          f"C={C} T={T} n_r={nr} decode steps={nds}", file=sys.stderr, flush=True)

    x, k, v, q, k_out, v_out, bp, bws, idx, dps, dws, out, lse, sel = setup(w, nds)
    flush = None
    if not args.no_flush:
        flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")    # 512 MiB
    calib = torch.empty(2, 64 << 20, dtype=torch.float32, device="cuda")     # 2 x 256 MiB
    calib[1].copy_(calib[0])                                                 # calibration copy

    # start / end events of every kernel: build = norms, seeds, T x (assign, sort),
    # (T - 1) x update, finalise, steady; decode = score, [histogram: heads of more than 8192
    # clusters], gather, retrieve
    n_build_ev = 2 * (3 * T + 3)
    n_dec_ev = 8
    dec_recorded = []
    def events(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in ev:
            e.record()
        return ev

    def one_step(bev, dev_, timed=None):
        """One build + nds decode calls. bev / dev_: per-kernel event lists (traced pass);
        timed: (build pair, [decode pairs]) of events around each call (untraced pass)."""
        if timed:
            timed[0][0].record()
        wi.wave_index_build(bp, k, v, k_out, v_out, idx, bws,
                            events=None if bev is None else [e.cuda_event for e in bev])
        if timed:
            timed[0][1].record()
        for s in range(nds):
            if flush is not None:
                flush.sum()
            if timed:
                timed[1][s][0].record()
            n_ev = wi.wave_decode_attention(dps[s], q[s], k_out, v_out, idx, out, lse, sel[s], dws,
                                            events=None if dev_ is None else
                                            [e.cuda_event for e in dev_[s]])
            if dev_ is not None:
                dec_recorded.append(n_ev)
            if timed:
                timed[1][s][1].record()

    for _ in range(args.warmup):
        one_step(None, None)
    torch.cuda.synchronize()

    # ---- timed pass: untraced calls, HIP events around each call on the stream
    pair = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(2)]  # noqa: E731
    tev = [(pair(), [pair() for _ in range(nds)]) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(None, None, tev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    el = lambda a, b: a.elapsed_time(b)  # noqa: E731
    build_ms = [el(*t[0]) for t in tev]
    call_ms = [el(*c) for t in tev for c in t[1]]

    # ---- traced pass (one step): each kernel's duration from its start / end events
    bev = events(n_build_ev)
    dev_ = [events(n_dec_ev) for _ in range(nds)]
    torch.cuda.synchronize()
    one_step(bev, dev_)
    torch.cuda.synchronize()
    kd = lambda ev, i: el(ev[2 * i], ev[2 * i + 1])  # noqa: E731
    assign_ms, sort_ms, update_ms, fin_ms = [], [], [], []
    i = 2                          # after norms, seeds
    for p in range(T):
        assign_ms.append(kd(bev, i))
        sort_ms.append(kd(bev, i + 1))
        i += 2
        if p < T - 1:
            update_ms.append(kd(bev, i))
            i += 1
    fin_ms.append(kd(bev, i))
    has_hist = dec_recorded[0] == 8
    assert all(n == dec_recorded[0] for n in dec_recorded) and dec_recorded[0] in (6, 8)
    score_ms = [kd(e, 0) for e in dev_]
    hist_ms = [kd(e, 1) for e in dev_] if has_hist else []
    gather_ms = [kd(e, 1 + has_hist) for e in dev_]
    retrieve_ms = [kd(e, 2 + has_hist) for e in dev_]
    med = statistics.median

    # ---- algorithmic work (per decode call and per assignment launch)
    E, Er = exact_rows(w, idx, sel, nds)
    BH = B * H
    call_bytes = decode_call_bytes(w, E)
    # score kernel: centroids and sizes in; every head's logit and the group score out; q
    score_bytes = (2 * C * d + 4 * C + 4 * C * G + 4 * C + 2 * G * d) * BH
    # histogram kernel (large heads): the group scores
    hist_bytes = 4 * C * BH
    # gather kernel: the group scores (selection: each selection workgroup reads its own share;
    # the histogram's re-reads of the head's scores hit L2) and the published list; every cluster's
    # value sum, size and logits (estimate); the steady rows; q
    steady_mean = w.n_sink + w.n_recent + (nds + 1) / 2
    gather_bytes = (4 * C + 8 * nr + 12 * nr + 2 * C * d + 4 * C + 4 * C * G
                    + 4 * d * steady_mean + 2 * G * d) * BH
    # retrieve kernel: retrieved K/V rows, the removed clusters' value sums and logits, the
    # list entries, q, out
    retrieve_bytes = (4 * d * Er + (2 * d + 4 * G + 12) * nr + 2 * G * d + 4 * G * d) * BH
    n_idx = [max(0, min((s + 1) * w.segment_size, L0 - w.n_recent) - max(s * w.segment_size,
                                                                           w.n_sink))
             for s in range(w.n_segments)]
    assign_flop = sum(2.0 * n * w.clusters_per_segment * d for n in n_idx) * BH

    decode_tok_s = B / (med(call_ms) * 1e-3)
    build_tok_s = B * L0 / (med(build_ms) * 1e-3)
    call_gbs = call_bytes / (med(call_ms) * 1e-3) / 1e9
    mean = statistics.mean
    traffic = load_traffic()

    def roof(kernel, bound, work, launches_ms, extra=None):
        t = mean(launches_ms) * 1e-3
        if bound == "mfma":
            ach, peak, unit, key = work / t / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "flop_per_launch"
        else:
            ach, peak, unit, key = work / t / 1e9, HBM_PEAK_GBS, "GB/s", "bytes_per_launch"
        r = {"kernel": kernel, "bound": bound, "achieved": round(ach, 2), "peak": peak,
             "unit": unit, "frac": round(ach / peak, 4), "traffic": traffic.get(kernel),
             key: work, "avg_launch_us": round(mean(launches_ms) * 1e3, 2)}
        r.update(extra or {})
        return r

    roofs = {
        "k_assign": roof("k_assign", "mfma", assign_flop, assign_ms),
        "k_dec_score": roof("k_dec_score", "hbm", score_bytes, score_ms),
        **({"k_dec_hist": roof("k_dec_hist", "hbm", hist_bytes, hist_ms)} if has_hist else {}),
        "k_dec_gather": roof("k_dec_gather", "hbm", gather_bytes, gather_ms),
        "k_dec_retrieve": roof("k_dec_retrieve", "hbm", retrieve_bytes, retrieve_ms),
    }
    per_step = {"k_assign": T * mean(assign_ms), "k_dec_score": nds * mean(score_ms),
                **({"k_dec_hist": nds * mean(hist_ms)} if has_hist else {}),
                "k_dec_gather": nds * mean(gather_ms),
                "k_dec_retrieve": nds * mean(retrieve_ms)}
    dominant = max(per_step, key=per_step.get)
    roof_call = roof("decode call", "hbm", call_bytes, call_ms,
                     {"median_launch_us": round(med(call_ms) * 1e3, 2)})
    roof_call.pop("traffic")
    # The call is a chain of dependent kernels: at 128K its bytes take a few microseconds at
    # the peak while the chain's steps (kernel launches, memory round trips, the one-workgroup
    # selection) take most of the call. Each kernel's median traced time, what remains of the
    # untraced call between them, and the call's bytes at the HBM peak.
    chain = {"k_dec_score": med(score_ms) * 1e3}
    if has_hist:
        chain["k_dec_hist"] = med(hist_ms) * 1e3
    chain.update({"k_dec_gather": med(gather_ms) * 1e3, "k_dec_retrieve": med(retrieve_ms) * 1e3})
    roof_call["latency_chain_us"] = {
        **{k: round(v, 2) for k, v in chain.items()},
        "between_kernels": round(med(call_ms) * 1e3 - sum(chain.values()), 2),
        "bytes_at_peak": round(call_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}

    res = {
        "metric": "decode attn tokens/s + achieved HBM GB/s at 128K/1M ctx; index-build tok/s",
        "value": round(decode_tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded topic-structured RoPE keys, Gaussian values)",
        "config": {"workload": w.name, "batch": B, "context": L0, "n_q_heads": Hq,
                   "n_kv_heads": H, "head_dim": d, "segment_size": w.segment_size,
                   "clusters": C, "iters": T, "steady": [w.n_sink, w.n_recent],
                   "n_retrieve": nr, "decode_steps": nds, "cache_flush": flush is not None},
        "decode_call_us": round(med(call_ms) * 1e3, 2),
        "retrieved_tokens_per_kv_head": round(Er, 1),
        "decode_hbm_GBps": round(call_gbs, 1),
        "decode_hbm_frac": round(call_gbs / HBM_PEAK_GBS, 4),
        "decode_bytes_per_call": call_bytes,
        "exact_tokens_per_kv_head": round(E, 1),
        "index_build_tok_s": round(build_tok_s, 1),
        "index_build_ms": round(med(build_ms), 3),
        "kernel_us": {"assign": round(mean(assign_ms) * 1e3, 2),
                      "sort": round(statistics.mean(sort_ms) * 1e3, 2),
                      "update": round(statistics.mean(update_ms) * 1e3, 2) if update_ms else None,
                      "finalise": round(statistics.mean(fin_ms) * 1e3, 2),
                      "decode_call": round(med(call_ms) * 1e3, 2),
                      "dec_score": round(statistics.mean(score_ms) * 1e3, 2),
                      **({"dec_hist": round(statistics.mean(hist_ms) * 1e3, 2)}
                         if has_hist else {}),
                      "dec_gather": round(statistics.mean(gather_ms) * 1e3, 2),
                      "dec_retrieve": round(statistics.mean(retrieve_ms) * 1e3, 2)},
        "dominant_kernel": dominant,
        "step_ms_by_kernel": {k: round(v, 3) for k, v in per_step.items()},
        "roofline": roofs[dominant],
        "roofline_by_kernel": roofs,
        "roofline_decode_call": roof_call,
    }
    cs = sorted(call_ms)
    res["decode_call_us_p10_p90"] = [round(cs[int(0.1 * (len(cs) - 1))] * 1e3, 2),
                                     round(cs[int(0.9 * (len(cs) - 1))] * 1e3, 2)]
    if args.anns != "none" and args.anns == w.name:
        res["anns"] = anns_leg(w, nds, x, k, v, q, k_out, v_out, idx, dps, dws, flush)
        torch.cuda.empty_cache()
    if args.tier != "none":
        res["tier"] = tier_leg(w, nds, k_out, v_out, q, idx, dps, dws, out, lse, flush,
                               [float(f) for f in args.tier.split(",")], med(call_ms))
        torch.cuda.empty_cache()
    del k, v, q, k_out, v_out, bws, idx, dws, flush, calib
    torch.cuda.empty_cache()
    if args.extend != "none":
        res["extend"] = extend_leg(args.extend, 5)
        torch.cuda.empty_cache()
    if args.prefill != "none":
        res["prefill_fused_build"] = prefill_leg(args.prefill)
        torch.cuda.empty_cache()
    if args.stack8 != "none":
        res["stack_b8"] = stack_leg(args.stack8, args.stack_steps, 2, dense=True)
        torch.cuda.empty_cache()
    if args.stack1m != "none":
        res["stack_1m"] = stack_leg(args.stack1m, args.stack_steps, 2, dense=False)
        torch.cuda.empty_cache()
    if args.sweep != "none":
        res["sweep"] = sweep_leg(args.sweep, 3, 1)
        torch.cuda.empty_cache()
    if "stack_b8" in res and res["stack_b8"].get("dense_hbm_GBps"):
        # a measured streaming reference: the library's dense flash-decode over the batch-8
        # stack (every K and V row read once, in order)
        ref = res["stack_b8"]["dense_hbm_GBps"]
        res["decode_frac_of_stream"] = {
            "reference": "dense flash-decode of the batch-8 stack", "reference_GBps": ref,
            w.name: round(res["decode_hbm_GBps"] / ref, 4),
            **{res[k]["workload"]: round(res[k]["decode_hbm_GBps"] / ref, 4)
               for k in ("stack_b8", "stack_1m") if k in res}}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_decode_steps)
    print(json.dumps(res), flush=True)



def setup(w, nds):
    """Synthetic layer of workload w resident on the GPU, index and decode buffers."""
    import numpy as np
    import torch

    import kv_vector_index_amd as wi
    import synth

    B, H, Hq, d = w.batch, w.n_kv_heads, w.n_q_heads, 128
    L0, C, nr = w.context, w.n_clusters, w.n_retrieve
    t = time.time()
    x = synth.generate_layer(w)
    print(f"[bench] generated {w.name} inputs in {time.time() - t:.1f}s", file=sys.stderr,
          flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    k, v = dev(x.k), dev(x.v)
    q = dev(x.q)                                              # [steps, B, Hq, d]
    k_out, v_out = torch.zeros_like(k), torch.zeros_like(v)
    k_out[:, :, L0:] = k[:, :, L0:]                           # decode-appended rows
    v_out[:, :, L0:] = v[:, :, L0:]
    bp = wi.wave_build_params(B, Hq, H, d, L0, w.capacity, w.segment_size,
                              w.clusters_per_segment, w.n_iters, w.n_sink, w.n_recent)
    bws = torch.empty(wi.wave_index_workspace_size(bp), dtype=torch.uint8, device="cuda")
    idx = wi.alloc_index(B, H, C, L0, optional=False)
    scale = 1.0 / math.sqrt(d)
    dps = [wi.wave_decode_params(B, Hq, H, d, L0 + s + 1, L0, w.capacity, C, w.n_sink,
                                 w.n_recent, nr, scale) for s in range(nds)]
    dws = wi.alloc_decode_workspace(dps[0])
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    sel = torch.empty(nds, B, H, max(nr, 1), dtype=torch.int32, device="cuda")
    return x, k, v, q, k_out, v_out, bp, bws, idx, dps, dws, out, lse, sel


def exact_rows(w, idx, sel, nds):
    """Mean exact rows (steady + retrieved tokens) and retrieved tokens per (b, kv-head)
    over the decode calls, from the published selections and the cluster sizes."""
    import numpy as np

    B, H, nr = w.batch, w.n_kv_heads, w.n_retrieve
    csize = idx.cluster_size.cpu().numpy()
    selh = sel.cpu().numpy()
    e_tok, r_tok = [], []
    for s in range(nds):
        steady = w.n_sink + w.n_recent + s + 1
        tot = rt = 0
        for b in range(B):
            for g in range(H):
                ids = selh[s, b, g, :nr]
                ids = ids[ids >= 0]
                rt += int(csize[b, g, ids].sum())
                tot += steady + int(csize[b, g, ids].sum())
        e_tok.append(tot / (B * H))
        r_tok.append(rt / (B * H))
    return float(np.mean(e_tok)), float(np.mean(r_tok))


def decode_call_bytes(w, E):
    """Algorithmic HBM bytes of one decode call: centroids and sizes, the value sums of the
    unretrieved clusters, the exact K/V rows (E per (b, kv-head)), q in and out."""
    C, nr, G, d = w.n_clusters, w.n_retrieve, w.group, 128
    BH = w.batch * w.n_kv_heads
    return (2 * C * d + 4 * C + 2 * (C - nr) * d + 4 * d * E + 2 * G * d + 4 * G * d) * BH


def anns_leg(w, nds, x, k, v, q, k_out, v_out, idx, dps, dws, flush, n_pos=1024, M=32, R=32,
             E=16, ef=512, W=64, n_ret=256, err_steps=8):
    """The decode steps of the main leg through the attention-aware vector search on the raw
    (position-ordered) cache: the graph of the group's prefill queries at the last n_pos
    positions (n_pos * G training queries per KV head), then per step the search and the
    attention over the steady zone and the n_ret retrieved tokens. Reports the build, the
    call (median, cache flushed before each call as in the main leg) and its kernels, the
    rounds and nodes scored per search, the recall of the exact top-n_ret by the fp32 score,
    and the relative l2 error against dense attention per (b, q head) beside the wave
    index's error on the same steps."""
    import numpy as np
    import torch

    import kv_vector_index_amd as wi
    import synth

    B, H, Hq, G, d = w.batch, w.n_kv_heads, w.n_q_heads, w.group, 128
    L0, ns, nr = w.context, w.n_sink, w.n_recent
    N = L0 - ns - nr
    T = synth.training_queries(w, n_pos)
    t_dev = torch.from_numpy(T.view(np.int16)).view(torch.bfloat16).cuda()
    mk = lambda L: wi.wave_anns_params(B, Hq, H, d, L, L0, w.capacity, ns, nr, n_pos * G, M,  # noqa: E731
                                       R, E, ef, W, n_ret, 100000, 1.0 / math.sqrt(d))
    p0 = mk(L0)
    index = wi.alloc_anns_index(p0, t_dev)
    bws = torch.empty(wi.wave_anns_build_workspace_size(p0), dtype=torch.uint8, device="cuda")
    aws = torch.empty(wi.wave_anns_decode_workspace_size(p0), dtype=torch.uint8, device="cuda")
    ev = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(2)]  # noqa: E731
    bt = []
    for _ in range(3):
        e = ev()
        e[0].record()
        wi.wave_anns_build(p0, k, index, bws)
        e[1].record()
        bt.append(e)
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(16)]
    for e in kev:
        e.record()
    n_bk = wi.wave_anns_build(p0, k, index, bws, events=[e.cuda_event for e in kev])
    torch.cuda.synchronize()
    build_ms = statistics.median(a.elapsed_time(b) for a, b in bt[1:])
    names = ["lists", "zero", "count", "scan", "scatter", "link"][:n_bk // 2]
    build_k = {nm: round(kev[2 * i].elapsed_time(kev[2 * i + 1]) * 1e3, 1)
               for i, nm in enumerate(names)}
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    ret = torch.empty(nds, B, H, n_ret, dtype=torch.int32, device="cuda")
    st = torch.empty(nds, B, H, 2, dtype=torch.int32, device="cuda")
    ps = [mk(p.seq_len) for p in dps]
    for s in range(min(4, nds)):                                   # warm-up
        wi.wave_anns_decode_attention(ps[s], q[s], k, v, index, out, None, ret[s], st[s], aws)
    cev = [ev() for _ in range(nds)]
    for s in range(nds):
        if flush is not None:
            flush.sum()
        cev[s][0].record()
        wi.wave_anns_decode_attention(ps[s], q[s], k, v, index, out, None, ret[s], st[s], aws)
        cev[s][1].record()
    dk = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(nds)]
    for s in range(nds):
        if flush is not None:
            flush.sum()
        for e in dk[s]:
            e.record()
        wi.wave_anns_decode_attention(ps[s], q[s], k, v, index, out, None, ret[s], st[s], aws,
                                      events=[e.cuda_event for e in dk[s]])
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in cev]
    kern = lambda i: statistics.mean(dk[s][2 * i].elapsed_time(dk[s][2 * i + 1])  # noqa: E731
                                     for s in range(nds))
    stats = st.cpu().numpy()
    # recall of the exact best n_ret nodes by the group-sum score (fp32 products on the GPU)
    kn = k[:, :, ns:L0 - nr].float()
    rec = []
    for s in range(nds):
        u = q[s].float().view(B, H, G, d).sum(dim=2)                   # [B, H, d]
        sc = torch.matmul(kn, u.unsqueeze(-1)).squeeze(-1)             # fp32 [B, H, N]
        best = sc.topk(n_ret, dim=-1).indices + ns
        got = ret[s].long()
        hit = (best.unsqueeze(-1) == got.unsqueeze(-2)).any(-1).float().mean(-1)
        rec.append(hit.mean().item())
    # error against dense attention, beside the wave index's, over err_steps steps
    ref = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    wout = torch.empty_like(ref)
    lse_ref = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    lse_a = torch.empty_like(lse_ref)
    dws_dense = torch.empty(wi.wave_decode_workspace_size(dps[0]), dtype=torch.uint8,
                            device="cuda")
    ea, ew, mass = [], [], []
    for s in range(min(err_steps, nds)):
        wi.wave_dense_decode_attention(dps[s], q[s], k, v, ref, lse_ref, dws_dense)
        wi.wave_anns_decode_attention(ps[s], q[s], k, v, index, out, lse_a, None, None, aws)
        mass.append(torch.exp(lse_a - lse_ref).flatten())
        wi.wave_decode_attention(dps[s], q[s], k_out, v_out, idx, wout, None, None, dws)
        den = ref.norm(dim=-1)
        ea.append(((out - ref).norm(dim=-1) / den).flatten())
        ew.append(((wout - ref).norm(dim=-1) / den).flatten())
    ea, ew, mass = torch.cat(ea), torch.cat(ew), torch.cat(mass)
    rounds, visited = stats[..., 0].astype(float), stats[..., 1].astype(float)
    # bytes a search touches: the scored key rows and the expanded rows' neighbour lists (the
    # seed kernel reads the training queries); the attention: K and V of the steady zone and
    # the retrieved rows
    search_bytes = float(np.mean(visited * 256 + rounds * W * R * 4)) * B * H
    n_steady = ns + nr + (nds + 1) / 2
    attn_bytes = (n_steady + n_ret) * 512 * B * H
    t_seed, t_search, t_part, t_merge = kern(0), kern(1), kern(2), kern(3)
    r = {"workload": w.name, "training_queries": n_pos * G, "list_len": M, "degree": R,
         "n_entry": E, "pool": ef, "expand": W, "retrieved": n_ret, "nodes": N,
         "build_ms": round(build_ms, 3), "build_kernel_us": build_k,
         "call_us": round(statistics.median(call_ms) * 1e3, 2),
         "decode_tok_s": round(B / (statistics.median(call_ms) * 1e-3), 1),
         "kernel_us": {"seed": round(t_seed * 1e3, 2), "search": round(t_search * 1e3, 2),
                       "partial": round(t_part * 1e3, 2),
                       "merge": round(t_merge * 1e3, 2)},
         "rounds_mean": round(float(rounds.mean()), 1),
         "nodes_scored_mean": round(float(visited.mean()), 1),
         "nodes_scored_frac": round(float(visited.mean()) / N, 4),
         "recall_at_k": round(float(np.mean(rec)), 4),
         "search_GBps": round(search_bytes / (t_search * 1e-3) / 1e9, 1),
         "search_bytes_per_launch": round(search_bytes),
         "attention_GBps": round(attn_bytes / ((t_part + t_merge) * 1e-3) / 1e9, 1),
         "softmax_mass_on_attended_rows": round(mass.mean().item(), 4),
         "rel_l2_err_vs_dense": {"anns_mean": round(ea.mean().item(), 4),
                                 "anns_max": round(ea.max().item(), 4),
                                 "wave_mean": round(ew.mean().item(), 4),
                                 "wave_max": round(ew.max().item(), 4)}}
    print(f"[bench] anns: {r}", file=sys.stderr, flush=True)
    return r


def tier_leg(w, nds, k_out, v_out, q, idx, dps, dws, out, lse, flush, fracs, resident_ms):
    """The decode steps of the main leg through the host-memory tier: K/V in pinned host
    memory, the steady zone in its own device buffer, a device block cache of `frac` of the
    layer's 32-row blocks. Per cache size, after a reset: the first call (every retrieved row
    read over the bus), then the median call over the steps after the first quarter (in which
    the cache warms), the share of retrieved rows read from the block cache there, and the
    bytes that crossed the bus per call (the rows read from host memory: a row read over the
    bus is written into the cache on the device, not fetched again)."""
    import torch

    import kv_vector_index_amd as wi

    L0, ns, nr = w.context, w.n_sink, w.n_recent
    p_last = dps[-1]
    blocks = w.batch * w.n_kv_heads * -(-w.capacity // wi.TIER_BLOCK)
    block_bytes = 2 * wi.TIER_BLOCK * 128 * 2
    n_warm = max(1, nds // 4)
    pts = []
    for frac in fracs:
        n_slots = max(1, int(round(frac * blocks)))
        tier = wi.alloc_tier(p_last, n_slots)
        tier.host_k.copy_(k_out)
        tier.host_v.copy_(v_out)
        tier.steady_k.copy_(torch.cat([k_out[:, :, :ns], k_out[:, :, L0 - nr:]], dim=2))
        tier.steady_v.copy_(torch.cat([v_out[:, :, :ns], v_out[:, :, L0 - nr:]], dim=2))
        wi.wave_tier_reset(p_last, tier)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nds)]
        c0 = None
        for s in range(nds):
            if s == n_warm:
                c0 = wi.wave_tier_counters(p_last, tier)     # (synchronizes)
            if flush is not None:
                flush.sum()
            ev[s][0].record()
            wi.wave_decode_attention_tiered(dps[s], q[s], tier, idx, out, lse, None, dws)
            ev[s][1].record()
        c1 = wi.wave_tier_counters(p_last, tier)
        ms = [a.elapsed_time(b) for a, b in ev]
        d = {key: c1[key] - c0[key] for key in c1}
        n_t = nds - n_warm
        rows = d["rows_cached"] + d["rows_host"]
        bus = d["rows_host"] * 4 * 128 / n_t
        m = statistics.median(ms[n_warm:])
        pts.append({"block_cache_frac": frac, "slots": n_slots,
                    "block_cache_MiB": round(n_slots * block_bytes / 2**20, 1),
                    "first_call_us": round(ms[0] * 1e3, 1),
                    "call_us": round(m * 1e3, 1),
                    "resident_call_us": round(resident_ms * 1e3, 1),
                    "slowdown": round(m / resident_ms, 2),
                    "cached_row_share": round(d["rows_cached"] / max(rows, 1), 4),
                    "bus_MB_per_call": round(bus / 1e6, 3),
                    "bus_GBps": round(bus / (m * 1e-3) / 1e9, 1),
                    "rows_written_per_call": round(d["rows_written"] / n_t, 1),
                    "slots_claimed_per_call": round(d["blocks_admitted"] / n_t, 1),
                    "claims_refused_per_call": round(d["blocks_refused"] / n_t, 1)})
        print(f"[bench] tier {frac}: {pts[-1]}", file=sys.stderr, flush=True)
        del tier
    return {"workload": w.name, "timed_steps": nds - n_warm, "points": pts}


def extend_leg(name, n_rep):
    """Index extension in a decode loop: a workload's index built for its context minus one
    segment while that segment's tokens were generated (they sit in the recent zone), then
    extended to the full context (wave_index_extend: the last, partly indexed segment and
    the new one are clustered, the rest is copied), against a full build of the same
    context; with the decode call before the extension (on the earlier index, the generated
    tokens attended exactly) and after it. Median of n_rep timed calls each (HIP events),
    after one untimed call."""
    import numpy as np
    import torch

    import kv_vector_index_amd as wi
    import synth

    w = synth.WORKLOADS[name]
    B, H, Hq, d = w.batch, w.n_kv_heads, w.n_q_heads, 128
    L0, S, K = w.context, w.segment_size, w.clusters_per_segment
    prev_len = L0 - S
    x = synth.generate_layer(w, rows=L0 + 1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    k, v, q = dev(x.k), dev(x.v), dev(x.q[0])
    del x
    k_out, v_out = torch.zeros_like(k), torch.zeros_like(v)

    def params(n):
        return wi.wave_build_params(B, Hq, H, d, n, L0 + 1, S, K, w.n_iters, w.n_sink,
                                    w.n_recent)

    bp_prev, bp = params(prev_len), params(L0)
    ws = torch.empty(wi.wave_index_workspace_size(bp), dtype=torch.uint8, device="cuda")
    C_prev, C = -(-prev_len // S) * K, -(-L0 // S) * K
    prev = wi.alloc_index(B, H, C_prev, prev_len, optional=False)
    idx = wi.alloc_index(B, H, C, L0, optional=False)
    wi.wave_index_build(bp_prev, k, v, k_out, v_out, prev, ws)
    k_out[:, :, prev_len:] = k[:, :, prev_len:]            # the tokens generated since
    v_out[:, :, prev_len:] = v[:, :, prev_len:]
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    nr_prev, nr = (int(math.ceil(w.budget * c - 1e-9)) for c in (C_prev, C))
    # decode with the earlier index while S generated tokens sit in the recent zone
    dp_before = wi.wave_decode_params(B, Hq, H, d, L0, prev_len, L0 + 1, C_prev, w.n_sink,
                                      w.n_recent, nr_prev, scale)
    dws = wi.alloc_decode_workspace(dp_before)

    def timed(call):
        call()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_rep)]
        for e in ev:
            e[0].record()
            call()
            e[1].record()
        torch.cuda.synchronize()
        return statistics.median(e[0].elapsed_time(e[1]) for e in ev)

    before_us = timed(lambda: wi.wave_decode_attention(dp_before, q, k_out, v_out, prev, out,
                                                       None, None, dws)) * 1e3
    ext_ms = timed(lambda: wi.wave_index_extend(bp, prev_len, k, v, k_out, v_out, prev, idx,
                                                ws))
    dp_after = wi.wave_decode_params(B, Hq, H, d, L0 + 1, L0, L0 + 1, C, w.n_sink, w.n_recent,
                                     nr, scale)
    dws = wi.alloc_decode_workspace(dp_after)
    after_us = timed(lambda: wi.wave_decode_attention(dp_after, q, k_out, v_out, idx, out, None,
                                                      None, dws)) * 1e3
    k_full, v_full = torch.zeros_like(k), torch.zeros_like(v)
    full_ms = timed(lambda: wi.wave_index_build(bp, k, v, k_full, v_full, idx, ws))
    s0 = (prev_len - w.n_recent) // S
    return {"workload": w.name, "prev_len": prev_len, "seq_len": L0,
            "segments_built": -(-L0 // S) - s0, "segments_total": -(-L0 // S),
            "extend_ms": round(ext_ms, 3), "full_build_ms": round(full_ms, 3),
            "speedup_vs_full_build": round(full_ms / ext_ms, 2),
            "new_tok_s": round(B * (L0 - prev_len) / (ext_ms * 1e-3), 1),
            "decode_call_us_before": round(before_us, 2),
            "decode_call_us_after": round(after_us, 2),
            "extend_cost_per_generated_token_us": round(ext_ms * 1e3 / (L0 - prev_len), 4)}


def prefill_leg(name, standin_calls=8):
    """Prefill-fused index build: the context arrives one segment of S tokens at a time, and
    after each chunk the index is extended from the previous length (wave_index_extend; the
    first chunk is a plain build) on a second stream, while the first stream runs a stand-in
    for the chunk's prefill attention (standin_calls dense decode calls over the prefix that
    has arrived). Both streams keep the default priority; a chunk's extension waits for that
    chunk's stand-in (an event). Reported: the same work serially on one stream against the
    two streams, and whether the final index and cache equal one full build bit for bit."""
    import numpy as np
    import torch

    import kv_vector_index_amd as wi
    import synth

    w = synth.WORKLOADS[name]
    B, H, Hq, d = w.batch, w.n_kv_heads, w.n_q_heads, 128
    L0, S, K = w.context, w.segment_size, w.clusters_per_segment
    x = synth.generate_layer(w, rows=L0 + 1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    k, v, q = dev(x.k), dev(x.v), dev(x.q[0])
    del x
    lens = list(range(S, L0, S)) + [L0]
    Lcap = L0 + 1

    def params(n):
        return wi.wave_build_params(B, Hq, H, d, n, Lcap, S, K, w.n_iters, w.n_sink, w.n_recent)

    ws = torch.empty(wi.wave_index_workspace_size(params(L0)), dtype=torch.uint8, device="cuda")
    idxs = [wi.alloc_index(B, H, -(-n // S) * K, n) for n in lens]
    for i in idxs:
        i.objective = None
    # (the shortest prefix needs the largest workspace: its partial count grows with the
    # rows past the index)
    dp = wi.wave_decode_params(B, Hq, H, d, lens[0], lens[0], Lcap, 1, 0, 0, 0,
                               1.0 / math.sqrt(d))
    dws = wi.alloc_decode_workspace(dp)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    k_out, v_out = torch.zeros_like(k), torch.zeros_like(v)
    main_s = torch.cuda.current_stream()
    build_s = torch.cuda.Stream()

    def standin(n):
        p = wi.wave_decode_params(B, Hq, H, d, n, n, Lcap, 1, 0, 0, 0, 1.0 / math.sqrt(d))
        for _ in range(standin_calls):
            wi.wave_dense_decode_attention(p, q, k, v, out, None, dws)

    def build(c, stream):
        if c == 0:
            wi.wave_index_build(params(lens[0]), k, v, k_out, v_out, idxs[0], ws, stream)
        else:
            wi.wave_index_extend(params(lens[c]), lens[c - 1], k, v, k_out, v_out, idxs[c - 1],
                                 idxs[c], ws, stream)

    def run(overlap):
        t0, t1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        torch.cuda.synchronize()
        t0.record(main_s)
        build_s.wait_event(t0)
        for c, n in enumerate(lens):
            standin(n)
            if overlap:
                e = torch.cuda.Event()
                e.record(main_s)
                build_s.wait_event(e)
                build(c, build_s)
            else:
                build(c, main_s)
        if overlap:
            e = torch.cuda.Event()
            e.record(build_s)
            main_s.wait_event(e)
        t1.record(main_s)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    run(True)                                          # warm
    serial_ms = statistics.median(run(False) for _ in range(3))
    overlap_ms = statistics.median(run(True) for _ in range(3))
    t0, t1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    t0.record()
    for n in lens:
        standin(n)
    t1.record()
    torch.cuda.synchronize()
    standin_ms = t0.elapsed_time(t1)
    full = wi.alloc_index(B, H, -(-L0 // S) * K, L0)
    full.objective = None
    k_full, v_full = torch.zeros_like(k), torch.zeros_like(v)
    wi.wave_index_build(params(L0), k, v, k_full, v_full, full, ws)
    torch.cuda.synchronize()
    same = all(torch.equal(getattr(idxs[-1], f).view(torch.int16) if getattr(full, f).dtype ==
                           torch.bfloat16 else getattr(idxs[-1], f),
                           getattr(full, f).view(torch.int16) if getattr(full, f).dtype ==
                           torch.bfloat16 else getattr(full, f))
               for f in ("centroid_mean", "value_sum", "cluster_size", "cluster_offset",
                         "labels", "perm", "last_centroids"))
    same = same and torch.equal(k_out[:, :, :L0].view(torch.int16),
                                k_full[:, :, :L0].view(torch.int16))
    build_ms = max(0.0, serial_ms - standin_ms)
    return {"workload": name, "chunks": len(lens), "chunk_tokens": S,
            "standin": f"{standin_calls} dense decode calls over the arrived prefix per chunk",
            "standin_ms": round(standin_ms, 3), "serial_ms": round(serial_ms, 3),
            "overlapped_ms": round(overlap_ms, 3),
            "chunked_build_ms_serial": round(build_ms, 3),
            "build_hidden_frac": round((serial_ms - overlap_ms) / build_ms, 3) if build_ms else None,
            "equal_to_full_build": bool(same)}


def kernel_sources_hash() -> str:
    """Hash of the HIP sources: traffic figures are only valid for the kernels they measured."""
    import hashlib
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "kv_vector_index_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic() -> dict:
    """HBM bytes per launch of each kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE scaled by the calibration copy), if it was taken from the
    current kernel sources; otherwise no figures."""
    path = os.path.join(ROOT, "profiles", "traffic_llama128k.json")
    if not os.path.exists(path):
        return {}
    t = json.load(open(path))
    if t.get("sources_sha1") != kernel_sources_hash():
        return {}
    return t.get("bytes_per_launch", {})


def stack_leg(name, n_steps, n_warm, dense):
    """A whole model's attention layers resident in HBM: n_layers layers of the workload,
    each with its own permuted K/V cache and index (distinct buffers; the contents of layer 0
    replicated, since drawing every layer on the host would take minutes), built from the
    raw cache one layer after the other (the build timed over the whole stack), then decode
    steps of one call per layer (a model is layer-sequential; the other layers evict the
    caches, so no flush). Layer l decodes step s with the queries of step (s + l) mod steps
    so that the layers select different clusters. HIP events around each step's layer loop;
    with `dense`, the same steps with dense flash-decode over every layer's whole cache."""
    import numpy as np
    import torch

    import kv_vector_index_amd as wi
    import synth

    nq = n_steps + n_warm
    w = synth.WORKLOADS[name].with_(steps=nq)
    nL = w.n_layers
    B, H, Hq, G, d = w.batch, w.n_kv_heads, w.n_q_heads, w.group, 128
    L0, C, nr = w.context, w.n_clusters, w.n_retrieve
    t = time.time()
    x = synth.generate_layer(w)
    print(f"[bench] stack leg {name}: {nL} layers, B={B} L0={L0} C={C} n_r={nr}; generated "
          f"inputs in {time.time() - t:.1f}s", file=sys.stderr, flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    k, v, q = dev(x.k), dev(x.v), dev(x.q)
    del x
    bp = wi.wave_build_params(B, Hq, H, d, L0, w.capacity, w.segment_size,
                              w.clusters_per_segment, w.n_iters, w.n_sink, w.n_recent)
    bws = torch.empty(wi.wave_index_workspace_size(bp), dtype=torch.uint8, device="cuda")
    layers = []
    for _ in range(nL):
        ko, vo = torch.empty_like(k), torch.empty_like(v)
        ko[:, :, L0:] = k[:, :, L0:]                       # decode-appended rows
        vo[:, :, L0:] = v[:, :, L0:]
        layers.append((ko, vo, wi.alloc_index(B, H, C, L0, optional=False)))
    ev = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(2)]  # noqa: E731
    be = [ev() for _ in range(nL)]
    torch.cuda.synchronize()
    for l, (ko, vo, idx) in enumerate(layers):
        be[l][0].record()
        wi.wave_index_build(bp, k, v, ko, vo, idx, bws)
        be[l][1].record()
    torch.cuda.synchronize()
    build_ms = [e[0].elapsed_time(e[1]) for e in be]
    stack_build_ms = be[0][0].elapsed_time(be[-1][1])
    del k, v, bws
    torch.cuda.empty_cache()
    scale = 1.0 / math.sqrt(d)
    dps = [wi.wave_decode_params(B, Hq, H, d, L0 + s + 1, L0, w.capacity, C, w.n_sink,
                                 w.n_recent, nr, scale) for s in range(nq)]
    dws = wi.alloc_decode_workspace(dps[0])
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    sel = torch.empty(nL, nq, B, H, max(nr, 1), dtype=torch.int32, device="cuda")

    def steps(call):
        step_ev = [ev() for _ in range(nq)]
        l0_ev = [ev() for _ in range(nq)]
        for s in range(nq):
            step_ev[s][0].record()
            for l in range(nL):
                if l == 0:
                    l0_ev[s][0].record()
                call(s, l)
                if l == 0:
                    l0_ev[s][1].record()
            step_ev[s][1].record()
        torch.cuda.synchronize()
        st = sorted(e[0].elapsed_time(e[1]) for e in step_ev[n_warm:])
        l0 = statistics.median(e[0].elapsed_time(e[1]) for e in l0_ev[n_warm:])
        return st, l0

    def wave_call(s, l):
        ko, vo, idx = layers[l]
        wi.wave_decode_attention(dps[s], q[(s + l) % nq], ko, vo, idx, out, lse, sel[l, s], dws)

    st, l0_ms = steps(wave_call)
    med = statistics.median(st)
    # algorithmic bytes of every timed (layer, step) call, from the selections
    csize = [layers[l][2].cluster_size.cpu().numpy() for l in range(nL)]
    selh = sel.cpu().numpy()
    step_bytes = []
    for s in range(n_warm, nq):
        tot = 0.0
        for l in range(nL):
            ids = selh[l, s, :, :, :nr]
            E = 0.0
            for b in range(B):
                for g in range(H):
                    i = ids[b, g]
                    E += w.n_sink + w.n_recent + s + 1 + float(csize[l][b, g, i[i >= 0]].sum())
            tot += decode_call_bytes(w, E / (B * H))
        step_bytes.append(tot)
    nbytes = float(np.mean(step_bytes))
    gbs = nbytes / (med * 1e-3) / 1e9
    # per-kernel times of one traced call (layer 0, last step)
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for e in kev:
        e.record()
    ko, vo, idx = layers[0]
    n_ev = wi.wave_decode_attention(dps[-1], q[-1], ko, vo, idx, out, lse, sel[0, -1], dws,
                                    events=[e.cuda_event for e in kev])
    torch.cuda.synchronize()
    names = ["score", "hist", "gather", "retrieve"] if n_ev == 8 else ["score", "gather",
                                                                        "retrieve"]
    kernel_us = {nm: round(kev[2 * i].elapsed_time(kev[2 * i + 1]) * 1e3, 2)
                 for i, nm in enumerate(names)}
    res = {"workload": w.name, "layers": nL, "batch": B, "context": L0, "n_q_heads": Hq,
           "n_kv_heads": H, "clusters": C, "n_retrieve": nr, "steady": [w.n_sink, w.n_recent],
           "layer_contents": "layer 0 replicated into every layer's own buffers; layer l "
                             "decodes with the queries of step (s + l) mod steps",
           "decode_steps": n_steps, "warmup_steps": n_warm,
           "step_ms": round(med, 4),
           "step_ms_p10_p90": [round(st[int(0.1 * (len(st) - 1))], 4),
                               round(st[int(0.9 * (len(st) - 1))], 4)],
           "decode_tok_s": round(B / (med * 1e-3), 1),
           "decode_bytes_per_step": nbytes, "decode_hbm_GBps": round(gbs, 1),
           "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "layer0_call_us": round(l0_ms * 1e3, 2),
           "step_vs_layers_x_layer0_call": round(med / (nL * l0_ms), 3),
           "kernel_us_one_call": kernel_us,
           "index_build_ms_stack": round(stack_build_ms, 3),
           "index_build_ms_per_layer": round(statistics.median(build_ms), 3),
           "index_build_tok_s_stack": round(B * L0 * nL / (stack_build_ms * 1e-3), 1)}
    if dense:
        def dense_call(s, l):
            ko, vo, _ = layers[l]
            wi.wave_dense_decode_attention(dps[s], q[(s + l) % nq], ko, vo, out, lse, dws)
        dst, _ = steps(dense_call)
        dmed = statistics.median(dst)
        L_mid = L0 + (n_warm + 1 + nq) / 2
        dense_bytes = (4 * d * L_mid + 2 * G * d + 4 * G * d) * B * H * nL
        dgbs = dense_bytes / (dmed * 1e-3) / 1e9
        res.update({"dense_step_ms": round(dmed, 4),
                    "dense_tok_s": round(B / (dmed * 1e-3), 1),
                    "dense_bytes_per_step": dense_bytes, "dense_hbm_GBps": round(dgbs, 1),
                    "dense_hbm_frac": round(dgbs / HBM_PEAK_GBS, 4),
                    "speedup_vs_dense": round(dmed / med, 2)})
    del layers, dws
    torch.cuda.empty_cache()
    return res


def sweep_leg(name, n_steps, n_warm, cluster_sizes=(8, 16, 32),
              budgets=(0.005, 0.01, 0.018, 0.04), err_steps=4):
    """The Qwen-shaped stack (28 resident layers, layer 0 replicated as in stack_leg) over
    cluster sizes x retrieval budgets: per point, the decode step time of the layer loop
    (tokens/s, HBM GB/s on algorithmic bytes) and the error of layer 0's wave decode against
    exact attention (dense decode over all L rows, itself checked against the oracle's full
    attention in the tests): relative l2 error per (b, q head) over err_steps steps (mean /
    p99 / max), and the share of the exact softmax mass on the exactly attended rows (batch
    element 0, KV group 0, first step). Budget 1.0 (every cluster retrieved) is also run on
    layer 0 as a check of the comparison (rounding-level error)."""
    import numpy as np
    import torch

    import kv_vector_index_amd as wi
    import synth

    nq = max(n_steps + n_warm, err_steps)
    base = synth.WORKLOADS[name].with_(steps=nq)
    nL, B, H, Hq, G, d = base.n_layers, base.batch, base.n_kv_heads, base.n_q_heads, base.group, 128
    L0 = base.context
    t = time.time()
    x = synth.generate_layer(base)
    print(f"[bench] sweep leg {name}: {nL} layers; generated inputs in {time.time() - t:.1f}s",
          file=sys.stderr, flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    k, v, q = dev(x.k), dev(x.v), dev(x.q)
    del x
    scale = 1.0 / math.sqrt(d)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    ref = torch.empty(err_steps, B, Hq, d, dtype=torch.float32, device="cuda")
    ev = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(2)]  # noqa: E731
    grid = []
    for cs in cluster_sizes:
        w = base.with_(cluster_size=cs)
        C = w.n_clusters
        bp = wi.wave_build_params(B, Hq, H, d, L0, w.capacity, w.segment_size,
                                  w.clusters_per_segment, w.n_iters, w.n_sink, w.n_recent)
        bws = torch.empty(wi.wave_index_workspace_size(bp), dtype=torch.uint8, device="cuda")
        layers = []
        be = ev()
        for l in range(nL):
            ko, vo = torch.empty_like(k), torch.empty_like(v)
            ko[:, :, L0:] = k[:, :, L0:]
            vo[:, :, L0:] = v[:, :, L0:]
            idx = wi.alloc_index(B, H, C, L0, optional=False)
            if l == 0:
                be[0].record()
            wi.wave_index_build(bp, k, v, ko, vo, idx, bws)
            layers.append((ko, vo, idx))
        be[1].record()
        del bws
        # exact reference of layer 0
        ko0, vo0, idx0 = layers[0]
        for s in range(err_steps):
            p = wi.wave_decode_params(B, Hq, H, d, L0 + s + 1, L0, w.capacity, C, w.n_sink,
                                      w.n_recent, 0, scale)
            wi.wave_dense_decode_attention(p, q[s], ko0, vo0, ref[s], None,
                                           wi.alloc_decode_workspace(p))
        torch.cuda.synchronize()
        build_ms = be[0].elapsed_time(be[1])
        for beta in tuple(budgets) + (1.0,):
            nr = int(math.ceil(beta * C - 1e-9))
            dps = [wi.wave_decode_params(B, Hq, H, d, L0 + s + 1, L0, w.capacity, C, w.n_sink,
                                         w.n_recent, nr, scale) for s in range(nq)]
            dws = wi.alloc_decode_workspace(dps[0])
            sel = torch.empty(nq, B, H, nr, dtype=torch.int32, device="cuda")
            point = {"cluster_size": cs, "clusters": C, "budget": beta, "n_retrieve": nr}
            if beta < 1.0:
                step_ev = [ev() for _ in range(nq)]
                for s in range(nq):
                    step_ev[s][0].record()
                    for l in range(nL):
                        ko, vo, idx = layers[l]
                        wi.wave_decode_attention(dps[s], q[(s + l) % nq], ko, vo, idx, out,
                                                 None, sel[s] if l == 0 else None, dws)
                    step_ev[s][1].record()
                torch.cuda.synchronize()
                med = statistics.median(e[0].elapsed_time(e[1]) for e in step_ev[n_warm:])
                csz = idx0.cluster_size.cpu().numpy()
                selh = sel.cpu().numpy()
                E = np.mean([w.n_sink + w.n_recent + s + 1 +
                             float(csz[b, g, selh[s, b, g][selh[s, b, g] >= 0]].sum())
                             for s in range(n_warm, nq) for b in range(B) for g in range(H)])
                nbytes = decode_call_bytes(w, E) * nL
                gbs = nbytes / (med * 1e-3) / 1e9
                point.update({"step_ms": round(med, 4), "decode_tok_s": round(B / (med * 1e-3), 1),
                              "decode_bytes_per_step": nbytes, "decode_hbm_GBps": round(gbs, 1),
                              "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
            errs = []
            for s in range(err_steps):
                wi.wave_decode_attention(dps[s], q[s], ko0, vo0, idx0, out, None, sel[s], dws)
                errs.append(((out - ref[s]).norm(dim=-1) / ref[s].norm(dim=-1)).flatten())
            e = torch.cat(errs).double().cpu().numpy()
            # exact softmax mass on the exactly attended rows: batch 0, KV group 0, step 0
            L = L0 + 1
            m_np = np.zeros(L, dtype=bool)
            m_np[:w.n_sink] = True
            m_np[L0 - w.n_recent:L] = True
            ids = sel[0, 0, 0].cpu().numpy()
            off = idx0.cluster_offset[0, 0].cpu().numpy()
            size = idx0.cluster_size[0, 0].cpu().numpy()
            for j in ids[ids >= 0]:
                m_np[int(off[j]):int(off[j]) + int(size[j])] = True
            mask = torch.from_numpy(m_np).cuda()
            logits = (ko0[0, 0, :L].float() @ q[0][0, :G].float().T) * scale  # [L, G]
            mass = torch.softmax(logits, dim=0)[mask].sum(dim=0).mean().item()
            point.update({"rel_l2_mean": float(f"{e.mean():.3e}"),
                          "rel_l2_p99": float(f"{np.percentile(e, 99):.3e}"),
                          "rel_l2_max": float(f"{e.max():.3e}"),
                          "exact_zone_mass": round(mass, 4),
                          "index_build_ms_stack": round(build_ms, 3)})
            grid.append(point)
            del dws, sel
        del layers, idx0, ko0, vo0
        torch.cuda.empty_cache()
    return {"workload": name, "layers": nL, "batch": B, "context": L0, "n_q_heads": Hq,
            "n_kv_heads": H, "decode_steps": n_steps, "warmup_steps": n_warm,
            "error_steps": err_steps,
            "layer_contents": "layer 0 replicated into every layer's own buffers; layer l "
                              "decodes with the queries of step (s + l) mod steps",
            "reference": "dense decode over all L rows (layer 0)", "grid": grid}


def cpu_baseline(w, x, n_dec_steps=64):
    """The oracle, untuned, on the host cores: with one thread and with all of them
    (os.sched_getaffinity; BLAS threads limited by threadpoolctl, the oracle's own loops
    being single-threaded).
      * the 128K layer (w, inputs x): build = 24 segments (sample i: KV head i mod H, segment
        2 i + i // H mod the segments, three distinct segments per KV head) through all passes,
        extrapolated to the layer by the exact work ratio (segments x KV heads / 24);
        decode = n_dec_steps steps of KV head 0 (its index built by the oracle with one pass,
        untimed: decode work does not depend on the pass count), extrapolated to all KV heads;
      * the 4K layer ('tiny'): the whole build (all heads, all passes) and all its decode
        steps, measured whole.
    `value` is the 128K decode rate at all cores (tokens/s), like the GPU's."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import wave_oracle as wo

    cores = len(os.sched_getaffinity(0))
    g = 0
    segs = wo.segment_ranges(w.context, w.segment_size, w.n_sink, w.n_recent)
    H = w.n_kv_heads
    picks = [(i % H, (2 * i + i // H) % len(segs)) for i in range(3 * H)]
    Ks = [wo.bf16_to_f64(x.k[0, gg, segs[ss][0]:segs[ss][1]]) for gg, ss in picks]
    n_pts = sum(K.shape[0] for K in Ks)
    print("[bench] cpu baseline: oracle index of KV head 0 (decode input, untimed)",
          file=sys.stderr, flush=True)
    with threadpool_limits(cores):
        hidx, ko, vo = wo.build_head(x.k[0, g], x.v[0, g], w.context, w.segment_size,
                                     w.clusters_per_segment, 1, w.n_sink, w.n_recent)
    kc = np.concatenate([ko, x.k[0, g, w.context:]])
    vc = np.concatenate([vo, x.v[0, g, w.context:]])
    G = w.group
    n_dec = min(n_dec_steps, x.q.shape[0])
    tw = synth.WORKLOADS["tiny"]
    tx = synth.generate_layer(tw)
    runs = {}
    for threads in (1, cores):
        print(f"[bench] cpu baseline: {threads} thread(s)", file=sys.stderr, flush=True)
        with threadpool_limits(threads):
            t = time.perf_counter()
            for K in Ks:
                wo.cluster_segment(K, w.clusters_per_segment, w.n_iters)
            t_seg = (time.perf_counter() - t) / len(Ks)
            t = time.perf_counter()
            for s in range(n_dec):
                wo.decode_group(x.q[s][0, g * G:(g + 1) * G], kc, vc, hidx, w.context,
                                w.context + s + 1, w.n_sink, w.n_recent, w.n_retrieve)
            t_head = (time.perf_counter() - t) / n_dec
            t = time.perf_counter()
            tlay = wo.build_layer(tx.k, tx.v, tw.context, tw.segment_size,
                                  tw.clusters_per_segment, tw.n_iters, tw.n_sink, tw.n_recent)
            t_tiny_build = time.perf_counter() - t
            kct = np.concatenate([tlay.k_out, tx.k[:, :, tw.context:]], axis=2)
            vct = np.concatenate([tlay.v_out, tx.v[:, :, tw.context:]], axis=2)
            t = time.perf_counter()
            for s in range(tw.steps):
                wo.decode_layer(tx.q[s], kct, vct, tlay, tw.context, tw.context + s + 1,
                                tw.n_sink, tw.n_recent, tw.n_retrieve)
            t_tiny_dec = (time.perf_counter() - t) / tw.steps
        n_units = w.batch * w.n_kv_heads
        runs[threads] = {
            "threads": threads,
            "llama128k_decode_tok_s": round(w.batch / (t_head * n_units), 3),
            "llama128k_decode_step_s": round(t_head * n_units, 4),
            "llama128k_index_build_tok_s": round(n_pts / len(Ks) / t_seg, 1),
            "llama128k_index_build_s": round(t_seg * len(segs) * n_units, 2),
            "tiny_index_build_s": round(t_tiny_build, 3),
            "tiny_index_build_tok_s": round(tw.batch * tw.context / t_tiny_build, 1),
            "tiny_decode_step_s": round(t_tiny_dec, 4),
            "tiny_decode_tok_s": round(tw.batch / t_tiny_dec, 3)}
    allc = runs[cores]
    return {"value": allc["llama128k_decode_tok_s"], "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"128K layer: decode {n_dec} steps of KV head 0 (index by the oracle, 1 "
                       f"pass, untimed), extrapolated x{w.batch * w.n_kv_heads} to every KV "
                       f"head; build {len(picks)} segments ({n_pts} tokens) x {w.n_iters} "
                       f"passes, extrapolated x{len(segs) * w.batch * w.n_kv_heads / len(picks):g} "
                       f"(segments x KV heads / {len(picks)}); 4K layer: whole build and all "
                       f"{tw.steps} decode steps, measured"),
            "extrapolated": {"llama128k_decode": w.batch * w.n_kv_heads,
                             "llama128k_index_build": len(segs) * w.batch * w.n_kv_heads / len(picks)},
            "one_thread": runs[1], "all_cores": allc}

if __name__ == "__main__":
    main()
