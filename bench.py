#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

One step = one decode step of a whole model's attention on one batch: plan
the batch once (work list shared by every layer), then for each of
``--layers`` layers append the batch's new K/V rows into that layer's paged
cache and run paged attention over every sequence's context. Each layer
has its own cache, so no call finds its KV warm in the caches
(32 layers x ~0.7 GB >> the 256 MB Infinity Cache). The step is captured
once in a HIP graph and replayed, so host launch overhead is not timed.

The default workload is the Llama-3-8B-shaped decode batch: 64 sequences,
contexts uniform on [128, 4096], 32 query / 8 KV heads, head_dim 128, bf16,
16-token blocks drawn from a shuffled pool 1.25x the blocks needed.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "KV-read HBM GB/s (% of peak) + decode attention tokens/s, Llama-3-8B shape"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published


def _threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# parity bounds of the check before timing: per element |gpu - ref| /
# max(1, |ref|), and relative RMS over the sample (same as the test suite)
TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 3e-2}
RRMS = {"f32": 1e-6, "bf16": 4e-3, "fp8": 4e-3}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_inputs(wl, vals) -> dict:
    """Host copies of the GPU run's own inputs, taken before any append:
    q and this step's new K/V rows (stored bits), and the pre-append cache
    (for an fp8 cache: the source values and scales, which the oracle
    leg encodes with its own e4m3 arithmetic)."""
    import torch

    def bits(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    h = {"q": bits(vals.q), "k_new": bits(vals.k_new), "v_new": bits(vals.v_new)}
    if wl.kv_dtype == "fp8":
        h["k_src"], h["v_src"] = bits(vals.k_src), bits(vals.v_src)
        h["k_scale"], h["v_scale"] = bits(vals.k_scale), bits(vals.v_scale)
    else:
        h["k_cache"], h["v_cache"] = bits(vals.k_cache), bits(vals.v_cache)
    return h


def parity_sample(wl) -> np.ndarray:
    """Sequences checked before timing: the shortest, the longest, the
    median, the first and last, the first sequence with more than one
    query token, and six spread over the batch."""
    L = wl.context_lens
    order = np.argsort(L, kind="stable")
    pick = {int(order[0]), int(order[-1]), int(order[len(order) // 2]), 0, wl.num_seqs - 1}
    spans = np.nonzero(wl.query_lens > 1)[0]
    if spans.size:
        pick.add(int(spans[0]))
    pick |= set(int(i) for i in np.linspace(0, wl.num_seqs - 1, 6).astype(int))
    return np.array(sorted(pick), np.int32)


def oracle_leg(wl, host, gpu_out, budget_s: float = 10.0):
    """The CPU oracle on the GPU run's own inputs. First it checks the timed
    configuration's output (``gpu_out``, float64 [T][Hq][D]) on sampled
    sequences against the oracle, then it times the oracle as it stands
    on the host's cores (about ``budget_s``) and on one thread."""
    import oracle

    h = dict(host)
    if wl.kv_dtype == "fp8":
        h["k_cache"] = oracle.fp8_encode_blocks(h.pop("k_src"), h["k_scale"])
        h["v_cache"] = oracle.fp8_encode_blocks(h.pop("v_src"), h["v_scale"])
    else:
        h["k_cache"], h["v_cache"] = h["k_cache"].copy(), h["v_cache"].copy()
    oracle.kv_append(h["k_cache"], h["v_cache"], h["k_new"], h["v_new"], wl.slot_mapping,
                     kv_dtype=wl.kv_dtype, new_dtype=wl.q_dtype, k_scale=h.get("k_scale"),
                     v_scale=h.get("v_scale"), num_kv_heads=wl.num_kv_heads,
                     head_dim=wl.head_dim)
    threads = _threads()
    # parity of the timed configuration on sampled sequences
    sample = parity_sample(wl)
    ref, _ = oracle.run_workload(wl, h, seq_subset=sample, threads=threads)
    qsl = wl.query_start_loc
    rows = np.concatenate([np.arange(qsl[i], qsl[i + 1]) for i in sample])
    g, r = gpu_out[rows], ref[rows]
    key = "fp8" if wl.kv_dtype == "fp8" else wl.q_dtype
    diff = np.abs(g - r)
    err = float(np.max(diff / np.maximum(1.0, np.abs(r)))) if r.size else 0.0
    rrms = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)) if r.size else 0.0
    parity = {"sequences": int(sample.size), "rows": int(rows.size), "max_tol_err": err,
              "rel_rms": rrms, "tol": TOL[key], "rrms_bound": RRMS[key],
              "ok": bool(np.all(np.isfinite(g)) and err <= TOL[key] and rrms <= RRMS[key])}
    # timing: a prefix of the batch's sequences, doubled until the budget
    # is spent (then whole-batch repeats)
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.kv_elem_bytes

    def timed(nthreads, budget, n0):
        reps, t_total, seqs_done, bytes_done = 0, 0.0, 0, 0
        n_sub = max(1, min(wl.num_seqs, n0))
        while t_total < budget and reps < 1000:
            sub = np.arange(n_sub, dtype=np.int32)
            t0 = time.perf_counter()
            oracle.run_workload(wl, h, seq_subset=sub, threads=nthreads)
            dt = time.perf_counter() - t0
            t_total += dt
            seqs_done += n_sub
            bytes_done += int(wl.context_lens[:n_sub].astype(np.int64).sum()) * per_tok
            reps += 1
            if n_sub < wl.num_seqs and dt < budget / 4:
                n_sub = min(wl.num_seqs, n_sub * 2)
        return reps, t_total, seqs_done, bytes_done

    reps, t_total, seqs_done, bytes_done = timed(threads, budget_s, 4)
    r1, t1, s1, b1 = timed(1, max(budget_s / 5, 1.0), 1)
    cpu = {
        "value": round(bytes_done / t_total / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{seqs_done} sequence-layer calls of this batch ({reps} oracle calls over "
                  f"prefixes of the batch, {t_total:.1f} s, float64 gather-then-softmax, "
                  f"{threads} threads) on the GPU run's own input arrays",
        "tokens_per_s": round(seqs_done / t_total, 2),
        "single_thread": {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s",
                          "tokens_per_s": round(s1 / t1, 2),
                          "sample": f"{s1} sequence-layer calls, {t1:.1f} s, 1 thread"},
        "cpu_model": cpu_model(),
    }
    return parity, cpu


PROFILE_FILES = {
    "c1": "kernels_tiny_paged_decode_fp32.md",
    "c2": "kernels_llama3_8b_decode_bf16.md",
    "c3": "kernels_long_context_split_kv_bf16.md",
    "c4": "kernels_hybrid_chunked_prefill_bf16.md",
    "c5": "kernels_70b_decode_fp8_kv.md",
}


def attention_source_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_213_amd",
                        "csrc")
    for f in ("pa_attention.hip", "pa_span.hip", "pa_device.h", "pa_internal.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(config: str, cascade: bool, fp8_qk: bool = False, partition_size: int = 0):
    """HBM bytes per attention launch recorded by the profiler counters for
    this workload and method (profiles/), or None when none are recorded or
    the attention source has changed since they were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        PROFILE_FILES.get(config, ""))
    if not os.path.isfile(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            k, sep, v = line.partition(":")
            if sep and k in ("traffic_bytes_per_launch", "attention_source_sha256", "cascade",
                             "fp8_qk", "partition_size"):
                fields[k] = v.strip()
    if fields.get("attention_source_sha256") != attention_source_sha256():
        return None
    if fields.get("cascade", "off") != ("on" if cascade else "off"):
        return None
    if fields.get("fp8_qk", "off") != ("on" if fp8_qk else "off"):
        return None
    if fields.get("partition_size", "0") != str(int(partition_size)):
        return None
    t = fields.get("traffic_bytes_per_launch")
    return int(t) if t and t.isdigit() else None


def cascade_read_bytes(wl, members_per_tile: int) -> int:
    """K/V bytes cascade attention reads: each group tile reads its group's
    prefix once, each member with keys past the prefix reads only those,
    everything else its whole context (same per-token bytes as the logical
    count, whole prefix blocks)."""
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * wl.kv_elem_bytes
    L = wl.context_lens.astype(np.int64)
    toks = int(L.sum())
    blocks = int(((L + 15) // 16).sum())
    for grp, pb in zip(wl.shared_groups, wl.shared_prefix_blocks):
        tiles = -(-len(grp) // members_per_tile)
        toks += tiles * 16 * pb
        blocks += tiles * pb
        for i in grp:
            if int(wl.query_lens[i]) == 1 and int(L[i]) > 16 * pb:
                toks -= 16 * pb
                blocks -= pb
    b = toks * per_tok
    if wl.kv_dtype == "fp8":
        b += blocks * wl.num_kv_heads * 2 * 4
    return b


def stream_read_probe(pa, torch, dev, mib: int = 4096, reps: int = 10) -> float:
    """GB/s of the library's streaming-read probe over a buffer 16x the
    Infinity Cache: what a plain read of HBM reaches on this device."""
    buf = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(8 * 1024, dtype=torch.int32, device=dev)
    for _ in range(2):
        pa.probe_stream_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pa.probe_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del buf, sink
    return round((mib << 20) / sec / 1e9, 1)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", help="c1..c5 (c2 is the headline workload)")
    ap.add_argument("--layers", type=int, default=32,
                    help="layers per step, each with its own cache (capped so the caches "
                         "fit in about 40 GB; one layer of a large batch already exceeds "
                         "the on-chip caches many times)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=0,
                    help="split-KV piece in tokens (0: balanced over resident waves)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (its parity check before timing and the CPU "
                         "baseline)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a graph")
    ap.add_argument("--cascade", choices=("auto", "on", "off"), default="auto",
                    help="read shared prefixes once per group (auto: when the workload's "
                         "sequences share prefix blocks)")
    ap.add_argument("--append", choices=("fused", "separate"), default="fused",
                    help="decode batches: append the step's K/V rows in the attention pass "
                         "(fused) or with their own launch before it (separate); chunked-"
                         "prefill batches always use the separate launch")
    ap.add_argument("--fp8-qk", action="store_true",
                    help="fp8 cache: S = K q^T on the fp8 matrix cores (two-term fp8 q)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run the library's plain copy kernel over this many MiB, a "
                         "kernel of known traffic for calibrating profiler byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the paged-attention path "
                                   "runs on a single device (sharding is described, not run)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import paged_kv_cache_213_amd as pa
    from paged_kv_cache_213_amd import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    pa.load_library()  # fails loudly if the HIP library is missing

    wl = W.make_config(args.config, seed=args.seed)
    P = args.partition_size
    dev = torch.device("cuda")
    torch.cuda.set_device(0)
    vals = W.materialize(wl, dev)
    # the oracle leg runs on host copies of these very inputs (before any append)
    host = None if args.no_cpu_baseline else host_inputs(wl, vals)
    k_scale = v_scale = None
    if wl.kv_dtype == "fp8":
        # build the e4m3 cache with the library's own append: every valid slot
        # of the pool (finite source rows), quantized with its block's scale
        k_scale, v_scale = vals.k_scale, vals.v_scale
        NB, Hkv, D = wl.num_blocks, wl.num_kv_heads, wl.head_dim
        valid = torch.isfinite(vals.k_src[:, 0, :, 0])  # [NB][16]
        b_idx, o_idx = torch.nonzero(valid, as_tuple=True)
        rows_k = vals.k_src.permute(0, 2, 1, 3)[b_idx, o_idx].to(torch.bfloat16).contiguous()
        rows_v = vals.v_src.permute(0, 3, 1, 2)[b_idx, o_idx].to(torch.bfloat16).contiguous()
        slots_all = (b_idx * 16 + o_idx).to(torch.int32).contiguous()
        vals.k_cache = torch.full((NB, Hkv, 16, D), 0x7F, dtype=torch.uint8, device=dev)
        vals.v_cache = torch.full((NB, Hkv, D, 16), 0x7F, dtype=torch.uint8, device=dev)
        pa.kv_append(vals.k_cache, vals.v_cache, rows_k, rows_v, slots_all, k_scale=k_scale,
                     v_scale=v_scale)
        torch.cuda.synchronize()
        del rows_k, rows_v, slots_all, b_idx, o_idx, valid
        vals.k_src = vals.v_src = None
    per_layer = (vals.k_cache.numel() * vals.k_cache.element_size()) * 2
    layers = max(1, min(args.layers, int(40e9 // per_layer)))
    kc = [vals.k_cache] + [vals.k_cache.clone() for _ in range(layers - 1)]
    vc = [vals.v_cache] + [vals.v_cache.clone() for _ in range(layers - 1)]
    qs = [vals.q] + [vals.q.clone() for _ in range(layers - 1)]
    outs = [torch.empty_like(vals.q) for _ in range(layers)]
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    qsl = None if wl.is_decode else torch.from_numpy(wl.query_start_loc).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    lse = torch.empty(wl.num_tokens, wl.num_q_heads, dtype=torch.float32, device=dev)
    use_cascade = args.cascade == "on" or (args.cascade == "auto" and bool(wl.shared_groups))
    if args.fp8_qk and wl.kv_dtype != "fp8":
        print(json.dumps({"error": "--fp8-qk needs a workload with an fp8 cache"}))
        sys.exit(2)
    shape = pa.make_shape(vals.q, vals.k_cache, bt, P, cascade=use_cascade, fp8_qk=args.fp8_qk)
    groups = pa.PrefixGroups(wl.shared_groups, wl.shared_prefix_blocks, dev) if use_cascade \
        else None
    nbytes = pa.workspace_bytes(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len,
                                wl.max_query_len)
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    mq = 1 if wl.is_decode else wl.max_query_len
    fused = args.append == "fused" and wl.is_decode
    app_kw = dict(k_new=vals.k_new, v_new=vals.v_new) if fused else {}

    def model_step(stream):
        if groups is not None:
            pa.plan_cascade(shape, cl, ws, groups, query_start_loc=qsl,
                            num_q_tokens=wl.num_tokens, max_query_len=mq,
                            max_context_len=wl.max_context_len, stream=stream)
        else:
            pa.plan(shape, cl, ws, query_start_loc=qsl, num_q_tokens=wl.num_tokens,
                    max_query_len=mq, max_context_len=wl.max_context_len, stream=stream)
        for L_ in range(layers):
            if not fused:
                pa.kv_append(kc[L_], vc[L_], vals.k_new, vals.v_new, slots, k_scale=k_scale,
                             v_scale=v_scale, stream=stream)
            pa.run(shape, qs[L_], kc[L_], vc[L_], bt, cl, wl.scale, ws, query_start_loc=qsl,
                   max_query_len=mq, max_context_len=wl.max_context_len, out=outs[L_],
                   lse=lse, stream=stream, passes="partial", k_scale=k_scale, v_scale=v_scale,
                   **app_kw)
            pa.run(shape, qs[L_], kc[L_], vc[L_], bt, cl, wl.scale, ws, query_start_loc=qsl,
                   max_query_len=mq, max_context_len=wl.max_context_len, out=outs[L_],
                   lse=lse, stream=stream, passes="merge")

    def model_step_plan(stream):
        if groups is not None:
            pa.plan_cascade(shape, cl, ws, groups, query_start_loc=qsl,
                            num_q_tokens=wl.num_tokens, max_query_len=mq,
                            max_context_len=wl.max_context_len, stream=stream)
        else:
            pa.plan(shape, cl, ws, query_start_loc=qsl, num_q_tokens=wl.num_tokens,
                    max_query_len=mq, max_context_len=wl.max_context_len, stream=stream)

    if args.calibrate_copy_mib > 0:
        nb = args.calibrate_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        pa.probe_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    s = torch.cuda.Stream()
    graph = None
    with torch.cuda.stream(s):
        for _ in range(2):
            model_step(s)  # eager warm-up (also sets the occupancy caches)
        s.synchronize()
        if not args.no_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=s):
                model_step(s)

    def replay():
        with torch.cuda.stream(s):
            if graph is not None:
                graph.replay()
            else:
                model_step(s)

    for _ in range(args.warmup):
        replay()
    torch.cuda.synchronize()
    if not all(bool(torch.isfinite(o.float()).all()) for o in outs):
        raise SystemExit("non-finite attention output")
    # before timing: the timed configuration's output against the oracle on
    # sampled sequences, then the oracle's own timing (CPU baseline)
    parity = cpu = None
    if host is not None:
        gpu_out = outs[0].float().cpu().numpy().astype(np.float64)
        parity, cpu = oracle_leg(wl, host, gpu_out, args.cpu_budget)
        del host, gpu_out
        if not parity["ok"]:
            print(json.dumps({"error": "parity check before timing failed", "parity": parity}))
            sys.exit(3)

    # timed region: exactly `steps` model steps
    att_ms = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # spread: each of max(50, steps) further steps timed on its own
    n_spread = max(50, args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread + 1)]
    evs[0].record(s)
    for i in range(n_spread):
        replay()
        evs[i + 1].record(s)
    torch.cuda.synchronize()
    step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n_spread)])
    # the attention kernel's own duration: one event pair around the pass-1
    # launches of every layer, back to back on the stream (they are
    # independent); a GPU spin first lets the host enqueue ahead of the GPU,
    # so the interval holds only those kernels
    with torch.cuda.stream(s):
        for _ in range(min(args.steps, 10)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(2_000_000)
            e0.record(s)
            for L_ in range(layers):
                pa.run(shape, qs[L_], kc[L_], vc[L_], bt, cl, wl.scale, ws, query_start_loc=qsl,
                       max_query_len=mq, max_context_len=wl.max_context_len, out=outs[L_],
                       lse=lse, stream=s, passes="partial", k_scale=k_scale, v_scale=v_scale,
                       **app_kw)
            e1.record(s)
            s.synchronize()
            att_ms.append(e0.elapsed_time(e1) / layers)
    att_ms = np.array(att_ms)

    def back_to_back_us(enqueue_layer, reps=5):
        """Mean duration of one launch, timed over every layer's launch back
        to back (same method as the attention pass above)."""
        per = []
        with torch.cuda.stream(s):
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(2_000_000)
                e0.record(s)
                for L_ in range(layers):
                    enqueue_layer(L_)
                e1.record(s)
                s.synchronize()
                per.append(e0.elapsed_time(e1) * 1e3 / layers)
        return round(float(np.mean(per)), 2)

    # (a fused append is inside the attention pass's time)
    append_us = None if fused else back_to_back_us(lambda L_: pa.kv_append(
        kc[L_], vc[L_], vals.k_new, vals.v_new, slots, k_scale=k_scale, v_scale=v_scale,
        stream=s))
    merge_us = back_to_back_us(lambda L_: pa.run(
        shape, qs[L_], kc[L_], vc[L_], bt, cl, wl.scale, ws, query_start_loc=qsl,
        max_query_len=mq, max_context_len=wl.max_context_len, out=outs[L_], lse=lse, stream=s,
        passes="merge"))
    plan_us = back_to_back_us(lambda L_: model_step_plan(s))
    probe_gbs = stream_read_probe(pa, torch, dev)
    ms_per_step = wall * 1e3 / args.steps
    kv_bytes = wl.kv_bytes_logical()
    value = layers * kv_bytes / (ms_per_step / 1e3) / 1e9
    att_mean = float(att_ms.mean())
    # the roofline counts what the method must read: the logical bytes, or
    # with cascade the group prefixes once per group tile
    # members per group tile, as the library's layout gives them
    mpt = pa.workspace_layout(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len, mq,
                              decode=wl.is_decode).members_per_tile
    read_bytes = cascade_read_bytes(wl, mpt) if use_cascade else kv_bytes
    achieved = read_bytes / (att_mean / 1e3) / 1e9
    layer_ms = ms_per_step / layers
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 KV, bf16 q"}[wl.kv_dtype],
        "data": "synthetic (seeded N(0,1) values, shuffled block pool)",
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(wl.num_tokens / (ms_per_step / 1e3), 1),
        "tokens_per_s_per_layer_call": round(wl.num_tokens / (layer_ms / 1e3), 1),
        "kv_tokens_per_s_per_layer_call": round(float(wl.context_lens.sum()) / (layer_ms / 1e3), 1),
        "config": {
            "workload": f"{wl.name}: {W.CONFIG_TITLES[wl.name]}",
            "num_seqs": wl.num_seqs,
            "num_q_tokens": wl.num_tokens,
            "q_heads": wl.num_q_heads,
            "kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim,
            "block_size": 16,
            "sum_context_len": int(wl.context_lens.sum()),
            "kv_bytes_per_layer": kv_bytes,
            "layers_per_step": layers,
            "partition_size": P,
            "graph": graph is not None,
            "cascade": use_cascade,
            "fp8_qk": bool(args.fp8_qk),
            "append": "fused into the attention pass" if fused else "separate launch",
            "kv_bytes_read_per_layer": read_bytes,
            "kv_bytes_unique_per_layer": wl.kv_bytes_unique() if wl.shared_groups else kv_bytes,
            "seed": wl.seed,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": recorded_traffic(wl.name, use_cascade, args.fp8_qk, P),
            "traffic_note": "HBM bytes per attention pass launch (calibrated FETCH_SIZE + "
                            "WRITE_SIZE, profiles/); null if not recorded for the current "
                            "attention source",
            "kernel": "attention pass (attention_narrow per layer, beside attention_span "
                      "on the library's second stream when the batch has chunked-prefill "
                      "spans; decode batches append the step's K/V rows in it unless "
                      "--append separate); HIP events on the caller's stream around the "
                      "back-to-back pass-1 calls of all layers, divided by the layers",
            "launch_us_mean": round(att_mean * 1e3, 2),
            "launch_us_min_max": [round(float(att_ms.min()) * 1e3, 2),
                                  round(float(att_ms.max()) * 1e3, 2)],
            "stream_read_probe_gbs": probe_gbs,
            "frac_of_stream_read_probe": round(achieved / probe_gbs, 4),
        },
        "launch_us": {"plan_per_step": plan_us, "kv_append": append_us,
                      "attention": round(att_mean * 1e3, 2), "merge": merge_us},
        "step_ms_spread": {"n": n_spread, "p10": round(float(np.percentile(step_ms, 10)), 5),
                           "median": round(float(np.median(step_ms)), 5),
                           "p90": round(float(np.percentile(step_ms, 90)), 5),
                           "note": "each step timed alone with HIP events on the replay stream, "
                                   "after the timed region"},
    }
    if parity is not None:
        res["parity_before_timing"] = parity
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
