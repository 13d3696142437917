#!/usr/bin/env python3
"""Benchmark of one GDN layer's speculative verify + commit step on one MI355X.

A step is the whole hot path over one batch of synthetic drafts for one GDN
layer (h = 8, d_k = d_v = 256, FP32 state): verification (chain kernel for
chain workloads, tree-masked factorized kernel otherwise) and the commit of
an accepted path from a factor record.  By default the commit is delayed: the
step's single launch first commits the accepted path of the draft that the
same state verified on its previous visit, then verifies the new draft
(bitwise the same as commit followed by verify); --separate-commit runs the
plain verification and then gdn_commit_path as two launches.  Steps rotate
over enough distinct layer states (default 1 GiB in total, several times the
256 MB Infinity Cache) that every state read comes from HBM.  The
decode24-b1-h8-d256 workload runs the 24-layer decode loop instead.

The default workload is tree64-b8-h8-d256 (batch 8, 64-node trees: the
largest single-GPU per-layer configuration); the 8-node chain
(chain8-b1-h8-d256) is measured in the same run for the HBM half of the
metric.

Prints one JSON line:
  value           verified draft nodes per second (B * N per step); K steps
                  replayed as one HIP graph, timed with HIP events on the
                  stream the kernels run on (no host launch overhead)
  ms_per_step     that time per step; with the delayed commit a step is one
                  launch, so it is also the kernel's average launch duration
  roofline        of the step's kernel, every fraction from ms_per_step: for
                  the tree kernel its FP32-equivalent contraction flops per
                  launch against the 157.3 TFLOP/s FP32 peak (frac), the bf16
                  MFMA work it actually issues and the matrix units' busy
                  fraction from the committed rocprofv3 counters
                  (issued_mfma), and its algorithmic HBM bytes against 8 TB/s
                  (hbm); for the chain kernel its algorithmic bytes against
                  8 TB/s; `traffic` = HBM bytes per launch from the
                  rocprofv3 counter summaries in profiles/
  chain8          the 8-node chain's step with its HBM roofline
  cpu_baseline    the CPU oracle (per-path fp64 replay + commit replay):
                  median of 5 trials on all threads and on one thread
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_gdn_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0
CLOCK_HZ = 2.4e9  # peak engine clock, for MFMA-busy fractions
# the configuration the bench line is quoted on: the largest single-GPU
# per-layer workload (batch-8 64-node trees), with the 8-node chain's HBM
# figures alongside
DEFAULT_WORKLOAD = "tree64-b8-h8-d256"
CHAIN_WORKLOAD = "chain8-b1-h8-d256"
CSRC = os.path.join(ROOT, "linear_attention_gdn_amd", "csrc")
# the sources each entry point's kernels are built from (tree verification at
# batch x heads >= 256 runs the split-role kernel of tree_verify_ws.hip)
KERNEL_SOURCES = {
    "gdn_chain_verify": ["chain_verify.hip"],
    "gdn_chain_verify_delayed": ["chain_verify.hip"],
    "gdn_tree_verify": ["tree_verify.hip", "tree_verify_ws.hip", "tree_common.h"],
    "gdn_tree_verify_delayed": ["tree_verify.hip", "tree_verify_ws.hip", "tree_common.h"],
    "gdn_layer_verify": ["tree_verify.hip", "tree_verify_ws.hip", "tree_common.h"],
    "gdn_commit_path": ["commit.hip"],
    "gdn_linear": ["layer.hip"],
}


def source_digest(kernel: str) -> str:
    """Short hash of a kernel's sources (and the shared header) to tie counters to code."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["gdn_common.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def _counter_summary(kind: str, kernel: str, workload: str):
    """Fields of a committed rocprofv3 counter summary (profiles/<kind>_<kernel>_<workload>.txt)
    if it was taken on the current source of that kernel, else None."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_digest") != source_digest(kernel):
        return None
    return fields


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current source of that kernel (else None)."""
    fields = _counter_summary("traffic", kernel, workload)
    try:
        return float(fields["hbm_bytes_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def measured_mfma(kernel: str, workload: str, avg_us: float):
    """Issued bf16 MFMA work per launch from the committed counter summary
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP; MFMA-busy cycles per SIMD), as
    rates over this run's measured launch time; None if absent or stale."""
    fields = _counter_summary("mfma", kernel, workload)
    if not fields:
        return None
    try:
        f = float(fields["bf16_mfma_flop_per_launch"])
        busy = float(fields["mfma_busy_cycles_per_simd"])
    except (KeyError, ValueError):
        return None
    t_s = avg_us * 1e-6
    return {"bf16_flop_per_launch": f, "issued_tflops": round(f / t_s / 1e12, 2),
            "issued_frac": round(f / t_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "busy_cycles_per_simd": busy,
            "busy_frac_at_2p4ghz": round(busy / (t_s * CLOCK_HZ), 4)}


def calibrate_copy(mib: int, iters: int) -> None:
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    n = (mib << 20) // 4
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "iters": iters}), flush=True)


def bytes_verify(d: W.Draft, tree: bool) -> int:
    """Algorithmic HBM bytes of one verification launch (inputs read once,
    outputs and factor record written once; no scratch)."""
    es = 2 if d.dtype == "bf16" else 4
    B, N, H, dk, dv = d.B, d.N, d.H, d.dk, d.dv
    state = B * H * dv * dk * 4
    qkv = B * N * H * (2 * dk + dv) * es
    bg = B * N * H * 8
    out = B * N * H * dv * 4
    rec = B * H * N * (dv * 4 + 4 + dk * es) + B * N * 12
    par = B * N * 4 if tree else 0
    return state + qkv + bg + out + rec + par


def bytes_commit(d: W.Draft, plens: np.ndarray) -> float:
    """Algorithmic bytes of one commit: every sequence with a non-empty path
    reads and writes its state once and reads its path's u', k and G."""
    es = 2 if d.dtype == "bf16" else 4
    B, N, H, dk, dv = d.B, d.N, d.H, d.dk, d.dv
    tot = 0.0
    for n in plens:
        if n > 0:
            tot += 2 * H * dv * dk * 4 + H * n * (dv * 4 + dk * es + 4) + N * 8
    return tot + B * 4


def bytes_delayed(d: W.Draft, plens: np.ndarray, tree: bool) -> float:
    """Algorithmic bytes of one delayed-commit verification: the verification's
    own bytes, plus, for every sequence with a non-empty accepted path, the
    state written back once and the path's u', k and G read from the previous
    record (the state read is shared with the verification)."""
    es = 2 if d.dtype == "bf16" else 4
    B, N, H, dk, dv = d.B, d.N, d.H, d.dk, d.dv
    tot = float(bytes_verify(d, tree)) + B * N * 8 + B * 4
    for n in plens:
        if n > 0:
            tot += H * dv * dk * 4 + H * n * (dv * 4 + dk * es + 4)
    return tot


def draw_lasts(d: W.Draft, rng, count: int, chain: bool) -> np.ndarray:
    out = np.empty((count, d.B), dtype=np.int32)
    for i in range(count):
        for b in range(d.B):
            if chain:
                out[i, b] = int(rng.integers(0, d.N + 1)) - 1
            else:
                mean = 3.0 if d.N <= 32 else 4.0
                out[i, b] = W.accept_leaf_geometric(d.parents[b], rng, mean)
    return out


def path_lengths(d: W.Draft, lasts: np.ndarray) -> np.ndarray:
    depth = np.stack([W.depths_of(d.parents[b]) for b in range(d.B)])
    return np.array([[0 if l < 0 else depth[b, l] for b, l in enumerate(row)] for row in lasts])


def _median_rate(run_once, units_per_call, trials: int, min_s: float):
    """Median over `trials` of (units done / seconds) where each trial repeats
    run_once() for at least min_s seconds (and at least once)."""
    rates, calls = [], 0
    for _ in range(trials):
        n, t0 = 0, time.perf_counter()
        while True:
            run_once(calls)
            n += 1
            calls += 1
            el = time.perf_counter() - t0
            if el >= min_s:
                break
        rates.append(n * units_per_call / el)
    return float(np.median(rates)), calls


def cpu_baseline(d: W.Draft, lasts: np.ndarray, budget_s: float):
    """The oracle (per-path fp64 replay + commit replay) on the host: median of
    5 timed trials on all OpenMP threads and median of 5 on one thread, each
    trial at least budget_s / 10 seconds."""
    from oracle import oracle as O

    q, k, v = d.q64(), d.k64(), d.v64()

    def step(i):
        O.tree_verify(d.S0, d.parents, q, k, v, d.beta, d.g, d.scale)
        O.commit(d.S0, d.parents, k, v, d.beta, d.g, lasts[i % len(lasts)])

    threads = O.set_threads(0)
    t0 = time.perf_counter()
    step(0)  # warm-up (library load, page-in)
    many, n_many = _median_rate(step, d.B * d.N, 5, budget_s / 10)
    O.set_threads(1)
    one, n_one = _median_rate(step, d.B * d.N, 5, budget_s / 10)
    O.set_threads(threads)
    el = time.perf_counter() - t0
    return {"value": round(many, 1), "unit": "nodes/s", "cores": threads, "kind": "oracle",
            "value_1_thread": round(one, 1), "trials": 5, "statistic": "median",
            "sample": f"{d.name}: one step = verify by per-path fp64 replay + commit replay of "
                      f"a drawn accepted path; median of 5 trials on {threads} threads "
                      f"({n_many} steps) and of 5 on 1 thread ({n_one} steps); {el:.1f} s "
                      f"of CPU work in total"}


def layer_run(args, workload: str, extras: bool) -> dict:
    """One GDN layer's verify + commit steps on `workload`: the timed graph of
    K steps (HIP events on the launching stream), the roofline of the step's
    kernel, and with `extras` the separate kernels, the latency floor and the
    timing variants as context."""
    import torch

    from linear_attention_gdn_amd import gdnspec as G

    dev = torch.device("cuda:0")
    d = W.WORKLOADS[workload](0)
    chain = workload.startswith("chain")
    B, N, H, dk, dv = d.B, d.N, d.H, d.dk, d.dv
    code = G.GDN_BF16 if d.dtype == "bf16" else G.GDN_F32

    state_bytes = B * H * dv * dk * 4
    R = max(1, (args.rotate_mib << 20) // state_bytes)
    S0 = torch.from_numpy(d.S0).to(dev)
    states = [S0.clone() for _ in range(R)]
    bf = lambda x: torch.from_numpy(x.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    f = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    q, k, v = bf(d.q), bf(d.k), bf(d.v)
    beta, g = f(d.beta), f(d.g)
    parents = torch.from_numpy(d.parents).to(dev)
    out = torch.empty(B, N, H, dv, device=dev)
    rec = G.FactorRecord.empty(B, N, H, dk, dv, code, device=dev)
    rng = np.random.default_rng(1234)
    total = args.warmup + args.steps
    lasts_np = draw_lasts(d, rng, total, chain)
    lasts = torch.from_numpy(lasts_np).to(dev)

    def verify(i):
        S = states[i % R]
        if chain:
            G.gdn_chain_verify(S, q, k, v, beta, g, out, rec)
        else:
            G.gdn_tree_verify(S, parents, q, k, v, beta, g, out, rec)

    def commit(i):
        G.gdn_commit_path(states[i % R], rec, lasts[i])

    # Delayed commit: step i commits, on state i % R, the draft that state
    # verified on its previous visit (accepted node lasts[i]) and verifies
    # the new draft, in one launch.  Each state keeps two record slots used
    # alternately.
    delayed = not args.separate_commit
    if delayed:
        recs = [[G.FactorRecord.empty(B, N, H, dk, dv, code, device=dev) for _ in range(2)]
                for _ in range(R)]
        for j in range(R):  # every state's "previous visit": a plain verify
            if chain:
                G.gdn_chain_verify(states[j], q, k, v, beta, g, out, recs[j][1])
            else:
                G.gdn_tree_verify(states[j], parents, q, k, v, beta, g, out, recs[j][1])
        torch.cuda.synchronize()

    def fused(i):
        j, vis = i % R, i // R
        if chain:
            G.gdn_chain_verify_delayed(states[j], recs[j][(vis + 1) % 2], lasts[i], q, k, v, beta,
                                       g, out, recs[j][vis % 2])
        else:
            G.gdn_tree_verify_delayed(states[j], recs[j][(vis + 1) % 2], lasts[i], parents, q, k,
                                      v, beta, g, out, recs[j][vis % 2])

    def step(i):
        if delayed:
            fused(i)
        else:
            verify(i)
            commit(i)

    # warmup (eager)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    timed = range(args.warmup, total)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if args.no_graph:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in timed:
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in timed:
                    step(i)
        stream.wait_stream(s)
        graph.replay()  # first replay uploads the graph; not timed
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        graph.replay()  # on the current stream: the stream every kernel of the step runs on
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    elapsed = e0.elapsed_time(e1) * 1e-3  # seconds, HIP events
    ms_per_step = elapsed * 1e3 / args.steps
    value = B * N / (elapsed / args.steps)
    res = {"d": d, "chain": chain, "delayed": delayed, "R": R, "ms_per_step": ms_per_step,
           "wall_ms_per_step": wall * 1e3 / args.steps, "value": value}

    # algorithmic bytes of the step's kernel(s), over the accepted paths drawn
    # for the timed steps
    plens = path_lengths(d, lasts_np[args.warmup:total])
    b_step = (np.mean([bytes_delayed(d, p, not chain) for p in plens]) if delayed else
              bytes_verify(d, not chain) + np.mean([bytes_commit(d, p) for p in plens]))
    res["step_bytes"] = float(b_step)
    res["step_kernel"] = (("gdn_chain_verify_delayed" if chain else "gdn_tree_verify_delayed")
                          if delayed else None)
    if not extras:
        return res

    # Per-kernel durations: each kernel alone, `nper` back-to-back launches
    # captured in a HIP graph, timed with events on the stream it runs on.
    nper = min(args.steps, 400)

    def graph_time(fn):
        gph = torch.cuda.CUDAGraph()
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):
            with torch.cuda.graph(gph, stream=gs):
                for j in range(nper):
                    fn(args.warmup + j)
        stream.wait_stream(gs)
        gph.replay()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        gph.replay()
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / nper

    if args.no_graph:  # eager: event pairs around single launches
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4 * nper)]
        for j in range(nper):
            i = args.warmup + j
            evs[4 * j].record(stream)
            verify(i)
            evs[4 * j + 1].record(stream)
            evs[4 * j + 2].record(stream)
            commit(i)
            evs[4 * j + 3].record(stream)
        torch.cuda.synchronize()
        t_ver = np.array([evs[4 * j].elapsed_time(evs[4 * j + 1]) for j in range(nper)])
        t_com = np.array([evs[4 * j + 2].elapsed_time(evs[4 * j + 3]) for j in range(nper)])
    else:
        t_ver = np.array([graph_time(verify)])
        t_com = np.array([graph_time(commit)])
    # The latency floor of one step on this GPU, in the same harness: an empty
    # kernel, and a plain device copy that reads one step's states (rotating
    # like the steps, so from HBM) and writes as many bytes.
    floor = None
    if not args.no_graph:
        scratch = torch.empty_like(states[0])
        t_empty = graph_time(lambda i: torch.cuda._sleep(0))
        t_copy = graph_time(lambda i: scratch.copy_(states[i % R]))
        floor = {"empty_kernel_us": round(t_empty * 1e3, 3),
                 "state_copy_us": round(t_copy * 1e3, 3),
                 "state_copy_bytes": 2 * state_bytes,
                 "state_copy_gbs": round(2 * state_bytes / (t_copy * 1e-3) / 1e9, 1)}
    # The same step on one resident state (hot: back-to-back in a graph, the
    # state served from the caches), and single steps called eagerly from
    # Python and waited for (host call to completion, rotating states), median.
    variants = None
    if not args.no_graph:
        def step_on(j, i):
            if delayed:
                if chain:
                    G.gdn_chain_verify_delayed(states[j], recs[j][(i + 1) % 2], lasts[i], q, k,
                                               v, beta, g, out, recs[j][i % 2])
                else:
                    G.gdn_tree_verify_delayed(states[j], recs[j][(i + 1) % 2], lasts[i], parents,
                                              q, k, v, beta, g, out, recs[j][i % 2])
            else:
                if chain:
                    G.gdn_chain_verify(states[j], q, k, v, beta, g, out, rec)
                else:
                    G.gdn_tree_verify(states[j], parents, q, k, v, beta, g, out, rec)
                G.gdn_commit_path(states[j], rec, lasts[i])

        t_hot = graph_time(lambda i: step_on(0, i))
        ts = []
        for j in range(min(60, args.steps)):  # step indices stay within the drawn lasts
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            step_on(j % R, args.warmup + j)
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        variants = {"hot_state_graph_us_per_step": round(t_hot * 1e3, 3),
                    "eager_single_step_us_median":
                        round(float(np.median(ts[len(ts) // 6:])) * 1e6, 2)}
    plens_k = path_lengths(d, lasts_np[args.warmup:args.warmup + nper])
    b_ver = bytes_verify(d, not chain)
    b_com = np.mean([bytes_commit(d, p) for p in plens_k])
    kernels = {
        "verify": {"name": "gdn_chain_verify" if chain else "gdn_tree_verify",
                   "avg_us": round(float(t_ver.mean() * 1e3), 3), "bytes": int(b_ver),
                   "gbs": round(float(b_ver / (t_ver.mean() * 1e-3) / 1e9), 1)},
        "commit": {"name": "gdn_commit_path", "avg_us": round(float(t_com.mean() * 1e3), 3),
                   "bytes": float(b_com),
                   "gbs": round(float(b_com / (t_com.mean() * 1e-3) / 1e9), 1)},
    }
    if not chain:
        flops = 4.0 * B * H * N * dk * dv
        kernels["verify"]["fp32_equiv_tflops"] = round(float(flops / (t_ver.mean() * 1e-3) / 1e12), 2)
    # The pages' baselines on this GPU (root-to-leaf replay against tree
    # verification, token replay against the factor-buffer commit) and the
    # chain-decomposed hybrid verifier, timed the same way as the kernels above.
    replay = None
    if not args.no_graph:
        leaves = [W.leaves_of(p) for p in d.parents]
        P = max(len(l) for l in leaves)
        ends_np = np.full((B, P), -1, np.int32)
        for b, l in enumerate(leaves):
            ends_np[b, :len(l)] = l
        ends = torch.from_numpy(ends_np).to(dev)
        t_rv = graph_time(lambda i: G.gdn_replay_verify(states[i % R], parents, q, k, v, beta, g,
                                                        ends, out))
        t_rc = graph_time(lambda i: G.gdn_replay_commit(states[i % R], parents, k, v, beta, g,
                                                        lasts[i]))
        hplan = G.HybridPlan(d.parents, device=dev)
        t_hy = graph_time(lambda i: G.gdn_hybrid_verify(states[i % R], parents, q, k, v, beta, g,
                                                        out, rec, hplan))
        replay = {"root_to_leaf_replay_us": round(t_rv * 1e3, 3), "paths_per_sequence": P,
                  "hybrid_chain_verify_us": round(t_hy * 1e3, 3),
                  "hybrid_levels": hplan.levels,
                  "hybrid_chains_per_level": [int(c) for c in
                                              hplan.chains_per_level[:hplan.levels]],
                  "verify_us": round(float(t_ver.mean() * 1e3), 3),
                  "verify_speedup_over_replay": round(t_rv / float(t_ver.mean()), 2),
                  "token_replay_commit_us": round(t_rc * 1e3, 3),
                  "commit_us": round(float(t_com.mean() * 1e3), 3),
                  "commit_speedup_over_replay": round(t_rc / float(t_com.mean()), 2)}
    res.update(kernels=kernels, floor=floor, variants=variants, replay=replay)
    return res


def prune_timing(args) -> dict:
    """Confidence-guided pruning of batch-8 candidate trees shaped like the
    pages' drafter (top-4 continuations to depth 4: 341 candidates, budget 16
    nodes, margin 3 nats), HIP-graph timing of back-to-back launches."""
    import torch

    from linear_attention_gdn_amd import gdnspec as G
    B, T, tau = 8, 16, 3.0
    par, conf = W.candidate_batch(B, seed=5, top_k=4, depth=4)
    dev = torch.device("cuda:0")
    pt = torch.from_numpy(par).to(dev)
    ct = torch.from_numpy(conf).to(dev)
    kept = torch.empty(B, T, dtype=torch.int32, device=dev)
    newp = torch.empty(B, T, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    n = 200
    gph = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        with torch.cuda.graph(gph, stream=gs):
            for _ in range(n):
                G.gdn_prune_draft(pt, ct, tau, kept, newp, cnt)
    stream.wait_stream(gs)
    gph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    gph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    return {"B": B, "candidates": int(par.shape[1]), "budget": T, "tau": tau, "avg_us": round(us, 3),
            "mean_kept": round(float(cnt.float().mean()), 2)}


def roofline_of(res: dict) -> dict:
    """Roofline of the step's kernel.  The step is one launch (the delayed
    commit fused into the verification), so the kernel's average launch
    duration is the event-timed step itself (ms_per_step), and every fraction
    below is computed from it."""
    d, chain = res["d"], res["chain"]
    t_s = res["ms_per_step"] * 1e-3
    kern = res["step_kernel"] or ("gdn_chain_verify + gdn_commit_path" if chain
                                  else "gdn_tree_verify + gdn_commit_path")
    gbs = res["step_bytes"] / t_s / 1e9
    traffic = measured_traffic(res["step_kernel"], d.name) if res["step_kernel"] else None
    hbm = {"achieved_gbs": round(gbs, 2), "peak_gbs": HBM_PEAK_GBS,
           "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": round(res["step_bytes"])}
    if chain:  # the serial chain kernel streams the state: HBM roofline
        return {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kern,
                "duration_us": round(t_s * 1e6, 3), "algorithmic_bytes": round(res["step_bytes"])}
    # the tree kernel's S0 contraction, FP32-accurate on bf16 matrix cores
    B, N, H, dk, dv = d.B, d.N, d.H, d.dk, d.dv
    flops = 4.0 * B * H * N * dk * dv  # algorithmic (FP32-equivalent) per launch
    tflops = flops / t_s / 1e12
    mf = measured_mfma(res["step_kernel"], d.name, t_s * 1e6) if res["step_kernel"] else None
    issued = None
    if mf:
        issued = {"type": "bf16 (v_mfma_f32_16x16x32_bf16, v_mfma_f32_16x16x16_bf16)",
                  "flop_per_launch": mf["bf16_flop_per_launch"],
                  "achieved_tflops": mf["issued_tflops"], "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                  "frac": mf["issued_frac"],
                  "busy_cycles_per_simd": mf["busy_cycles_per_simd"],
                  "busy_frac": mf["busy_frac_at_2p4ghz"]}
    return {"bound": "mfma", "achieved": round(tflops, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic, "kernel": kern, "duration_us": round(t_s * 1e6, 3),
            "algorithmic_flops": flops,
            "fp32_equiv": {"achieved_tflops": round(tflops, 2),
                           "peak_tflops": FP32_MFMA_PEAK_TFLOPS,
                           "frac": round(tflops / FP32_MFMA_PEAK_TFLOPS, 4)},
            "issued_mfma": issued, "hbm": hbm}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(W.WORKLOADS) + sorted(W.STACK_WORKLOADS))
    ap.add_argument("--rotate-mib", type=int, default=1024,
                    help="total size of the rotating layer states")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the 8-node chain's HBM figures that accompany a tree workload")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    ap.add_argument("--separate-commit", action="store_true",
                    help="verify and commit as two launches per step instead of the delayed "
                         "commit fused into the next verification")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 20)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the verify/commit path shards over "
              "(sequence, head, state-row tile) units with no exchange, so there is no "
              "multi-GPU step to time; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload in W.STACK_WORKLOADS:
        bench_decode_loop(args)
        return

    import torch

    torch.cuda.set_device(0)
    res = layer_run(args, args.workload, extras=True)
    d = res["d"]
    roofline = roofline_of(res)
    # The 8-node chain (the HBM half of the metric), measured in the same run
    # with the same step count and timing.
    chain8 = None
    if not res["chain"] and not args.no_chain:
        rc = layer_run(args, CHAIN_WORKLOAD, extras=False)
        rr = roofline_of(rc)
        chain8 = {"workload": CHAIN_WORKLOAD, "ms_per_step": round(rc["ms_per_step"], 6),
                  "value": round(rc["value"], 1), "unit": "nodes/s", "kernel": rr["kernel"],
                  "bound": "hbm", "achieved": rr["achieved"], "peak": HBM_PEAK_GBS,
                  "unit_roofline": "GB/s", "frac": rr["frac"], "traffic": rr["traffic"],
                  "algorithmic_bytes": rr["algorithmic_bytes"]}

    pruning = None if args.no_graph else prune_timing(args)

    cpu = None
    if not args.no_cpu_baseline:
        rng = np.random.default_rng(99)
        cpu = cpu_baseline(d, draw_lasts(d, rng, 64, res["chain"]), args.cpu_seconds)

    B, N, H, dk, dv = d.B, d.N, d.H, d.dk, d.dv
    line = {
        "metric": "verified draft nodes/sec per GDN layer (h=8,d=256)",
        "value": round(res["value"], 1),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": d.name, "B": B, "N": N, "H": H, "dk": dk, "dv": dv,
                   "qkv_dtype": d.dtype, "state_dtype": "f32", "rotating_states": res["R"],
                   "timing": "eager" if args.no_graph else "hip_graph",
                   "commit": "delayed, fused into the next verification" if res["delayed"]
                             else "separate launch after each verification",
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "chain8": chain8,
        "wall_ms_per_step": round(res["wall_ms_per_step"], 6),
        "latency_floor": res["floor"],
        "timing_variants": res["variants"],
        "kernels": res["kernels"],
        "replay_baselines": res["replay"],
        "pruning": pruning,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# the decode loop over a stack of layers
# ---------------------------------------------------------------------------


def _graph_of(fn, count, stream):
    """Capture `count` calls fn(0..count-1) in one HIP graph (uploaded by a
    first replay)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for j in range(count):
                fn(j)
    stream.wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    return g


def _time_graph(g, stream, reps=1):
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3  # seconds


def _time_eager(fn, count, stream, reps=1):
    """Seconds for reps * count direct calls fn(0..count-1) on `stream`."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        for j in range(count):
            fn(j)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def stack_cpu_baseline(shape, layers, S0, parents, lasts, x0_bits, budget_s):
    """Oracle steps (24-layer verify + commit, fp64 with bf16 rounding at the
    projection inputs and q/k/v) on the host for about `budget_s` seconds."""
    from oracle import layer as LY
    from oracle import oracle as O

    threads = O.set_threads(0)
    wide = lambda b: W.bf16_bits_to_f32(b).astype(np.float64)
    wt = LY.StackWeights([wide(w) for w, _, _ in layers], [c for _, c, _ in layers],
                         [wide(w) for _, _, w in layers], shape.H, shape.dk, shape.dv, bf16=True)
    states = [S0[l][0].astype(np.float64) for l in range(shape.layers)]
    hists = [np.zeros((3, shape.n_conv)) for _ in range(shape.layers)]
    steps, t0 = 0, time.perf_counter()
    while True:
        i = steps % len(lasts)
        x, per_layer = LY.stack_spec_step(wt, wide(x0_bits[i]), parents[i], states, hists)
        states, hists = LY.stack_commit(wt, parents[i], states, hists, per_layer, int(lasts[i]))
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    N = parents.shape[1]
    return {"value": steps * N * shape.layers / el, "unit": "nodes/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} full {shape.layers}-layer verify+commit steps of {N}-node "
                      f"trees (fp64, numpy BLAS + OpenMP C oracle) in {el:.1f} s; value counts "
                      f"nodes x layers per second like the GPU value"}


def bench_decode_loop(args):
    import torch

    from linear_attention_gdn_amd import gdnspec as G
    from linear_attention_gdn_amd.stack import GdnStack

    cfg = W.STACK_WORKLOADS[args.workload]
    shape = W.StackShape(cfg["layers"], cfg["D"], cfg["H"], cfg["dk"], cfg["dv"])
    N, L = cfg["N"], cfg["layers"]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(0)
    layers = [W.stack_layer_weights(shape, rng) for _ in range(L)]
    S0 = W.stack_states(shape, 1, rng)
    st = GdnStack(shape, B=1, N=N, device=dev)
    for l, (w_in, conv, w_o) in enumerate(layers):
        st.load_layer(l, w_in, conv, w_o, S0=S0[l])

    # per-step inputs: `chunk` distinct drafts captured in one graph
    chunk = min(args.steps, 20)  # even: the two buffer sets line up across graph replays
    slots = max(chunk, args.warmup)
    parents_np, lasts_np = W.stack_drafts(rng, slots, N=N, accept_mean=cfg["accept_mean"])
    x0_bits = np.stack([W.stack_inputs(rng, N, shape.D) for _ in range(slots)])
    xt_bits = W.stack_inputs(rng, slots, shape.D)  # one token per autoregressive step
    bfd = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(
        torch.bfloat16)
    fd = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    parents = torch.from_numpy(parents_np[:, None, :].copy()).to(dev)   # [slots][1][N]
    lasts = torch.from_numpy(lasts_np[:, None].copy()).to(dev)          # [slots][1]
    x0b = bfd(x0_bits)
    x0f = fd(W.bf16_bits_to_f32(x0_bits))
    xtb = bfd(xt_bits)
    xtf = fd(W.bf16_bits_to_f32(xt_bits))

    def spec_step(i):  # commits step i - 1's accepted path inside step i's verification
        st.set_inputs(x0f[i], x0b[i])
        j = (i - 1) % slots
        st.step(parents[i], last_prev=lasts[j], parents_prev=parents[j])

    def ar_step(i):
        st.ar_step(xtf[i:i + 1], xtb[i:i + 1])

    stream = torch.cuda.current_stream()
    st.set_inputs(x0f[slots - 1], x0b[slots - 1])
    st.verify(parents[slots - 1])  # the step before the first: its commit is pending
    for i in range(args.warmup):
        spec_step(i % slots)
        ar_step(i % slots)
    torch.cuda.synchronize()
    st.check_status()

    def timed(step_fn):
        reps, rem = divmod(args.steps, chunk)
        if args.no_graph:
            return _time_eager(step_fn, chunk, stream, reps) + _time_eager(step_fn, rem, stream)
        el = _time_graph(_graph_of(step_fn, chunk, stream), stream, reps)
        if rem:
            el += _time_graph(_graph_of(step_fn, rem, stream), stream)
        return el

    t_spec = timed(spec_step)
    t_ar = timed(ar_step)
    ms_step = t_spec * 1e3 / args.steps
    ms_tok = t_ar * 1e3 / args.steps
    depth = np.stack([W.depths_of(p) for p in parents_np])
    acc = np.array([0 if l < 0 else depth[i, l] for i, l in enumerate(lasts_np)])
    reps, rem = divmod(args.steps, chunk)
    acc_per_step = (reps * acc[:chunk].sum() + acc[:rem].sum()) / args.steps

    # per-kernel durations: each kernel alone, back-to-back in a graph,
    # rotating over the layers (the weights of 24 layers exceed the MALL)
    nper = 4 * L
    M, sh = N, shape
    npj = sh.n_proj
    PK = G.GDN_W_PACKED
    g0, g1 = st.gate_cols
    P2 = lambda l: st.P[st.cur, l].view(M, npj)
    xb3 = st.xb.view(1, N, sh.D)
    kern = {
        "linear_in": (lambda j: G.gdn_linear(st.xb, st.W_in[j % L], C=P2(j % L), w_layout=PK),
                      npj * sh.D * 2 + M * sh.D * 2 + M * npj * 4),
        "layer_prep": (lambda j: G.gdn_layer_prep(st.P[st.cur, j % L], xb3, st.W_ab[j % L],
                                                  parents[0], st.conv_w[j % L], st.hist[j % L],
                                                  st.q, st.k, st.v, st.beta, st.g), None),
        "layer_prep_delayed": (lambda j: G.gdn_layer_prep_delayed(
            st.P[st.cur, j % L], xb3, st.W_ab[j % L], parents[0], st.conv_w[j % L],
            st.hists[st.hc, j % L], st.q, st.k, st.v, st.beta, st.g, st.P[1 - st.cur, j % L],
            parents[0], lasts[0], st.hists[1 - st.hc, j % L]), None),
        "tree_verify": (lambda j: G.gdn_tree_verify(st.S[j % L], parents[0], st.q, st.k, st.v,
                                                    st.beta, st.g, st.out,
                                                    st.rec[st.cur][j % L]), None),
        "tree_verify_delayed": (lambda j: G.gdn_tree_verify_delayed(
            st.S[j % L], st.rec[st.cur][j % L], lasts[0], parents[0], st.q, st.k, st.v, st.beta,
            st.g, st.out, st.rec[1 - st.cur][j % L]), None),
        "layer_verify": (lambda j: G.gdn_layer_verify(
            st.S[j % L], parents[0], st.q, st.k, st.v, st.beta, st.g, P2(j % L)[:, g0:g1], st.Y,
            st.rec[1 - st.cur][j % L], prev_factors=st.rec[st.cur][j % L],
            last_accepted=lasts[0]), None),
        "gate_merge": (lambda j: G.gdn_gate_merge(st.out.view(M, sh.H * sh.dv),
                                                  P2(j % L)[:, g0:g1], st.Y), None),
        "linear_out": (lambda j: G.gdn_linear(st.Y, st.W_o[j % L], C=st.x, R=st.x,
                                              C_bf16=st.xb, w_layout=PK),
                       sh.D * sh.H * sh.dv * 2 + M * sh.H * sh.dv * 2 + M * sh.D * 10),
        "commit_path": (lambda j: G.gdn_commit_path(st.S[j % L], st.rec[st.cur][j % L],
                                                    lasts[0]), None),
        "conv_commit": (lambda j: G.gdn_conv_commit(st.P[st.cur, j % L], parents[0], lasts[0],
                                                    st.hist[j % L]), None),
        "linear_in_m1": (lambda j: G.gdn_linear(st.x1b, st.W_in[j % L],
                                                C=st.P1.view(1, npj), w_layout=PK),
                         npj * sh.D * 2 + sh.D * 2 + npj * 4),
        "decode_step": (lambda j: G.gdn_decode_step(
            st.S[j % L], st.q1.view(1, sh.H, sh.dk), st.k1.view(1, sh.H, sh.dk),
            st.v1.view(1, sh.H, sh.dv), st.beta1.view(1, sh.H), st.g1.view(1, sh.H), st.out1),
            2 * sh.H * sh.dv * sh.dk * 4),
    }
    kernels = {}
    for name, (fn, nbytes) in kern.items():
        if args.no_graph:
            us = _time_eager(fn, nper, stream) * 1e6 / nper
        else:
            us = _time_graph(_graph_of(fn, nper, stream), stream) * 1e6 / nper
        kernels[name] = {"avg_us": round(us, 3)}
        if nbytes:
            kernels[name]["bytes"] = int(nbytes)
            kernels[name]["gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    kd = kernels["linear_in"]
    roofline = {"bound": "hbm", "achieved": kd["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kd["gbs"] / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("gdn_linear", args.workload),
                "kernel": "gdn_linear", "algorithmic_bytes": kd["bytes"]}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = stack_cpu_baseline(shape, layers, S0, parents_np, lasts_np, x0_bits,
                                 args.cpu_seconds)
    value = N * L / (ms_step * 1e-3)
    line = {
        "metric": "verified draft nodes/sec per GDN layer (h=8,d=256)",
        "value": round(value, 1),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": L, "hidden": shape.D, "B": 1, "N": N,
                   "H": shape.H, "dk": shape.dk, "dv": shape.dv, "weights": "bf16",
                   "state_dtype": "f32", "timing": "eager" if args.no_graph else "hip_graph",
                   "parallelism": "single-gpu"},
        "decode_loop": {
            "stack_nodes_per_s": round(N / (ms_step * 1e-3), 1),
            "mean_accepted_per_step": round(float(acc_per_step), 3),
            "accepted_tokens_per_s": round(acc_per_step / (ms_step * 1e-3), 1),
            "ar_ms_per_token": round(ms_tok, 6),
            "ar_tokens_per_s": round(1e3 / ms_tok, 1),
            "speedup_accepted_vs_ar": round(acc_per_step / (ms_step * 1e-3) / (1e3 / ms_tok), 3),
        },
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
