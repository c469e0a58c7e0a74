#!/usr/bin/env python3
"""Tree-verify step benchmark on one GPU.

One step takes every node of a batch of 64 draft trees (22 nodes each) through one
gated delta-rule layer -- ``lin_tree_verify_commit``: the commit of the path the same
sequences accepted in their previous step, then the verify of this step's tree, in one
pass over the state -- and one tree-masked attention layer (``attn_tree_verify``, Q8_0
cache of 4096 committed slots, window 2048).  ``linear_unfused`` times the separate
``lin_tree_verify`` and ``lin_tree_commit`` calls on the same inputs; ``linear_bank`` the
pending bank (``lin_tree_verify_bank``, a 32-entry bank per sequence: the state is written
only when the bank fills).  Widths: linear 16 key / 48 value heads
of 128, fp32 state; attention 24 query / 4 KV heads of 256.

value = node-layers per second = 2 * (tree nodes in the batch) / step time, i.e. the
harmonic mean of the linear layer's and the attention layer's nodes/s.

Inputs are seeded synthetic tensors (workloads.workload_batched); a pool of three distinct
input sets (about 2 GB) rotates between steps so the 256 MB last-level cache cannot
hold a step's working set.  Per-kernel durations come from HIP events recorded on the
stream the kernels are launched on (torch's current stream) around every call in the
timed region.

Output: one JSON line.  ``roofline`` is for the kernel with the largest mean duration;
its ``traffic`` is read from the committed hardware-counter summary under ``profiles/``
when that summary was taken on the current kernel source (else null).  ``next_kernels``
times, after the step and outside ``value``, the tree convolution and its window commit,
the greedy acceptance of the step's trees (vocabulary 151936, bf16 logits) and the
compaction of the attention cache to the accepted paths.  ``workload2`` times the step's
three calls on the second workload (budgets 8, 16 and 40 with a Q8_0 K cache and a Q4_0
V cache).  ``single_sequence`` times one
sequence through each layer on its own (the tiny layer, the 27B-width linear and attention
layers) as HIP-graph replays.  ``long_context`` times one step of a long-context model at one sequence (16
linear and 4 attention layers, 131072 committed Q4_0 slots, windows 0 and 2048); its
full-window attention is the matrix-core-bound case and also reports its fraction of the
fp16 matrix peak.  ``cpu_baseline`` times the fp64 CPU oracle over whole sequences of the same
workload for about ten seconds.

Warm-up runs at least --warmup steps and keeps going until --min-warmup-s (0.3 s) have
passed: the clock ramps up over the first ~40 ms of sustained work, and timings taken
inside the ramp read up to 15% slow.  ``warmup`` in the JSON line is the requested minimum,
``warmup_steps_run`` the number of warm-up steps actually run.  ``copy_ceiling`` is a
device-to-device copy measured on the same GPU; every kernel also reports its fraction of it.

    python bench.py [--gpus 1] [--steps 100] [--warmup 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
COUNTER_FILE = os.path.join(ROOT, "profiles", "hbm_counters_batched64.txt")
KERNEL_SOURCES = {
    "lin_tree_verify": "tree_verify_linear_amd/csrc/lin_tree.hip",
    "lin_tree_commit": "tree_verify_linear_amd/csrc/lin_tree.hip",
    "lin_tree_verify_commit": "tree_verify_linear_amd/csrc/lin_tree.hip",
    "lin_tree_verify_bank": "tree_verify_linear_amd/csrc/lin_tree.hip",
    "attn_tree_verify": "tree_verify_linear_amd/csrc/attn_tree.hip",
    "tree_accept_greedy": "tree_verify_linear_amd/csrc/accept.hip",
    "kv_tree_compact": "tree_verify_linear_amd/csrc/accept.hip",
    "conv_tree_verify": "tree_verify_linear_amd/csrc/conv_tree.hip",
    "conv_tree_commit": "tree_verify_linear_amd/csrc/conv_tree.hip",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--min-warmup-s", type=float, default=0.3,
                    help="keep running untimed warm-up steps until this many seconds have passed (the "
                         "GPU clock ramps up over the first ~40 ms of sustained work)")
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--no-workload2", action="store_true",
                    help="skip the second workload (budgets 8/16/40, Q8_0 K + Q4_0 V)")
    ap.add_argument("--no-single-sequence", action="store_true",
                    help="skip the single-sequence layer timings (tiny layer, 27B-width linear and attention layers)")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the long-context model step (131072 committed Q4_0 slots, 16 linear + 4 attention layers)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- bytes

def lin_verify_bytes(L) -> int:
    """Algorithmic HBM bytes of one lin_tree_verify call: the committed state once, the
    per-node inputs, the outputs and captured deltas (valid nodes only)."""
    B, Hv, dv, dk = L.state.shape
    Hk = L.q.shape[2]
    eb = 2 if L.dtype == "bf16" else 4
    nodes = int(L.n_nodes.sum())
    per_node = 2 * Hk * dk * eb + Hv * dv * eb + 2 * Hv * eb + 2 * Hv * dv * 4
    return B * Hv * dv * dk * 4 + nodes * per_node + L.parent.nbytes + L.n_nodes.nbytes


def lin_verify_commit_bytes(L) -> int:
    """The fused call: the verify's bytes, the committed state written once, and the previous
    step's accepted k rows, captured deltas and decays (the same sequences' previous step)."""
    B, Hv, dv, dk = L.state.shape
    Hk = L.k.shape[2]
    eb = 2 if L.dtype == "bf16" else 4
    acc = int(L.path_len.sum())
    return lin_verify_bytes(L) + B * Hv * dv * dk * 4 + acc * (Hk * dk * eb + Hv * dv * 4 + Hv * eb) + L.path.nbytes


def lin_commit_bytes(L) -> int:
    """State read + written once, plus k, captured delta and g of every accepted node."""
    B, Hv, dv, dk = L.state.shape
    Hk = L.k.shape[2]
    eb = 2 if L.dtype == "bf16" else 4
    acc = int(L.path_len.sum())
    return 2 * B * Hv * dv * dk * 4 + acc * (Hk * dk * eb + Hv * dv * 4 + Hv * eb) + L.path.nbytes


def attn_bytes(A) -> int:
    """Quantised K and V rows of the union of visible slots per (sequence, KV head), the
    bf16 queries and the fp32 outputs and log-sum-exps."""
    from workloads import row_bytes
    B, N, Hq, D = A.q.shape
    rb = row_bytes(A.k_type, D) + row_bytes(A.v_type, D)
    total = 0
    for b in range(B):
        n, T = int(A.n_nodes[b]), int(A.n_past[b])
        committed = T if A.window == 0 else min(T, A.window - 1)
        total += A.Hkv * (committed + n) * rb + n * Hq * (D * 2 + D * 4 + 4)
    return total


def accept_bytes(X) -> int:
    """Logits of every valid node read once, the tree and draft tokens, and the outputs
    (argmax per node, path, its length, the next token)."""
    B, N, V = X.logits.shape
    eb = X.logits.itemsize
    return int(X.n_nodes.sum()) * V * eb + X.parent.nbytes + X.tokens.nbytes + X.n_nodes.nbytes + 4 * (2 * B * N + 2 * B)


def compact_bytes(path, path_len, Hkv, rk, rv) -> int:
    """Each moved row (accepted node not already in place) read once and written once in
    both caches, plus the path."""
    import numpy as np
    moved = sum(int(np.count_nonzero(path[b][:path_len[b]] != np.arange(path_len[b]))) for b in range(len(path_len)))
    return moved * Hkv * (rk + rv) * 2 + path.nbytes + path_len.nbytes


def conv_verify_bytes(X) -> int:
    """Every valid node's input row read once and its output row written once, the committed
    window and the weights read once."""
    eb = X.x.itemsize
    nodes = int(X.n_nodes.sum())
    B = X.x.shape[0]
    return nodes * X.C * (eb + 4) + B * (X.K - 1) * X.C * 4 + X.C * X.K * 4 + X.parent.nbytes + X.n_nodes.nbytes


def conv_commit_bytes(X) -> int:
    """Per sequence with an accepted path: the K-1 new window rows read (from the window or
    the accepted inputs) and written."""
    eb = X.x.itemsize
    total = 0
    for L in X.path_len:
        m = min(int(L), X.K - 1)
        if L > 0:
            total += X.C * ((X.K - 1 - m) * 4 + m * eb + (X.K - 1) * 4)
    return total + X.path.nbytes + X.path_len.nbytes


def attn_flops(A) -> float:
    """2 * D flops for each of QK and PV, over each row's visible slots."""
    from workloads import row_bytes  # noqa: F401  (same module as the byte model)
    B, N, Hq, D = A.q.shape
    total = 0
    for b in range(B):
        n, T, W = int(A.n_nodes[b]), int(A.n_past[b]), A.window
        parent = A.parent[b]
        dep = [0] * n
        for i in range(1, n):
            dep[i] = dep[parent[i]] + 1
        for i in range(n):
            vis_c = T if W == 0 else max(0, min(T, W - 1 - dep[i]))
            vis_t = dep[i] + 1 if W == 0 else min(dep[i] + 1, W)
            total += Hq * (vis_c + vis_t)
    return 4.0 * D * total


# ----------------------------------------------------------------------------- helpers

def sha256_of(rel: str) -> str:
    """SHA-256 of a kernel source with // comments and blank lines removed, so that a
    comment edit does not disown counters taken on unchanged code."""
    with open(os.path.join(ROOT, rel)) as f:
        lines = [ln.split("//", 1)[0].rstrip() for ln in f]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def counter_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, if it matches the source."""
    if not os.path.exists(COUNTER_FILE):
        return None
    fields = {}
    with open(COUNTER_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    src = KERNEL_SOURCES[kernel]
    if fields.get(f"{kernel}.source_sha256") != sha256_of(src):
        return None
    try:
        return float(fields[f"{kernel}.hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


UTIL_FILE = os.path.join(ROOT, "profiles", "util_counters_batched64.txt")


def counter_util(kernel: str):
    """Matrix-core and vector-ALU utilisation of ``kernel`` from the committed counter summary
    (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES etc.), if it was taken on the current source."""
    if not os.path.exists(UTIL_FILE):
        return None
    fields = {}
    with open(UTIL_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get(f"{kernel}.source_sha256") != sha256_of(KERNEL_SOURCES[kernel]):
        return None
    out = {}
    for key in ("mfma_util", "mfma_useful_frac", "valu_busy", "mfma_valu_coexec"):
        try:
            out[key] = float(fields[f"{kernel}.{key}"])
        except (KeyError, ValueError):
            pass
    return out or None


def to_device(L, A, dev):
    import numpy as np
    import torch

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    d = dict(q=bits(L.q), k=bits(L.k), v=bits(L.v), g=bits(L.g), beta=bits(L.beta),
             state=torch.from_numpy(L.state).to(dev), parent=i32(L.parent), n_nodes=i32(L.n_nodes),
             path=i32(L.path), path_len=i32(L.path_len),
             aq=bits(A.q), kc=torch.from_numpy(A.k_cache).to(dev), vc=torch.from_numpy(A.v_cache).to(dev),
             n_past=i32(A.n_past), aparent=i32(A.parent), an_nodes=i32(A.n_nodes))
    B, N, Hv, dv = L.v.shape
    d["out"] = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=dev)
    d["cap"] = torch.empty_like(d["out"])
    d["caps"] = [d["cap"], torch.empty_like(d["out"])]      # this step's and the previous step's deltas
    Bq, Nq, Hq, D = A.q.shape
    d["aout"] = torch.empty((Bq, Nq, Hq, D), dtype=torch.float32, device=dev)
    d["lse"] = torch.empty((Bq, Nq, Hq), dtype=torch.float32, device=dev)
    return d


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=None)
    except Exception:
        return None


def cpu_baseline(L, A, budget_s: float):
    """fp64 oracle over whole sequences (verify, attention, commit) for about budget_s."""
    import numpy as np
    import oracle

    def sl(x, b):
        return x[b:b + 1]

    B = L.q.shape[0]
    nodes = 0
    seqs = 0
    w0, c0 = time.perf_counter(), time.process_time()
    for b in range(B):
        oracle.lin_tree_verify(sl(L.q, b), sl(L.k, b), sl(L.v, b), sl(L.g, b), sl(L.beta, b), sl(L.state, b),
                               sl(L.parent, b), sl(L.n_nodes, b), L.scale, L.dtype)
        oracle.lin_commit_replay(sl(L.state, b), sl(L.path, b), sl(L.path_len, b), sl(L.k, b), sl(L.v, b),
                                 sl(L.g, b), sl(L.beta, b), sl(L.parent, b), sl(L.n_nodes, b), L.dtype)
        oracle.attn_tree_verify(sl(A.q, b), sl(A.k_cache, b), sl(A.v_cache, b), A.k_type, A.v_type,
                                sl(A.n_past, b), sl(A.parent, b), sl(A.n_nodes, b), A.window, A.scale, A.Hkv)
        nodes += int(L.n_nodes[b])
        seqs += 1
        if time.perf_counter() - w0 >= budget_s:
            break
    wall = time.perf_counter() - w0
    cpu = time.process_time() - c0
    return {
        "value": 2.0 * nodes / wall,
        "unit": "node-layers/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{seqs} of {B} sequences of the batched step (linear verify + commit + attention, "
                  f"{nodes} nodes), fp64 NumPy, {wall:.1f} s wall, {cpu:.1f} s CPU",
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
        "blas_threads": _blas_threads(),
    }


def cpu_baseline_configs(long_w):
    """The same oracle on the other workloads, one call each (the long-context step from one
    of its linear and one of its attention layers): wall seconds and nodes/s per layer call."""
    import dataclasses
    import oracle
    from workloads import workload_tiny_linear, workload_linear_27b, workload_attention_27b

    def timed(fn):
        w0, c0 = time.perf_counter(), time.process_time()
        fn()
        return time.perf_counter() - w0, time.process_time() - c0

    def lin(L):
        oracle.lin_tree_verify(L.q, L.k, L.v, L.g, L.beta, L.state, L.parent, L.n_nodes, L.scale, L.dtype)
        oracle.lin_commit_replay(L.state, L.path, L.path_len, L.k, L.v, L.g, L.beta, L.parent, L.n_nodes, L.dtype)

    def attn(A, dense=False):
        f = oracle.attn_tree_verify_dense if dense else oracle.attn_tree_verify
        f(A.q, A.k_cache, A.v_cache, A.k_type, A.v_type, A.n_past, A.parent, A.n_nodes, A.window, A.scale, A.Hkv)

    res = {}
    L0 = workload_tiny_linear().lin[0]
    reps = 20
    w, c = timed(lambda: [lin(L0) for _ in range(reps)])
    res["tiny_linear"] = {"wall_s_per_call": round(w / reps, 5), "nodes_per_s": round(reps * int(L0.n_nodes.sum()) / w, 1),
                          "what": "verify + commit replay, 1 head, dk=dv=16, fp32, 8 nodes"}
    L1 = workload_linear_27b(1).lin[0]
    w, c = timed(lambda: lin(L1))
    res["linear_27b"] = {"wall_s_per_call": round(w, 4), "nodes_per_s": round(int(L1.n_nodes.sum()) / w, 1),
                         "what": "verify + commit replay, Hk16/Hv48 dk=dv=128, 22 nodes"}
    A2 = workload_attention_27b(1).attn[0]
    w, c = timed(lambda: attn(A2))
    res["attention_27b"] = {"wall_s_per_call": round(w, 4), "nodes_per_s": round(int(A2.n_nodes.sum()) / w, 1),
                            "what": "Hq24/Hkv4 D256, Q8_0, 4096 committed slots, window 2048, 22 nodes"}
    if long_w is not None:
        Ll, Al = long_w.lin[0], long_w.attn[0]
        wl, _ = timed(lambda: lin(Ll))
        out = {"linear_layer_wall_s": round(wl, 4)}
        for window in (0, 2048):
            Aw = dataclasses.replace(Al, window=window)
            wa, _ = timed(lambda: attn(Aw, dense=True))
            step = 16 * wl + 4 * wa
            out[f"window{window}"] = {"attention_layer_wall_s": round(wa, 4), "step_wall_s": round(step, 3),
                                      "node_layers_per_s": round(20 * int(Ll.n_nodes.sum()) / step, 1)}
        out["what"] = ("one 22-node step of 16 linear + 4 attention layers (131072 Q4_0 slots), from one timed "
                       "linear layer (verify + commit replay) and one attention layer (the oracle's dense masked "
                       "softmax) per window")
        res["long_context"] = out
    return res


def time_next_rows(args, tvl, torch, dev, d, A, B):
    """Greedy acceptance over the step's trees (vocabulary 151936, bf16 logits) and the
    compaction of the attention layer's cache to the accepted paths.  Timed on their own,
    after the step; they are not part of ``value``."""
    import numpy as np
    from workloads import workload_accept, row_bytes

    sets = [workload_accept(B), workload_accept(B, seq_ids=list(range(B, 2 * B)))]
    devs = []
    for X in sets:
        lg = torch.from_numpy(np.ascontiguousarray(X.logits).view(np.int16)).view(torch.bfloat16).to(dev)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
        devs.append(dict(logits=lg, parent=i32(X.parent), n_nodes=i32(X.n_nodes), tokens=i32(X.tokens)))
    N, V = sets[0].logits.shape[1], sets[0].logits.shape[2]
    ws = torch.empty(max(tvl.tree_accept_workspace_bytes(B, N, V), 256), dtype=torch.uint8, device=dev)
    outs = [torch.empty((B, N), dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev),
            torch.empty((B,), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev)]

    def accept(i):
        x = devs[i % 2]
        return tvl.tree_accept_greedy(x["logits"], x["parent"], x["n_nodes"], x["tokens"], *outs, workspace=ws)

    reps = max(args.steps, 5)
    w0 = time.perf_counter()
    i = 0
    while i < 2 or time.perf_counter() - w0 < args.min_warmup_s / 3:
        accept(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        accept(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    acc_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]

    # Compaction of the attention cache along the paths accepted by the last call above.
    path, plen = outs[1].clone(), outs[2].clone()
    torch.cuda.synchronize()
    ph, lh = path.cpu().numpy(), plen.cpu().numpy()
    rk, rv = row_bytes(A.k_type, A.D), row_bytes(A.v_type, A.D)
    # One call moves well under a megabyte, faster than Python can issue calls, so the
    # calls are captured into a HIP graph and timed as replays (reps calls per replay).
    def compact():
        tvl.kv_tree_compact(d["kc"], d["vc"], A.k_type, A.v_type, d["n_past"], path, plen)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        compact()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            compact()
    graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    cmp_ms = []
    for j in range(3):
        ev[0].record()
        graph.replay()
        ev[1].record()
        torch.cuda.synchronize()
        cmp_ms.append(ev[0].elapsed_time(ev[1]) / reps)

    def entry(ms_list, nbytes, extra):
        ms = sum(ms_list) / len(ms_list)
        gbs = nbytes / (ms * 1e-3) / 1e9
        return dict(mean_us=round(ms * 1e3, 2), median_us=round(sorted(ms_list)[len(ms_list) // 2] * 1e3, 2),
                    algorithmic_MB=round(nbytes / 1e6, 3), GB_per_s=round(gbs, 1),
                    frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4), **extra)

    # Tree convolution over the step's trees at the linear layer's q|k|v width (10240
    # channels, window width 4), then the commit of its window along the accepted paths.
    from workloads import workload_conv
    csets = [workload_conv(B), workload_conv(B, seq_ids=list(range(B, 2 * B)))]
    cdev = []
    for X in csets:
        xd = torch.from_numpy(np.ascontiguousarray(X.x).view(np.int16)).view(torch.bfloat16).to(dev)
        cdev.append(dict(x=xd, w=torch.from_numpy(X.weight).to(dev), st=torch.from_numpy(X.state).to(dev),
                         parent=i32(X.parent), n=i32(X.n_nodes), path=i32(X.path), plen=i32(X.path_len),
                         y=torch.empty((B, X.x.shape[1], X.C), dtype=torch.float32, device=dev)))

    def conv(i):
        c = cdev[i % 2]
        tvl.conv_tree_verify(c["x"], c["w"], c["st"], c["parent"], c["n"], "silu", y=c["y"])

    for i in range(4):
        conv(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        conv(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    conv_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]

    cc = cdev[0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tvl.conv_tree_commit(cc["st"], cc["x"], cc["path"], cc["plen"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    cgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cgraph):
        for _ in range(reps):
            tvl.conv_tree_commit(cc["st"], cc["x"], cc["path"], cc["plen"])
    cgraph.replay()
    torch.cuda.synchronize()
    ccommit_ms = []
    for j in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cgraph.replay()
        e1.record()
        torch.cuda.synchronize()
        ccommit_ms.append(e0.elapsed_time(e1) / reps)

    ab = sum(accept_bytes(X) for X in sets) / len(sets)
    cb = compact_bytes(ph, lh, A.Hkv, rk, rv)
    print(f"# timed acceptance and compaction ({reps} calls each)", file=sys.stderr, flush=True)
    return {
        "tree_accept_greedy": entry(acc_ms, ab, {"counter_traffic_bytes": counter_traffic("tree_accept_greedy"),
                                                 "workload": f"{B} sequences x 22-node trees, vocabulary {V}, "
                                                             "bf16 logits (argmax + walk, two launches)"}),
        "conv_tree_verify": entry(conv_ms, sum(conv_verify_bytes(X) for X in csets) / 2,
                                  {"counter_traffic_bytes": counter_traffic("conv_tree_verify"),
                                   "workload": f"{B} sequences x 22-node trees, 10240 channels, window 4, bf16 "
                                               "inputs, SiLU"}),
        "conv_tree_commit": entry(ccommit_ms, conv_commit_bytes(csets[0]),
                                  {"counter_traffic_bytes": counter_traffic("conv_tree_commit"),
                                   "workload": f"{B} sequences, 10240 channels, window 4, accepted paths; timed "
                                               f"as graph replays of {reps} calls"}),
        "kv_tree_compact": entry(cmp_ms, cb, {"counter_traffic_bytes": counter_traffic("kv_tree_compact"),
                                              "workload": f"{B} sequences, Hkv {A.Hkv}, D {A.D}, {A.k_type}/"
                                                          f"{A.v_type}, accepted paths (mean length "
                                                          f"{float(lh.mean()):.2f}); timed as graph "
                                                          f"replays of {reps} calls"}),
    }


def time_unfused_linear(args, tvl, torch, pool, sets):
    """The linear layer's separate calls (verify, then commit) on the step's inputs, for
    comparison with the fused call.  Iteration i verifies input set i and commits the set
    verified in iteration i - 1 (with that verify's deltas), so neither call finds its state
    in the last-level cache from the call just before it (the sets rotate through about 2 GB)."""
    K = max(args.steps, 10)
    n = len(pool)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        d, L = pool[i % n], sets[i % n].lin[0]
        c = pool[(i - 1) % n]
        ev[i][0].record()
        tvl.lin_tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"], d["n_nodes"],
                            L.scale, out=d["out"], cap_delta=d["cap"])
        ev[i][1].record()
        tvl.lin_tree_commit(c["state"], c["path"], c["path_len"], c["k"], c["g"], c["cap"])
        ev[i][2].record()
    torch.cuda.synchronize()
    res = {}
    for j, (nme, fn) in enumerate((("lin_tree_verify", lin_verify_bytes), ("lin_tree_commit", lin_commit_bytes))):
        ms = sum(e[j].elapsed_time(e[j + 1]) for e in ev) / K
        nb = sum(fn(W.lin[0]) for W in sets) / len(sets)
        gbs = nb / (ms * 1e-3) / 1e9
        res[nme] = {"mean_us": round(ms * 1e3, 2), "algorithmic_MB": round(nb / 1e6, 2), "GB_per_s": round(gbs, 1),
                    "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "counter_traffic_bytes": counter_traffic(nme)}
    return res


def lin_bank_entry_bytes(L) -> int:
    """HBM bytes of one pending-bank entry per sequence: its key row per key head, its
    captured delta row and decay per value head."""
    Hv, dv = L.state.shape[1], L.state.shape[2]
    Hk, dk = L.k.shape[2], L.k.shape[3]
    eb = 2 if L.dtype == "bf16" else 4
    return Hk * dk * eb + Hv * (dv * 4 + 4)


def time_bank_linear(args, tvl, torch, pool, sets, Emax: int = 32):
    """The linear layer with the pending bank (``lin_tree_verify_bank``): each step verifies
    from the stored state plus the bank plus the previous step's path, then appends that
    path to the bank, or -- for the sequences whose bank it would overflow -- stores the
    committed state and empties the bank.  The state is read every step and written once
    per bank fill.  The three input sets rotate as in the step, each with its own state and
    bank; after enough untimed steps for the banks to reach their steady cycle, K steps are
    timed.  Bytes per step follow each sequence's bank length (simulated on the host with
    the same rule)."""
    import numpy as np
    n = len(pool)
    L0 = sets[0].lin[0]
    B, Hk, dk = L0.k.shape[0], L0.k.shape[2], L0.k.shape[3]
    Hv, dv = L0.state.shape[1], L0.state.shape[2]
    eb = 2 if L0.dtype == "bf16" else 4
    banks = [tvl.lin_bank_empty(B, Hk, Hv, dk, dv, Emax, torch.bfloat16, "cuda") for _ in range(n)]
    E = [np.zeros(B, np.int64) for _ in range(n)]
    entry = lin_bank_entry_bytes(L0)
    tile = Hv * dv * dk * 4

    def one(i, ev=None):
        d, L = pool[i % n], sets[i % n].lin[0]
        v = i // n
        cap, prev_cap = d["caps"][v % 2], d["caps"][(v + 1) % 2]
        plen = d["path_len"] if v > 0 else d["zero_len"]
        if ev:
            ev[0].record()
        tvl.lin_tree_verify_bank(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"], d["n_nodes"],
                                 L.scale, d["path"], plen, d["k"], d["g"], prev_cap, banks[i % n], out=d["out"],
                                 cap_delta=cap)
        if ev:
            ev[1].record()
        # host model of the same step: bytes beyond the plain verify's
        Lp = L.path_len.astype(np.int64) if v > 0 else np.zeros(B, np.int64)
        e = E[i % n]
        flushed = Lp > Emax - e
        extra = (int(e.sum()) * entry                     # the bank's entries read
                 + int(Lp.sum()) * (Hk * dk * eb + Hv * dv * 4 + Hv * eb)   # the previous path read
                 + int(Lp[~flushed].sum()) * entry          # appended
                 + int((flushed & (e + Lp > 0)).sum()) * tile)   # committed tiles stored
        E[i % n] = np.where(flushed, 0, e + Lp)
        return extra, int(flushed.sum()), float(e.mean())

    for p in pool:
        p["zero_len"] = torch.zeros_like(p["path_len"])
    warm = n * (Emax + 2)                            # every bank past its first fill
    for i in range(warm):
        one(i)
    torch.cuda.synchronize()
    K = max(args.steps, 4 * n)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    extra, flushes, emean = 0, 0, 0.0
    for i in range(K):
        x, f, e = one(warm + i, ev[i])
        extra += x
        flushes += f
        emean += e
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    nb = sum(lin_verify_bytes(W.lin[0]) for W in sets) / n + extra / K
    nodes = sum(int(W.lin[0].n_nodes.sum()) for W in sets) / n
    gbs = nb / (ms * 1e-3) / 1e9
    return {"Emax": Emax, "steps_timed": K, "mean_us": round(ms * 1e3, 2),
            "algorithmic_MB": round(nb / 1e6, 2), "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "nodes_per_s": round(nodes / (ms * 1e-3), 1),
            "flushed_fraction": round(flushes / (K * B), 4), "bank_entries_mean": round(emean / K, 2),
            "counter_traffic_bytes": counter_traffic("lin_tree_verify_bank")}


def time_workload2(args, tvl, torch, dev, B):
    """The second workload: budgets 8 (a chain), 16 and 40, with a Q8_0 K cache and a Q4_0 V
    cache, through the same three calls as the step.  One input set per variant (each is
    larger than the 256 MB last-level cache); not part of ``value``."""
    from workloads import workload_batched
    res = {}
    for budget in (8, 16, 40):
        W = workload_batched(B, budget=budget, k_type="q8_0", v_type="q4_0")
        L, A = W.lin[0], W.attn[0]
        d = to_device(L, A, dev)
        N, Hkv, Tcap = A.q.shape[1], A.k_cache.shape[1], A.k_cache.shape[2]
        ws = torch.empty(max(tvl.attn_tree_workspace_bytes(B, N, A.Hq, Hkv, A.D, Tcap, A.window), 256),
                         dtype=torch.uint8, device=dev)
        st0 = d["state"].clone()

        def step(ev=None):
            if ev:
                ev[0].record()
            tvl.lin_tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"],
                                d["n_nodes"], L.scale, out=d["out"], cap_delta=d["cap"])
            if ev:
                ev[1].record()
            tvl.attn_tree_verify(d["aq"], d["kc"], d["vc"], A.k_type, A.v_type, d["n_past"], d["aparent"],
                                 d["an_nodes"], A.window, A.scale, out=d["aout"], lse=d["lse"], workspace=ws)
            if ev:
                ev[2].record()
            tvl.lin_tree_commit(d["state"], d["path"], d["path_len"], d["k"], d["g"], d["cap"])
            if ev:
                ev[3].record()

        w0 = time.perf_counter()
        while time.perf_counter() - w0 < 0.1:
            step()
            torch.cuda.synchronize()
        K = max(args.steps, 10)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for i in range(K):
            step(evs[i])
        torch.cuda.synchronize()
        d["state"].copy_(st0)
        names = ["lin_tree_verify", "attn_tree_verify", "lin_tree_commit"]
        byts = {"lin_tree_verify": lin_verify_bytes(L), "attn_tree_verify": attn_bytes(A),
                "lin_tree_commit": lin_commit_bytes(L)}
        ks = {}
        for j, nme in enumerate(names):
            ms = sum(e[j].elapsed_time(e[j + 1]) for e in evs) / K
            gbs = byts[nme] / (ms * 1e-3) / 1e9
            ks[nme] = {"mean_us": round(ms * 1e3, 2), "algorithmic_MB": round(byts[nme] / 1e6, 2),
                       "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        ms_step = evs[0][0].elapsed_time(evs[-1][3]) / K
        nodes = int(L.n_nodes.sum())
        res[f"budget{budget}"] = {"workload": f"{B} sequences x {budget}-node DDTree"
                                              f"{' (a chain)' if budget == 8 else ''}, linear Hk16/Hv48 "
                                              f"dk=dv=128 + commit, attention Hq24/Hkv4 D256 Q8_0 K / Q4_0 V "
                                              f"T=4096 window 2048",
                                  "ms_per_step": round(ms_step, 4),
                                  "node_layers_per_s": round(2 * nodes / (ms_step * 1e-3), 1),
                                  "kernels": ks}
        del d, ws
        print(f"# timed second workload, budget {budget}", file=sys.stderr, flush=True)
    return res


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak, vendor figure


def measure_copy_ceiling(torch, dev, mib: int = 1024, reps: int = 10):
    """A STREAM-style copy ceiling on this GPU: device-to-device copies of ``mib`` MiB (read
    once, written once), timed with events; GB/s counts both directions."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del src, dst
    best = min(ms)
    gbs = 2 * mib * (1 << 20) / (best * 1e-3) / 1e9
    return {"GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "what": f"device-to-device copy of {mib} MiB (read + write), best of {reps}"}


def graph_us(torch, fn, reps=20):
    """Median microseconds per call of ``fn`` over replays of a HIP graph holding ``reps``
    calls (one sequence's calls are latency-bound: the graph removes the launch cost)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    w0 = time.perf_counter()
    while time.perf_counter() - w0 < 0.05:
        g.replay()
        torch.cuda.synchronize()
    ts = []
    for _ in range(7):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / reps)
    return sorted(ts)[len(ts) // 2]


def time_single_sequence(args, tvl, torch, dev):
    """One sequence through each layer on its own: the tiny linear layer (1 head, dk = dv =
    16, fp32, 8 nodes), the 27B-width linear layer (22-node tree: verify, commit, and the fused
    call) and the 27B-width attention layer (Q8_0, 4096 committed slots, windows 2048 and 0).
    These calls are latency-bound (a handful of workgroups); each is timed as HIP-graph replays
    of 20 calls.  Not part of ``value``."""
    import numpy as np
    from workloads import workload_tiny_linear, workload_linear_27b, workload_attention_27b

    def t(a, bf16):
        if bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    res = {}
    for name, W in (("tiny_linear", workload_tiny_linear()), ("linear_27b", workload_linear_27b(1))):
        L = W.lin[0]
        bf = L.dtype == "bf16"
        d = dict(q=t(L.q, bf), k=t(L.k, bf), v=t(L.v, bf), g=t(L.g, bf), beta=t(L.beta, bf),
                 state=torch.from_numpy(L.state).to(dev), parent=i32(L.parent), n_nodes=i32(L.n_nodes),
                 path=i32(L.path), path_len=i32(L.path_len))
        d["out"] = torch.empty(tuple(L.v.shape), dtype=torch.float32, device=dev)
        d["cap"] = torch.empty_like(d["out"])
        d["cap2"] = torch.empty_like(d["out"])

        def verify():
            tvl.lin_tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"], d["n_nodes"],
                                L.scale, out=d["out"], cap_delta=d["cap"])

        def commit():
            tvl.lin_tree_commit(d["state"], d["path"], d["path_len"], d["k"], d["g"], d["cap"])

        def fused():
            tvl.lin_tree_verify_commit(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"],
                                       d["n_nodes"], L.scale, d["path"], d["path_len"], d["k"], d["g"], d["cap"],
                                       out=d["out"], cap_delta=d["cap2"])

        verify()
        n = int(L.n_nodes.sum())
        entry = {}
        for cname, fn in (("lin_tree_verify", verify), ("lin_tree_commit", commit), ("lin_tree_verify_commit", fused)):
            us = graph_us(torch, fn)
            entry[cname] = {"us": round(us, 2), "nodes_per_s": round(n / (us * 1e-6), 1)}
        entry["workload"] = (f"1 sequence, {n}-node tree, Hk{L.q.shape[2]}/Hv{L.v.shape[2]} dk={L.q.shape[3]} "
                             f"dv={L.v.shape[3]}, {L.dtype} inputs, fp32 state; path of {int(L.path_len[0])}")
        res[name] = entry
        del d
    for window in (2048, 0):
        W = workload_attention_27b(1, window=window)
        A = W.attn[0]
        B, N, Hq, D = A.q.shape
        Hkv, Tcap = A.k_cache.shape[1], A.k_cache.shape[2]
        x = dict(q=t(A.q, True), kc=torch.from_numpy(A.k_cache).to(dev), vc=torch.from_numpy(A.v_cache).to(dev),
                 n_past=i32(A.n_past), parent=i32(A.parent), n_nodes=i32(A.n_nodes),
                 out=torch.empty((B, N, Hq, D), dtype=torch.float32, device=dev),
                 lse=torch.empty((B, N, Hq), dtype=torch.float32, device=dev),
                 ws=torch.empty(max(tvl.attn_tree_workspace_bytes(B, N, Hq, Hkv, D, Tcap, window), 256),
                                dtype=torch.uint8, device=dev))

        def attn():
            tvl.attn_tree_verify(x["q"], x["kc"], x["vc"], A.k_type, A.v_type, x["n_past"], x["parent"],
                                 x["n_nodes"], A.window, A.scale, out=x["out"], lse=x["lse"], workspace=x["ws"])

        us = graph_us(torch, attn)
        n = int(A.n_nodes.sum())
        nb = attn_bytes(A)
        res[f"attention_27b_window{window}"] = {
            "attn_tree_verify": {"us": round(us, 2), "nodes_per_s": round(n / (us * 1e-6), 1),
                                 "algorithmic_MB": round(nb / 1e6, 3),
                                 "GB_per_s": round(nb / (us * 1e-6) / 1e9, 1)},
            "workload": f"1 sequence, {n}-node tree, Hq{Hq}/Hkv{Hkv} D{D}, {A.k_type} K and V, "
                        f"{int(A.n_past[0])} committed slots, window {window}"}
        del x
    print("# timed the single-sequence layers", file=sys.stderr, flush=True)
    return res


def time_long_context(args, tvl, torch, dev):
    """One decoding step of a long-context model at one sequence: four groups of four linear
    layers (27B widths, fused commit + verify) followed by one attention layer over 131072
    committed slots in Q4_0 (K and V), with one shared 22-node tree; full attention
    (window 0) and window 2048.  Four distinct attention layers (604 MB of cache, over twice
    the 256 MB last-level cache), so no attention layer is served from that cache at window 0.
    At window 2048 a step touches about 60 MB, so it runs cache-resident; those figures are
    latency-bound either way.  Not part of ``value``.  Returns (results, workload)."""
    import dataclasses
    import numpy as np
    from workloads import workload_long_context

    t0 = time.perf_counter()
    W = workload_long_context(window=0, n_lin=16, n_attn=4)
    print(f"# generated the long-context layers in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    lins = []
    for L in W.lin:
        d = dict(q=bits(L.q), k=bits(L.k), v=bits(L.v), g=bits(L.g), beta=bits(L.beta),
                 state=torch.from_numpy(L.state).to(dev), parent=i32(L.parent), n_nodes=i32(L.n_nodes),
                 path=i32(L.path), path_len=i32(L.path_len))
        d["out"] = torch.empty(tuple(L.v.shape), dtype=torch.float32, device=dev)
        d["caps"] = [torch.empty_like(d["out"]), torch.empty_like(d["out"])]
        lins.append(d)
    attns = []
    for A in W.attn:
        B, N, Hq, D = A.q.shape
        Hkv, Tcap = A.k_cache.shape[1], A.k_cache.shape[2]
        ws_bytes = max(max(tvl.attn_tree_workspace_bytes(B, N, Hq, Hkv, D, Tcap, w) for w in (0, 2048)), 256)
        attns.append(dict(q=bits(A.q), kc=torch.from_numpy(A.k_cache).to(dev), vc=torch.from_numpy(A.v_cache).to(dev),
                          n_past=i32(A.n_past), parent=i32(A.parent), n_nodes=i32(A.n_nodes),
                          out=torch.empty((B, N, Hq, D), dtype=torch.float32, device=dev),
                          lse=torch.empty((B, N, Hq), dtype=torch.float32, device=dev),
                          ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev)))
    order = []
    for a in range(4):
        order += [("lin", 4 * a + j) for j in range(4)] + [("attn", a)]
    # the first visit of each linear layer has no previous path: a plain verify fills its deltas
    for i, d in enumerate(lins):
        L = W.lin[i]
        tvl.lin_tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"], d["n_nodes"],
                            L.scale, out=d["out"], cap_delta=d["caps"][0])
    torch.cuda.synchronize()
    visit = [1]

    def call(kind, idx, window):
        if kind == "lin":
            d, L = lins[idx], W.lin[idx]
            v = visit[0]
            tvl.lin_tree_verify_commit(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"],
                                       d["n_nodes"], L.scale, d["path"], d["path_len"], d["k"], d["g"],
                                       d["caps"][(v + 1) % 2], out=d["out"], cap_delta=d["caps"][v % 2])
        else:
            x, A = attns[idx], W.attn[idx]
            tvl.attn_tree_verify(x["q"], x["kc"], x["vc"], A.k_type, A.v_type, x["n_past"], x["parent"],
                                 x["n_nodes"], window, A.scale, out=x["out"], lse=x["lse"], workspace=x["ws"])

    res = {"workload": "one sequence, 22-node DDTree, [4 linear layers (Hk16/Hv48 dk=dv=128, fused commit + "
                       "verify), 1 attention layer (Hq24/Hkv4 D256, K and V Q4_0, 131072 committed slots)] x 4"}
    lin_b = sum(lin_verify_commit_bytes(L) for L in W.lin) / len(W.lin)
    nodes = int(W.lin[0].n_nodes.sum())
    for window in (0, 2048):
        steps = max(args.steps, 10)
        w0 = time.perf_counter()
        while time.perf_counter() - w0 < 0.2:
            for kind, idx in order:
                call(kind, idx, window)
            visit[0] += 1
            torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)] for _ in range(steps)]
        for k in range(steps):
            evs[k][0].record()
            for j, (kind, idx) in enumerate(order):
                call(kind, idx, window)
                evs[k][j + 1].record()
            visit[0] += 1
        torch.cuda.synchronize()
        lin_ms, attn_ms = [], []
        for e in evs:
            for j, (kind, _) in enumerate(order):
                (lin_ms if kind == "lin" else attn_ms).append(e[j].elapsed_time(e[j + 1]))
        step_ms = sum(e[0].elapsed_time(e[-1]) for e in evs) / steps
        la = sum(lin_ms) / len(lin_ms)
        aa = sum(attn_ms) / len(attn_ms)
        Aw = [dataclasses.replace(A, window=window) for A in W.attn]
        ab = sum(attn_bytes(A) for A in Aw) / len(Aw)
        af = sum(attn_flops(A) for A in Aw) / len(Aw)
        a_gbs = ab / (aa * 1e-3) / 1e9
        a_tfs = af / (aa * 1e-3) / 1e12
        l_gbs = lin_b / (la * 1e-3) / 1e9
        res[f"window{window}"] = {
            "ms_per_step": round(step_ms, 4),
            "node_layers_per_s": round(20 * nodes / (step_ms * 1e-3), 1),
            "lin_tree_verify_commit": {"mean_us": round(la * 1e3, 2), "algorithmic_MB": round(lin_b / 1e6, 3),
                                       "GB_per_s": round(l_gbs, 1), "frac_hbm_peak": round(l_gbs / HBM_PEAK_GBS, 4)},
            "attn_tree_verify": {"mean_us": round(aa * 1e3, 2), "algorithmic_MB": round(ab / 1e6, 3),
                                 "GB_per_s": round(a_gbs, 1), "frac_hbm_peak": round(a_gbs / HBM_PEAK_GBS, 4),
                                 "TFLOP_per_s": round(a_tfs, 1),
                                 "frac_mfma_f16_peak": round(a_tfs / MFMA_F16_PEAK_TFLOPS, 4)},
        }
        print(f"# timed the long-context step, window {window}", file=sys.stderr, flush=True)
    del lins, attns
    return res, W


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the tree-verify kernels need no exchange between GPUs and no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import tree_verify_linear_amd as tvl
    from workloads import workload_batched

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    tvl.lib()

    B = args.batch
    t_gen = time.perf_counter()
    sets = [workload_batched(B, seq_ids=list(range(k * B, (k + 1) * B))) for k in range(3)]
    print(f"# generated {len(sets)} input sets in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    pool = [to_device(W.lin[0], W.attn[0], dev) for W in sets]
    L0, A0 = sets[0].lin[0], sets[0].attn[0]
    Hkv, Tcap = A0.k_cache.shape[1], A0.k_cache.shape[2]
    ws_bytes = max(tvl.attn_tree_workspace_bytes(B, A0.q.shape[1], A0.Hq, Hkv, A0.D, Tcap, A0.window), 256)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    names = ["lin_tree_verify_commit", "attn_tree_verify"]

    def step(i, ev=None):
        # One step per input set: the linear layer's verify, which first commits the path the
        # same sequences accepted in their previous step (fused), and the attention layer.
        d = pool[i % len(pool)]
        W = sets[i % len(sets)]
        L, A = W.lin[0], W.attn[0]
        visit = i // len(pool)
        cap, prev_cap = d["caps"][visit % 2], d["caps"][(visit + 1) % 2]
        if ev:
            ev[0].record()
        if visit == 0:
            tvl.lin_tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"], d["n_nodes"],
                                L.scale, out=d["out"], cap_delta=cap)
        else:
            tvl.lin_tree_verify_commit(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"],
                                       d["n_nodes"], L.scale, d["path"], d["path_len"], d["k"], d["g"], prev_cap,
                                       out=d["out"], cap_delta=cap)
        if ev:
            ev[1].record()
        tvl.attn_tree_verify(d["aq"], d["kc"], d["vc"], A.k_type, A.v_type, d["n_past"], d["aparent"],
                             d["an_nodes"], A.window, A.scale, out=d["aout"], lse=d["lse"], workspace=ws)
        if ev:
            ev[2].record()

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    copy_ceiling = measure_copy_ceiling(torch, dev)

    # Warm-up: at least --warmup steps, and untimed steps until --min-warmup-s have passed, so
    # the timed steps run at the clock the GPU holds under sustained load.
    w0 = time.perf_counter()
    warm = 0
    while warm < max(args.warmup, 2 * len(pool)) or time.perf_counter() - w0 < args.min_warmup_s:
        step(warm)
        warm += 1
        if warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(f"# warmup done: {warm} steps in {time.perf_counter() - w0:.2f} s", file=sys.stderr, flush=True)

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(K):
        step(warm + i, evs[i])
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - h0) * 1e3 / K
    per = {n: [] for n in names}
    for e in evs:
        for j, n in enumerate(names):
            per[n].append(e[j].elapsed_time(e[j + 1]))
    ms_step = evs[0][0].elapsed_time(evs[-1][2]) / K
    print(f"# timed {K} steps", file=sys.stderr, flush=True)

    nodes = sum(int(W.lin[0].n_nodes.sum()) for W in sets) / len(sets)
    value = 2.0 * nodes / (ms_step * 1e-3)
    byts = {
        "lin_tree_verify_commit": sum(lin_verify_commit_bytes(W.lin[0]) for W in sets) / len(sets),
        "attn_tree_verify": sum(attn_bytes(W.attn[0]) for W in sets) / len(sets),
    }
    kernels = {}
    for n in names:
        ms = sum(per[n]) / len(per[n])
        med = sorted(per[n])[len(per[n]) // 2]
        gbs = byts[n] / (ms * 1e-3) / 1e9
        kernels[n] = {"mean_us": round(ms * 1e3, 2), "median_us": round(med * 1e3, 2),
                      "algorithmic_MB": round(byts[n] / 1e6, 2), "GB_per_s": round(gbs, 1),
                      "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "nodes_per_s": round(nodes / (ms * 1e-3), 1), "counter_traffic_bytes": counter_traffic(n)}
    fl = sum(attn_flops(W.attn[0]) for W in sets) / len(sets)
    kernels["attn_tree_verify"]["TFLOP_per_s"] = round(fl / (kernels["attn_tree_verify"]["mean_us"] * 1e-6) / 1e12, 2)
    dom = max(names, key=lambda n: kernels[n]["mean_us"])
    achieved = kernels[dom]["GB_per_s"]
    roofline = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic(dom),
                "algorithmic_bytes_per_launch": int(byts[dom]),
                "frac_copy_ceiling": round(achieved / copy_ceiling["GB_per_s"], 4)}
    for n in names:
        kernels[n]["frac_copy_ceiling"] = round(kernels[n]["GB_per_s"] / copy_ceiling["GB_per_s"], 4)
    util = counter_util("attn_tree_verify")
    if util:
        kernels["attn_tree_verify"].update(util)

    unfused = None if args.no_workload2 else time_unfused_linear(args, tvl, torch, pool, sets)
    bank = None if args.no_workload2 else time_bank_linear(args, tvl, torch, pool, sets)
    next_kernels = time_next_rows(args, tvl, torch, dev, pool[0], A0, B)
    workload2 = None if args.no_workload2 else time_workload2(args, tvl, torch, dev, B)
    single = None if args.no_single_sequence else time_single_sequence(args, tvl, torch, dev)
    long_context, long_w = (None, None) if args.no_long_context else time_long_context(args, tvl, torch, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(L0, A0, args.cpu_seconds)
        cpu["per_config"] = cpu_baseline_configs(long_w)
        print("# timed the CPU oracle", file=sys.stderr, flush=True)

    line = {
        "metric": "tree-verify nodes/s per layer (22-node tree) + achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "node-layers/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "ms_per_step": round(ms_step, 4),
        "host_ms_per_step": round(host_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"batched tree verify: {B} sequences x 22-node DDTree, linear layer Hk16/Hv48 "
                               f"dk=dv=128 fp32 state + commit, attention Hq24/Hkv4 D256 Q8_0 T=4096 window 2048",
                   "global_batch": B, "tree_nodes": 22, "kv_type": "q8_0", "window": 2048, "n_past": 4096},
        "kernels": kernels,
        "linear_unfused": unfused,
        "linear_bank": bank,
        "next_kernels": next_kernels,
        "workload2": workload2,
        "single_sequence": single,
        "long_context": long_context,
        "roofline": roofline,
        "copy_ceiling": copy_ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
