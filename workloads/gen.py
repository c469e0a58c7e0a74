"""Seeded input generators (trees, paths, linear-attention and attention inputs).

Seeding: every tensor is drawn from its own stream,
``Generator(PCG64(SeedSequence([cfg, b, layer, tensor_id])))``, so a sequence's inputs
do not depend on the batch size it is generated in.

Shapes follow the library's layouts (row-major, innermost last):

* linear layer: q, k ``[B][N][Hk][dk]``; v ``[B][N][Hv][dv]``; g, beta ``[B][N][Hv]``;
  state ``[B][Hv][dv][dk]`` (fp32, one row of ``dk`` keys per value channel).
* attention layer: q ``[B][N][Hq][D]``; K/V cache ``[B][Hkv][Tcap][D/32 blocks]`` of
  Q8_0 (34 bytes per block) or Q4_0 (18 bytes per block) blocks.
* tree: ``parent[B][Nmax]`` int32 (``-1`` for the root and for padding rows beyond
  ``n_nodes[b]``); ``n_nodes[B]`` int32.
* accepted path: ``path[B][Lmax]`` int32 (``-1`` padding), ``path_len[B]`` int32.
* tree convolution: inputs ``x[B][N][C]`` (bf16 bits or fp32), weight ``[C][K]`` fp32,
  committed window ``state[B][K-1][C]`` fp32 (oldest first).
* acceptance: draft ``tokens[B][N]`` int32 (distinct among siblings; node 0 holds the last
  committed token) and target ``logits[B][N][V]`` (bf16 bits or fp32).

bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even from fp32).
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field

import numpy as np

# Tensor ids used in the seed tuple.
T_TREE, T_PATH, T_Q, T_K, T_V, T_G, T_BETA, T_STATE, T_AQ, T_KC, T_VC, T_LOGITS, T_DTOK, T_TLOGIT = range(14)
T_CX, T_CW, T_CSTATE = 14, 15, 16

QK8_0_BYTES = 34   # fp16 scale + 32 int8
QK4_0_BYTES = 18   # fp16 scale + 16 bytes of packed nibbles
BLOCK = 32
KV_TYPES = {"q8_0": 0, "q4_0": 1}
ROW_BYTES_PER_BLOCK = {"q8_0": QK8_0_BYTES, "q4_0": QK4_0_BYTES}


def rng_for(cfg: int, b: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, b, layer, tensor_id])))


# ----------------------------------------------------------------------------- rounding

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest-even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + (((u >> 16) & 1) + 0x7FFF)) >> 16
    return u.astype(np.uint16)


def f32_to_f16_bits(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------------------- trees

def tree_small(rng: np.random.Generator) -> np.ndarray:
    """8 nodes: a root chain 0-1-2-3 plus two 2-node branches hung off chain nodes 0..2."""
    parent = np.array([-1, 0, 1, 2, 0, 4, 0, 6], dtype=np.int32)
    parent[4] = int(rng.integers(0, 3))
    parent[6] = int(rng.integers(0, 3))
    return parent


def tree_ddtree(rng: np.random.Generator, budget: int = 22, topk: int = 4, max_depth: int = 8,
                tau: float = 6.0, vocab: int = 1024, logit_std: float = 2.0,
                chain_seed: bool = True) -> np.ndarray:
    """Best-first draft tree over seeded per-depth draft logits.

    A block-diffusion draft gives one distribution per depth that does not depend on
    the parent, so the greedy chain has the best cumulative log-probability at every
    depth.  The chain is seeded first; the remaining budget is filled best-first from
    the top-k children of every node; a candidate more than ``tau`` below the best
    cumulative log-probability at its depth is pruned.  Nodes are numbered in the order
    they are added, so ``parent[i] < i``.  Ties: higher log-prob, then shallower, then
    lower parent index, then lower top-k rank.
    """
    logits = rng.normal(0.0, logit_std, size=(max_depth, vocab))
    m = logits.max(axis=1, keepdims=True)
    lp = logits - (m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True)))
    top_lp = -np.sort(-lp, axis=1)[:, :topk]          # [depth-1][rank], descending
    best = np.concatenate([[0.0], np.cumsum(top_lp[:, 0])])

    parent, depth, cum, rank = [-1], [0], [0.0], [0]
    if chain_seed:
        while len(parent) < budget and depth[-1] < max_depth:
            d = depth[-1] + 1
            parent.append(len(parent) - 1)
            depth.append(d)
            cum.append(best[d])
            rank.append(0)
    on_chain = set(range(len(parent))) if chain_seed else {0}

    heap: list = []

    def push_children(n: int) -> None:
        d = depth[n] + 1
        if d > max_depth:
            return
        for r in range(topk):
            if chain_seed and n in on_chain and r == 0 and n + 1 < len(parent) and parent[n + 1] == n:
                continue  # the seeded chain child
            c = cum[n] + top_lp[d - 1, r]
            heapq.heappush(heap, (-c, d, n, r))

    for n in range(len(parent)):
        push_children(n)
    while heap and len(parent) < budget:
        negc, d, p, r = heapq.heappop(heap)
        c = -negc
        if c < best[d] - tau:
            continue
        parent.append(p)
        depth.append(d)
        cum.append(c)
        rank.append(r)
        push_children(len(parent) - 1)
    return np.array(parent, dtype=np.int32)


def tree_chain(n: int) -> np.ndarray:
    p = np.arange(-1, n - 1, dtype=np.int32)
    return p


def random_root_leaf_path(rng: np.random.Generator, parent: np.ndarray, n: int) -> np.ndarray:
    """Uniformly random child at each node, from the root until a leaf."""
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[int(parent[i])].append(i)
    path = [0]
    while children[path[-1]]:
        ch = children[path[-1]]
        path.append(ch[int(rng.integers(0, len(ch)))])
    return np.array(path, dtype=np.int32)


def pad_trees(parents, nmax: int | None = None):
    nmax = nmax or max(len(p) for p in parents)
    out = np.full((len(parents), nmax), -1, dtype=np.int32)
    n = np.zeros(len(parents), dtype=np.int32)
    for b, p in enumerate(parents):
        out[b, :len(p)] = p
        n[b] = len(p)
    return out, n


def pad_paths(paths, lmax: int | None = None):
    lmax = lmax or max(len(p) for p in paths)
    out = np.full((len(paths), lmax), -1, dtype=np.int32)
    ln = np.zeros(len(paths), dtype=np.int32)
    for b, p in enumerate(paths):
        out[b, :len(p)] = p
        ln[b] = len(p)
    return out, ln


# ----------------------------------------------------------------------------- quantised blocks

def quantize_q8_0(x: np.ndarray) -> np.ndarray:
    """fp32 ``[..., D]`` -> Q8_0 bytes ``[..., D/32*34]``: per block {fp16 d, int8 q[32]}."""
    x = np.asarray(x, dtype=np.float32)
    lead, D = x.shape[:-1], x.shape[-1]
    assert D % BLOCK == 0
    blk = x.reshape(*lead, D // BLOCK, BLOCK)
    amax = np.abs(blk).max(axis=-1)
    d16 = (amax / 127.0).astype(np.float16)
    d = d16.astype(np.float32)
    inv = np.divide(1.0, d, out=np.zeros_like(d), where=d > 0)
    q = np.clip(np.rint(blk * inv[..., None]), -127, 127).astype(np.int8)
    out = np.empty((*lead, D // BLOCK, QK8_0_BYTES), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(*lead, D // BLOCK, 2)
    out[..., 2:] = q.view(np.uint8)
    return out.reshape(*lead, D // BLOCK * QK8_0_BYTES)


def quantize_q4_0(x: np.ndarray) -> np.ndarray:
    """fp32 ``[..., D]`` -> Q4_0 bytes: per block {fp16 d, uint8 qs[16]}; element e<16 is the
    low nibble of qs[e], element e+16 the high nibble; value = d * (nibble - 8)."""
    x = np.asarray(x, dtype=np.float32)
    lead, D = x.shape[:-1], x.shape[-1]
    assert D % BLOCK == 0
    blk = x.reshape(*lead, D // BLOCK, BLOCK)
    idx = np.abs(blk).argmax(axis=-1)
    mx = np.take_along_axis(blk, idx[..., None], axis=-1)[..., 0]
    d16 = (mx / -8.0).astype(np.float16)
    d = d16.astype(np.float32)
    inv = np.divide(1.0, d, out=np.zeros_like(d), where=d != 0)
    nib = np.clip(np.rint(blk * inv[..., None]) + 8, 0, 15).astype(np.uint8)
    qs = nib[..., :16] | (nib[..., 16:] << 4)
    out = np.empty((*lead, D // BLOCK, QK4_0_BYTES), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(*lead, D // BLOCK, 2)
    out[..., 2:] = qs
    return out.reshape(*lead, D // BLOCK * QK4_0_BYTES)


QUANTIZERS = {"q8_0": quantize_q8_0, "q4_0": quantize_q4_0}


def row_bytes(kv_type: str, D: int) -> int:
    return D // BLOCK * ROW_BYTES_PER_BLOCK[kv_type]


# ----------------------------------------------------------------------------- layer inputs

def _unit_rows(rng, shape):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


@dataclass
class LinInputs:
    """One linear-attention layer's inputs for B sequences (see module docstring)."""
    dtype: str                 # "f32" or "bf16"
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state: np.ndarray          # fp32 [B][Hv][dv][dk]
    parent: np.ndarray
    n_nodes: np.ndarray
    path: np.ndarray
    path_len: np.ndarray
    scale: float
    Hk: int
    Hv: int
    dk: int
    dv: int


def gen_lin_seq(cfg: int, b: int, layer: int, N: int, Hk: int, Hv: int, dk: int, dv: int,
                dtype: str, state_std: float = 0.1):
    """Per-sequence draws (fp32, before any rounding)."""
    q = _unit_rows(rng_for(cfg, b, layer, T_Q), (N, Hk, dk))
    k = _unit_rows(rng_for(cfg, b, layer, T_K), (N, Hk, dk))
    v = rng_for(cfg, b, layer, T_V).standard_normal((N, Hv, dv), dtype=np.float32)
    x = rng_for(cfg, b, layer, T_G).standard_normal((N, Hv))
    g = np.exp(-np.logaddexp(0.0, x)).astype(np.float32)          # exp(-softplus(x))
    y = rng_for(cfg, b, layer, T_BETA).standard_normal((N, Hv))
    beta = (1.0 / (1.0 + np.exp(-y))).astype(np.float32)           # sigmoid(y)
    state = rng_for(cfg, b, layer, T_STATE).normal(0.0, state_std, (Hv, dv, dk)).astype(np.float32)
    return q, k, v, g, beta, state


def gen_lin(cfg: int, parents, paths, Hk: int, Hv: int, dk: int, dv: int, dtype: str,
            layer: int = 0, scale: float | None = None, seq_ids=None) -> LinInputs:
    B = len(parents)
    parent, n_nodes = pad_trees(parents)
    path, path_len = pad_paths(paths)
    Nmax = parent.shape[1]
    seq_ids = list(range(B)) if seq_ids is None else list(seq_ids)
    qs = np.zeros((B, Nmax, Hk, dk), np.float32)
    ks = np.zeros((B, Nmax, Hk, dk), np.float32)
    vs = np.zeros((B, Nmax, Hv, dv), np.float32)
    gs = np.zeros((B, Nmax, Hv), np.float32)
    bs = np.zeros((B, Nmax, Hv), np.float32)
    st = np.zeros((B, Hv, dv, dk), np.float32)
    for b in range(B):
        n = int(n_nodes[b])
        q, k, v, g, beta, s = gen_lin_seq(cfg, seq_ids[b], layer, n, Hk, Hv, dk, dv, dtype)
        qs[b, :n], ks[b, :n], vs[b, :n], gs[b, :n], bs[b, :n], st[b] = q, k, v, g, beta, s
    if dtype == "bf16":
        qs, ks, vs, gs, bs = (f32_to_bf16_bits(a) for a in (qs, ks, vs, gs, bs))
    elif dtype != "f32":
        raise ValueError(dtype)
    return LinInputs(dtype, qs, ks, vs, gs, bs, st, parent, n_nodes, path, path_len,
                     float(scale if scale is not None else 1.0 / np.sqrt(dk)), Hk, Hv, dk, dv)


@dataclass
class AttnInputs:
    q: np.ndarray              # bf16 bits [B][N][Hq][D]
    k_cache: np.ndarray        # uint8 [B][Hkv][Tcap][row_bytes]
    v_cache: np.ndarray
    k_type: str
    v_type: str
    n_past: np.ndarray         # int32 [B]
    parent: np.ndarray
    n_nodes: np.ndarray
    window: int
    scale: float
    Hq: int
    Hkv: int
    D: int
    Tcap: int


def gen_kv_head(cfg: int, b: int, layer: int, head: int, which: int, slots: int, D: int,
                kv_type: str, chunk: int = 32768) -> np.ndarray:
    """Quantised rows for one (sequence, kv-head): values N(0,1), then blocked."""
    rng = rng_for(cfg, b, layer, which * 4096 + head)
    out = np.empty((slots, row_bytes(kv_type, D)), dtype=np.uint8)
    qz = QUANTIZERS[kv_type]
    for s0 in range(0, slots, chunk):
        s1 = min(slots, s0 + chunk)
        out[s0:s1] = qz(rng.standard_normal((s1 - s0, D), dtype=np.float32))
    return out


def gen_attn(cfg: int, parents, Hq: int, Hkv: int, D: int, T, k_type: str, v_type: str,
             window: int, layer: int = 0, scale: float | None = None, seq_ids=None,
             tcap: int | None = None) -> AttnInputs:
    B = len(parents)
    parent, n_nodes = pad_trees(parents)
    Nmax = parent.shape[1]
    T = np.broadcast_to(np.asarray(T, dtype=np.int64), (B,)).astype(np.int32)
    Tcap = int(tcap if tcap is not None else int(T.max()) + Nmax)
    seq_ids = list(range(B)) if seq_ids is None else list(seq_ids)
    q = np.zeros((B, Nmax, Hq, D), np.float32)
    kc = np.zeros((B, Hkv, Tcap, row_bytes(k_type, D)), np.uint8)
    vc = np.zeros((B, Hkv, Tcap, row_bytes(v_type, D)), np.uint8)
    for b in range(B):
        n = int(n_nodes[b])
        sb = seq_ids[b]
        q[b, :n] = rng_for(cfg, sb, layer, T_AQ).standard_normal((n, Hq, D), dtype=np.float32)
        live = int(T[b]) + n
        for h in range(Hkv):
            kc[b, h, :live] = gen_kv_head(cfg, sb, layer, h, T_KC, live, D, k_type)
            vc[b, h, :live] = gen_kv_head(cfg, sb, layer, h, T_VC, live, D, v_type)
    return AttnInputs(f32_to_bf16_bits(q), kc, vc, k_type, v_type, T, parent, n_nodes, int(window),
                      float(scale if scale is not None else 1.0 / np.sqrt(D)), Hq, Hkv, D, Tcap)


# ----------------------------------------------------------------------------- named workloads

@dataclass
class Workload:
    name: str
    lin: list = field(default_factory=list)     # LinInputs per linear layer
    attn: list = field(default_factory=list)    # AttnInputs per attention layer
    order: list = field(default_factory=list)   # ("lin", i) / ("attn", i) in layer order


def trees_for(cfg: int, B: int, kind: str, seq_ids=None, **kw):
    seq_ids = list(range(B)) if seq_ids is None else list(seq_ids)
    parents, paths = [], []
    for sb in seq_ids:
        rt = rng_for(cfg, sb, 0, T_TREE)
        p = tree_small(rt) if kind == "small" else tree_ddtree(rt, **kw)
        parents.append(p)
        paths.append(random_root_leaf_path(rng_for(cfg, sb, 0, T_PATH), p, len(p)))
    return parents, paths


def workload_tiny_linear() -> Workload:
    """One linear layer, 1 head, dk=dv=16, fp32, 8-node tree, seeded root-to-leaf path."""
    parents, paths = trees_for(0, 1, "small")
    return Workload("tiny-linear-8", lin=[gen_lin(0, parents, paths, 1, 1, 16, 16, "f32")],
                    order=[("lin", 0)])


def workload_linear_27b(B: int = 1, cfg: int = 1, seq_ids=None) -> Workload:
    """One linear layer: Hk=16, Hv=48, dk=dv=128, bf16 inputs, fp32 state, 22-node trees."""
    parents, paths = trees_for(cfg, B, "ddtree", seq_ids)
    return Workload(f"linear-27b-b{B}", lin=[gen_lin(cfg, parents, paths, 16, 48, 128, 128, "bf16",
                                                     seq_ids=seq_ids)], order=[("lin", 0)])


def workload_attention_27b(B: int = 1, cfg: int = 2, T: int = 4096, window: int = 2048,
                           kv_type: str = "q8_0", seq_ids=None) -> Workload:
    """One attention layer: Hq=24, Hkv=4, D=256, bf16 Q, quantised KV, 22-node trees."""
    parents, _ = trees_for(cfg, B, "ddtree", seq_ids)
    return Workload(f"attention-27b-b{B}-t{T}-w{window}-{kv_type}",
                    attn=[gen_attn(cfg, parents, 24, 4, 256, T, kv_type, kv_type, window, seq_ids=seq_ids)],
                    order=[("attn", 0)])


def workload_batched(B: int = 64, cfg: int = 3, seq_ids=None, budget: int = 22, k_type: str = "q8_0",
                     v_type: str = "q8_0") -> Workload:
    """64 sequences, each with its own 22-node tree and accepted path, through one linear
    layer (27B widths) and one attention layer (T=4096 Q8_0, window 2048).  ``budget`` and
    the K/V types select the second workload's variants (budgets 8, 16, 40; asymmetric K/V)."""
    kw = {} if budget == 22 else {"budget": budget}
    parents, paths = trees_for(cfg, B, "ddtree", seq_ids, **kw)
    lin = gen_lin(cfg, parents, paths, 16, 48, 128, 128, "bf16", seq_ids=seq_ids)
    attn = gen_attn(cfg, parents, 24, 4, 256, 4096, k_type, v_type, 2048, seq_ids=seq_ids)
    name = f"batched-b{B}" if (budget, k_type, v_type) == (22, "q8_0", "q8_0") else \
        f"batched-b{B}-budget{budget}-{k_type}-{v_type}"
    return Workload(name, lin=[lin], attn=[attn], order=[("lin", 0), ("attn", 0)])


def workload_long_context(window: int = 0, T: int = 131072, n_lin: int = 16, n_attn: int = 4,
                          cfg: int = 4) -> Workload:
    """[4 linear, 1 attention] x 4 with a shared 22-node tree; KV in Q4_0 for K and V."""
    parents, paths = trees_for(cfg, 1, "ddtree")
    lins = [gen_lin(cfg, parents, paths, 16, 48, 128, 128, "bf16", layer=l) for l in range(n_lin)]
    attns = [gen_attn(cfg, parents, 24, 4, 256, T, "q4_0", "q4_0", window, layer=100 + a)
             for a in range(n_attn)]
    per = n_lin // n_attn if n_attn else n_lin
    order = []
    li = 0
    for a in range(n_attn):
        for _ in range(per):
            order.append(("lin", li)); li += 1
        order.append(("attn", a))
    while li < n_lin:
        order.append(("lin", li)); li += 1
    return Workload(f"long-context-t{T}-w{window}", lin=lins, attn=attns, order=order)


# ----------------------------------------------------------------------------- acceptance

@dataclass
class AcceptInputs:
    dtype: str
    logits: np.ndarray      # [B][N][V] bf16 bits (uint16) or float32
    tokens: np.ndarray      # [B][N] int32 draft tokens
    parent: np.ndarray
    n_nodes: np.ndarray
    V: int


def gen_accept(cfg: int, parents, V: int, dtype: str = "bf16", match_p: float = 0.75, tie_p: float = 0.0,
               layer: int = 0, seq_ids=None) -> AcceptInputs:
    """Draft tokens (distinct among the children of each node) and target logits ~ N(0, 1)
    with one planted maximum (8 + |N(0, 0.5)|) per node.  With probability ``match_p`` the
    planted token is a random child's draft token, so the greedy walk descends; with
    probability ``tie_p`` a second random index receives exactly the same value."""
    seq_ids = list(range(len(parents))) if seq_ids is None else list(seq_ids)
    parent, n_nodes = pad_trees(parents)
    B, N = parent.shape
    tokens = np.zeros((B, N), dtype=np.int32)
    logits = np.zeros((B, N, V), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b, sid in enumerate(seq_ids):
        n = int(n_nodes[b])
        rt = rng_for(cfg, sid, layer, T_DTOK)
        tok = rt.integers(0, V, size=N).astype(np.int64)
        kids = [[c for c in range(1, n) if int(parent[b, c]) == p] for p in range(n)]
        for ch in kids:
            seen = set()
            for c in ch:
                # distinct among siblings while the vocabulary allows it
                while int(tok[c]) in seen and len(seen) < V:
                    tok[c] = int(rt.integers(0, V))
                seen.add(int(tok[c]))
        tokens[b] = tok
        rl = rng_for(cfg, sid, layer, T_TLOGIT)
        x = rl.standard_normal((N, V), dtype=np.float32)
        for i in range(n):
            if kids[i] and rl.random() < match_p:
                t = int(tok[kids[i][int(rl.integers(0, len(kids[i])))]])
            else:
                t = int(rl.integers(0, V))
            x[i, t] = np.float32(8.0 + abs(rl.normal(0.0, 0.5)))
            if tie_p > 0 and rl.random() < tie_p:
                x[i, int(rl.integers(0, V))] = x[i, t]
        logits[b] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return AcceptInputs(dtype, logits, tokens, parent, n_nodes, V)


def workload_accept(B: int = 64, V: int = 151936, dtype: str = "bf16", cfg: int = 3, seq_ids=None,
                    tie_p: float = 0.0) -> AcceptInputs:
    """Greedy acceptance over the batched step's trees (same seeds as ``workload_batched``)."""
    parents, _ = trees_for(cfg, B, "ddtree", seq_ids=seq_ids)
    return gen_accept(cfg, parents, V, dtype, tie_p=tie_p, layer=50, seq_ids=seq_ids)


# ----------------------------------------------------------------------------- tree convolution

@dataclass
class ConvInputs:
    dtype: str
    x: np.ndarray           # [B][N][C] bf16 bits (uint16) or float32
    weight: np.ndarray      # [C][K] float32
    state: np.ndarray       # [B][K-1][C] float32, oldest first
    parent: np.ndarray
    n_nodes: np.ndarray
    path: np.ndarray
    path_len: np.ndarray
    K: int
    C: int


def gen_conv(cfg: int, parents, paths, C: int, K: int, dtype: str = "bf16", layer: int = 0,
             seq_ids=None) -> ConvInputs:
    """Inputs ~ N(0, 1) (the layer's q|k|v projections, rounded to bf16), weights ~ N(0, 1/K)
    (one set per layer, drawn from sequence 0's stream), committed window ~ N(0, 1) fp32."""
    seq_ids = list(range(len(parents))) if seq_ids is None else list(seq_ids)
    parent, n_nodes = pad_trees(parents)
    path, path_len = pad_paths(paths, lmax=parent.shape[1])
    B, N = parent.shape
    x = np.zeros((B, N, C), dtype=np.uint16 if dtype == "bf16" else np.float32)
    state = np.zeros((B, K - 1, C), dtype=np.float32)
    for b, sid in enumerate(seq_ids):
        xb = rng_for(cfg, sid, layer, T_CX).standard_normal((N, C), dtype=np.float32)
        x[b] = f32_to_bf16_bits(xb) if dtype == "bf16" else xb
        state[b] = rng_for(cfg, sid, layer, T_CSTATE).standard_normal((K - 1, C), dtype=np.float32)
    w = (rng_for(cfg, 0, layer, T_CW).standard_normal((C, K), dtype=np.float32) / np.float32(np.sqrt(K)))
    return ConvInputs(dtype, x, w.astype(np.float32), state, parent, n_nodes, path, path_len, K, C)


def workload_conv(B: int = 64, cfg: int = 3, C: int = 2 * 16 * 128 + 48 * 128, K: int = 4, dtype: str = "bf16",
                  seq_ids=None) -> ConvInputs:
    """The batched step's trees and accepted paths, at the linear layer's q|k|v width
    (2 x 16 key heads x 128 + 48 value heads x 128 = 10240 channels), window width 4."""
    parents, paths = trees_for(cfg, B, "ddtree", seq_ids=seq_ids)
    return gen_conv(cfg, parents, paths, C, K, dtype, layer=60, seq_ids=seq_ids)
