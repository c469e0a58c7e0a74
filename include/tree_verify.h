/*
 * tree_verify.h -- C ABI of libtreeverify.so: the tree-verify step of a DFlash/DDTree
 * speculative decoder on AMD Instinct MI355X (gfx950).
 *
 * One verify step scores every node of a draft tree (given as parent indices) through
 * each layer of a hybrid model in one pass.  Three calls cover it:
 *
 *   lin_tree_verify   gated delta-rule (linear attention) layer: runs the recurrence along
 *                     every node's root path from the committed state and captures the
 *                     per-node factors needed to commit later;
 *   lin_tree_commit   after acceptance, moves the committed state in place to the end of
 *                     the accepted root path, using the captured factors (or, fused,
 *                     lin_tree_verify_commit applies it inside the next step's verify,
 *                     and lin_tree_verify_bank keeps several steps pending in a bank and
 *                     writes the state only when the bank fills);
 *   attn_tree_verify  full-attention layer: tree-masked softmax attention over a Q8_0 /
 *                     Q4_0 quantised KV cache with an optional sliding window.
 *
 * Two more close the loop from scores to the next step:
 *
 *   tree_accept_greedy  argmax of every node's logits and the greedy walk that picks the
 *                       accepted root path (the path the commit calls take);
 *   kv_tree_compact     moves the accepted nodes' K/V rows to the committed prefix.
 *
 * and two cover the short causal convolution in front of the linear layers:
 *
 *   conv_tree_verify    each node's convolution over its window of earlier inputs taken
 *                       along its parent chain;
 *   conv_tree_commit    moves the committed window to the end of the accepted path.
 *
 * Sources (page title, section):
 *   "Luce DFlash" server README -- "How it works" (DDTree tree verify: one forward scores
 *     the whole tree through a mask derived from parent pointers; per-step rollback of the
 *     recurrent state and KV cache to the committed prefix; tree-mode gated-delta-net
 *     kernels), "Architecture note" (Gated DeltaNet layers with a recurrent state cache;
 *     attention layers with 24 query / 4 KV heads of length 256), "Asymmetric K/V
 *     quantization" (per-side KV types, q8_0 default; unsupported pairs are refused with
 *     the list of supported ones) and the long-context table and flags (sliding-window
 *     flash attention, --fa-window N, 0 = full attention).
 *   PR #606 "perf(qwen36): add SpecLA factor-capture speculative decoding" -- "Paper
 *     mapping" (the method consumes scored candidates plus parent topology; a chain is a
 *     degenerate tree), "CLI" (options are validated up front; invalid combinations are
 *     rejected, not silently changed) and the review comment naming the commit routines
 *     (factor capture during verify, flush into the raw state on commit).
 *
 * Conventions for every call
 *   - All tensors are row-major with the innermost dimension last, laid out exactly as
 *     stated per argument.  "device" pointers are HIP device memory (or managed memory);
 *     "host" pointers are ordinary host memory.
 *   - The caller owns every buffer.  The library allocates nothing, keeps no state between
 *     calls (apart from the thread-local error message) and never synchronises: work is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream) and may run after the
 *     call returns.  The calls can therefore be captured into a HIP graph.
 *   - Return value: TV_OK, or an error code with a message readable through
 *     tv_last_error().  Errors are detected on the host, before anything is enqueued; a
 *     call that returns an error has enqueued nothing (TV_EDEVICE excepted: the launch
 *     itself failed).
 *   - Tree metadata lives in device memory and is not read back.  Kernels clamp every
 *     index taken from it (parent, n_nodes, path, path_len, n_past) into range, so a
 *     malformed tree or path can give wrong numbers but never an out-of-bounds access.
 *     Use tv_validate_tree / tv_validate_path on host copies to check them exactly, or
 *     tv_check_metadata to check them on the device without reading them back.
 *
 * Tree representation (both layer types)
 *   parent  [B][N] int32, device.  parent[b][0] = -1 (node 0 is the root: the last
 *           committed token, not yet processed); for 0 < i < n_nodes[b],
 *           0 <= parent[b][i] < i (any topological numbering).  Entries at or beyond
 *           n_nodes[b] are ignored.
 *   n_nodes [B] int32, device.  1 <= n_nodes[b] <= N; N <= 64.  Rows at or beyond
 *           n_nodes[b] of every output are left untouched.
 *   depth(0) = 0, depth(i) = depth(parent[i]) + 1.
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_ABI_VERSION 1
#define TV_MAX_NODES 64
#define TV_BANK_MAX_ENTRIES 256   /* largest pending-bank capacity (lin_tree_verify_bank) */

typedef enum {
    TV_OK = 0,
    TV_EINVAL = 1,        /* null pointer, non-positive size, window < 0, non-finite scale */
    TV_EUNSUPPORTED = 2,  /* dtype, head size or K/V type pair not built (message lists them) */
    TV_ERANGE = 3,        /* N > 64, Lmax > N, workspace too small, size overflow */
    TV_ETOPO = 4,         /* tv_validate_tree: not a rooted topological parent array */
    TV_EPATH = 5,         /* tv_validate_path: not a root path of the tree */
    TV_EDEVICE = 6        /* a kernel launch failed (message carries the HIP error) */
} tv_status;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* Which key head a value head reads (linear layer, Hv a multiple of Hk).
 * CONTIGUOUS: value head h reads key head h / (Hv / Hk)   (default)
 * TILED:      value head h reads key head h % Hk                      */
typedef enum { TV_HEADS_CONTIGUOUS = 0, TV_HEADS_TILED = 1 } tv_head_group;

/* KV cache block formats (GGUF block convention, 32 elements per block):
 * Q8_0: 34 bytes {fp16 d (little-endian); int8 q[32]}, x[e] = d * q[e].
 * Q4_0: 18 bytes {fp16 d; uint8 qs[16]}, x[e] = d * ((qs[e] & 15) - 8) for e < 16 and
 *       x[e + 16] = d * ((qs[e] >> 4) - 8).                                          */
typedef enum { TV_Q8_0 = 0, TV_Q4_0 = 1 } tv_kv_type;

/* Activation after the tree convolution. */
typedef enum { TV_ACT_NONE = 0, TV_ACT_SILU = 1 } tv_activation;

/*
 * lin_tree_verify -- one gated delta-rule layer over the draft tree.
 * ("Luce DFlash" README, "How it works" and "Architecture note"; PR #606, "Paper mapping".)
 *
 * For sequence b, value head h (key head kh per head_group) and node i with parent p, with
 * S_{-1} the committed state S0 (a dk x dv matrix mapping keys to values):
 *     u_i     = S_p^T k_i
 *     delta_i = beta_i * (v_i - g_i * u_i)
 *     S_i     = g_i * S_p + k_i delta_i^T
 *     out_i   = scale * S_i^T q_i
 * Per-node states S_i are never materialised and `state` is not modified: rolling back is
 * free.  delta_i is written to cap_delta for lin_tree_commit.
 *
 *   B, N       sequences; tree rows per sequence (1 <= N <= 64)
 *   Hk, Hv     key heads, value heads (Hv % Hk == 0)
 *   dk, dv     head sizes, each one of 16, 32, 64, 128
 *   dtype      TV_F32 or TV_BF16: element type of q, k, v, g, beta
 *   head_group tv_head_group
 *   scale      output scale (usually 1/sqrt(dk)); finite
 *   parent, n_nodes   device, see "Tree representation"
 *   q, k       device, [B][N][Hk][dk]   (already normalised by the caller)
 *   v          device, [B][N][Hv][dv]
 *   g, beta    device, [B][N][Hv]       (g: multiplicative decay in (0, 1])
 *   state      device, fp32 [B][Hv][dv][dk]: state[b][h][c][r] = S0[r][c] (one row of dk
 *              keys per value channel c).  Read only.
 *   out        device, fp32 [B][N][Hv][dv]
 *   cap_delta  device, fp32 [B][N][Hv][dv]: delta_i, consumed by lin_tree_commit
 * q, k, v, state, out and cap_delta must be 16-byte aligned (TV_EINVAL otherwise).
 */
int lin_tree_verify(int B, int N, int Hk, int Hv, int dk, int dv, int dtype, int head_group,
                    float scale, const int32_t* parent, const int32_t* n_nodes,
                    const void* q, const void* k, const void* v, const void* g, const void* beta,
                    const float* state, float* out, float* cap_delta, void* stream);

/*
 * lin_tree_commit -- move the committed state to the end of the accepted root path.
 * ("Luce DFlash" README, "How it works": after accept, the recurrent state is the
 * committed prefix; PR #606 review comment: captured factors are flushed into the raw
 * state on commit.)
 *
 * With accepted path a_0 = 0, a_1, ..., a_{L-1} (each a child of the previous) and
 * c_m = prod_{m < m' < L} g_{a_m'} (empty product = 1):
 *     S <- (prod_{m < L} g_{a_m}) * S0 + sum_m c_m * k_{a_m} delta_{a_m}^T
 * which equals replaying the recurrence over the accepted tokens alone.  path_len[b] = 0
 * leaves sequence b's state unchanged.
 *
 *   B, N, Hk, Hv, dk, dv, dtype, head_group   as for lin_tree_verify (same call's values)
 *   path       device, int32 [B][Lmax]; entries at or beyond path_len[b] are ignored
 *   path_len   device, int32 [B]; 0 <= path_len[b] <= min(Lmax, n_nodes[b])
 *   Lmax       1 <= Lmax <= N
 *   k          device, [B][N][Hk][dk] (the tensor given to lin_tree_verify)
 *   g          device, [B][N][Hv]
 *   cap_delta  device, fp32 [B][N][Hv][dv], written by lin_tree_verify
 *   state      device, fp32 [B][Hv][dv][dk], updated in place
 * state, k and cap_delta must be 16-byte aligned (TV_EINVAL otherwise).
 */
int lin_tree_commit(int B, int N, int Hk, int Hv, int dk, int dv, int dtype, int head_group,
                    const int32_t* path, const int32_t* path_len, int Lmax,
                    const void* k, const void* g, const float* cap_delta, float* state,
                    void* stream);

/*
 * attn_tree_workspace_bytes -- device workspace attn_tree_verify needs for these sizes
 * (0 if the sizes are invalid).  The workspace holds per-split partial results.
 */
size_t attn_tree_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int Tcap, int window);

/*
 * lin_tree_verify_commit -- the previous step's commit and this step's verify in one pass.
 * (PR #606 "SpecLA factor-capture speculative decoding": the captured factors are applied
 * to the state while the next verify loads it, instead of a separate pass over the state.)
 *
 * For every (sequence, value head), the state is first moved to the end of the previous
 * step's accepted path exactly as lin_tree_commit would (from that step's k, g and captured
 * deltas) and stored back into `state`; then this step's tree is verified from it exactly as
 * lin_tree_verify would.  Each state tile is read once and written once, where a separate
 * commit would read it a second time.  A sequence with prev_path_len = 0 keeps its state
 * (and it is not written).
 *
 *   B, N, Hk, Hv, dk, dv, dtype, head_group, scale, parent, n_nodes, q, k, v, g, beta, out,
 *   cap_delta             as for lin_tree_verify (this step)
 *   state                 device, fp32 [B][Hv][dv][dk], in/out: the committed state
 *   prev_N                tree rows per sequence of the previous step (1..64)
 *   prev_path, prev_path_len, prev_Lmax   the previous step's accepted paths (as for
 *                         lin_tree_commit; prev_Lmax <= prev_N)
 *   prev_k, prev_g        device, the previous step's k [B][prev_N][Hk][dk] and
 *                         g [B][prev_N][Hv], of dtype
 *   prev_cap_delta        device, fp32 [B][prev_N][Hv][dv]: the previous verify's
 *                         cap_delta.  Must not be the same buffer as cap_delta.
 * prev_k and prev_cap_delta must be 16-byte aligned in addition to lin_tree_verify's
 * arguments.
 */
int lin_tree_verify_commit(int B, int N, int Hk, int Hv, int dk, int dv, int dtype, int head_group,
                           float scale, const int32_t* parent, const int32_t* n_nodes,
                           const void* q, const void* k, const void* v, const void* g,
                           const void* beta, float* state, float* out, float* cap_delta,
                           int prev_N, const int32_t* prev_path, const int32_t* prev_path_len,
                           int prev_Lmax, const void* prev_k, const void* prev_g,
                           const float* prev_cap_delta, void* stream);

/*
 * Pending bank -- several steps' commits kept pending, flushed when the bank fills.
 * (PR #606 "SpecLA factor-capture speculative decoding": "CLI", the fused-commit option that
 * is on by default, and the review comment on the pending bank, its pending count and the
 * fused flush of the pending factors into the raw state.)
 *
 * A bank holds, per sequence, accepted entries (key, decay, captured delta) of earlier steps
 * that are not yet in the stored state, in acceptance order: E = bank_len[b] entries.  The
 * committed state is the stored state, then the bank's entries, then the accepted path of
 * the step verified last (pending until the next call, as with lin_tree_verify_commit):
 *     S = G S_stored + sum_e c_e k_e delta_e^T,  G = prod_e g_e,  c_e = prod_{e' > e} g_e'
 * over all of those entries in order -- exactly where committing each step's path in turn
 * with lin_tree_commit would have moved the state.  lin_tree_verify_bank verifies this step's
 * tree from S and then either appends the previous path to the bank, leaving `state` alone,
 * or stores S into `state` and empties the bank: when the path does not fit (E + L > Emax) or
 * a flush is asked for.  So the state is written once per bank fill instead of every step.
 * lin_bank_flush stores S without a verify (e.g. before the state is read elsewhere).
 *
 * Bank buffers (caller-owned, device; Emax a multiple of 32 in [32, TV_BANK_MAX_ENTRIES]):
 *   bank_k      [B][Hk][dk][Emax] of dtype (each key channel's entries contiguous)
 *   bank_g      fp32 [B][Hv][Emax]
 *   bank_delta  fp32 [B][Hv][dv][Emax] (each value channel's entries contiguous)
 *   bank_len    int32 [B]: E per sequence, in [0, Emax] (clamped into it); 0 for an empty
 *               bank (set it to 0 whenever `state` is replaced by the caller).
 * Entries at or beyond E are never used and need no initialisation.  The bank, the state and
 * the previous step's buffers belong together: calls that use one bank must not overlap.
 *
 * lin_tree_verify_bank -- lin_tree_verify from the committed state S above.
 *   B .. cap_delta         as for lin_tree_verify (this step); state is in/out
 *   prev_N .. prev_cap_delta   the previous step's accepted path and its k, g and captured
 *                          deltas, as for lin_tree_verify_commit (prev_path_len[b] = 0 when
 *                          nothing is pending, e.g. at the first step)
 *   Emax, bank_k, bank_g, bank_delta, bank_len   the bank (updated)
 *   flush                  0 or 1: 1 stores S and empties every sequence's bank
 * Alignment as for lin_tree_verify_commit, plus bank_k and bank_delta 16-byte, bank_g and
 * bank_len 4-byte.  Accuracy: bank keys enter exactly (bf16) or as bf16 hi + lo (fp32),
 * c_e delta_e as bf16 hi + lo, accumulated in fp32 (about 2^-16 relative per term).
 */
int lin_tree_verify_bank(int B, int N, int Hk, int Hv, int dk, int dv, int dtype, int head_group,
                         float scale, const int32_t* parent, const int32_t* n_nodes,
                         const void* q, const void* k, const void* v, const void* g,
                         const void* beta, float* state, float* out, float* cap_delta,
                         int prev_N, const int32_t* prev_path, const int32_t* prev_path_len,
                         int prev_Lmax, const void* prev_k, const void* prev_g,
                         const float* prev_cap_delta, int Emax, int flush, void* bank_k,
                         float* bank_g, float* bank_delta, int32_t* bank_len, void* stream);

/*
 * lin_bank_flush -- store the committed state S (stored state + bank + previous step's
 * path) into `state` and empty the bank.  Arguments as for lin_tree_verify_bank; no tree is
 * verified and no node input is read.
 */
int lin_bank_flush(int B, int Hk, int Hv, int dk, int dv, int dtype, int head_group, float* state,
                   int prev_N, const int32_t* prev_path, const int32_t* prev_path_len,
                   int prev_Lmax, const void* prev_k, const void* prev_g,
                   const float* prev_cap_delta, int Emax, void* bank_k, float* bank_g,
                   float* bank_delta, int32_t* bank_len, void* stream);

/*
 * attn_tree_verify -- one full-attention layer over the draft tree.
 * ("Luce DFlash" README, "How it works", "Architecture note", the FA-window flag and
 * "Asymmetric K/V quantization".)
 *
 * Sequence b has T = n_past[b] committed slots; tree node j's K/V are in slot T + j.
 * Committed slot t sits at position t and tree node j at T + depth(j).  Query node i (at
 * position T + depth(i)) attends to committed slot t iff window == 0 or
 * T + depth(i) - t < window, and to tree slot T + j iff j is on i's root path (itself
 * included) and (window == 0 or depth(i) - depth(j) < window).  Query head h reads KV
 * head h / (Hq / Hkv).
 *     out[b][i][h] = sum_t softmax_t(scale * <q, K_t>) V_t        lse = log sum_t exp(...)
 *
 *   B, N       sequences; tree rows per sequence (1 <= N <= 64)
 *   Hq, Hkv    query heads, KV heads (Hq % Hkv == 0, Hq / Hkv <= 8)
 *   D          head size: 256
 *   Tcap       slots per (sequence, KV head) row of the cache; n_past[b] + n_nodes[b] <= Tcap
 *   k_type, v_type   tv_kv_type of each cache ({Q8_0, Q4_0} x {Q8_0, Q4_0})
 *   window     0 = full attention, else the window W > 0
 *   scale      score scale (usually 1/sqrt(D)); finite
 *   parent, n_nodes  device, see "Tree representation"
 *   n_past     device, int32 [B]
 *   q          device, bf16 [B][N][Hq][D], any finite values (each row is rescaled by a power
 *              of two before entering the matrix cores, so its range is not limited to fp16's);
 *              the scores scale * <q, k> must stay within fp32 range
 *   k_cache    device, bytes [B][Hkv][Tcap][D/32 blocks of k_type]
 *   v_cache    device, bytes [B][Hkv][Tcap][D/32 blocks of v_type]
 *   out        device, fp32 [B][N][Hq][D], 16-byte aligned
 *   lse        device, fp32 [B][N][Hq] (natural log) or NULL
 *   workspace  device, >= attn_tree_workspace_bytes(...) bytes, 256-byte aligned; its
 *              contents need no initialisation and are garbage afterwards
 */
int attn_tree_verify(int B, int N, int Hq, int Hkv, int D, int Tcap, int k_type, int v_type,
                     int window, float scale, const int32_t* parent, const int32_t* n_nodes,
                     const int32_t* n_past, const void* q, const void* k_cache,
                     const void* v_cache, float* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * attn_tree_verify_noalloc -- attn_tree_verify for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as attn_tree_verify, without the workspace:
 * the split partials go to a scratch array the library holds on each device for the life of
 * the process (64 MiB, reserved when the library's code is first loaded on a device).  The
 * call allocates nothing.
 *   - Sizes whose partials need more than the scratch (attn_tree_workspace_bytes(...) above
 *     64 MiB) are rejected with TV_ERANGE before anything is enqueued.
 *   - Every call on a device shares that device's scratch, so calls that can overlap on one
 *     GPU (different streams, or different threads without ordering) race: serialise them.
 *     Nothing in the scratch needs to start at zero; its contents are garbage afterwards.
 */
int attn_tree_verify_noalloc(int B, int N, int Hq, int Hkv, int D, int Tcap, int k_type, int v_type,
                             int window, float scale, const int32_t* parent, const int32_t* n_nodes,
                             const int32_t* n_past, const void* q, const void* k_cache,
                             const void* v_cache, float* out, float* lse, void* stream);

/* Bytes of workspace tree_accept_greedy needs (0 for invalid sizes or dtype). */
size_t tree_accept_workspace_bytes(int B, int N, int V, int dtype);

/*
 * tree_accept_greedy -- greedy acceptance of the draft tree from the target's logits.
 * ("Luce DFlash" README, "How it works": one forward scores the whole tree, then the
 * committed prefix is advanced to the accepted path; "Scope and limits": verification is
 * argmax, and temperature 0 keeps the committed tokens exactly the greedy ones.)
 *
 *   target[b][i] = argmax_v logits[b][i][v] for i < n_nodes[b]: the lowest index holding
 *                  the largest value, NaN entries never selected, 0 for a row that is all
 *                  NaN; -1 for n_nodes[b] <= i < N.  +0 and -0 compare equal.
 *   The walk starts at the root (node 0, always accepted).  From accepted node p the next
 *   accepted node is the lowest-index child c of p (parent[c] == p, c < n_nodes[b]) whose
 *   draft token tokens[b][c] equals target[b][p]; it stops when no child matches.
 *   path[b][m]     the m-th accepted node, root first, -1 for m >= path_len[b] (m < N)
 *   path_len[b]    accepted nodes, root included (1 <= path_len[b] <= n_nodes[b])
 *   next_token[b]  target[b][last accepted node]: the token committed after the accepted
 *                  draft tokens.
 *
 *   B, N       sequences; tree rows per sequence (1 <= N <= 64)
 *   V          vocabulary size (logits per row)
 *   dtype      TV_BF16 or TV_F32: the logits' element type
 *   logits     device, [B][N][V] of dtype, 16-byte aligned; rows beyond n_nodes are not read
 *   parent, n_nodes  device, see "Tree representation" (n_nodes is clamped into [1, N])
 *   tokens     device, int32 [B][N]: draft token of each node (the root's is ignored)
 *   target     device, int32 [B][N]          path  device, int32 [B][N]
 *   path_len, next_token   device, int32 [B]
 *   workspace  device, >= tree_accept_workspace_bytes(B, N, V, dtype) bytes, 256-byte
 *              aligned; needs no initialisation, garbage afterwards
 * The outputs feed lin_tree_commit (path, path_len, Lmax = N) and kv_tree_compact.
 */
int tree_accept_greedy(int B, int N, int V, int dtype, const void* logits,
                       const int32_t* parent, const int32_t* n_nodes, const int32_t* tokens,
                       int32_t* target, int32_t* path, int32_t* path_len,
                       int32_t* next_token, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * kv_tree_compact -- moves the accepted tree nodes' K/V rows to the committed prefix.
 * ("Luce DFlash" README, "How it works": after acceptance the KV cache is restored to the
 * committed prefix, which then ends with the accepted path.)
 *
 * For each sequence b with T = n_past[b] and m < path_len[b]: the row of every KV head at
 * slot T + path[b][m] (where verify stored node path[b][m]) is copied byte for byte to slot
 * T + m, in both caches.  All sources are read before any destination is written, so the
 * result does not depend on the order of the moves.  Every other slot keeps its bytes.
 * Moves whose source or destination slot falls outside [0, Tcap), or whose node index is
 * negative, are skipped; path_len is clamped into [0, Lmax].  The caller advances n_past
 * by path_len afterwards.
 *
 *   B, Hkv, D, Tcap, k_type, v_type   as for attn_tree_verify; D a multiple of 32, <= 512
 *   n_past     device, int32 [B]
 *   path       device, int32 [B][Lmax] (as written by tree_accept_greedy with Lmax = N)
 *   path_len   device, int32 [B]
 *   Lmax       row stride of path, 1 <= Lmax <= 64
 *   k_cache, v_cache   device, in/out, 16-byte aligned, layouts as for attn_tree_verify
 */
int kv_tree_compact(int B, int Hkv, int D, int Tcap, int k_type, int v_type,
                    const int32_t* n_past, const int32_t* path, const int32_t* path_len,
                    int Lmax, void* k_cache, void* v_cache, void* stream);

/*
 * conv_tree_verify -- causal depthwise convolution of width K over the draft tree.
 * ("Luce DFlash" README, "How it works": the recurrent state rolled back after acceptance
 * includes the convolution window, and the tree-aware convolution gathers each node's
 * window of earlier inputs along its parent chain, not in node order.)
 *
 * For sequence b, node i < n_nodes[b] and channel c:
 *     y[b][i][c] = act( sum_{k<K} weight[c][k] * u_k )
 * where u_{K-1} = x[b][i][c], u_{K-2} = x[b][parent(i)][c], ... up the root path, and
 * positions above the root come from the committed window: the j-th step above the root
 * reads conv_state[b][K-1-j][c] (oldest first, so conv_state[b][K-2] is the most recent
 * committed input).  On a chain this is ordinary causal 1-D convolution with the window
 * as left context.  act is the identity or SiLU (v * sigmoid(v)).
 *
 *   B, N       sequences; tree rows per sequence (1 <= N <= 64)
 *   C          channels, a multiple of 8 (the linear layer's q|k|v projections)
 *   K          convolution width, 2..8 (a model parameter)
 *   dtype      TV_F32 or TV_BF16: element type of x
 *   activation tv_activation
 *   parent, n_nodes   device, see "Tree representation"
 *   x          device, [B][N][C] of dtype
 *   weight     device, fp32 [C][K]; weight[c][K-1] multiplies the node's own input
 *   conv_state device, fp32 [B][K-1][C], read only
 *   y          device, fp32 [B][N][C]
 * x, weight, conv_state and y must be 16-byte aligned.
 */
int conv_tree_verify(int B, int N, int C, int K, int dtype, int activation,
                     const int32_t* parent, const int32_t* n_nodes, const void* x,
                     const float* weight, const float* conv_state, float* y, void* stream);

/*
 * conv_tree_commit -- moves the committed window to the end of the accepted path, in place.
 * ("Luce DFlash" README, "How it works": after accept the window is restored to the
 * committed prefix, which now ends with the accepted path.)
 *
 * With L = path_len[b] (clamped into [0, Lmax]) and the accepted inputs x[b][path[b][m]],
 * the new window is the last K-1 entries of (conv_state[b][0..K-2], accepted inputs in path
 * order).  L = 0 leaves it unchanged.  Path entries are clamped into [0, N-1].
 *
 *   B, N, C, K, dtype   as for conv_tree_verify
 *   path, path_len      device, int32 [B][Lmax] and [B] (as for lin_tree_commit)
 *   Lmax                row stride of path, 1 <= Lmax <= N
 *   x                   device, [B][N][C] of dtype (the inputs the verify call saw)
 *   conv_state          device, fp32 [B][K-1][C], in/out
 */
int conv_tree_commit(int B, int N, int C, int K, int dtype, const int32_t* path,
                     const int32_t* path_len, int Lmax, const void* x, float* conv_state,
                     void* stream);

/* Device-side check of the same metadata, for metadata that never leaves the device
 * (PR #606 "CLI": inputs are validated, invalid ones reported rather than silently used).
 * Enqueues one small kernel on `stream` and reads nothing back: status[b] (device int32
 * [B]) receives a bit mask per sequence, 0 when the sequence passes every check that
 * tv_validate_tree / tv_validate_path make.  path and path_len may both be NULL: then only
 * the tree is checked and Lmax is ignored (else 1 <= Lmax <= N).  Each bit is judged on its
 * own, with n_nodes[b] clamped to [0, N].  Every index read is clamped, so any metadata is
 * safe to check.  B >= 1, 1 <= N <= 64. */
#define TV_BAD_N_NODES   1   /* n_nodes[b] not in [1, N] */
#define TV_BAD_ROOT      2   /* parent[b][0] != -1 */
#define TV_BAD_PARENT    4   /* some parent[b][i], 0 < i < n_nodes[b], not in [0, i) */
#define TV_BAD_PATH_LEN  8   /* path_len[b] not in [0, min(Lmax, n_nodes[b])] */
#define TV_BAD_PATH_ROOT 16  /* path_len[b] > 0 and path[b][0] != 0 */
#define TV_BAD_PATH_STEP 32  /* some path[b][m], 0 < m < path_len[b], is not a child of path[b][m-1] */
int tv_check_metadata(const int32_t* parent, const int32_t* n_nodes, const int32_t* path,
                      const int32_t* path_len, int B, int N, int Lmax, int32_t* status,
                      void* stream);

/* Host-side checks of tree metadata (host pointers).  TV_OK or TV_ETOPO / TV_EPATH /
 * TV_EINVAL / TV_ERANGE with a message naming the first offending entry. */
int tv_validate_tree(const int32_t* parent, const int32_t* n_nodes, int B, int N);
int tv_validate_path(const int32_t* parent, const int32_t* n_nodes, const int32_t* path,
                     const int32_t* path_len, int B, int N, int Lmax);

/* Message of the last error on the calling thread ("" if none).  Valid until the next
 * call from the same thread. */
const char* tv_last_error(void);
int tv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TREE_VERIFY_H */
