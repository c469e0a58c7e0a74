// Greedy acceptance over the draft tree and KV-cache compaction (gfx950).
//
// tree_accept_greedy = two launches:
//   argmax_chunk_kernel  one workgroup per (sequence, node, chunk of the vocabulary): 256
//                        threads stream 32 KiB of logits with 16-byte loads, reduce an
//                        order-preserving integer key to the chunk maximum, and locate its
//                        first index; writes one 64-bit partial (key, index) per chunk;
//   accept_walk_kernel   one wavefront per sequence, one lane per node: folds the chunk
//                        partials into the node's argmax, then walks the tree from the root
//                        with a ballot per step (the child whose draft token matches).
// kv_tree_compact = one launch: one workgroup per (sequence, KV head) stages the accepted
// rows of both caches in LDS, then writes them to their compacted slots, so sources that
// other moves overwrite are always read first.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int ARG_THREADS = 256;
constexpr int ARG_VEC = 8;    // 16-byte loads per thread per chunk

template <bool BF16>
struct LogitFmt {
    static constexpr int kEsz = BF16 ? 2 : 4;              // bytes per logit
    static constexpr int kEpv = 16 / kEsz;                 // logits per 16-byte load
    static constexpr int kChunk = ARG_THREADS * ARG_VEC * kEpv;
    // Keys at or above this come from non-NaN values; every NaN maps below it.
    static constexpr uint32_t kNonNan = BF16 ? 0x00FFu : 0x00FFFFFFu;
    // A NaN bit pattern (two per word for bf16): padding whose key is below kNonNan.
    static constexpr uint32_t kPad = BF16 ? 0x7F817F81u : 0x7F800001u;
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// Order-preserving keys.  A float's sign-magnitude bits are turned into the two's
// complement of its magnitude (so +0 and -0 coincide and order follows value), then offset
// so that -inf lands just above every NaN:
//   non-NaN values map monotonically onto [kNonNan, max]; every NaN maps below kNonNan.
// Larger key = larger value; equal keys = equal values (floating-point equality).
__device__ __forceinline__ u16x2 keys_bf16x2(uint32_t w) {
    const u16x2 s = __builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, w) >> static_cast<short>(15));
    const u16x2 mag = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    return ((mag ^ s) - s) + static_cast<unsigned short>(0x807F);
}

__device__ __forceinline__ uint32_t key_f32(uint32_t u) {
    const uint32_t s = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);
    return ((u & 0x7FFFFFFFu) ^ s) - s + 0x807FFFFFu;
}

template <bool BF16>
__device__ __forceinline__ uint32_t key_at(const uint8_t* rowp, int e) {
    if constexpr (BF16) {
        const uint32_t h = reinterpret_cast<const uint16_t*>(rowp)[e];
        return keys_bf16x2(h).x;
    } else {
        return key_f32(reinterpret_cast<const uint32_t*>(rowp)[e]);
    }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = max(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off)));
    return x;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = min(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off)));
    return x;
}

struct ArgmaxArgs {
    int N, V, chunks;
    const uint8_t* logits;      // [B][N][V] of bf16 or f32
    const int32_t* n_nodes;     // [B]
    uint64_t* partial;          // [B][N][chunks]
};

// Partial of one chunk: (key << 32) | (0xFFFFFFFF - index), so the larger partial holds the
// larger value and, among equal values, the lower index; 0 = the chunk has no non-NaN logit.
template <bool BF16>
__global__ __launch_bounds__(ARG_THREADS) void argmax_chunk_kernel(ArgmaxArgs a) {
    using F = LogitFmt<BF16>;
    const int C = a.chunks;
    const int row = blockIdx.x / C, c = blockIdx.x % C;
    const int b = row / a.N, i = row % a.N;
    const int n = clampi(a.n_nodes[b], 1, a.N);
    if (i >= n) return;                                     // uniform over the workgroup

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t lo = static_cast<int64_t>(c) * F::kChunk;
    const int cnt = static_cast<int>(min(static_cast<int64_t>(F::kChunk), static_cast<int64_t>(a.V) - lo));
    const uint8_t* rowp = a.logits + (static_cast<size_t>(row) * a.V + lo) * F::kEsz;
    const bool vec = (reinterpret_cast<uintptr_t>(rowp) & 15) == 0;
    const int nvec = vec ? cnt / F::kEpv : 0;              // whole 16-byte loads in the chunk
    const int stail = nvec * F::kEpv;                       // first logit read one at a time

    uint4 r[ARG_VEC];
#pragma unroll
    for (int j = 0; j < ARG_VEC; ++j) {
        const int vi = j * ARG_THREADS + t;
        // the logits are read once: non-temporal loads keep them out of the caches
        r[j] = make_uint4(F::kPad, F::kPad, F::kPad, F::kPad);
        if (vi < nvec) {
            typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
            const u32v4 x = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(rowp) + vi);
            r[j] = make_uint4(x[0], x[1], x[2], x[3]);
        }
    }

    uint32_t best;
    if constexpr (BF16) {
        u16x2 acc = {0, 0};
#pragma unroll
        for (int j = 0; j < ARG_VEC; ++j) {
            acc = __builtin_elementwise_max(acc, keys_bf16x2(r[j].x));
            acc = __builtin_elementwise_max(acc, keys_bf16x2(r[j].y));
            acc = __builtin_elementwise_max(acc, keys_bf16x2(r[j].z));
            acc = __builtin_elementwise_max(acc, keys_bf16x2(r[j].w));
        }
        best = max(static_cast<uint32_t>(acc.x), static_cast<uint32_t>(acc.y));
    } else {
        best = 0;
#pragma unroll
        for (int j = 0; j < ARG_VEC; ++j)
            best = max(max(max(best, key_f32(r[j].x)), key_f32(r[j].y)), max(key_f32(r[j].z), key_f32(r[j].w)));
    }
    for (int e = stail + t; e < cnt; e += ARG_THREADS) best = max(best, key_at<BF16>(rowp, e));

    __shared__ uint32_t red_key[ARG_THREADS / 64];
    __shared__ uint32_t red_idx[ARG_THREADS / 64];
    const uint32_t wbest = wave_max_u32(best);
    if (lane == 0) red_key[wave] = wbest;
    __syncthreads();
    uint32_t M = red_key[0];
#pragma unroll
    for (int w = 1; w < ARG_THREADS / 64; ++w) M = max(M, red_key[w]);

    // Only the lanes that hold the maximum look for its first position among their logits.
    uint32_t idx = 0xFFFFFFFFu;
    if (M >= F::kNonNan && best == M) {
#pragma unroll
        for (int j = 0; j < ARG_VEC; ++j) {
            const int vi = j * ARG_THREADS + t;
            const uint32_t wd[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (BF16) {
                    const u16x2 k = keys_bf16x2(wd[q]);
                    const uint32_t e0 = static_cast<uint32_t>(vi * 8 + 2 * q);
                    if (k.y == M) idx = min(idx, e0 + 1);
                    if (k.x == M) idx = min(idx, e0);
                } else {
                    if (key_f32(wd[q]) == M) idx = min(idx, static_cast<uint32_t>(vi * 4 + q));
                }
            }
        }
        for (int e = stail + t; e < cnt; e += ARG_THREADS)
            if (key_at<BF16>(rowp, e) == M) idx = min(idx, static_cast<uint32_t>(e));
    }
    const uint32_t widx = wave_min_u32(idx);
    if (lane == 0) red_idx[wave] = widx;
    __syncthreads();
    if (t == 0) {
        uint32_t first = red_idx[0];
#pragma unroll
        for (int w = 1; w < ARG_THREADS / 64; ++w) first = min(first, red_idx[w]);
        uint64_t p = 0;
        if (M >= F::kNonNan)
            p = (static_cast<uint64_t>(M) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(lo + first));
        a.partial[static_cast<size_t>(row) * C + c] = p;
    }
}

struct WalkArgs {
    int N, chunks;
    const uint64_t* partial;
    const int32_t* parent;
    const int32_t* n_nodes;
    const int32_t* tokens;
    int32_t* target;
    int32_t* path;
    int32_t* path_len;
    int32_t* next_token;
};

__global__ __launch_bounds__(64) void accept_walk_kernel(WalkArgs a) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const int N = a.N, n = clampi(a.n_nodes[b], 1, N);
    const size_t rb = static_cast<size_t>(b) * N;

    int tgt = -1;
    if (lane < n) {
        const uint64_t* p = a.partial + (rb + lane) * a.chunks;
        uint64_t best = 0;
        for (int c = 0; c < a.chunks; ++c) best = max(best, p[c]);
        tgt = best ? static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best)) : 0;
    }
    if (lane < N) a.target[rb + lane] = tgt;

    const int par = lane < n ? a.parent[rb + lane] : -2;
    const int tok = lane < n ? a.tokens[rb + lane] : 0;
    // Each step moves to a strictly later node, so the walk ends within n steps even when
    // the parent array is malformed; on a valid tree every child already comes later.
    int cur = 0, L = 1, mine = lane == 0 ? 0 : -1;
    for (;;) {
        const int want = __shfl(tgt, cur);
        const unsigned long long m = __ballot(lane > cur && lane < n && par == cur && tok == want);
        if (m == 0) break;
        const int child = __ffsll(m) - 1;
        if (lane == L) mine = child;
        ++L;
        cur = child;
    }
    const int last_tgt = __shfl(tgt, cur);
    if (lane < N) a.path[rb + lane] = mine;
    if (lane == 0) {
        a.path_len[b] = L;
        a.next_token[b] = last_tgt;
    }
}

struct CompactArgs {
    int Hkv, Tcap, Lmax, rk, rv;    // rk, rv: bytes per (slot, head) row of each cache
    const int32_t* n_past;
    const int32_t* path;
    const int32_t* path_len;
    uint8_t* k_cache;
    uint8_t* v_cache;
};

// U = the copy unit: 16 bytes when both row sizes and bases allow it, else 2 bytes.
template <typename U>
__global__ __launch_bounds__(256) void kv_compact_kernel(CompactArgs a) {
    extern __shared__ uint4 smem_raw[];
    U* stage = reinterpret_cast<U*>(smem_raw);
    __shared__ int src_node[TV_MAX_NODES];
    const int b = blockIdx.x / a.Hkv, h = blockIdx.x % a.Hkv;
    const int64_t T = max(a.n_past[b], 0);
    const int L = clampi(a.path_len[b], 0, a.Lmax);
    const int t = threadIdx.x;
    if (t < L) {
        // A move is kept only when it changes something and both slots are in the cache.
        const int p = a.path[static_cast<size_t>(b) * a.Lmax + t];
        const bool ok = p != t && p >= 0 && T + p < a.Tcap && T + t < a.Tcap;
        src_node[t] = ok ? p : -1;
    }
    __syncthreads();

    const int uk = a.rk / static_cast<int>(sizeof(U)), uv = a.rv / static_cast<int>(sizeof(U));
    const int per = uk + uv, total = L * per;
    const size_t head_row = (static_cast<size_t>(b) * a.Hkv + h) * static_cast<size_t>(a.Tcap);
    const U* kc = reinterpret_cast<const U*>(a.k_cache);
    const U* vc = reinterpret_cast<const U*>(a.v_cache);
    for (int e = t; e < total; e += 256) {
        const int m = e / per, r = e - m * per;
        const int p = src_node[m];
        if (p < 0) continue;
        const size_t slot = head_row + static_cast<size_t>(T + p);
        stage[e] = r < uk ? kc[slot * uk + r] : vc[slot * uv + (r - uk)];
    }
    __syncthreads();
    U* kd = reinterpret_cast<U*>(a.k_cache);
    U* vd = reinterpret_cast<U*>(a.v_cache);
    for (int e = t; e < total; e += 256) {
        const int m = e / per, r = e - m * per;
        if (src_node[m] < 0) continue;
        const size_t slot = head_row + static_cast<size_t>(T + m);
        if (r < uk) kd[slot * uk + r] = stage[e];
        else vd[slot * uv + (r - uk)] = stage[e];
    }
}

// Device-side metadata check: one wave per sequence, lane = node (tree) and = path entry
// (path); every lane's findings are OR-reduced across the wave and lane 0 writes the mask.
// Every index read is clamped, so malformed metadata is reported, never dereferenced.
__global__ __launch_bounds__(64) void check_metadata_kernel(const int32_t* parent, const int32_t* n_nodes,
                                                            const int32_t* path, const int32_t* path_len, int N,
                                                            int Lmax, int32_t* status) {
    const int b = blockIdx.x, i = threadIdx.x;
    const int nraw = n_nodes[b];
    const int n = clampi(nraw, 0, N);
    int bad = 0;
    if (i == 0 && (nraw < 1 || nraw > N)) bad |= TV_BAD_N_NODES;
    const int p = i < N ? parent[static_cast<size_t>(b) * N + i] : -1;
    if (i == 0 && p != -1) bad |= TV_BAD_ROOT;
    if (i > 0 && i < n && (p < 0 || p >= i)) bad |= TV_BAD_PARENT;
    if (path) {
        const int Lraw = path_len[b];
        const int lim = Lmax < n ? Lmax : n;
        if (i == 0 && (Lraw < 0 || Lraw > lim)) bad |= TV_BAD_PATH_LEN;
        const int L = clampi(Lraw, 0, lim);
        const int a = i < Lmax ? path[static_cast<size_t>(b) * Lmax + i] : 0;
        if (i == 0 && L > 0 && a != 0) bad |= TV_BAD_PATH_ROOT;
        const int pa = __shfl(p, clampi(a, 0, 63));          // parent of this entry's node
        const int prev = __shfl(a, i > 0 ? i - 1 : 0);       // the entry before it
        if (i > 0 && i < L && (a < 0 || a >= n || pa != prev)) bad |= TV_BAD_PATH_STEP;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bad |= __shfl_xor(bad, off);
    if (i == 0) status[b] = bad;
}

}  // namespace

int accept_chunks(int V, bool bf16) {
    const int ce = bf16 ? LogitFmt<true>::kChunk : LogitFmt<false>::kChunk;
    return (V + ce - 1) / ce;
}

size_t accept_workspace_bytes(int B, int N, int V, bool bf16) {
    const size_t bytes = static_cast<size_t>(B) * N * accept_chunks(V, bf16) * sizeof(uint64_t);
    return (bytes + 255) / 256 * 256;
}

int launch_accept(const AcceptArgs& a, hipStream_t stream) {
    const int C = accept_chunks(a.V, a.bf16);
    ArgmaxArgs g{a.N, a.V, C, static_cast<const uint8_t*>(a.logits), a.n_nodes, static_cast<uint64_t*>(a.workspace)};
    const size_t wgs = static_cast<size_t>(a.B) * a.N * C;
    if (wgs > 0x7FFFFFFFu) return set_error(TV_ERANGE, "tree_accept_greedy: %zu workgroups exceed the grid limit", wgs);
    if (a.bf16)
        hipLaunchKernelGGL((argmax_chunk_kernel<true>), dim3(static_cast<unsigned>(wgs)), dim3(ARG_THREADS), 0, stream, g);
    else
        hipLaunchKernelGGL((argmax_chunk_kernel<false>), dim3(static_cast<unsigned>(wgs)), dim3(ARG_THREADS), 0, stream, g);
    WalkArgs w{a.N, C, static_cast<const uint64_t*>(a.workspace), a.parent, a.n_nodes, a.tokens,
               a.target, a.path, a.path_len, a.next_token};
    hipLaunchKernelGGL(accept_walk_kernel, dim3(static_cast<unsigned>(a.B)), dim3(64), 0, stream, w);
    return launch_status("tree_accept_greedy");
}

int launch_check_metadata(const int32_t* parent, const int32_t* n_nodes, const int32_t* path, const int32_t* path_len,
                          int B, int N, int Lmax, int32_t* status, hipStream_t stream) {
    hipLaunchKernelGGL(check_metadata_kernel, dim3(static_cast<unsigned>(B)), dim3(64), 0, stream, parent, n_nodes, path,
                       path_len, N, Lmax, status);
    return launch_status("tv_check_metadata");
}

int launch_kv_compact(const KvCompactArgs& a, hipStream_t stream) {
    CompactArgs c{a.Hkv, a.Tcap, a.Lmax, a.rk, a.rv, a.n_past, a.path, a.path_len,
                  static_cast<uint8_t*>(a.k_cache), static_cast<uint8_t*>(a.v_cache)};
    const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.Hkv));
    const size_t shmem = static_cast<size_t>(a.Lmax) * (a.rk + a.rv);
    if (a.rk % 16 == 0 && a.rv % 16 == 0)
        hipLaunchKernelGGL((kv_compact_kernel<uint4>), grid, dim3(256), shmem, stream, c);
    else
        hipLaunchKernelGGL((kv_compact_kernel<uint16_t>), grid, dim3(256), shmem, stream, c);
    return launch_status("kv_tree_compact");
}

}  // namespace tv
