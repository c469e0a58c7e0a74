// Tree-aware causal short convolution and its window commit (gfx950).
//
// ("Luce DFlash" README, "How it works": the rolled-back recurrent state includes the
// convolution window, and the tree-aware convolution gathers each node's window of earlier
// inputs along its parent chain in the draft tree rather than in node order.)
//
//   y_i[c] = sum_{k<K} w[c][k] * u_{i,k}[c],  u_{i,K-1} = x_i, u_{i,K-2} = x_parent(i), ...,
//   above the root the committed window (oldest first); optionally SiLU.
//
// Both kernels are bandwidth work: one thread handles 8 channels, four at 4t .. 4t+3 and four
// at 1024 + 4t .. 1024 + 4t + 3 of its workgroup's 2048, so every load and store instruction
// of a wave covers one contiguous run of memory (whole 128-byte lines of the fp32 outputs).
// The weights of those channels stay in registers, and every input row a node's window needs
// is read with coalesced vector loads (a parent's row is usually still in L2 from the
// parent's own thread).
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int CPT = 8;                 // channels per thread
constexpr int CONV_THREADS = 256;      // 2048 channels per workgroup
constexpr int NPW = 8;                 // nodes per workgroup (each thread walks all of them)

struct ConvArgs {
    int B, N, C, K, silu, Lmax;
    const int32_t* parent;
    const int32_t* n_nodes;
    const void* x;
    const float* weight;
    const float* state;
    float* y;
    float* state_rw;
    const int32_t* path;
    const int32_t* path_len;
};

constexpr int HALF = CONV_THREADS * CPT / 2;    // offset of a thread's second four channels

// A thread's channels: c0 .. c0+3 and c0+HALF .. c0+HALF+3 (c0 = chunk base + 4t), present
// as whole halves (C is a multiple of 8).  Absent halves read as zero and are not stored.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t elem, bool okb, float (&u)[CPT]) {
    if constexpr (BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(base) + elem;
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        uint2 b = make_uint2(0u, 0u);
        if (okb) b = *reinterpret_cast<const uint2*>(p + HALF);
        const uint32_t w[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[2 * e] = __uint_as_float(w[e] << 16);
            u[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
        const float* p = static_cast<const float*>(base) + elem;
        const float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
        if (okb) b = *reinterpret_cast<const float4*>(p + HALF);
        u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w;
        u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
    }
}

__device__ __forceinline__ void load8f(const float* p, bool okb, float (&u)[CPT]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (okb) b = *reinterpret_cast<const float4*>(p + HALF);
    u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w;
    u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
}

__device__ __forceinline__ void store8f(float* p, bool okb, const float (&u)[CPT]) {
    *reinterpret_cast<float4*>(p) = make_float4(u[0], u[1], u[2], u[3]);
    if (okb) *reinterpret_cast<float4*>(p + HALF) = make_float4(u[4], u[5], u[6], u[7]);
}

// The same for outputs that are written once and read by a later call: streamed past the
// caches (a wave's store covers whole lines).
__device__ __forceinline__ void store8f_stream(float* p, bool okb, const float (&u)[CPT]) {
    typedef float f32v4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f32v4{u[0], u[1], u[2], u[3]}, reinterpret_cast<f32v4*>(p));
    if (okb) __builtin_nontemporal_store(f32v4{u[4], u[5], u[6], u[7]}, reinterpret_cast<f32v4*>(p + HALF));
}

// SiLU with the hardware exp2 and reciprocal (each about 1 ulp).
__device__ __forceinline__ float silu(float v) {
    return v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v));
}

// Work unit: (sequence, group of 8 nodes, 2048 channels); thread = 8 channels, all 8 nodes,
// so each thread loads its weights once.
template <int K, bool BF16>
__global__ __launch_bounds__(CONV_THREADS) void conv_tree_kernel(ConvArgs a) {
    __shared__ int par[TV_MAX_NODES];
    const int chunks = (a.C + CONV_THREADS * CPT - 1) / (CONV_THREADS * CPT);
    const int nblocks = (a.N + NPW - 1) / NPW;
    int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int chunk = wg % chunks;
    wg /= chunks;
    const int nb = wg % nblocks;
    const int b = wg / nblocks;
    const int n = clampi(a.n_nodes[b], 0, a.N);
    const int t = threadIdx.x;
    // parents clamped to an earlier node, so every walk moves toward the root
    if (t < n) par[t] = t == 0 ? -1 : clampi(a.parent[static_cast<size_t>(b) * a.N + t], 0, t - 1);
    __syncthreads();
    const int c0 = chunk * CONV_THREADS * CPT + 4 * t;
    const bool okb = c0 + HALF < a.C;
    const int i0 = nb * NPW;
    if (c0 >= a.C || i0 >= n) return;

    float w[CPT][K];
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        const int ch = e < 4 ? c0 + e : (okb ? c0 + HALF + e - 4 : c0);
#pragma unroll
        for (int k = 0; k < K; ++k) w[e][k] = a.weight[static_cast<size_t>(ch) * K + k];
    }

    const size_t xrow = static_cast<size_t>(b) * a.N;
    const float* win = a.state + static_cast<size_t>(b) * (K - 1) * a.C + c0;
    // Nodes past the tree are computed on node 0's rows and not stored: the loop stays
    // branch-free, so the loads of all its nodes can be in flight together.
#pragma unroll
    for (int q = 0; q < NPW; ++q) {
        const int i = i0 + q < n ? i0 + q : 0;
        float acc[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) acc[e] = 0.f;
        int node = i, above = 0;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
            float u[CPT];
            if (node >= 0) {
                load8<BF16>(a.x, (xrow + node) * a.C + c0, okb, u);
                node = node > 0 ? par[node] : -1;
            } else {
                ++above;
                load8f(win + static_cast<size_t>(K - 1 - above) * a.C, okb, u);
            }
#pragma unroll
            for (int e = 0; e < CPT; ++e) acc[e] = __builtin_fmaf(w[e][k], u[e], acc[e]);
        }
        if (a.silu) {
#pragma unroll
            for (int e = 0; e < CPT; ++e) acc[e] = silu(acc[e]);
        }
        if (i0 + q < n) store8f_stream(a.y + (xrow + i) * a.C + c0, okb, acc);
    }
}

// Work unit: (sequence, 2048 channels); thread = 8 channels of the sequence's window.  All K-1
// new rows are read before any is written, so the in-place shift is safe.
template <int K, bool BF16>
__global__ __launch_bounds__(CONV_THREADS) void conv_commit_kernel(ConvArgs a) {
    const int chunks = (a.C + CONV_THREADS * CPT - 1) / (CONV_THREADS * CPT);
    const int wg = blockIdx.x;
    const int b = wg / chunks;
    const int c0 = (wg % chunks) * CONV_THREADS * CPT + 4 * static_cast<int>(threadIdx.x);
    const bool okb = c0 + HALF < a.C;
    const int L = clampi(a.path_len[b], 0, a.Lmax);
    if (c0 >= a.C || L == 0) return;
    float* st = a.state_rw + static_cast<size_t>(b) * (K - 1) * a.C + c0;
    float rows[K - 1][CPT];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        const int s = j + L;          // position in (committed window, accepted inputs)
        if (s < K - 1) {
            load8f(st + static_cast<size_t>(s) * a.C, okb, rows[j]);
        } else {
            const int node = clampi(a.path[static_cast<size_t>(b) * a.Lmax + (s - (K - 1))], 0, a.N - 1);
            load8<BF16>(a.x, (static_cast<size_t>(b) * a.N + node) * a.C + c0, okb, rows[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < K - 1; ++j) store8f(st + static_cast<size_t>(j) * a.C, okb, rows[j]);
}

template <bool BF16>
void launch_conv_k(const ConvArgs& a, bool commit, dim3 grid, hipStream_t stream) {
#define TV_CONV_CASE(KK)                                                                                  \
    case KK:                                                                                              \
        if (commit) hipLaunchKernelGGL((conv_commit_kernel<KK, BF16>), grid, dim3(CONV_THREADS), 0, stream, a); \
        else hipLaunchKernelGGL((conv_tree_kernel<KK, BF16>), grid, dim3(CONV_THREADS), 0, stream, a);     \
        break;
    switch (a.K) {
        TV_CONV_CASE(2)
        TV_CONV_CASE(3)
        TV_CONV_CASE(4)
        TV_CONV_CASE(5)
        TV_CONV_CASE(6)
        TV_CONV_CASE(7)
        TV_CONV_CASE(8)
        default: break;
    }
#undef TV_CONV_CASE
}

}  // namespace

int launch_conv_verify(const ConvVerifyArgs& v, hipStream_t stream) {
    ConvArgs a{v.B, v.N, v.C, v.K, v.silu, 0, v.parent, v.n_nodes, v.x, v.weight, v.state, v.y,
               nullptr, nullptr, nullptr};
    const long long chunks = (v.C + CONV_THREADS * CPT - 1) / (CONV_THREADS * CPT);
    const long long wgs = static_cast<long long>(v.B) * ((v.N + NPW - 1) / NPW) * chunks;
    if (wgs > 0x7fffffffLL) return set_error(TV_ERANGE, "conv_tree_verify: too many work units");
    if (v.bf16) launch_conv_k<true>(a, false, dim3(static_cast<unsigned>(wgs)), stream);
    else launch_conv_k<false>(a, false, dim3(static_cast<unsigned>(wgs)), stream);
    return launch_status("conv_tree_verify");
}

int launch_conv_commit(const ConvCommitArgs& c, hipStream_t stream) {
    ConvArgs a{c.B, c.N, c.C, c.K, 0, c.Lmax, nullptr, nullptr, c.x, nullptr, nullptr, nullptr,
               c.state, c.path, c.path_len};
    const long long chunks = (c.C + CONV_THREADS * CPT - 1) / (CONV_THREADS * CPT);
    const long long wgs = static_cast<long long>(c.B) * chunks;
    if (wgs > 0x7fffffffLL) return set_error(TV_ERANGE, "conv_tree_commit: too many work units");
    if (c.bf16) launch_conv_k<true>(a, true, dim3(static_cast<unsigned>(wgs)), stream);
    else launch_conv_k<false>(a, true, dim3(static_cast<unsigned>(wgs)), stream);
    return launch_status("conv_tree_commit");
}

}  // namespace tv
