// Gated delta-rule layer over a draft tree: verify (factor capture) and commit, gfx950.
//
// Method ("Luce DFlash" README, "How it works" / "Architecture note"; PR #606 "SpecLA
// factor-capture speculative decoding"): for node i with parent p and committed state S0
//     u_i = S_p^T k_i,  delta_i = beta_i (v_i - g_i u_i),  S_i = g_i S_p + k_i delta_i^T,
//     o_i = scale S_i^T q_i.
// Unrolling the recurrence along the root path gives, for any vector x,
//     S_p^T x = G_p S0^T x + sum_{m on path(p)} gamma(p, m) (k_m . x) delta_m
// with G_p the product of g over path(p) and gamma(p, m) the product of g over the path
// nodes strictly below m.  So only S0^T k_i and S0^T q_i (2N products per value channel)
// touch the state; everything else is O(N * depth) per channel plus the key Gram matrix.
//
// Verify: one wave per (sequence, value head, tile of <= 64 value channels).
//   * The tile of S0 (64 channels x dk fp32, one row per channel) is loaded once, split into
//     bf16 hi + lo parts (|x - hi - lo| <= 2^-16 |x|) and contracted with [k_0..k_{n-1},
//     q_0..q_{n-1}] on the matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulate); bf16
//     keys and queries are exact operands.  fp32 inputs are split too (hi*hi+hi*lo+lo*hi).
//   * The same MFMA gives the key Gram matrix k_m . k_i and k_m . q_i.
//   * The tree is then walked in index order with one lane per value channel: delta_i and
//     o_i need only on-chip data (the projections, the Gram matrix and the ancestors'
//     deltas in LDS).  Per-node states are never formed; S0 is never written.
// Commit: the accepted path's captured deltas are flushed into the state in place,
//     S <- (prod_m g_{a_m}) S0 + sum_m c_m k_{a_m} delta_{a_m}^T,  c_m = prod_{m'>m} g_{a_m'},
//   a streaming rank-L update (HBM bound).
#include "tv_internal.h"

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 fp32 values -> bf16 hi and lo with x = hi + lo + O(2^-16 |x|).
__device__ __forceinline__ void split_bf16(const float4& x0, const float4& x1, bf16x8& hi, bf16x8& lo) {
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(v[e]);
        hi[e] = h;
        lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(h));
    }
}

// Contraction-index order used for both MFMA operands: lane group g (lane / 16) of K-step
// ks holds rows ks*32 + {4g..4g+3} and ks*32 + 16 + {4g..4g+3}, so one 16-byte load per
// half covers a contiguous 64-byte run per row across the four groups.
template <int DK>
__device__ __forceinline__ bool second_half_valid(int ks) { return ks * 32 + 16 < DK; }

template <bool BF16IN>
__device__ __forceinline__ float load_scalar(const void* base, size_t idx) {
    if constexpr (BF16IN) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
    else return static_cast<const float*>(base)[idx];
}

// Loads the 8 contraction elements of one key/query row for K-step ks as bf16 hi (and lo
// for fp32 inputs).  `row` points at element 0 of the row.
template <int DK, bool BF16IN>
__device__ __forceinline__ void load_row_operand(const void* row, int ks, int g4, bool valid,
                                                 bf16x8& hi, bf16x8& lo) {
    const int r0 = ks * 32 + 4 * g4;
    if constexpr (BF16IN) {
        const uint16_t* p = static_cast<const uint16_t*>(row) + r0;
        uint2 a = make_uint2(0, 0), c = make_uint2(0, 0);
        if (valid) {
            a = *reinterpret_cast<const uint2*>(p);
            if (second_half_valid<DK>(ks)) c = *reinterpret_cast<const uint2*>(p + 16);
        }
        u32x4 w = {a.x, a.y, c.x, c.y};
        hi = __builtin_bit_cast(bf16x8, w);
        lo = bf16x8{};
    } else {
        const float* p = static_cast<const float*>(row) + r0;
        float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
        if (valid) {
            x0 = *reinterpret_cast<const float4*>(p);
            if (second_half_valid<DK>(ks)) x1 = *reinterpret_cast<const float4*>(p + 16);
        }
        split_bf16(x0, x1, hi, lo);
    }
}

template <int DK, int NT, bool BF16IN>
__global__ __launch_bounds__(64) void lin_verify_kernel(LinVerifyArgs a) {
    constexpr int KS = (DK + 31) / 32;        // MFMA K-steps over dk
    constexpr int NMAX = NT * 8;              // 2n columns fit in NT tiles of 16
    constexpr int GT = (NMAX + 15) / 16;      // Gram row tiles
    constexpr int CST = 68;                   // padded row stride of Cs (floats)
    constexpr int GST = NT * 16 + 4;          // padded row stride of Gm

    __shared__ __align__(16) float Cs[NT * 16][CST];   // Cs[c][j] = (S0^T x_c)[j0 + j]
    __shared__ float Gm[GT * 16][GST];        // Gm[m][c] = k_m . x_c
    __shared__ float Dl[NMAX][64];            // delta_i per value channel
    __shared__ float Vl[NMAX][64];            // v_i per value channel
    __shared__ float gl[NMAX], bl[NMAX];
    __shared__ int par[NMAX], dep[NMAX];
    __shared__ int anc[NMAX][NMAX];           // anc[i][t]: t-th strict ancestor (nearest first)

    const int lane = threadIdx.x;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int CW = a.dv < 64 ? a.dv : 64;
    const int MT = CW >> 4;
    const int ctiles = a.dv / CW;
    int unit = xcd_remap(blockIdx.x, gridDim.x);
    const int ct = unit % ctiles;
    unit /= ctiles;
    const int h = unit % a.Hv;
    const int b = unit / a.Hv;
    const int kh = a.tiled ? h % a.Hk : h / a.group_div;
    const int n = clampi(a.n_nodes[b], 0, a.N < NMAX ? a.N : NMAX);
    if (n <= 0) return;
    const int j0 = ct * CW;

    // 1. committed-state tile as MFMA A operand (rows = value channels); issued first.
    float4 sa[4][KS][2];
    const float* srow = a.state + (static_cast<size_t>(b) * a.Hv + h) * a.dv * DK + static_cast<size_t>(j0) * DK;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            sa[mt][ks][0] = sa[mt][ks][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (mt < MT) {
                const float* p = srow + (mt * 16 + l16) * DK + ks * 32 + 4 * g4;
                sa[mt][ks][0] = *reinterpret_cast<const float4*>(p);
                if (second_half_valid<DK>(ks)) sa[mt][ks][1] = *reinterpret_cast<const float4*>(p + 16);
            }
        }

    // 2. B operand columns: c < n -> k_c, n <= c < 2n -> q_{c-n}, beyond -> zero.
    bf16x8 bh[NT][KS], bo[NT][KS];
    {
        const size_t esz = BF16IN ? 2 : 4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int c = nt * 16 + l16;
            const bool isk = c < n;
            const int node = isk ? c : c - n;
            const bool valid = c < 2 * n;
            const void* base = isk ? a.k : a.q;
            const size_t rowoff = ((static_cast<size_t>(b) * a.N + (valid ? node : 0)) * a.Hk + kh) * DK;
            const void* row = static_cast<const char*>(base) + rowoff * esz;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) load_row_operand<DK, BF16IN>(row, ks, g4, valid, bh[nt][ks], bo[nt][ks]);
        }
    }

    // 3. tree metadata, gates and values.
    if (lane < n) {
        const int p = lane == 0 ? -1 : clampi(a.parent[static_cast<size_t>(b) * a.N + lane], 0, lane - 1);
        par[lane] = p;
        const size_t gi = (static_cast<size_t>(b) * a.N + lane) * a.Hv + h;
        gl[lane] = load_scalar<BF16IN>(a.g, gi);
        bl[lane] = load_scalar<BF16IN>(a.beta, gi);
    }
    for (int i = 0; i < n; ++i) {
        const size_t vi = ((static_cast<size_t>(b) * a.N + i) * a.Hv + h) * a.dv + j0 + lane;
        Vl[i][lane] = lane < CW ? load_scalar<BF16IN>(a.v, vi) : 0.f;
    }

    // 4. Gram matrix: rows are the key columns (tiles 0..GT-1 of the B operand).
#pragma unroll
    for (int gt = 0; gt < GT; ++gt) {
        if (gt * 16 >= n) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                acc = mfma16x16x32(bh[gt][ks], bh[nt][ks], acc);
                if constexpr (!BF16IN) {
                    acc = mfma16x16x32(bh[gt][ks], bo[nt][ks], acc);
                    acc = mfma16x16x32(bo[gt][ks], bh[nt][ks], acc);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Gm[gt * 16 + 4 * g4 + e][nt * 16 + l16] = acc[e];
        }
    }

    // 5. S0^T x_c for this tile's channels.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        if (mt >= MT) continue;
        bf16x8 ah[KS], al[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) split_bf16(sa[mt][ks][0], sa[mt][ks][1], ah[ks], al[ks]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                acc = mfma16x16x32(ah[ks], bh[nt][ks], acc);
                acc = mfma16x16x32(al[ks], bh[nt][ks], acc);
                if constexpr (!BF16IN) acc = mfma16x16x32(ah[ks], bo[nt][ks], acc);
            }
            *reinterpret_cast<float4*>(&Cs[nt * 16 + l16][mt * 16 + 4 * g4]) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
    __syncthreads();

    // 6. ancestor lists: lane i follows its own parent chain once.
    if (lane < n) {
        int t = 0;
        for (int m = par[lane]; m >= 0; m = par[m]) anc[lane][t++] = m;
        dep[lane] = t;
    }
    __syncthreads();

    // 7. the tree walk, nodes in index order, one lane per value channel.
    const int j = lane;
    for (int i = 0; i < n; ++i) {
        float u = 0.f, w = 0.f, gam = 1.f;
        const int d = dep[i];
#pragma unroll 4
        for (int t = 0; t < d; ++t) {
            const int m = anc[i][t];
            const float dm = Dl[m][j];
            u = fmaf(gam * Gm[m][i], dm, u);
            w = fmaf(gam * Gm[m][n + i], dm, w);
            gam *= gl[m];
        }
        u = fmaf(gam, Cs[i][j], u);        // gam = G_parent
        w = fmaf(gam, Cs[n + i][j], w);
        const float gi = gl[i], bi = bl[i];
        const float dl = bi * (Vl[i][j] - gi * u);
        Dl[i][j] = dl;
        const float o = a.scale * fmaf(gi, w, Gm[i][n + i] * dl);
        if (j < CW) {
            const size_t off = ((static_cast<size_t>(b) * a.N + i) * a.Hv + h) * a.dv + j0 + j;
            a.out[off] = o;
            a.cap_delta[off] = dl;
        }
    }
}

template <bool BF16IN>
__global__ __launch_bounds__(256) void lin_commit_kernel(LinCommitArgs a, int rows, int rtiles) {
    extern __shared__ __align__(16) float smem[];   // Kc[L][dk] then cd[L][rows]
    __shared__ int ap[TV_MAX_NODES];
    __shared__ float ga[TV_MAX_NODES];
    __shared__ float coef[TV_MAX_NODES + 4];

    const int t = threadIdx.x;
    int unit = xcd_remap(blockIdx.x, gridDim.x);
    const int rt = unit % rtiles;
    unit /= rtiles;
    const int h = unit % a.Hv;
    const int b = unit / a.Hv;
    const int L = clampi(a.path_len[b], 0, a.Lmax);
    if (L == 0) return;
    const int kh = a.tiled ? h % a.Hk : h / a.group_div;
    const int dk = a.dk, j0 = rt * rows;

    // committed state: this workgroup's rows x dk, at most two float4 per thread, issued first
    float4* S = reinterpret_cast<float4*>(a.state + ((static_cast<size_t>(b) * a.Hv + h) * a.dv + j0) * dk);
    const int nvec = rows * dk / 4;
    float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
    if (t < nvec) s0 = S[t];
    if (t + 256 < nvec) s1 = S[t + 256];

    if (t < L) {
        const int node = clampi(a.path[static_cast<size_t>(b) * a.Lmax + t], 0, a.N - 1);
        ap[t] = node;
        ga[t] = load_scalar<BF16IN>(a.g, (static_cast<size_t>(b) * a.N + node) * a.Hv + h);
    }
    __syncthreads();
    if (t == 0) {
        float c = 1.f;
        for (int m = L - 1; m >= 0; --m) {
            coef[m] = c;
            c *= ga[m];
        }
        coef[L] = c;                            // product over the whole path
    }
    float* Kc = smem;
    float* cd = smem + L * dk;
    for (int idx = t; idx < L * dk; idx += 256) {
        const int m = idx / dk, r = idx - m * dk;
        Kc[idx] = load_scalar<BF16IN>(a.k, ((static_cast<size_t>(b) * a.N + ap[m]) * a.Hk + kh) * dk + r);
    }
    __syncthreads();
    for (int idx = t; idx < L * rows; idx += 256) {
        const int m = idx / rows, jj = idx - m * rows;
        cd[idx] = coef[m] * a.cap_delta[((static_cast<size_t>(b) * a.N + ap[m]) * a.Hv + h) * a.dv + j0 + jj];
    }
    __syncthreads();

    const float G = coef[L];
    auto update = [&](float4 s, int v) {
        const int e = v * 4, jj = e / dk, r = e - jj * dk;
        s.x *= G; s.y *= G; s.z *= G; s.w *= G;
        for (int m = 0; m < L; ++m) {
            const float c = cd[m * rows + jj];
            const float4 kk = *reinterpret_cast<const float4*>(&Kc[m * dk + r]);
            s.x = fmaf(c, kk.x, s.x);
            s.y = fmaf(c, kk.y, s.y);
            s.z = fmaf(c, kk.z, s.z);
            s.w = fmaf(c, kk.w, s.w);
        }
        S[v] = s;
    };
    if (t < nvec) update(s0, t);
    if (t + 256 < nvec) update(s1, t + 256);
}

template <int DK, int NT>
int launch_verify_dk_nt(const LinVerifyArgs& a, bool bf16, hipStream_t stream) {
    const int CW = a.dv < 64 ? a.dv : 64;
    const long long units = static_cast<long long>(a.B) * a.Hv * (a.dv / CW);
    if (units > 0x7fffffffLL) return set_error(TV_ERANGE, "lin_tree_verify: too many work units (%lld)", units);
    dim3 grid(static_cast<unsigned>(units)), block(64);
    if (bf16) hipLaunchKernelGGL((lin_verify_kernel<DK, NT, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((lin_verify_kernel<DK, NT, false>), grid, block, 0, stream, a);
    return launch_status("lin_tree_verify");
}

template <int DK>
int launch_verify_dk(const LinVerifyArgs& a, bool bf16, hipStream_t stream) {
    const int cols = 2 * a.N;
    if (cols <= 16) return launch_verify_dk_nt<DK, 1>(a, bf16, stream);
    if (cols <= 32) return launch_verify_dk_nt<DK, 2>(a, bf16, stream);
    if (cols <= 48) return launch_verify_dk_nt<DK, 3>(a, bf16, stream);
    if (cols <= 64) return launch_verify_dk_nt<DK, 4>(a, bf16, stream);
    return launch_verify_dk_nt<DK, 8>(a, bf16, stream);
}

}  // namespace

int launch_lin_verify(const LinVerifyArgs& a, bool bf16, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_verify_dk<16>(a, bf16, stream);
        case 32: return launch_verify_dk<32>(a, bf16, stream);
        case 64: return launch_verify_dk<64>(a, bf16, stream);
        case 128: return launch_verify_dk<128>(a, bf16, stream);
        default: return set_error(TV_EUNSUPPORTED, "lin_tree_verify: dk=%d not built (16, 32, 64, 128)", a.dk);
    }
}

int launch_lin_commit(const LinCommitArgs& a, bool bf16, hipStream_t stream) {
    const int elems = a.dv * a.dk < 2048 ? a.dv * a.dk : 2048;   // per workgroup: <= 2 float4 per thread
    const int rows = elems / a.dk;
    const int rtiles = a.dv / rows;
    const long long units = static_cast<long long>(a.B) * a.Hv * rtiles;
    if (units > 0x7fffffffLL) return set_error(TV_ERANGE, "lin_tree_commit: too many work units (%lld)", units);
    const size_t shmem = static_cast<size_t>(a.Lmax) * (a.dk + rows) * sizeof(float);
    dim3 grid(static_cast<unsigned>(units)), block(256);
    if (bf16) hipLaunchKernelGGL((lin_commit_kernel<true>), grid, block, shmem, stream, a, rows, rtiles);
    else hipLaunchKernelGGL((lin_commit_kernel<false>), grid, block, shmem, stream, a, rows, rtiles);
    return launch_status("lin_tree_commit");
}

}  // namespace tv
