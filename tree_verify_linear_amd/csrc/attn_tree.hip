// Tree-masked softmax attention over a Q8_0 / Q4_0 KV cache, gfx950.
//
// Method ("Luce DFlash" README, "How it works": one target forward verifies the whole draft
// tree through a causal mask derived from parent pointers; "Architecture note": 24 query
// heads share 4 KV heads of length 256; the FA-window flag: a sliding window, 0 = full;
// "Asymmetric K/V quantization": K and V each Q8_0 or Q4_0).  Query node i sits at position
// T + depth(i); it sees committed slot t iff window == 0 or T + depth(i) - t < window, and
// tree slot T + j iff j is on its root path and (window == 0 or depth(i) - depth(j) < window).
//
// Work unit: (sequence, KV head, row block, KV split).  The rows are the (node, query head)
// pairs that share the KV head -- 22 nodes x 6 heads = 132 rows for the 27B layer -- so every
// K/V byte is read from HBM once per split and reused by all of them.
//   * K/V slot tiles (32 slots) are copied raw into LDS with 16-byte loads, then dequantised
//     cooperatively.  Every value d*q is split exactly into fp16 hi + lo (d is fp16 and q has
//     at most 8 bits, so d*q has <= 19 significant bits and the fp16 residual is exact); K
//     is kept row-major, V transposed (slots contiguous) for the PV operand.
//   * S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulate): Q (bf16,
//     exactly representable in fp16 within range) stays in registers as the B operand, K hi
//     and lo come from LDS as the A operand.  The scores of one row then sit in one lane
//     group in exactly the layout the PV product wants for P, so no transpose is needed.
//   * Mask, scale and an online softmax in the exp2 domain; P is rounded once to fp16 (the
//     only rounding of the whole contraction) and O += P V_hi + P V_lo.
//   * Each split writes unnormalised O, its running max and sum; a combine pass rescales and
//     sums the splits.  With a single split the kernel normalises and writes the output.
#include <cmath>

#include "tv_internal.h"

namespace tv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TS = 32;                 // slots per tile
constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr int MAXRT = 3;               // row tiles (of 16 rows) per wave
constexpr int ROWS_PER_BLOCK = WAVES * MAXRT * 16;   // 192
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int blk_bytes(int type) { return type == TV_Q8_0 ? 34 : 18; }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Exact split of x = d*q (d fp16, |q| <= 127) into two fp16 values.
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
    hi = static_cast<_Float16>(x);
    lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

struct AttnLaunch {
    AttnArgs a;
    int G;              // query heads per KV head
    int rows;           // N * G
    int rows_pad;       // rows rounded up to row tiles of 16, per KV head
    int rblocks;        // row blocks of ROWS_PER_BLOCK rows
    int nsplit;         // KV splits per (sequence, KV head)
    int chunk;          // slots per split (multiple of TS)
    float* opart;       // [B][Hkv][nsplit][rows_pad][D]
    float* mpart;       // [B][Hkv][nsplit][rows_pad]  running max (log2 domain)
    float* lpart;       // [B][Hkv][nsplit][rows_pad]  running sum
};

template <int D>
struct AttnSmem {
    static constexpr int NB = D / 32;
    static constexpr int KST = D + 8;              // fp16 row stride of the K tile (padded)
    static constexpr int VST = TS + 4;             // fp16 row stride of the transposed V tile
    __align__(16) uint8_t kraw[TS * NB * 34];
    __align__(16) uint8_t vraw[TS * NB * 34];
    __align__(16) _Float16 khi[TS][KST];
    __align__(16) _Float16 klo[TS][KST];
    __align__(16) _Float16 vhi[D][VST];
    __align__(16) _Float16 vlo[D][VST];
    uint64_t anc[TV_MAX_NODES];
    int dep[TV_MAX_NODES];
    int par[TV_MAX_NODES];
};

// Decodes 8 consecutive elements (e0 .. e0+7, e0 % 8 == 0) of one quantised block at `blk`.
__device__ __forceinline__ void decode8(const uint8_t* blk, int type, int e0, float (&x)[8]) {
    const float d = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(blk));
    if (type == TV_Q8_0) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(blk + 2 + e0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint16_t w = p[k];
            x[2 * k] = d * static_cast<float>(static_cast<int8_t>(w & 0xff));
            x[2 * k + 1] = d * static_cast<float>(static_cast<int8_t>(w >> 8));
        }
    } else {
        const bool high = e0 >= 16;
        const uint16_t* p = reinterpret_cast<const uint16_t*>(blk + 2 + (e0 & 15));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint16_t w = p[k];
            const int b0 = w & 0xff, b1 = w >> 8;
            const int n0 = high ? (b0 >> 4) : (b0 & 15), n1 = high ? (b1 >> 4) : (b1 & 15);
            x[2 * k] = d * static_cast<float>(n0 - 8);
            x[2 * k + 1] = d * static_cast<float>(n1 - 8);
        }
    }
}

template <int D>
__global__ __launch_bounds__(THREADS, 1) void attn_kernel(AttnLaunch L) {
    constexpr int NB = D / 32, KS = D / 32, NTD = D / 16;
    using SM = AttnSmem<D>;
    __shared__ SM sm;
    const AttnArgs& a = L.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, l16 = lane & 15;

    int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int split = wg % L.nsplit;
    wg /= L.nsplit;
    const int rb = wg % L.rblocks;
    wg /= L.rblocks;
    const int kvh = wg % a.Hkv;
    const int b = wg / a.Hkv;

    const int n = clampi(a.n_nodes[b], 0, a.N);
    const int T = clampi(a.n_past[b], 0, a.Tcap - n);
    const int W = a.window;
    const int lo_b = W ? (T - W + 1 > 0 ? T - W + 1 : 0) : 0;   // first committed slot any node sees
    const int hi_b = T + n;
    const int s0 = lo_b + split * L.chunk;
    const int s1 = s0 + L.chunk < hi_b ? s0 + L.chunk : hi_b;

    // tree metadata (depth, ancestor sets) for this sequence
    if (tid < n) sm.par[tid] = tid == 0 ? -1 : clampi(a.parent[static_cast<size_t>(b) * a.N + tid], 0, tid - 1);
    __syncthreads();
    if (tid == 0) {
        for (int i = 0; i < n; ++i) {
            const int p = sm.par[i];
            sm.dep[i] = p < 0 ? 0 : sm.dep[p] + 1;
            sm.anc[i] = (p < 0 ? 0ull : sm.anc[p]) | (1ull << i);
        }
    }

    // this lane's rows: Q as the MFMA B operand, and the row's mask parameters
    const int kt = a.k_type, vt = a.v_type;
    f16x8 qop[MAXRT][KS];
    int rnode[MAXRT], rlo[MAXRT], rdep[MAXRT];
    uint64_t ranc[MAXRT];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MAXRT; ++t) {
        const int r = rb * ROWS_PER_BLOCK + (wave + WAVES * t) * 16 + l16;
        const int node = r / L.G, hh = r - node * L.G;
        const bool ok = r < L.rows && node < n;
        rnode[t] = ok ? node : -1;
        rdep[t] = ok ? sm.dep[node] : 0;
        ranc[t] = ok ? sm.anc[node] : 0ull;
        rlo[t] = W ? T + rdep[t] - W + 1 : 0;
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               ((static_cast<size_t>(b) * a.N + (ok ? node : 0)) * a.Hq + kvh * L.G + hh) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (ok) w = *reinterpret_cast<const uint4*>(qrow + ks * 32 + 8 * g4);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qop[t][ks][2 * e] = static_cast<_Float16>(__uint_as_float(u[e] << 16));
                qop[t][ks][2 * e + 1] = static_cast<_Float16>(__uint_as_float(u[e] & 0xffff0000u));
            }
        }
    }

    f32x4 oacc[MAXRT][NTD];
#pragma unroll
    for (int t = 0; t < MAXRT; ++t)
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt) oacc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrow[MAXRT], lrow[MAXRT];
#pragma unroll
    for (int t = 0; t < MAXRT; ++t) {
        mrow[t] = -INFINITY;
        lrow[t] = 0.f;
    }
    const float sl2 = a.scale * kLog2e;
    const int kbb = blk_bytes(kt), vbb = blk_bytes(vt);
    const int krow = NB * kbb, vrow = NB * vbb;
    const uint8_t* kbase = a.k_cache + (static_cast<size_t>(b) * a.Hkv + kvh) * a.Tcap * krow;
    const uint8_t* vbase = a.v_cache + (static_cast<size_t>(b) * a.Hkv + kvh) * a.Tcap * vrow;

    for (int t0 = s0; t0 < s1; t0 += TS) {
        // 1. raw K and V rows of slots t0 .. t0+TS-1 into LDS (16-byte pieces; rows past the
        //    cache end are zero, rows past s1 are masked below)
        {
            const int kch = TS * krow / 16, vch = TS * vrow / 16;
            const int slots_ok = a.Tcap - t0 < TS ? a.Tcap - t0 : TS;
            for (int c = tid; c < kch; c += THREADS) {
                uint4 w = make_uint4(0, 0, 0, 0);
                if (c * 16 < slots_ok * krow) w = *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(t0) * krow + c * 16);
                *reinterpret_cast<uint4*>(&sm.kraw[c * 16]) = w;
            }
            for (int c = tid; c < vch; c += THREADS) {
                uint4 w = make_uint4(0, 0, 0, 0);
                if (c * 16 < slots_ok * vrow) w = *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(t0) * vrow + c * 16);
                *reinterpret_cast<uint4*>(&sm.vraw[c * 16]) = w;
            }
        }
        __syncthreads();
        // 2. dequantise: K row-major (one (slot, 8 elements) piece per item), V transposed
        //    (4 slots x 8 elements per item)
        for (int item = tid; item < TS * (D / 8); item += THREADS) {
            const int slot = item / (D / 8), e0 = (item % (D / 8)) * 8;
            float x[8];
            decode8(&sm.kraw[slot * krow + (e0 / 32) * kbb], kt, e0 % 32, x);
            f16x8 h, l;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                _Float16 hh_, ll_;
                split_f16(x[e], hh_, ll_);
                h[e] = hh_;
                l[e] = ll_;
            }
            *reinterpret_cast<f16x8*>(&sm.khi[slot][e0]) = h;
            *reinterpret_cast<f16x8*>(&sm.klo[slot][e0]) = l;
        }
        for (int item = tid; item < (TS / 4) * (D / 8); item += THREADS) {
            const int sq = item / (D / 8), e0 = (item % (D / 8)) * 8;
            float x[4][8];
#pragma unroll
            for (int s = 0; s < 4; ++s) decode8(&sm.vraw[(4 * sq + s) * vrow + (e0 / 32) * vbb], vt, e0 % 32, x[s]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                f16x4 h, l;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    _Float16 hh_, ll_;
                    split_f16(x[s][e], hh_, ll_);
                    h[s] = hh_;
                    l[s] = ll_;
                }
                *reinterpret_cast<f16x4*>(&sm.vhi[e0 + e][4 * sq]) = h;
                *reinterpret_cast<f16x4*>(&sm.vlo[e0 + e][4 * sq]) = l;
            }
        }
        __syncthreads();

        // 3. S^T = K Q^T for the wave's row tiles: sacc[st][t][e] = score of slot
        //    t0 + 16 st + 4 g4 + e against row l16 of row tile t
        f32x4 sacc[2][MAXRT];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int t = 0; t < MAXRT; ++t) sacc[st][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 ah = *reinterpret_cast<const f16x8*>(&sm.khi[st * 16 + l16][ks * 32 + 8 * g4]);
                const f16x8 al = *reinterpret_cast<const f16x8*>(&sm.klo[st * 16 + l16][ks * 32 + 8 * g4]);
#pragma unroll
                for (int t = 0; t < MAXRT; ++t) {
                    sacc[st][t] = mfma_f16(ah, qop[t][ks], sacc[st][t]);
                    sacc[st][t] = mfma_f16(al, qop[t][ks], sacc[st][t]);
                }
                __builtin_amdgcn_sched_barrier(0);     // bound the operands kept live
            }
        }

        // 4. mask, online softmax (exp2 domain), P in fp16 as the PV A operand
        f16x8 pa[MAXRT];
#pragma unroll
        for (int t = 0; t < MAXRT; ++t) {
            float sv[8];
            float mt = -INFINITY;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int slot = t0 + (k < 4 ? 4 * g4 + k : 16 + 4 * g4 + (k - 4));
                bool vis = rnode[t] >= 0 && slot < s1;
                if (slot < T) {
                    vis = vis && slot >= rlo[t];
                } else {
                    const int j = slot - T;
                    vis = vis && j < 64 && ((ranc[t] >> j) & 1ull) && (W == 0 || rdep[t] - sm.dep[j < 64 ? j : 0] < W);
                }
                const float s = (k < 4 ? sacc[0][t][k] : sacc[1][t][k - 4]) * sl2;
                sv[k] = vis ? s : -INFINITY;
                mt = fmaxf(mt, sv[k]);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            // Lazy rescaling: P is taken against a reference max that moves only when a row's
            // max grows by more than 2^8 (so P <= 256, still exact to fp16's relative
            // precision); O and the sum are rescaled only then, for the whole wave at once.
            const bool grow = mt > mrow[t] + 8.f;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float mnew = grow ? mt : mrow[t];
                const float alpha = (mnew == -INFINITY || mrow[t] == -INFINITY) ? 0.f : exp2f(mrow[t] - mnew);
                lrow[t] *= alpha;
                mrow[t] = mnew;
                float af[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) af[e] = __shfl(alpha, 4 * g4 + e);
#pragma unroll
                for (int nt = 0; nt < NTD; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) oacc[t][nt][e] *= af[e];
            }
            float psum = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float p = mrow[t] == -INFINITY ? 0.f : exp2f(sv[k] - mrow[t]);
                pa[t][k] = static_cast<_Float16>(p);
                psum += static_cast<float>(pa[t][k]);       // the weights actually applied
            }
            lrow[t] += psum;
        }

        // 5. O += P V (hi and lo parts of V)
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt) {
            const int e = nt * 16 + l16;
            const f16x4 h0 = *reinterpret_cast<const f16x4*>(&sm.vhi[e][4 * g4]);
            const f16x4 h1 = *reinterpret_cast<const f16x4*>(&sm.vhi[e][16 + 4 * g4]);
            const f16x4 l0 = *reinterpret_cast<const f16x4*>(&sm.vlo[e][4 * g4]);
            const f16x4 l1 = *reinterpret_cast<const f16x4*>(&sm.vlo[e][16 + 4 * g4]);
            const f16x8 bh = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
            const f16x8 bl = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
#pragma unroll
            for (int t = 0; t < MAXRT; ++t) {
                oacc[t][nt] = mfma_f16(pa[t], bh, oacc[t][nt]);
                oacc[t][nt] = mfma_f16(pa[t], bl, oacc[t][nt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();                               // LDS tiles are rewritten next
    }

    // 6. per-row sums across the four lane groups, then write
#pragma unroll
    for (int t = 0; t < MAXRT; ++t) {
        lrow[t] += __shfl_xor(lrow[t], 16);
        lrow[t] += __shfl_xor(lrow[t], 32);
    }
    const size_t part = (static_cast<size_t>(b) * a.Hkv + kvh) * L.nsplit + split;
#pragma unroll
    for (int t = 0; t < MAXRT; ++t) {
        const int rt = wave + WAVES * t;
        const int rbase = rb * ROWS_PER_BLOCK + rt * 16;
        if (rbase >= L.rows) continue;
        if (L.nsplit == 1) {
            // normalise here: O rows 4 g4 + e need their row's sum and max
            float inv[4], mx[4], sm_[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sm_[e] = __shfl(lrow[t], 4 * g4 + e);
                mx[e] = __shfl(mrow[t], 4 * g4 + e);
                inv[e] = sm_[e] > 0.f ? 1.f / sm_[e] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = rbase + 4 * g4 + e;
                const int node = r / L.G, hh = r - node * L.G;
                if (r >= L.rows || node >= n) continue;
                float* orow = a.out + ((static_cast<size_t>(b) * a.N + node) * a.Hq + kvh * L.G + hh) * D;
#pragma unroll
                for (int nt = 0; nt < NTD; ++nt) orow[nt * 16 + l16] = oacc[t][nt][e] * inv[e];
                if (a.lse && l16 == 0)
                    a.lse[(static_cast<size_t>(b) * a.N + node) * a.Hq + kvh * L.G + hh] =
                        (mx[e] + log2f(sm_[e])) * kLn2;
            }
        } else {
            float* op = L.opart + (part * L.rows_pad + rbase) * D;
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int nt = 0; nt < NTD; ++nt) op[(4 * g4 + e) * D + nt * 16 + l16] = oacc[t][nt][e];
            if (g4 == 0) {
                L.mpart[part * L.rows_pad + rbase + l16] = mrow[t];
                L.lpart[part * L.rows_pad + rbase + l16] = lrow[t];
            }
        }
    }
}

// Merges the splits of one row: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnLaunch L) {
    const AttnArgs& a = L.a;
    int wg = blockIdx.x;
    const int r = wg % L.rows;
    wg /= L.rows;
    const int kvh = wg % a.Hkv;
    const int b = wg / a.Hkv;
    const int n = clampi(a.n_nodes[b], 0, a.N);
    const int node = r / L.G, hh = r - node * L.G;
    if (node >= n) return;
    const size_t p0 = (static_cast<size_t>(b) * a.Hkv + kvh) * L.nsplit;
    float M = -INFINITY;
    for (int s = 0; s < L.nsplit; ++s) M = fmaxf(M, L.mpart[(p0 + s) * L.rows_pad + r]);
    float Lsum = 0.f;
    float acc[D / 64];
#pragma unroll
    for (int k = 0; k < D / 64; ++k) acc[k] = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < L.nsplit; ++s) {
            const float ms = L.mpart[(p0 + s) * L.rows_pad + r];
            if (ms == -INFINITY) continue;
            const float w = exp2f(ms - M);
            Lsum += w * L.lpart[(p0 + s) * L.rows_pad + r];
            const float* op = L.opart + ((p0 + s) * L.rows_pad + r) * D;
#pragma unroll
            for (int k = 0; k < D / 64; ++k) acc[k] += w * op[k * 64 + threadIdx.x];
        }
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    float* orow = a.out + ((static_cast<size_t>(b) * a.N + node) * a.Hq + kvh * L.G + hh) * D;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) orow[k * 64 + threadIdx.x] = acc[k] * inv;
    if (a.lse && threadIdx.x == 0)
        a.lse[(static_cast<size_t>(b) * a.N + node) * a.Hq + kvh * L.G + hh] = (M + log2f(Lsum)) * kLn2;
}

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

// Split policy: about one workgroup per CU, splits of at least 256 slots.  Depends only on
// host-known sizes (n_past lives on the device), using the widest visible span.
struct SplitPlan {
    int G, rows, rows_pad, rblocks, nsplit, chunk;
};
SplitPlan plan_splits(int B, int N, int Hq, int Hkv, int Tcap, int window, int cus) {
    SplitPlan p;
    p.G = Hq / Hkv;
    p.rows = N * p.G;
    p.rows_pad = (p.rows + 15) / 16 * 16;
    p.rblocks = (p.rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    long long span = window ? static_cast<long long>(window) - 1 + N : Tcap;
    if (span > Tcap) span = Tcap;
    if (span < 1) span = 1;
    const long long units = static_cast<long long>(B) * Hkv * p.rblocks;
    long long ns = (cus + units - 1) / units;
    const long long maxns = (span + 255) / 256;
    if (ns > maxns) ns = maxns;
    if (ns < 1) ns = 1;
    long long chunk = (span + ns - 1) / ns;
    chunk = (chunk + TS - 1) / TS * TS;
    p.nsplit = static_cast<int>((span + chunk - 1) / chunk);
    p.chunk = static_cast<int>(chunk);
    return p;
}

size_t workspace_for(const SplitPlan& p, int B, int Hkv, int D) {
    if (p.nsplit <= 1) return 256;
    const size_t parts = static_cast<size_t>(B) * Hkv * p.nsplit * p.rows_pad;
    const size_t bytes = parts * (static_cast<size_t>(D) + 2) * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

}  // namespace

size_t attn_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int Tcap, int window) {
    const SplitPlan p = plan_splits(B, N, Hq, Hkv, Tcap, window, cu_count());
    return workspace_for(p, B, Hkv, D);
}

int launch_attn(const AttnArgs& a, hipStream_t stream) {
    const SplitPlan p = plan_splits(a.B, a.N, a.Hq, a.Hkv, a.Tcap, a.window, cu_count());
    AttnLaunch L;
    L.a = a;
    L.G = p.G;
    L.rows = p.rows;
    L.rows_pad = p.rows_pad;
    L.rblocks = p.rblocks;
    L.nsplit = p.nsplit;
    L.chunk = p.chunk;
    const size_t parts = static_cast<size_t>(a.B) * a.Hkv * p.nsplit * p.rows_pad;
    float* ws = static_cast<float*>(a.workspace);
    L.opart = ws;
    L.mpart = ws + parts * a.D;
    L.lpart = L.mpart + parts;
    const long long wgs = static_cast<long long>(a.B) * a.Hkv * p.rblocks * p.nsplit;
    const long long rowsall = static_cast<long long>(a.B) * a.Hkv * p.rows;
    if (wgs > 0x7fffffffLL || rowsall > 0x7fffffffLL)
        return set_error(TV_ERANGE, "attn_tree_verify: too many work units");
    if (a.D != 256) return set_error(TV_EUNSUPPORTED, "attn_tree_verify: D=%d not built", a.D);
    hipLaunchKernelGGL(attn_kernel<256>, dim3(static_cast<unsigned>(wgs)), dim3(THREADS), 0, stream, L);
    if (p.nsplit > 1)
        hipLaunchKernelGGL(attn_combine_kernel<256>, dim3(static_cast<unsigned>(rowsall)), dim3(64), 0, stream, L);
    return launch_status("attn_tree_verify");
}

}  // namespace tv
