// Gated delta-rule layer over a draft tree: verify (factor capture) and commit, gfx950.
//
// Method ("Luce DFlash" README, "How it works" / "Architecture note"; PR #606 "SpecLA
// factor-capture speculative decoding"): for node i with parent p and committed state S0
//     u_i = S_p^T k_i,  delta_i = beta_i (v_i - g_i u_i),  S_i = g_i S_p + k_i delta_i^T,
//     o_i = scale S_i^T q_i.
// Unrolling the recurrence along the root path gives, for any vector x,
//     S_p^T x = G_p S0^T x + sum_{m strict ancestor of i} gamma(i, m) (k_m . x) delta_m
// with G_p the product of g over the root path of p and gamma(i, m) the product of g over
// the strict ancestors of i below m.  So only S0^T k_i and S0^T q_i (2n products per value
// channel) touch the state; the rest is O(n * depth) per channel plus the key Gram matrix:
//     delta_i = beta_i v_i - beta_i g_i G_p a_i + sum_m Pu[i][m] delta_m
//     o_i     = scale g_i G_p b_i + scale (k_i . q_i) delta_i + sum_m Pw[i][m] delta_m
// with a_i = (S0^T k_i)[j], b_i = (S0^T q_i)[j] for value channel j and, for each strict
// ancestor m of i, Pu[i][m] = -beta_i g_i gamma(i, m) (k_m . k_i) and
// Pw[i][m] = scale g_i gamma(i, m) (k_m . q_i).
//
// Verify: a work unit is (sequence, value head, tile of <= 64 value channels).
//   * The unit's S0 tile (one row of dk fp32 per channel) is split into bf16 hi + lo parts
//     (|x - hi - lo| <= 2^-16 |x|) and contracted with [k_0..k_{n-1}, q_0..q_{n-1}] on the
//     matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulate); bf16 keys and queries are
//     exact operands, fp32 ones are split too (hi*hi + hi*lo + lo*hi).  The same MFMA gives
//     the key Gram matrix.
//   * Lane i computes node i's ancestor set and walk coefficients and writes them as LDS
//     row i.  The walk then runs one lane per value channel, nodes in index order, in
//     branch-free straight-line code whose LDS addresses are compile-time offsets (nodes
//     beyond the tree have zero coefficients); deltas stay in registers.  Per-node states
//     are never formed; S0 is never written.
//   * One wave per unit; several units stay resident per CU, so one unit's loads overlap
//     another's arithmetic.  No load address depends on loaded data.
// Commit: the accepted path's captured deltas are flushed into the state in place,
//     S <- (prod_m g_{a_m}) S0 + sum_m c_m k_{a_m} delta_{a_m}^T,  c_m = prod_{m'>m} g_{a_m'},
//   a streaming rank-L update (HBM bound).  Fused variant: the next step's verify applies
//   the same update to the state tile it has just loaded, stores the committed tile and
//   verifies from it, so the state is read once per step instead of twice.
#include <type_traits>

#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kMinChannels = 16;                // narrowest verify unit (one MFMA row tile)
// Units of the bank verify hold at most 32 value channels: the bank's operands then fit beside
// the state tile and the unit's inputs without spilling registers.
constexpr int kBankTiles = 4;
// bf16 units copy their key / query rows and value rows straight from memory into LDS
// (global-to-LDS copies) instead of holding them in registers while the state tile streams in.
constexpr bool kStageBf16 = true;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 x 16 x 4 in fp32: lane (g, l) holds A[l][g] and B[g][l]; the accumulator layout is that
// of every 16 x 16 matrix-core tile (lane (g, l): rows 4g .. 4g+3 of column l).
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
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

// 8 fp32 values -> three bf16 terms with x = hi + mid + lo + O(2^-24 |x|) (each residual is
// exact in fp32).
__device__ __forceinline__ void split3_bf16(const float4& x0, const float4& x1, bf16x8& hi, bf16x8& mid,
                                            bf16x8& lo) {
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(v[e]);
        const float r = v[e] - static_cast<float>(h);
        const __bf16 m = static_cast<__bf16>(r);
        hi[e] = h;
        mid[e] = m;
        lo[e] = static_cast<__bf16>(r - static_cast<float>(m));
    }
}

// Contraction order shared by every MFMA operand over the keys: lane group g (lane / 16) of
// K-step ks holds keys ks*32 + 4g .. 4g+3 (half 0) and ks*32 + 16 + 4g .. 16 + 4g + 3 (half 1)
// of its row, zero past dk.  (Any order gives the same dot products; this one is also the
// accumulator layout of a 16 x 16 matrix-core tile over 16 keys, so a state tile held this way
// can be updated by matrix instructions in place.)
template <int DK>
__device__ __forceinline__ bool kvalid(int ks, int g4, int half) { return ks * 32 + 16 * half + 4 * g4 < DK; }
__device__ __forceinline__ int kfirst(int ks, int g4, int half) { return ks * 32 + 16 * half + 4 * g4; }

// A verify unit is one wave: its LDS accesses execute in issue order, so ordering them needs
// only that the compiler keeps them in place and that their results have returned -- never a
// wait for the wave's outstanding global stores (committed state tiles, bank entries), which
// __syncthreads would add.
__device__ __forceinline__ void wave_lds_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);             // lgkmcnt(0); vector memory not waited for
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait for every vector memory operation of the wave, the global-to-LDS row copies included.
__device__ __forceinline__ void wait_all_vm() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

template <bool BF16IN>
__device__ __forceinline__ float load_scalar(const void* base, size_t idx) {
    if constexpr (BF16IN) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
    else return static_cast<const float*>(base)[idx];
}

// One key/query row's 8 contraction elements for K-step ks, as bf16 hi (and lo for fp32).
template <int DK, bool BF16IN>
__device__ __forceinline__ void load_row_operand(const void* row, int ks, int g4, bool valid, bf16x8& hi,
                                                 bf16x8& lo) {
    const int r0 = kfirst(ks, g4, 0), r1 = kfirst(ks, g4, 1);
    const bool ok0 = valid && kvalid<DK>(ks, g4, 0), ok1 = valid && kvalid<DK>(ks, g4, 1);
    if constexpr (BF16IN) {
        uint2 w0 = make_uint2(0, 0), w1 = w0;
        if (ok0) w0 = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(row) + r0);
        if (ok1) w1 = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(row) + r1);
        u32x4 u = {w0.x, w0.y, w1.x, w1.y};
        hi = __builtin_bit_cast(bf16x8, u);
        lo = bf16x8{};
    } else {
        float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
        if (ok0) x0 = *reinterpret_cast<const float4*>(static_cast<const float*>(row) + r0);
        if (ok1) x1 = *reinterpret_cast<const float4*>(static_cast<const float*>(row) + r1);
        split_bf16(x0, x1, hi, lo);
    }
}

// A unit's S0 tile (MT x 16 value channels x dk) in MFMA A-operand order.
// Global loads issued by load_state_tile: one per 16-key piece inside dk (dk is a multiple of
// 16) and channel piece.
template <int DK, int MTX>
constexpr int state_tile_loads() { return MTX * (DK / 16); }

// 16 zero bytes in global memory: the source of loads that fall outside a unit's tile.
__device__ __align__(16) const float kZeros[4] = {0.f, 0.f, 0.f, 0.f};
typedef const __attribute__((address_space(1))) float gfloat;
typedef const __attribute__((address_space(1))) f32x4 gf32x4;

template <int DK, int MTX>
__device__ __forceinline__ void load_state_tile(float4 (&sa)[MTX][(DK + 31) / 32][2], const float* tile, int MT,
                                                int l16, int g4) {
    constexpr int KS = (DK + 31) / 32;
    // Every lane loads: pieces past the unit's width or past dk read 16 zero bytes instead (a
    // select of the address, not of the loaded value, which the compiler may turn back into a
    // load under a lane-dependent branch, making the wave wait for each load in turn).
#pragma unroll
    for (int mt = 0; mt < MTX; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // a 16-key piece past dk: zero, with no load (see state_tile_loads)
                if (ks * 32 + 16 * h >= DK) {
                    sa[mt][ks][h] = make_float4(0.f, 0.f, 0.f, 0.f);
                    continue;
                }
                // both addresses are global memory: kept in that address space, the loads stay
                // global loads (a generic pointer would make them flat loads, whose counts the
                // waits below cannot rely on)
                const bool ok = mt < MT && kvalid<DK>(ks, g4, h);
                const gfloat* src = ok ? (const gfloat*)(tile + (mt * 16 + l16) * DK + kfirst(ks, g4, h))
                                       : (const gfloat*)kZeros;
                const f32x4 x = *(const gf32x4*)src;
                sa[mt][ks][h] = make_float4(x[0], x[1], x[2], x[3]);
            }
        }
}

struct UnitIds {
    int b, h, kh, ct, j0;
};

__device__ __forceinline__ UnitIds unit_ids(const LinVerifyArgs& a, int unit, int ctiles, int CW) {
    UnitIds u;
    u.ct = unit % ctiles;
    u.h = (unit / ctiles) % a.Hv;
    u.b = unit / ctiles / a.Hv;
    u.kh = a.tiled ? u.h % a.Hk : u.h / a.group_div;
    u.j0 = u.ct * CW;
    return u;
}

// Shared memory of one verify wave, kept at or under 20 KiB for trees of up to 24 nodes so
// that eight units stay resident per CU (the LDS is allocated in 512-byte granules).
template <int NT, bool BF16IN>
struct VerifySmem {
    static constexpr int NMAX = NT * 8;
    static constexpr int GT = (NMAX + 15) / 16;
    static constexpr int GC = NT * 16;              // Gm columns: x_0 .. x_{2N-1} and padding
    static constexpr int GST = GC + 4;              // padded row stride of Gm
    // Cs[c][j] = (S0^T x_c)[j0 + j], rows of 64 floats with the float4 slots of row c permuted
    // by c mod 16 (see cs_at), so the matrix-core stores of 16 rows spread over the banks.
    // Rows N.. become the outputs, rows 0.. the deltas once the walks have read them.
    __align__(16) float Cs[NT * 16][64];
    // Three lifetimes in one place (one wave reads each before the next is written):
    union {
        // Gm[m][c] = k_m . x_c, until the coefficients are built; column GC holds node m's
        // decay and column GC + 1 its parent
        float Gm[NMAX][GST];
        struct {
            __align__(16) float Pu[NMAX][NMAX];    // Pu[i][m], zero unless m is a strict ancestor of i
            __align__(16) float Pw[NMAX][NMAX];    //   (both read by the walks)
            float cv[NMAX], ca[NMAX], cb[NMAX], cd[NMAX];   // per-node scalars of the walks
        };
        struct {                                    // before all of those: a pending commit
            __align__(16) float pk[4][128];         //   key rows of four accepted nodes
            __align__(16) float pd[4][64];          //   c_l * delta_l for the unit's channels
            int pn[TV_MAX_NODES];                   //   accepted node of entry l
            float pg[TV_MAX_NODES], pc[TV_MAX_NODES];   // its decay; c_l = prod_{l' > l} g
        };
    };
    __align__(16) uint8_t Vs[NMAX * 64 * (BF16IN ? 2 : 4)];   // v rows of the unit, [node][channel]
};

// Element (row, col) of Cs; col % 4 == 0 addresses a whole float4 slot.
template <typename SM>
__device__ __forceinline__ float* cs_at(SM& sm, int row, int col) {
    return &sm.Cs[row][col ^ ((row & 15) << 2)];
}

// Everything one unit reads from global memory, held in registers while in flight.  MTX: the
// most 16-channel pieces a unit holds (4: up to 64 channels).
template <int DK, int NT, bool BF16IN, int MTX = 4>
struct UnitIn {
    static constexpr int KS = (DK + 31) / 32;
    static constexpr int NMAX = NT * 8;
    static constexpr int ESZ = BF16IN ? 2 : 4;
    static constexpr int VL = (NMAX * 64 * ESZ + 1023) / 1024;   // 16-byte v loads per lane
    float4 sa[MTX][KS][2];
    bf16x8 bh[NT][KS], bo[NT][KS];
    uint4 vraw[VL];
    uint32_t graw, braw;                             // lane i: node i's g and beta, raw input bits
    int praw, nraw;                                  // lane i: parent[i]; n_nodes[b] (unclamped)
    // a pending commit (previous step's path): its length, lane l's entry (node, decay) and
    // the first four entries' key / delta segments (lane -> entry lane / 16, segment lane % 16)
    int pL, pnode;
    int bE;                                          // bank mode: entries already in the bank
    float bg[4];                                     // bank mode: decays of entries 4 lane .. +3
    // bank mode, bf16 inputs: the first 32 entries' operands, loaded with the unit's inputs --
    // key tile t's A operand (keys 16 t + l16, entries 8 g4 .. +7) and the deltas of channel
    // 16 mt + l16, entries 8 g4 .. +7
    uint4 bk[2 * KS];
    float4 bd[MTX][2];
    // kept as loaded (raw input bits, converted where used): a conversion or select right at
    // the load would make the wave wait for it, and so for everything issued before it
    uint32_t pgraw;                                  // lane l: entry l's decay
    uint4 pkraw[BF16IN ? 1 : 2];                     // key segment (8 bf16 or 8 fp32)
    float4 pdv;                                      // delta segment
};

// Issues every load of a unit.  Only the previous path's operands depend on loaded data (its
// entries, loaded first, their dependent loads last); everything else is issued without
// waiting (the tree size n is applied at compute time; rows up to N are loaded).
template <int DK, int NT, bool BF16IN, bool STAGE, bool PRELOAD = true, int MTX = 4, bool BANK = false,
          bool PEND = true>
__device__ __forceinline__ void load_unit(UnitIn<DK, NT, BF16IN, MTX>& in, VerifySmem<NT, BF16IN>& sm,
                                          const LinVerifyArgs& a, int unit, int ctiles, int CW, int lane) {
    using U = UnitIn<DK, NT, BF16IN, MTX>;
    const int g4 = lane >> 4, l16 = lane & 15;
    const UnitIds id = unit_ids(a, unit, ctiles, CW);
    const int N = a.N;                              // <= NMAX by dispatch
    // wave-uniform: read through the constant address space (a scalar load, counted apart
    // from the vector loads and stores, so nothing waits on them for it)
    in.nraw = N > 0 ? ((const __attribute__((address_space(4))) int32_t*)(a.n_nodes))[id.b] : 0;
    // A pending path's entries first: the loads that depend on them (its decays, keys and
    // deltas) are issued after the state tile's, and vector loads return in issue order, so
    // the entries are back long before the tile (every lane loads; entries past Lmax unused).
    int pentry = 0;
    if (PEND && a.pend_path_len)
        pentry = a.pend_path[static_cast<size_t>(id.b) * a.pend_Lmax + (lane < a.pend_Lmax ? lane : a.pend_Lmax - 1)];
    if (BANK && a.bank_len) {                       // the bank's decays (entries 4 lane .. +3)
        const float* gb = a.bank_g + (static_cast<size_t>(id.b) * a.Hv + id.h) * a.bank_Emax;
#pragma unroll
        for (int i = 0; i < 4; ++i) in.bg[i] = gb[min(4 * lane + i, a.bank_Emax - 1)];
    }
    in.praw = -1;
    in.graw = in.braw = 0u;
    if (N > 0) {                                    // every lane loads (node clamped)
        const int nd = lane < N ? lane : N - 1;
        const int pr = a.parent[static_cast<size_t>(id.b) * N + nd];
        const size_t gi = (static_cast<size_t>(id.b) * N + nd) * a.Hv + id.h;
        uint32_t gr, br;
        if constexpr (BF16IN) {
            gr = static_cast<const uint16_t*>(a.g)[gi];
            br = static_cast<const uint16_t*>(a.beta)[gi];
        } else {
            gr = static_cast<const uint32_t*>(a.g)[gi];
            br = static_cast<const uint32_t*>(a.beta)[gi];
        }
        in.praw = pr;                               // lanes >= n are masked where used
        in.graw = gr;
        in.braw = br;
    }
    if constexpr (STAGE) {
        static_assert(BF16IN, "staged rows are bf16");
        if (N > 0) {                                // (N = 0: a flush without a tree)
            // B operand columns c (< N: k_c; < 2N: q_{c-N}; beyond: k_0, never used) as LDS rows of
            // Cs, row c at byte 2 DK c; its 16-byte pieces are stored XOR-rotated by the row index
            // (piece p at slot p ^ (c mod LPR)), so the 16 rows a matrix-core operand read touches
            // fall in different banks.  One copy instruction moves 1 KiB: RPI whole rows.
            constexpr int LPR = DK / 8, RPI = 64 / LPR, NI = (NT * 16 + RPI - 1) / RPI;   // <= Cs
            const uint32_t cs = lds_address(&sm.Cs[0][0]);
            const int rr = lane / LPR, ck = lane % LPR;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int c = j * RPI + rr;
                const bool isq = c >= N && c < 2 * N;
                const int node = c < N ? c : (isq ? c - N : 0);
                const uint16_t* row = static_cast<const uint16_t*>(isq ? a.q : a.k) +
                                      ((static_cast<size_t>(id.b) * N + node) * a.Hk + id.kh) * DK;
                copy16_to_lds(row + (ck ^ (c & (LPR - 1))) * 8, __builtin_amdgcn_readfirstlane(cs + j * 1024));
            }
            // v rows of the unit's channels into Vs, row i at byte 2 CW i (rows past N repeat N - 1)
            const int lprv = CW / 8, rpiv = 64 / lprv, niv = (U::NMAX + rpiv - 1) / rpiv;
            const uint32_t vs = lds_address(&sm.Vs[0]);
            for (int j = 0; j < niv; ++j) {
                const int row = j * rpiv + lane / lprv;
                const int node = row < N ? row : N - 1;
                const uint16_t* src = static_cast<const uint16_t*>(a.v) +
                                      ((static_cast<size_t>(id.b) * N + node) * a.Hv + id.h) * a.dv + id.j0 + (lane % lprv) * 8;
                copy16_to_lds(src, __builtin_amdgcn_readfirstlane(vs + j * 1024));
            }
        }
    } else {
        // B operand columns: c < N -> k_c, N <= c < 2N -> q_{c-N}, beyond -> zero.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int c = nt * 16 + l16;
            const bool isk = c < N;
            const bool valid = c < 2 * N;
            const int node = valid ? (isk ? c : c - N) : 0;
            const size_t rowoff = ((static_cast<size_t>(id.b) * N + node) * a.Hk + id.kh) * DK;
            const void* row = static_cast<const char*>(isk ? a.k : a.q) + rowoff * U::ESZ;
#pragma unroll
            for (int ks = 0; ks < U::KS; ++ks) load_row_operand<DK, BF16IN>(row, ks, g4, valid, in.bh[nt][ks], in.bo[nt][ks]);
        }
        // v rows of this unit's channels: 16 bytes per lane, several nodes per instruction.
        const int epl = 16 / U::ESZ;                    // elements per lane
        const int lpr = CW / epl;                       // lanes per node row
        const int rpi = 64 / lpr;                       // node rows per instruction
#pragma unroll
        for (int t = 0; t < U::VL; ++t) {
            const int row = t * rpi + lane / lpr, col = (lane % lpr) * epl;
            in.vraw[t] = make_uint4(0, 0, 0, 0);
            if (row < N)
                in.vraw[t] = *reinterpret_cast<const uint4*>(
                    static_cast<const char*>(a.v) +
                    (((static_cast<size_t>(id.b) * N + row) * a.Hv + id.h) * a.dv + id.j0 + col) * U::ESZ);
        }
    }
    const float* tile = a.state + (static_cast<size_t>(id.b) * a.Hv + id.h) * a.dv * DK + static_cast<size_t>(id.j0) * DK;
    load_state_tile<DK, MTX>(in.sa, tile, CW >> 4, l16, g4);
    if constexpr (BANK && BF16IN) {
        // The bank's first 32 entries, whatever its length (entries past it are masked when
        // applied; Emax >= 32, so every address is inside the bank).
        const size_t Emax = static_cast<size_t>(a.bank_Emax);
        const uint16_t* kb = static_cast<const uint16_t*>(a.bank_k) + (static_cast<size_t>(id.b) * a.Hk + id.kh) * DK * Emax;
#pragma unroll
        for (int t = 0; t < 2 * U::KS; ++t)
            if (t * 16 < DK) in.bk[t] = *reinterpret_cast<const uint4*>(kb + static_cast<size_t>(t * 16 + l16) * Emax + 8 * g4);
        const float* db = a.bank_delta + ((static_cast<size_t>(id.b) * a.Hv + id.h) * a.dv + id.j0) * Emax;
        const int MT = CW >> 4;
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) {
            const float* dr = db + static_cast<size_t>((mt < MT ? mt : MT - 1) * 16 + l16) * Emax + 8 * g4;
            in.bd[mt][0] = *reinterpret_cast<const float4*>(dr);
            in.bd[mt][1] = *reinterpret_cast<const float4*>(dr + 4);
        }
    }
    in.pL = 0;
    if (PEND && a.pend_path_len) {
        // Issued last (the entries were loaded first): the decays and the first four entries'
        // key and delta segments, so the other loads are already in flight.
        const int PN = a.pend_N;
        in.pL = clampi(((const __attribute__((address_space(4))) int32_t*)(a.pend_path_len))[id.b], 0, a.pend_Lmax);
        const int node = lane < a.pend_Lmax ? clampi(pentry, 0, PN - 1) : 0;
        in.pnode = node;
        const size_t gi = (static_cast<size_t>(id.b) * PN + node) * a.Hv + id.h;
        if constexpr (BF16IN) in.pgraw = static_cast<const uint16_t*>(a.pend_g)[gi];
        else in.pgraw = static_cast<const uint32_t*>(a.pend_g)[gi];
        if constexpr (!PRELOAD) return;             // apply_pending loads every entry itself
        // lane -> (entry q, segment sg): 8 keys and 4 channels; segments past dk or past the
        // unit's channels read zeros (every lane loads; the address is selected, not the value)
        const int q = lane >> 4, sg = lane & 15;
        const int nq = __shfl(node, q);
        const size_t ko = ((static_cast<size_t>(id.b) * PN + nq) * a.Hk + id.kh) * DK + sg * 8;
        const gfloat* zero = (const gfloat*)kZeros;
        if constexpr (BF16IN) {
            const gfloat* kp = sg * 8 < DK ? (const gfloat*)(static_cast<const uint16_t*>(a.pend_k) + ko) : zero;
            in.pkraw[0] = __builtin_bit_cast(uint4, *(const gf32x4*)kp);
        } else {
            const gfloat* kp = sg * 8 < DK ? (const gfloat*)(static_cast<const float*>(a.pend_k) + ko) : zero;
            const gfloat* kp4 = sg * 8 < DK ? kp + 4 : zero;
            in.pkraw[0] = __builtin_bit_cast(uint4, *(const gf32x4*)kp);
            in.pkraw[1] = __builtin_bit_cast(uint4, *(const gf32x4*)kp4);
        }
        const gfloat* dp = sg * 4 < CW ? (const gfloat*)(a.pend_delta + ((static_cast<size_t>(id.b) * PN + nq) * a.Hv + id.h) * a.dv +
                                                         id.j0 + sg * 4)
                                       : zero;
        const f32x4 d = *(const gf32x4*)dp;
        in.pdv = make_float4(d[0], d[1], d[2], d[3]);
    }
}

// This lane's matrix-core operand (K-step ks) of column c from the staged LDS rows: keys
// kfirst(ks, g4, 0..1) .. +3, i.e. 16-byte piece ks*4 + 2h + g4/2 of row c, half g4 & 1 of it,
// at its XOR-rotated slot.
template <int DK>
__device__ __forceinline__ bf16x8 staged_operand(const float* rows, int c, int ks, int g4) {
    constexpr int LPR = DK / 8;
    const uint8_t* row = reinterpret_cast<const uint8_t*>(rows) + c * DK * 2;
    uint2 w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int slot = ((ks * 4 + 2 * h + (g4 >> 1)) ^ (c & (LPR - 1))) & (LPR - 1);
        w[h] = make_uint2(0, 0);
        if (kvalid<DK>(ks, g4, h)) w[h] = *reinterpret_cast<const uint2*>(row + slot * 16 + (g4 & 1) * 8);
    }
    u32x4 u = {w[0].x, w[0].y, w[1].x, w[1].y};
    return __builtin_bit_cast(bf16x8, u);
}

// EARLY (a plain verify, whose state tile's loads were the unit's last): the walk
// coefficients, which need only the tree and the k/q rows, are built before the state
// contraction, while the tile is still arriving; the wave waits for the staged rows only.
template <int DK, int NT, bool BF16IN, bool STAGE, bool EARLY, int MTX>
__device__ __forceinline__ int compute_unit(const UnitIn<DK, NT, BF16IN, MTX>& in, VerifySmem<NT, BF16IN>& sm,
                                            const LinVerifyArgs& a, int unit, int ctiles, int CW, int lane,
                                            bool staged_wait_done) {
    using U = UnitIn<DK, NT, BF16IN, MTX>;
    constexpr int KS = U::KS, NMAX = U::NMAX, GT = (NMAX + 15) / 16;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int N = a.N;
    // staged rows: every copy of this wave has landed (also before an early exit, so that none
    // is still writing LDS when the workgroup ends).  After a commit the wait was made before
    // the commit's first store, so that this one does not wait for the stores too.  EARLY:
    // the state tile's loads, issued after the copies, may still be in flight (the count is
    // checked against the code by tests/test_codegen.py).
    if constexpr (STAGE) {
        if constexpr (EARLY) wait_vm<state_tile_loads<DK, MTX>()>();
        else if (!staged_wait_done) wait_all_vm();
    }
    const int n = clampi(in.nraw, 0, N);
    if (n <= 0) {
        if constexpr (EARLY) wait_all_vm();         // nothing left in flight when the wave ends
        return 0;
    }
    const int MT = CW >> 4;
    // the B operands: from the staged LDS rows, or loaded into registers with the unit's inputs
    bf16x8 opnd[STAGE ? NT : 1][KS];
    if constexpr (STAGE) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) opnd[nt][ks] = staged_operand<DK>(&sm.Cs[0][0], nt * 16 + l16, ks, g4);
    }
    auto bop = [&](int nt, int ks) -> const bf16x8& {
        if constexpr (STAGE) return opnd[nt][ks];
        else return in.bh[nt][ks];
    };
    // this lane's node (lane < n): parent, decay and write strength; zero beyond the tree
    const bool real = lane < n;
    // The node's raw parent, decay and strength pass through an empty asm statement here, so
    // the compiler cannot hoist their first use (and so the wait for them) to right after
    // their loads, ahead of the unit's other loads.
    uint32_t praw = static_cast<uint32_t>(in.praw), graw = in.graw, braw = in.braw;
    asm volatile("" : "+v"(praw), "+v"(graw), "+v"(braw));
    const int pme = real && lane > 0 ? clampi(static_cast<int>(praw), 0, lane - 1) : -1;
    float gme = 0.f, bme = 0.f;
    if constexpr (BF16IN) {
        gme = real ? bf16_bits_to_f32(static_cast<uint16_t>(graw)) : 0.f;
        bme = real ? bf16_bits_to_f32(static_cast<uint16_t>(braw)) : 0.f;
    } else {
        gme = real ? __uint_as_float(graw) : 0.f;
        bme = real ? __uint_as_float(braw) : 0.f;
    }

    // 1. tree metadata and v rows into LDS; the key Gram matrix.
    constexpr int GC = VerifySmem<NT, BF16IN>::GC;
    if (lane < NMAX) {
        sm.Gm[lane][GC] = gme;
        sm.Gm[lane][GC + 1] = __int_as_float(pme);
    }
    if constexpr (!STAGE) {
        const int epl = 16 / U::ESZ, lpr = CW / epl, rpi = 64 / lpr;
#pragma unroll
        for (int t = 0; t < U::VL; ++t) {
            const int row = t * rpi + lane / lpr, col = (lane % lpr) * epl;
            if (row < NMAX) *reinterpret_cast<uint4*>(&sm.Vs[(row * 64 + col) * U::ESZ]) = in.vraw[t];
        }
    }
#pragma unroll
    for (int gt = 0; gt < GT; ++gt) {
        if (gt * 16 >= n) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                acc = mfma16x16x32(bop(gt, ks), bop(nt, ks), acc);
                if constexpr (!BF16IN) {
                    acc = mfma16x16x32(in.bh[gt][ks], in.bo[nt][ks], acc);
                    acc = mfma16x16x32(in.bo[gt][ks], in.bh[nt][ks], acc);
                }
            }
            if (gt * 16 + 4 * g4 < NMAX) {          // rows past the largest tree are not kept
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.Gm[gt * 16 + 4 * g4 + e][nt * 16 + l16] = acc[e];
            }
        }
    }

    // 3. lane = node: ancestor set and the walk coefficients of node `lane`, written as rows
    //    of LDS so the walk reads four of them per broadcast load (after the Gram matrix;
    //    before the contraction when EARLY).
    auto coefficients = [&]() {
        if (lane < NMAX) {
            uint64_t am = 0;
            for (int m = pme; m >= 0; m = __float_as_int(sm.Gm[m][GC + 1])) am |= 1ull << m;
            const int li = real ? lane : 0;
            const float cdv = a.scale * sm.Gm[li][N + li];   // before the rows below replace Gm
            float run = 1.f;                            // product of g over ancestors below m
            float pu[NMAX], pw[NMAX];
#pragma unroll
            for (int m = NMAX - 1; m >= 0; --m) {
                const bool an = (am >> m) & 1ull;
                pu[m] = an ? -bme * gme * run * sm.Gm[m][li] : 0.f;
                pw[m] = an ? a.scale * gme * run * sm.Gm[m][N + li] : 0.f;
                run = an ? run * sm.Gm[m < n ? m : 0][GC] : run;
            }
#pragma unroll
            for (int m = 0; m < NMAX; m += 4) {
                *reinterpret_cast<float4*>(&sm.Pu[lane][m]) = make_float4(pu[m], pu[m + 1], pu[m + 2], pu[m + 3]);
                *reinterpret_cast<float4*>(&sm.Pw[lane][m]) = make_float4(pw[m], pw[m + 1], pw[m + 2], pw[m + 3]);
            }
            sm.cv[lane] = bme;                          // run is now G_parent
            sm.ca[lane] = bme * gme * run;
            sm.cb[lane] = a.scale * gme * run;
            sm.cd[lane] = cdv;
        }
        wave_lds_sync();
    };

    if constexpr (EARLY) {
        wave_lds_sync();                            // the Gram rows are in LDS
        coefficients();
    }

    // 2. S0^T x_c for the unit's channels.
#pragma unroll
    for (int mt = 0; mt < MTX; ++mt) {
        if (mt >= MT) continue;
        bf16x8 ah[KS], al[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) split_bf16(in.sa[mt][ks][0], in.sa[mt][ks][1], ah[ks], al[ks]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                acc = mfma16x16x32(ah[ks], bop(nt, ks), acc);
                acc = mfma16x16x32(al[ks], bop(nt, ks), acc);
                if constexpr (!BF16IN) acc = mfma16x16x32(ah[ks], in.bo[nt][ks], acc);
            }
            *reinterpret_cast<float4*>(cs_at(sm, nt * 16 + l16, mt * 16 + 4 * g4)) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
    wave_lds_sync();

    if constexpr (!EARLY) coefficients();
    const int vst = STAGE ? CW : 64;                // Vs row stride (elements)
    auto v_of = [&](int i) {
        if constexpr (BF16IN) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(sm.Vs)[i * vst + lane]);
        else return reinterpret_cast<const float*>(sm.Vs)[i * 64 + lane];
    };

    // 4. the delta walk: lane = value channel, nodes in index order.  Branch-free, with
    //    every LDS address a compile-time offset, so loads of later nodes overlap earlier
    //    arithmetic: nodes at or beyond n have zero coefficients and values (delta 0).
    float dr[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        float d0 = sm.cv[i] * v_of(i) - sm.ca[i] * *cs_at(sm, i, lane), d1 = 0.f;
#pragma unroll
        for (int m = 0; m + 1 < i; m += 2) {
            d0 = fmaf(sm.Pu[i][m], dr[m], d0);
            d1 = fmaf(sm.Pu[i][m + 1], dr[m + 1], d1);
        }
        if (i & 1) d0 = fmaf(sm.Pu[i][i - 1], dr[i - 1], d0);
        dr[i] = i < n ? d0 + d1 : 0.f;              // padding rows may hold anything
    }

    // 5. outputs, now that every delta is known (independent per node).
    float orow[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        float o0 = fmaf(sm.cb[i], *cs_at(sm, N + i, lane), sm.cd[i] * dr[i]), o1 = 0.f;
#pragma unroll
        for (int m = 0; m + 1 < i; m += 2) {
            o0 = fmaf(sm.Pw[i][m], dr[m], o0);
            o1 = fmaf(sm.Pw[i][m + 1], dr[m + 1], o1);
        }
        if (i & 1) o0 = fmaf(sm.Pw[i][i - 1], dr[i - 1], o0);
        orow[i] = o0 + o1;
    }
    // No LDS writes inside the walks (they would order every later read after them).  Both
    // walks are done with the rows: row i < n now holds delta_i, row N + i holds o_i (the
    // outputs go second, so they win where a padding row i >= N meets output row N + i - N).
#pragma unroll
    for (int i = 0; i < NMAX; ++i) *cs_at(sm, i, lane) = dr[i];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) *cs_at(sm, N + i, lane) = orow[i];
    wave_lds_sync();

    return n;
}

// The unit's deltas (Cs rows 0..n-1) and outputs (Cs rows N..N+n-1): 16-byte stores, four
// rows per instruction.  Issued after the next unit's inputs have landed, so the wait for
// those inputs never includes these stores.
template <int NT, bool BF16IN>
__device__ __forceinline__ void store_unit(VerifySmem<NT, BF16IN>& sm, const LinVerifyArgs& a, int unit, int n,
                                           int ctiles, int CW, int lane) {
    const int N = a.N;
    const UnitIds id = unit_ids(a, unit, ctiles, CW);
    const size_t rowbase = (static_cast<size_t>(id.b) * a.N * a.Hv + id.h) * a.dv + id.j0;
    const size_t ostep = static_cast<size_t>(a.Hv) * a.dv;
    const int c4 = (lane & 15) * 4;
    for (int r = lane >> 4; r < 2 * n; r += 4) {
        const bool isd = r < n;
        const int i = isd ? r : r - n;
        if (c4 < CW) {
            // written once and read by a later call: streamed past the caches (whole lines)
            float* dst = (isd ? a.cap_delta : a.out) + rowbase + i * ostep + c4;
            const float4 x = *reinterpret_cast<const float4*>(cs_at(sm, isd ? i : N + i, c4));
            __builtin_nontemporal_store(f32x4{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4*>(dst));
        }
    }
    wave_lds_sync();                                // LDS is reused by the next unit
}

// Stores the unit's state tile (held in the key order of kfirst) at its place in the state.
template <int DK, int MTX>
__device__ __forceinline__ void store_state_tile(const float4 (&sa)[MTX][(DK + 31) / 32][2], float* state, const UnitIds& id,
                                                 int Hv, int dv, int MT, int g4, int l16) {
    constexpr int KS = (DK + 31) / 32;
    float* tile = state + (static_cast<size_t>(id.b) * Hv + id.h) * dv * DK + static_cast<size_t>(id.j0) * DK;
#pragma unroll
    for (int mt = 0; mt < MTX; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                if (mt < MT && kvalid<DK>(ks, g4, h))
                    *reinterpret_cast<float4*>(tile + (mt * 16 + l16) * DK + kfirst(ks, g4, h)) = sa[mt][ks][h];
}

// Commits the previous step's accepted path a_0 .. a_{L-1} into the unit's state tile, in
// registers:  S <- G S + sum_l c_l k_{a_l} delta_{a_l}^T with G = prod_l g_{a_l} and
// c_l = prod_{l' > l} g_{a_l'} (the commit's formula).  Entries are staged four at a time
// through LDS that the unit's own computation overwrites later, and each group of four is
// added by fp32 matrix instructions.  `store`: the committed tile is stored.  `to_bank`: the path's entries are also written to the pending bank after its
// first `E0` entries -- the unit's channels of each captured delta, the decays (by the unit of
// channel tile 0) and the keys (by the first value head that reads the key head).
template <int DK, int NT, bool BF16IN, bool PRE = true, int MTX = 4>
__device__ __forceinline__ void apply_pending(UnitIn<DK, NT, BF16IN, MTX>& in, VerifySmem<NT, BF16IN>& sm,
                                              const LinVerifyArgs& a, int unit, int ctiles, int CW, int lane,
                                              bool store = true, bool to_bank = false, int E0 = 0) {
    constexpr int KS = (DK + 31) / 32;
    auto& sa = in.sa;
    const UnitIds id = unit_ids(a, unit, ctiles, CW);
    const int L = in.pL;
    if (L == 0) return;                             // nothing accepted: the state is unchanged
    const int g4 = lane >> 4, l16 = lane & 15, MT = CW >> 4;
    const int PN = a.pend_N;
    if (lane < L) {
        sm.pn[lane] = in.pnode;
        sm.pg[lane] = BF16IN ? bf16_bits_to_f32(static_cast<uint16_t>(in.pgraw)) : __uint_as_float(in.pgraw);
    }
    // the bank's slices this unit writes (wave-uniform)
    const size_t Emax = static_cast<size_t>(a.bank_Emax);
    const bool key_writer = to_bank && id.ct == 0 && id.h == (a.tiled ? id.kh : id.kh * a.group_div);
    float* bdel = to_bank ? a.bank_delta + ((static_cast<size_t>(id.b) * a.Hv + id.h) * a.dv + id.j0) * Emax + E0
                          : nullptr;
    if (to_bank && id.ct == 0 && lane < L)
        a.bank_g[(static_cast<size_t>(id.b) * a.Hv + id.h) * Emax + E0 + lane] =
            BF16IN ? bf16_bits_to_f32(static_cast<uint16_t>(in.pgraw)) : __uint_as_float(in.pgraw);
    wave_lds_sync();
    if (lane < L) {
        float c = 1.f;
        for (int l = lane + 1; l < L; ++l) c *= sm.pg[l];
        sm.pc[lane] = c;
    }
    wave_lds_sync();
    const float G = sm.pc[0] * sm.pg[0];
#pragma unroll
    for (int mt = 0; mt < MTX; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                sa[mt][ks][hh].x *= G; sa[mt][ks][hh].y *= G; sa[mt][ks][hh].z *= G; sa[mt][ks][hh].w *= G;
            }
    for (int c0 = 0; c0 < L; c0 += 4) {
        {   // lane -> (entry q, segment s): 8 key elements and 4 channels of c_l * delta_l
            const int q = lane >> 4, s = lane & 15, l = c0 + q;
            float kv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float4 draw = make_float4(0.f, 0.f, 0.f, 0.f);   // delta_l, this lane's 4 channels
            if (PRE && c0 == 0) {                   // loaded with the unit's inputs (as raw bits)
                const bool lv = l < L;              // entries past the path: zero (selects)
                if constexpr (BF16IN) {
                    const uint32_t u[4] = {in.pkraw[0].x, in.pkraw[0].y, in.pkraw[0].z, in.pkraw[0].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kv[2 * e] = lv ? __uint_as_float(u[e] << 16) : 0.f;
                        kv[2 * e + 1] = lv ? __uint_as_float(u[e] & 0xffff0000u) : 0.f;
                    }
                } else {
                    const uint32_t u[8] = {in.pkraw[0].x, in.pkraw[0].y, in.pkraw[0].z, in.pkraw[0].w,
                                           in.pkraw[1].x, in.pkraw[1].y, in.pkraw[1].z, in.pkraw[1].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) kv[e] = lv ? __uint_as_float(u[e]) : 0.f;
                }
                const float4 pd = in.pdv;
                draw = make_float4(lv ? pd.x : 0.f, lv ? pd.y : 0.f, lv ? pd.z : 0.f, lv ? pd.w : 0.f);
            } else {
                // every lane loads (clamped to entry L - 1 and to the first key / channel
                // segment) and then selects: no lane-dependent branch around the loads
                const int node = sm.pn[l < L ? l : L - 1];
                const bool kok = l < L && s * 8 < DK, dok = l < L && s * 4 < CW;
                const size_t ko = ((static_cast<size_t>(id.b) * PN + node) * a.Hk + id.kh) * DK + (s * 8 < DK ? s * 8 : 0);
                if constexpr (BF16IN) {
                    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.pend_k) + ko);
                    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kv[2 * e] = kok ? __uint_as_float(u[e] << 16) : 0.f;
                        kv[2 * e + 1] = kok ? __uint_as_float(u[e] & 0xffff0000u) : 0.f;
                    }
                } else {
                    const float4 x0 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.pend_k) + ko);
                    const float4 x1 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.pend_k) + ko + 4);
                    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) kv[e] = kok ? xv[e] : 0.f;
                }
                const float4 d = *reinterpret_cast<const float4*>(
                    a.pend_delta + ((static_cast<size_t>(id.b) * PN + node) * a.Hv + id.h) * a.dv + id.j0 +
                    (s * 4 < CW ? s * 4 : 0));
                if (dok) draw = d;
            }
            float4 dv4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (l < L) {
                const float cl = sm.pc[l];
                dv4 = make_float4(cl * draw.x, cl * draw.y, cl * draw.z, cl * draw.w);
            }
            if (to_bank && l < L) {
                // raw entries (c_l is applied when the bank is read), at entry E0 + l
                if (s * 4 < CW) {
                    bdel[(s * 4 + 0) * Emax + l] = draw.x;
                    bdel[(s * 4 + 1) * Emax + l] = draw.y;
                    bdel[(s * 4 + 2) * Emax + l] = draw.z;
                    bdel[(s * 4 + 3) * Emax + l] = draw.w;
                }
                if (key_writer && s * 8 < DK) {
                    using E = typename std::conditional<BF16IN, uint16_t, uint32_t>::type;
                    E* kb = static_cast<E*>(a.bank_k) + ((static_cast<size_t>(id.b) * a.Hk + id.kh) * DK + s * 8) * Emax +
                            E0 + l;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        if constexpr (BF16IN) kb[i * Emax] = static_cast<uint16_t>(__float_as_uint(kv[i]) >> 16);
                        else kb[i * Emax] = __float_as_uint(kv[i]);
                    }
                }
            }
            if (s * 8 < 128) {
                *reinterpret_cast<float4*>(&sm.pk[q][s * 8]) = make_float4(kv[0], kv[1], kv[2], kv[3]);
                *reinterpret_cast<float4*>(&sm.pk[q][s * 8 + 4]) = make_float4(kv[4], kv[5], kv[6], kv[7]);
            }
            *reinterpret_cast<float4*>(&sm.pd[q][s * 4]) = dv4;
        }
        wave_lds_sync();
        // The rank-4 update on the matrix cores in fp32, the tile itself the accumulator:
        // C[key][channel] += sum_q k_q[key] (c_q delta_q)[channel], one 16 x 16 x 4 instruction per
        // 16-key x 16-channel piece, lane group q holding entry q (entries past L were staged as
        // zeros).  Products and sums are fp32, as a fused multiply-add loop would give.
        float bd[MTX];
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) bd[mt] = sm.pd[g4][mt * 16 + l16];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (ks * 32 + 16 * h >= DK) continue;             // the key tile is past dk
                const float ak = sm.pk[g4][ks * 32 + 16 * h + l16];
#pragma unroll
                for (int mt = 0; mt < MTX; ++mt) {
                    float4& t = sa[mt][ks][h];
                    f32x4 acc = {t.x, t.y, t.z, t.w};
                    acc = mfma16x16x4f32(ak, bd[mt], acc);
                    t = make_float4(acc[0], acc[1], acc[2], acc[3]);
                }
            }
        wave_lds_sync();
    }
    if (store) store_state_tile<DK, MTX>(sa, a.state_out, id, a.Hv, a.dv, MT, g4, l16);
}

// Applies the pending bank's E entries (earlier steps' accepted paths, in order) to the unit's
// state tile in registers:  S <- G S + sum_e c_e k_e delta_e^T  with G = prod_e g_e and
// c_e = prod_{e' > e} g_e' -- the same update as committing each step's path in turn.  The
// bank is channel-major (bank_k[b][kh][key][e], bank_delta[b][h][channel][e]), so the rank-E
// update runs on the matrix cores with the tile itself as the accumulator: for every 16-key x
// 16-channel piece, C[key][ch] += K^T[key][e] (c . delta)[e][ch] over 32 entries per
// instruction.  bf16 inputs: the keys enter exactly and c_e delta_e as bf16 hi + lo (each term
// exact to about 2^-17 relative; the tolerance of a bf16 step is 2e-3).  fp32 inputs: keys and
// c_e delta_e are each split into three bf16 terms and the six products above 2^-24 relative
// are kept, so the update is as exact as fp32 arithmetic.
template <int DK, int NT, bool BF16IN, int MTX>
__device__ __forceinline__ void apply_bank(UnitIn<DK, NT, BF16IN, MTX>& in, VerifySmem<NT, BF16IN>& sm,
                                           const LinVerifyArgs& a, int unit, int ctiles, int CW, int lane) {
    constexpr int KS = (DK + 31) / 32;
    constexpr int ESZ = BF16IN ? 2 : 4;
    auto& sa = in.sa;
    const int E = in.bE;                            // in [0, Emax]
    const int Emax = a.bank_Emax;                   // a multiple of 32, at most 256
    if (E == 0) return;                             // an empty bank: the tile is the stored state
    const UnitIds id = unit_ids(a, unit, ctiles, CW);
    const int g4 = lane >> 4, l16 = lane & 15, MT = CW >> 4;
    // suffix products of the decays: lane l holds entries 4l .. 4l+3 (loaded with the unit's
    // inputs from clamped indices; decay 1 past E, a select, not a lane-dependent branch)
    float gl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) gl[i] = 4 * lane + i < E ? in.bg[i] : 1.f;
    float inc = (gl[0] * gl[1]) * (gl[2] * gl[3]);   // becomes the product over lanes >= this one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_down(inc, off);
        if (lane + off < 64) inc *= o;
    }
    float ex = __shfl_down(inc, 1);                 // product over the lanes after this one
    if (lane == 63) ex = 1.f;
    const float G = __shfl(inc, 0);
    float* cbuf = &sm.pk[0][0];                     // free until the pending path is staged
    *reinterpret_cast<float4*>(&cbuf[4 * lane]) =
        make_float4(gl[1] * gl[2] * gl[3] * ex, gl[2] * gl[3] * ex, gl[3] * ex, ex);
    wave_lds_sync();
#pragma unroll
    for (int mt = 0; mt < MTX; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                sa[mt][ks][h].x *= G; sa[mt][ks][h].y *= G; sa[mt][ks][h].z *= G; sa[mt][ks][h].w *= G;
            }
    const uint8_t* kb = static_cast<const uint8_t*>(a.bank_k) +
                        (static_cast<size_t>(id.b) * a.Hk + id.kh) * DK * Emax * ESZ;
    const float* db = a.bank_delta + ((static_cast<size_t>(id.b) * a.Hv + id.h) * a.dv + id.j0) * Emax;
    for (int e0 = 0; e0 < E; e0 += 32) {
        const int ef = e0 + 8 * g4;                 // first of this lane's eight entries
        const int nv = clampi(E - ef, 0, 8);        // how many of them are pending
        const float4 c0 = *reinterpret_cast<const float4*>(&cbuf[ef]), c1 = *reinterpret_cast<const float4*>(&cbuf[ef + 4]);
        // bf16 inputs: this chunk's key and delta operands, in in.bk / in.bd -- the first chunk's
        // were loaded with the unit's inputs, later ones are loaded here (e0 is wave-uniform: a
        // scalar branch)
        if constexpr (BF16IN) {
            if (e0 > 0) {
#pragma unroll
                for (int t = 0; t < 2 * KS; ++t)
                    if (t * 16 < DK)
                        in.bk[t] = *reinterpret_cast<const uint4*>(kb + (static_cast<size_t>(t * 16 + l16) * Emax + ef) * ESZ);
#pragma unroll
                for (int mt = 0; mt < MTX; ++mt) {
                    const float* dr = db + static_cast<size_t>((mt < MT ? mt : MT - 1) * 16 + l16) * Emax + ef;
                    in.bd[mt][0] = *reinterpret_cast<const float4*>(dr);
                    in.bd[mt][1] = *reinterpret_cast<const float4*>(dr + 4);
                }
            }
        }
        // Two passes of two 16-channel pieces each (fewer live operands; fp32 keys are
        // re-read from the cache in the second pass).
#pragma unroll
        for (int mp = 0; mp < MTX; mp += 2) {
            // B operands: c_e delta_e[channel] for entries ef .. ef+7 of channel mt*16 + l16
            // (fp32 inputs: a third term, bmid, see below)
            bf16x8 bhi[2], blo[2], bmid[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int mt = mp + m;
                float4 d0 = make_float4(0.f, 0.f, 0.f, 0.f), d1 = d0;
                if constexpr (BF16IN) {
                    // mt >= MT: a zero B operand, a zero tile.  (A select on values: a
                    // conditional between two float4 lvalues would select their addresses and
                    // keep the unit's arrays out of registers.)
                    const float4 x0 = in.bd[mt][0], x1 = in.bd[mt][1];
                    const bool ok = mt < MT;
                    d0 = make_float4(ok ? x0.x : 0.f, ok ? x0.y : 0.f, ok ? x0.z : 0.f, ok ? x0.w : 0.f);
                    d1 = make_float4(ok ? x1.x : 0.f, ok ? x1.y : 0.f, ok ? x1.z : 0.f, ok ? x1.w : 0.f);
                } else if (mt < MT) {
                    const float* dr = db + static_cast<size_t>(mt * 16 + l16) * Emax + ef;
                    d0 = *reinterpret_cast<const float4*>(dr);
                    d1 = *reinterpret_cast<const float4*>(dr + 4);
                }
                float4 m0, m1;                      // entries past E contribute exactly zero
                m0.x = 0 < nv ? c0.x * d0.x : 0.f; m0.y = 1 < nv ? c0.y * d0.y : 0.f;
                m0.z = 2 < nv ? c0.z * d0.z : 0.f; m0.w = 3 < nv ? c0.w * d0.w : 0.f;
                m1.x = 4 < nv ? c1.x * d1.x : 0.f; m1.y = 5 < nv ? c1.y * d1.y : 0.f;
                m1.z = 6 < nv ? c1.z * d1.z : 0.f; m1.w = 7 < nv ? c1.w * d1.w : 0.f;
                if constexpr (BF16IN) split_bf16(m0, m1, bhi[m], blo[m]);
                else split3_bf16(m0, m1, bhi[m], bmid[m], blo[m]);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (ks * 32 + 16 * h >= DK) continue;     // the key tile is past dk
                    // A operand: K^T[key][ef .. ef+7] for key ks*32 + 16h + l16
                    bf16x8 ahi, alo, amid;
                    if constexpr (BF16IN) {
                        const uint4 w = in.bk[2 * ks + h];
                        uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t keep = (2 * j < nv ? 0x0000ffffu : 0u) | (2 * j + 1 < nv ? 0xffff0000u : 0u);
                            u[j] &= keep;
                        }
                        u32x4 uv = {u[0], u[1], u[2], u[3]};
                        ahi = __builtin_bit_cast(bf16x8, uv);
                        alo = bf16x8{};
                    } else {
                        const uint8_t* kr = kb + (static_cast<size_t>(ks * 32 + 16 * h + l16) * Emax + ef) * ESZ;
                        float4 x0 = *reinterpret_cast<const float4*>(kr), x1 = *reinterpret_cast<const float4*>(kr + 16);
                        x0.x = 0 < nv ? x0.x : 0.f; x0.y = 1 < nv ? x0.y : 0.f; x0.z = 2 < nv ? x0.z : 0.f;
                        x0.w = 3 < nv ? x0.w : 0.f; x1.x = 4 < nv ? x1.x : 0.f; x1.y = 5 < nv ? x1.y : 0.f;
                        x1.z = 6 < nv ? x1.z : 0.f; x1.w = 7 < nv ? x1.w : 0.f;
                        split3_bf16(x0, x1, ahi, amid, alo);
                    }
#pragma unroll
                    for (int m = 0; m < 2; ++m) {   // mt >= MT: a zero B operand, a zero tile
                        float4& t = sa[mp + m][ks][h];
                        f32x4 acc = {t.x, t.y, t.z, t.w};
                        // smallest terms first; bf16 keys are exact, fp32 keys and every c delta
                        // are split, and the terms kept are those above 2^-24 relative
                        if constexpr (!BF16IN) {
                            acc = mfma16x16x32(alo, bhi[m], acc);
                            acc = mfma16x16x32(amid, bmid[m], acc);
                            acc = mfma16x16x32(ahi, blo[m], acc);
                            acc = mfma16x16x32(amid, bhi[m], acc);
                            acc = mfma16x16x32(ahi, bmid[m], acc);
                        } else {
                            acc = mfma16x16x32(ahi, blo[m], acc);
                        }
                        acc = mfma16x16x32(ahi, bhi[m], acc);
                        t = make_float4(acc[0], acc[1], acc[2], acc[3]);
                    }
                }
        }
    }
    wave_lds_sync();                                // cbuf is read before Cs is rewritten
}

// Bank mode: the committed state is the stored tile, then the bank's entries, then the
// previous step's path.  All three are applied in registers; then either the path is
// appended to the bank (the stored tile is left alone), or -- when it would not fit
// (E + L > Emax) or a flush is asked for -- the committed tile is stored and the bank's
// length is reset after the launch.  Every unit of a sequence takes the same decision.
template <int DK, int NT, bool BF16IN, int MTX>
__device__ __forceinline__ void commit_with_bank(UnitIn<DK, NT, BF16IN, MTX>& in, VerifySmem<NT, BF16IN>& sm,
                                                 const LinVerifyArgs& a, int unit, int ctiles, int CW, int lane) {
    const UnitIds id = unit_ids(a, unit, ctiles, CW);
    in.bE = clampi(((const __attribute__((address_space(4))) int32_t*)(a.bank_len))[id.b], 0, a.bank_Emax);
    const bool flush = a.bank_flush || in.pL > a.bank_Emax - in.bE;
    apply_bank<DK, NT, BF16IN, MTX>(in, sm, a, unit, ctiles, CW, lane);
    apply_pending<DK, NT, BF16IN, true, MTX>(in, sm, a, unit, ctiles, CW, lane, false, !flush, in.bE);
    if (flush && in.bE + in.pL > 0)
        store_state_tile<DK, MTX>(in.sa, a.state_out, id, a.Hv, a.dv, CW >> 4, lane >> 4, lane & 15);
}

// Waves per SIMD the verify kernel is compiled for: two, except for fp32 inputs with trees of
// 25..32 nodes, whose k/q operands (bf16 hi + lo, held in registers: fp32 rows are not staged)
// and 32 KiB of LDS per unit leave room for one.
template <int NT, bool BF16IN>
constexpr int verify_waves_per_simd() { return (!BF16IN && NT == 4) ? 1 : 2; }

// Verify for trees of up to 32 nodes: one unit per workgroup of one wave.  The hardware
// dispatcher keeps several units resident per CU (bf16 inputs: registers allow two waves per
// SIMD, the LDS footprint eight workgroups per CU up to 24 nodes), so one unit's memory
// latency hides behind another's arithmetic.
// BANK: the pending-bank call; COMMIT: the fused call (the previous step's path committed
// first); neither: the plain verify.  Separate instantiations, so that the plain verify's
// registers are not allocated for the commit's.
template <int DK, int NT, bool BF16IN, bool BANK, bool COMMIT>
__global__ __launch_bounds__(64, (verify_waves_per_simd<NT, BF16IN>())) void lin_verify_kernel(LinVerifyArgs a) {
    static_assert(NT <= 4, "register walk is for trees of up to 32 nodes");
    __shared__ VerifySmem<NT, BF16IN> sm;
    const int lane = threadIdx.x;
    const int CW = a.cw;
    const int ctiles = a.dv / CW;
    const int u = xcd_remap(blockIdx.x, gridDim.x);
    constexpr bool STAGE = BF16IN && kStageBf16;
    UnitIn<DK, NT, BF16IN, BANK ? kBankTiles : 4> in;
    load_unit<DK, NT, BF16IN, STAGE, true, BANK ? kBankTiles : 4, BANK, BANK || COMMIT>(in, sm, a, u, ctiles, CW, lane);
    constexpr bool commits = BANK || COMMIT;
    if (STAGE && commits) wait_all_vm();             // before the commit's stores (see compute_unit)
    if constexpr (BANK) commit_with_bank(in, sm, a, u, ctiles, CW, lane);
    else if constexpr (COMMIT) apply_pending<DK, NT, BF16IN>(in, sm, a, u, ctiles, CW, lane);
    const int n = compute_unit<DK, NT, BF16IN, STAGE, !commits>(in, sm, a, u, ctiles, CW, lane, commits);
    store_unit(sm, a, u, n, ctiles, CW, lane);
}

// Verify for trees of 33..64 nodes: the same unit, with up to 512 registers per lane (one
// wave per SIMD per workgroup slot) for the wider operand set and the longer register walk.
template <int DK, int NT, bool BF16IN, bool BANK, bool COMMIT>
__global__ __launch_bounds__(64, 1) void lin_verify_wide_kernel(LinVerifyArgs a) {
    static_assert(NT > 4 && NT <= 8, "wide register walk is for trees of 33..64 nodes");
    __shared__ VerifySmem<NT, BF16IN> sm;
    const int lane = threadIdx.x;
    const int CW = a.cw;
    const int ctiles = a.dv / CW;
    const int u = xcd_remap(blockIdx.x, gridDim.x);
    constexpr bool STAGE = BF16IN && kStageBf16;
    UnitIn<DK, NT, BF16IN, BANK ? kBankTiles : 4> in;
    load_unit<DK, NT, BF16IN, STAGE, true, BANK ? kBankTiles : 4, BANK, BANK || COMMIT>(in, sm, a, u, ctiles, CW, lane);
    constexpr bool commits = BANK || COMMIT;
    if (STAGE && commits) wait_all_vm();             // before the commit's stores (see compute_unit)
    if constexpr (BANK) commit_with_bank(in, sm, a, u, ctiles, CW, lane);
    else if constexpr (COMMIT) apply_pending<DK, NT, BF16IN>(in, sm, a, u, ctiles, CW, lane);
    const int n = compute_unit<DK, NT, BF16IN, STAGE, false>(in, sm, a, u, ctiles, CW, lane, commits);
    store_unit(sm, a, u, n, ctiles, CW, lane);
}

template <bool BF16IN>
__global__ __launch_bounds__(256) void lin_commit_kernel(LinCommitArgs a, int rows, int rtiles) {
    extern __shared__ __align__(16) float smem[];  // Kc[L][dk] then cd[L][rows]
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
    // the state is streamed once: non-temporal loads and stores keep it out of the caches
    f32x4* Sv = reinterpret_cast<f32x4*>(S);
    auto ld = [&](int v) {
        const f32x4 x = __builtin_nontemporal_load(&Sv[v]);
        return make_float4(x[0], x[1], x[2], x[3]);
    };
    if (t < nvec) s0 = ld(t);
    if (t + 256 < nvec) s1 = ld(t + 256);

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
        coef[L] = c;                                // product over the whole path
    }
    float* Kc = smem;
    float* cd = smem + L * dk;
    if constexpr (BF16IN) {
        // eight bf16 keys per 16-byte load (dk is a multiple of 16)
        for (int idx = t; idx < L * dk / 8; idx += 256) {
            const int m = idx / (dk / 8), r = (idx - m * (dk / 8)) * 8;
            const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) +
                                                          ((static_cast<size_t>(b) * a.N + ap[m]) * a.Hk + kh) * dk + r);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
            float* dst = &Kc[m * dk + r];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dst[2 * e] = __uint_as_float(u[e] << 16);
                dst[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
            }
        }
    } else {
        for (int idx = t; idx < L * dk; idx += 256) {
            const int m = idx / dk, r = idx - m * dk;
            Kc[idx] = load_scalar<BF16IN>(a.k, ((static_cast<size_t>(b) * a.N + ap[m]) * a.Hk + kh) * dk + r);
        }
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
        __builtin_nontemporal_store(f32x4{s.x, s.y, s.z, s.w}, &Sv[v]);
    };
    if (t < nvec) update(s0, t);
    if (t + 256 < nvec) update(s1, t + 256);
}

// A bank verify's length update, once every unit has read the old length: 0 where the verify
// flushed (a flush was asked for, or E + L > Emax), else E + L.
__global__ void lin_bank_len_kernel(int32_t* bank_len, const int32_t* path_len, int Lmax, int B, int Emax,
                                    int flush) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int E = clampi(bank_len[b], 0, Emax);
    const int L = clampi(path_len[b], 0, Lmax);
    bank_len[b] = flush || L > Emax - E ? 0 : E + L;
}

// Value channels per unit: 64 (one per lane of the walk), narrowed to 32 or 16 while the
// launch would give fewer than two units per CU.  A narrower unit still walks the whole tree
// (the walk's instruction count does not shrink) but loads, commits and contracts a
// proportionally smaller state tile, which shortens the critical path of small batches.
int verify_channels(int B, int Hv, int dv) {
    int cw = dv < 64 ? dv : 64;
    const long long target = 2LL * device_cu_count();
    while (cw > kMinChannels && static_cast<long long>(B) * Hv * (dv / cw) < target) cw /= 2;
    return cw;
}

template <int DK, int NT>
int launch_verify_dk_nt(const LinVerifyArgs& args, bool bf16, hipStream_t stream) {
    LinVerifyArgs a = args;
    a.cw = verify_channels(a.B, a.Hv, a.dv);
    if (a.bank_len && a.cw > 16 * kBankTiles) a.cw = 16 * kBankTiles;
    const int CW = a.cw;
    const long long units = static_cast<long long>(a.B) * a.Hv * (a.dv / CW);
    if (units > 0x7fffffffLL) return set_error(TV_ERANGE, "lin_tree_verify: too many work units (%lld)", units);
    dim3 block(64);
    dim3 grid(static_cast<unsigned>(units));
    const bool bank = a.bank_len != nullptr;
    const bool commit = a.pend_path_len != nullptr;
    if constexpr (NT <= 4) {
        if (bank) {
            if (bf16) hipLaunchKernelGGL((lin_verify_kernel<DK, NT, true, true, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((lin_verify_kernel<DK, NT, false, true, true>), grid, block, 0, stream, a);
        } else if (commit) {
            if (bf16) hipLaunchKernelGGL((lin_verify_kernel<DK, NT, true, false, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((lin_verify_kernel<DK, NT, false, false, true>), grid, block, 0, stream, a);
        } else {
            if (bf16) hipLaunchKernelGGL((lin_verify_kernel<DK, NT, true, false, false>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((lin_verify_kernel<DK, NT, false, false, false>), grid, block, 0, stream, a);
        }
    } else {
        if (bank) {
            if (bf16) hipLaunchKernelGGL((lin_verify_wide_kernel<DK, NT, true, true, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((lin_verify_wide_kernel<DK, NT, false, true, true>), grid, block, 0, stream, a);
        } else if (commit) {
            if (bf16) hipLaunchKernelGGL((lin_verify_wide_kernel<DK, NT, true, false, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((lin_verify_wide_kernel<DK, NT, false, false, true>), grid, block, 0, stream, a);
        } else {
            if (bf16) hipLaunchKernelGGL((lin_verify_wide_kernel<DK, NT, true, false, false>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((lin_verify_wide_kernel<DK, NT, false, false, false>), grid, block, 0, stream, a);
        }
    }
    return launch_status("lin_tree_verify");
}

template <int DK>
int launch_verify_dk(const LinVerifyArgs& a, bool bf16, hipStream_t stream) {
    const int cols = 2 * a.N;
    if (cols <= 16) return launch_verify_dk_nt<DK, 1>(a, bf16, stream);
    if (cols <= 32) return launch_verify_dk_nt<DK, 2>(a, bf16, stream);
    if (cols <= 48) return launch_verify_dk_nt<DK, 3>(a, bf16, stream);
    if (cols <= 64) return launch_verify_dk_nt<DK, 4>(a, bf16, stream);
    if (cols <= 80) return launch_verify_dk_nt<DK, 5>(a, bf16, stream);
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

int launch_lin_bank_len(int32_t* bank_len, const int32_t* path_len, int Lmax, int B, int Emax, int flush,
                        hipStream_t stream) {
    hipLaunchKernelGGL(lin_bank_len_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, bank_len, path_len, Lmax, B,
                       Emax, flush);
    return launch_status("lin_tree_verify_bank");
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
