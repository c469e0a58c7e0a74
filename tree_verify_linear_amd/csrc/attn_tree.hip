// Tree-masked softmax attention over a Q8_0 / Q4_0 KV cache, gfx950.
//
// Method ("Luce DFlash" README, "How it works": one target forward verifies the whole draft
// tree through a causal mask derived from parent pointers; "Architecture note": 24 query
// heads share 4 KV heads of length 256; the FA-window flag: a sliding window, 0 = full;
// "Asymmetric K/V quantization": K and V each Q8_0 or Q4_0).  Query node i sits at position
// T + depth(i); it sees committed slot t iff window == 0 or T + depth(i) - t < window, and
// tree slot T + j iff j is on its root path and (window == 0 or depth(i) - depth(j) < window).
//
// Work unit: (sequence, KV head, block of <= 144 rows, KV split).  The rows are the (node,
// query head) pairs that share the KV head -- 22 nodes x 6 heads = 132 rows, 9 row tiles of
// 16 -- so every K/V byte is read from HBM once per split and reused by all of them.
//
// Layout of the work inside a workgroup (8 waves, two per SIMD, in two roles):
//   * K/V slot tiles (32 slots, one contiguous run of rows each) are copied raw from HBM into
//     rings of LDS slots by direct global-to-LDS loads, K three tiles and V two tiles ahead of
//     their first use, so several tiles per CU are in flight without holding registers.
//   * Queries are pre-scaled per row by a power of two 2^-e (the row's largest magnitude lands
//     in [2^14, 2^15)), so every bf16 query converts to fp16 exactly whatever its range; 2^e
//     is folded into the row's score scale.
//   * K enters the matrix cores as exact integers: one tile step ahead, the scoring waves
//     convert the raw Q8_0 / Q4_0 codes into fp16 integers in the QK operand layout (plus
//     each block's fp16 scale as fp32).  The QK^T product of each 32-element block is one
//     v_mfma_f32_16x16x32_f16 (K integers x Q), and the block's per-slot scale is applied to
//     the fp32 result: scores are exact products summed in fp32.
//   * Scoring waves (4): wave w owns row tiles w and w + 4 over the whole head dimension, and
//     wave 0 also row tile 8 (more than 128 rows; it then leaves its share of the K
//     conversion to waves 1..3), so no partial score leaves a wave.  The row
//     tiles of a sequence's rows are spread evenly over its row blocks.  Each wave masks its
//     rows, runs an online softmax in
//     the exp2 domain (the reference max moves only when a row max grows by more than 2^8; O
//     is then rescaled) and writes P as an fp16 pair hi + lo (P to about 2^-22) to LDS in the
//     PV A-operand layout (the score layout of S^T already is that layout).
//   * PV waves (4): PV wave w owns output columns 64w .. 64w+63 of all rows.  It dequantises
//     its columns of V exactly into fp16 hi/lo registers (d*q has at most 19 significant
//     bits, so hi = RN(d*q) and lo = d*q - hi) and accumulates
//     O += P_hi V_hi + P_hi V_lo + P_lo V_hi (the dropped P_lo V_lo is ~2^-22 relative), one
//     tile behind the scores.
//   * One barrier per tile step, one wave of each role per SIMD: in step k the scoring waves
//     score tile k, run its softmax and convert K of tile k+1 while the PV waves dequantise V
//     of tile k-1 and accumulate its PV products, so the matrix work of one role runs beside
//     the vector work of the other without a barrier between them.
//   * Each split writes unnormalised O, its running max and sum; a combine pass rescales and
//     sums the splits.  With a single split the kernel normalises and writes the output.
#include <cfloat>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "tv_internal.h"

// Split partials for callers that cannot allocate (attn_tree_verify_noalloc): one array per
// device, held for the life of the process.  Host code never passes this name to a kernel
// (on the host it is only a stand-in); it uses the device address looked up once per device.
static constexpr size_t kAttnScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

namespace tv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 256;
constexpr int TS = 32;                       // slots per tile
constexpr int WAVES = 8;                     // 4 scoring + 4 PV waves
constexpr int THREADS = 64 * WAVES;
constexpr int RTMAX = 9;                     // row tiles per row block
constexpr int OWNMAX = (RTMAX + 3) / 4;      // softmax tiles owned per scoring wave
constexpr int ROWS_PER_BLOCK = RTMAX * 16;   // 144
constexpr int MAXROW = 8 * 34;               // bytes of one slot's row (Q8_0, the larger)
// Raw K/V tiles are copied straight from HBM into rings of LDS slots by direct global-to-LDS
// loads (1 KiB per wave instruction), DK (K) and DV (V) tiles ahead of their first use.
#ifndef TV_DK
#define TV_DK 3
#endif
#ifndef TV_DV
#define TV_DV 2
#endif
constexpr int DK = TV_DK, DV = TV_DV;
constexpr int RK = DK + 2, RV = DV + 2;      // ring slots (see the schedule in attn_kernel)
constexpr int SLOT = (TS * MAXROW + 1023) / 1024 * 1024;   // 9 KiB: whole wave instructions
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS offset of a generic pointer into a __shared__ array: its low 32 bits (a generic LDS
// address is the shared aperture base plus the offset).  Taken this way rather than by a cast
// to the LDS address space, whose null check this compiler has been seen to miscompile
// ("operand has incorrect register class" on the aperture register) in some inlining contexts.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are complete, then the
// barrier.  Unlike __syncthreads it does not wait for outstanding global-to-LDS copies, which
// must stay in flight across barriers; each copy is waited for explicitly before the barrier
// that publishes it.  The signal fences keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0), other counters unchanged
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int TYPE>
struct Fmt {
    static constexpr int BLK = TYPE == TV_Q8_0 ? 34 : 18;   // bytes per 32-element block
    static constexpr int ROW = 8 * BLK;                      // bytes per slot (256 elements)
};

__device__ __forceinline__ _Float16 block_scale(const uint8_t* blk) {
    return __builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(blk));
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// The same with the alignment known only at run time (o % 4 is 0 or 2).
__device__ __forceinline__ uint32_t bytes4_rt(const uint8_t* row, int o) {
    const uint8_t* p = row + (o & ~3);
    return __builtin_amdgcn_alignbyte(lds_u32(p + 4), lds_u32(p), static_cast<uint32_t>(o & 3));
}

// Bytes 0, 1 (resp. 2, 3) of x placed under the fp16 exponent of 1024: the pair of fp16
// values 1024 + byte.
__device__ __forceinline__ f16x2 biased_lo(uint32_t x) {
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u));
}
__device__ __forceinline__ f16x2 biased_hi(uint32_t x) {
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u));
}

// Four quantised integers per dword -> biased byte form: Q8_0 flips the sign bit (q + 128),
// Q4_0 selects the low or high nibbles (q + 8).  `ints_bias` undoes the bias exactly.
template <int TYPE>
__device__ __forceinline__ uint32_t to_biased(uint32_t w, int nib_shift) {
    if constexpr (TYPE == TV_Q8_0) return w ^ 0x80808080u;
    else return (w >> nib_shift) & 0x0f0f0f0fu;
}
template <int TYPE>
constexpr float ints_bias() { return TYPE == TV_Q8_0 ? 1152.f : 1032.f; }

// Elements 8g .. 8g+7 of block kb of a slot row (the MFMA operand of lane group g) are 8 bytes
// (Q8_0) or the low or high nibbles of 8 bytes (Q4_0: elements 16.. are the high nibbles of
// bytes 0..).  The integer part of a block starts two bytes after its scale, so it is dword
// aligned in odd blocks and two bytes off in even ones (34- and 18-byte blocks alike): KRaw
// holds the aligned dwords covering those bytes, two or three, loaded ahead of the conversion.
template <bool ODD>
struct KRaw {
    uint32_t d[ODD ? 2 : 3];
};
template <int TYPE, bool ODD>
__device__ __forceinline__ KRaw<ODD> load_kraw(const uint8_t* row, int kb, int g) {
    const int o = TYPE == TV_Q8_0 ? 34 * kb + 2 + 8 * g : 18 * kb + 2 + 8 * (g & 1);
    KRaw<ODD> r;
    if constexpr (ODD) {
        r.d[0] = lds_u32(row + o);
        r.d[1] = lds_u32(row + o + 4);
    } else {
        r.d[0] = lds_u32(row + o - 2);
        r.d[1] = lds_u32(row + o + 2);
        r.d[2] = lds_u32(row + o + 6);
    }
    return r;
}
// Those elements as exact fp16 integers.  Block kb is even iff !ODD.
template <int TYPE, bool ODD>
__device__ __forceinline__ f16x8 kraw_ints8(const KRaw<ODD>& r, int g) {
    const int sh = TYPE == TV_Q8_0 ? 0 : (g >= 2 ? 4 : 0);
    uint32_t a, b;
    if constexpr (ODD) {
        a = r.d[0];
        b = r.d[1];
    } else {
        a = __builtin_amdgcn_alignbyte(r.d[1], r.d[0], 2u);
        b = __builtin_amdgcn_alignbyte(r.d[2], r.d[1], 2u);
    }
    const uint32_t w0 = to_biased<TYPE>(a, sh);
    const uint32_t w1 = to_biased<TYPE>(b, sh);
    const f16x2 bias = static_cast<_Float16>(ints_bias<TYPE>());
    const f16x2 p0 = biased_lo(w0) - bias, p1 = biased_hi(w0) - bias;
    const f16x2 p2 = biased_lo(w1) - bias, p3 = biased_hi(w1) - bias;
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Two probabilities as fp16 pairs: hi = RN(p) (packed convert) and lo = RN(p - hi), the
// residual taken in fp32 by v_fma_mix (hi widened exactly) and written straight into the
// halves of one register.
__device__ __forceinline__ void split_p2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const f16x2 h = {static_cast<_Float16>(p0), static_cast<_Float16>(p1)};
    hi = __builtin_bit_cast(uint32_t, h);
    uint32_t l;
    asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(l) : "v"(p0), "v"(hi));
    asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "+v"(l) : "v"(p1), "v"(hi));
    lo = l;
}

// d*q = hi + lo exactly (see the file comment): hi rounds the exact product once, the fused
// multiply-add returns the residual, which needs at most 8 significant bits.
template <typename V>
__device__ __forceinline__ void split_exact(const V& q, const V& d, V& hi, V& lo) {
    hi = d * q;
    lo = __builtin_elementwise_fma(d, q, -hi);
}

struct AttnLaunch {
    AttnArgs a;
    int G;              // query heads per KV head
    int rows;           // N * G
    int rows_pad;       // rows rounded up to row tiles of 16, per KV head
    int rblocks;        // row blocks (at most ROWS_PER_BLOCK rows each)
    int rtb;            // row tiles per row block (<= RTMAX; the last block may hold fewer)
    int nsplit;         // KV splits per (sequence, KV head)
    int chunk;          // slots per split (multiple of TS)
    float* opart;       // [B][Hkv][nsplit][rows_pad][D]
    float* mpart;       // [B][Hkv][nsplit][rows_pad]  running max (log2 domain)
    float* lpart;       // [B][Hkv][nsplit][rows_pad]  running sum
};

struct AttnSmem {
    __align__(16) f16x8 kop[2][2][8][64];                   // K integers in the QK operand layout
    __align__(16) float kd[2][8][TS];                       // K block scales [block][slot]
    __align__(16) f16x8 pbuf[2][RTMAX][64];                 // P hi in the PV operand layout
    __align__(16) f16x8 pbuf_lo[2][RTMAX][64];              // P lo = P - P hi, same layout
    __align__(16) float alpha[2][RTMAX][16];                // O rescale factor per row
    int grow[2][RTMAX];                                     // row tile needs a rescale
    float mfin[ROWS_PER_BLOCK], lfin[ROWS_PER_BLOCK];
    uint64_t anc[TV_MAX_NODES];
    int dep[TV_MAX_NODES];
    int par[TV_MAX_NODES];
};

// Softmax state of one owned row tile (this lane's row l16).
struct RowState {
    int node, dep, rlo;         // rlo: first committed slot the row sees
    uint64_t anc;
    float m, l;                 // running max (log2 domain, lane-group uniform), lane's sum
    float sl2;                  // log2(e) * |scale| * 2^e of the row's query pre-scale
    bool on;                    // the row exists
};


// One query row (bf16) as this lane's QK operand pieces: elements kb*32 + 8*g4 .. +7 for the 8
// blocks.  The row is pre-scaled by 2^-e, e chosen per row so that its largest magnitude lands
// in [2^14, 2^15): every bf16 value then converts to fp16 exactly (down to 2^-32 of the row's
// maximum), whatever the query's range, and 2^e is folded into the row's score scale.  The
// scale's sign is folded in too (exact), so the scores see a positive factor.
// (The row address is always valid -- rows past the tree read node 0's row -- so the loads are
// unconditional and absent rows are zeroed after them.)
__device__ __forceinline__ int load_qrow(const uint16_t* qrow, bool ok, int g4, uint4 (&w)[8]) {
    uint32_t mx = 0;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const uint4 x = *reinterpret_cast<const uint4*>(qrow + kb * 32 + 8 * g4);
        w[kb] = ok ? x : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const uint32_t u[4] = {w[kb].x, w[kb].y, w[kb].z, w[kb].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = (u[e] << 16) & 0x7fff0000u, hi = u[e] & 0x7fff0000u;
            mx = lo > mx ? lo : mx;
            mx = hi > mx ? hi : mx;
        }
    }
    // the row's maximum magnitude as fp32 bits (order of non-negative floats = order of bits)
    uint32_t t = __shfl_xor(mx, 16);
    mx = t > mx ? t : mx;
    t = __shfl_xor(mx, 32);
    mx = t > mx ? t : mx;
    const int E = static_cast<int>(mx >> 23) - 127;          // exponent of the maximum
    return (mx == 0u || E > 126) ? 0 : clampi(E - 14, -100, 100);
}
__device__ __forceinline__ f16x8 qrow_op(const uint4& w, int e, uint32_t qflip) {
    const float s = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);   // 2^-e
    const uint32_t u[4] = {w.x ^ qflip, w.y ^ qflip, w.z ^ qflip, w.w ^ qflip};
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = static_cast<_Float16>(__uint_as_float(u[i] << 16) * s);
        o[2 * i + 1] = static_cast<_Float16>(__uint_as_float(u[i] & 0xffff0000u) * s);
    }
    return o;
}

// FULL: every row block of the launch has all RTMAX row tiles (the last one more than 128
// rows), so the row-tile count is a constant and the tile loops have no branch between row
// tiles: the next row tile's operand loads can then be scheduled under the current MFMAs.
template <int KT, int VT, bool FULL>
__global__ __launch_bounds__(THREADS, 1) void attn_kernel(AttnLaunch L) {
    using KF = Fmt<KT>;
    using VF = Fmt<VT>;
    constexpr int KCH = TS * KF::ROW / 16, VCH = TS * VF::ROW / 16;    // 16-byte pieces per tile
    __shared__ AttnSmem sm;
    __shared__ __align__(1024) uint8_t ringk[RK][SLOT];     // raw K tiles (see dma_tile)
    __shared__ __align__(1024) uint8_t ringv[RV][SLOT];     // raw V tiles
    const AttnArgs& a = L.a;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (WAVES - 1);   // wave-uniform
    const bool scorer = wave < 4;
    const int wl = wave & 3;
    const int g4 = lane >> 4, l16 = lane & 15;

    int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int split = wg % L.nsplit;
    wg /= L.nsplit;
    const int rb = wg % L.rblocks;
    wg /= L.rblocks;
    const int kvh = wg % a.Hkv;
    const int b = wg / a.Hkv;

    const int N = a.N;
    const int n = clampi(a.n_nodes[b], 0, N);
    const int T = clampi(a.n_past[b], 0, a.Tcap - n);
    const int W = a.window;
    const int lo_b = W ? (T - W + 1 > 0 ? T - W + 1 : 0) : 0;   // first committed slot any node sees
    const int hi_b = T + n;
    const int s0 = lo_b + split * L.chunk;
    const int s1 = s0 + L.chunk < hi_b ? s0 + L.chunk : hi_b;
    const int ntiles = s1 > s0 ? (s1 - s0 + TS - 1) / TS : 0;
    const int rowbase = rb * L.rtb * 16;
    const int RT = FULL ? RTMAX : ((L.rows - rowbase + 15) / 16 < L.rtb ? (L.rows - rowbase + 15) / 16 : L.rtb);
    const size_t part = (static_cast<size_t>(b) * a.Hkv + kvh) * L.nsplit + split;

    // tree metadata (depth, ancestor sets) for this sequence
    if (tid < n) sm.par[tid] = tid == 0 ? -1 : clampi(a.parent[static_cast<size_t>(b) * N + tid], 0, tid - 1);
    __syncthreads();
    if (tid == 0) {
        for (int i = 0; i < n; ++i) {
            const int p = sm.par[i];
            sm.dep[i] = p < 0 ? 0 : sm.dep[p] + 1;
            sm.anc[i] = (p < 0 ? 0ull : sm.anc[p]) | (1ull << i);
        }
    }

    const uint8_t* kbase = a.k_cache + (static_cast<size_t>(b) * a.Hkv + kvh) * a.Tcap * KF::ROW;
    const uint8_t* vbase = a.v_cache + (static_cast<size_t>(b) * a.Hkv + kvh) * a.Tcap * VF::ROW;
    // Raw tiles in LDS rings, copied by direct global-to-LDS loads.  Instruction i of a tile
    // moves bytes 1024 i .. 1024 i + 1023 of the tile's contiguous run of rows (lane l: 16 bytes
    // at 1024 i + 16 l).  Pieces past the tile (the last instruction's upper half) or past the
    // cache end re-read the tile's last piece inside the cache: they land in the slot's padding
    // or in rows that are never visible (masked scores, zeroed V scales).  The PV waves copy K,
    // the scoring waves copy V, so no wave reads a ring it has copies in flight for: waits are
    // explicit (wait_vm before the barrier that publishes a tile), never implied by a read.
    constexpr int NIK = (TS * KF::ROW + 1023) / 1024, NIV = (TS * VF::ROW + 1023) / 1024;
    // Staging work of the scoring waves: the V copies (a quarter each) and the K conversion
    // (a quarter each, except that a wave 0 scoring three row tiles, with more than 128 rows,
    // leaves its K blocks to waves 1..3).  A wave issues copy instructions i = w, w + 4, ... of
    // each tile: the same count for every tile, so a fixed number of tiles still in flight is
    // a fixed vmcnt.
    const bool has8 = RT > 8;
    const int cntk = (NIK - wl + 3) / 4, cntv = (NIV - wl + 3) / 4;
    auto dma_tile = [&](const uint8_t* base, int rowbytes, int nch, uint8_t* slot, int tile) {
        const int t0 = s0 + tile * TS;
        const int last = (a.Tcap - t0 < TS ? a.Tcap - t0 : TS) * rowbytes / 16 - 1;   // t0 < Tcap
        const uint8_t* src = base + static_cast<size_t>(t0) * rowbytes;
        const int ni = (TS * rowbytes + 1023) / 1024;
        for (int i = wl; i < ni; i += 4) {
            int c = i * 64 + lane;
            c = c < nch ? c : nch - 1;
            c = c < last ? c : last;
            copy16_to_lds(src + c * 16, __builtin_amdgcn_readfirstlane(lds_offset(slot + i * 1024)));
        }
    };
    auto dma_k = [&](int tile) { dma_tile(kbase, KF::ROW, KCH, &ringk[tile % RK][0], tile); };
    auto dma_v = [&](int tile) { dma_tile(vbase, VF::ROW, VCH, &ringv[tile % RV][0], tile); };
    // Wait for a copied tile: `after` tiles copied since by this wave may stay in flight; a
    // count short of the steady state (the last tiles) waits for everything.
    auto wait_k = [&](int after) {
        if (after == DK) {
            if (cntk == 1) wait_vm<DK>();
            else if (cntk == 2) wait_vm<2 * DK>();
            else if (cntk == 3) wait_vm<3 * DK>();
            else wait_vm<0>();
        } else if (after == DK + 1) {
            if (cntk == 1) wait_vm<DK + 1>();
            else if (cntk == 2) wait_vm<2 * (DK + 1)>();
            else if (cntk == 3) wait_vm<3 * (DK + 1)>();
            else wait_vm<0>();
        } else {
            wait_vm<0>();
        }
    };
    auto wait_v = [&](int after) {
        if (after == DV) {
            if (cntv == 1) wait_vm<DV>();
            else if (cntv == 2) wait_vm<2 * DV>();
            else if (cntv == 3) wait_vm<3 * DV>();
            else wait_vm<0>();
        } else {
            wait_vm<0>();
        }
    };
    // K integers of tile `tile` (raw rows in its ring slot) into the QK operand buffer
    // kop[tile&1] and their block scales into kd[tile&1], NB consecutive blocks from kb0 (odd
    // iff ODD0) per wave: blocks 2w, 2w + 1, or with wave 0 not staging, {0,1,2}, {3,4,5},
    // {6,7} for waves 1..3.  Lane (g4, l16) of slot half st holds slot 16 st + l16, elements
    // 8 g4 .. 8 g4 + 7 of the block: exactly the MFMA A operand of that (half, block), so the
    // scoring waves read it back with one conflict-free 16-byte load per lane.  Every LDS read
    // of a conversion is issued before its first write (one round trip, not one per block);
    // lanes g4 < NB convert the scale of block kb0 + g4.
    auto convert_blocks = [&](int tile, int kb0, auto nbc, auto odd0c) {
        constexpr int NB = decltype(nbc)::value;
        constexpr bool ODD0 = decltype(odd0c)::value;
        const int buf = tile & 1;
        const int kbs = kb0 + (g4 < NB ? g4 : NB - 1);
        KRaw<ODD0> r0[2], r2[2];
        KRaw<!ODD0> r1[2];
        _Float16 sc[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const uint8_t* krow = &ringk[tile % RK][(16 * st + l16) * KF::ROW];
            r0[st] = load_kraw<KT, ODD0>(krow, kb0, g4);
            r1[st] = load_kraw<KT, !ODD0>(krow, kb0 + 1, g4);
            if constexpr (NB > 2) r2[st] = load_kraw<KT, ODD0>(krow, kb0 + 2, g4);
            sc[st] = block_scale(krow + kbs * KF::BLK);
        }
        // (the scales are used only by lanes g4 < NB; keep their loads with the others rather
        // than inside the branch that writes them)
        asm volatile("" : : "v"(sc[0]), "v"(sc[1]));
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            sm.kop[buf][st][kb0][lane] = kraw_ints8<KT, ODD0>(r0[st], g4);
            sm.kop[buf][st][kb0 + 1][lane] = kraw_ints8<KT, !ODD0>(r1[st], g4);
            if constexpr (NB > 2) sm.kop[buf][st][kb0 + 2][lane] = kraw_ints8<KT, ODD0>(r2[st], g4);
            if (g4 < NB) sm.kd[buf][kbs][16 * st + l16] = static_cast<float>(sc[st]);
        }
    };
    auto convert_k = [&](int tile) {
        using N2 = std::integral_constant<int, 2>;
        using N3 = std::integral_constant<int, 3>;
        using EV = std::integral_constant<bool, false>;
        using OD = std::integral_constant<bool, true>;
        if (!has8) convert_blocks(tile, 2 * wl, N2{}, EV{});
        else if (wl == 1) convert_blocks(tile, 0, N3{}, EV{});
        else if (wl == 2) convert_blocks(tile, 3, N3{}, OD{});
        else if (wl == 3) convert_blocks(tile, 6, N2{}, EV{});
    };

    // Prologue: K tiles 0 .. DK+1 and V tiles 0 .. DV-1 in flight; K tile 0 converted.
    const int nk0 = ntiles < DK + 2 ? ntiles : DK + 2, nv0 = ntiles < DV ? ntiles : DV;
    if (!scorer) {
        for (int t = 0; t < nk0; ++t) dma_k(t);
        wait_k(nk0 - 1);                                     // tile 0
    } else {
        for (int t = 0; t < nv0; ++t) dma_v(t);
    }
    lds_barrier();
    if (scorer && ntiles > 0) convert_k(0);
    if (!scorer) wait_k(nk0 - 2);                           // tile 1 (converted in step 0)
    lds_barrier();

    // Barrier sequence, identical in both roles: two above, one per tile step k = 0..ntiles,
    // one before the epilogue's output writes.
    if (scorer) {
        // ------------------------------------------------------------ scoring waves
        // Wave w scores row tiles w and w + 4 over the whole head dimension, and wave 0 also
        // row tile 8 (present only for more than 128 rows), so no partial score leaves a wave
        // and a tile's scores, softmax and P need no barrier inside the tile step.
        const uint32_t qflip = a.scale < 0.f ? 0x80008000u : 0u;
        const float sl2b = fabsf(a.scale) * kLog2e;
        f16x8 qop[OWNMAX][8];
        RowState rs[OWNMAX];
        int rlo_max[OWNMAX];
#pragma unroll
        for (int j = 0; j < OWNMAX; ++j) {
            rs[j].on = false;
            rs[j].node = rs[j].dep = rs[j].rlo = 0;
            rs[j].anc = 0ull;
            rs[j].m = -INFINITY;
            rs[j].l = 0.f;
            rs[j].sl2 = FLT_MIN;
        }
        auto setup_row = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int r = j < 2 ? wl + 4 * j : 8;
            const int row = rowbase + r * 16 + l16;
            const int node = row / L.G, hh = row - node * L.G;
            const bool on = r < RT && row < L.rows && node < n;
            const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                                   ((static_cast<size_t>(b) * N + (on ? node : 0)) * a.Hq + kvh * L.G + hh) * D;
            uint4 qw[8];
            const int qe = load_qrow(qrow, on, g4, qw);
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) qop[j][kb] = qrow_op(qw[kb], qe, qflip);
            rs[j].on = on;
            rs[j].node = on ? node : 0;
            rs[j].dep = on ? sm.dep[node] : 0;
            rs[j].anc = on ? sm.anc[node] : 0ull;
            rs[j].rlo = W ? T + rs[j].dep - W + 1 : 0;
            // |scale| * log2(e) * 2^e, kept positive (a zero scale becomes the smallest normal
            // float: the scores then vanish and the weights are uniform, as for scale 0)
            rs[j].sl2 = fmaxf(ldexpf(sl2b, qe), FLT_MIN);
        };
        setup_row(std::integral_constant<int, 0>{});
        setup_row(std::integral_constant<int, 1>{});
        if (RT > 8 && wl == 0) setup_row(std::integral_constant<int, 2>{});   // row tile 8
#pragma unroll
        for (int j = 0; j < OWNMAX; ++j) {
            // a committed tile is unmasked for this row tile when every row sees all its slots
            // (rows that do not exist are cleared separately)
            int rm = rs[j].on ? rs[j].rlo : -0x7fffffff;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const int t = __shfl_xor(rm, o);
                rm = t > rm ? t : rm;
            }
            rlo_max[j] = __builtin_amdgcn_readfirstlane(rm);
        }
        const bool own0 = wl < RT, own1 = wl + 4 < RT;       // wave-uniform

        // The tile loop of one scoring wave, specialised on what the wave holds so that the
        // inner loop has no branches: NJ row tiles among w, w + 4 (0..2) and, for wave 0, row
        // tile 8 (S8).  One barrier per tile step: scores and softmax of tile k, K conversion of
        // tile k + 1 and the copy of V tile k + DV, then the barrier that publishes P, K and V.
        auto scoring_loop = [&](auto njc, auto s8c) {
            constexpr int NJ = decltype(njc)::value;
            constexpr bool S8 = decltype(s8c)::value;
            constexpr int NS = NJ + (S8 ? 1 : 0);          // row tiles scored (row tile jj < 2: w + 4 jj; 2: 8)
            f32x4 own[OWNMAX][2];
            for (int k = 0; k <= ntiles; ++k) {
                if (k < ntiles && NS > 0) {
                    // scores of tile k.  Per slot half: the K integers of all 8 blocks against Q
                    // on the matrix cores (independent products, issued back to back), then each
                    // block's per-slot scale applied and summed in fp32.
                    const int buf = k & 1;
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        f32x4 sa[NS > 0 ? NS : 1];
#pragma unroll
                        for (int h = 0; h < 4; ++h) {                // blocks 2h, 2h+1
                            f16x8 ka[2];
                            f32x4 d4[2];
#pragma unroll
                            for (int x = 0; x < 2; ++x) {
                                ka[x] = sm.kop[buf][st][2 * h + x][lane];
                                d4[x] = *reinterpret_cast<const f32x4*>(&sm.kd[buf][2 * h + x][16 * st + 4 * g4]);
                            }
                            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                            f32x4 acc[NS > 0 ? NS : 1][2];
#pragma unroll
                            for (int x = 0; x < 2; ++x) {
#pragma unroll
                                for (int jj = 0; jj < NS; ++jj)
                                    acc[jj][x] = mfma_f16(ka[x], qop[jj][2 * h + x], z);
                            }
#pragma unroll
                            for (int jj = 0; jj < NS; ++jj) {
#pragma unroll
                                for (int x = 0; x < 2; ++x) {
                                    if (h == 0 && x == 0) sa[jj] = d4[0] * acc[jj][0];
                                    else sa[jj] += d4[x] * acc[jj][x];
                                }
                            }
                        }
#pragma unroll
                        for (int jj = 0; jj < NS; ++jj) own[jj][st] = sa[jj];
                    }
                }
                // K of tile k+1 into the other operand buffer (read by the scores of step k+1)
                if (k + 1 < ntiles) convert_k(k + 1);
                if (k < ntiles && NS > 0) {
                    // softmax of tile k for the row tiles scored (two, three for wave 0), which go
                    // through each step together, so their independent chains interleave
                    const int t0 = s0 + k * TS;
                    const int bufk = k & 1;
                    float x[NS > 0 ? NS : 1][8];        // unscaled scores
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x[jj][e] = own[jj][0][e];
                            x[jj][4 + e] = own[jj][1][e];
                        }
                    }
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj) {
                        const bool fast = t0 + TS <= (T < s1 ? T : s1) && t0 >= rlo_max[jj];
                        if (!fast) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const int slot = t0 + (e < 4 ? 4 * g4 + e : 16 + 4 * g4 + (e - 4));
                                bool vis = rs[jj].on && slot < s1;
                                if (slot < T) {
                                    vis = vis && slot >= rs[jj].rlo;
                                } else {
                                    const int jn = slot - T;     // < n <= 64 whenever slot < s1
                                    vis = vis && jn < TV_MAX_NODES && ((rs[jj].anc >> (jn & 63)) & 1ull) &&
                                          (W == 0 || rs[jj].dep - sm.dep[jn & 63] < W);
                                }
                                x[jj][e] = vis ? x[jj][e] : -INFINITY;
                            }
                        }
                    }
                    // (rows past the tree are not masked on unmasked tiles: their Q is zero, so
                    // their weights stay finite, and nothing reads their results)
                    float mt[NS > 0 ? NS : 1];
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj) {
                        mt[jj] = x[jj][0];
#pragma unroll
                        for (int e = 1; e < 8; ++e) mt[jj] = fmaxf(mt[jj], x[jj][e]);
                    }
                    // the row's 32 slots sit in the four lane groups: max over l, l^16, l^32
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj) {
                        const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt[jj]), __float_as_uint(mt[jj]), false, false);
                        mt[jj] = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
                    }
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj) {
                        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt[jj]), __float_as_uint(mt[jj]), false, false);
                        mt[jj] = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1])) * rs[jj].sl2;
                    }
#pragma unroll
                    for (int jj = 0; jj < NS; ++jj) {
                        const int r = jj < 2 ? wl + 4 * jj : 8;
                        // Lazy rescaling: P is taken against a reference max that moves only when
                        // the row max grows by more than 2^8 (so P <= 256); alpha is 1 otherwise.
                        const bool grow = mt[jj] > rs[jj].m + 8.f;
                        const bool anyg = __builtin_amdgcn_ballot_w64(grow) != 0;
                        const float mnew = grow ? mt[jj] : rs[jj].m;
                        const float al = rs[jj].m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rs[jj].m - mnew);
                        rs[jj].m = mnew;
                        const float m = mnew == -INFINITY ? 0.f : mnew;      // then every x is -inf
                        // P = hi + lo in fp16 (lo is the rounding residual of hi), so P enters
                        // the PV products to about 2^-22 relative
                        float pe[8];
                        float ps = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[jj][e], rs[jj].sl2, -m));
                            ps += pe[e];
                        }
                        uint32_t ph[4], pl[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) split_p2(pe[2 * e], pe[2 * e + 1], ph[e], pl[e]);
                        rs[jj].l = rs[jj].l * al + ps;
                        *reinterpret_cast<uint4*>(&sm.pbuf[bufk][r][lane]) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
                        *reinterpret_cast<uint4*>(&sm.pbuf_lo[bufk][r][lane]) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
                        if (g4 == 0) sm.alpha[bufk][r][l16] = al;          // row l16's factor
                        if (lane == 0) sm.grow[bufk][r] = anyg;
                    }
                }
                // copy V tile k+DV into the slot of tile k-2 (dequantised in step k-1; the PV
                // waves read tile k-1's slot during this step); V tile k is dequantised in the
                // next step
                if (k + DV < ntiles) dma_v(k + DV);
                wait_v(ntiles - 1 - k < DV ? ntiles - 1 - k : DV);
                lds_barrier();
            }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using BF = std::integral_constant<bool, false>;
        using BT = std::integral_constant<bool, true>;
        if (has8 && wl == 0) {
            scoring_loop(I2{}, BT{});
        } else if (own1) {
            scoring_loop(I2{}, BF{});
        } else if (own0) {
            scoring_loop(I1{}, BF{});              // small trees: one row tile
        } else {
            scoring_loop(I0{}, BF{});              // no row tile: staging and barriers only
        }
        // epilogue: row maxima and sums for the PV waves (and the split partials)
#pragma unroll
        for (int j = 0; j < OWNMAX; ++j) {
            const int r = j < 2 ? wl + 4 * j : 8;
            if (j == 2 && wl != 0) continue;
            float l = rs[j].l;
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            if (r < RT && g4 == 0) {
                sm.mfin[r * 16 + l16] = rs[j].m;
                sm.lfin[r * 16 + l16] = l;
                const int row = rowbase + r * 16 + l16;
                if (L.nsplit > 1 && row < L.rows) {
                    L.mpart[part * L.rows_pad + row] = rs[j].m;
                    L.lpart[part * L.rows_pad + row] = l;
                }
            }
        }
        __syncthreads();
    } else {
        // ------------------------------------------------------------ PV waves
        f32x4 oacc[RTMAX][4];
#pragma unroll
        for (int r = 0; r < RTMAX; ++r)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) oacc[r][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

        // O += P V for one row tile of tile k-1 (P hi/lo from LDS, V operands in registers)
        auto pv_rowtile = [&](auto rc, int bufp, const f16x8 (&bh)[4], const f16x8 (&bl)[4]) {
            constexpr int r = decltype(rc)::value;
            if (r >= RT) return;
            const f16x8 pa = sm.pbuf[bufp][r][lane];
            const f16x8 pl = sm.pbuf_lo[bufp][r][lane];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) oacc[r][jj] = mfma_f16(pa, bh[jj], oacc[r][jj]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) oacc[r][jj] = mfma_f16(pa, bl[jj], oacc[r][jj]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) oacc[r][jj] = mfma_f16(pl, bh[jj], oacc[r][jj]);
        };
        using R0 = std::integral_constant<int, 0>;
        using R1 = std::integral_constant<int, 1>;
        using R2 = std::integral_constant<int, 2>;
        using R3 = std::integral_constant<int, 3>;
        using R4 = std::integral_constant<int, 4>;
        using R5 = std::integral_constant<int, 5>;
        using R6 = std::integral_constant<int, 6>;
        using R7 = std::integral_constant<int, 7>;
        using R8 = std::integral_constant<int, 8>;
        for (int k = 0; k <= ntiles; ++k) {
            // this wave's 64 columns of V for tile k-1 as the PV B operands, fp16
            // hi/lo, straight from the raw rows into registers.  Column tile jj, lane (g4, l16)
            // holds column 4*l16 + jj of the wave's 64 (four adjacent columns = one dword per
            // slot) at the slots of the P operand's lane
            // group: 4g4 .. 4g4+3 and 16+4g4 .. 16+4g4+3.
            f16x8 bh[4], bl[4];
            if (k >= 1) {
                const uint8_t* raw = &ringv[(k - 1) % RV][0];
                const int kb = 2 * wl + (l16 >> 3), c4 = 4 * (l16 & 7);
                const int o = VT == TV_Q8_0 ? 34 * kb + 2 + c4 : 18 * kb + 2 + (c4 & 15);
                const int sh = c4 >= 16 ? 4 : 0;
                const f16x2 bias = static_cast<_Float16>(ints_bias<VT>());
                uint32_t w[8];
                _Float16 dd[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const uint8_t* row = raw + (t < 4 ? 4 * g4 + t : 12 + 4 * g4 + t) * VF::ROW;
                    w[t] = to_biased<VT>(bytes4_rt(row, o), sh);
                    dd[t] = block_scale(row + kb * VF::BLK);
                }
                // slots past the split's end hold bytes of no concern here (possibly not even
                // finite scales): their weights are zero, and a zero scale keeps 0 * V exact
                const int tv0 = s0 + (k - 1) * TS;
                if (tv0 + TS > s1) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int slot = tv0 + (t < 4 ? 4 * g4 + t : 12 + 4 * g4 + t);
                        dd[t] = slot < s1 ? dd[t] : static_cast<_Float16>(0.f);
                    }
                }
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    // u0 = [w_a.b0, w_b.b0, w_a.b1, w_b.b1], u1 = the same for bytes 2, 3
                    const uint32_t u0 = __builtin_amdgcn_perm(w[2 * pp + 1], w[2 * pp], 0x05010400u);
                    const uint32_t u1 = __builtin_amdgcn_perm(w[2 * pp + 1], w[2 * pp], 0x07030602u);
                    const f16x2 q[4] = {biased_lo(u0) - bias, biased_hi(u0) - bias, biased_lo(u1) - bias,
                                        biased_hi(u1) - bias};
                    const f16x2 d2 = {dd[2 * pp], dd[2 * pp + 1]};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        f16x2 h, l;
                        split_exact(q[c], d2, h, l);
                        bh[c][2 * pp] = h[0];
                        bh[c][2 * pp + 1] = h[1];
                        bl[c][2 * pp] = l[0];
                        bl[c][2 * pp + 1] = l[1];
                    }
                }
                // O rescale for tile k-1, then O += P V for its row tiles
                const int bufp = (k - 1) & 1;
                int anyg = 0;
#pragma unroll
                for (int r = 0; r < RTMAX; ++r) anyg |= r < RT ? sm.grow[bufp][r] : 0;
                if (anyg) {
#pragma unroll
                    for (int r = 0; r < RTMAX; ++r) {
                        if (r >= RT || !sm.grow[bufp][r]) continue;
                        const f32x4 al = *reinterpret_cast<const f32x4*>(&sm.alpha[bufp][r][4 * g4]);
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) oacc[r][jj] *= al;
                    }
                }
                pv_rowtile(R0{}, bufp, bh, bl);
                pv_rowtile(R1{}, bufp, bh, bl);
                pv_rowtile(R2{}, bufp, bh, bl);
                pv_rowtile(R3{}, bufp, bh, bl);
                pv_rowtile(R4{}, bufp, bh, bl);
                pv_rowtile(R5{}, bufp, bh, bl);
                pv_rowtile(R6{}, bufp, bh, bl);
                pv_rowtile(R7{}, bufp, bh, bl);
                pv_rowtile(R8{}, bufp, bh, bl);
            }
            // copy K tile k+2+DK (its slot's tile k was converted in step k-1); K tile k+2 is
            // converted in the next step
            if (k + 2 + DK < ntiles) dma_k(k + 2 + DK);
            wait_k(ntiles - 3 - k < DK ? ntiles - 3 - k : DK);
            lds_barrier();
        }
        __syncthreads();
        // epilogue: this wave's 64 columns of every row
#pragma unroll
        for (int r = 0; r < RTMAX; ++r) {
            if (r >= RT) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rl = r * 16 + 4 * g4 + e;
                const int row = rowbase + rl;
                const int node = row / L.G, hh = row - node * L.G;
                if (row >= L.rows || node >= n) continue;
                if (L.nsplit == 1) {
                    const float lsum = sm.lfin[rl];
                    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
                    float* orow = a.out + ((static_cast<size_t>(b) * N + node) * a.Hq + kvh * L.G + hh) * D + 64 * wl;
                    // written once and read by a later call: streamed past the caches (whole lines)
                    __builtin_nontemporal_store(f32x4{oacc[r][0][e] * inv, oacc[r][1][e] * inv, oacc[r][2][e] * inv,
                                                      oacc[r][3][e] * inv},
                                                reinterpret_cast<f32x4*>(orow + 4 * l16));
                    if (a.lse && wl == 0 && l16 == 0)
                        a.lse[(static_cast<size_t>(b) * N + node) * a.Hq + kvh * L.G + hh] =
                            (sm.mfin[rl] + log2f(lsum)) * kLn2;
                } else {
                    float* op = L.opart + (part * L.rows_pad + row) * D + 64 * wl;
                    *reinterpret_cast<float4*>(op + 4 * l16) =
                        make_float4(oacc[r][0][e], oacc[r][1][e], oacc[r][2][e], oacc[r][3][e]);
                }
            }
        }
    }
}

// Merges the splits of one row: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.  Lane t
// takes splits t, t + 64, ... and merges their (max, sum) pairs online, so one pass of loads
// gives the row's M and sum (one memory round trip up to 64 splits); the wave then broadcasts
// each split's weight from the lane that holds it and loads the partial outputs of up to 32
// splits at once (four columns per lane), so the merge costs two or three round trips.
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnLaunch L) {
    const AttnArgs& a = L.a;
    const int t = threadIdx.x;
    int wg = blockIdx.x;
    const int r = wg % L.rows;
    wg /= L.rows;
    const int kvh = wg % a.Hkv;
    const int b = wg / a.Hkv;
    const int node = r / L.G, hh = r - node * L.G;
    const size_t p0 = (static_cast<size_t>(b) * a.Hkv + kvh) * L.nsplit;
    const int ns = L.nsplit;
    // pass 1: this lane's splits, merged online (the first one is this lane's own split t)
    float mt = -INFINITY, lt = 0.f;
    for (int s = t; s < ns; s += 64) {
        const float ms = L.mpart[(p0 + s) * L.rows_pad + r];
        const float ls = L.lpart[(p0 + s) * L.rows_pad + r];
        if (ms == -INFINITY) continue;
        const float mn = fmaxf(mt, ms);
        lt = (mt == -INFINITY ? 0.f : lt * exp2f(mt - mn)) + ls * exp2f(ms - mn);
        mt = mn;
    }
    float M = mt;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float Lsum = M == -INFINITY || mt == -INFINITY ? 0.f : lt * exp2f(mt - M);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Lsum += __shfl_xor(Lsum, o);
    const int n = clampi(a.n_nodes[b], 0, a.N);
    if (node >= n) return;
    // weight of split t (lane t's first split); splits past 64 reload their max
    const float m0 = t < ns ? L.mpart[(p0 + t) * L.rows_pad + r] : -INFINITY;
    const float w0 = m0 == -INFINITY || M == -INFINITY ? 0.f : exp2f(m0 - M);
    float acc[D / 64];
#pragma unroll
    for (int k = 0; k < D / 64; ++k) acc[k] = 0.f;
    if (M != -INFINITY) {
        constexpr int U = 32;
        for (int s0 = 0; s0 < ns; s0 += U) {
            float ov[U][D / 64];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = s0 + u < ns ? s0 + u : ns - 1;
                const float* op = L.opart + ((p0 + s) * L.rows_pad + r) * D;
#pragma unroll
                for (int k = 0; k < D / 64; ++k) ov[u][k] = op[k * 64 + t];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = s0 + u;
                if (s >= ns) break;
                float w = __shfl(w0, s & 63);
                if (s >= 64) {
                    const float ms = L.mpart[(p0 + s) * L.rows_pad + r];
                    w = ms == -INFINITY ? 0.f : exp2f(ms - M);
                }
#pragma unroll
                for (int k = 0; k < D / 64; ++k) acc[k] += w * ov[u][k];
            }
        }
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    float* orow = a.out + ((static_cast<size_t>(b) * a.N + node) * a.Hq + kvh * L.G + hh) * D;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) orow[k * 64 + t] = acc[k] * inv;
    if (a.lse && t == 0)
        a.lse[(static_cast<size_t>(b) * a.N + node) * a.Hq + kvh * L.G + hh] = (M + log2f(Lsum)) * kLn2;
}

// Split policy: about one workgroup per CU (the LDS footprint allows one), splits of at least
// four tiles (below that the per-split set-up, partial writes and merge outweigh the extra
// parallelism).  Depends only on host-known sizes (n_past lives on the device), using the
// widest visible span.
struct SplitPlan {
    int G, rows, rows_pad, rblocks, rtb, nsplit, chunk;
};
SplitPlan plan_splits(int B, int N, int Hq, int Hkv, int Tcap, int window, int cus) {
    SplitPlan p;
    p.G = Hq / Hkv;
    p.rows = N * p.G;
    p.rows_pad = (p.rows + 15) / 16 * 16;
    p.rblocks = (p.rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    // the row tiles spread evenly over the blocks (240 rows: 8 + 7 tiles, not 9 + 6)
    p.rtb = (p.rows_pad / 16 + p.rblocks - 1) / p.rblocks;
    long long span = window ? static_cast<long long>(window) - 1 + N : Tcap;
    if (span > Tcap) span = Tcap;
    if (span < 1) span = 1;
    const long long units = static_cast<long long>(B) * Hkv * p.rblocks;
    long long ns = (cus + units - 1) / units;
    const long long maxns = (span + 4 * TS - 1) / (4 * TS);
    if (ns > maxns) ns = maxns;
    if (ns < 1) ns = 1;
    long long chunk = (span + ns - 1) / ns;
    chunk = (chunk + TS - 1) / TS * TS;
    p.nsplit = static_cast<int>((span + chunk - 1) / chunk);
    p.chunk = static_cast<int>(chunk);
    return p;
}

size_t workspace_for(const SplitPlan& p, int B, int Hkv, int D_) {
    if (p.nsplit <= 1) return 256;
    const size_t parts = static_cast<size_t>(B) * Hkv * p.nsplit * p.rows_pad;
    const size_t bytes = parts * (static_cast<size_t>(D_) + 2) * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

template <int KT, int VT>
void launch_pair(const AttnLaunch& L, unsigned wgs, hipStream_t stream) {
    const bool full = L.rtb == RTMAX && L.rows - (L.rblocks - 1) * ROWS_PER_BLOCK > (RTMAX - 1) * 16;
    if (full) hipLaunchKernelGGL((attn_kernel<KT, VT, true>), dim3(wgs), dim3(THREADS), 0, stream, L);
    else hipLaunchKernelGGL((attn_kernel<KT, VT, false>), dim3(wgs), dim3(THREADS), 0, stream, L);
}

}  // namespace

int device_cu_count() {
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

size_t attn_scratch_capacity() { return kAttnScratchBytes; }

void* attn_scratch_device_ptr() {
    static std::mutex mu;
    static void* ptrs[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        set_error(TV_EDEVICE, "attn_tree_verify_noalloc: no current HIP device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error(TV_EDEVICE, "attn_tree_verify_noalloc: scratch lookup failed on device %d: %s", dev,
                      hipGetErrorString(e));
            return nullptr;
        }
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

size_t attn_workspace_bytes(int B, int N, int Hq, int Hkv, int D_, int Tcap, int window) {
    const SplitPlan p = plan_splits(B, N, Hq, Hkv, Tcap, window, device_cu_count());
    return workspace_for(p, B, Hkv, D_);
}

int launch_attn(const AttnArgs& a, hipStream_t stream) {
    if (a.D != D) return set_error(TV_EUNSUPPORTED, "attn_tree_verify: D=%d not built", a.D);
    const SplitPlan p = plan_splits(a.B, a.N, a.Hq, a.Hkv, a.Tcap, a.window, device_cu_count());
    AttnLaunch L;
    L.a = a;
    L.G = p.G;
    L.rows = p.rows;
    L.rows_pad = p.rows_pad;
    L.rblocks = p.rblocks;
    L.rtb = p.rtb;
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
    const unsigned w = static_cast<unsigned>(wgs);
    if (a.k_type == TV_Q8_0 && a.v_type == TV_Q8_0) launch_pair<TV_Q8_0, TV_Q8_0>(L, w, stream);
    else if (a.k_type == TV_Q8_0 && a.v_type == TV_Q4_0) launch_pair<TV_Q8_0, TV_Q4_0>(L, w, stream);
    else if (a.k_type == TV_Q4_0 && a.v_type == TV_Q8_0) launch_pair<TV_Q4_0, TV_Q8_0>(L, w, stream);
    else if (a.k_type == TV_Q4_0 && a.v_type == TV_Q4_0) launch_pair<TV_Q4_0, TV_Q4_0>(L, w, stream);
    else return set_error(TV_EUNSUPPORTED, "attn_tree_verify: K/V type pair not built");
    if (p.nsplit > 1)
        hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<unsigned>(rowsall)), dim3(64), 0, stream, L);
    return launch_status("attn_tree_verify");
}

}  // namespace tv
