// Internal declarations shared by the library's translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tree_verify.h"

namespace tv {

// ---------------------------------------------------------------- host-side error state
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int launch_status(const char* what);   // TV_OK or TV_EDEVICE from hipGetLastError
int device_cu_count();                // compute units of the current device (cached per device)

// ---------------------------------------------------------------- launchers (host)
struct LinVerifyArgs {
    int B, N, Hk, Hv, dk, dv, group_div, tiled;
    float scale;
    const int32_t* parent;
    const int32_t* n_nodes;
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* state;
    float* out;
    float* cap_delta;
    // The previous step's accepted path, committed into the state tile before this verify
    // (pend_path_len == nullptr: nothing pending, the state is only read).
    int pend_N, pend_Lmax;
    const int32_t* pend_path;
    const int32_t* pend_path_len;
    const void* pend_k;
    const void* pend_g;
    const float* pend_delta;
    float* state_out;                 // == state when a commit is pending
    int cw;                           // value channels per work unit (set by the launcher)
    // A pending bank (earlier steps' accepted entries, channel-major; see lin_tree_verify_bank):
    // applied to each state tile before the pending path; the previous step's path is then
    // appended to it, or, when it would not fit or a flush is asked for, the whole committed
    // tile is stored and the bank emptied.
    int bank_Emax;                    // entries per bank (a multiple of 32, at most 256)
    const int32_t* bank_len;          // nullptr: no bank
    void* bank_k;                     // [B][Hk][dk][Emax] of the input type
    float* bank_g;                    // [B][Hv][Emax]
    float* bank_delta;                // [B][Hv][dv][Emax]
    int bank_flush;
};
int launch_lin_verify(const LinVerifyArgs& a, bool bf16, hipStream_t stream);

struct LinCommitArgs {
    int B, N, Hk, Hv, dk, dv, group_div, tiled, Lmax;
    const int32_t* path;
    const int32_t* path_len;
    const void* k;
    const void* g;
    const float* cap_delta;
    float* state;
};
int launch_lin_commit(const LinCommitArgs& a, bool bf16, hipStream_t stream);

// After a bank verify: each bank's new length (0 where the verify flushed, else E + L).
int launch_lin_bank_len(int32_t* bank_len, const int32_t* path_len, int Lmax, int B, int Emax, int flush,
                        hipStream_t stream);

struct AttnArgs {
    int B, N, Hq, Hkv, D, Tcap, k_type, v_type, window;
    float scale;
    const int32_t* parent;
    const int32_t* n_nodes;
    const int32_t* n_past;
    const void* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    float* out;
    float* lse;
    void* workspace;
};
size_t attn_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int Tcap, int window);
int launch_attn(const AttnArgs& a, hipStream_t stream);
size_t attn_scratch_capacity();       // bytes of the library's own split-partial scratch
void* attn_scratch_device_ptr();      // its address on the current device (nullptr + error on failure)

struct AcceptArgs {
    int B, N, V;
    bool bf16;
    const void* logits;
    const int32_t* parent;
    const int32_t* n_nodes;
    const int32_t* tokens;
    int32_t* target;
    int32_t* path;
    int32_t* path_len;
    int32_t* next_token;
    void* workspace;
};
int accept_chunks(int V, bool bf16);
size_t accept_workspace_bytes(int B, int N, int V, bool bf16);
int launch_accept(const AcceptArgs& a, hipStream_t stream);

int launch_check_metadata(const int32_t* parent, const int32_t* n_nodes, const int32_t* path, const int32_t* path_len,
                          int B, int N, int Lmax, int32_t* status, hipStream_t stream);

struct KvCompactArgs {
    int B, Hkv, Tcap, Lmax, rk, rv;
    const int32_t* n_past;
    const int32_t* path;
    const int32_t* path_len;
    void* k_cache;
    void* v_cache;
};
int launch_kv_compact(const KvCompactArgs& a, hipStream_t stream);

struct ConvVerifyArgs {
    int B, N, C, K, silu;
    bool bf16;
    const int32_t* parent;
    const int32_t* n_nodes;
    const void* x;
    const float* weight;
    const float* state;
    float* y;
};
int launch_conv_verify(const ConvVerifyArgs& a, hipStream_t stream);

struct ConvCommitArgs {
    int B, N, C, K, Lmax;
    bool bf16;
    const int32_t* path;
    const int32_t* path_len;
    const void* x;
    float* state;
};
int launch_conv_commit(const ConvCommitArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- device helpers
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
// Consecutive workgroup ids are dealt round-robin to the 8 XCDs (each with its own L2).
// Remap so that every XCD works through one contiguous range of work units: units that
// share inputs (neighbouring heads of one sequence) then share an L2.  Bijective for any
// total.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
    constexpr int kXcd = 8;
    const int q = total / kXcd, r = total % kXcd;
    const int x = wg % kXcd, idx = wg / kXcd;
    return x * q + (x < r ? x : r) + idx;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Wait until at most N of this wave's vector memory operations (loads, stores and
// global-to-LDS copies) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One direct global-to-LDS copy instruction: lane l moves the 16 bytes at its `src` to LDS
// byte address lds + 16 l (lds is wave-uniform, passed in M0).  Written as a statement of its
// own so that the compiler neither waits for it before unrelated LDS accesses nor assumes it
// complete: the caller waits for it explicitly (wait_vm) before reading what it wrote.
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}
#endif

}  // namespace tv
