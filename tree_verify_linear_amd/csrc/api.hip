// C entry points of libtreeverify.so: argument checks, error reporting, dispatch.
// Every check runs on the host before anything is enqueued; see include/tree_verify.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "tv_internal.h"

namespace tv {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = '\0'; }

int launch_status(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(TV_EDEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return TV_OK;
}

static bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

static bool head_size_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

static int check_common_lin(const char* fn, int B, int N, int Hk, int Hv, int dk, int dv, int dtype,
                            int head_group) {
    if (B <= 0 || N <= 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0)
        return set_error(TV_EINVAL, "%s: sizes must be positive (B=%d N=%d Hk=%d Hv=%d dk=%d dv=%d)", fn, B, N,
                         Hk, Hv, dk, dv);
    if (N > TV_MAX_NODES) return set_error(TV_ERANGE, "%s: N=%d exceeds %d tree nodes", fn, N, TV_MAX_NODES);
    if (Hv % Hk != 0) return set_error(TV_EINVAL, "%s: Hv=%d is not a multiple of Hk=%d", fn, Hv, Hk);
    if (!head_size_ok(dk) || !head_size_ok(dv))
        return set_error(TV_EUNSUPPORTED, "%s: dk=%d dv=%d not built; supported head sizes: 16, 32, 64, 128", fn,
                         dk, dv);
    if (dtype != TV_F32 && dtype != TV_BF16)
        return set_error(TV_EUNSUPPORTED, "%s: dtype %d not built; supported: TV_F32, TV_BF16", fn, dtype);
    if (head_group != TV_HEADS_CONTIGUOUS && head_group != TV_HEADS_TILED)
        return set_error(TV_EINVAL, "%s: head_group %d is not TV_HEADS_CONTIGUOUS or TV_HEADS_TILED", fn,
                         head_group);
    const double elems = static_cast<double>(B) * N * (Hv > Hk ? Hv : Hk) * (dk > dv ? dk : dv);
    if (elems > 9.0e15) return set_error(TV_ERANGE, "%s: tensor sizes overflow", fn);
    return TV_OK;
}

}  // namespace tv

using namespace tv;

extern "C" {

int tv_abi_version(void) { return TV_ABI_VERSION; }

const char* tv_last_error(void) { return g_err; }

int tv_check_metadata(const int32_t* parent, const int32_t* n_nodes, const int32_t* path, const int32_t* path_len,
                      int B, int N, int Lmax, int32_t* status, void* stream) {
    clear_error();
    const char* fn = "tv_check_metadata";
    if (!parent || !n_nodes || !status) return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if ((path == nullptr) != (path_len == nullptr))
        return set_error(TV_EINVAL, "%s: path and path_len must both be given or both be NULL", fn);
    if (B <= 0 || N <= 0) return set_error(TV_EINVAL, "%s: B=%d N=%d must be positive", fn, B, N);
    if (N > TV_MAX_NODES) return set_error(TV_ERANGE, "%s: N=%d exceeds %d tree nodes", fn, N, TV_MAX_NODES);
    if (path && (Lmax < 1 || Lmax > N)) return set_error(TV_ERANGE, "%s: Lmax=%d not in [1, N=%d]", fn, Lmax, N);
    return launch_check_metadata(parent, n_nodes, path, path_len, B, N, path ? Lmax : 1, status,
                                 static_cast<hipStream_t>(stream));
}
int tv_validate_tree(const int32_t* parent, const int32_t* n_nodes, int B, int N) {
    clear_error();
    if (!parent || !n_nodes) return set_error(TV_EINVAL, "tv_validate_tree: null pointer");
    if (B <= 0 || N <= 0) return set_error(TV_EINVAL, "tv_validate_tree: B=%d N=%d must be positive", B, N);
    if (N > TV_MAX_NODES) return set_error(TV_ERANGE, "tv_validate_tree: N=%d exceeds %d", N, TV_MAX_NODES);
    for (int b = 0; b < B; ++b) {
        const int n = n_nodes[b];
        if (n < 1 || n > N) return set_error(TV_ETOPO, "tv_validate_tree: n_nodes[%d]=%d not in [1, %d]", b, n, N);
        const int32_t* p = parent + static_cast<size_t>(b) * N;
        if (p[0] != -1) return set_error(TV_ETOPO, "tv_validate_tree: parent[%d][0]=%d, the root must be -1", b, p[0]);
        for (int i = 1; i < n; ++i)
            if (p[i] < 0 || p[i] >= i)
                return set_error(TV_ETOPO, "tv_validate_tree: parent[%d][%d]=%d is not an earlier node", b, i, p[i]);
    }
    return TV_OK;
}

int tv_validate_path(const int32_t* parent, const int32_t* n_nodes, const int32_t* path, const int32_t* path_len,
                     int B, int N, int Lmax) {
    const int st = tv_validate_tree(parent, n_nodes, B, N);
    if (st != TV_OK) return st;
    if (!path || !path_len) return set_error(TV_EINVAL, "tv_validate_path: null pointer");
    if (Lmax < 1 || Lmax > N) return set_error(TV_ERANGE, "tv_validate_path: Lmax=%d not in [1, N=%d]", Lmax, N);
    for (int b = 0; b < B; ++b) {
        const int L = path_len[b], n = n_nodes[b];
        if (L < 0 || L > Lmax || L > n)
            return set_error(TV_EPATH, "tv_validate_path: path_len[%d]=%d not in [0, min(Lmax, n_nodes)]", b, L);
        const int32_t* a = path + static_cast<size_t>(b) * Lmax;
        const int32_t* p = parent + static_cast<size_t>(b) * N;
        if (L > 0 && a[0] != 0) return set_error(TV_EPATH, "tv_validate_path: path[%d][0]=%d, must start at the root", b, a[0]);
        for (int m = 1; m < L; ++m)
            if (a[m] < 0 || a[m] >= n || p[a[m]] != a[m - 1])
                return set_error(TV_EPATH, "tv_validate_path: path[%d][%d]=%d is not a child of path[%d][%d]=%d", b, m,
                                 a[m], b, m - 1, a[m - 1]);
    }
    return TV_OK;
}

int lin_tree_verify(int B, int N, int Hk, int Hv, int dk, int dv, int dtype, int head_group, float scale,
                    const int32_t* parent, const int32_t* n_nodes, const void* q, const void* k, const void* v,
                    const void* g, const void* beta, const float* state, float* out, float* cap_delta,
                    void* stream) {
    clear_error();
    const char* fn = "lin_tree_verify";
    int st = check_common_lin(fn, B, N, Hk, Hv, dk, dv, dtype, head_group);
    if (st != TV_OK) return st;
    if (!std::isfinite(scale)) return set_error(TV_EINVAL, "%s: scale is not finite", fn);
    if (!parent || !n_nodes || !q || !k || !v || !g || !beta || !state || !out || !cap_delta)
        return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16) || !aligned(out, 16) ||
        !aligned(cap_delta, 16))
        return set_error(TV_EINVAL, "%s: q, k, v, state, out and cap_delta must be 16-byte aligned", fn);
    LinVerifyArgs a{B, N, Hk, Hv, dk, dv, Hv / Hk, head_group == TV_HEADS_TILED, scale, parent, n_nodes,
                    q, k, v, g, beta, state, out, cap_delta};
    return launch_lin_verify(a, dtype == TV_BF16, static_cast<hipStream_t>(stream));
}

int lin_tree_verify_commit(int B, int N, int Hk, int Hv, int dk, int dv, int dtype, int head_group, float scale,
                           const int32_t* parent, const int32_t* n_nodes, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, float* state, float* out, float* cap_delta, int prev_N,
                           const int32_t* prev_path, const int32_t* prev_path_len, int prev_Lmax, const void* prev_k,
                           const void* prev_g, const float* prev_cap_delta, void* stream) {
    clear_error();
    const char* fn = "lin_tree_verify_commit";
    int st = check_common_lin(fn, B, N, Hk, Hv, dk, dv, dtype, head_group);
    if (st != TV_OK) return st;
    if (prev_N < 1 || prev_N > TV_MAX_NODES) return set_error(TV_ERANGE, "%s: prev_N=%d not in [1, %d]", fn, prev_N, TV_MAX_NODES);
    if (prev_Lmax < 1 || prev_Lmax > prev_N)
        return set_error(TV_ERANGE, "%s: prev_Lmax=%d not in [1, prev_N=%d]", fn, prev_Lmax, prev_N);
    if (!std::isfinite(scale)) return set_error(TV_EINVAL, "%s: scale is not finite", fn);
    if (!parent || !n_nodes || !q || !k || !v || !g || !beta || !state || !out || !cap_delta || !prev_path ||
        !prev_path_len || !prev_k || !prev_g || !prev_cap_delta)
        return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16) || !aligned(out, 16) ||
        !aligned(cap_delta, 16) || !aligned(prev_k, 16) || !aligned(prev_cap_delta, 16))
        return set_error(TV_EINVAL, "%s: q, k, v, state, out, cap_delta, prev_k and prev_cap_delta must be 16-byte "
                         "aligned", fn);
    if (static_cast<const void*>(cap_delta) == static_cast<const void*>(prev_cap_delta))
        return set_error(TV_EINVAL, "%s: cap_delta and prev_cap_delta must be different buffers", fn);
    LinVerifyArgs a{B, N, Hk, Hv, dk, dv, Hv / Hk, head_group == TV_HEADS_TILED, scale, parent, n_nodes,
                    q, k, v, g, beta, state, out, cap_delta, prev_N, prev_Lmax, prev_path, prev_path_len, prev_k,
                    prev_g, prev_cap_delta, state};
    return launch_lin_verify(a, dtype == TV_BF16, static_cast<hipStream_t>(stream));
}

static int check_bank(const char* fn, int Emax) {
    if (Emax < 32 || Emax > TV_BANK_MAX_ENTRIES || Emax % 32 != 0)
        return set_error(TV_ERANGE, "%s: Emax=%d must be a multiple of 32 in [32, %d]", fn, Emax, TV_BANK_MAX_ENTRIES);
    return TV_OK;
}

static int check_prev(const char* fn, int prev_N, int prev_Lmax) {
    if (prev_N < 1 || prev_N > TV_MAX_NODES) return set_error(TV_ERANGE, "%s: prev_N=%d not in [1, %d]", fn, prev_N, TV_MAX_NODES);
    if (prev_Lmax < 1 || prev_Lmax > prev_N)
        return set_error(TV_ERANGE, "%s: prev_Lmax=%d not in [1, prev_N=%d]", fn, prev_Lmax, prev_N);
    return TV_OK;
}

static int check_bank_buffers(const char* fn, const void* bank_k, const float* bank_g, const float* bank_delta,
                              const int32_t* bank_len) {
    if (!bank_k || !bank_g || !bank_delta || !bank_len) return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(bank_k, 16) || !aligned(bank_delta, 16) || !aligned(bank_g, 4) || !aligned(bank_len, 4))
        return set_error(TV_EINVAL, "%s: bank_k and bank_delta must be 16-byte aligned (bank_g and bank_len 4-byte)",
                         fn);
    return TV_OK;
}

int lin_tree_verify_bank(int B, int N, int Hk, int Hv, int dk, int dv, int dtype, int head_group, float scale,
                         const int32_t* parent, const int32_t* n_nodes, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, float* state, float* out, float* cap_delta, int prev_N,
                         const int32_t* prev_path, const int32_t* prev_path_len, int prev_Lmax, const void* prev_k,
                         const void* prev_g, const float* prev_cap_delta, int Emax, int flush, void* bank_k,
                         float* bank_g, float* bank_delta, int32_t* bank_len, void* stream) {
    clear_error();
    const char* fn = "lin_tree_verify_bank";
    int st = check_common_lin(fn, B, N, Hk, Hv, dk, dv, dtype, head_group);
    if (st != TV_OK) return st;
    if ((st = check_prev(fn, prev_N, prev_Lmax)) != TV_OK) return st;
    if ((st = check_bank(fn, Emax)) != TV_OK) return st;
    if (flush != 0 && flush != 1) return set_error(TV_EINVAL, "%s: flush=%d is not 0 or 1", fn, flush);
    if (!std::isfinite(scale)) return set_error(TV_EINVAL, "%s: scale is not finite", fn);
    if (!parent || !n_nodes || !q || !k || !v || !g || !beta || !state || !out || !cap_delta || !prev_path ||
        !prev_path_len || !prev_k || !prev_g || !prev_cap_delta)
        return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if ((st = check_bank_buffers(fn, bank_k, bank_g, bank_delta, bank_len)) != TV_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16) || !aligned(out, 16) ||
        !aligned(cap_delta, 16) || !aligned(prev_k, 16) || !aligned(prev_cap_delta, 16))
        return set_error(TV_EINVAL, "%s: q, k, v, state, out, cap_delta, prev_k and prev_cap_delta must be 16-byte "
                         "aligned", fn);
    if (static_cast<const void*>(cap_delta) == static_cast<const void*>(prev_cap_delta))
        return set_error(TV_EINVAL, "%s: cap_delta and prev_cap_delta must be different buffers", fn);
    LinVerifyArgs a{B, N, Hk, Hv, dk, dv, Hv / Hk, head_group == TV_HEADS_TILED, scale, parent, n_nodes,
                    q, k, v, g, beta, state, out, cap_delta, prev_N, prev_Lmax, prev_path, prev_path_len, prev_k,
                    prev_g, prev_cap_delta, state};
    a.bank_Emax = Emax;
    a.bank_len = bank_len;
    a.bank_k = bank_k;
    a.bank_g = bank_g;
    a.bank_delta = bank_delta;
    a.bank_flush = flush;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = launch_lin_verify(a, dtype == TV_BF16, s)) != TV_OK) return st;
    return launch_lin_bank_len(bank_len, prev_path_len, prev_Lmax, B, Emax, flush, s);
}

int lin_bank_flush(int B, int Hk, int Hv, int dk, int dv, int dtype, int head_group, float* state, int prev_N,
                   const int32_t* prev_path, const int32_t* prev_path_len, int prev_Lmax, const void* prev_k,
                   const void* prev_g, const float* prev_cap_delta, int Emax, void* bank_k, float* bank_g,
                   float* bank_delta, int32_t* bank_len, void* stream) {
    clear_error();
    const char* fn = "lin_bank_flush";
    int st = check_common_lin(fn, B, 1, Hk, Hv, dk, dv, dtype, head_group);
    if (st != TV_OK) return st;
    if ((st = check_prev(fn, prev_N, prev_Lmax)) != TV_OK) return st;
    if ((st = check_bank(fn, Emax)) != TV_OK) return st;
    if (!state || !prev_path || !prev_path_len || !prev_k || !prev_g || !prev_cap_delta)
        return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if ((st = check_bank_buffers(fn, bank_k, bank_g, bank_delta, bank_len)) != TV_OK) return st;
    if (!aligned(state, 16) || !aligned(prev_k, 16) || !aligned(prev_cap_delta, 16))
        return set_error(TV_EINVAL, "%s: state, prev_k and prev_cap_delta must be 16-byte aligned", fn);
    // the bank verify with an empty tree (N = 0): no node input is read and nothing is written
    // but the committed state
    LinVerifyArgs a{B, 0, Hk, Hv, dk, dv, Hv / Hk, head_group == TV_HEADS_TILED, 1.f, nullptr, nullptr,
                    nullptr, nullptr, nullptr, nullptr, nullptr, state, nullptr, nullptr, prev_N, prev_Lmax, prev_path,
                    prev_path_len, prev_k, prev_g, prev_cap_delta, state};
    a.bank_Emax = Emax;
    a.bank_len = bank_len;
    a.bank_k = bank_k;
    a.bank_g = bank_g;
    a.bank_delta = bank_delta;
    a.bank_flush = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = launch_lin_verify(a, dtype == TV_BF16, s)) != TV_OK) return st;
    return launch_lin_bank_len(bank_len, prev_path_len, prev_Lmax, B, Emax, 1, s);
}

int lin_tree_commit(int B, int N, int Hk, int Hv, int dk, int dv, int dtype, int head_group, const int32_t* path,
                    const int32_t* path_len, int Lmax, const void* k, const void* g, const float* cap_delta,
                    float* state, void* stream) {
    clear_error();
    const char* fn = "lin_tree_commit";
    int st = check_common_lin(fn, B, N, Hk, Hv, dk, dv, dtype, head_group);
    if (st != TV_OK) return st;
    if (Lmax < 1 || Lmax > N) return set_error(TV_ERANGE, "%s: Lmax=%d not in [1, N=%d]", fn, Lmax, N);
    if (!path || !path_len || !k || !g || !cap_delta || !state) return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(state, 16) || !aligned(k, 16) || !aligned(cap_delta, 16))
        return set_error(TV_EINVAL, "%s: state, k and cap_delta must be 16-byte aligned", fn);
    LinCommitArgs a{B, N, Hk, Hv, dk, dv, Hv / Hk, head_group == TV_HEADS_TILED, Lmax, path, path_len, k, g,
                    cap_delta, state};
    return launch_lin_commit(a, dtype == TV_BF16, static_cast<hipStream_t>(stream));
}

size_t attn_tree_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int Tcap, int window) {
    clear_error();
    if (B <= 0 || N <= 0 || N > TV_MAX_NODES || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || Tcap <= 0 || window < 0)
        return 0;
    return attn_workspace_bytes(B, N, Hq, Hkv, D, Tcap, window);
}

}  // extern "C"

// Host checks shared by attn_tree_verify and attn_tree_verify_noalloc (everything but the
// workspace).
static int check_attn(const char* fn, int B, int N, int Hq, int Hkv, int D, int Tcap, int k_type, int v_type,
                      int window, float scale, const int32_t* parent, const int32_t* n_nodes, const int32_t* n_past,
                      const void* q, const void* k_cache, const void* v_cache, const float* out) {
    if (B <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Tcap <= 0)
        return set_error(TV_EINVAL, "%s: sizes must be positive (B=%d N=%d Hq=%d Hkv=%d D=%d Tcap=%d)", fn, B, N, Hq,
                         Hkv, D, Tcap);
    if (N > TV_MAX_NODES) return set_error(TV_ERANGE, "%s: N=%d exceeds %d tree nodes", fn, N, TV_MAX_NODES);
    if (Hq % Hkv) return set_error(TV_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
    if (Hq / Hkv > 8) return set_error(TV_EUNSUPPORTED, "%s: Hq/Hkv=%d query heads per KV head not built (<= 8)", fn, Hq / Hkv);
    if (D != 256) return set_error(TV_EUNSUPPORTED, "%s: D=%d not built; supported head size: 256", fn, D);
    const bool kt_ok = k_type == TV_Q8_0 || k_type == TV_Q4_0, vt_ok = v_type == TV_Q8_0 || v_type == TV_Q4_0;
    if (!kt_ok || !vt_ok)
        return set_error(TV_EUNSUPPORTED,
                         "%s: K/V type pair (%d, %d) not built; supported pairs: (Q8_0, Q8_0), (Q8_0, Q4_0), "
                         "(Q4_0, Q8_0), (Q4_0, Q4_0)", fn, k_type, v_type);
    if (window < 0) return set_error(TV_EINVAL, "%s: window=%d must be >= 0 (0 = full attention)", fn, window);
    if (!std::isfinite(scale)) return set_error(TV_EINVAL, "%s: scale is not finite", fn);
    if (!parent || !n_nodes || !n_past || !q || !k_cache || !v_cache || !out)
        return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return set_error(TV_EINVAL, "%s: q, the caches and out must be 16-byte aligned", fn);
    return TV_OK;
}

extern "C" {

int attn_tree_verify(int B, int N, int Hq, int Hkv, int D, int Tcap, int k_type, int v_type, int window, float scale,
                     const int32_t* parent, const int32_t* n_nodes, const int32_t* n_past, const void* q,
                     const void* k_cache, const void* v_cache, float* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream) {
    clear_error();
    const char* fn = "attn_tree_verify";
    const int st = check_attn(fn, B, N, Hq, Hkv, D, Tcap, k_type, v_type, window, scale, parent, n_nodes, n_past, q,
                              k_cache, v_cache, out);
    if (st != TV_OK) return st;
    if (!workspace) return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(workspace, 256)) return set_error(TV_EINVAL, "%s: workspace must be 256-byte aligned", fn);
    const size_t need = attn_workspace_bytes(B, N, Hq, Hkv, D, Tcap, window);
    if (need == 0) return set_error(TV_ERANGE, "%s: sizes overflow", fn);
    if (workspace_bytes < need)
        return set_error(TV_ERANGE, "%s: workspace of %zu bytes is smaller than the %zu needed", fn, workspace_bytes, need);
    AttnArgs a{B, N, Hq, Hkv, D, Tcap, k_type, v_type, window, scale, parent, n_nodes, n_past, q,
               static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache), out, lse, workspace};
    return launch_attn(a, static_cast<hipStream_t>(stream));
}

int attn_tree_verify_noalloc(int B, int N, int Hq, int Hkv, int D, int Tcap, int k_type, int v_type, int window,
                             float scale, const int32_t* parent, const int32_t* n_nodes, const int32_t* n_past,
                             const void* q, const void* k_cache, const void* v_cache, float* out, float* lse,
                             void* stream) {
    clear_error();
    const char* fn = "attn_tree_verify_noalloc";
    const int st = check_attn(fn, B, N, Hq, Hkv, D, Tcap, k_type, v_type, window, scale, parent, n_nodes, n_past, q,
                              k_cache, v_cache, out);
    if (st != TV_OK) return st;
    const size_t need = attn_workspace_bytes(B, N, Hq, Hkv, D, Tcap, window);
    if (need == 0) return set_error(TV_ERANGE, "%s: sizes overflow", fn);
    if (need > attn_scratch_capacity())
        return set_error(TV_ERANGE, "%s: these sizes need %zu bytes of split partials, more than the %zu bytes of "
                         "built-in scratch; use attn_tree_verify with a workspace", fn, need, attn_scratch_capacity());
    void* ws = attn_scratch_device_ptr();
    if (!ws) return TV_EDEVICE;                     // message set by the lookup
    AttnArgs a{B, N, Hq, Hkv, D, Tcap, k_type, v_type, window, scale, parent, n_nodes, n_past, q,
               static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache), out, lse, ws};
    return launch_attn(a, static_cast<hipStream_t>(stream));
}

size_t tree_accept_workspace_bytes(int B, int N, int V, int dtype) {
    clear_error();
    if (B <= 0 || N <= 0 || N > TV_MAX_NODES || V <= 0 || (dtype != TV_F32 && dtype != TV_BF16)) return 0;
    return accept_workspace_bytes(B, N, V, dtype == TV_BF16);
}

int tree_accept_greedy(int B, int N, int V, int dtype, const void* logits, const int32_t* parent,
                       const int32_t* n_nodes, const int32_t* tokens, int32_t* target, int32_t* path,
                       int32_t* path_len, int32_t* next_token, void* workspace, size_t workspace_bytes,
                       void* stream) {
    clear_error();
    const char* fn = "tree_accept_greedy";
    if (B <= 0 || N <= 0 || V <= 0)
        return set_error(TV_EINVAL, "%s: sizes must be positive (B=%d N=%d V=%d)", fn, B, N, V);
    if (N > TV_MAX_NODES) return set_error(TV_ERANGE, "%s: N=%d exceeds %d tree nodes", fn, N, TV_MAX_NODES);
    if (dtype != TV_F32 && dtype != TV_BF16)
        return set_error(TV_EUNSUPPORTED, "%s: dtype %d not built; supported: TV_F32, TV_BF16", fn, dtype);
    if (!logits || !parent || !n_nodes || !tokens || !target || !path || !path_len || !next_token || !workspace)
        return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(logits, 16) || !aligned(workspace, 256))
        return set_error(TV_EINVAL, "%s: logits must be 16-byte aligned, workspace 256-byte aligned", fn);
    if (static_cast<double>(B) * N * V > 9.0e15) return set_error(TV_ERANGE, "%s: tensor sizes overflow", fn);
    const size_t need = accept_workspace_bytes(B, N, V, dtype == TV_BF16);
    if (workspace_bytes < need)
        return set_error(TV_ERANGE, "%s: workspace of %zu bytes is smaller than the %zu needed", fn, workspace_bytes, need);
    AcceptArgs a{B, N, V, dtype == TV_BF16, logits, parent, n_nodes, tokens, target, path, path_len, next_token,
                 workspace};
    return launch_accept(a, static_cast<hipStream_t>(stream));
}

int kv_tree_compact(int B, int Hkv, int D, int Tcap, int k_type, int v_type, const int32_t* n_past,
                    const int32_t* path, const int32_t* path_len, int Lmax, void* k_cache, void* v_cache,
                    void* stream) {
    clear_error();
    const char* fn = "kv_tree_compact";
    if (B <= 0 || Hkv <= 0 || D <= 0 || Tcap <= 0)
        return set_error(TV_EINVAL, "%s: sizes must be positive (B=%d Hkv=%d D=%d Tcap=%d)", fn, B, Hkv, D, Tcap);
    if (D % 32 != 0 || D > 512)
        return set_error(TV_EUNSUPPORTED, "%s: D=%d not built; supported: multiples of 32 up to 512", fn, D);
    const bool kt_ok = k_type == TV_Q8_0 || k_type == TV_Q4_0, vt_ok = v_type == TV_Q8_0 || v_type == TV_Q4_0;
    if (!kt_ok || !vt_ok)
        return set_error(TV_EUNSUPPORTED,
                         "%s: K/V type pair (%d, %d) not built; supported pairs: (Q8_0, Q8_0), (Q8_0, Q4_0), "
                         "(Q4_0, Q8_0), (Q4_0, Q4_0)", fn, k_type, v_type);
    if (Lmax < 1 || Lmax > TV_MAX_NODES)
        return set_error(TV_ERANGE, "%s: Lmax=%d not in [1, %d]", fn, Lmax, TV_MAX_NODES);
    if (!n_past || !path || !path_len || !k_cache || !v_cache) return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
        return set_error(TV_EINVAL, "%s: the caches must be 16-byte aligned", fn);
    const int rk = D / 32 * (k_type == TV_Q8_0 ? 34 : 18), rv = D / 32 * (v_type == TV_Q8_0 ? 34 : 18);
    if (static_cast<double>(B) * Hkv * Tcap * (rk > rv ? rk : rv) > 9.0e15)
        return set_error(TV_ERANGE, "%s: cache sizes overflow", fn);
    KvCompactArgs a{B, Hkv, Tcap, Lmax, rk, rv, n_past, path, path_len, k_cache, v_cache};
    return launch_kv_compact(a, static_cast<hipStream_t>(stream));
}

static int check_conv(const char* fn, int B, int N, int C, int K, int dtype) {
    if (B <= 0 || N <= 0 || C <= 0 || K <= 0)
        return set_error(TV_EINVAL, "%s: sizes must be positive (B=%d N=%d C=%d K=%d)", fn, B, N, C, K);
    if (N > TV_MAX_NODES) return set_error(TV_ERANGE, "%s: N=%d exceeds %d tree nodes", fn, N, TV_MAX_NODES);
    if (K < 2 || K > 8) return set_error(TV_EUNSUPPORTED, "%s: K=%d not built; supported widths: 2..8", fn, K);
    if (C % 8) return set_error(TV_EUNSUPPORTED, "%s: C=%d not built; channels must be a multiple of 8", fn, C);
    if (dtype != TV_F32 && dtype != TV_BF16)
        return set_error(TV_EUNSUPPORTED, "%s: dtype %d not built; supported: TV_F32, TV_BF16", fn, dtype);
    if (static_cast<double>(B) * N * C > 9.0e15) return set_error(TV_ERANGE, "%s: tensor sizes overflow", fn);
    return TV_OK;
}

int conv_tree_verify(int B, int N, int C, int K, int dtype, int activation, const int32_t* parent,
                     const int32_t* n_nodes, const void* x, const float* weight, const float* conv_state, float* y,
                     void* stream) {
    clear_error();
    const char* fn = "conv_tree_verify";
    const int st = check_conv(fn, B, N, C, K, dtype);
    if (st != TV_OK) return st;
    if (activation != TV_ACT_NONE && activation != TV_ACT_SILU)
        return set_error(TV_EINVAL, "%s: activation %d is not TV_ACT_NONE or TV_ACT_SILU", fn, activation);
    if (!parent || !n_nodes || !x || !weight || !conv_state || !y) return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(x, 16) || !aligned(weight, 16) || !aligned(conv_state, 16) || !aligned(y, 16))
        return set_error(TV_EINVAL, "%s: x, weight, conv_state and y must be 16-byte aligned", fn);
    ConvVerifyArgs a{B, N, C, K, activation == TV_ACT_SILU, dtype == TV_BF16, parent, n_nodes, x, weight, conv_state, y};
    return launch_conv_verify(a, static_cast<hipStream_t>(stream));
}

int conv_tree_commit(int B, int N, int C, int K, int dtype, const int32_t* path, const int32_t* path_len, int Lmax,
                     const void* x, float* conv_state, void* stream) {
    clear_error();
    const char* fn = "conv_tree_commit";
    const int st = check_conv(fn, B, N, C, K, dtype);
    if (st != TV_OK) return st;
    if (Lmax < 1 || Lmax > N) return set_error(TV_ERANGE, "%s: Lmax=%d not in [1, N=%d]", fn, Lmax, N);
    if (!path || !path_len || !x || !conv_state) return set_error(TV_EINVAL, "%s: null pointer argument", fn);
    if (!aligned(x, 16) || !aligned(conv_state, 16))
        return set_error(TV_EINVAL, "%s: x and conv_state must be 16-byte aligned", fn);
    ConvCommitArgs a{B, N, C, K, Lmax, dtype == TV_BF16, path, path_len, x, conv_state};
    return launch_conv_commit(a, static_cast<hipStream_t>(stream));
}

}  // extern "C"
