// C ABI entry points of the KDA library: argument validation and dispatch.
// Every check runs on the host before any HIP call, so a bad argument returns
// a status and enqueues nothing.
#include <stdint.h>
#include <string.h>

#include "kda_internal.hpp"

namespace {

// A C caller may pass any int where an enum is declared.  In C++, reading an
// enum object whose value lies outside the range its enumerators span is
// undefined, so every enum argument is first read as its raw integer and
// validated; only valid values are used as enums afterwards.
template <typename E>
int raw(const E& e)
{
    static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}
bool valid_mode(int m) { return m == KDA_GATE_CHANNEL || m == KDA_GATE_SCALAR || m == KDA_GATE_NONE; }
bool valid_dtype(int d) { return d == KDA_F32 || d == KDA_BF16; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool supported_dk(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_dv(int d) { return supported_dk(d) || d == 256; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }

kda_status check_common(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const void* o, int B, int T, int H, int Hqk, int Dk,
                        int Dv, int mode, int dtype, int o_dtype)
{
    if (B < 1 || H < 1 || T < 0) return KDA_ERROR_INVALID_VALUE;
    if (Hqk < 1 || Hqk > H || H % Hqk != 0) return KDA_ERROR_INVALID_VALUE;
    if (!valid_mode(mode) || !valid_dtype(dtype) || !valid_dtype(o_dtype))
        return KDA_ERROR_INVALID_VALUE;
    if (!supported_dk(Dk) || !supported_dv(Dv)) return KDA_ERROR_NOT_SUPPORTED;
    // sizes must fit the 64-bit index arithmetic of the kernels comfortably
    const double tok = (double)B * (double)T * (double)H;
    if (tok * (double)(Dk > Dv ? Dk : Dv) > 9.0e15) return KDA_ERROR_INVALID_VALUE;
    if ((double)B * H > 2.0e9) return KDA_ERROR_INVALID_VALUE;
    if (T > 0) {
        if (!q || !k || !v || !beta || !o) return KDA_ERROR_INVALID_VALUE;
        if (mode != KDA_GATE_NONE && !g) return KDA_ERROR_INVALID_VALUE;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(o))
            return KDA_ERROR_MISALIGNED;
        if (g && !aligned16(g)) return KDA_ERROR_MISALIGNED;
    }
    return KDA_SUCCESS;
}

}  // namespace

namespace kda {

// Every argument check of kda_chunk_fwd except those of the workspace, on
// the host, before any HIP call.
kda_status chunk_fwd_checks(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* initial_state,
                            const float* final_state, const void* o, int B, int T, int H, int Hqk,
                            int Dk, int Dv, int chunk, const kda_gate_mode& mode,
                            const kda_dtype& dtype, const kda_dtype& o_dtype, int prologue)
{
    if (prologue & ~KDA_PROLOGUE_ALL) return KDA_ERROR_INVALID_VALUE;
    kda_status st = check_common(q, k, v, g, beta, o, B, T, H, Hqk, Dk, Dv, raw(mode), raw(dtype),
                                 raw(o_dtype));
    if (st != KDA_SUCCESS) return st;
    if (!supported_chunk(chunk) || !chunk_fwd_supported(Dk, Dv, chunk, dtype))
        return KDA_ERROR_NOT_SUPPORTED;
    // chunk records and state workgroups are counted in 32-bit integers
    const double nrec = (double)B * H * ((T + chunk - 1) / chunk);
    if (nrec > 1073741824.0 || (double)B * H * (Dv / 16) + 64.0 > 2147483647.0)
        return KDA_ERROR_INVALID_VALUE;
    if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
        return KDA_ERROR_MISALIGNED;
    return KDA_SUCCESS;
}

}  // namespace kda

// Launch errors are read with hipGetLastError after each launch.  An error
// left on this thread by an earlier, unrelated runtime call (one the caller
// already recovered from) would be read there as well, so it is discarded
// before the entry point launches anything.
static inline void discard_stale_error() { (void)hipGetLastError(); }

extern "C" {

const char* kda_status_string(kda_status s)
{
    switch (raw(s)) {
        case KDA_SUCCESS: return "KDA_SUCCESS";
        case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
        case KDA_ERROR_NOT_SUPPORTED: return "KDA_ERROR_NOT_SUPPORTED";
        case KDA_ERROR_MISALIGNED: return "KDA_ERROR_MISALIGNED";
        case KDA_ERROR_WORKSPACE: return "KDA_ERROR_WORKSPACE";
        case KDA_ERROR_HIP: return "KDA_ERROR_HIP";
        case KDA_ERROR_SCRATCH: return "KDA_ERROR_SCRATCH";
    }
    return "KDA_ERROR_UNKNOWN";
}

int kda_version(void) { return 10300; }

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, float* state, void* o, int B, int T, int H,
                              int Hqk, int Dk, int Dv, float scale, kda_gate_mode mode,
                              kda_dtype dtype, kda_dtype o_dtype, int prologue, void* stream)
{
    if (prologue & ~KDA_PROLOGUE_ALL) return KDA_ERROR_INVALID_VALUE;
    kda_status st = check_common(q, k, v, g, beta, o, B, T, H, Hqk, Dk, Dv, raw(mode), raw(dtype),
                                 raw(o_dtype));
    if (st != KDA_SUCCESS) return st;
    if (T == 0) return KDA_SUCCESS;
    if (!state) return KDA_ERROR_INVALID_VALUE;
    if (!aligned16(state)) return KDA_ERROR_MISALIGNED;
    kda::RecArgs a{q, k, v, g, beta, state, o, B, T, H, Dk, Dv, Hqk, scale, mode, dtype, o_dtype, nullptr,
                   prologue};
    discard_stale_error();
    hipError_t e = kda::launch_recurrent(a, (hipStream_t)stream);
    return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
}

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv, int chunk,
                                    kda_gate_mode mode, kda_dtype dtype)
{
    (void)mode;
    if (B < 1 || H < 1 || T <= 0) return 0;
    if (!supported_dk(Dk) || !supported_dv(Dv) || !supported_chunk(chunk)) return 0;
    if (!valid_dtype(raw(dtype))) return 0;
    return kda::chunk_workspace_bytes(B, T, H, Dk, Dv, chunk, dtype);
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, float* final_state,
                         void* o, int B, int T, int H, int Hqk, int Dk, int Dv, int chunk,
                         float scale, kda_gate_mode mode, kda_dtype dtype, kda_dtype o_dtype,
                         int prologue, void* workspace, size_t workspace_bytes, void* stream)
{
    kda_status st = kda::chunk_fwd_checks(q, k, v, g, beta, initial_state, final_state, o, B, T,
                                          H, Hqk, Dk, Dv, chunk, mode, dtype, o_dtype, prologue);
    if (st != KDA_SUCCESS) return st;
    const size_t need = kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, chunk, mode, dtype);
    if (T > 0) {
        if (!workspace || workspace_bytes < need) return KDA_ERROR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return KDA_ERROR_MISALIGNED;
    }
    if (T == 0 && !final_state) return KDA_SUCCESS;
    kda::ChunkArgs a{q, k, v, g, beta, initial_state, final_state, o, B, T, H, Dk, Dv, chunk, Hqk,
                     scale, mode, dtype, o_dtype, workspace, workspace_bytes, nullptr, 0, prologue};
    discard_stale_error();
    hipError_t e = kda::launch_chunk(a, (hipStream_t)stream);
    return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
}

kda_status kda_recurrent_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, float* state, void* o, const int* cu_seqlens,
                                int N, int T, int H, int Hqk, int Dk, int Dv, float scale,
                                kda_gate_mode mode, kda_dtype dtype, kda_dtype o_dtype,
                                int prologue, void* stream)
{
    if (N < 0 || (prologue & ~KDA_PROLOGUE_ALL)) return KDA_ERROR_INVALID_VALUE;
    kda_status st = check_common(q, k, v, g, beta, o, 1, T, H, Hqk, Dk, Dv, raw(mode), raw(dtype),
                                 raw(o_dtype));
    if (st != KDA_SUCCESS) return st;
    if ((double)N * H > 2.0e9) return KDA_ERROR_INVALID_VALUE;
    if (N == 0 || T == 0) return KDA_SUCCESS;   // every sequence is empty: states unchanged
    if (!state || !cu_seqlens) return KDA_ERROR_INVALID_VALUE;
    if (!aligned16(state) || ((uintptr_t)cu_seqlens & 3u) != 0) return KDA_ERROR_MISALIGNED;
    kda::RecArgs a{q, k, v, g, beta, state, o, N, T, H, Dk, Dv, Hqk, scale, mode, dtype, o_dtype,
                   cu_seqlens, prologue};
    discard_stale_error();
    hipError_t e = kda::launch_recurrent(a, (hipStream_t)stream);
    return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
}

size_t kda_chunk_fwd_varlen_workspace_size(int N, int T, int H, int Dk, int Dv, int chunk,
                                           kda_gate_mode mode, kda_dtype dtype)
{
    (void)mode;
    if (N < 1 || H < 1 || T < 0) return 0;
    if (!supported_dk(Dk) || !supported_dv(Dv) || !supported_chunk(chunk)) return 0;
    if (!valid_dtype(raw(dtype))) return 0;
    return kda::chunk_varlen_workspace_bytes(N, T, H, Dk, Dv, chunk, dtype);
}

kda_status kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* initial_state, float* final_state,
                                void* o, const int* cu_seqlens, int N, int T, int H, int Hqk,
                                int Dk, int Dv, int chunk, float scale, kda_gate_mode mode,
                                kda_dtype dtype, kda_dtype o_dtype, int prologue, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    if (N < 0 || (prologue & ~KDA_PROLOGUE_ALL)) return KDA_ERROR_INVALID_VALUE;
    kda_status st = check_common(q, k, v, g, beta, o, 1, T, H, Hqk, Dk, Dv, raw(mode), raw(dtype),
                                 raw(o_dtype));
    if (st != KDA_SUCCESS) return st;
    if (!supported_chunk(chunk) || !kda::chunk_fwd_supported(Dk, Dv, chunk, dtype))
        return KDA_ERROR_NOT_SUPPORTED;
    // chunk records and state workgroups are counted in 32-bit integers
    const double gmax = (double)((T + chunk - 1) / chunk) + (double)N;
    if (gmax * H > 1073741824.0 || (double)N * H * (Dv / 16) + 64.0 > 2147483647.0)
        return KDA_ERROR_INVALID_VALUE;
    if (N == 0) return KDA_SUCCESS;
    if (!cu_seqlens) return KDA_ERROR_INVALID_VALUE;
    if (((uintptr_t)cu_seqlens & 3u) != 0) return KDA_ERROR_MISALIGNED;
    if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
        return KDA_ERROR_MISALIGNED;
    const size_t need = kda_chunk_fwd_varlen_workspace_size(N, T, H, Dk, Dv, chunk, mode, dtype);
    if (!workspace || workspace_bytes < need) return KDA_ERROR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return KDA_ERROR_MISALIGNED;
    if (T == 0 && !final_state) return KDA_SUCCESS;
    kda::ChunkArgs a{q, k, v, g, beta, initial_state, final_state, o, 1, T, H, Dk, Dv, chunk, Hqk,
                     scale, mode, dtype, o_dtype, workspace, workspace_bytes, cu_seqlens, N, prologue};
    discard_stale_error();
    hipError_t e = kda::launch_chunk(a, (hipStream_t)stream);
    return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
}

size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int Hqk, int Dk, int Dv, int chunk,
                                    kda_gate_mode mode, kda_dtype dtype)
{
    (void)mode;
    if (B < 1 || H < 1 || T <= 0) return 0;
    if (Hqk < 1 || Hqk > H || H % Hqk != 0) return 0;
    if (!supported_dk(Dk) || !supported_dv(Dv) || !supported_chunk(chunk)) return 0;
    if (!valid_dtype(raw(dtype))) return 0;
    return kda::chunk_bwd_workspace_bytes(B, T, H, Hqk, Dk, Dv, chunk);
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, const void* d_o,
                         const float* d_final_state, void* dq, void* dk, void* dv, float* dg,
                         float* dbeta, float* d_initial_state, int B, int T, int H, int Hqk,
                         int Dk, int Dv, int chunk, float scale, kda_gate_mode mode,
                         kda_dtype dtype, kda_dtype grad_dtype, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    kda_status st = check_common(q, k, v, g, beta, d_o, B, T, H, Hqk, Dk, Dv, raw(mode), raw(dtype),
                                 raw(grad_dtype));
    if (st != KDA_SUCCESS) return st;
    if (!supported_chunk(chunk)) return KDA_ERROR_NOT_SUPPORTED;
    const double nrec = (double)B * H * ((T + chunk - 1) / chunk);
    if (nrec > 1073741824.0 || (double)B * H * 2.0 > 65535.0 * 1024.0)
        return KDA_ERROR_INVALID_VALUE;
    if (T > 0) {
        if (!dq || !dk || !dv || !dbeta) return KDA_ERROR_INVALID_VALUE;
        if (mode != KDA_GATE_NONE && !dg) return KDA_ERROR_INVALID_VALUE;
        if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dbeta))
            return KDA_ERROR_MISALIGNED;
        if (dg && !aligned16(dg)) return KDA_ERROR_MISALIGNED;
    }
    if ((initial_state && !aligned16(initial_state)) || (d_final_state && !aligned16(d_final_state)) ||
        (d_initial_state && !aligned16(d_initial_state)))
        return KDA_ERROR_MISALIGNED;
    const size_t need = kda_chunk_bwd_workspace_size(B, T, H, Hqk, Dk, Dv, chunk, mode, dtype);
    if (T > 0) {
        if (!workspace || workspace_bytes < need) return KDA_ERROR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return KDA_ERROR_MISALIGNED;
    }
    if (T == 0 && !d_initial_state) return KDA_SUCCESS;
    kda::ChunkBwdArgs a{q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                        d_initial_state, B, T, H, Hqk, Dk, Dv, chunk, scale, mode, dtype,
                        grad_dtype, workspace, workspace_bytes};
    discard_stale_error();
    hipError_t e = kda::launch_chunk_bwd(a, (hipStream_t)stream);
    return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
}

size_t kda_chunk_bwd_varlen_workspace_size(int N, int T, int H, int Hqk, int Dk, int Dv, int chunk,
                                           kda_gate_mode mode, kda_dtype dtype)
{
    (void)mode;
    if (N < 1 || H < 1 || T < 0) return 0;
    if (Hqk < 1 || Hqk > H || H % Hqk != 0) return 0;
    if (!supported_dk(Dk) || !supported_dv(Dv) || !supported_chunk(chunk)) return 0;
    if (!valid_dtype(raw(dtype))) return 0;
    return kda::chunk_bwd_varlen_workspace_bytes(N, T, H, Hqk, Dk, Dv, chunk);
}

kda_status kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* initial_state, const void* d_o,
                                const float* d_final_state, void* dq, void* dk, void* dv,
                                float* dg, float* dbeta, float* d_initial_state,
                                const int* cu_seqlens, int N, int T, int H, int Hqk, int Dk,
                                int Dv, int chunk, float scale, kda_gate_mode mode,
                                kda_dtype dtype, kda_dtype grad_dtype, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    if (N < 0) return KDA_ERROR_INVALID_VALUE;
    kda_status st = check_common(q, k, v, g, beta, d_o, 1, T, H, Hqk, Dk, Dv, raw(mode), raw(dtype),
                                 raw(grad_dtype));
    if (st != KDA_SUCCESS) return st;
    if (!supported_chunk(chunk)) return KDA_ERROR_NOT_SUPPORTED;
    const double gmax = (double)((T + chunk - 1) / chunk) + (double)N;
    if (gmax * H > 1073741824.0 || (double)N * H * 2.0 > 65535.0 * 1024.0)
        return KDA_ERROR_INVALID_VALUE;
    if (N == 0) return KDA_SUCCESS;
    if (!cu_seqlens) return KDA_ERROR_INVALID_VALUE;
    if (((uintptr_t)cu_seqlens & 3u) != 0) return KDA_ERROR_MISALIGNED;
    if (T > 0) {
        if (!dq || !dk || !dv || !dbeta) return KDA_ERROR_INVALID_VALUE;
        if (mode != KDA_GATE_NONE && !dg) return KDA_ERROR_INVALID_VALUE;
        if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dbeta))
            return KDA_ERROR_MISALIGNED;
        if (dg && !aligned16(dg)) return KDA_ERROR_MISALIGNED;
    }
    if ((initial_state && !aligned16(initial_state)) || (d_final_state && !aligned16(d_final_state)) ||
        (d_initial_state && !aligned16(d_initial_state)))
        return KDA_ERROR_MISALIGNED;
    const size_t need = kda_chunk_bwd_varlen_workspace_size(N, T, H, Hqk, Dk, Dv, chunk, mode, dtype);
    if (!workspace || workspace_bytes < need) return KDA_ERROR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return KDA_ERROR_MISALIGNED;
    if (T == 0 && !d_initial_state) return KDA_SUCCESS;
    kda::ChunkBwdArgs a{q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                        d_initial_state, 1, T, H, Hqk, Dk, Dv, chunk, scale, mode, dtype,
                        grad_dtype, workspace, workspace_bytes, cu_seqlens, N};
    discard_stale_error();
    hipError_t e = kda::launch_chunk_bwd(a, (hipStream_t)stream);
    return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_HIP;
}

}  // extern "C"
