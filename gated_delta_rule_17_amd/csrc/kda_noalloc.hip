// kda_chunk_fwd_noalloc: the chunkwise forward with a fixed, library-owned
// scratch array in place of the caller's workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// hosts that forbid allocation).
//
// The chunk records of kda_chunk_fwd live in `scratch`, a file-scope device
// array of KDA_NOALLOC_SCRATCH_BYTES.  Each device the library runs on holds
// its own copy of it from module load until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and that address is what the kernels receive.
//
// Every call on one device shares that device's array.  The forward writes
// every record before any kernel reads it, so no contents carry over from
// an earlier call and nothing needs clearing; two calls that overlap in
// time on one device (different streams, or different host threads) race on
// the records.
#include <atomic>
#include <mutex>

#include "kda_internal.hpp"

namespace {

__device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDev = 64;
std::atomic<void*> g_scratch[kMaxDev];
std::mutex g_scratch_mu;

// Device address of this device's scratch array (looked up on first use per
// device, with that device current).
hipError_t scratch_address(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                            const float* g, const float* beta,
                                            const float* initial_state, float* final_state,
                                            void* o, int B, int T, int H, int Hqk, int Dk, int Dv,
                                            int chunk, float scale, kda_gate_mode mode,
                                            kda_dtype dtype, kda_dtype o_dtype, int prologue,
                                            void* stream)
{
    // every check of kda_chunk_fwd but the workspace's, before any HIP call
    // (the enum arguments are validated there by their bytes)
    const kda_status st = kda::chunk_fwd_checks(q, k, v, g, beta, initial_state, final_state, o, B,
                                                T, H, Hqk, Dk, Dv, chunk, mode, dtype, o_dtype,
                                                prologue);
    if (st != KDA_SUCCESS) return st;
    const size_t need = kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, chunk, mode, dtype);
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERROR_SCRATCH;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return KDA_ERROR_HIP;
    return kda_chunk_fwd(q, k, v, g, beta, initial_state, final_state, o, B, T, H, Hqk, Dk, Dv,
                         chunk, scale, mode, dtype, o_dtype, prologue, ws,
                         (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}
