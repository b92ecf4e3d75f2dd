// Host-side interfaces between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kda.h"

namespace kda {

// epsilon of the fused L2 normalisation: x / sqrt(sum x^2 + eps)
constexpr float kNormEps = 1e-6f;

struct RecArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    float* state; void* o;
    int B, T, H, Dk, Dv;
    int Hq;               // query/key heads (H is a multiple; value head h reads h / (H / Hq))
    float scale;
    kda_gate_mode mode;
    kda_dtype dtype;      // q, k, v
    kda_dtype o_dtype;    // o
    // packed variable-length batch: device offsets [N + 1] (B is N, T the
    // packed token count), or null for a dense [B, T] batch
    const int* cu;
    int prologue;         // kda_prologue flags
};

struct ChunkArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    const float* h0; float* hT; void* o;
    int B, T, H, Dk, Dv, chunk;
    int Hq;               // query/key heads (H is a multiple; value head h reads h / (H / Hq))
    float scale;
    kda_gate_mode mode;
    kda_dtype dtype;      // q, k, v
    kda_dtype o_dtype;    // o
    void* ws; size_t ws_bytes;
    // packed variable-length batch: device offsets [N + 1] and N (T is the
    // packed token count, B unused), or null for a dense [B, T] batch
    const int* cu;
    int N;
    int prologue;         // kda_prologue flags
    // packed: the chunk and sequence tables in the workspace (set by the
    // dispatcher after it has built them)
    const void* ctab = nullptr;
    const void* stab = nullptr;
};

struct ChunkBwdArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta; const float* h0;
    const void* dO; const float* dhT;
    void* dq; void* dk; void* dv;
    float* dg; float* dbeta; float* dh0;
    int B, T, H, Hq, Dk, Dv, chunk;
    float scale;
    kda_gate_mode mode;
    kda_dtype dtype;      // q, k, v, dO
    kda_dtype grad_dtype; // dq, dk, dv
    void* ws; size_t ws_bytes;
    // packed variable-length batch: device offsets [N + 1] (T is the packed
    // token count, B is 1), or null for a dense [B, T] batch
    const int* cu = nullptr;
    int N = 0;
};

hipError_t launch_recurrent(const RecArgs& a, hipStream_t s);

// Every argument check of kda_chunk_fwd except those of the workspace (host
// only, no HIP call).  The enum arguments are taken by reference and read by
// their bytes: a C caller may pass any int, and only validated values are
// used as enums.
kda_status chunk_fwd_checks(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* initial_state,
                            const float* final_state, const void* o, int B, int T, int H, int Hqk,
                            int Dk, int Dv, int chunk, const kda_gate_mode& mode,
                            const kda_dtype& dtype, const kda_dtype& o_dtype, int prologue);

// Workspace layout of the chunk path (bytes); 0 if unsupported.
size_t chunk_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dtype);
size_t chunk_varlen_workspace_bytes(int N, int Ttot, int H, int Dk, int Dv, int chunk, kda_dtype dtype);
hipError_t launch_chunk(const ChunkArgs& a, hipStream_t s);

// Chunk and sequence tables of a packed batch (one workgroup, asynchronous):
// gmax chunk slots of (first token, length) and N sequences of (first token,
// length, first slot, 0), from device offsets cu[N + 1].
size_t packed_chunk_slots(int N, int T, int chunk);
// Whether the chunk forward is built for this (Dk, Dv, chunk, dtype): every
// supported pair except float32 operands with chunk 64, Dk 128 and Dv 256,
// whose staging does not fit a compute unit's LDS.
bool chunk_fwd_supported(int Dk, int Dv, int chunk, kda_dtype dtype);
hipError_t build_varlen_tables(const int* cu, int N, int T, int chunk, size_t gmax, void* ctab,
                               void* stab, hipStream_t s);

// Gradient of the chunk path: workspace bytes and launch.
size_t chunk_bwd_workspace_bytes(int B, int T, int H, int Hq, int Dk, int Dv, int chunk);
size_t chunk_bwd_varlen_workspace_bytes(int N, int T, int H, int Hq, int Dk, int Dv, int chunk);
hipError_t launch_chunk_bwd(const ChunkBwdArgs& a, hipStream_t s);

}  // namespace kda
