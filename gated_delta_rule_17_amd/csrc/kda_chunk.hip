// Chunkwise KDA forward: dispatch over the chunk length, the workspace
// layout, and the tables of packed variable-length batches.
#include "kda_chunk.hpp"

namespace kda {

// ---------------------------------------------------------------------------
// Packed variable-length batches: the chunk and sequence tables (one
// workgroup).  Sequence n covers tokens p_n .. p_{n+1}-1 with
// p_m = max_{j <= m} clamp(cu[j], 0, Ttot): for a well-formed cu (0 = cu[0]
// <= cu[1] <= ... <= cu[N] = Ttot) that is exactly [cu[n], cu[n+1]); for any
// other content the sequences still tile a subrange of [0, Ttot] without
// overlap, so no access leaves the buffers and at most
// ceil(Ttot / C) + N chunks arise (the table's size, Gmax).  The sequence
// table entry n is (first token, length, first chunk, 0); the chunk table
// entry g is (first token, length), and the entries after the last chunk are
// (0, 0).
__global__ void __launch_bounds__(1024)
varlen_tables(const int* __restrict__ cu, int N, int Ttot, int C, int Gmax,
              int2* __restrict__ ctab, int4* __restrict__ stab)
{
    __shared__ int smax[1024], ssum[1024];
    const int tid = threadIdx.x;
    int pcarry = 0, ccarry = 0;    // boundary maximum and chunk count of the earlier tiles
    for (int base = 0; base < N; base += 1024) {
        const int n = base + tid;
        int e0 = 0, e1 = 0;
        if (n < N) {
            e0 = min(max(cu[n], 0), Ttot);
            e1 = min(max(cu[n + 1], 0), Ttot);
        }
        int x = e0;                // inclusive prefix maximum over the tile
        smax[tid] = x;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int y = tid >= off ? smax[tid - off] : 0;
            __syncthreads();
            x = max(x, y);
            smax[tid] = x;
            __syncthreads();
        }
        const int start = max(x, pcarry);
        const int len = n < N ? max(start, e1) - start : 0;
        const int nch = (len + C - 1) / C;
        int cs = nch;              // inclusive prefix sum of the chunk counts
        ssum[tid] = cs;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int y = tid >= off ? ssum[tid - off] : 0;
            __syncthreads();
            cs += y;
            ssum[tid] = cs;
            __syncthreads();
        }
        const int first = ccarry + cs - nch;
        if (n < N) {
            stab[n] = make_int4(start, len, first, 0);
            for (int c = 0; c < nch && first + c < Gmax; ++c)
                ctab[first + c] = make_int2(start + c * C, min(C, len - c * C));
        }
        pcarry = max(pcarry, smax[1023]);
        ccarry += ssum[1023];
        __syncthreads();           // smax / ssum are rewritten by the next tile
    }
    for (int gch = ccarry + tid; gch < Gmax; gch += 1024) ctab[gch] = make_int2(0, 0);
}

static size_t records_bytes_any(int C, size_t nrec, int Dk, int Dv, kda_dtype dtype)
{
    switch (C) {
        case 16: return records_bytes_c16(nrec, Dk, Dv, dtype);
        case 32: return records_bytes_c32(nrec, Dk, Dv, dtype);
        case 64: return records_bytes_c64(nrec, Dk, Dv, dtype);
    }
    return 0;
}

// Workspace of the packed form: the records of Gmax * H chunks, then the
// chunk table, then the sequence table.
struct PackedLayout {
    size_t gmax, tab_off, seq_off, total;
};
static PackedLayout packed_layout(int N, int T, int H, int Dk, int Dv, int C, kda_dtype dtype)
{
    PackedLayout p;
    p.gmax = varlen_gmax(N, T, C);
    const size_t rec = records_bytes_any(C, p.gmax * H, Dk, Dv, dtype);
    p.tab_off = align_up(rec, 256);
    p.seq_off = p.tab_off + align_up(p.gmax * sizeof(int2), 16);
    p.total = rec == 0 ? 0 : p.seq_off + (size_t)N * sizeof(int4);
    return p;
}

size_t chunk_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dtype)
{
    // the records, then (segmented state pass only) the segment states
    const size_t NC = (size_t)(T + chunk - 1) / chunk;
    const size_t rec = records_bytes_any(chunk, (size_t)B * H * NC, Dk, Dv, dtype);
    const size_t sb = seg_bytes(B, T, H, Dk, Dv, chunk);
    return rec == 0 || sb == 0 ? rec : align_up(rec, 256) + sb;
}

size_t chunk_varlen_workspace_bytes(int N, int Ttot, int H, int Dk, int Dv, int chunk, kda_dtype dtype)
{
    return packed_layout(N, Ttot, H, Dk, Dv, chunk, dtype).total;
}

size_t packed_chunk_slots(int N, int T, int chunk) { return varlen_gmax(N, T, chunk); }

bool chunk_fwd_supported(int Dk, int Dv, int chunk, kda_dtype dtype)
{
    return records_bytes_any(chunk, 1, Dk, Dv, dtype) != 0;
}

hipError_t build_varlen_tables(const int* cu, int N, int T, int chunk, size_t gmax, void* ctab,
                               void* stab, hipStream_t s)
{
    hipLaunchKernelGGL(varlen_tables, dim3(1), dim3(1024), 0, s, cu, N, T, chunk, (int)gmax,
                       (int2*)ctab, (int4*)stab);
    return hipGetLastError();
}

hipError_t launch_chunk(const ChunkArgs& a0, hipStream_t s)
{
    ChunkArgs a = a0;
    if (a.cu) {
        const PackedLayout p = packed_layout(a.N, a.T, a.H, a.Dk, a.Dv, a.chunk, a.dtype);
        int2* ct = (int2*)((char*)a.ws + p.tab_off);
        int4* st = (int4*)((char*)a.ws + p.seq_off);
        if (a.N > 0) {
            hipLaunchKernelGGL(varlen_tables, dim3(1), dim3(1024), 0, s, a.cu, a.N, a.T, a.chunk,
                               (int)p.gmax, ct, st);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        a.ctab = ct;
        a.stab = st;
    }
    switch (a.chunk) {
        case 16: return launch_chunk_c16(a, s);
        case 32: return launch_chunk_c32(a, s);
        case 64: return launch_chunk_c64(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
