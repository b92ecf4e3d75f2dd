// Gradient of the chunkwise form: workspace layout and dispatch.
#include <algorithm>

#include "kda_bwd.hpp"

namespace kda {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Layout of the workspace: one float block per (sequence, head, chunk)
// record holding all of its fields (see bwd::Records) one after another, so
// that a workgroup working on a chunk touches one contiguous region; then
// the grouped-head partials.  Every field is a multiple of 1 KiB.
struct BwdLayout {
    size_t G, W, WT, Kr, KrT, U, Ut, P, Tm, Ap, Hs, E, dH, dE;   // float offsets in a record
    size_t rs;                                                  // floats per record
    size_t dqp, dkp, ctab, stab, total;                         // bytes
    size_t gmax;                                                // packed: chunk slots
};

// Dense batch: B * H * ceil(T / C) records.  Packed batch (N > 0, B = 1):
// H * gmax records, gmax = ceil(T / C) + N chunk slots, then the chunk and
// sequence tables.
BwdLayout bwd_layout(int B, int T, int H, int Hq, int Dk, int Dv, int C, int N = 0)
{
    BwdLayout l{};
    const size_t NC = (size_t)((T + C - 1) / C);
    l.gmax = N > 0 ? packed_chunk_slots(N, T, C) : 0;
    const size_t R = N > 0 ? (size_t)H * l.gmax : (size_t)B * H * NC;
    size_t o = 0;
    auto take = [&](size_t floats) { const size_t at = o; o += floats; return at; };
    l.G = take((size_t)C * Dk);
    l.W = take((size_t)C * Dk);
    l.WT = take((size_t)C * Dk);
    l.Kr = take((size_t)C * Dk);
    l.KrT = take((size_t)C * Dk);
    l.U = take((size_t)C * Dv);
    l.Ut = take((size_t)C * Dv);
    l.P = take((size_t)Dk * Dv);
    l.Tm = take((size_t)C * C);
    l.Ap = take((size_t)C * C);
    l.Hs = take((size_t)Dk * Dv);
    l.E = take((size_t)C * Dv);
    l.dH = take((size_t)Dk * Dv);
    l.dE = take((size_t)C * Dv);
    l.rs = o;
    size_t b = align256(R * l.rs * sizeof(float));
    const size_t part = Hq < H ? (size_t)B * T * H * Dk * sizeof(float) : 0;
    l.dqp = b;
    b = align256(b + part);
    l.dkp = b;
    b = align256(b + part);
    if (N > 0) {
        l.ctab = b;
        b = align256(b + l.gmax * sizeof(int2));
        l.stab = b;
        b = align256(b + (size_t)N * sizeof(int4));
    }
    l.total = b;
    return l;
}

// Dense batches run in groups of whole batch entries, so that the records of
// one group stay within kRecordCap bytes (at least one entry per group): the
// workspace is sized for one group and reused by the next.  A group of one
// entry still holds H * ceil(T / C) chunks, which fills the device.
constexpr size_t kRecordCap = (size_t)4 << 30;

int bwd_group(int B, int T, int H, int Hq, int Dk, int Dv, int C)
{
    const BwdLayout one = bwd_layout(1, T, H, Hq, Dk, Dv, C);
    const size_t per = (size_t)H * (size_t)((T + C - 1) / C) * one.rs * sizeof(float);
    const size_t fit = per > 0 ? kRecordCap / per : (size_t)B;
    return (int)std::max<size_t>(1, std::min<size_t>((size_t)B, fit));
}

// The three kernels (and the grouped-head sum) over the batch entries and
// records that `a` describes.
hipError_t run_bwd(const bwd::Args& a, const ChunkBwdArgs& h, hipStream_t s)
{
    hipError_t e = hipErrorInvalidValue;
    if (h.chunk == 16) e = launch_bwd_c16(a, h.Dk, h.Dv, h.dtype, s);
    else if (h.chunk == 32) e = launch_bwd_c32(a, h.Dk, h.Dv, h.dtype, s);
    else if (h.chunk == 64) e = launch_bwd_c64(a, h.Dk, h.Dv, h.dtype, s);
    if (e != hipSuccess || !a.dqp) return e;
    const size_t n = (size_t)a.B * a.T * a.Hq * h.Dk;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    const int G = a.H / a.Hq;
    if (a.gdt == KDA_BF16)
        hipLaunchKernelGGL(bwd::bwd_group_sum<bf16_t>, dim3(blocks), dim3(256), 0, s, a.dqp, a.dkp,
                           (bf16_t*)a.dq, (bf16_t*)a.dk, n, a.Hq, G, h.Dk);
    else
        hipLaunchKernelGGL(bwd::bwd_group_sum<float>, dim3(blocks), dim3(256), 0, s, a.dqp, a.dkp,
                           (float*)a.dq, (float*)a.dk, n, a.Hq, G, h.Dk);
    return hipGetLastError();
}

}  // namespace

size_t chunk_bwd_workspace_bytes(int B, int T, int H, int Hq, int Dk, int Dv, int chunk)
{
    if (T <= 0) return 0;
    return bwd_layout(bwd_group(B, T, H, Hq, Dk, Dv, chunk), T, H, Hq, Dk, Dv, chunk).total;
}

size_t chunk_bwd_varlen_workspace_bytes(int N, int T, int H, int Hq, int Dk, int Dv, int chunk)
{
    if (N <= 0) return 0;
    return bwd_layout(1, T, H, Hq, Dk, Dv, chunk, N).total;
}

hipError_t launch_chunk_bwd(const ChunkBwdArgs& h, hipStream_t s)
{
    const int C = h.chunk;
    const bool packed = h.cu != nullptr;
    const int Bg = packed ? 1 : bwd_group(h.B, h.T, h.H, h.Hq, h.Dk, h.Dv, C);
    const BwdLayout l = bwd_layout(Bg, h.T, h.H, h.Hq, h.Dk, h.Dv, C, packed ? h.N : 0);
    char* ws = (char*)h.ws;
    bwd::Args a{};
    a.q = h.q; a.k = h.k; a.v = h.v; a.dO = h.dO;
    a.g = h.g; a.beta = h.beta; a.h0 = h.h0; a.dhT = h.dhT;
    a.dq = h.dq; a.dk = h.dk; a.dv = h.dv;
    a.dg = h.dg; a.dbeta = h.dbeta; a.dh0 = h.dh0;
    const bool grouped = h.Hq < h.H && h.T > 0;
    a.dqp = grouped ? (float*)(ws + l.dqp) : nullptr;
    a.dkp = grouped ? (float*)(ws + l.dkp) : nullptr;
    if (h.T > 0) {
        float* f = (float*)ws;
        a.r.G = f + l.G;
        a.r.W = f + l.W;
        a.r.WT = f + l.WT;
        a.r.Kr = f + l.Kr;
        a.r.KrT = f + l.KrT;
        a.r.U = f + l.U;
        a.r.Ut = f + l.Ut;
        a.r.P = f + l.P;
        a.r.Tm = f + l.Tm;
        a.r.Ap = f + l.Ap;
        a.r.Hs = f + l.Hs;
        a.r.E = f + l.E;
        a.r.dH = f + l.dH;
        a.r.dE = f + l.dE;
        a.r.rs = l.rs;
    }
    a.B = h.B; a.T = h.T; a.H = h.H; a.Hq = h.Hq;
    a.NC = (h.T + C - 1) / C;
    a.ctab = nullptr;
    a.stab = nullptr;
    a.N = 0;
    a.Gmax = 0;
    a.mode = (int)h.mode;
    a.gdt = (int)h.grad_dtype;
    a.scale = h.scale;
    if (packed) {
        if (h.N == 0) return hipSuccess;
        a.B = 1;
        a.N = h.N;
        a.Gmax = (int)l.gmax;
        a.ctab = (const int2*)(ws + l.ctab);
        a.stab = (const int4*)(ws + l.stab);
        hipError_t e = build_varlen_tables(h.cu, h.N, h.T, C, l.gmax, ws + l.ctab, ws + l.stab, s);
        if (e != hipSuccess) return e;
        return run_bwd(a, h, s);
    }
    if (h.T == 0 && !h.dh0) return hipSuccess;
    // per batch entry: elements of each tensor (storage sizes apply below)
    const size_t tq = (size_t)h.T * h.Hq * h.Dk, tv = (size_t)h.T * h.H * h.Dv;
    const size_t tr = (size_t)h.T * h.H, tg = h.mode == KDA_GATE_CHANNEL ? tr * h.Dk : tr;
    const size_t st = (size_t)h.H * h.Dk * h.Dv;
    const size_t io = h.dtype == KDA_BF16 ? 2 : 4, gs = h.grad_dtype == KDA_BF16 ? 2 : 4;
    auto at = [](const void* p, size_t bytes) -> void* {
        return p ? (void*)((const char*)p + bytes) : nullptr;
    };
    for (int b0 = 0; b0 < h.B; b0 += Bg) {
        bwd::Args x = a;
        const size_t e = (size_t)b0;
        x.B = std::min(Bg, h.B - b0);
        x.q = at(h.q, e * tq * io);
        x.k = at(h.k, e * tq * io);
        x.v = at(h.v, e * tv * io);
        x.dO = at(h.dO, e * tv * io);
        x.g = (const float*)at(h.g, e * tg * 4);
        x.beta = (const float*)at(h.beta, e * tr * 4);
        x.h0 = (const float*)at(h.h0, e * st * 4);
        x.dhT = (const float*)at(h.dhT, e * st * 4);
        x.dq = at(h.dq, e * tq * gs);
        x.dk = at(h.dk, e * tq * gs);
        x.dv = at(h.dv, e * tv * gs);
        x.dg = (float*)at(h.dg, e * tg * 4);
        x.dbeta = (float*)at(h.dbeta, e * tr * 4);
        x.dh0 = (float*)at(h.dh0, e * st * 4);
        const hipError_t err = run_bwd(x, h, s);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace kda
