// Gradient of the chunkwise form: workspace layout and dispatch.
#include "kda_bwd.hpp"

namespace kda {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte offsets of the per-chunk records (see bwd::Records) and of the
// grouped-head partials inside the caller's workspace.
struct BwdLayout {
    size_t G, W, WT, Kr, KrT, U, Ut, P, Tm, Ap, Hs, E, dH, dE, dqp, dkp, total;
};

BwdLayout bwd_layout(int B, int T, int H, int Hq, int Dk, int Dv, int C)
{
    BwdLayout l{};
    const size_t NC = (size_t)((T + C - 1) / C);
    const size_t R = (size_t)B * H * NC;
    const size_t f = sizeof(float);
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
    l.G = take(R * C * Dk * f);
    l.W = take(R * C * Dk * f);
    l.WT = take(R * C * Dk * f);
    l.Kr = take(R * C * Dk * f);
    l.KrT = take(R * C * Dk * f);
    l.U = take(R * C * Dv * f);
    l.Ut = take(R * C * Dv * f);
    l.P = take(R * Dk * Dv * f);
    l.Tm = take(R * C * C * f);
    l.Ap = take(R * C * C * f);
    l.Hs = take(R * Dk * Dv * f);
    l.E = take(R * C * Dv * f);
    l.dH = take(R * Dk * Dv * f);
    l.dE = take(R * C * Dv * f);
    const size_t part = Hq < H ? (size_t)B * T * H * Dk * f : 0;
    l.dqp = take(part);
    l.dkp = take(part);
    l.total = o;
    return l;
}

}  // namespace

size_t chunk_bwd_workspace_bytes(int B, int T, int H, int Hq, int Dk, int Dv, int chunk)
{
    if (T <= 0) return 0;
    return bwd_layout(B, T, H, Hq, Dk, Dv, chunk).total;
}

hipError_t launch_chunk_bwd(const ChunkBwdArgs& h, hipStream_t s)
{
    const int C = h.chunk;
    const BwdLayout l = bwd_layout(h.B, h.T, h.H, h.Hq, h.Dk, h.Dv, C);
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
        a.r.G = (float*)(ws + l.G);
        a.r.W = (float*)(ws + l.W);
        a.r.WT = (float*)(ws + l.WT);
        a.r.Kr = (float*)(ws + l.Kr);
        a.r.KrT = (float*)(ws + l.KrT);
        a.r.U = (float*)(ws + l.U);
        a.r.Ut = (float*)(ws + l.Ut);
        a.r.P = (float*)(ws + l.P);
        a.r.Tm = (float*)(ws + l.Tm);
        a.r.Ap = (float*)(ws + l.Ap);
        a.r.Hs = (float*)(ws + l.Hs);
        a.r.E = (float*)(ws + l.E);
        a.r.dH = (float*)(ws + l.dH);
        a.r.dE = (float*)(ws + l.dE);
    }
    a.B = h.B; a.T = h.T; a.H = h.H; a.Hq = h.Hq;
    a.NC = (h.T + C - 1) / C;
    a.mode = (int)h.mode;
    a.gdt = (int)h.grad_dtype;
    a.scale = h.scale;
    if (h.T == 0 && !h.dh0) return hipSuccess;
    hipError_t e = hipErrorInvalidValue;
    if (C == 16) e = launch_bwd_c16(a, h.Dk, h.Dv, h.dtype, s);
    else if (C == 32) e = launch_bwd_c32(a, h.Dk, h.Dv, h.dtype, s);
    else if (C == 64) e = launch_bwd_c64(a, h.Dk, h.Dv, h.dtype, s);
    if (e != hipSuccess || !grouped) return e;
    const size_t n = (size_t)h.B * h.T * h.Hq * h.Dk;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    const int G = h.H / h.Hq;
    if (h.grad_dtype == KDA_BF16)
        hipLaunchKernelGGL(bwd::bwd_group_sum<bf16_t>, dim3(blocks), dim3(256), 0, s, a.dqp, a.dkp,
                           (bf16_t*)h.dq, (bf16_t*)h.dk, n, h.Hq, G, h.Dk);
    else
        hipLaunchKernelGGL(bwd::bwd_group_sum<float>, dim3(blocks), dim3(256), 0, s, a.dqp, a.dkp,
                           (float*)h.dq, (float*)h.dk, n, h.Hq, G, h.Dk);
    return hipGetLastError();
}

}  // namespace kda
