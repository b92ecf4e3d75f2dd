// Gradient of the chunkwise form (training backward) for gfx950.
//
// The pages train Kimi Delta Attention with the chunkwise algorithm (F29
// course outline, "Paper: Gated DeltaNet -> Kimi Delta Attention"; GeekNews
// #31925, section "Fused recurrent kernel for decode": chunkwise for training
// and prefill) but print no backward formulas.  The kernels here apply
// reverse mode to the chunk map of the forward (per chunk of C tokens, with
// H the transposed state entering it, G the inclusive prefix of the log
// gates, Gamma_ij = exp(G_i - G_j)):
//
//   A = strict lower part of beta_i sum_c k_i k_j Gamma_ij ; T = (I + A)^-1
//   U = T Diag(beta) V ; W = T Diag(beta) (K e^G) ; E = U - W H
//   Aqk = inclusive lower part of sum_c (scale q_i) k_j Gamma_ij
//   O = (scale Q e^G) H + Aqk E ;  H' = Diag(e^{G_last}) H + Kr^T E,
//   Kr = K e^{G_last - G}
//
// Four launches:
//   1. bwd_prep   one workgroup per (sequence, head, chunk): G, A (before the
//                 beta scaling), Aqk, T, W, U, Kr and Q e^G into per-chunk
//                 float32 records.
//   2. bwd_states one launch, two roles: workgroups of the first half carry
//                 the state forward through the chunks (storing the state
//                 entering each chunk and E), those of the second half carry
//                 the state gradient backward,
//                   dE = Aqk^T dO + Kr dH' ;
//                   dH = Diag(e^{G_last}) dH' + (scale Q e^G)^T dO - W^T dE,
//                 storing dH' and dE per chunk.  Each workgroup owns one
//                 16-column tile of the value dimension of one head.
//   3. bwd_grad   one workgroup per chunk, one wave per 16 key channels:
//                 dUt = T^T dE, dv = beta dUt, the products with the chunk
//                 state and its gradient, dA = -(strict lower dUt E^T),
//                 dAqk = lower dO E^T, then dq, dk, dbeta and the gate
//                 gradient (suffix sums of dG inside the chunk).
//   4. bwd_group_sum (grouped value heads only) adds the query/key gradients
//                 of the value heads that share a query/key head.
//
// Every product runs on v_mfma_f32_16x16x4_f32 with float32 operands from
// LDS.  Operand convention of that instruction (lane l, r = l % 16,
// g = l / 16): A[r][g], B[g][r]; accumulator element i is D[4g + i][r].
//
// Decays inside a chunk come from differences of G.  Products that sum
// over the tokens of a chunk with a decay between the two tokens are split
// at a reference row per 16-row output block: the first row of the block for
// sums over earlier tokens, the last row for sums over later ones.  Every
// factor is then either at most 1 or spans at most 15 tokens, so the path
// stays finite while no key channel decays by more than about e^-80 across
// 16 consecutive tokens.
#pragma once

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace bwd {

// Per-chunk float32 records in the workspace; record r = unit * NC + chunk,
// unit = b * H + h.  Rows of a ragged last chunk beyond its length are zero
// (G repeats its last valid row).
struct Records {
    float* G;    // [C][DK]  inclusive prefix of the log gates
    float* W;    // [C][DK]
    float* Kr;   // [C][DK]  K e^{G_last - G}
    float* Qg;   // [C][DK]  scale Q e^G
    float* U;    // [C][DV]
    float* Tm;   // [C][C]   (I + A)^-1
    float* Aq;   // [C][C]   Aqk (inclusive lower)
    float* Ap;   // [C][C]   A before the beta scaling (strict lower)
    float* Hs;   // [DK][DV] state entering the chunk
    float* E;    // [C][DV]  pseudo-values
    float* dH;   // [DK][DV] gradient of the state leaving the chunk
    float* dE;   // [C][DV]
};

struct Args {
    const void* q; const void* k; const void* v; const void* dO;
    const float* g; const float* beta; const float* h0; const float* dhT;
    void* dq; void* dk; void* dv;
    float* dg; float* dbeta; float* dh0;
    float* dqp; float* dkp;   // grouped heads: float partials per value head, else null
    Records r;
    int B, T, H, Hq, NC, mode;
    int gdt;                  // storage type of dq, dk, dv (kda_dtype)
    float scale;
};

// Store one gradient element in the gradient storage type.
__device__ __forceinline__ void store_grad(void* base, size_t i, float x, int gdt) {
    if (gdt == KDA_BF16) io<bf16_t>::store((bf16_t*)base + i, x);
    else ((float*)base)[i] = x;
}

__device__ __forceinline__ size_t tok_qk(const Args& a, int b, int t, int hq) {
    return ((size_t)b * a.T + t) * a.Hq + hq;
}
__device__ __forceinline__ size_t tok_v(const Args& a, int b, int t, int h) {
    return ((size_t)b * a.T + t) * a.H + h;
}

__device__ __forceinline__ float ex(float x) { return __expf(x); }

// Index of the n-th lower block tile (I, J), J <= I, of an NB x NB grid.
__device__ __forceinline__ void lower_tile(int n, int& I, int& J) {
    I = 0;
    while (n > I) { n -= I + 1; ++I; }
    J = n;
}

// ---------------------------------------------------------------------------
// 1. per-chunk preparation
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, typename IO>
__global__ void __launch_bounds__(256) bwd_prep(Args a)
{
    constexpr int NB = C / 16;
    constexpr int LK = DK + 2;
    constexpr int DM = DK > DV ? DK : DV;
    constexpr int LS = DM + 2;
    constexpr int LC = C + 2;
    __shared__ float sG[C][LK];
    __shared__ float sS[C][LS];
    __shared__ float sAk[16][LK];
    __shared__ float sAq[16][LK];
    __shared__ float sAp[C][LC];
    __shared__ float sT[C][LC];
    __shared__ float sBeta[C];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int rec = blockIdx.x;
    const int u = rec / a.NC, ch = rec % a.NC;
    const int b = u / a.H, h = u % a.H, hq = h / (a.H / a.Hq);
    const int t0 = ch * C;
    const int L = min(C, a.T - t0);
    const IO* q = (const IO*)a.q;
    const IO* k = (const IO*)a.k;
    const IO* v = (const IO*)a.v;
    const size_t R = (size_t)rec;
    float* const gG = a.r.G + R * C * DK;

    // G: inclusive prefix of the log gates per key channel (zero past the end)
    for (int c = tid; c < DK; c += 256) {
        float acc = 0.f;
        for (int i = 0; i < C; ++i) {
            float gi = 0.f;
            if (i < L) {
                if (a.mode == KDA_GATE_CHANNEL) gi = a.g[tok_v(a, b, t0 + i, h) * DK + c];
                else if (a.mode == KDA_GATE_SCALAR) gi = a.g[tok_v(a, b, t0 + i, h)];
            }
            acc += gi;
            sG[i][c] = acc;
            gG[i * DK + c] = acc;
        }
    }
    for (int i = tid; i < C; i += 256) sBeta[i] = i < L ? a.beta[tok_v(a, b, t0 + i, h)] : 0.f;
    __syncthreads();

    // coupling before beta (strict lower) and Aqk (inclusive lower), one
    // 16-row block I at a time, reference row 16 I
    for (int I = 0; I < NB; ++I) {
        const int rows = 16 * (I + 1);
        for (int e = tid; e < rows * DK; e += 256) {
            const int j = e / DK, c = e % DK;
            const float kv = j < L ? io<IO>::load(k + tok_qk(a, b, t0 + j, hq) * DK + c) : 0.f;
            sS[j][c] = kv * ex(sG[16 * I][c] - sG[j][c]);
        }
        for (int e = tid; e < 16 * DK; e += 256) {
            const int m = e / DK, c = e % DK, i = 16 * I + m;
            const float f = ex(sG[i][c] - sG[16 * I][c]);
            float kv = 0.f, qv = 0.f;
            if (i < L) {
                kv = io<IO>::load(k + tok_qk(a, b, t0 + i, hq) * DK + c);
                qv = io<IO>::load(q + tok_qk(a, b, t0 + i, hq) * DK + c);
            }
            sAk[m][c] = kv * f;
            sAq[m][c] = a.scale * qv * f;
        }
        __syncthreads();
        for (int job = w; job < 2 * (I + 1); job += 4) {
            const int which = job & 1, J = job >> 1;
            const float* A = which ? &sAq[0][0] : &sAk[0][0];
            f32x4 acc = zero4();
#pragma unroll 8
            for (int kk = 0; kk < DK; kk += 4)
                acc = mma4(A[r16 * LK + kk + q4], sS[16 * J + r16][kk + q4], acc);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * I + 4 * q4 + ii, j = 16 * J + r16;
                if (which == 0) {
                    const float val = j < i ? acc[ii] : 0.f;
                    sAp[i][j] = val;
                    a.r.Ap[R * C * C + i * C + j] = val;
                } else {
                    a.r.Aq[R * C * C + i * C + j] = j <= i ? acc[ii] : 0.f;
                }
            }
        }
        if (rows < C) {
            for (int e = tid; e < 16 * (C - rows); e += 256) {
                const int i = 16 * I + e / (C - rows), j = rows + e % (C - rows);
                sAp[i][j] = 0.f;
                a.r.Ap[R * C * C + i * C + j] = 0.f;
                a.r.Aq[R * C * C + i * C + j] = 0.f;
            }
        }
        __syncthreads();
    }

    // T = (I + A)^-1 by forward substitution, one column per thread:
    // T[i][c] = delta_ic - beta_i sum_{c <= j < i} Ap[i][j] T[j][c]
    if (tid < C) {
        const int cc = tid;
        for (int i = 0; i < C; ++i) {
            float t;
            if (i < cc) {
                t = 0.f;
            } else if (i == cc) {
                t = 1.f;
            } else {
                float s = 0.f;
                for (int j = cc; j < i; ++j) s += sAp[i][j] * sT[j][cc];
                t = -sBeta[i] * s;
            }
            sT[i][cc] = t;
        }
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += 256) a.r.Tm[R * C * C + e] = sT[e / C][e % C];

    // W = T Diag(beta) (K e^G)
    for (int e = tid; e < C * DK; e += 256) {
        const int j = e / DK, c = e % DK;
        const float kv = j < L ? io<IO>::load(k + tok_qk(a, b, t0 + j, hq) * DK + c) : 0.f;
        sS[j][c] = sBeta[j] * kv * ex(sG[j][c]);
    }
    __syncthreads();
    for (int job = w; job < NB * (DK / 16); job += 4) {
        const int I = job / (DK / 16), Rc = job % (DK / 16);
        f32x4 acc = zero4();
        for (int kk = 0; kk < 16 * (I + 1); kk += 4)
            acc = mma4(sT[16 * I + r16][kk + q4], sS[kk + q4][16 * Rc + r16], acc);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            a.r.W[R * C * DK + (16 * I + 4 * q4 + ii) * DK + 16 * Rc + r16] = acc[ii];
    }
    __syncthreads();

    // U = T Diag(beta) V
    for (int e = tid; e < C * DV; e += 256) {
        const int j = e / DV, c = e % DV;
        const float vv = j < L ? io<IO>::load(v + tok_v(a, b, t0 + j, h) * DV + c) : 0.f;
        sS[j][c] = sBeta[j] * vv;
    }
    __syncthreads();
    for (int job = w; job < NB * (DV / 16); job += 4) {
        const int I = job / (DV / 16), Rc = job % (DV / 16);
        f32x4 acc = zero4();
        for (int kk = 0; kk < 16 * (I + 1); kk += 4)
            acc = mma4(sT[16 * I + r16][kk + q4], sS[kk + q4][16 * Rc + r16], acc);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            a.r.U[R * C * DV + (16 * I + 4 * q4 + ii) * DV + 16 * Rc + r16] = acc[ii];
    }

    // Kr = K e^{G_last - G}, Qg = scale Q e^G
    for (int e = tid; e < C * DK; e += 256) {
        const int i = e / DK, c = e % DK;
        float kv = 0.f, qv = 0.f;
        if (i < L) {
            kv = io<IO>::load(k + tok_qk(a, b, t0 + i, hq) * DK + c);
            qv = io<IO>::load(q + tok_qk(a, b, t0 + i, hq) * DK + c);
        }
        a.r.Kr[R * C * DK + e] = kv * ex(sG[C - 1][c] - sG[i][c]);
        a.r.Qg[R * C * DK + e] = a.scale * qv * ex(sG[i][c]);
    }
}

// ---------------------------------------------------------------------------
// 2. sequential state passes (forward carry and reverse gradient carry)
// ---------------------------------------------------------------------------
template <int C, int DK, int DV>
struct StateLds {
    static constexpr int VT = 16;
    static constexpr int LW = DK + 2;    // rows read along the row index (normal A operand)
    static constexpr int LX = DK + 16;   // rows read along the column index (transposed A)
    static constexpr int LA = C + 16;
    // forward role
    static constexpr int fH = 0, fW = fH + DK * VT, fKr = fW + C * LW, fE = fKr + C * LX,
                         fGam = fE + C * VT, F_END = fGam + DK;
    // reverse role
    static constexpr int rdH = 0, rAq = rdH + DK * VT, rKr = rAq + C * LA, rQg = rKr + C * LW,
                         rW = rQg + C * LX, rdO = rW + C * LX, rdE = rdO + C * VT,
                         rGam = rdE + C * VT, R_END = rGam + DK;
    static constexpr int SIZE = F_END > R_END ? F_END : R_END;
};

// copy a [rows][cols] float record into LDS rows of stride ld
template <int ROWS, int COLS, int NT>
__device__ __forceinline__ void stage(float* dst, int ld, const float* src, int tid) {
    for (int e4 = tid; e4 < ROWS * COLS / 4; e4 += NT) {
        const int row = e4 / (COLS / 4), c4 = (e4 % (COLS / 4)) * 4;
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + row * COLS + c4);
        float* d = dst + row * ld + c4;
        d[0] = x[0]; d[1] = x[1]; d[2] = x[2]; d[3] = x[3];
    }
}

template <int C, int DK, int DV, typename IO>
__global__ void __launch_bounds__(256) bwd_states(Args a)
{
    using S = StateLds<C, DK, DV>;
    constexpr int NB = C / 16, VT = S::VT;
    __shared__ __align__(16) float smem[S::SIZE];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int units = a.B * a.H;
    const bool reverse = (int)blockIdx.y >= units;
    const int u = reverse ? blockIdx.y - units : blockIdx.y;
    const int b = u / a.H, h = u % a.H;
    const int v0 = blockIdx.x * VT;
    const size_t DD = (size_t)DK * DV;

    if (!reverse) {
        float* sH = smem + S::fH;
        float* sW = smem + S::fW;
        float* sKr = smem + S::fKr;
        float* sE = smem + S::fE;
        float* sGam = smem + S::fGam;
        for (int e = tid; e < DK * VT; e += 256) {
            const int c = e / VT, n = e % VT;
            sH[e] = a.h0 ? a.h0[(size_t)u * DD + c * DV + v0 + n] : 0.f;
        }
        for (int ch = 0; ch < a.NC; ++ch) {
            const size_t R = (size_t)u * a.NC + ch;
            stage<C, DK, 256>(sW, S::LW, a.r.W + R * C * DK, tid);
            stage<C, DK, 256>(sKr, S::LX, a.r.Kr + R * C * DK, tid);
            for (int c = tid; c < DK; c += 256) sGam[c] = ex(a.r.G[R * C * DK + (C - 1) * DK + c]);
            __syncthreads();
            for (int e = tid; e < DK * VT; e += 256) {
                const int c = e / VT, n = e % VT;
                a.r.Hs[R * DD + c * DV + v0 + n] = sH[e];
            }
            if (w < NB) {
                const int I = w;
                f32x4 acc = zero4();
#pragma unroll 8
                for (int kk = 0; kk < DK; kk += 4)
                    acc = mma4(sW[(16 * I + r16) * S::LW + kk + q4], sH[(kk + q4) * VT + r16], acc);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int i = 16 * I + 4 * q4 + ii;
                    const float e = a.r.U[R * C * DV + i * DV + v0 + r16] - acc[ii];
                    sE[i * VT + r16] = e;
                    a.r.E[R * C * DV + i * DV + v0 + r16] = e;
                }
            }
            __syncthreads();
            for (int Rt = w; Rt < DK / 16; Rt += 4) {
                f32x4 acc = zero4();
#pragma unroll 8
                for (int kk = 0; kk < C; kk += 4)
                    acc = mma4(sKr[(kk + q4) * S::LX + 16 * Rt + r16], sE[(kk + q4) * VT + r16], acc);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int c = 16 * Rt + 4 * q4 + ii;
                    sH[c * VT + r16] = sGam[c] * sH[c * VT + r16] + acc[ii];
                }
            }
            __syncthreads();
        }
        return;
    }

    // reverse role
    const IO* dO = (const IO*)a.dO;
    float* sdH = smem + S::rdH;
    float* sAq = smem + S::rAq;
    float* sKr = smem + S::rKr;
    float* sQg = smem + S::rQg;
    float* sW = smem + S::rW;
    float* sdO = smem + S::rdO;
    float* sdE = smem + S::rdE;
    float* sGam = smem + S::rGam;
    for (int e = tid; e < DK * VT; e += 256) {
        const int c = e / VT, n = e % VT;
        sdH[e] = a.dhT ? a.dhT[(size_t)u * DD + c * DV + v0 + n] : 0.f;
    }
    for (int ch = a.NC - 1; ch >= 0; --ch) {
        const size_t R = (size_t)u * a.NC + ch;
        const int t0 = ch * C;
        const int L = min(C, a.T - t0);
        stage<C, C, 256>(sAq, S::LA, a.r.Aq + R * C * C, tid);
        stage<C, DK, 256>(sKr, S::LW, a.r.Kr + R * C * DK, tid);
        stage<C, DK, 256>(sQg, S::LX, a.r.Qg + R * C * DK, tid);
        stage<C, DK, 256>(sW, S::LX, a.r.W + R * C * DK, tid);
        for (int e = tid; e < C * VT; e += 256) {
            const int i = e / VT, n = e % VT;
            sdO[e] = i < L ? io<IO>::load(dO + tok_v(a, b, t0 + i, h) * DV + v0 + n) : 0.f;
        }
        for (int c = tid; c < DK; c += 256) sGam[c] = ex(a.r.G[R * C * DK + (C - 1) * DK + c]);
        __syncthreads();
        for (int e = tid; e < DK * VT; e += 256) {
            const int c = e / VT, n = e % VT;
            a.r.dH[R * DD + c * DV + v0 + n] = sdH[e];
        }
        if (w < NB) {
            const int I = w;
            f32x4 acc = zero4();
            for (int kk = 16 * I; kk < C; kk += 4)
                acc = mma4(sAq[(kk + q4) * S::LA + 16 * I + r16], sdO[(kk + q4) * VT + r16], acc);
#pragma unroll 8
            for (int kk = 0; kk < DK; kk += 4)
                acc = mma4(sKr[(16 * I + r16) * S::LW + kk + q4], sdH[(kk + q4) * VT + r16], acc);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * I + 4 * q4 + ii;
                sdE[i * VT + r16] = acc[ii];
                a.r.dE[R * C * DV + i * DV + v0 + r16] = acc[ii];
            }
        }
        __syncthreads();
        for (int Rt = w; Rt < DK / 16; Rt += 4) {
            f32x4 pos = zero4(), neg = zero4();
#pragma unroll 8
            for (int kk = 0; kk < C; kk += 4) {
                pos = mma4(sQg[(kk + q4) * S::LX + 16 * Rt + r16], sdO[(kk + q4) * VT + r16], pos);
                neg = mma4(sW[(kk + q4) * S::LX + 16 * Rt + r16], sdE[(kk + q4) * VT + r16], neg);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int c = 16 * Rt + 4 * q4 + ii;
                sdH[c * VT + r16] = sGam[c] * sdH[c * VT + r16] + pos[ii] - neg[ii];
            }
        }
        __syncthreads();
    }
    if (a.dh0) {
        for (int e = tid; e < DK * VT; e += 256) {
            const int c = e / VT, n = e % VT;
            a.dh0[(size_t)u * DD + c * DV + v0 + n] = sdH[e];
        }
    }
}

// ---------------------------------------------------------------------------
// 3. per-chunk gradients
// ---------------------------------------------------------------------------
template <int C, int DK, int DV>
struct GradLds {
    static constexpr int NB = C / 16, NW = DK / 16;
    static constexpr int VS = DV < 32 ? DV : 32;
    static constexpr int LT = C + 16, LV = VS + 2, LE = VS + 16, LA = C + 2;
    // value-slice phase
    static constexpr int oT = 0, oH = oT + C * LT, odH = oH + DK * LV, oE = odH + DK * LV,
                         odO = oE + C * LV, odU = odO + C * LV, oV = odU + C * LV,
                         odE = oV + C * LV, S_END = odE + C * LE;
    // output phase
    static constexpr int oAq = 0, oAb = oAq + C * LA, oSrc = oAb + C * LA,
                         oRow = oSrc + NW * 2 * C * 16, oRowG = oRow + NW * C,
                         E_END = oRowG + NW * C;
    static constexpr int SIZE = S_END > E_END ? S_END : E_END;
};

template <int C, int DK, int DV, typename IO>
__global__ void __launch_bounds__(4 * DK) bwd_grad(Args a)
{
    using S = GradLds<C, DK, DV>;
    constexpr int NB = S::NB, NW = S::NW, NT = 64 * NW;
    constexpr int VS = S::VS, NS = DV / VS;
    constexpr int LT = S::LT, LV = S::LV, LE = S::LE, LA = S::LA;
    constexpr int NY = NB * (NB + 1) / 2;
    constexpr int NYS = (2 * NY + NW - 1) / NW;
    __shared__ __align__(16) float smem[S::SIZE];
    __shared__ float sPart[C][NB];
    __shared__ float sDb[C];
    __shared__ float sBeta[C];
    __shared__ float sDgam[DK];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int rec = blockIdx.x;
    const int u = rec / a.NC, ch = rec % a.NC;
    const int b = u / a.H, h = u % a.H, hq = h / (a.H / a.Hq);
    const int t0 = ch * C;
    const int L = min(C, a.T - t0);
    const size_t R = (size_t)rec;
    const size_t DD = (size_t)DK * DV;
    const IO* q = (const IO*)a.q;
    const IO* k = (const IO*)a.k;
    const IO* v = (const IO*)a.v;
    const IO* dO = (const IO*)a.dO;

    float* sT = smem + S::oT;
    float* sH = smem + S::oH;
    float* sdH = smem + S::odH;
    float* sE = smem + S::oE;
    float* sdO = smem + S::odO;
    float* sdU = smem + S::odU;
    float* sV = smem + S::oV;
    float* sdE = smem + S::odE;

    for (int e = tid; e < C * C; e += NT) sT[(e / C) * LT + e % C] = a.r.Tm[R * C * C + e];
    for (int i = tid; i < C; i += NT) sBeta[i] = i < L ? a.beta[tok_v(a, b, t0 + i, h)] : 0.f;
    for (int e = tid; e < C * NB; e += NT) sPart[e / NB][e % NB] = 0.f;

    f32x4 X1[NB], X2[NB], X3[NB], Y[NYS];
#pragma unroll
    for (int I = 0; I < NB; ++I) { X1[I] = zero4(); X2[I] = zero4(); X3[I] = zero4(); }
#pragma unroll
    for (int s = 0; s < NYS; ++s) Y[s] = zero4();
    float zacc = 0.f, gacc = 0.f;

    for (int s = 0; s < NS; ++s) {
        const int v0 = s * VS;
        __syncthreads();
        for (int e = tid; e < DK * VS; e += NT) {
            const int c = e / VS, n = e % VS;
            sH[c * LV + n] = a.r.Hs[R * DD + c * DV + v0 + n];
            sdH[c * LV + n] = a.r.dH[R * DD + c * DV + v0 + n];
        }
        for (int e = tid; e < C * VS; e += NT) {
            const int i = e / VS, n = e % VS;
            sE[i * LV + n] = a.r.E[R * C * DV + i * DV + v0 + n];
            sdE[i * LE + n] = a.r.dE[R * C * DV + i * DV + v0 + n];
            float dov = 0.f, vv = 0.f;
            if (i < L) {
                dov = io<IO>::load(dO + tok_v(a, b, t0 + i, h) * DV + v0 + n);
                vv = io<IO>::load(v + tok_v(a, b, t0 + i, h) * DV + v0 + n);
            }
            sdO[i * LV + n] = dov;
            sV[i * LV + n] = vv;
        }
        __syncthreads();
        // dUt = T^T dE (upper triangular: rows i take j >= 16 I), dv = beta dUt
        for (int job = w; job < NB * (VS / 16); job += NW) {
            const int I = job / (VS / 16), Vt = job % (VS / 16);
            f32x4 acc = zero4();
            for (int kk = 16 * I; kk < C; kk += 4)
                acc = mma4(sT[(kk + q4) * LT + 16 * I + r16], sdE[(kk + q4) * LE + 16 * Vt + r16], acc);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * I + 4 * q4 + ii, n = 16 * Vt + r16;
                sdU[i * LV + n] = acc[ii];
                if (i < L)
                    store_grad(a.dv, tok_v(a, b, t0 + i, h) * DV + v0 + n, sBeta[i] * acc[ii], a.gdt);
            }
        }
        __syncthreads();
        if (tid < C) {
            for (int n = 0; n < VS; ++n) zacc += sdU[tid * LV + n] * sV[tid * LV + n];
        }
        if (tid < DK) {
            for (int n = 0; n < VS; ++n) gacc += sH[tid * LV + n] * sdH[tid * LV + n];
        }
        // products with the state and its gradient for this wave's 16 channels
#pragma unroll
        for (int I = 0; I < NB; ++I) {
#pragma unroll
            for (int kk = 0; kk < VS; kk += 4) {
                const float bH = sH[(16 * w + r16) * LV + kk + q4];
                const float bdH = sdH[(16 * w + r16) * LV + kk + q4];
                X1[I] = mma4(sdO[(16 * I + r16) * LV + kk + q4], bH, X1[I]);
                X2[I] = mma4(sE[(16 * I + r16) * LV + kk + q4], bdH, X2[I]);
                X3[I] = mma4(sdU[(16 * I + r16) * LV + kk + q4], bH, X3[I]);
            }
        }
        // C x C products dO E^T and dUt E^T on the lower block tiles
#pragma unroll
        for (int sl = 0; sl < NYS; ++sl) {
            const int job = w + sl * NW;
            if (job < 2 * NY) {
                int I, J;
                lower_tile(job % NY, I, J);
                const float* A = job >= NY ? sdU : sdO;
#pragma unroll
                for (int kk = 0; kk < VS; kk += 4)
                    Y[sl] = mma4(A[(16 * I + r16) * LV + kk + q4], sE[(16 * J + r16) * LV + kk + q4], Y[sl]);
            }
        }
    }
    __syncthreads();

    // dAqk (inclusive lower) and beta_i dA_ij, dA = -(strict lower of dUt E^T);
    // the dbeta term sum_j dA_ij Ap_ij per tile goes to sPart
    float* sdAq = smem + S::oAq;
    float* sdAb = smem + S::oAb;
    if (tid < DK) sDgam[tid] = gacc;
#pragma unroll
    for (int sl = 0; sl < NYS; ++sl) {
        const int job = w + sl * NW;
        if (job < 2 * NY) {
            int I, J;
            lower_tile(job % NY, I, J);
            if (job < NY) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int i = 16 * I + 4 * q4 + ii, j = 16 * J + r16;
                    sdAq[i * LA + j] = j <= i ? Y[sl][ii] : 0.f;
                }
            } else {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int i = 16 * I + 4 * q4 + ii, j = 16 * J + r16;
                    const float dA = j < i ? -Y[sl][ii] : 0.f;
                    float part = dA * a.r.Ap[R * C * C + i * C + j];
                    part += __shfl_xor(part, 1);
                    part += __shfl_xor(part, 2);
                    part += __shfl_xor(part, 4);
                    part += __shfl_xor(part, 8);
                    if (r16 == 0) sPart[i][J] = part;
                    sdAb[i * LA + j] = sBeta[i] * dA;
                }
            }
        }
    }
    __syncthreads();
    if (tid < C) {
        float s = zacc;
        for (int J = 0; J < NB; ++J) s += sPart[tid][J];
        sDb[tid] = s;
    }

    // output phase: wave w owns key channels 16 w .. 16 w + 15; lane (r16, q4)
    // holds rows 16 I + 4 q4 + ii of channel 16 w + r16
    const int c = 16 * w + r16;
    float* src0 = smem + S::oSrc + w * 2 * C * 16;
    float* src1 = src0 + C * 16;
    float* sRow = smem + S::oRow;
    float* sRowG = smem + S::oRowG;
    float Gd[NB][4], kd[NB][4], qd[NB][4];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * I + 4 * q4 + ii;
            Gd[I][ii] = a.r.G[R * C * DK + i * DK + c];
            float kv = 0.f, qv = 0.f;
            if (i < L) {
                kv = io<IO>::load(k + tok_qk(a, b, t0 + i, hq) * DK + c);
                qv = io<IO>::load(q + tok_qk(a, b, t0 + i, hq) * DK + c);
            }
            kd[I][ii] = kv;
            qd[I][ii] = qv;
        }
    }
    f32x4 dq[NB], Pg[NB], Pinv[NB];
    // sums over earlier tokens j <= i, reference row 16 I
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        const float Gs = __shfl(Gd[I][0], r16);
#pragma unroll
        for (int J = 0; J <= I; ++J) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                src0[(16 * J + 4 * q4 + ii) * 16 + r16] = kd[J][ii] * ex(Gs - Gd[J][ii]);
        }
        __syncthreads();
        f32x4 ra = zero4(), rb = zero4();
        for (int kk = 0; kk < 16 * (I + 1); kk += 4) {
            const float bs = src0[(kk + q4) * 16 + r16];
            ra = mma4(sdAq[(16 * I + r16) * LA + kk + q4], bs, ra);
            rb = mma4(sdAb[(16 * I + r16) * LA + kk + q4], bs, rb);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * I + 4 * q4 + ii;
            const float f = ex(Gd[I][ii] - Gs), eg = ex(Gd[I][ii]);
            dq[I][ii] = a.scale * (eg * X1[I][ii] + f * ra[ii]);
            Pg[I][ii] = -sBeta[i] * eg * X3[I][ii] + f * rb[ii];
        }
        __syncthreads();
    }
    // sums over later tokens i >= j, reference row 16 J + 15
#pragma unroll
    for (int J = NB - 1; J >= 0; --J) {
        const float Ge = __shfl(Gd[J][3], 48 + r16);
#pragma unroll
        for (int I = J; I < NB; ++I) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int row = 16 * I + 4 * q4 + ii;
                const float f = ex(Gd[I][ii] - Ge);
                src0[row * 16 + r16] = kd[I][ii] * f;
                src1[row * 16 + r16] = a.scale * qd[I][ii] * f;
            }
        }
        __syncthreads();
        f32x4 acc = zero4();
        for (int kk = 16 * J; kk < C; kk += 4) {
            acc = mma4(sdAb[(kk + q4) * LA + 16 * J + r16], src0[(kk + q4) * 16 + r16], acc);
            acc = mma4(sdAq[(kk + q4) * LA + 16 * J + r16], src1[(kk + q4) * 16 + r16], acc);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) Pinv[J][ii] = ex(Ge - Gd[J][ii]) * acc[ii];
        __syncthreads();
    }

    // dk, dq, dG; the dbeta term -sum_c (dUt H^T)_ic k_ic e^G_ic
    const float Gl = __shfl(Gd[NB - 1][3], 48 + r16);
    const bool grouped = a.dqp != nullptr;
    float dG[NB][4];
    float colPr = 0.f;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * I + 4 * q4 + ii;
            const float pr = ex(Gl - Gd[I][ii]) * X2[I][ii];
            const float dkv = Pg[I][ii] + Pinv[I][ii] + pr;
            dG[I][ii] = kd[I][ii] * (Pg[I][ii] - Pinv[I][ii] - pr) + qd[I][ii] * dq[I][ii];
            colPr += pr * kd[I][ii];
            float x3 = X3[I][ii] * kd[I][ii] * ex(Gd[I][ii]);
            x3 += __shfl_xor(x3, 1);
            x3 += __shfl_xor(x3, 2);
            x3 += __shfl_xor(x3, 4);
            x3 += __shfl_xor(x3, 8);
            if (r16 == 0) sRow[w * C + i] = x3;
            if (i < L) {
                if (grouped) {
                    const size_t o = tok_v(a, b, t0 + i, h) * DK + c;
                    a.dqp[o] = dq[I][ii];
                    a.dkp[o] = dkv;
                } else {
                    const size_t o = tok_qk(a, b, t0 + i, hq) * DK + c;
                    store_grad(a.dq, o, dq[I][ii], a.gdt);
                    store_grad(a.dk, o, dkv, a.gdt);
                }
            }
        }
    }
    colPr += __shfl_xor(colPr, 16);
    colPr += __shfl_xor(colPr, 32);
    if (q4 == 3) dG[NB - 1][3] += colPr + sDgam[c] * ex(Gl);

    if (a.mode == KDA_GATE_CHANNEL) {
        // dg = suffix sums of dG over the rows of the chunk, per channel
#pragma unroll
        for (int I = 0; I < NB; ++I) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) src0[(16 * I + 4 * q4 + ii) * 16 + r16] = dG[I][ii];
        }
        __syncthreads();
        float seg[16];
        float tot = 0.f;
        if (16 * q4 < C) {
#pragma unroll
            for (int m = 15; m >= 0; --m) {
                tot += src0[(16 * q4 + m) * 16 + r16];
                seg[m] = tot;
            }
        }
        const float t1 = __shfl(tot, r16 + 16), t2 = __shfl(tot, r16 + 32), t3 = __shfl(tot, r16 + 48);
        const float after = (q4 < 1 ? t1 : 0.f) + (q4 < 2 ? t2 : 0.f) + (q4 < 3 ? t3 : 0.f);
        if (16 * q4 < C) {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int i = 16 * q4 + m;
                if (i < L) a.dg[tok_v(a, b, t0 + i, h) * DK + c] = seg[m] + after;
            }
        }
    } else if (a.mode == KDA_GATE_SCALAR) {
#pragma unroll
        for (int I = 0; I < NB; ++I) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                float x = dG[I][ii];
                x += __shfl_xor(x, 1);
                x += __shfl_xor(x, 2);
                x += __shfl_xor(x, 4);
                x += __shfl_xor(x, 8);
                if (r16 == 0) sRowG[w * C + 16 * I + 4 * q4 + ii] = x;
            }
        }
    }
    __syncthreads();
    if (a.mode == KDA_GATE_SCALAR && w == 0) {
        float x = 0.f;
        if (lane < C) {
            for (int ww = 0; ww < NW; ++ww) x += sRowG[ww * C + lane];
        }
        // suffix sums over the rows of the chunk
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(x, off);
            if (lane + off < 64) x += y;
        }
        if (lane < L) a.dg[tok_v(a, b, t0 + lane, h)] = x;
    }
    if (tid < L) {
        float db = sDb[tid];
        for (int ww = 0; ww < NW; ++ww) db -= sRow[ww * C + tid];
        a.dbeta[tok_v(a, b, t0 + tid, h)] = db;
    }
}

// ---------------------------------------------------------------------------
// 4. grouped value heads: dq, dk of a query/key head = sum over its value heads
// ---------------------------------------------------------------------------
template <typename IO>
__global__ void __launch_bounds__(256) bwd_group_sum(const float* dqp, const float* dkp, IO* dq, IO* dk,
                                                     size_t n, int Hq, int G, int DK)
{
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const int c = (int)(e % DK);
    const size_t th = e / DK;                    // (b * T + t) * Hq + hq
    const size_t base = ((th / Hq) * Hq * G + (th % Hq) * G) * DK + c;
    float sq = 0.f, sk = 0.f;
    for (int gg = 0; gg < G; ++gg) {
        sq += dqp[base + (size_t)gg * DK];
        sk += dkp[base + (size_t)gg * DK];
    }
    io<IO>::store(dq + e, sq);
    io<IO>::store(dk + e, sk);
}

}  // namespace bwd
}  // namespace kda

namespace kda {
namespace bwd {

// Launch the three per-chunk / per-tile kernels for one shape.
template <int C, int DK, int DV, typename IO>
hipError_t launch3(const Args& a, hipStream_t s)
{
    const int units = a.B * a.H;
    const unsigned nrec = (unsigned)units * (unsigned)a.NC;
    if (nrec > 0) {
        hipLaunchKernelGGL((bwd_prep<C, DK, DV, IO>), dim3(nrec), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_states<C, DK, DV, IO>), dim3(DV / 16, 2 * units), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nrec > 0) {
        hipLaunchKernelGGL((bwd_grad<C, DK, DV, IO>), dim3(nrec), dim3(4 * DK), 0, s, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace bwd

#define KDA_BWD_CASES(CC)                                                                      \
    KDA_BWD_CASE(CC, 16, 16) KDA_BWD_CASE(CC, 16, 32) KDA_BWD_CASE(CC, 16, 64) KDA_BWD_CASE(CC, 16, 128) \
    KDA_BWD_CASE(CC, 32, 16) KDA_BWD_CASE(CC, 32, 32) KDA_BWD_CASE(CC, 32, 64) KDA_BWD_CASE(CC, 32, 128) \
    KDA_BWD_CASE(CC, 64, 16) KDA_BWD_CASE(CC, 64, 32) KDA_BWD_CASE(CC, 64, 64) KDA_BWD_CASE(CC, 64, 128) \
    KDA_BWD_CASE(CC, 128, 16) KDA_BWD_CASE(CC, 128, 32) KDA_BWD_CASE(CC, 128, 64) KDA_BWD_CASE(CC, 128, 128)

hipError_t launch_bwd_c16(const bwd::Args& a, int Dk, int Dv, kda_dtype dtype, hipStream_t s);
hipError_t launch_bwd_c32(const bwd::Args& a, int Dk, int Dv, kda_dtype dtype, hipStream_t s);
hipError_t launch_bwd_c64(const bwd::Args& a, int Dk, int Dv, kda_dtype dtype, hipStream_t s);

}  // namespace kda
