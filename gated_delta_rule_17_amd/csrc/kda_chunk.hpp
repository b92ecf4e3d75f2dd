// Chunkwise-parallel KDA forward (prefill / training forward): kernels and
// launch templates.  kda_chunk_c16.hip, kda_chunk_c32.hip and kda_chunk_c64.hip
// instantiate them for one chunk length each; kda_chunk.hip dispatches.
//
// GeekNews #31925, section "Chunkwise KDA: recasting the recurrence as matrix
// products" with "Cumulative decay and provisional errors" and "Restoring
// causal dependence"; F29 course outline, Objectives ("pseudo-values from a
// triangular solve; log-space decay ratios", "WY/UT form").
//
// Per (batch, head) and chunk of C tokens i = 0..C-1 entering with state H
// (transposed, Dk x Dv):
//   G_i   = g_0 + ... + g_i                       cumulative log-decay per key channel
//   A_ij  = beta_i sum_c k_i[c] k_j[c] exp(G_i[c] - G_j[c])    j < i
//   T     = (I + A)^-1                            (unit lower triangular)
//   W     = T Diag(beta) (K * exp(G)),  U = T Diag(beta) V    (pseudo-values: E = U - W H)
//   o     = (Q~ * exp(G)) H + Aqk E,  Aqk_ij = sum_c q~_i[c] k_j[c] exp(G_i[c] - G_j[c]), j <= i
//   H'    = Diag(exp G_last) H + (K * exp(G_last - G))^T E
//
// Two kernels:
//  chunk_prepare  persistent workgroups striding over the (b, h, chunk) items,
//                 fully parallel, one wavefront per 16-token x 32-channel tile.
//                 Everything that does not depend on the incoming state: G,
//                 A and Aqk on the matrix cores, the inverted diagonal blocks of
//                 I + A by a column sweep, W and U by block forward
//                 substitution carried in matrix-core accumulators.  Writes one
//                 record per chunk.
//  chunk_state    one workgroup per (b, h, 16 value columns), sequential over
//                 the chunks.  The 16 state columns live in matrix-core
//                 accumulators (float32) for the whole sequence; per chunk:
//                 E = U - W H, o = Qg H + Aqk E, H = gl * H + Kr^T E.
//
// Overflow-free decay ratios.  exp(G_i - G_j) is split into factors that
// each stay <= 1 using reference tokens at 16-token block boundaries: for
// blocks J < I, exp(G_i - G_s(I)) * exp(G_s(I) - G_e(J)) * exp(G_e(J) - G_j)
// with s = first and e = last token of a block.  Inside a diagonal block the
// key side exp(G_s(I) - G_j) >= 1 grows with the decay inside the block; any
// key channel whose decay across one block exceeds kRangeMax is removed from
// that diagonal block's matrix-core product and added exactly, term by term,
// on the vector units instead.
#pragma once

#include <atomic>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

constexpr float kRangeMax = 80.f;
constexpr float kLog2e = 1.4426950408889634f;

// 2^x on the transcendental unit (x in log2 units; underflows to 0)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// log(sigmoid(a)) = min(a, 0) - log(1 + exp(-|a|)), without overflow, on the
// transcendental unit: exp(-|a|) lies in (0, 1], so 1 + exp(-|a|) lies in
// (1, 2] and its log2 carries an absolute error of about 1e-7.  That absolute
// error is what the decays see (they are exponentials of differences of
// prefix sums of these logs).
__device__ __forceinline__ float log_sigmoid(float a) {
    const float e = exp2_fast(-fabsf(a) * kLog2e);
    return fminf(a, 0.f) - __builtin_amdgcn_logf(1.f + e) * (1.f / kLog2e);
}

template <int C, int DK, int DV, typename OT>
struct CS {
    static constexpr int NB = C / 16;                 // 16-token blocks per chunk
    static constexpr int CP = C < 32 ? 32 : C;        // token dim padded to the 32-wide k step
    static constexpr int DKP = DK < 32 ? 32 : DK;     // key dim padded likewise
    static constexpr int PAD = 16 / (int)sizeof(OT);  // LDS row padding (16 bytes)
    static constexpr int SK = DKP + PAD;              // stride of [token][channel] operands
    static constexpr int SKF = DKP + 4;               // stride of the float32 key array
    static constexpr int DVP = DV < 32 ? 32 : DV;     // value dim padded likewise
    static constexpr int SV = DVP + PAD;              // stride of [token][value channel] operands
    static constexpr int VJ = (DVP + DKP - 1) / DKP;  // value loads per lane (8 channels each)
    static constexpr int SC = CP + PAD;               // stride of [channel][token] operands
    static constexpr int SA = C + 4;                  // stride of float32 A / T
    static constexpr int KSN = DKP / 32;              // 32-channel slices
    static constexpr int NW = NB * KSN;               // chunk_prepare wavefronts: one per 16 x 32 tile
    static constexpr int NT = 64 * NW;                // and threads
    static constexpr int NPAIR = NB * (NB - 1) / 2;
    static constexpr bool SPLIT = sizeof(OT) == 2;    // bf16: precise operands are hi/lo pairs
    static constexpr int NP = SPLIT ? 2 : 1;
    static constexpr int SZ = (int)sizeof(OT);
    // per-chunk record, elements per part
    static constexpr size_t W_N = (size_t)C * DKP;    // -W      [C][DKP]   plain
    static constexpr size_t Q_N = (size_t)C * DKP;    // Qg      [C][DKP]   plain
    static constexpr size_t KR_N = (size_t)DK * CP;   // Kr^T    [DK][CP]   precise
    static constexpr size_t AQ_N = (size_t)C * CP;    // Aqk     [C][CP]    precise
    static constexpr size_t U_N = (size_t)DV * C;     // U^T     [DV][C]    float32
    // LDS, stage A: Qk (plain), Qq and Kd (precise), Kk (float32)
    static constexpr int STAGE_A = (1 + 2 * NP) * C * SK * SZ + C * SKF * 4;
    // stage B: the right-hand sides Bk (plain) and Bv (precise) as [token][channel],
    // A off its diagonal blocks (precise), the inverted diagonal blocks of
    // I + A (precise; the Aqk staging of the exact fallback aliases them) and
    // -W staged row-major
    static constexpr int TB_BYTES = (C * SA * 4 > NP * C * SC * SZ) ? C * SA * 4 : NP * C * SC * SZ;
    static constexpr int WS_BYTES = C * SK * SZ;
    static constexpr int STAGE_B = C * SK * SZ + NP * C * SV * SZ + NP * C * SC * SZ + TB_BYTES + WS_BYTES;
    static constexpr int BIG = STAGE_A > STAGE_B ? STAGE_A : STAGE_B;
    static_assert((C * SV * SZ) % 16 == 0, "alignment");
    static_assert(NT <= 1024, "one workgroup");
    static_assert((C * SK * SZ) % 16 == 0 && (C * SC * SZ) % 16 == 0, "alignment");
};

// The per-chunk records inside the workspace: one array per record field
// (hi and lo parts of precise operands are separate arrays of equal layout).
template <int C, int DK, int DV, typename OT>
struct WsLayout {
    using S = CS<C, DK, DV, OT>;
    OT *wneg, *qg, *krt_h, *krt_l, *aqk_h, *aqk_l;
    float *ut, *gl;
    __host__ __device__ WsLayout(void* base, size_t nrec) {
        char* p = (char*)base;
        auto take = [&](size_t elems, size_t sz) { char* r = p; p += nrec * elems * sz; return r; };
        wneg = (OT*)take(S::W_N, S::SZ);
        qg = (OT*)take(S::Q_N, S::SZ);
        krt_h = (OT*)take(S::KR_N, S::SZ);
        krt_l = S::SPLIT ? (OT*)take(S::KR_N, S::SZ) : krt_h;
        aqk_h = (OT*)take(S::AQ_N, S::SZ);
        aqk_l = S::SPLIT ? (OT*)take(S::AQ_N, S::SZ) : aqk_h;
        ut = (float*)take(S::U_N, 4);
        gl = (float*)p;
    }
    static size_t bytes(size_t nrec) {
        return nrec * ((S::W_N + S::Q_N + S::NP * (S::KR_N + S::AQ_N)) * S::SZ + S::U_N * 4 + DK * 4);
    }
    __device__ OT* wneg_rec(size_t rec) const { return wneg + rec * S::W_N; }
    __device__ OT* qg_rec(size_t rec) const { return qg + rec * S::Q_N; }
    __device__ PArr<OT> krt(size_t rec) const { return {krt_h + rec * S::KR_N, krt_l + rec * S::KR_N}; }
    __device__ PArr<OT> aqk(size_t rec) const { return {aqk_h + rec * S::AQ_N, aqk_l + rec * S::AQ_N}; }
};

template <typename OT>
__device__ __forceinline__ void store_op(OT* p, float x) { io<OT>::store(p, x); }

// Fragment-major record layout.  A record operand of logical shape [rows][K]
// (K = 32 * KS) is stored as its 16x32 matrix-core fragments, each fragment as
// 64 lanes x 8 consecutive k-values, so that one wave's fragment load reads
// 1 KiB of contiguous memory.  Element (row, k) lives at:
__device__ __forceinline__ int fragidx(int row, int k, int KS) {
    return (((row >> 4) * KS + (k >> 5)) * 64 + (row & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
}
// start of fragment (row tile, k step) for this lane
__device__ __forceinline__ int fragbase(int rtile, int ks, int KS, int lane) {
    return ((rtile * KS + ks) * 64 + lane) * 8;
}
// U^T is stored accumulator-major: block (value tile nt, token tile it) holds
// 64 lanes x 4 floats, lane (r, g) holding U[16it + 4g + u][16nt + r], u = 0..3.
__device__ __forceinline__ int accbase(int nt, int it, int NB, int lane) {
    return ((nt * NB + it) * 64 + lane) * 4;
}

// Store N consecutive values (N a power of two, p aligned to N elements) of
// a plain operand with one vector store.
template <typename OT, int N>
__device__ __forceinline__ void store_run(OT* p, const float* x)
{
    if constexpr (sizeof(OT) == 2 && N >= 2) {
        typedef uint16_t vec __attribute__((ext_vector_type(N)));
        vec u;
#pragma unroll
        for (int e = 0; e < N; ++e) u[e] = f32_to_bf16(x[e]);
        *reinterpret_cast<vec*>(p) = u;
    } else if constexpr (sizeof(OT) == 4 && N >= 4) {
#pragma unroll
        for (int e = 0; e < N; e += 4)
            *reinterpret_cast<f32x4*>(p + e) = (f32x4){x[e], x[e + 1], x[e + 2], x[e + 3]};
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) io<OT>::store(p + e, x[e]);
    }
}

// Column swizzle of a [row][CP] operand that is written column-wise: the
// 8-column group of (row, j) is XOR-ed with row / 8, so that the rows 8 apart
// written by one store instruction fall into different LDS banks.  Runs of 8
// columns stay contiguous, so fragment reads are unchanged in cost.
template <int CP>
__device__ __forceinline__ int swz(int row, int j) {
    return ((((j >> 3) ^ (row >> 3)) & (CP / 8 - 1)) << 3) | (j & 7);
}

// Store N consecutive values of a precise operand with the widest aligned stores
// (N is a power of two; idx is a multiple of N).
template <typename OT, int N>
__device__ __forceinline__ void store_run(const PArr<OT>& a, int idx, const float* x)
{
    if constexpr (N >= 4) {
#pragma unroll
        for (int u = 0; u < N; u += 4)
            store4_p(a, idx + u, (f32x4){x[u], x[u + 1], x[u + 2], x[u + 3]});
    } else {
#pragma unroll
        for (int u = 0; u < N; ++u) store_p(a, idx + u, x[u]);
    }
}

// Value held by lane J of this lane's 16-lane row (DPP row broadcast).
template <int J>
__device__ __forceinline__ float row_lane(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + J, 0xf, 0xf, false));
}

// Column sweep of forward substitution for X = (I + A)^-1 of one 16x16 unit
// lower triangular block: lane (r, g) holds row r of A in arow and
// X[r][4g .. 4g+3] in x (initially the identity).  Step J eliminates column J
// from every later row using row J of X, broadcast within each 16-lane row.
template <int J>
__device__ __forceinline__ void sweep16(float (&x)[4], const float (&arow)[16], int r) {
    if constexpr (J < 15) {
        float xj[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xj[u] = row_lane<J>(x[u]);
        if (r > J) {
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] -= arow[J] * xj[u];
        }
        sweep16<J + 1>(x, arow, r);
    }
}

// ---------------------------------------------------------------------------
// chunk_prepare
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 16 lanes of a row (DPP row shifts; a lane
// shifted in from outside the row contributes 0).
__device__ __forceinline__ float row_scan16(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
    return x;
}

// Right operand (32 x 16) that picks columns 16hh .. 16hh+15 out of a 16 x 32
// left operand: lane (r, g) holds B[8g + e][r] = (8g + e == 16hh + r).  The
// product D = A B is then an exact transpose into the accumulator layout,
// lane (r, g) receiving A[4g + u][16hh + r] (one nonzero term per sum).
template <typename OT>
__device__ __forceinline__ Frag<OT> select_frag(int hh, int lane) {
    Frag<OT> f;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.set(e, (8 * g + e == 16 * hh + r) ? 1.f : 0.f);
    return f;
}
// bf16: the single one (0x3f80) is placed into its 32-bit word directly
template <>
__device__ __forceinline__ Frag<bf16_t> select_frag<bf16_t>(int hh, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const int e = 16 * hh + r - 8 * g;                       // position of the one, if in [0, 8)
    const uint32_t one = (unsigned)e < 8u ? (0x3f80u << (16 * (e & 1))) : 0u;
    const int d = e >> 1;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {d == 0 ? one : 0u, d == 1 ? one : 0u, d == 2 ? one : 0u, d == 3 ? one : 0u};
    Frag<bf16_t> f;
    f.v = __builtin_bit_cast(u16x8, w);
    return f;
}

// PRO: the fused prologue is compiled in (its flags are then read from
// `pro`); without it the prologue code is absent and `pro` is ignored.
template <int C, int DK, int DV, typename OT, bool PRO>
__global__ void __launch_bounds__((CS<C, DK, DV, OT>::NT))
chunk_prepare(const OT* __restrict__ q, const OT* __restrict__ k, const OT* __restrict__ v,
              const float* __restrict__ g, const float* __restrict__ beta,
              int T, int H, int HQ, int NC, int NITEM, float scale, int mode, void* __restrict__ ws,
              size_t nrec, const int2* __restrict__ ctab, int pro)
{
    using S = CS<C, DK, DV, OT>;
    constexpr int NB = S::NB, CP = S::CP, DKP = S::DKP, SK = S::SK, SKF = S::SKF, SC = S::SC,
                  SA = S::SA, NP = S::NP, KSN = S::KSN, SV = S::SV, DVP = S::DVP, VJ = S::VJ;
    // grouped value heads: value head h reads query/key head h / GH
    const int GH = H / HQ;

    // Where an item's chunk lives: the token index of its first token (tokens
    // are [*, H, D] rows) and its number of valid tokens.  Dense batches: item
    // = (b*H + h) * NC + chunk over [B, T].  Packed variable-length batches
    // (ctab != null): item = g * H + h over the chunk table, whose entry g is
    // (first token, length); entries past the last chunk have length 0.
    struct Loc { size_t tok0; int L, h; };
    auto locate = [&](int item) {
        Loc l;
        if (ctab) {
            const int gch = item / H;
            l.h = item - gch * H;
            const int2 e = ctab[gch];
            l.tok0 = (size_t)e.x;
            l.L = e.y;
        } else {
            const int bh = item / NC, c_idx = item - bh * NC;
            const int b = bh / H;
            l.h = bh - b * H;
            l.tok0 = (size_t)b * T + (size_t)c_idx * C;
            l.L = min(C, T - c_idx * C);
        }
        return l;
    };

    __shared__ __align__(16) char big[S::BIG];
    __shared__ float sb[C];
    __shared__ __align__(16) float btot[NB][DKP];       // per-block totals of the log2 decay
    __shared__ __align__(16) float bfirst[NB][DKP];     // and its first term
    __shared__ __align__(16) float eSb[NB][DKP];        // exp(G at the block's first token)
    __shared__ __align__(16) float eLb[NB][DKP];        // exp(G_last - G at the block's last token)
    __shared__ float nrm[KSN][2][C];                    // partial sums of k^2, q^2 per slice
    __shared__ float inrm[2][C];                        // 1 / norm of k and of q per token
    __shared__ __align__(16) float fpair[S::NPAIR > 0 ? S::NPAIR : 1][DKP];
    __shared__ __align__(8) unsigned char flag[NB][DKP];
    __shared__ int anyflag;
    __shared__ __align__(16) float Ads[NB * 16 * 20];   // diagonal blocks of A (float32)

    const WsLayout<C, DK, DV, OT> W(ws, nrec);

    // Work layout: wavefront (I, ks) owns the 16 x 32 tile of tokens
    // 16I .. 16I+15 and key channels 32ks .. 32ks+31 of its chunk, lane (r, gq)
    // the token 16I + r and the channels 32ks + 8gq .. +7: the matrix-core
    // fragment layout of the [token][channel] operands.  Every global load
    // and every operand store is then 16 bytes wide, and the cumulative decay
    // inside a block is a scan over the 16 lanes of a row.  The value
    // channels follow the same pattern, ch + DKP*j for j < VJ.
    struct In {
        f32x4 g0, g1;          // per-channel log-gates of the 8 channels
        float gt;              // per-token log-gate
        Frag<OT> k, q, v[VJ];
        float b;               // beta of the token
    };
    auto load_in = [&](In& x, int item, int tid, int grp) {
        const int wv = tid >> 6, ln = tid & 63;
        const int I = wv / KSN, ksl = wv - I * KSN;
        const int ch = 32 * ksl + 8 * (ln >> 4);
        const int chc = ch < DK ? ch : 0;                  // padded channels read channel 0
        const Loc l = locate(item);
        const int i = 16 * I + (ln & 15);
        const size_t row = l.tok0 + (size_t)(i < l.L ? i : max(l.L - 1, 0));
        const size_t tok = row * H + l.h;                  // value-head row: v, g, beta
        const size_t tkq = row * HQ + l.h / GH;            // its query/key row
        // Both gate forms are loaded unconditionally, from valid addresses, so
        // that no branch joins loaded registers (a join would force a wait for
        // the loads right where they are issued); the unused form is never
        // read.  Without per-channel gates the 32 bytes at the start of the
        // token's key row (DK >= 16) stand in, without a per-token gate beta.
        if (grp == 0) {
            const float* gch = mode == KDA_GATE_CHANNEL ? g + tok * DK + chc
                                                        : reinterpret_cast<const float*>(k + tkq * DK);
            x.g0 = *reinterpret_cast<const f32x4*>(gch);
            x.g1 = *reinterpret_cast<const f32x4*>(gch + 4);
            x.gt = *(mode == KDA_GATE_SCALAR ? g + tok : beta + tok);
        } else if (grp == 1) {
            x.k.load(k + tkq * DK + chc);
            x.b = beta[tok];
        } else if (grp == 2) {
            x.q.load(q + tkq * DK + chc);
        } else {
#pragma unroll
            for (int j = 0; j < VJ; ++j) {
                const int vch = ch + DKP * j;
                x.v[j].load(v + tok * DV + (vch < DV ? vch : 0));   // padded channels read channel 0
            }
        }
    };
    // Make loaded values available at this point (the wait for their loads
    // is placed here).
    auto settle = [&](In& x) {
        asm volatile("" : "+v"(x.g0), "+v"(x.g1), "+v"(x.gt), "+v"(x.b));
        x.k.settle();
        x.q.settle();
#pragma unroll
        for (int j = 0; j < VJ; ++j) x.v[j].settle();
    };
    // eight consecutive values of a precise operand, hi and lo parts
    auto store8_p = [&](const PArr<OT>& a, int idx, const float* x) {
        PFrag<OT> f;
        f.from_f32(x);
        f.h.store(a.h + idx);
        if constexpr (S::SPLIT) f.l.store(a.l + idx);
    };

    // Persistent workgroups: item = (b*H + h) * NC + chunk, strided by the
    // grid.  The inputs of the next item are requested at the start of the
    // current one and taken after its matrix-core phases.
    int item = blockIdx.x;
    if (item >= NITEM) return;
    In cur;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) load_in(cur, item, threadIdx.x, grp);
    settle(cur);
    for (; item < NITEM; item += gridDim.x) {
        // Thread indices are re-derived in every iteration from a value the
        // compiler cannot see through, so that it does not hoist every
        // per-lane address of the item out of the loop (which would keep them
        // all live at once and spill).
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int r = lane & 15, gq = lane >> 4;
        const int Ib = wave / KSN, ksl = wave - Ib * KSN;   // this wave's block and channel slice
        const int ch = 32 * ksl + 8 * gq;                   // this lane's first channel
        const int it = 16 * Ib + r;                         // this lane's token
        // stage-A arrays
        OT* Qk = (OT*)big;                                             // [C][SK] plain
        const PArr<OT> Qq{Qk + C * SK, Qk + 2 * C * SK};               // [C][SK] precise
        const PArr<OT> Kd{Qk + (1 + NP) * C * SK, Qk + (2 + NP) * C * SK};  // [C][SK] precise
        float* Kk = (float*)(Qk + (1 + 2 * NP) * C * SK);              // [C][SKF] float32

        const int nitem = min(item + (int)gridDim.x, NITEM - 1);
        // the next item's inputs, requested in four groups over the phases
        // (gates here, then k and beta, q, v), so that their transfer overlaps
        // the computation instead of stalling instruction issue in one burst
        In nxt;

        const Loc loc = locate(item);
        const int L = loc.L;                // valid tokens
        const int h = loc.h;
        // the chunk table ends in empty entries, and the items of one workgroup
        // only grow: nothing is left for this workgroup (uniform)
        if (L <= 0) break;
        const size_t rec = (size_t)item;
        OT* const Wq = W.qg_rec(rec);
        OT* const Wwn = W.wneg_rec(rec);
        const PArr<OT> Wkr = W.krt(rec), Waq = W.aqk(rec);
        float* Wut = W.ut + rec * S::U_N;
        if (tid == 0) anyflag = 0;
        const bool tv = it < L;
        // beta, or sigmoid of a pre-activation
        const float bet = (PRO && (pro & KDA_BETA_SIGMOID)) ? 1.f / (1.f + expf(-cur.b)) : cur.b;
        if (ksl == 0 && gq == 0) sb[it] = tv ? bet : 0.f;
        float gl[8], kv[8], qv[8];
        float pk = 0.f, pq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool ok = tv && (DK % 32 == 0 || ch + e < DK);   // (padded channels only when DK < 32)
            float gv = mode == KDA_GATE_CHANNEL ? (e < 4 ? cur.g0[e] : cur.g1[e - 4]) : cur.gt;
            if (PRO && (pro & KDA_GATE_LOGSIGMOID)) gv = log_sigmoid(gv);
            gl[e] = (ok && mode != KDA_GATE_NONE) ? gv * kLog2e : 0.f;   // log2 units
            kv[e] = ok ? cur.k.get(e) : 0.f;
            qv[e] = ok ? cur.q.get(e) * scale : 0.f;
            if constexpr (PRO) {
                pk += kv[e] * kv[e];
                pq += qv[e] * qv[e];
            }
        }
        // L2 normalisation of q and k: the sums of squares of token `it` over
        // this wave's 32 channels (the four lanes holding them), one partial
        // per slice to LDS; the scales are taken after the next barrier
        if (PRO && (pro & KDA_NORMALIZE_QK)) {
            pk += __shfl_xor(pk, 16);
            pk += __shfl_xor(pk, 32);
            pq += __shfl_xor(pq, 16);
            pq += __shfl_xor(pq, 32);
            if (gq == 0) {
                nrm[ksl][0][it] = pk;
                nrm[ksl][1][it] = pq;
            }
        }

        // ---- cumulative log-decay, in log2 units from here on (every decay
        // factor is one 2^x): inside the block by a scan over the row, the
        // block totals through LDS.
#pragma unroll
        for (int e = 0; e < 8; ++e) gl[e] = row_scan16(gl[e]);
        if (r == 0) {
            *reinterpret_cast<f32x4*>(&bfirst[Ib][ch]) = (f32x4){gl[0], gl[1], gl[2], gl[3]};
            *reinterpret_cast<f32x4*>(&bfirst[Ib][ch + 4]) = (f32x4){gl[4], gl[5], gl[6], gl[7]};
        }
        if (r == 15) {
            *reinterpret_cast<f32x4*>(&btot[Ib][ch]) = (f32x4){gl[0], gl[1], gl[2], gl[3]};
            *reinterpret_cast<f32x4*>(&btot[Ib][ch + 4]) = (f32x4){gl[4], gl[5], gl[6], gl[7]};
        }
        __syncthreads();
        load_in(nxt, nitem, tid, 0);
        if (PRO && (pro & KDA_NORMALIZE_QK)) {
            float sk2 = 0.f, sq2 = 0.f;
#pragma unroll
            for (int j = 0; j < KSN; ++j) {
                sk2 += nrm[j][0][it];
                sq2 += nrm[j][1][it];
            }
            const float fk = rsqrtf(sk2 + kNormEps);
            // qv holds scale * q: its norm is taken over q itself
            const float fq = scale != 0.f ? rsqrtf(sq2 / (scale * scale) + kNormEps) : 1.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kv[e] *= fk;
                qv[e] *= fq;
            }
            if (ksl == 0 && gq == 0) {
                inrm[0][it] = fk;
                inrm[1][it] = fq;
            }
        }
        // ---- the factors of one (block I, channel c): a left-to-right pass
        // over the block totals (the same order everywhere) gives G at the
        // block boundaries; from them exp(G_s(I)), exp(G_last - G_e(I)), the
        // cross-block factors exp(G_s(I) - G_e(J)), J < I, the range flag and,
        // once per channel, the exp(G_last) record
        for (int job = tid; job < NB * DKP; job += S::NT) {
            const int I = job / DKP, c = job - I * DKP;
            float acc = 0.f, off = 0.f, gend[NB];
#pragma unroll
            for (int J = 0; J < NB; ++J) {
                if (J == I) off = acc;
                acc += btot[J][c];
                gend[J] = acc;
            }
            const float g0 = bfirst[I][c], gt = btot[I][c];
            eSb[I][c] = exp2_fast(off + g0);
            eLb[I][c] = exp2_fast(acc - (off + gt));
            const bool bad = (g0 - gt) > kRangeMax * kLog2e;
            flag[I][c] = bad ? 1 : 0;
            if (bad) anyflag = 1;
#pragma unroll
            for (int J = 0; J < NB - 1; ++J)
                if (J < I) fpair[I * (I - 1) / 2 + J][c] = exp2_fast(off + g0 - gend[J]);
            if (I == 0 && c < DK) W.gl[rec * DK + c] = exp2_fast(acc);
        }
        __syncthreads();
        load_in(nxt, nitem, tid, 1);

        // ---- element-wise operands of token `it`, channels ch .. ch+7, each
        // group stored as soon as it is formed
        float gs[8], ge[8], eg[8];
        unsigned int badbits = 0;
        {
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(&bfirst[Ib][ch]);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(&bfirst[Ib][ch + 4]);
            const f32x4 t0v = *reinterpret_cast<const f32x4*>(&btot[Ib][ch]);
            const f32x4 t1v = *reinterpret_cast<const f32x4*>(&btot[Ib][ch + 4]);
            const uint64_t fb = *reinterpret_cast<const uint64_t*>(&flag[Ib][ch]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gs[e] = e < 4 ? s0[e] : s1[e - 4];     // at the block's first token (local)
                ge[e] = e < 4 ? t0v[e] : t1v[e - 4];   // at the block's last token (local)
                badbits |= ((fb >> (8 * e)) & 1u) << e;
            }
        }
        {
            const f32x4 es0 = *reinterpret_cast<const f32x4*>(&eSb[Ib][ch]);
            const f32x4 es1 = *reinterpret_cast<const f32x4*>(&eSb[Ib][ch + 4]);
            float qk[8], qq[8], qg[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = exp2_fast(gl[e] - gs[e]);              // <= 1
                eg[e] = x * (e < 4 ? es0[e] : es1[e - 4]);             // exp(G_i) <= 1
                qk[e] = kv[e] * x;
                qq[e] = qv[e] * x;
                qg[e] = qv[e] * eg[e];
            }
            store_run<OT, 8>(Qk + it * SK + ch, qk);
            store8_p(Qq, it * SK + ch, qq);
            // Qg record: one 16-byte store per lane, a wave's tile is 1 KiB of
            // contiguous record
            store_run<OT, 8>(Wq + fragidx(it, ch, KSN), qg);
        }
        {
            float kd[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                kd[e] = (badbits >> e) & 1u ? 0.f : kv[e] * exp2_fast(gs[e] - gl[e]);   // >= |k|, bounded
            store8_p(Kd, it * SK + ch, kd);
        }
        {
            const f32x4 el0 = *reinterpret_cast<const f32x4*>(&eLb[Ib][ch]);
            const f32x4 el1 = *reinterpret_cast<const f32x4*>(&eLb[Ib][ch + 4]);
            float kk[8], kr[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kk[e] = kv[e] * exp2_fast(ge[e] - gl[e]);              // <= |k|
                kr[e] = kk[e] * (e < 4 ? el0[e] : el1[e - 4]);         // k exp(G_last - G_i)
            }
            *reinterpret_cast<f32x4*>(Kk + it * SKF + ch) = (f32x4){kk[0], kk[1], kk[2], kk[3]};
            *reinterpret_cast<f32x4*>(Kk + it * SKF + ch + 4) = (f32x4){kk[4], kk[5], kk[6], kk[7]};
            // Kr^T record, transposed on the matrix cores: a lane then holds
            // four consecutive tokens of one channel
            PFrag<OT> kf;
            kf.from_f32(kr);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                if (32 * ksl + 16 * hh < DK) {
                    const Frag<OT> sel = select_frag<OT>(hh, lane);
                    const int idx = fragidx(32 * ksl + 16 * hh + r, 16 * Ib + 4 * gq, CP / 32);
                    Vec4<OT>::store(Wkr.h + idx, mma(kf.h, sel, zero4()));
                    if constexpr (S::SPLIT) Vec4<OT>::store(Wkr.l + idx, mma(kf.l, sel, zero4()));
                }
            }
        }
        load_in(nxt, nitem, tid, 2);
        // beta_i k_i exp(G_i), kept (in the plain operand type) for the
        // right-hand side of the solve
        Frag<OT> bk;
#pragma unroll
        for (int e = 0; e < 8; ++e) bk.set(e, bet * kv[e] * eg[e]);
        if (CP > C) {   // zero the padded token columns of Kr^T and Aqk
            for (int p = tid; p < DK * (CP - C); p += S::NT) {
                const int cc = p / (CP - C), i = C + p % (CP - C);
                store_p(Wkr, fragidx(cc, i, CP / 32), 0.f);
            }
            for (int p = tid; p < C * (CP - C); p += S::NT) {
                const int i = p / (CP - C), j = C + p % (CP - C);
                store_p(Waq, fragidx(i, j, CP / 32), 0.f);
            }
        }
        __syncthreads();


        // ---- A^T and Aqk^T tiles on the matrix cores: tile (J, I), J <= I
        // lane result: A[i = 16I + r][j = 16J + 4gq + u]
        constexpr int NTILE = NB * (NB + 1) / 2;
        constexpr int NW = S::NW;
        constexpr int TPW = (NTILE + NW - 1) / NW;
        f32x4 accA[TPW], accQ[TPW];
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            accA[s] = zero4();
            accQ[s] = zero4();
            const int tix = wave + NW * s;
            if (tix < NTILE) {
                int I = 0, base = 0;
                while (base + I + 1 <= tix) { base += I + 1; ++I; }
                const int J = tix - base;
                const bool diag = (I == J);
                const int pi = diag ? 0 : I * (I - 1) / 2 + J;
#pragma unroll
                for (int ks = 0; ks < DKP / 32; ++ks) {
                    const int ch = 32 * ks + 8 * gq;
                    PFrag<OT> key;
                    if (diag) {
                        key = Kd.frag((16 * J + r) * SK + ch);
                    } else {
                        float t8[8];
                        const f32x4 k0 = *reinterpret_cast<const f32x4*>(Kk + (16 * J + r) * SKF + ch);
                        const f32x4 k1 = *reinterpret_cast<const f32x4*>(Kk + (16 * J + r) * SKF + ch + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            t8[e] = k0[e] * fpair[pi][ch + e];
                            t8[4 + e] = k1[e] * fpair[pi][ch + 4 + e];
                        }
                        key.from_f32(t8);
                    }
                    Frag<OT> bk;
                    bk.load(Qk + (16 * I + r) * SK + ch);
                    const PFrag<OT> bq = Qq.frag((16 * I + r) * SK + ch);
                    accA[s] = mma(key.h, bk, accA[s]);
                    accQ[s] = mma3(key, bq, accQ[s]);
                }
            }
        }
        __syncthreads();   // stage-A operands are dead from here on
        load_in(nxt, nitem, tid, 3);

        // stage-B layout (aliases stage A)
        OT* const XW = (OT*)big;                            // [C][SK] beta_j k_j exp(G_j), plain
        OT* const xu_h = XW + C * SK;
        const PArr<OT> XU{xu_h, xu_h + C * SV};           // [C][SV] beta_j v_j, precise
        OT* const m_h = xu_h + NP * C * SV;
        const PArr<OT> Mp{m_h, m_h + C * SC};             // [C][SC] A below the diagonal blocks, precise
        OT* const tb_h = m_h + NP * C * SC;
        const PArr<OT> Tb{tb_h, tb_h + C * SC};           // [C][SC] (I + A_II)^-1 on the diagonal blocks
        float* const Aq32 = (float*)tb_h;                  // [C][SA] Aqk staging of the exact fallback (dead before Tb)
        OT* const Wst = (OT*)((char*)tb_h + S::TB_BYTES);  // [C][SK] -W, plain, row-major (staging of the record)
        auto ad = [&](int I, int ii, int jj) -> float& { return Ads[(I * 16 + ii) * 20 + jj]; };
        const bool fallback = anyflag != 0;

#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int tix = wave + NW * s;
            if (tix < NTILE) {
                int I = 0, base = 0;
                while (base + I + 1 <= tix) { base += I + 1; ++I; }
                const int J = tix - base;
                const int i = 16 * I + r;
                const int j0 = 16 * J + 4 * gq;
                f32x4 av = accA[s] * sb[i];
                f32x4 qv = accQ[s];
                if (I == J) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (j0 + u >= i) av[u] = 0.f;
                        if (j0 + u > i) qv[u] = 0.f;
                    }
                    *reinterpret_cast<f32x4*>(&ad(I, r, 4 * gq)) = av;
                } else {
                    store4_p(Mp, i * SC + j0, av);
                }
                if (fallback) *reinterpret_cast<f32x4*>(Aq32 + i * SA + j0) = qv;
                else store4_p(Waq, fragidx(i, j0, CP / 32), qv);
            }
        }
        // zero the strictly upper blocks of the Aqk staging / record, eight
        // columns at a time (a run of 8 is contiguous in the fragment layout)
        for (int p = tid; p < C * (C / 8); p += S::NT) {
            const int i = p / (C / 8), j8 = 8 * (p % (C / 8));
            if ((j8 >> 4) > (i >> 4)) {
                if (fallback) {
                    *reinterpret_cast<f32x4*>(Aq32 + i * SA + j8) = zero4();
                    *reinterpret_cast<f32x4*>(Aq32 + i * SA + j8 + 4) = zero4();
                } else {
                    store4_p(Waq, fragidx(i, j8, CP / 32), zero4());
                    store4_p(Waq, fragidx(i, j8, CP / 32) + 4, zero4());
                }
            }
        }
        // beta_j k_j exp(G_j) and beta_j v_j, rows of 8 channels
        bk.store(XW + it * SK + ch);
#pragma unroll
        for (int j = 0; j < VJ; ++j) {
            const int vch = ch + DKP * j;
            if (vch < DVP) {
                float bv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) bv[e] = (tv && vch + e < DV) ? bet * cur.v[j].get(e) : 0.f;
                store8_p(XU, it * SV + vch, bv);
            }
        }
        __syncthreads();

        if (fallback) {
            // Exact diagonal-block terms for the key channels whose decay across a
            // block exceeds kRangeMax (their factorised key side was zeroed above).
            // Wave (Ib, ksl) owns block Ib and the 32 channels of slice ksl and
            // walks its flagged channels in ascending order.  For each, every lane
            // (r, gq) reloads token 16 Ib + r of that channel (the four lane groups
            // hold the same values), the block-local log2 prefix of the gate is a
            // row scan, and lane (r, gq) sums the terms of the entries
            // (i = 16 Ib + r, j = 16 Ib + 4 gq + u):
            //   Aqk_ij += q_i k_j 2^(G_i - G_j),   A_ij += beta_i k_i k_j 2^(G_i - G_j),
            // every factor <= 1.  The next channel's values are requested before
            // the current one is summed.  The slices then add their sums to the
            // block one after another, so the result does not depend on wave timing.
            uint32_t fmask = 0;
#pragma unroll
            for (int c = 0; c < 32; ++c)
                if (32 * ksl + c < DK && flag[Ib][32 * ksl + c]) fmask |= 1u << c;
            float pq[4] = {0.f, 0.f, 0.f, 0.f}, pa[4] = {0.f, 0.f, 0.f, 0.f};
            if (fmask) {   // uniform over the wave
                const size_t row = loc.tok0 + (tv ? it : 0);
                const float* grow = mode == KDA_GATE_CHANNEL ? g + (row * H + h) * DK + 32 * ksl
                                                             : g + row * H + h;
                const OT* krow = k + (row * HQ + h / GH) * DK + 32 * ksl;
                const OT* qrow = q + (row * HQ + h / GH) * DK + 32 * ksl;
                const int gstep = mode == KDA_GATE_CHANNEL ? 1 : 0;
                const float fk = (PRO && (pro & KDA_NORMALIZE_QK)) ? inrm[0][it] : 1.f;
                const float fq = (PRO && (pro & KDA_NORMALIZE_QK)) ? inrm[1][it] : 1.f;
                const float bi = sb[it];
                uint32_t m = fmask;
                int cn = __builtin_ctz(m);
                float gn = grow[gstep * cn], kn = io<OT>::load(krow + cn), qn = io<OT>::load(qrow + cn);
                while (m) {
                    m &= m - 1;
                    float gv = gn;
                    const float kv = tv ? kn * fk : 0.f, qv = tv ? qn * scale * fq : 0.f;
                    cn = m ? __builtin_ctz(m) : cn;            // uniform
                    gn = grow[gstep * cn];
                    kn = io<OT>::load(krow + cn);
                    qn = io<OT>::load(qrow + cn);
                    if (PRO && (pro & KDA_GATE_LOGSIGMOID)) gv = log_sigmoid(gv);
                    const float G = row_scan16(tv ? gv * kLog2e : 0.f);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int jj = 4 * gq + u;
                        const float Gj = __shfl(G, 16 * gq + jj), kj = __shfl(kv, 16 * gq + jj);
                        if (jj <= r) {
                            const float w = exp2_fast(G - Gj) * kj;
                            pq[u] += qv * w;
                            if (jj < r) pa[u] += bi * kv * w;
                        }
                    }
                }
            }
            for (int sl = 0; sl < KSN; ++sl) {
                if (ksl == sl && fmask) {
                    const int i = 16 * Ib + r, j0 = 16 * Ib + 4 * gq;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        Aq32[i * SA + j0 + u] += pq[u];
                        ad(Ib, r, 4 * gq + u) += pa[u];
                    }
                }
                __syncthreads();
            }
            for (int p = tid; p < C * C; p += S::NT) {
                const int i = p / C, j = p % C;
                store_p(Waq, fragidx(i, j, CP / 32), Aq32[i * SA + j]);
            }
            __syncthreads();
        }

        // ---- diagonal blocks of T = (I + A)^-1 by a column sweep (one wave each)
        if (wave < NB) {
            const int I = wave;
            float arow[16];
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) arow[jj] = ad(I, r, jj);
            float x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = (4 * gq + u == r) ? 1.f : 0.f;
            sweep16<0>(x, arow, r);
            store4_p(Tb, (16 * I + r) * SC + 16 * I + 4 * gq, (f32x4){x[0], x[1], x[2], x[3]});
        }
        __syncthreads();
        // the next item's inputs were requested several phases ago: take them now,
        // before the record stores of the last phases (whose completion a later
        // wait would also include)
        settle(nxt);

        // ---- W = T Diag(beta) (K exp(G)) and U = T Diag(beta) V by block forward
        // substitution over the 16-token block rows:
        //   X_I = T_II (B_I - sum_{J<I} A_IJ X_J)      (X = W with B = Bk, X = U with B = Bv)
        // One wavefront per 16-column tile of W or U carries the whole recursion
        // in registers: an accumulator (lane: rows 4gq..4gq+3, column r) is
        // exactly the right operand of a 16-wide matrix-core product, so X_J
        // feeds the products with A_IJ and T_II without leaving the registers.
        {
            // the right-hand side at tokens jb .. jb+3 of channel `row`
            // (accumulator layout) from a [token][channel] array
            auto col4 = [&](const OT* a, int jb, int row, int stride) {
                f32x4 x;
#pragma unroll
                for (int u = 0; u < 4; ++u) x[u] = io<OT>::load(a + (jb + u) * stride + row);
                return x;
            };
            constexpr int MW = DK / 16, NTL = DK / 16 + DV / 16;
            for (int tix = wave; tix < NTL; tix += S::NW) {
                const bool isw = tix < MW;
                const int n = isw ? tix : tix - MW;
                const int row = 16 * n + r;      // channel of the right-hand side
                if constexpr (S::SPLIT) {
                    // bf16 operands: U from precise products throughout; W (stored
                    // plain) from plain products with A_IJ and a precise one with
                    // T_II; -X_J is split into bf16 parts once.  Every LDS operand
                    // of the recursion (right-hand sides, A_IJ, T_II) is read up
                    // front, so that only the matrix-core chain remains serial.
                    constexpr int NPR = NB * (NB - 1) / 2 > 0 ? NB * (NB - 1) / 2 : 1;
                    auto ld4 = [&](const OT* p) { return *reinterpret_cast<const s16x4*>(p); };
                    f32x4 R[NB];
                    s16x4 th[NB], tl[NB], mh[NPR], ml[NPR];
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        const int jb = 16 * I + 4 * gq;
                        R[I] = isw ? col4(XW, jb, row, SK) : col4(XU.h, jb, row, SV) + col4(XU.l, jb, row, SV);
                        const int ti = (16 * I + r) * SC + 16 * I + 4 * gq;
                        th[I] = ld4(Tb.h + ti);
                        tl[I] = ld4(Tb.l + ti);
#pragma unroll
                        for (int J = 0; J < I; ++J) {
                            const int mi = (16 * I + r) * SC + 16 * J + 4 * gq;
                            mh[I * (I - 1) / 2 + J] = ld4(Mp.h + mi);
                            if (!isw) ml[I * (I - 1) / 2 + J] = ld4(Mp.l + mi);
                        }
                    }
                    B16 negx[NB];                // -X_J, lane: X[16J + 4gq + u][16n + r]
                    if (isw) {
#pragma unroll
                        for (int I = 0; I < NB; ++I) {
                            f32x4 x = R[I];
#pragma unroll
                            for (int J = 0; J < I; ++J) x = mma16v(mh[I * (I - 1) / 2 + J], negx[J].h, x);
                            const f32x4 y = mma16v_p(th[I], tl[I], B16::from(x), zero4());
                            negx[I] = B16::plain(-y);
                            const int jb = 16 * I + 4 * gq;
#pragma unroll
                            for (int u = 0; u < 4; ++u) store_op(Wst + (jb + u) * SK + 16 * n + r, -y[u]);
                        }
                    } else {
#pragma unroll
                        for (int I = 0; I < NB; ++I) {
                            f32x4 x = R[I];
#pragma unroll
                            for (int J = 0; J < I; ++J)
                                x = mma16v_p(mh[I * (I - 1) / 2 + J], ml[I * (I - 1) / 2 + J], negx[J], x);
                            const f32x4 y = mma16v_p(th[I], tl[I], B16::from(x), zero4());
                            negx[I] = B16::from(-y);
                            // accumulator-major block (n, I) of the U^T record
                            Vec4<float>::store(Wut + accbase(n, I, NB, lane), y);
                        }
                    }
                } else {
                    f32x4 negx[NB];
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        const int jb = 16 * I + 4 * gq;
                        f32x4 R = isw ? col4(XW, jb, row, SK) : col4(XU.h, jb, row, SV);
#pragma unroll
                        for (int J = 0; J < I; ++J) {
                            const int mi = (16 * I + r) * SC + 16 * J + 4 * gq;
                            R = mma16_p(Mp.h + mi, Mp.l + mi, negx[J], R);
                        }
                        const int ti = (16 * I + r) * SC + 16 * I + 4 * gq;
                        const f32x4 y = mma16_p(Tb.h + ti, Tb.l + ti, R, zero4());
                        negx[I] = -y;
                        if (isw) {
#pragma unroll
                            for (int u = 0; u < 4; ++u) store_op(Wst + (jb + u) * SK + 16 * n + r, -y[u]);
                        } else {
                            Vec4<float>::store(Wut + accbase(n, I, NB, lane), y);
                        }
                    }
                }
            }
            __syncthreads();
            // the -W record from its row-major staging, eight channels per store
            // (padded key channels are zero)
            for (int p = tid; p < C * (DKP / 8); p += S::NT) {
                const int i = p / (DKP / 8), c8 = 8 * (p % (DKP / 8));
                Frag<OT> f;
                if (c8 < DK) f.load(Wst + i * SK + c8);
                else f.zero();
                f.store(Wwn + fragidx(i, c8, DKP / 32));
            }
        }

        __syncthreads();   // LDS is reused by the next item
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// chunk_state: sequential pass over the chunks of one (b, h), 16 value columns
// (h0 and hT may be the same buffer: each workgroup reads exactly the state
// entries it later writes, and reads them first)
//
// Eight wavefronts in two roles, two per SIMD:
//   waves 0-3, the chain:  E = U - W H and H = Diag(gl) H + Kr^T E, the
//                          sequential dependence from chunk to chunk;
//   waves 4-7, the output: o = Qg H + Aqk E, which nothing later depends on.
// Both roles meet at the two barriers of every chunk step (E published;
// H published), so the output work and its operand loads run beside the
// chain on the same SIMDs instead of in series with it.
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, typename OT, typename OUT, int NT2, bool C8>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
chunk_state(const float* h0, float* hT, OUT* __restrict__ o,
            int T, int H, int BH, int NC, const void* ws, size_t nrec, const int4* __restrict__ stab,
            float* seg, int nseg, int seglen, int phase)
{
    // (ws is deliberately not __restrict__: with it, the record loads count as
    // invariant and the compiler sinks the next chunk's operand loads past the
    // barriers to the point of use, which undoes the prefetch)
    using S = CS<C, DK, DV, OT>;
    constexpr int NB = S::NB, CP = S::CP, DKP = S::DKP, SK = S::SK, SC = S::SC, NP = S::NP;
    constexpr int NCOL = 16 * NT2;        // value columns of one workgroup (NT2 16-column tiles)
    constexpr int NCT = DV / NCOL;        // workgroups per head
    constexpr int MH = DK / 16;           // 16-row tiles of the state
    constexpr int MHW = (MH + 3) / 4;     // state tiles per chain wave
    constexpr int KS = DKP / 32, KC = CP / 32;
    constexpr bool ALLE = NB >= 4;        // every wave of a role owns a token tile
    constexpr bool ALLH = (MH % 4) == 0;  // every chain wave owns MHW state tiles
    // C8 (chains alone, no outputs: phase 1 of the segmented pass): all eight
    // waves are chain waves, in two groups of four that each carry half of
    // the workgroup's tiles, so two chains share every SIMD instead of one
    constexpr int NTW = C8 ? NT2 / 2 : NT2;   // 16-column tiles per chain wave
    // bf16 operands with one tile per wave: three operand sets in rotation (a
    // chunk's operands are requested two steps ahead); otherwise two (with two
    // tiles a third fits the registers but measured no faster)
    constexpr bool THREE = S::SPLIT && NTW == 1;
    static_assert(DV % NCOL == 0, "whole tiles per workgroup");
    static_assert(!C8 || NT2 % 2 == 0, "two groups of whole tiles");

    __shared__ __align__(16) OT HTs[NP * NCOL * SK];   // H^T [n][c] (precise operand)
    __shared__ __align__(16) OT ETs[NP * NCOL * SC];   // E^T [n][j] (precise operand)
    const PArr<OT> HT{HTs, HTs + NCOL * SK};
    const PArr<OT> ET{ETs, ETs + NCOL * SC};

    // Workgroups come in groups of G, one group per (sequence-head, segment).
    // XCD-aware mapping: all workgroups of a group on the same XCD (id % 8),
    // so the chunk records they all read are shared through that XCD's L2.
    //
    // phase 0: one segment per sequence, every workgroup a state chain with
    //   outputs (role 0), from h0 to hT.
    // Segmented sequences (nseg segments of seglen chunks; seg holds three
    // sets of nseg states [BH, DK, DV]: the true states entering the
    // segments, the segments' final states from a zero state, and the
    // segments' transition matrices):
    // phase 1 (no outputs: every workgroup of this pass is a chain alone):
    //   segment 0 runs role 1 from h0, keeps h0 as the state entering segment
    //   0 and leaves its final state as the state entering segment 1; every
    //   later segment runs role 1 from a zero state in its first NCT
    //   workgroups and role 2 (the transition matrix: the same chain from
    //   the identity, with U = 0) in the next NCT;
    // phase 3: every segment runs role 0 (outputs) from its true entering
    //   state (chunk_seg_combine forms those of segments 2 .. nseg-1 in
    //   between); the last one writes hT.  h0 itself is not read here, so a
    //   final state written over the initial one is safe.
    const int id = blockIdx.x;
    const int xcd = id & 7, slot = id >> 3;
    const int G = phase == 1 ? 2 * NCT : NCT;
    const int nsl = phase == 0 ? 1 : nseg;
    const int grp = (slot / G) * 8 + xcd;
    const int wg = slot % G;
    const int bh = grp / nsl;
    if (bh >= BH) return;
    const int segi = grp - bh * nsl;
    int role = 0;
    if (C8 && phase != 1) return;      // (not launched that way)
    if (phase == 1) {
        if (wg >= NCT) {
            if (segi == 0) return;
            role = 2;
        } else {
            role = 1;
        }
    }
    const int ct = wg % NCT;
    const int h = bh - (bh / H) * H;
    const int n0 = NCOL * ct;
    const size_t SS = (size_t)BH * DK * DV;   // one set of states
    const float* h0p = h0;
    float* hTp = hT;
    if (phase == 1) {
        if (segi == 0) {
            hTp = seg + SS;                    // the state entering segment 1
        } else {
            h0p = nullptr;
            hTp = seg + ((size_t)role * nseg + segi) * SS;
        }
    } else if (phase == 3) {
        h0p = seg + (size_t)segi * SS;
        hTp = segi == nseg - 1 ? hT : nullptr;
    }
    // The sequence of this workgroup: its first token, its length, its number
    // of chunks and where its chunk records start.  Dense batches: sequence b
    // of [B, T], records (b*H + h) * NC + chunk.  Packed variable-length
    // batches (stab != null): entry n = (first token, length, first chunk),
    // records g * H + h for global chunk g.
    size_t tokbase, recbase, recstride;
    int seqlen, NCs;
    if (stab) {
        const int4 e = stab[bh / H];
        tokbase = (size_t)e.x;
        seqlen = e.y;
        NCs = (seqlen + C - 1) / C;
        recbase = (size_t)e.z * H + h;
        recstride = (size_t)H;
    } else {
        tokbase = (size_t)(bh / H) * T;
        seqlen = T;
        NCs = NC;
        recbase = (size_t)bh * NC;
        recstride = 1;
    }
    // this workgroup's chunks: c0 .. c0 + NCs - 1 of its sequence
    const int c0 = phase == 0 ? 0 : segi * seglen;
    if (phase != 0) NCs = max(0, min(seglen, NCs - c0));
    const WsLayout<C, DK, DV, OT> W(const_cast<void*>(ws), nrec);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, gq = lane >> 4;
    const bool chain = C8 || wave < 4;
    const int tb = C8 ? (wave >> 2) * NTW : 0;             // first tile of this wave's group
    const int wr = wave & 3;                               // index within the role
    const int we = ALLE ? wr : (wr < NB ? wr : NB - 1);    // token tile of E / o
    const bool has_t = ALLE || wr < NB;

    // zero the operand tiles (padding stays zero)
    for (int p = tid; p < NP * NCOL * SK; p += 512) store_op(HTs + p, 0.f);
    for (int p = tid; p < NP * NCOL * SC; p += 512) store_op(ETs + p, 0.f);
    __syncthreads();

    auto rec_of = [&](int cidx) { return recbase + (size_t)(c0 + cidx) * recstride; };

    if (chain) {
        f32x4 hacc[MHW][NTW];
#pragma unroll
        for (int s = 0; s < MHW; ++s) {
            const int mt = wr + 4 * s;
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                hacc[s][n] = zero4();
                if (mt < MH && role == 2) {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        hacc[s][n][u] = (16 * mt + 4 * gq + u == n0 + 16 * (tb + n) + r) ? 1.f : 0.f;
                } else if (mt < MH && h0p) {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        hacc[s][n][u] = h0p[((size_t)bh * DK + 16 * mt + 4 * gq + u) * DV + n0 + 16 * (tb + n) + r];
                }
                if (mt < MH && phase == 1 && segi == 0) {   // the state entering segment 0, for phase 3
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        seg[((size_t)bh * DK + 16 * mt + 4 * gq + u) * DV + n0 + 16 * (tb + n) + r] = hacc[s][n][u];
                }
                if (mt < MH) store4_p(HT, (16 * (tb + n) + r) * SK + 16 * mt + 4 * gq, hacc[s][n]);
            }
        }
        __syncthreads();

        // Operands of one chunk step, shared by the workgroup's NT2 column
        // tiles (only U is per tile).  The loads are unconditional
        // straight-line code (indices clamped; zero padding in the records
        // makes the extra fragments harmless) so that the wait for one set
        // never includes the loads of another.
        struct Ops {
            Frag<OT> wn[KS];         // -W rows 16*we.. (A operand of E)
            PFrag<OT> kr[MHW][KC];   // Kr^T rows 16*mt.. (A operand of the state update)
            f32x4 u[NTW];            // U^T init of E
            float gl;                // exp(G_last) of one state row (see gl_of)
        };
        auto mt_of = [&](int s) { return ALLH ? wr + 4 * s : min(wr + 4 * s, MH - 1); };
        // The decays exp(G_last) of a wave's state rows are one 4-byte load per
        // lane (lane l: row l % 16 of state tile (l / 16) % MHW) rather than a
        // 16-byte load per lane and tile of which every 16 lanes share each
        // value; each lane takes its four rows of a tile by lane exchange.
        auto gl_of = [&](size_t rec) {
            return W.gl[rec * DK + 16 * mt_of((lane >> 4) % MHW) + (lane & 15)];
        };
        auto load_ops = [&](Ops& P, int cidx) {
            const size_t rec = rec_of(cidx);
            const OT* wn = W.wneg_rec(rec);
            const PArr<OT> kr = W.krt(rec);
#pragma unroll
            for (int n = 0; n < NTW; ++n)
                P.u[n] = Vec4<float>::load(W.ut + rec * S::U_N + accbase(NT2 * ct + tb + n, we, NB, lane));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) P.wn[ks].load(wn + fragbase(we, ks, KS, lane));
            P.gl = gl_of(rec);
#pragma unroll
            for (int s = 0; s < MHW; ++s) {
#pragma unroll
                for (int ks = 0; ks < KC; ++ks) P.kr[s][ks] = kr.frag(fragbase(mt_of(s), ks, KC, lane));
            }
        };
        // One chunk step with operands P.  The operands of chunk `nxt` are
        // loaded into Q in the order the next step consumes them (U, -W, gl,
        // Kr^T): the memory counter retires in order, so every wait of the
        // next step covers only loads issued a whole step before.  U and -W
        // are requested in the E phase, gl and Kr^T in the update phase, so
        // the record traffic of a step is spread over both of its phases (the
        // load unit of the compute unit, not the matrix cores, bounds the
        // step).  Accumulations are split into independent chains so that the
        // matrix-core latency is not paid once per k step.
        auto step = [&](const Ops& P, Ops& Q, int nxt) {
            const size_t rec = rec_of(nxt);
            const OT* wn = W.wneg_rec(rec);
            const PArr<OT> kr = W.krt(rec);
#pragma unroll
            for (int n = 0; n < NTW; ++n)
                Q.u[n] = Vec4<float>::load(W.ut + rec * S::U_N + accbase(NT2 * ct + tb + n, we, NB, lane));
            // this lane's rows 4 gq .. 4 gq + 3 of each state tile
            f32x4 g4[MHW];
#pragma unroll
            for (int s = 0; s < MHW; ++s) {
#pragma unroll
                for (int u = 0; u < 4; ++u) g4[s][u] = __shfl(P.gl, 16 * s + 4 * gq + u);
            }
            f32x4 ea[NTW], eb[NTW];
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                ea[n] = role == 2 ? zero4() : P.u[n];   // the transition matrix has no U term
                eb[n] = zero4();
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Q.wn[ks].load(wn + fragbase(we, ks, KS, lane));
                if (has_t) {
#pragma unroll
                    for (int n = 0; n < NTW; ++n) {
                        const PFrag<OT> hf = HT.frag((16 * (tb + n) + r) * SK + 32 * ks + 8 * gq);
                        if (ks & 1) eb[n] = mma2(P.wn[ks], hf, eb[n]);
                        else ea[n] = mma2(P.wn[ks], hf, ea[n]);
                    }
                }
            }
            if (has_t) {
#pragma unroll
                for (int n = 0; n < NTW; ++n)
                    store4_p(ET, (16 * (tb + n) + r) * SC + 16 * wr + 4 * gq, ea[n] + eb[n]);
            }
#pragma unroll
            for (int g2 = 0; g2 < KS; ++g2) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * NTW, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x020, NTW, 0);
            __syncthreads();
            // H = Diag(gl) H + Kr^T E
            f32x4 part[MHW][NTW];
#pragma unroll
            for (int s = 0; s < MHW; ++s) {
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    if (ALLH || wr + 4 * s < MH) hacc[s][n] *= g4[s];
                    part[s][n] = zero4();
                }
            }
            Q.gl = gl_of(rec);
#pragma unroll
            for (int ks = 0; ks < KC; ++ks) {
                PFrag<OT> et[NTW];
#pragma unroll
                for (int n = 0; n < NTW; ++n) et[n] = ET.frag((16 * (tb + n) + r) * SC + 32 * ks + 8 * gq);
#pragma unroll
                for (int s = 0; s < MHW; ++s) {
                    Q.kr[s][ks] = kr.frag(fragbase(mt_of(s), ks, KC, lane));
                    if (ALLH || wr + 4 * s < MH) {
#pragma unroll
                        for (int n = 0; n < NTW; ++n) {
                            if (ks & 1) part[s][n] = mma3(P.kr[s][ks], et[n], part[s][n]);
                            else hacc[s][n] = mma3(P.kr[s][ks], et[n], hacc[s][n]);
                        }
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < MHW; ++s) {
                const int mt = wr + 4 * s;
                if (ALLH || mt < MH) {
#pragma unroll
                    for (int n = 0; n < NTW; ++n) {
                        hacc[s][n] += part[s][n];
                        store4_p(HT, (16 * (tb + n) + r) * SK + 16 * mt + 4 * gq, hacc[s][n]);
                    }
                }
            }
            __syncthreads();
        };
        if (NCs > 0 && THREE) {
            // three operand sets in rotation: a chunk's operands are requested
            // two steps before they are used (the records come from beyond the
            // L2, whose latency one step does not cover)
            Ops A, B, D;
            load_ops(A, 0);
            load_ops(B, min(1, NCs - 1));
            for (int cidx = 0; cidx < NCs; cidx += 3) {
                step(A, D, min(cidx + 2, NCs - 1));
                if (cidx + 1 < NCs) step(B, A, min(cidx + 3, NCs - 1));
                if (cidx + 2 < NCs) step(D, B, min(cidx + 4, NCs - 1));
            }
        } else if (NCs > 0) {
            Ops A, B;
            load_ops(A, 0);
            for (int cidx = 0; cidx < NCs; cidx += 2) {
                step(A, B, min(cidx + 1, NCs - 1));
                if (cidx + 1 < NCs) step(B, A, min(cidx + 2, NCs - 1));
            }
        }
        if (hTp) {
#pragma unroll
            for (int s = 0; s < MHW; ++s) {
                const int mt = wr + 4 * s;
                if (mt < MH) {
#pragma unroll
                    for (int n = 0; n < NTW; ++n) {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            hTp[((size_t)bh * DK + 16 * mt + 4 * gq + u) * DV + n0 + 16 * (tb + n) + r] = hacc[s][n][u];
                    }
                }
            }
        }
    } else if (role != 0) {
        // no outputs: the output waves only keep the chain's barriers
        __syncthreads();
        for (int cidx = 0; cidx < NCs; ++cidx) {
            __syncthreads();
            __syncthreads();
        }
    } else {
        __syncthreads();   // initial state published
        struct Ops {
            Frag<OT> qg[KS];         // Qg rows 16*we.. (B operand of o^T)
            PFrag<OT> aq[KC];        // Aqk rows 16*we.. (B operand of o^T)
        };
        // Aqk is lower triangular: the 32-column fragments right of this
        // wave's token tile are zero and are neither loaded nor multiplied
        // (a condition uniform over the wave)
        const int weu = __builtin_amdgcn_readfirstlane(we);
        auto aq_live = [&](int ks) { return 32 * ks <= 16 * weu + 15; };
        auto load_ops = [&](Ops& P, int cidx) {
            const size_t rec = rec_of(cidx);
            const OT* qg = W.qg_rec(rec);
            const PArr<OT> aq = W.aqk(rec);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) P.qg[ks].load(qg + fragbase(we, ks, KS, lane));
#pragma unroll
            for (int ks = 0; ks < KC; ++ks)
                if (aq_live(ks)) P.aq[ks] = aq.frag(fragbase(we, ks, KC, lane));
        };
        auto step = [&](const Ops& P, int cidx, Ops& Q, int nxt) {
            const size_t rec = rec_of(nxt);
            const OT* qg = W.qg_rec(rec);
            const PArr<OT> aq = W.aqk(rec);
            f32x4 oa[NT2], ob[NT2];   // two independent accumulation chains per tile
#pragma unroll
            for (int n = 0; n < NT2; ++n) {
                oa[n] = zero4();
                ob[n] = zero4();
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Q.qg[ks].load(qg + fragbase(we, ks, KS, lane));
                if (has_t) {
#pragma unroll
                    for (int n = 0; n < NT2; ++n) {
                        const PFrag<OT> hf = HT.frag((16 * n + r) * SK + 32 * ks + 8 * gq);
                        if (ks & 1) ob[n] = mma2(hf, P.qg[ks], ob[n]);
                        else oa[n] = mma2(hf, P.qg[ks], oa[n]);
                    }
                }
            }
#pragma unroll
            for (int g2 = 0; g2 < KS; ++g2) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * NT2, 0);
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < KC; ++ks) {
                if (!aq_live(ks)) continue;
                Q.aq[ks] = aq.frag(fragbase(we, ks, KC, lane));
                if (has_t) {
#pragma unroll
                    for (int n = 0; n < NT2; ++n) {
                        const PFrag<OT> ef = ET.frag((16 * n + r) * SC + 32 * ks + 8 * gq);
                        if (ks & 1) ob[n] = mma3(ef, P.aq[ks], ob[n]);
                        else oa[n] = mma3(ef, P.aq[ks], oa[n]);
                    }
                }
            }
            if (has_t) {
                // lane holds o^T[n = 4gq + u][i = 16*wr + r] of each tile
                const int t0 = (c0 + cidx) * C;
                const int i = 16 * wr + r;
                if (i < min(C, seqlen - t0)) {
                    OUT* op = o + ((tokbase + t0 + i) * H + h) * DV + n0 + 4 * gq;
#pragma unroll
                    for (int n = 0; n < NT2; ++n) Vec4<OUT>::store(op + 16 * n, oa[n] + ob[n]);
                }
            }
            __syncthreads();
        };
        if (NCs > 0 && THREE) {
            Ops A, B, D;
            load_ops(A, 0);
            load_ops(B, min(1, NCs - 1));
            for (int cidx = 0; cidx < NCs; cidx += 3) {
                step(A, cidx, D, min(cidx + 2, NCs - 1));
                if (cidx + 1 < NCs) step(B, cidx + 1, A, min(cidx + 3, NCs - 1));
                if (cidx + 2 < NCs) step(D, cidx + 2, B, min(cidx + 4, NCs - 1));
            }
        } else if (NCs > 0) {
            Ops A, B;
            load_ops(A, 0);
            for (int cidx = 0; cidx < NCs; cidx += 2) {
                step(A, cidx, B, min(cidx + 1, NCs - 1));
                if (cidx + 1 < NCs) step(B, cidx + 1, A, min(cidx + 2, NCs - 1));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Segmented sequences: the true state entering each segment, in order,
//   H_{s+1} = M_s H_s + Z_s,   s = 1 .. nseg - 2,
// from H_1 (left by segment 0) with the segments' transition matrices M_s and
// their final states from zero Z_s (the chunk carry is affine in the state
// it starts from).  One workgroup per (sequence-head, 16 value columns), one
// wave per 16 rows of the state, float32 products on the matrix cores
// (v_mfma_f32_16x16x4_f32: exact float32 products, float32 sums).
template <int DK, int DV>
__global__ void __launch_bounds__(4 * DK) chunk_seg_combine(float* seg, int BH, int nseg)
{
    static_assert(DK == DV, "square transition matrices");
    // Wave t forms rows 16t .. 16t+15 of the new state tile.  Lane (r, g)
    // holds them as an accumulator (rows 16t + 4g + u, column r) and, for
    // the product, supplies M_s[16t + r][k] and H_s[k][r] for the keys
    // k = KQ*g .. KQ*g + KQ-1, one per 16x16x4 step (any fixed assignment of
    // the keys to the steps gives the same sum).  The state tile sits in LDS
    // transposed ([column][row]), in two buffers used in turn, so that one
    // barrier per segment suffices.  The next segment's operands (this
    // lane's keys of its row of M, and its Z entries) are requested before
    // this segment's products, into the other of two register sets, from a
    // clamped (always valid) segment index.
    constexpr int D = DK, NCT = DV / 16, KQ = D / 4, SH = D + 4;
    __shared__ __align__(16) float HsT[2][16 * SH];
    const int bh = blockIdx.x / NCT, ct = blockIdx.x % NCT;
    if (bh >= BH) return;
    const size_t SS = (size_t)BH * D * DV;
    const int tid = threadIdx.x, lane = tid & 63, t = tid >> 6, r = lane & 15, g = lane >> 4;
    const size_t base = (size_t)bh * D * DV;
    const int row0 = 16 * t + 4 * g;                              // this lane's accumulator rows
    const size_t ooff = base + (size_t)row0 * DV + 16 * ct + r;   // (row0, column r) of a state
    {
        f32x4 h;
#pragma unroll
        for (int u = 0; u < 4; ++u) h[u] = seg[SS + ooff + (size_t)u * DV];
        *reinterpret_cast<f32x4*>(&HsT[0][r * SH + row0]) = h;
    }
    struct Ops {
        f32x4 m[KQ / 4];   // M_s[16t + r][KQ*g ..]
        f32x4 z;           // Z_s[row0 + u][column r]
    };
    const int last = nseg - 2;     // the last segment whose map is applied
    auto load = [&](Ops& P, int s2) {
        const f32x4* M = reinterpret_cast<const f32x4*>(seg + ((size_t)2 * nseg + s2) * SS + base +
                                                        (size_t)(16 * t + r) * DV + KQ * g);
#pragma unroll
        for (int j = 0; j < KQ / 4; ++j) P.m[j] = M[j];
        const float* Z = seg + ((size_t)nseg + s2) * SS + ooff;
#pragma unroll
        for (int u = 0; u < 4; ++u) P.z[u] = Z[(size_t)u * DV];
    };
    auto step = [&](const Ops& P, Ops& Q, int s2, int buf) {
        load(Q, min(s2 + 1, last));
        const float* hb = &HsT[buf][r * SH + KQ * g];
        f32x4 acc[4] = {P.z, zero4(), zero4(), zero4()};   // four independent chains
#pragma unroll
        for (int j = 0; j < KQ / 4; ++j) {
            const f32x4 hv = *reinterpret_cast<const f32x4*>(hb + 4 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = mma4(P.m[j][e], hv[e], acc[e]);
        }
        const f32x4 hn = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        *reinterpret_cast<f32x4*>(&HsT[buf ^ 1][r * SH + row0]) = hn;
        float* out = seg + (size_t)(s2 + 1) * SS + ooff;
#pragma unroll
        for (int u = 0; u < 4; ++u) out[(size_t)u * DV] = hn[u];
        __syncthreads();
    };
    if (last < 1) return;
    Ops A, B;
    load(A, 1);
    __syncthreads();               // H_1 in LDS
    for (int s2 = 1; s2 <= last; s2 += 2) {
        step(A, B, s2, 0);
        if (s2 + 1 <= last) step(B, A, s2 + 1, 1);
    }
}

// ---------------------------------------------------------------------------
// Number of workgroups of `kernel` (with `threads` threads) that the current
// device holds at once: compute units times the occupancy limit, queried once
// per kernel and device.
template <typename K>
int resident_blocks(K kernel, int threads)
{
    constexpr int MAXDEV = 64;
    static std::atomic<int> cache[MAXDEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < MAXDEV ? dev : MAXDEV - 1;
    int n = cache[slot].load(std::memory_order_relaxed);
    if (n > 0 && dev < MAXDEV) return n;
    int ncu = 0, per = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        ncu = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess || per < 1)
        per = 1;
    n = ncu * per;
    if (dev < MAXDEV) cache[slot].store(n, std::memory_order_relaxed);
    return n;
}

// Upper bound of the number of chunks of a packed batch, and the workspace
// layout of the packed form: the records of Gmax * H chunks, then the chunk
// table, then the sequence table.
inline size_t varlen_gmax(int N, int Ttot, int C) { return (size_t)(Ttot + C - 1) / C + (size_t)N; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Segments per sequence of the dense state pass.  A long sequence over few
// heads walks a long serial chain on a small part of the device (one
// workgroup per head and 32 value columns; 256 of them fill an MI355X); it is
// cut into up to 8 segments of at least 32 chunks that run side by side.
// 1 (no segments) unless d_k = d_v >= 32 and the sequence has at least 256
// chunks.  A function of the shape alone, so that the workspace size does not
// depend on the device.
inline int seg_count(int B, int T, int H, int Dk, int Dv, int C)
{
    if (Dk != Dv || Dv < 32) return 1;
    const long nc = (T + C - 1) / C;
    if (nc < 256) return 1;
    const long tiles = (long)B * H * (Dv / 32);
    long s = 256 / (tiles > 0 ? tiles : 1);
    if (s > 8) s = 8;
    while (s > 1 && nc < 32 * s) --s;
    return s < 2 ? 1 : (int)s;
}
// Bytes of the segment states (three sets of nseg states [B, H, Dk, Dv]).
inline size_t seg_bytes(int B, int T, int H, int Dk, int Dv, int C)
{
    const int ns = seg_count(B, T, H, Dk, Dv, C);
    return ns > 1 ? (size_t)3 * ns * B * H * Dk * Dv * 4 : 0;
}

// LDS of chunk_prepare (its staging arrays, then the per-block gate terms,
// norms, pair factors, flags and the diagonal blocks of A, as declared in the
// kernel) against the 160 KiB of a compute unit: the shapes beyond it (float32
// operands with chunk 64, d_k 128 and d_v 256) are not instantiated.
template <int C, int DK, int DV, typename OT>
constexpr bool chunk_shape_fits()
{
    using S = CS<C, DK, DV, OT>;
    constexpr long other = C * 4 + 4L * S::NB * S::DKP * 4 + S::KSN * 2L * C * 4 + 2L * C * 4 +
                           (S::NPAIR > 0 ? S::NPAIR : 1) * (long)S::DKP * 4 + (long)S::NB * S::DKP + 4 +
                           S::NB * 16L * 20 * 4;
    return S::BIG + other <= 160L * 1024;
}

// The state pass: one workgroup per (sequence, head, NT2 16-column value
// tiles).  Two tiles per workgroup share every record load and halve the
// pass's compute-unit time; one tile per workgroup gives the most
// workgroups.  Two tiles are taken once one tile per workgroup would need
// more workgroups than the device holds at once (the pass then runs in
// several waves of workgroups anyway).
template <int C, int DK, int DV, typename OT, int NT2, bool C8 = false>
hipError_t launch_state_nt(const ChunkArgs& a, int BH, int NC, size_t nrec, const int4* stab,
                           float* seg, int nseg, int seglen, int phase, hipStream_t s)
{
    constexpr int NCT = DV / (16 * NT2);
    const int nsl = phase == 0 ? 1 : nseg;
    const int G = phase == 1 ? 2 * NCT : NCT;
    const long groups = ((long)BH * nsl + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * G));
    if (a.o_dtype == KDA_F32)
        hipLaunchKernelGGL((chunk_state<C, DK, DV, OT, float, NT2, C8>), grid, dim3(512), 0, s,
                           a.h0, a.hT, (float*)a.o, a.T, a.H, BH, NC, (const void*)a.ws, nrec, stab,
                           seg, nseg, seglen, phase);
    else
        hipLaunchKernelGGL((chunk_state<C, DK, DV, OT, bf16_t, NT2, C8>), grid, dim3(512), 0, s,
                           a.h0, a.hT, (bf16_t*)a.o, a.T, a.H, BH, NC, (const void*)a.ws, nrec, stab,
                           seg, nseg, seglen, phase);
    return hipGetLastError();
}

// The state pass, in one of two shapes.
// Plain: one workgroup per (sequence, head, NT2 16-column value tiles).  Two
// tiles per workgroup share every record load and halve the pass's
// compute-unit time; one tile per workgroup gives the most workgroups.  Two
// tiles are taken once one tile per workgroup would need more workgroups
// than the device holds at once (the pass then runs in several waves of
// workgroups anyway), and four (bf16 operands) once two would.
// Segmented (nseg > 1, see seg_count): phase 1, chunk_seg_combine, phase 3,
// two tiles per workgroup.
template <int C, int DK, int DV, typename OT>
hipError_t launch_state(const ChunkArgs& a, int BH, int NC, size_t nrec, const int4* stab,
                        float* seg, int nseg, hipStream_t s)
{
    if constexpr (DV >= 32) {
        if (nseg > 1) {
            if constexpr (DK == DV) {
                const int seglen = (NC + nseg - 1) / nseg;
                // phase 1 runs two chains per later segment (its zero-state
                // part and its transition matrix): four tiles per workgroup
                // (bf16 operands) keep it to one workgroup per compute unit;
                // it has no outputs, so all eight waves carry chains
                hipError_t e;
                if constexpr (std::is_same<OT, bf16_t>::value && DV % 64 == 0)
                    e = launch_state_nt<C, DK, DV, OT, 4, true>(a, BH, NC, nrec, stab, seg, nseg, seglen, 1, s);
                else
                    e = launch_state_nt<C, DK, DV, OT, 2, true>(a, BH, NC, nrec, stab, seg, nseg, seglen, 1, s);
                if (e != hipSuccess) return e;
                hipLaunchKernelGGL((chunk_seg_combine<DK, DV>), dim3(BH * (DV / 16)), dim3(4 * DK), 0, s,
                                   seg, BH, nseg);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                return launch_state_nt<C, DK, DV, OT, 2>(a, BH, NC, nrec, stab, seg, nseg, seglen,
                                                         3, s);
            }
            return hipErrorInvalidValue;
        }
        int ncu = 0, dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            ncu = 256;
        // four tiles (bf16 operands) once two would still need more than one
        // workgroup per compute unit
        if constexpr (std::is_same<OT, bf16_t>::value && DV % 64 == 0) {
            if ((double)BH * (DV / 32) > (double)ncu)
                return launch_state_nt<C, DK, DV, OT, 4>(a, BH, NC, nrec, stab, nullptr, 1, NC, 0, s);
        }
        if ((double)BH * (DV / 16) > (double)ncu)
            return launch_state_nt<C, DK, DV, OT, 2>(a, BH, NC, nrec, stab, nullptr, 1, NC, 0, s);
    }
    return launch_state_nt<C, DK, DV, OT, 1>(a, BH, NC, nrec, stab, nullptr, 1, NC, 0, s);
}

template <int C, int DK, int DV, typename OT>
hipError_t launch3(const ChunkArgs& a, hipStream_t s)
{
    if constexpr (!chunk_shape_fits<C, DK, DV, OT>()) {
        (void)a; (void)s;
        return hipErrorInvalidValue;
    } else {
    const bool packed = a.cu != nullptr;
    int BH, NC, nitem;
    size_t nrec;
    const int2* ctab = nullptr;
    const int4* stab = nullptr;
    if (packed) {   // the tables were built in the workspace by the caller
        const size_t gmax = varlen_gmax(a.N, a.T, C);
        BH = a.N * a.H;
        NC = 0;
        nrec = gmax * a.H;
        nitem = (int)nrec;
        ctab = (const int2*)a.ctab;
        stab = (const int4*)a.stab;
    } else {
        BH = a.B * a.H;
        NC = (a.T + C - 1) / C;
        nrec = (size_t)BH * NC;
        nitem = (int)nrec;
    }
    if (nitem > 0 && a.T > 0) {
        // persistent workgroups: as many as can be resident at once
        constexpr int NT = CS<C, DK, DV, OT>::NT;
        if (a.prologue) {
            const int grid = min(nitem, resident_blocks(chunk_prepare<C, DK, DV, OT, true>, NT));
            hipLaunchKernelGGL((chunk_prepare<C, DK, DV, OT, true>), dim3(grid), dim3(NT), 0, s,
                               (const OT*)a.q, (const OT*)a.k, (const OT*)a.v, a.g, a.beta,
                               a.T, a.H, a.Hq, NC, nitem, a.scale, (int)a.mode, a.ws, nrec, ctab,
                               a.prologue);
        } else {
            const int grid = min(nitem, resident_blocks(chunk_prepare<C, DK, DV, OT, false>, NT));
            hipLaunchKernelGGL((chunk_prepare<C, DK, DV, OT, false>), dim3(grid), dim3(NT), 0, s,
                               (const OT*)a.q, (const OT*)a.k, (const OT*)a.v, a.g, a.beta,
                               a.T, a.H, a.Hq, NC, nitem, a.scale, (int)a.mode, a.ws, nrec, ctab, 0);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (BH == 0) return hipSuccess;
    const int nseg = packed ? 1 : seg_count(a.B, a.T, a.H, a.Dk, a.Dv, C);
    float* seg = nseg > 1 ? (float*)((char*)a.ws + align_up(WsLayout<C, DK, DV, OT>::bytes(nrec), 256))
                          : nullptr;
    return launch_state<C, DK, DV, OT>(a, BH, NC, nrec, stab, seg, nseg, s);
    }
}

// Bytes of the chunk records of nrec (chunk, head) items; 0 for a shape that
// is not instantiated.
template <int C, int DK, int DV, typename OT>
size_t records_bytes(size_t nrec)
{
    if constexpr (!chunk_shape_fits<C, DK, DV, OT>()) {
        (void)nrec;
        return 0;
    } else {
        return WsLayout<C, DK, DV, OT>::bytes(nrec);
    }
}

// Every (Dk, Dv) the library supports, Dk in {16, 32, 64, 128} and Dv in
// {16, 32, 64, 128, 256}: F(C, DK, DV) is expanded for each.
#define KDA_FOR_DV(F, CC, DK) F(CC, DK, 16) F(CC, DK, 32) F(CC, DK, 64) F(CC, DK, 128) F(CC, DK, 256)
#define KDA_FOR_DKDV(F, CC) KDA_FOR_DV(F, CC, 16) KDA_FOR_DV(F, CC, 32) KDA_FOR_DV(F, CC, 64) KDA_FOR_DV(F, CC, 128)

// One chunk length each (kda_chunk_c<C>.hip).
hipError_t launch_chunk_c16(const ChunkArgs& a, hipStream_t s);
hipError_t launch_chunk_c32(const ChunkArgs& a, hipStream_t s);
hipError_t launch_chunk_c64(const ChunkArgs& a, hipStream_t s);
size_t records_bytes_c16(size_t nrec, int Dk, int Dv, kda_dtype dtype);
size_t records_bytes_c32(size_t nrec, int Dk, int Dv, kda_dtype dtype);
size_t records_bytes_c64(size_t nrec, int Dk, int Dv, kda_dtype dtype);

}  // namespace kda
